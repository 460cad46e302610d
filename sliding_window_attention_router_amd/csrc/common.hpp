// Device-side vocabulary shared by the SwiAttn kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SWI_DEV __device__ __forceinline__

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace swi {

constexpr int kWave = 64;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;

// bfloat16 storage type.  Conversions from float lower to the gfx950
// v_cvt_pk_bf16_f32 instruction (round to nearest even).
using bf16_t = __bf16;

SWI_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
SWI_DEV float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of lane l ^ 32 (the other half of the wave), through the gfx950
// v_permlane32_swap (a VALU op, no LDS round trip): swapping the upper half
// of one copy with the lower half of another leaves lane l's partner value
// in the second result for l < 32 and in the first for l >= 32.
SWI_DEV float xor32(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(__lane_id() < 32 ? r[1] : r[0]);
}

SWI_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
SWI_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
SWI_DEV int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  return v;
}
SWI_DEV int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
// Inclusive prefix sum over the lanes of the wave.
SWI_DEV int wave_incl_scan_i(int v) {
  const int lane = __lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}
SWI_DEV int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}

// Element type traits: storage type and bytes.
template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kBytes = 4;
  SWI_DEV static float load(const float* p) { return *p; }
  SWI_DEV static void store(float* p, float v) { *p = v; }
};
template <>
struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
  SWI_DEV static float load(const bf16_t* p) { return float(*p); }
  SWI_DEV static void store(bf16_t* p, float v) { *p = bf16_t(v); }
};

}  // namespace swi
