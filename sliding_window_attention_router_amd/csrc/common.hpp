// Device-side vocabulary shared by the SwiAttn kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

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

// Wave-wide reductions on the DPP network (VALU only, no LDS round trip):
// combine within quads, half-rows and rows of 16 lanes, then across rows
// (row_bcast15 into rows 1 and 3, row_bcast31 into rows 2 and 3); lane 63
// ends with the total, which is returned to every lane.  Lanes a step does
// not update read the identity.  The combining order is fixed.
template <int CTRL, int ROWS = 0xF>
SWI_DEV int dpp_src(int v, int identity) {
  return __builtin_amdgcn_update_dpp(identity, v, CTRL, ROWS, 0xF, false);
}
template <typename Op>
SWI_DEV int wave_reduce(int v, int identity, Op op) {
  v = op(v, dpp_src<0xB1>(v, identity));        // quad_perm [1,0,3,2]
  v = op(v, dpp_src<0x4E>(v, identity));        // quad_perm [2,3,0,1]
  v = op(v, dpp_src<0x141>(v, identity));       // row_half_mirror
  v = op(v, dpp_src<0x140>(v, identity));       // row_mirror
  v = op(v, dpp_src<0x142, 0xA>(v, identity));  // row_bcast15
  v = op(v, dpp_src<0x143, 0xC>(v, identity));  // row_bcast31
  return __builtin_amdgcn_readlane(v, 63);
}
SWI_DEV float wave_max(float v) {
  return __int_as_float(wave_reduce(__float_as_int(v), __float_as_int(-__builtin_huge_valf()),
                                    [](int a, int b) {
                                      return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b)));
                                    }));
}
SWI_DEV float wave_sum(float v) {
  return __int_as_float(wave_reduce(__float_as_int(v), 0, [](int a, int b) {
    return __float_as_int(__int_as_float(a) + __int_as_float(b));
  }));
}
SWI_DEV int wave_min_i(int v) {
  return wave_reduce(v, INT_MAX, [](int a, int b) { return min(a, b); });
}
SWI_DEV int wave_max_i(int v) {
  return wave_reduce(v, INT_MIN, [](int a, int b) { return max(a, b); });
}
SWI_DEV int wave_sum_i(int v) {
  return wave_reduce(v, 0, [](int a, int b) { return a + b; });
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
