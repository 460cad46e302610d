// Router logits + hard gate, and compaction of the full-branch tokens.
//
// SwiAttn report, section 2 (router paragraph): per layer and per token a
// linear map of the hidden state gives a logit; the forward gate is the
// indicator of sigmoid(logit) > 0.5, which is the indicator of logit > 0.
#include "common.hpp"
#include "kernels.hpp"

namespace swi {

// One wave per token.  Lane l accumulates the products of the 16-byte
// vectors l, l+64, l+128, ... of the hidden row in that order, then the wave
// reduces with a fixed xor tree, so the logit is bitwise reproducible.
template <typename T>
__global__ __launch_bounds__(256) void route_kernel(const T* __restrict__ H,
                                                    const T* __restrict__ r,
                                                    const float* __restrict__ bias,
                                                    uint8_t* __restrict__ gate,
                                                    float* __restrict__ z_out, int64_t tokens,
                                                    int hidden, int G) {
  constexpr int VEC = 16 / Elem<T>::kBytes;  // elements per 16-byte load
  const int lane = threadIdx.x & 63;
  const int64_t tok = int64_t(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (tok >= tokens) return;
  const T* row = H + tok * hidden;
  const bool vec_ok = (hidden % VEC) == 0;
  for (int g = 0; g < G; ++g) {
    float acc = 0.f;
    if (vec_ok) {
      const int nvec = hidden / VEC;
      for (int v = lane; v < nvec; v += 64) {
        u32x4 hv = *reinterpret_cast<const u32x4*>(row + int64_t(v) * VEC);
        const T* hp = reinterpret_cast<const T*>(&hv);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const int k = v * VEC + e;
          acc = fmaf(Elem<T>::load(hp + e), Elem<T>::load(r + int64_t(k) * G + g), acc);
        }
      }
    } else {
      for (int k = lane; k < hidden; k += 64)
        acc = fmaf(Elem<T>::load(row + k), Elem<T>::load(r + int64_t(k) * G + g), acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) {
      const float z = acc + bias[g];
      gate[tok * G + g] = z > 0.f ? 1 : 0;
      if (z_out) z_out[tok * G + g] = z;
    }
  }
}

// Single gate group, bf16/fp32 rows whose length is a multiple of the
// 16-byte vector: each wave takes kTok tokens, every lane issues all of its
// 16-byte loads (kTok rows x the vectors it owns) before reducing, and the
// weight vectors a lane owns are loaded once.  Same per-lane order and xor
// tree as route_kernel.
constexpr int kTok = 1;  // tokens per wave (1 measured fastest: more waves in flight than 2, 3, 4 or 8)
template <typename T, int NV>
__global__ __launch_bounds__(256) void route_g1_kernel(const T* __restrict__ H,
                                                       const T* __restrict__ r,
                                                       const float* __restrict__ bias,
                                                       uint8_t* __restrict__ gate,
                                                       float* __restrict__ z_out, int64_t tokens,
                                                       int hidden) {
  constexpr int VEC = 16 / Elem<T>::kBytes;
  const int lane = threadIdx.x & 63;
  const int64_t tok0 = (int64_t(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6)) * kTok;
  if (tok0 >= tokens) return;
  u32x4 rv[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) rv[j] = *reinterpret_cast<const u32x4*>(r + int64_t(lane + 64 * j) * VEC);
  u32x4 hv[kTok][NV];
#pragma unroll
  for (int t = 0; t < kTok; ++t)
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int64_t tok = min(tok0 + t, tokens - 1);
      // read once: the non-temporal hint keeps the stream out of the caches
      // (the plain load ran at 4.9 TB/s, a read probe reaches 7 TB/s with it)
      hv[t][j] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(H + tok * hidden + int64_t(lane + 64 * j) * VEC));
    }
  float acc[kTok];
#pragma unroll
  for (int t = 0; t < kTok; ++t) {
    acc[t] = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const T* hp = reinterpret_cast<const T*>(&hv[t][j]);
      const T* rp = reinterpret_cast<const T*>(&rv[j]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[t] = fmaf(Elem<T>::load(hp + e), Elem<T>::load(rp + e), acc[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < kTok; ++t) {
    const float sum = wave_sum(acc[t]);
    if (lane == 0 && tok0 + t < tokens) {
      const float z = sum + bias[0];
      gate[tok0 + t] = z > 0.f ? 1 : 0;
      if (z_out) z_out[tok0 + t] = z;
    }
  }
}

// One 1024-thread block per (batch, gate group).  Each thread owns a
// contiguous segment of positions, counts its routed tokens, a block-wide
// exclusive prefix sum (wave shuffles + one LDS pass) gives each segment its
// output offset, and each thread then writes its positions in ascending
// order.  The result is the unique ascending list.
constexpr int kCompactThreads = 1024;

__global__ __launch_bounds__(kCompactThreads) void compact_kernel(const uint8_t* __restrict__ gate,
                                                                  int32_t* __restrict__ idx,
                                                                  int32_t* __restrict__ cnt,
                                                                  int N, int G) {
  __shared__ int wave_tot[kCompactThreads / 64];
  __shared__ int carry_s;
  const int bg = blockIdx.x;  // b * G + g
  const int b = bg / G, g = bg - b * G;
  const uint8_t* gp = gate + int64_t(b) * N * G + g;
  int32_t* out = idx + int64_t(bg) * N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // segments of `seg` positions; loop in rounds when N is large
  const int seg = 32;
  const int round_len = seg * kCompactThreads;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < N; base += round_len) {
    const int s0 = base + tid * seg;
    const int s1 = min(s0 + seg, N);
    uint32_t bits = 0;
    if (G == 1 && s1 - s0 == seg && ((reinterpret_cast<uintptr_t>(gp + s0) & 15) == 0)) {
      // 32 gate bytes as two 16-byte loads
      const u32x4 w0 = *reinterpret_cast<const u32x4*>(gp + s0);
      const u32x4 w1 = *reinterpret_cast<const u32x4*>(gp + s0 + 16);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t wd = k < 4 ? w0[k] : w1[k - 4];
#pragma unroll
        for (int e = 0; e < 4; ++e) bits |= (((wd >> (8 * e)) & 0xffu) != 0 ? 1u : 0u) << (4 * k + e);
      }
    } else {
      for (int i = s0; i < s1; ++i) bits |= (gp[int64_t(i) * G] != 0 ? 1u : 0u) << (i - s0);
    }
    const int c = __popc(bits);
    // inclusive scan within the wave
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
      int v = lane < kCompactThreads / 64 ? wave_tot[lane] : 0;
      int w = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(w, o, 64);
        if (lane >= o) w += t;
      }
      if (lane < kCompactThreads / 64) wave_tot[lane] = w - v;  // exclusive
    }
    __syncthreads();
    const int carry = carry_s;
    int pos = carry + wave_tot[wave] + incl - c;
    while (bits) {
      const int j = __ffs(bits) - 1;
      bits &= bits - 1;
      out[pos++] = s0 + j;
    }
    __syncthreads();
    if (tid == kCompactThreads - 1) carry_s = pos;  // last thread's end = round total
    __syncthreads();
  }
  if (tid == 0) cnt[bg] = carry_s;
}

hipError_t launch_route(const void* H, const void* r, const float* bias, uint8_t* gate,
                        float* z_out, int B, int N, int hidden, int G, bool f32,
                        hipStream_t s) {
  const int64_t tokens = int64_t(B) * N;
  const int wpb = 4;
  const int VEC = f32 ? 4 : 8;
  const bool aligned = (reinterpret_cast<uintptr_t>(H) & 15) == 0 && (reinterpret_cast<uintptr_t>(r) & 15) == 0;
  if (G == 1 && aligned && hidden % (64 * VEC) == 0 && hidden / (64 * VEC) <= 8) {
    const int nv = hidden / (64 * VEC);
    dim3 g1(unsigned((tokens + wpb * kTok - 1) / (wpb * kTok)));
#define SWI_ROUTE_G1(NVV)                                                                         \
  case NVV:                                                                                       \
    if (f32)                                                                                      \
      hipLaunchKernelGGL((route_g1_kernel<float, NVV>), g1, dim3(64 * wpb), 0, s,                 \
                         static_cast<const float*>(H), static_cast<const float*>(r), bias, gate,  \
                         z_out, tokens, hidden);                                                  \
    else                                                                                          \
      hipLaunchKernelGGL((route_g1_kernel<bf16_t, NVV>), g1, dim3(64 * wpb), 0, s,                \
                         static_cast<const bf16_t*>(H), static_cast<const bf16_t*>(r), bias,      \
                         gate, z_out, tokens, hidden);                                            \
    return hipGetLastError();
    switch (nv) {
      SWI_ROUTE_G1(1)
      SWI_ROUTE_G1(2)
      SWI_ROUTE_G1(3)
      SWI_ROUTE_G1(4)
      SWI_ROUTE_G1(5)
      SWI_ROUTE_G1(6)
      SWI_ROUTE_G1(7)
      SWI_ROUTE_G1(8)
      default: break;
    }
#undef SWI_ROUTE_G1
  }
  dim3 grid(unsigned((tokens + wpb - 1) / wpb));
  if (f32)
    hipLaunchKernelGGL(route_kernel<float>, grid, dim3(64 * wpb), 0, s,
                       static_cast<const float*>(H), static_cast<const float*>(r), bias, gate,
                       z_out, tokens, hidden, G);
  else
    hipLaunchKernelGGL(route_kernel<bf16_t>, grid, dim3(64 * wpb), 0, s,
                       static_cast<const bf16_t*>(H), static_cast<const bf16_t*>(r), bias,
                       gate, z_out, tokens, hidden, G);
  return hipGetLastError();
}

hipError_t launch_compact(const uint8_t* gate, int32_t* idx, int32_t* cnt, int B, int N, int G,
                          hipStream_t s) {
  hipLaunchKernelGGL(compact_kernel, dim3(unsigned(B * G)), dim3(kCompactThreads), 0, s, gate,
                     idx, cnt, N, G);
  return hipGetLastError();
}

}  // namespace swi
