// Router gradient through SwiAttn's straight-through gate (one layer).
//
// SwiAttn report, section 2: the hard gate is sigma = 1(soft > 0.5) + soft -
// sg(soft) with soft = sigmoid(z) and z = R(H) = H.r + bias; its forward
// value is the 0/1 decision and its derivative the sigmoid's.  With
// O = sigma * O_FULL + (1 - sigma) * O_SWA the gradient that reaches the
// router is
//   dz[t,g]  = soft'(z) * sum over the heads h of group g and channels c of
//              dO[t,h,c] * (O_FULL - O_SWA)[t,h,c]
//   dH[t,k]  = sum_g dz[t,g] r[k,g]
//   dr[k,g]  = sum_t H[t,k] dz[t,g],   dbias[g] = sum_t dz[t,g]
// (the gradients that reach Q, K, V through the two branch outputs are not
// computed here).
//
//   router_grad_token_kernel   one wave per token: the group sums of
//                              dO * (O_FULL - O_SWA), dz, and the dH row
//   router_grad_weight_kernel  per split of kSplitTokens tokens: partial
//                              sums of H^T dz and of dz
//   router_grad_reduce_kernel  the partials summed: wave w of 16 adds the
//                              splits w, w+16, ... in order, then the wave
//                              sums are added in wave order
// Every reduction has a fixed order (bitwise reproducible).  All passes are
// bound by HBM: the three [tokens, Hq, d] tensors and H are read once, dH is
// written once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "kernels.hpp"

namespace swi {

constexpr int kRgThreads = 256;   // four waves
constexpr int kSplitTokens = 32;  // tokens per partial of the weight and bias sums
constexpr int kRedWaves = 16;     // waves that share one column block of the final sums
constexpr int kRgMaxG = 64;       // gate groups supported (dz of a token lives in LDS)

// Eight consecutive elements as float.
SWI_DEV void load8(const bf16_t* p, float (&x)[8]) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = float(v[j]);
}
SWI_DEV void load8(const float* p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = a[j];
    x[4 + j] = b[j];
  }
}
// The same for data read once: the non-temporal hint keeps the stream out
// of the caches.
SWI_DEV void load8_nt(const bf16_t* p, float (&x)[8]) {
  const bf16x8 v = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = float(v[j]);
}
SWI_DEV void load8_nt(const float* p, float (&x)[8]) {
  const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = a[j];
    x[4 + j] = b[j];
  }
}
SWI_DEV void store8(bf16_t* p, const float (&x)[8]) {
  bf16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = bf16_t(x[j]);
  *reinterpret_cast<bf16x8*>(p) = v;
}
SWI_DEV void store8(float* p, const float (&x)[8]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

// sigmoid'(x) = e^-|x| / (1 + e^-|x|)^2: symmetric, no cancellation in the
// tails (soft * (1 - soft) loses the small factor once soft rounds to 1).
SWI_DEV float sigmoid_grad(float x) {
  const float u = expf(-fabsf(x));
  const float v = 1.f + u;
  return u / (v * v);
}

// PPL > 0: a group has exactly PPL * 64 pieces of 8 elements, so a lane
// issues all 3 PPL of its loads before the first product (one memory round
// trip per token and group); PPL = 0: any size, piece by piece.  Either way
// a lane sums its pieces in the same order.
template <typename T, int PPL>
__global__ __launch_bounds__(kRgThreads) void router_grad_token_kernel(const T* dO, const T* Of,
                                                                       const T* Os, const float* z,
                                                                       const T* r, float* dz, T* dH,
                                                                       int64_t ntok, int row, int hidden,
                                                                       int G) {
  __shared__ float s_dz[kRgThreads / kWave][kRgMaxG];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int64_t nwaves = int64_t(gridDim.x) * (kRgThreads / kWave);
  const int per_group = row / G;      // the heads of a group are contiguous in a row
  const int pieces = per_group / 8;   // 8-element pieces per group
  for (int64_t t = int64_t(blockIdx.x) * (kRgThreads / kWave) + wave; t < ntok; t += nwaves) {
    const int64_t base = t * row;
    for (int g = 0; g < G; ++g) {
      float acc = 0.f;
      if constexpr (PPL > 0) {
        float a[PPL][8], f[PPL][8], w[PPL][8];
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
          const int64_t e = base + int64_t(g) * per_group + int64_t(lane + kWave * k) * 8;
          load8_nt(dO + e, a[k]);
          load8_nt(Of + e, f[k]);
          load8_nt(Os + e, w[k]);
        }
#pragma unroll
        for (int k = 0; k < PPL; ++k)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc = fmaf(a[k][j], f[k][j] - w[k][j], acc);
      } else {
        for (int p = lane; p < pieces; p += kWave) {
          const int64_t e = base + int64_t(g) * per_group + int64_t(p) * 8;
          float a[8], f[8], w[8];
          load8_nt(dO + e, a);
          load8_nt(Of + e, f);
          load8_nt(Os + e, w);
#pragma unroll
          for (int j = 0; j < 8; ++j) acc = fmaf(a[j], f[j] - w[j], acc);
        }
      }
      const float sgrp = wave_sum(acc);
      const float v = sgrp * sigmoid_grad(z[t * G + g]);
      if (lane == 0) {
        dz[t * G + g] = v;
        s_dz[wave][g] = v;
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    // dH row: 8 consecutive hidden units per lane and step (hidden % 8 == 0);
    // with one group the 8 weights are one 16-byte piece of r
    for (int p = lane; p < hidden / 8; p += kWave) {
      float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (G == 1) {
        float rr[8];
        load8(r + int64_t(p) * 8, rr);
        const float v = s_dz[wave][0];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = fmaf(v, rr[j], o[j]);
      } else {
        for (int g = 0; g < G; ++g) {
          const float v = s_dz[wave][g];
#pragma unroll
          for (int j = 0; j < 8; ++j) o[j] = fmaf(v, Elem<T>::load(r + int64_t(p * 8 + j) * G + g), o[j]);
        }
      }
      store8(dH + t * hidden + int64_t(p) * 8, o);
    }
    __builtin_amdgcn_wave_barrier();  // s_dz is rewritten for the wave's next token
  }
}

// Partial sums over the tokens of split s (blockIdx.x) for 8 hidden units per
// thread (blockIdx.y picks the column block): part[(s*G + g)*(hidden+1) + k]
// = sum_t H[t,k] dz[t,g], and at column `hidden` the sum of dz[t,g].
template <typename T>
__global__ __launch_bounds__(kRgThreads) void router_grad_weight_kernel(const T* H, const float* dz,
                                                                        float* part, int64_t ntok,
                                                                        int hidden, int G) {
  const int64_t t0 = int64_t(blockIdx.x) * kSplitTokens;
  const int64_t t1 = t0 + kSplitTokens < ntok ? t0 + kSplitTokens : ntok;
  const int k0 = (blockIdx.y * kRgThreads + threadIdx.x) * 8;
  const int64_t stride = int64_t(hidden) + 1;
  const bool cols = k0 < hidden;  // hidden % 8 == 0: a thread's 8 columns are all in range or none
  for (int g = 0; g < G; ++g) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float accb = 0.f;
#pragma unroll 8
    for (int64_t t = t0; t < t1; ++t) {
      const float w = dz[t * G + g];
      accb += w;
      if (cols) {
        float h[8];
        load8_nt(H + t * hidden + k0, h);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(w, h[j], acc[j]);
      }
    }
    float* out = part + (int64_t(blockIdx.x) * G + g) * stride;
    if (cols) {
#pragma unroll
      for (int j = 0; j < 8; ++j) out[k0 + j] = acc[j];
    }
    if (blockIdx.y == 0 && threadIdx.x == 0) out[hidden] = accb;
  }
}

// dr[k,g] and dbias[g]: one workgroup per 64 outputs (lane = output); wave
// w sums the splits w, w + kRedWaves, ... in order, then the wave partials
// are added in wave order.
__global__ __launch_bounds__(kRedWaves * kWave) void router_grad_reduce_kernel(const float* part, float* dr,
                                                                               float* dbias, int splits,
                                                                               int hidden, int G) {
  __shared__ float s_part[kRedWaves][kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int64_t stride = int64_t(hidden) + 1;
  const int64_t i = int64_t(blockIdx.x) * kWave + lane;  // over G * (hidden + 1)
  const bool live = i < int64_t(G) * stride;
  const int g = live ? int(i / stride) : 0;
  const int k = live ? int(i - int64_t(g) * stride) : 0;
  float s = 0.f;
  if (live) {
#pragma unroll 8
    for (int sp = wave; sp < splits; sp += kRedWaves) s += part[(int64_t(sp) * G + g) * stride + k];
  }
  s_part[wave][lane] = s;
  __syncthreads();
  if (wave != 0 || !live) return;
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kRedWaves; ++w) tot += s_part[w][lane];
  if (k < hidden)
    dr[int64_t(k) * G + g] = tot;
  else
    dbias[g] = tot;
}

size_t router_grad_workspace(int64_t ntok, int hidden, int G) {
  const int64_t splits = (ntok + kSplitTokens - 1) / kSplitTokens;
  return size_t(splits) * G * (size_t(hidden) + 1) * sizeof(float);
}

int router_grad_max_groups() { return kRgMaxG; }

template <typename T>
static hipError_t run_router_grad(const T* dO, const T* Of, const T* Os, const float* z, const T* H,
                                  const T* r, float* dz, T* dH, float* dr, float* dbias, int64_t ntok,
                                  int row, int hidden, int G, float* part, hipStream_t s) {
  const int64_t waves = ntok;
  const int64_t want = (waves + (kRgThreads / kWave) - 1) / (kRgThreads / kWave);
  const int grid = int(want < 8192 ? want : 8192);
  const int pieces = row / G / 8;
  if (pieces == 4 * kWave)
    hipLaunchKernelGGL((router_grad_token_kernel<T, 4>), dim3(grid), dim3(kRgThreads), 0, s, dO, Of, Os, z,
                       r, dz, dH, ntok, row, hidden, G);
  else if (pieces == 2 * kWave)
    hipLaunchKernelGGL((router_grad_token_kernel<T, 2>), dim3(grid), dim3(kRgThreads), 0, s, dO, Of, Os, z,
                       r, dz, dH, ntok, row, hidden, G);
  else
    hipLaunchKernelGGL((router_grad_token_kernel<T, 0>), dim3(grid), dim3(kRgThreads), 0, s, dO, Of, Os, z,
                       r, dz, dH, ntok, row, hidden, G);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t splits = (ntok + kSplitTokens - 1) / kSplitTokens;
  const int ycols = (hidden + kRgThreads * 8 - 1) / (kRgThreads * 8);
  hipLaunchKernelGGL((router_grad_weight_kernel<T>), dim3(unsigned(splits), unsigned(ycols)),
                     dim3(kRgThreads), 0, s, H, dz, part, ntok, hidden, G);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t outs = int64_t(G) * (int64_t(hidden) + 1);
  hipLaunchKernelGGL(router_grad_reduce_kernel, dim3(unsigned((outs + kWave - 1) / kWave)),
                     dim3(kRedWaves * kWave), 0, s, part, dr, dbias, int(splits), hidden, G);
  return hipGetLastError();
}

hipError_t launch_router_grad(const void* dO, const void* Of, const void* Os, const float* z,
                              const void* H, const void* r, float* dz, void* dH, float* dr,
                              float* dbias, int B, int N, int Hq, int d, int hidden, int G, bool f32,
                              void* ws, hipStream_t s) {
  const int64_t ntok = int64_t(B) * N;
  const int row = Hq * d;
  float* part = static_cast<float*>(ws);
  if (f32)
    return run_router_grad<float>(static_cast<const float*>(dO), static_cast<const float*>(Of),
                                  static_cast<const float*>(Os), z, static_cast<const float*>(H),
                                  static_cast<const float*>(r), dz, static_cast<float*>(dH), dr, dbias,
                                  ntok, row, hidden, G, part, s);
  return run_router_grad<bf16_t>(static_cast<const bf16_t*>(dO), static_cast<const bf16_t*>(Of),
                                 static_cast<const bf16_t*>(Os), z, static_cast<const bf16_t*>(H),
                                 static_cast<const bf16_t*>(r), dz, static_cast<bf16_t*>(dH), dr, dbias,
                                 ntok, row, hidden, G, part, s);
}

}  // namespace swi
