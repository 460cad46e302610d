// Attention backward of the hard-gated SwiAttn prefill.
//
// SwiAttn report, section 2: O = sigma * O_FULL + (1 - sigma) * O_SWA with a
// 0/1 forward gate, so row i of a head in gate group g is one softmax
// attention over its key set S_i = [0, i] (gate 1) or [max(0, i-W+1), i]
// (gate 0; weimeta SWA glossary, section "详细解释").  For L = sum(dO * O):
//   P_ij = exp(s_ij - LSE_i),  s_ij = scale <q_i, k_j>,  D_i = <dO_i, O_i>
//   dS_ij = P_ij (<dO_i, v_j> - D_i)
//   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
//   dV_j = sum_i P_ij dO_i   (K, V gradients summed over the query heads of
//   a KV head).
//
//   bwd_row_kernel  one wave per (token, query head): pass 1 forms LSE_i over
//                   S_i, pass 2 accumulates dQ_i; LSE_i and D_i go to the
//                   workspace for the column pass
//   bwd_col_kernel  one wave per (key j, KV head), keys fastest: walks the rows that see
//                   key j (the window rows j .. j+W-1 of every gate, then the
//                   gate=1 rows past the window from the compacted list) for
//                   each query head of the KV head and accumulates dK_j, dV_j
// A lane holds d/64 channels; every dot product is a lane product followed
// by the wave's DPP sum, four keys (or rows) at a time.  This is a plain
// VALU implementation (no matrix cores); every sum has a fixed order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "kernels.hpp"

namespace swi {

constexpr int kBwdThreads = 256;  // four waves
constexpr int kBwdGroup = 4;      // keys (rows) per step

struct BwdArgs {
  const void *Q, *K, *V, *O, *dO;
  const uint8_t* gate;
  const int32_t* idx;
  const int32_t* cnt;
  void *dQ, *dK, *dV;
  float* lse2;  // [B,Hq,N] row log-sum-exp, log2 units
  float* Drow;  // [B,Hq,N] <dO_i, O_i>
  int B, N, Hq, Hkv, G, W, HK, HG;
  float sl2;    // scale * log2(e)
  float scale;
};

template <typename T, int CPL>
SWI_DEV void load_ch(const T* p, float (&x)[CPL]) {
#pragma unroll
  for (int e = 0; e < CPL; ++e) x[e] = Elem<T>::load(p + e);
}

template <int CPL>
SWI_DEV float lane_dot(const float (&a)[CPL], const float (&b)[CPL]) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < CPL; ++e) s = fmaf(a[e], b[e], s);
  return s;
}

// Row pass: wave w -> (b, i, h).
template <typename T, int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_row_kernel(BwdArgs a) {
  constexpr int CPL = D / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t nrows = int64_t(a.B) * a.N * a.Hq;
  const int64_t nw = int64_t(gridDim.x) * (kBwdThreads / kWave);
  const T* Qp = static_cast<const T*>(a.Q);
  const T* Kp = static_cast<const T*>(a.K);
  const T* Vp = static_cast<const T*>(a.V);
  const T* Op = static_cast<const T*>(a.O);
  const T* dOp = static_cast<const T*>(a.dO);
  for (int64_t r = int64_t(blockIdx.x) * (kBwdThreads / kWave) + (threadIdx.x >> 6); r < nrows; r += nw) {
    const int h = int(r % a.Hq);
    const int64_t bi = r / a.Hq;  // b * N + i
    const int i = int(bi % a.N), b = int(bi / a.N);
    const int kvh = h / a.HK, g = h / a.HG;
    const bool full = a.gate[bi * a.G + g] != 0;
    const int lo = full ? 0 : max(0, i - a.W + 1);
    const int64_t qoff = (bi * a.Hq + h) * D + lane * CPL;
    const int64_t krow = int64_t(a.Hkv) * D;  // elements between key rows
    const T* kb = Kp + (int64_t(b) * a.N * a.Hkv + kvh) * D + lane * CPL;
    const T* vb = Vp + (int64_t(b) * a.N * a.Hkv + kvh) * D + lane * CPL;
    float q[CPL], go[CPL], o[CPL];
    load_ch<T, CPL>(Qp + qoff, q);
    load_ch<T, CPL>(dOp + qoff, go);
    load_ch<T, CPL>(Op + qoff, o);
    // pass 1: log-sum-exp over the key set (log2 units)
    float m = kNegInf, l = 0.f;
    for (int j0 = lo; j0 <= i; j0 += kBwdGroup) {
      float s[kBwdGroup];
#pragma unroll
      for (int u = 0; u < kBwdGroup; ++u) {
        const int j = min(j0 + u, i);
        float k[CPL];
        load_ch<T, CPL>(kb + int64_t(j) * krow, k);
        s[u] = lane_dot<CPL>(q, k);
      }
#pragma unroll
      for (int u = 0; u < kBwdGroup; ++u) s[u] = j0 + u <= i ? wave_sum(s[u]) * a.sl2 : kNegInf;
      float mb = m;
#pragma unroll
      for (int u = 0; u < kBwdGroup; ++u) mb = fmaxf(mb, s[u]);
      l *= exp2f(m - mb);
#pragma unroll
      for (int u = 0; u < kBwdGroup; ++u) l += exp2f(s[u] - mb);
      m = mb;
    }
    const float lse = m + log2f(l);
    const float Dv = wave_sum(lane_dot<CPL>(go, o));
    // pass 2: dQ
    float dq[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) dq[e] = 0.f;
    for (int j0 = lo; j0 <= i; j0 += kBwdGroup) {
      float s[kBwdGroup], dp[kBwdGroup], k[kBwdGroup][CPL];
#pragma unroll
      for (int u = 0; u < kBwdGroup; ++u) {
        const int j = min(j0 + u, i);
        float v[CPL];
        load_ch<T, CPL>(kb + int64_t(j) * krow, k[u]);
        load_ch<T, CPL>(vb + int64_t(j) * krow, v);
        s[u] = lane_dot<CPL>(q, k[u]);
        dp[u] = lane_dot<CPL>(go, v);
      }
#pragma unroll
      for (int u = 0; u < kBwdGroup; ++u) {
        const float p = j0 + u <= i ? exp2f(wave_sum(s[u]) * a.sl2 - lse) : 0.f;
        const float ds = p * (wave_sum(dp[u]) - Dv);
#pragma unroll
        for (int e = 0; e < CPL; ++e) dq[e] = fmaf(ds, k[u][e], dq[e]);
      }
    }
    T* dqp = static_cast<T*>(a.dQ) + qoff;
#pragma unroll
    for (int e = 0; e < CPL; ++e) Elem<T>::store(dqp + e, dq[e] * a.scale);
    if (lane == 0) {
      const int64_t sidx = (int64_t(b) * a.Hq + h) * a.N + i;
      a.lse2[sidx] = lse;
      a.Drow[sidx] = Dv;
    }
  }
}

// First position >= x in the ascending compacted list of (b, g), as an index.
SWI_DEV int lower_bound_idx(const int32_t* list, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (list[mid] < x)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// Column pass: wave w -> (b, j, kvh).
template <typename T, int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_col_kernel(BwdArgs a) {
  constexpr int CPL = D / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t ncols = int64_t(a.B) * a.N * a.Hkv;
  const int64_t nw = int64_t(gridDim.x) * (kBwdThreads / kWave);
  const T* Qp = static_cast<const T*>(a.Q);
  const T* Kp = static_cast<const T*>(a.K);
  const T* Vp = static_cast<const T*>(a.V);
  const T* dOp = static_cast<const T*>(a.dO);
  for (int64_t c = int64_t(blockIdx.x) * (kBwdThreads / kWave) + (threadIdx.x >> 6); c < ncols; c += nw) {
    // token fastest: the waves of a workgroup (and the workgroups an XCD
    // runs) take neighbouring keys of one KV head, whose rows overlap
    const int j = int(c % a.N);
    const int64_t bk = c / a.N;  // b * Hkv + kvh
    const int kvh = int(bk % a.Hkv), b = int(bk / a.Hkv);
    const int64_t bj = int64_t(b) * a.N + j;
    const int64_t koff = (bj * a.Hkv + kvh) * D + lane * CPL;
    float k[CPL], v[CPL], dk[CPL], dv[CPL];
    load_ch<T, CPL>(Kp + koff, k);
    load_ch<T, CPL>(Vp + koff, v);
#pragma unroll
    for (int e = 0; e < CPL; ++e) dk[e] = dv[e] = 0.f;
    const int64_t qrow = int64_t(a.Hq) * D;  // elements between query rows
    const int wend = int(min<int64_t>(int64_t(a.N) - 1, int64_t(j) + a.W - 1));  // last window row
    for (int hh = 0; hh < a.HK; ++hh) {
      const int h = kvh * a.HK + hh, g = h / a.HG;
      const T* qb = Qp + (int64_t(b) * a.N * a.Hq + h) * D + lane * CPL;
      const T* db = dOp + (int64_t(b) * a.N * a.Hq + h) * D + lane * CPL;
      const float* lrow = a.lse2 + (int64_t(b) * a.Hq + h) * a.N;
      const float* drow = a.Drow + (int64_t(b) * a.Hq + h) * a.N;
      const int32_t* list = a.idx + (int64_t(b) * a.G + g) * a.N;
      const int n = a.cnt[b * a.G + g];
      // rows: window rows j .. wend (any gate), then gate=1 rows > wend
      const int f0 = lower_bound_idx(list, n, wend + 1);
      const int nwin = wend - j + 1, total = nwin + (n - f0);
      for (int t0 = 0; t0 < total; t0 += kBwdGroup) {
        int row[kBwdGroup];
        float s[kBwdGroup], dp[kBwdGroup], qv[kBwdGroup][CPL], gv[kBwdGroup][CPL];
#pragma unroll
        for (int u = 0; u < kBwdGroup; ++u) {
          const int t = min(t0 + u, total - 1);
          row[u] = t < nwin ? j + t : list[f0 + (t - nwin)];
          load_ch<T, CPL>(qb + int64_t(row[u]) * qrow, qv[u]);
          load_ch<T, CPL>(db + int64_t(row[u]) * qrow, gv[u]);
          s[u] = lane_dot<CPL>(qv[u], k);
          dp[u] = lane_dot<CPL>(gv[u], v);
        }
#pragma unroll
        for (int u = 0; u < kBwdGroup; ++u) {
          const bool live = t0 + u < total;
          const float p = live ? exp2f(wave_sum(s[u]) * a.sl2 - lrow[row[u]]) : 0.f;
          const float ds = p * (wave_sum(dp[u]) - drow[row[u]]);
#pragma unroll
          for (int e = 0; e < CPL; ++e) {
            dv[e] = fmaf(p, gv[u][e], dv[e]);
            dk[e] = fmaf(ds, qv[u][e], dk[e]);
          }
        }
      }
    }
    T* dkp = static_cast<T*>(a.dK) + koff;
    T* dvp = static_cast<T*>(a.dV) + koff;
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      Elem<T>::store(dkp + e, dk[e] * a.scale);
      Elem<T>::store(dvp + e, dv[e]);
    }
  }
}

size_t backward_workspace(int B, int N, int Hq) { return size_t(2) * B * Hq * N * sizeof(float); }

template <typename T, int D>
static hipError_t run_backward(BwdArgs& a, hipStream_t s) {
  const int64_t rows = int64_t(a.B) * a.N * a.Hq;
  const int64_t cols = int64_t(a.B) * a.N * a.Hkv;
  const int wpb = kBwdThreads / kWave;
  const int64_t g1 = (rows + wpb - 1) / wpb, g2 = (cols + wpb - 1) / wpb;
  hipLaunchKernelGGL((bwd_row_kernel<T, D>), dim3(unsigned(g1 < 65536 ? g1 : 65536)), dim3(kBwdThreads), 0,
                     s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_col_kernel<T, D>), dim3(unsigned(g2 < 65536 ? g2 : 65536)), dim3(kBwdThreads), 0,
                     s, a);
  return hipGetLastError();
}

hipError_t launch_backward(const void* Q, const void* K, const void* V, const void* O,
                           const void* dO, const uint8_t* gate, const int32_t* idx,
                           const int32_t* cnt, void* dQ, void* dK, void* dV, int B, int N, int Hq,
                           int Hkv, int G, int d, int W, float scale, bool f32, void* ws,
                           hipStream_t s) {
  BwdArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.dO = dO;
  a.gate = gate;
  a.idx = idx;
  a.cnt = cnt;
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.lse2 = static_cast<float*>(ws);
  a.Drow = a.lse2 + size_t(B) * Hq * N;
  a.B = B;
  a.N = N;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.W = W;
  a.HK = Hq / Hkv;
  a.HG = Hq / G;
  a.sl2 = scale * kLog2e;
  a.scale = scale;
  if (f32) {
    if (d == 64) return run_backward<float, 64>(a, s);
    return run_backward<float, 128>(a, s);
  }
  if (d == 64) return run_backward<bf16_t, 64>(a, s);
  return run_backward<bf16_t, 128>(a, s);
}

}  // namespace swi
