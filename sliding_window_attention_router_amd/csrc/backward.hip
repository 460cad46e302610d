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
//   bwd_row_kernel  one 16-lane group per (token, query head): one online
//                   pass over S_i accumulates dQ_i and LSE_i (running
//                   maximum, rescaled sums); LSE_i and D_i go to the
//                   workspace for the column pass.  Two launches: the
//                   gate=0 rows in token order, the gate=1 rows gathered
//                   (neighbouring routed tokens share their keys)
//   bwd_col_kernel  one 16-lane group per (key j, KV head), keys fastest:
//                   walks the rows that see key j (the window rows j ..
//                   j+W-1 of every gate, then the gate=1 rows past the
//                   window from the compacted list) for each query head of
//                   the KV head and accumulates dK_j, dV_j
// A wave holds four groups of 16 lanes (one row or key each, d/16 channels
// per lane); a dot product is a lane product plus the 16-lane DPP row sum,
// four keys (or rows) at a time.  This is a plain vector-ALU implementation
// (no matrix cores); every sum has a fixed order.
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

constexpr int kGL = 16;               // lanes per group (one row or key each)
constexpr int kGroups = kWave / kGL;  // groups per wave

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

// Sum over the 16 lanes of a DPP row (quads, half-rows, rows); each step
// adds two equal-shaped partial sums, so all 16 lanes end with the same bits.
SWI_DEV float row16_sum(float v) {
  int x = __float_as_int(v);
  const auto add = [](int p, int q) { return __float_as_int(__int_as_float(p) + __int_as_float(q)); };
  x = add(x, dpp_src<0xB1>(x, 0));   // quad_perm [1,0,3,2]
  x = add(x, dpp_src<0x4E>(x, 0));   // quad_perm [2,3,0,1]
  x = add(x, dpp_src<0x141>(x, 0));  // row_half_mirror
  x = add(x, dpp_src<0x140>(x, 0));  // row_mirror
  return __int_as_float(x);
}

// Row pass, in two launches.  kFar = false: group grp of wave w -> item
// r = 4w + grp of the (b, i, h) order (heads fastest: the groups of a wave
// are the heads of one token); rows whose gate is 1 are left to the other
// launch.  kFar = true: item r of the (b, h, t) order with t fastest is the
// t-th gate=1 token of head h's gate group (from the compacted list), so
// the groups of a workgroup are 16 neighbouring routed tokens of one head,
// which walk the same keys [0, i] together.  The wave walks the union of its
// groups' key ranges; each group masks its own.
template <typename T, int D, bool kFar>
__global__ __launch_bounds__(kBwdThreads) void bwd_row_kernel(BwdArgs a) {
  constexpr int CPL = D / kGL;
  const int lane = threadIdx.x & (kWave - 1), grp = lane / kGL, gl = lane % kGL;
  const int64_t nrows = int64_t(a.B) * a.N * a.Hq;
  const int64_t nw = int64_t(gridDim.x) * (kBwdThreads / kWave);
  const T* Qp = static_cast<const T*>(a.Q);
  const T* Kp = static_cast<const T*>(a.K);
  const T* Vp = static_cast<const T*>(a.V);
  const T* Op = static_cast<const T*>(a.O);
  const T* dOp = static_cast<const T*>(a.dO);
  for (int64_t w = int64_t(blockIdx.x) * (kBwdThreads / kWave) + (threadIdx.x >> 6); w * kGroups < nrows;
       w += nw) {
    const int64_t r = w * kGroups + grp;
    bool act = r < nrows;
    const int64_t rr = act ? r : nrows - 1;
    int h, i, b;
    if constexpr (kFar) {
      const int t = int(rr % a.N);
      const int64_t bh = rr / a.N;  // b * Hq + h
      h = int(bh % a.Hq);
      b = int(bh / a.Hq);
      const int gg = h / a.HG;
      const int n = a.cnt[b * a.G + gg];
      act = act && t < n;
      i = a.idx[(int64_t(b) * a.G + gg) * a.N + (t < n ? t : 0)];
      if (!act) i = 0;
    } else {
      h = int(rr % a.Hq);
      const int64_t bi0 = rr / a.Hq;  // b * N + i
      i = int(bi0 % a.N);
      b = int(bi0 / a.N);
    }
    const int64_t bi = int64_t(b) * a.N + i;
    const int kvh = h / a.HK, g = h / a.HG;
    const bool full = a.gate[bi * a.G + g] != 0;
    if constexpr (!kFar) act = act && !full;  // gate=1 rows: the other launch
    const int lo = full ? 0 : max(0, i - a.W + 1);
    const int64_t qoff = (bi * a.Hq + h) * D + gl * CPL;
    const int64_t krow = int64_t(a.Hkv) * D;  // elements between key rows
    const T* kb = Kp + (int64_t(b) * a.N * a.Hkv + kvh) * D + gl * CPL;
    const T* vb = Vp + (int64_t(b) * a.N * a.Hkv + kvh) * D + gl * CPL;
    float q[CPL], go[CPL], o[CPL];
    load_ch<T, CPL>(Qp + qoff, q);
    load_ch<T, CPL>(dOp + qoff, go);
    load_ch<T, CPL>(Op + qoff, o);
    const int jlo = wave_min_i(act ? lo : INT_MAX), jhi = wave_max_i(act ? i : -1);
    // one online pass: with m the running maximum of the scores (log2
    // units), l = sum 2^(s - m) and dq = sum 2^(s - m) (dP - D) k; when m
    // rises both are rescaled.  D = <dO, O> is known before the pass, so
    // dQ = dq / l and LSE = m + log2(l) at the end.
    const float Dv = row16_sum(lane_dot<CPL>(go, o));
    float m = kNegInf, l = 0.f, dq[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) dq[e] = 0.f;
    for (int j0 = jlo; j0 <= jhi; j0 += kBwdGroup) {
      float s[kBwdGroup], dp[kBwdGroup], k[kBwdGroup][CPL];
#pragma unroll
      for (int u = 0; u < kBwdGroup; ++u) {
        const int j = min(j0 + u, jhi);
        float v[CPL];
        load_ch<T, CPL>(kb + int64_t(j) * krow, k[u]);
        load_ch<T, CPL>(vb + int64_t(j) * krow, v);
        s[u] = lane_dot<CPL>(q, k[u]);
        dp[u] = lane_dot<CPL>(go, v);
      }
      float mb = m;
#pragma unroll
      for (int u = 0; u < kBwdGroup; ++u) {
        const int j = j0 + u;
        const bool in = act && j <= jhi && j >= lo && j <= i;
        s[u] = in ? row16_sum(s[u]) * a.sl2 : kNegInf;
        dp[u] = row16_sum(dp[u]);
        mb = fmaxf(mb, s[u]);
      }
      if (mb == kNegInf) continue;  // no key of this group in the step (group-uniform)
      const float sc = exp2f(m - mb);  // 0 while m is -inf
      l *= sc;
#pragma unroll
      for (int e = 0; e < CPL; ++e) dq[e] *= sc;
#pragma unroll
      for (int u = 0; u < kBwdGroup; ++u) {
        const float p = exp2f(s[u] - mb);
        l += p;
        const float ds = p * (dp[u] - Dv);
#pragma unroll
        for (int e = 0; e < CPL; ++e) dq[e] = fmaf(ds, k[u][e], dq[e]);
      }
      m = mb;
    }
    const float lse = m + log2f(l);
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) dq[e] *= inv;
    if (act) {
      T* dqp = static_cast<T*>(a.dQ) + qoff;
#pragma unroll
      for (int e = 0; e < CPL; ++e) Elem<T>::store(dqp + e, dq[e] * a.scale);
      if (gl == 0) {
        const int64_t sidx = (int64_t(b) * a.Hq + h) * a.N + i;
        a.lse2[sidx] = lse;
        a.Drow[sidx] = Dv;
      }
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

// Column pass: group grp of wave w -> item c = 4w + grp of the (b, kvh, j)
// order (keys fastest: the groups of a wave are four neighbouring keys of
// one KV head, and neighbouring waves share their rows in cache).  For each
// query head of the KV head the wave walks the union of its groups' window
// rows (a row sees key j if i >= j and (i <= j+W-1 or its gate is 1)), then
// the gate=1 rows past that union from the compacted list.
template <typename T, int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_col_kernel(BwdArgs a) {
  constexpr int CPL = D / kGL;
  const int lane = threadIdx.x & (kWave - 1), grp = lane / kGL, gl = lane % kGL;
  const int64_t ncols = int64_t(a.B) * a.N * a.Hkv;
  const int64_t nw = int64_t(gridDim.x) * (kBwdThreads / kWave);
  const T* Qp = static_cast<const T*>(a.Q);
  const T* Kp = static_cast<const T*>(a.K);
  const T* Vp = static_cast<const T*>(a.V);
  const T* dOp = static_cast<const T*>(a.dO);
  for (int64_t w = int64_t(blockIdx.x) * (kBwdThreads / kWave) + (threadIdx.x >> 6); w * kGroups < ncols;
       w += nw) {
    const int64_t c = w * kGroups + grp;
    const bool act = c < ncols;
    const int64_t cc = act ? c : ncols - 1;
    const int j = int(cc % a.N);
    const int64_t bk = cc / a.N;  // b * Hkv + kvh
    const int kvh = int(bk % a.Hkv), b = int(bk / a.Hkv);
    const int64_t koff = ((int64_t(b) * a.N + j) * a.Hkv + kvh) * D + gl * CPL;
    float k[CPL], v[CPL], dk[CPL], dv[CPL];
    load_ch<T, CPL>(Kp + koff, k);
    load_ch<T, CPL>(Vp + koff, v);
#pragma unroll
    for (int e = 0; e < CPL; ++e) dk[e] = dv[e] = 0.f;
    const int64_t qrow = int64_t(a.Hq) * D;  // elements between query rows
    const int wend = int(min<int64_t>(int64_t(a.N) - 1, int64_t(j) + a.W - 1));  // last window row
    const int ilo = wave_min_i(act ? j : INT_MAX), ihi = wave_max_i(act ? wend : -1);
    for (int hh = 0; hh < a.HK; ++hh) {
      const int h = kvh * a.HK + hh, g = h / a.HG;
      const T* qb = Qp + (int64_t(b) * a.N * a.Hq + h) * D + gl * CPL;
      const T* db = dOp + (int64_t(b) * a.N * a.Hq + h) * D + gl * CPL;
      const float* lrow = a.lse2 + (int64_t(b) * a.Hq + h) * a.N;
      const float* drow = a.Drow + (int64_t(b) * a.Hq + h) * a.N;
      const uint8_t* grow = a.gate + int64_t(b) * a.N * a.G + g;
      const int32_t* list = a.idx + (int64_t(b) * a.G + g) * a.N;
      const int n = a.cnt[b * a.G + g];
      const auto visit = [&](const int (&row)[kBwdGroup], const bool (&sees)[kBwdGroup]) {
        float s[kBwdGroup], dp[kBwdGroup], qv[kBwdGroup][CPL], gv[kBwdGroup][CPL];
#pragma unroll
        for (int u = 0; u < kBwdGroup; ++u) {
          load_ch<T, CPL>(qb + int64_t(row[u]) * qrow, qv[u]);
          load_ch<T, CPL>(db + int64_t(row[u]) * qrow, gv[u]);
          s[u] = lane_dot<CPL>(qv[u], k);
          dp[u] = lane_dot<CPL>(gv[u], v);
        }
#pragma unroll
        for (int u = 0; u < kBwdGroup; ++u) {
          const float sv = row16_sum(s[u]), dpv = row16_sum(dp[u]);
          const float p = sees[u] ? exp2f(sv * a.sl2 - lrow[row[u]]) : 0.f;
          const float ds = p * (dpv - drow[row[u]]);
#pragma unroll
          for (int e = 0; e < CPL; ++e) {
            dv[e] = fmaf(p, gv[u][e], dv[e]);
            dk[e] = fmaf(ds, qv[u][e], dk[e]);
          }
        }
      };
      // the union of the groups' window rows
      for (int i0 = ilo; i0 <= ihi; i0 += kBwdGroup) {
        int row[kBwdGroup];
        bool sees[kBwdGroup];
#pragma unroll
        for (int u = 0; u < kBwdGroup; ++u) {
          const int i = i0 + u;
          row[u] = min(i, ihi);
          sees[u] = act && i <= ihi && i >= j && (i <= wend || grow[int64_t(row[u]) * a.G] != 0);
        }
        visit(row, sees);
      }
      // gate=1 rows past the union
      const int f0 = lower_bound_idx(list, n, ihi + 1);
      const int cnt_g = act ? n - f0 : 0;
      const int tmax = wave_max_i(cnt_g);
      for (int t0 = 0; t0 < tmax; t0 += kBwdGroup) {
        int row[kBwdGroup];
        bool sees[kBwdGroup];
#pragma unroll
        for (int u = 0; u < kBwdGroup; ++u) {
          const int t = t0 + u;
          sees[u] = t < cnt_g;
          row[u] = cnt_g > 0 ? list[f0 + min(t, cnt_g - 1)] : j;
        }
        visit(row, sees);
      }
    }
    if (act) {
      T* dkp = static_cast<T*>(a.dK) + koff;
      T* dvp = static_cast<T*>(a.dV) + koff;
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        Elem<T>::store(dkp + e, dk[e] * a.scale);
        Elem<T>::store(dvp + e, dv[e]);
      }
    }
  }
}

size_t backward_workspace(int B, int N, int Hq) { return size_t(2) * B * Hq * N * sizeof(float); }

template <typename T, int D>
static hipError_t run_backward(BwdArgs& a, hipStream_t s) {
  const int64_t rows = int64_t(a.B) * a.N * a.Hq;
  const int64_t cols = int64_t(a.B) * a.N * a.Hkv;
  const int per_wg = (kBwdThreads / kWave) * kGroups;  // items per workgroup
  const int64_t g1 = (rows + per_wg - 1) / per_wg, g2 = (cols + per_wg - 1) / per_wg;
  hipLaunchKernelGGL((bwd_row_kernel<T, D, false>), dim3(unsigned(g1 < 65536 ? g1 : 65536)),
                     dim3(kBwdThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_row_kernel<T, D, true>), dim3(unsigned(g1 < 65536 ? g1 : 65536)),
                     dim3(kBwdThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
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
