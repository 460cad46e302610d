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
// bfloat16, on the matrix cores (three launches):
//   bwd_q_mfma_kernel   a workgroup per 128 query rows of a head: one online
//                       pass over 64-key blocks gives dQ, LSE and D (the
//                       latter two go to the workspace); launched for the
//                       gate=0 rows in token order and for the gate=1 rows
//                       gathered from the compacted list
//   bwd_kv_mfma_kernel  a workgroup per 128 keys of a KV head walks 64-row
//                       tiles of the rows that see them (window rows of every
//                       gate, then gathered gate=1 rows) for each query head
//                       and accumulates dK, dV
// float32, on the vector ALU (three launches):
//   bwd_row_kernel  one 16-lane group per (token, query head): one online
//                   pass over S_i gives dQ_i, LSE_i and D_i; launched for
//                   the gate=0 rows in token order and for the gate=1 rows
//                   gathered (neighbouring routed tokens share their keys)
//   bwd_col_kernel  one 16-lane group per (key j, KV head), keys fastest:
//                   walks the rows that see key j (the window rows j ..
//                   j+W-1 of every gate, then the gate=1 rows past the
//                   window from the compacted list) for each query head of
//                   the KV head and accumulates dK_j, dV_j
// In the vector-ALU kernels a wave holds four groups of 16 lanes (one row
// or key each, d/16 channels per lane); a dot product is a lane product
// plus the 16-lane DPP row sum, four keys (or rows) at a time.  In every
// kernel each sum has a fixed order and no atomics are used, so two runs
// give the same bits.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// ---------------------------------------------------------------------------
// dK, dV on the matrix cores (bfloat16).  A workgroup owns kKvKeys keys of
// one KV head, 32 per wave; each wave keeps its keys' K and V rows in
// registers as MFMA B operands.  For every query head of the KV head the
// workgroup walks tiles of kRT query rows: first the window rows
// [k0, min(N, k0 + kKvKeys - 1 + W)) (any gate; masked per pair), then the
// gate=1 rows past them, gathered from the compacted list.  The four waves
// share each tile: Q and dO rows are staged once in LDS (double-buffered,
// one barrier per tile) with each row's LSE, D and visible key range.
//   S  = Q K^T,  dP = dO V^T         (per 32-row half: 32 rows x 32 keys,
//                                      k = channels)
//   P  = 2^(S sl2 - LSE) on visible pairs,  dS = P (dP - D)
//   dV^T += dO^T P,  dK^T += Q^T dS  (channels x 32 keys, k = rows)
// The 32x32 accumulator of S gives lane l the key l % 32 and rows
// 8(i/4) + 4(l/32) + i%4; those are exactly the contraction slots a B
// operand of the second products holds (rows permuted the same way on the
// A side), so P and dS feed the next MFMAs from registers, and the
// transposed A operands (dO^T, Q^T) come from ds_read_b64_tr_b16: within 16
// lanes, source lane 4r + k points at row r, channels c0 + 4k .. c0 + 4k + 3,
// and lane i receives channel c0 + i of rows 0..3.
// LDS rows are XOR-swizzled by 16-byte chunk so that both the plain 16-byte
// reads (16 lanes, 16 consecutive rows, one chunk) and the transposing
// reads (32 lanes, 4 rows x 4 chunks) hit distinct banks.
// ---------------------------------------------------------------------------
constexpr int kKvKeys = 128;  // keys per workgroup (4 waves x 32)
constexpr int kRT = 64;       // query rows per tile (a multiple of 32)

template <int D>
struct KvTile {
  static constexpr int kRowB = 2 * D;
  static constexpr int kMat = kRT * kRowB;           // one staged matrix (Q or dO)
  static constexpr int kInfo = 2 * kMat;             // lse2, D, first key, last key: [4][kRT]
  static constexpr int kBytes = kInfo + 4 * kRT * 4;
  static constexpr int kCPR = D / 8;                 // 16-byte chunks per row
  static constexpr int kPer = kRT * kCPR / kBwdThreads;  // chunks per thread and matrix
  static_assert(kPer >= 1 && kRT * kCPR % kBwdThreads == 0, "tile staging");
  SWI_DEV static constexpr int swz(int row) {
    return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
  }
  SWI_DEV static constexpr int pos(int row, int chunk) { return row * kRowB + ((chunk ^ swz(row)) << 4); }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

SWI_DEV s16x4 lds_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_kv_mfma_kernel(BwdArgs a) {
  using L = KvTile<D>;
  constexpr int KS = D / 16;  // k-steps of the channel contractions
  constexpr int MD = D / 32;  // 32-channel tiles of dK^T, dV^T
  __shared__ __attribute__((aligned(16))) char lds[2][L::kBytes];
  __shared__ int rowbuf[2][kRT];  // query row of each slot of the next tiles (-1: padding)
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int rl = lane & 31, hf = lane >> 5;
  const int nbk = a.B * a.Hkv;
  const int kblk = blockIdx.x / nbk, bk = blockIdx.x % nbk;  // heaviest key blocks first
  const int b = bk / a.Hkv, kvh = bk % a.Hkv;
  const int k0 = kblk * kKvKeys;
  const int j = k0 + wave * 32 + rl;  // this lane's key
  const int jc = min(j, a.N - 1);
  const bf16_t* Qp = static_cast<const bf16_t*>(a.Q);
  const bf16_t* dOp = static_cast<const bf16_t*>(a.dO);
  bf16x8 kreg[KS], vreg[KS];
  {
    const int64_t off = ((int64_t(b) * a.N + jc) * a.Hkv + kvh) * D + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kreg[ks] = *reinterpret_cast<const bf16x8*>(static_cast<const bf16_t*>(a.K) + off + 16 * ks);
      vreg[ks] = *reinterpret_cast<const bf16x8*>(static_cast<const bf16_t*>(a.V) + off + 16 * ks);
    }
  }
  f32x16 dk[MD], dv[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) dk[md] = dv[md] = f32x16{};
  const int wend = int(min<int64_t>(a.N, int64_t(k0) + kKvKeys - 1 + a.W));  // window rows end here
  const int nwt = (wend - k0 + kRT - 1) / kRT;
  const int64_t qrs = int64_t(a.Hq) * D;  // elements between query rows
  // transposing-read lane roles: row r of a 4-row group, channel quad kq,
  // 16-channel half c16 of a 32-channel tile
  const int tr_r = (lane >> 2) & 3, tr_kq = lane & 3, tr_c16 = (lane >> 4) & 1;
  for (int hh = 0; hh < a.HK; ++hh) {
    const int h = kvh * a.HK + hh, g = h / a.HG;
    const int32_t* list = a.idx + (int64_t(b) * a.G + g) * a.N;
    const int n = a.cnt[b * a.G + g];
    const int f0 = lower_bound_idx(list, n, wend);
    const int nt = nwt + (n - f0 + kRT - 1) / kRT;
    const bf16_t* qh = Qp + int64_t(b) * a.N * qrs + int64_t(h) * D;
    const bf16_t* dh = dOp + int64_t(b) * a.N * qrs + int64_t(h) * D;
    const float* lrow = a.lse2 + (int64_t(b) * a.Hq + h) * a.N;
    const float* drow = a.Drow + (int64_t(b) * a.Hq + h) * a.N;
    const uint8_t* grow = a.gate + int64_t(b) * a.N * a.G + g;
    // Row indices run one tile ahead of the row loads: the gathered rows of
    // tile t + 2 are looked up in the list while tile t is computed and kept
    // in LDS (rowbuf), so the loads of a tile never wait on a list lookup.
    // Every load is unconditional (clamped to a valid row) and consumed in
    // the iteration that issues it; padding slots are zeroed when the tile
    // is written to LDS.
    // (branch-free: the list is read for window tiles too, at a clamped
    // index, so the looked-up value is never merged with another one while
    // its load is in flight)
    int fw = 0, fl = 0;
    bool fok = false, fwin = true;
    const auto fetch_row = [&](int t) {  // slot tid % kRT of tile t
      const int m = tid % kRT;
      const int q = f0 + (t - nwt) * kRT + m;
      fl = list[min(max(q, 0), max(n - 1, 0))];
      fw = k0 + t * kRT + m;
      fwin = t < nwt;
      fok = fwin ? fw < wend : q < n;
    };
    const auto put_row = [&](int* rb) {
      if (tid < kRT) rb[tid] = fok ? (fwin ? fw : fl) : -1;
    };
    u32x4 sq[L::kPer], sd[L::kPer];
    bool sok[L::kPer + 1];
    float s_l = 0.f, s_d = 0.f;
    int s_row = 0;
    uint8_t s_g = 0;
    const auto load_tile = [&](const int* rb) {
#pragma unroll
      for (int p = 0; p < L::kPer; ++p) {
        const int u = tid + p * kBwdThreads, m = u / L::kCPR, c = u % L::kCPR;
        const int r = rb[m];
        sok[p] = r >= 0;
        const int rc = r >= 0 ? r : 0;
        sq[p] = *reinterpret_cast<const u32x4*>(qh + int64_t(rc) * qrs + 8 * c);
        sd[p] = *reinterpret_cast<const u32x4*>(dh + int64_t(rc) * qrs + 8 * c);
      }
      const int r = rb[tid % kRT];
      sok[L::kPer] = r >= 0;
      s_row = r >= 0 ? r : 0;
      s_l = lrow[s_row];
      s_d = drow[s_row];
      s_g = grow[int64_t(s_row) * a.G];
    };
    const auto store_tile = [&](char* buf) {
      const u32x4 z = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int p = 0; p < L::kPer; ++p) {
        const int u = tid + p * kBwdThreads, m = u / L::kCPR, c = u % L::kCPR;
        *reinterpret_cast<u32x4*>(buf + L::pos(m, c)) = sok[p] ? sq[p] : z;
        *reinterpret_cast<u32x4*>(buf + L::kMat + L::pos(m, c)) = sok[p] ? sd[p] : z;
      }
      if (tid < kRT) {
        const bool ok = sok[L::kPer];
        float* info = reinterpret_cast<float*>(buf + L::kInfo);
        info[tid] = ok ? s_l : __builtin_huge_valf();
        info[kRT + tid] = ok ? s_d : 0.f;
        reinterpret_cast<int*>(info)[2 * kRT + tid] = ok ? (s_g != 0 ? 0 : s_row - a.W + 1) : 0;
        reinterpret_cast<int*>(info)[3 * kRT + tid] = ok ? s_row : -1;
      }
    };
    // rows of tiles 0 and 1, then tile 0 itself
    fetch_row(0);
    put_row(rowbuf[0]);
    if (nt > 1) {
      fetch_row(1);
      put_row(rowbuf[1]);
    }
    __syncthreads();
    load_tile(rowbuf[0]);
    store_tile(lds[0]);
    __syncthreads();
    // iteration t: tile t is in LDS buffer t % 2 and the rows of tile t + 1
    // in rowbuf[(t + 1) % 2]; the rows of tile t + 2 are looked up and tile
    // t + 1 is loaded while tile t is computed; one barrier per tile
    for (int t = 0; t < nt; ++t) {
      const bool more = t + 1 < nt;
      if (t + 2 < nt) fetch_row(t + 2);
      if (more) load_tile(rowbuf[(t + 1) & 1]);
      const char* qt = lds[t & 1];
      const char* dt = qt + L::kMat;
      constexpr int RH = kRT / 32;  // 32-row halves of the tile
      f32x16 s[RH], dp[RH];
#pragma unroll
      for (int rh = 0; rh < RH; ++rh) {
        s[rh] = dp[rh] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(qt + L::pos(32 * rh + rl, 2 * ks + hf));
          const bf16x8 ad = *reinterpret_cast<const bf16x8*>(dt + L::pos(32 * rh + rl, 2 * ks + hf));
          s[rh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kreg[ks], s[rh], 0, 0, 0);
          dp[rh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, vreg[ks], dp[rh], 0, 0, 0);
        }
      }
      // P and dS for rows 32rh + 8q + 4hf + e (slot 4q + e of half rh); the
      // 16-row k-step st = 2rh + (slot / 8) of the second products
      const float* info = reinterpret_cast<const float*>(qt + L::kInfo);
      bf16x8 pb[2 * RH], sb[2 * RH];
#pragma unroll
      for (int rh = 0; rh < RH; ++rh)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m0 = 32 * rh + 8 * q + 4 * hf;
          const f32x4 lv = *reinterpret_cast<const f32x4*>(info + m0);
          const f32x4 dv4 = *reinterpret_cast<const f32x4*>(info + kRT + m0);
          typedef int i32x4 __attribute__((ext_vector_type(4)));
          const i32x4 lo = *reinterpret_cast<const i32x4*>(info + 2 * kRT + m0);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(info + 3 * kRT + m0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * q + e;
            const bool vis = j >= lo[e] && j <= hi[e];
            const float p = vis ? fast_exp2(s[rh][i] * a.sl2 - lv[e]) : 0.f;
            pb[2 * rh + (i >> 3)][i & 7] = bf16_t(p);
            sb[2 * rh + (i >> 3)][i & 7] = bf16_t(p * (dp[rh][i] - dv4[e]));
          }
        }
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const int c = 4 * md + 2 * tr_c16 + (tr_kq >> 1), cb = (tr_kq & 1) * 8;
#pragma unroll
        for (int st = 0; st < 2 * RH; ++st) {
          const int r0 = 16 * st + 4 * hf + tr_r, r1 = r0 + 8;
          const s16x4 d0 = lds_tr16(dt + L::pos(r0, c) + cb), d1 = lds_tr16(dt + L::pos(r1, c) + cb);
          const s16x4 q0 = lds_tr16(qt + L::pos(r0, c) + cb), q1 = lds_tr16(qt + L::pos(r1, c) + cb);
          const bf16x8 ad = __builtin_bit_cast(bf16x8, __builtin_shufflevector(d0, d1, 0, 1, 2, 3, 4, 5, 6, 7));
          const bf16x8 aq = __builtin_bit_cast(bf16x8, __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7));
          dv[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, pb[st], dv[md], 0, 0, 0);
          dk[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, sb[st], dk[md], 0, 0, 0);
        }
      }
      if (more) store_tile(lds[(t + 1) & 1]);
      if (t + 2 < nt) put_row(rowbuf[t & 1]);
      __syncthreads();
    }
  }
  if (j < a.N) {
    const int64_t off = ((int64_t(b) * a.N + j) * a.Hkv + kvh) * D;
    bf16_t* dkp = static_cast<bf16_t*>(a.dK) + off;
    bf16_t* dvp = static_cast<bf16_t*>(a.dV) + off;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ch = 32 * md + 8 * q + 4 * hf;
        bf16x4 vk, vv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vk[e] = bf16_t(dk[md][4 * q + e] * a.scale);
          vv[e] = bf16_t(dv[md][4 * q + e]);
        }
        *reinterpret_cast<bf16x4*>(dkp + ch) = vk;
        *reinterpret_cast<bf16x4*>(dvp + ch) = vv;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ on the matrix cores (bfloat16), with each row's LSE and D for the dK/dV
// kernel.  A workgroup owns kQRows query rows of one head, 32 per wave;
// each wave keeps its rows' Q and dO as MFMA B operands in registers, so
// the 32x32 accumulators put one query per lane column (lanes l and l^32
// share query l % 32).  Blocks of kQKeys keys of the KV head are staged in
// LDS (double-buffered, one barrier per block) and shared by the waves:
//   S^T = K Q^T,  dP^T = V dO^T            (keys x queries, k = channels)
//   one online pass: m = running maximum of S sl2 (raised only when a
//   block exceeds it; dq and the sum rescaled then), p = 2^(S sl2 - m),
//   dS^T = p (dP^T - D)
//   dQ^T += K^T dS^T                        (channels x queries, k = keys)
// and at the end dQ = scale dq / l, LSE = m + log2(l), D = <dO, O> (formed
// from the same registers before the pass).  K is read both ways (plain
// rows for the scores, ds_read_b64_tr_b16 for K^T), with the swizzle of
// KvTile.  kFar = false: rows in token order, only gate=0 rows written
// (their keys are the window); kFar = true: the gate=1 rows of the head's
// gate group, gathered from the compacted list (keys [0, i]), heaviest
// tiles first.
// ---------------------------------------------------------------------------
constexpr int kQRows = 128;  // query rows per workgroup (4 waves x 32)
constexpr int kQKeys = 64;   // keys per LDS block

template <int D, bool kFar>
__global__ __launch_bounds__(kBwdThreads) void bwd_q_mfma_kernel(BwdArgs a) {
  using L = KvTile<D>;
  constexpr int KS = D / 16;
  constexpr int MD = D / 32;
  constexpr int kMat = kQKeys * L::kRowB;             // one staged K or V block
  constexpr int kPer = kQKeys * L::kCPR / kBwdThreads;  // chunks per thread and matrix
  static_assert(kQKeys * L::kCPR % kBwdThreads == 0, "block staging");
  __shared__ __attribute__((aligned(16))) char lds[2][2 * kMat];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int rl = lane & 31, hf = lane >> 5;
  const int nbh = a.B * a.Hq;
  const int ntile = (a.N + kQRows - 1) / kQRows;
  const int bh = blockIdx.x % nbh;
  const int b = bh / a.Hq, h = bh % a.Hq, kvh = h / a.HK, g = h / a.HG;
  const int32_t* list = a.idx + (int64_t(b) * a.G + g) * a.N;
  int tile = blockIdx.x / nbh;
  int n = 0;
  if constexpr (kFar) {
    n = a.cnt[b * a.G + g];
    tile = ntile - 1 - tile;  // the last gathered tiles hold the longest rows: first
    if (tile * kQRows >= n) return;  // workgroup-uniform, before any barrier
  }
  // this lane's query row and its visible keys [lo, hi]; act: row written here
  const int slot = tile * kQRows + wave * 32 + rl;
  int row, lo, hi;
  bool act;
  if constexpr (kFar) {
    act = slot < n;
    row = list[act ? slot : n - 1];
    lo = 0;
    hi = act ? row : -1;
  } else {
    row = min(slot, a.N - 1);
    act = slot < a.N && a.gate[(int64_t(b) * a.N + row) * a.G + g] == 0;
    lo = act ? row - a.W + 1 : 1;
    hi = act ? row : 0;
  }
  // key blocks of the workgroup: the union of its rows' ranges
  int wlo, whi;
  if constexpr (kFar) {
    wlo = 0;
    whi = list[min(n, tile * kQRows + kQRows) - 1];
  } else {
    wlo = max(0, tile * kQRows - a.W + 1);
    whi = min(a.N, tile * kQRows + kQRows) - 1;
  }
  const int kb0 = wlo / kQKeys, kb1 = whi / kQKeys;
  const int vlo = wave_min_i(act ? lo : INT_MAX), vhi = wave_max_i(act ? hi : -1);  // this wave's keys
  const int64_t qrs = int64_t(a.Hq) * D;
  const int64_t qoff = (int64_t(b) * a.N + row) * qrs + int64_t(h) * D + 8 * hf;
  bf16x8 qreg[KS], oreg[KS];
  float Dv = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qreg[ks] = *reinterpret_cast<const bf16x8*>(static_cast<const bf16_t*>(a.Q) + qoff + 16 * ks);
    oreg[ks] = *reinterpret_cast<const bf16x8*>(static_cast<const bf16_t*>(a.dO) + qoff + 16 * ks);
    const bf16x8 ov = *reinterpret_cast<const bf16x8*>(static_cast<const bf16_t*>(a.O) + qoff + 16 * ks);
#pragma unroll
    for (int e = 0; e < 8; ++e) Dv = fmaf(float(oreg[ks][e]), float(ov[e]), Dv);
  }
  Dv += __shfl_xor(Dv, 32);
  const int64_t krs = int64_t(a.Hkv) * D;
  const bf16_t* kh = static_cast<const bf16_t*>(a.K) + int64_t(b) * a.N * krs + int64_t(kvh) * D;
  const bf16_t* vh = static_cast<const bf16_t*>(a.V) + int64_t(b) * a.N * krs + int64_t(kvh) * D;
  u32x4 sk[kPer], sv[kPer];
  const auto load_block = [&](int kb) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int u = tid + p * kBwdThreads, r = u / L::kCPR, c = u % L::kCPR;
      const int key = min(kb * kQKeys + r, a.N - 1);  // past the end: masked
      sk[p] = *reinterpret_cast<const u32x4*>(kh + int64_t(key) * krs + 8 * c);
      sv[p] = *reinterpret_cast<const u32x4*>(vh + int64_t(key) * krs + 8 * c);
    }
  };
  const auto store_block = [&](char* buf) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int u = tid + p * kBwdThreads, r = u / L::kCPR, c = u % L::kCPR;
      *reinterpret_cast<u32x4*>(buf + L::pos(r, c)) = sk[p];
      *reinterpret_cast<u32x4*>(buf + kMat + L::pos(r, c)) = sv[p];
    }
  };
  f32x16 dq[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) dq[md] = f32x16{};
  float m = kNegInf, l = 0.f;
  const int tr_r = (lane >> 2) & 3, tr_kq = lane & 3, tr_c16 = (lane >> 4) & 1;
  load_block(kb0);
  store_block(lds[0]);
  __syncthreads();
  for (int kb = kb0; kb <= kb1; ++kb) {
    const bool more = kb < kb1;
    if (more) load_block(kb + 1);
    const char* kt = lds[(kb - kb0) & 1];
    const char* vt = kt + kMat;
    const int key0 = kb * kQKeys;
    if (key0 + kQKeys - 1 >= vlo && key0 <= vhi) {  // wave-uniform: any of this wave's pairs here
      f32x16 s[2], dp[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        s[mt] = dp[mt] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 ak = *reinterpret_cast<const bf16x8*>(kt + L::pos(32 * mt + rl, 2 * ks + hf));
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(vt + L::pos(32 * mt + rl, 2 * ks + hf));
          s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qreg[ks], s[mt], 0, 0, 0);
          dp[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, oreg[ks], dp[mt], 0, 0, 0);
        }
      }
      // element i of slice mt: key key0 + 32 mt + 8 (i/4) + 4 hf + i%4
      float bmax = kNegInf;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 32 * mt + 8 * (i >> 2) + 4 * hf + (i & 3);
          const float x = (key >= lo && key <= hi) ? s[mt][i] * a.sl2 : kNegInf;
          s[mt][i] = x;
          bmax = fmaxf(bmax, x);
        }
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
      const bool raise = bmax > m;
      if (__any(raise)) {
        const float alpha = raise ? fast_exp2(m - bmax) : 1.f;  // 0 while m is -inf
        l *= alpha;
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
          for (int i = 0; i < 16; ++i) dq[md][i] *= alpha;
        if (raise) m = bmax;
      }
      bf16x8 sb[4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = s[mt][i];
          const float p = x == kNegInf ? 0.f : fast_exp2(x - m);
          l += p;
          sb[2 * mt + (i >> 3)][i & 7] = bf16_t(p * (dp[mt][i] - Dv));
        }
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const int c = 4 * md + 2 * tr_c16 + (tr_kq >> 1), cb = (tr_kq & 1) * 8;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int r0 = 16 * st + 4 * hf + tr_r, r1 = r0 + 8;
          const s16x4 k0 = lds_tr16(kt + L::pos(r0, c) + cb), k1 = lds_tr16(kt + L::pos(r1, c) + cb);
          const bf16x8 ak = __builtin_bit_cast(bf16x8, __builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7));
          dq[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, sb[st], dq[md], 0, 0, 0);
        }
      }
    }
    if (more) store_block(lds[(kb + 1 - kb0) & 1]);
    __syncthreads();
  }
  const float lt = l + __shfl_xor(l, 32);
  if (act) {
    const float inv = a.scale / lt;
    bf16_t* dqp = static_cast<bf16_t*>(a.dQ) + (int64_t(b) * a.N + row) * qrs + int64_t(h) * D;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = bf16_t(dq[md][4 * q + e] * inv);
        *reinterpret_cast<bf16x4*>(dqp + 32 * md + 8 * q + 4 * hf) = v;
      }
    if (hf == 0) {
      const int64_t sidx = (int64_t(b) * a.Hq + h) * a.N + row;
      a.lse2[sidx] = m + log2f(lt);
      a.Drow[sidx] = Dv;
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
  hipError_t e;
  if constexpr (std::is_same<T, bf16_t>::value) {
    const int64_t nq = (int64_t(a.N) + kQRows - 1) / kQRows * a.B * a.Hq;
    hipLaunchKernelGGL((bwd_q_mfma_kernel<D, false>), dim3(unsigned(nq)), dim3(kBwdThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_q_mfma_kernel<D, true>), dim3(unsigned(nq)), dim3(kBwdThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t nkb = (int64_t(a.N) + kKvKeys - 1) / kKvKeys;
    hipLaunchKernelGGL((bwd_kv_mfma_kernel<D>), dim3(unsigned(nkb * a.B * a.Hkv)), dim3(kBwdThreads), 0, s,
                       a);
  } else {
    hipLaunchKernelGGL((bwd_row_kernel<T, D, false>), dim3(unsigned(g1 < 65536 ? g1 : 65536)),
                       dim3(kBwdThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_row_kernel<T, D, true>), dim3(unsigned(g1 < 65536 ? g1 : 65536)),
                       dim3(kBwdThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_col_kernel<T, D>), dim3(unsigned(g2 < 65536 ? g2 : 65536)), dim3(kBwdThreads), 0,
                       s, a);
  }
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
