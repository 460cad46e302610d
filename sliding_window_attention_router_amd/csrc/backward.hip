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
// bfloat16, on the matrix cores (two launches):
//   bwd_q_mfma_kernel   a workgroup per 128 query rows of a head: one online
//                       pass over 64-key blocks gives dQ, LSE and D (the
//                       latter two go to the workspace); the gate=1 rows
//                       gathered from the compacted list, then the gate=0
//                       rows in token order, in one grid
//   bwd_kv_mfma_kernel  a workgroup per 64 keys of a KV head (16 a wave)
//                       walks 64-row tiles of the rows that see them (window
//                       rows of every gate, then gathered gate=1 rows) for
//                       each query head and accumulates dK, dV
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
// Staged K/V blocks of the dQ kernel and Q/dO row tiles (kRT rows).  LDS rows
// are XOR-swizzled by 16-byte chunk (KvTile) so that the dQ kernel's plain
// 16-byte reads (16 lanes, 16 consecutive rows, one chunk) and transposing
// reads (32 lanes, 4 rows x 4 chunks) hit distinct banks.
// ---------------------------------------------------------------------------
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

// ---------------------------------------------------------------------------
// dK, dV on the matrix cores (bfloat16), with v_mfma_f32_16x16x32_bf16.  A
// workgroup owns kKvKeys keys of one KV head, 16 per wave; each wave keeps
// its keys' K and V rows as MFMA B operands (lane l: key l % 16, channels
// 8 (l / 16) .. + 7 of each 32-channel step).  For every query head of the
// KV head the workgroup walks tiles of kRT query rows: first the window rows
// [k0, min(N, k0 + kKvKeys - 1 + W)) (any gate; masked per pair), then the
// gate=1 rows past them, gathered from the compacted list.  The four waves
// share each tile: its Q and dO rows are copied straight from global memory
// into LDS (global_load_lds_dwordx4, double-buffered, one barrier per tile;
// the lane -> source mapping applies the swizzle), with each row's LSE, D
// and visible key range beside them.
//   S  = Q K^T,  dP = dO V^T         (16-row tiles x 16 keys, k = channels)
//   P  = 2^(S sl2 - LSE) on visible pairs,  dS = P (dP - D)
//   dV^T += dO^T P,  dK^T += Q^T dS  (16-channel tiles x 16 keys, k = rows)
// The 16x16 accumulator of S gives lane l the key l % 16 and rows
// 4 (l / 16) + i of its 16-row tile; two tiles fill the eight contraction
// slots a B operand of the second products holds (slot 8g + i: row
// 32 st + 4g + i; slot 8g + 4 + i: row 32 st + 16 + 4g + i), so P and dS go
// from registers to the next MFMAs, and the transposed A operands (dO^T,
// Q^T) come from two ds_read_b64_tr_b16 each with the same row order
// (within 16 lanes, source lane 4r + k points at row r, channels
// c0 + 4k .. c0 + 4k + 3, and lane i receives channel c0 + i of rows
// 0..3).  With 243 VGPRs a wave (d = 128; no AGPRs, no scratch) two
// workgroups share a CU: two waves per SIMD, so one wave's exponentials and
// conversions can overlap the other's products.
// Layout of the row tiles (Kv16Tile), from LDS bank-conflict counts measured
// on gfx950 (64 banks of 4 bytes; ds_read_b128 serves the 16 lanes of a
// half-wave whose lane bits 2..4 have the same parity together, 8-byte reads
// serve a half-wave at a time): chunk c (16 bytes) of row r goes to plane
// c % 4, at r * (D / 2) bytes plus 16 * ((c / 4) ^ x(r, c)) inside the plane,
// with x = ((r / 4) % 2) + 2 (c % 2) for d = 128 and x = c % 2 for d = 64.
// Planes start at multiples of 256 bytes, so only the row and the slot pick
// the banks.  A plain operand read (lane: row 16 rt + l % 16, chunk
// 4 ks + l / 16) then finds the four lanes of a b128 group with equal l % 4
// on four different slots, and a half-wave's transposing reads (8 rows x two
// adjacent chunks x two 8-byte halves) on 32 different bank pairs.  (Whole
// rows with an XOR swizzle, or planes whose slot ignores either the row or
// the chunk parity, left one of the two reads with a two-way conflict.)
// ---------------------------------------------------------------------------
constexpr int kKvKeys = 64;  // keys per workgroup (4 waves x 16)

template <int D>
struct Kv16Tile {
  static constexpr int kRowB = 2 * D;
  static constexpr int kMat = kRT * kRowB;           // one staged matrix (Q or dO)
  static constexpr int kInfo = 2 * kMat;             // lse2, D, first key, last key: [4][kRT]
  static constexpr int kBytes = kInfo + 4 * kRT * 4;
  static constexpr int kCopies = kMat / 1024;        // 1 KB direct copies per matrix
  static constexpr int kPerWave = kCopies / (kBwdThreads / kWave);
  static_assert(kPerWave >= 1 && kCopies % (kBwdThreads / kWave) == 0, "tile copies");
  static constexpr int kPlaneRowB = kRowB / 4;       // bytes of a row in one plane
  static constexpr int kPlaneB = kRT * kPlaneRowB;   // bytes of one plane
  SWI_DEV static constexpr int x(int row, int chunk) {
    return D == 128 ? (((row >> 2) & 1) | ((chunk & 1) << 1)) : (chunk & 1);
  }
  SWI_DEV static constexpr int pos(int row, int chunk) {
    return (chunk & 3) * kPlaneB + row * kPlaneRowB + (((chunk >> 2) ^ x(row, chunk)) << 4);
  }
  // row and chunk held at byte offset o of a staged matrix (inverse of pos)
  SWI_DEV static constexpr int row_at(int o) { return (o % kPlaneB) / kPlaneRowB; }
  SWI_DEV static constexpr int chunk_at(int o) {
    const int plane = o / kPlaneB, r = row_at(o), slot = (o % kPlaneRowB) >> 4;
    return 4 * (slot ^ x(r, plane)) + plane;
  }
};

#define SWI_BWD_GLOBAL(p) ((__attribute__((address_space(1))) void*)(p))
#define SWI_BWD_LOCAL(p) ((__attribute__((address_space(3))) void*)(p))

template <int D>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_kv_mfma_kernel(BwdArgs a) {
  using L = Kv16Tile<D>;
  constexpr int KS = D / 32;  // 32-channel steps of the score products
  constexpr int CT = D / 16;  // 16-channel tiles of dK^T, dV^T
  constexpr int RT = kRT / 16;  // 16-row tiles of a row tile
  static_assert(kRT == 64, "two 32-row steps per row tile");
  __shared__ __attribute__((aligned(16))) char lds[2][L::kBytes];
  __shared__ int rowbuf[2][kRT];  // query row of each slot of the next tiles (-1: padding)
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int kl = lane & 15, grp = lane >> 4;
  const int nbk = a.B * a.Hkv;
  const int kblk = blockIdx.x / nbk, bk = blockIdx.x % nbk;  // heaviest key blocks first
  const int b = bk / a.Hkv, kvh = bk % a.Hkv;
  const int k0 = kblk * kKvKeys;
  const int j = k0 + wave * 16 + kl;  // this lane's key
  const int jc = min(j, a.N - 1);
  const bf16_t* Qp = static_cast<const bf16_t*>(a.Q);
  const bf16_t* dOp = static_cast<const bf16_t*>(a.dO);
  bf16x8 kreg[KS], vreg[KS];
  {
    const int64_t off = ((int64_t(b) * a.N + jc) * a.Hkv + kvh) * D + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kreg[ks] = *reinterpret_cast<const bf16x8*>(static_cast<const bf16_t*>(a.K) + off + 32 * ks);
      vreg[ks] = *reinterpret_cast<const bf16x8*>(static_cast<const bf16_t*>(a.V) + off + 32 * ks);
    }
  }
  f32x4 dk[CT], dv[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) dk[ct] = dv[ct] = f32x4{};
  const int wend = int(min<int64_t>(a.N, int64_t(k0) + kKvKeys - 1 + a.W));  // window rows end here
  const int nwt = (wend - k0 + kRT - 1) / kRT;
  const int64_t qrs = int64_t(a.Hq) * D;  // elements between query rows
  // transposing-read lane roles: row r of a 4-row group, channel quad kq
  const int tr_r = (lane >> 2) & 3, tr_kq = lane & 3;
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
    // Row indices run one tile ahead of the copies: the rows of tile t + 2
    // are looked up while tile t is computed and kept in LDS (rowbuf).  The
    // list is read for window tiles too, at a clamped index (branch-free).
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
    // each row's LSE, D and visible keys (one row per lane; wave w loads
    // and stores field w); the loads are issued before a tile's copies so
    // that waiting for them leaves the copies in flight
    static_assert(kRT == kWave && kBwdThreads / kWave == 4, "one info field per wave");
    float i_l = 0.f, i_d = 0.f;
    int i_row = 0, i_ok = 0;
    uint8_t i_g = 0;
    const auto load_info = [&](const int* rb) {
      const int r = rb[lane];
      i_ok = r >= 0;
      i_row = r >= 0 ? r : k0;
      if (wave == 0) i_l = lrow[i_row];
      else if (wave == 1) i_d = drow[i_row];
      else if (wave == 2) i_g = grow[int64_t(i_row) * a.G];
    };
    const auto store_info = [&](char* buf) {
      float* info = reinterpret_cast<float*>(buf + L::kInfo);
      if (wave == 0) info[lane] = i_ok ? i_l : __builtin_huge_valf();
      else if (wave == 1) info[kRT + lane] = i_ok ? i_d : 0.f;
      else if (wave == 2) reinterpret_cast<int*>(info)[2 * kRT + lane] = i_ok ? (i_g != 0 ? 0 : i_row - a.W + 1) : 0;
      else reinterpret_cast<int*>(info)[3 * kRT + lane] = i_ok ? i_row : -1;
    };
    // the copies of one tile: copy m covers LDS bytes [1024 m, 1024 m + 1024)
    // of each matrix; lane i writes 16 bytes at 16 i, which hold chunk
    // chunk_at(...) of row row_at(...) (padding slots read a valid row; their
    // pairs are masked by the info)
    const auto issue_tile = [&](char* buf, const int* rb) {
#pragma unroll
      for (int i = 0; i < L::kPerWave; ++i) {
        const int m = wave * L::kPerWave + i;
        const int byte = m * 1024 + lane * 16;
        const int row = rb[L::row_at(byte)];
        const int64_t src = int64_t(row >= 0 ? row : k0) * qrs + 8 * L::chunk_at(byte);
        __builtin_amdgcn_global_load_lds(SWI_BWD_GLOBAL(qh + src), SWI_BWD_LOCAL(buf + m * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(SWI_BWD_GLOBAL(dh + src), SWI_BWD_LOCAL(buf + L::kMat + m * 1024), 16,
                                         0, 0);
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
    load_info(rowbuf[0]);
    issue_tile(lds[0], rowbuf[0]);
    store_info(lds[0]);
    // iteration t: tile t lands in LDS buffer t % 2 (the wait + barrier at
    // the top make every wave's copies and the info visible, and make sure
    // every wave is done with tile t - 1, whose buffer the next copies
    // overwrite); tile t + 1 is copied and the rows of tile t + 2 looked up
    // while tile t is computed
    for (int t = 0; t < nt; ++t) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const bool more = t + 1 < nt;
      if (more) {
        load_info(rowbuf[(t + 1) & 1]);
        issue_tile(lds[(t + 1) & 1], rowbuf[(t + 1) & 1]);
      }
      if (t + 2 < nt) fetch_row(t + 2);
      const char* qt = lds[t & 1];
      const char* dt = qt + L::kMat;
      f32x4 s[RT], dp[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        s[rt] = dp[rt] = f32x4{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(qt + L::pos(16 * rt + kl, 4 * ks + grp));
          const bf16x8 ad = *reinterpret_cast<const bf16x8*>(dt + L::pos(16 * rt + kl, 4 * ks + grp));
          s[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, kreg[ks], s[rt], 0, 0, 0);
          dp[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ad, vreg[ks], dp[rt], 0, 0, 0);
        }
      }
      // instruction order for the scheduler: eight operand reads ahead, then
      // each product followed by the next read (LDS latency covered by the
      // products instead of waited for before each one)
      constexpr int kMfS = 2 * RT * KS;  // products and operand reads of this phase
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // LDS reads
#pragma unroll
      for (int i = 0; i < kMfS - 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      // P and dS of rows 16 rt + 4 grp + i; slot (rt % 2) * 4 + i of the
      // 32-row step rt / 2 of the second products.  Two kinds of tile see
      // every key of the workgroup and skip the visibility test: gathered
      // rows without padding (they lie past the window rows: i >= k0 + 63 + W)
      // and window tiles t >= 1 whose last row still has key k0 in its
      // window (k0 + 64 t + 63 - W + 1 <= k0) and lies before N.
      const float* info = reinterpret_cast<const float*>(qt + L::kInfo);
      typedef int i32x4 __attribute__((ext_vector_type(4)));
      bf16x8 pb[RT / 2], sb[RT / 2];
      const auto p_ds = [&](auto all_visible) {
        constexpr bool kAll = decltype(all_visible)::value;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int m0 = 16 * rt + 4 * grp;
          const f32x4 lv = *reinterpret_cast<const f32x4*>(info + m0);
          const f32x4 dv4 = *reinterpret_cast<const f32x4*>(info + kRT + m0);
          i32x4 lo = i32x4{}, hi = i32x4{};
          if constexpr (!kAll) {
            lo = *reinterpret_cast<const i32x4*>(info + 2 * kRT + m0);
            hi = *reinterpret_cast<const i32x4*>(info + 3 * kRT + m0);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool vis = kAll || (j >= lo[i] && j <= hi[i]);
            const float p = vis ? fast_exp2(s[rt][i] * a.sl2 - lv[i]) : 0.f;
            pb[rt >> 1][(rt & 1) * 4 + i] = bf16_t(p);
            sb[rt >> 1][(rt & 1) * 4 + i] = bf16_t(p * (dp[rt][i] - dv4[i]));
          }
        }
      };
      if ((t >= nwt && f0 + (t - nwt + 1) * kRT <= n) ||
          (t >= 1 && (t + 1) * kRT <= a.W && k0 + (t + 1) * kRT <= a.N))
        p_ds(std::true_type{});
      else
        p_ds(std::false_type{});
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int c = 2 * ct + (tr_kq >> 1), cb = (tr_kq & 1) * 8;
#pragma unroll
        for (int st = 0; st < RT / 2; ++st) {
          const int r0 = 32 * st + 4 * grp + tr_r, r1 = r0 + 16;
          const s16x4 d0 = lds_tr16(dt + L::pos(r0, c) + cb), d1 = lds_tr16(dt + L::pos(r1, c) + cb);
          const s16x4 q0 = lds_tr16(qt + L::pos(r0, c) + cb), q1 = lds_tr16(qt + L::pos(r1, c) + cb);
          const bf16x8 ad = __builtin_bit_cast(bf16x8, __builtin_shufflevector(d0, d1, 0, 1, 2, 3, 4, 5, 6, 7));
          const bf16x8 aq = __builtin_bit_cast(bf16x8, __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7));
          dv[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ad, pb[st], dv[ct], 0, 0, 0);
          dk[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, sb[st], dk[ct], 0, 0, 0);
        }
      }
      // the same for the second products: eight transposing reads ahead,
      // then two reads after each product
      constexpr int kMfP = 2 * CT * (RT / 2);  // products; twice as many reads
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < kMfP - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (more) store_info(lds[(t + 1) & 1]);
      if (t + 2 < nt) put_row(rowbuf[t & 1]);
    }
    __syncthreads();  // every wave is done with the last tile before the next head's copies
  }
  if (j < a.N) {
    const int64_t off = ((int64_t(b) * a.N + j) * a.Hkv + kvh) * D;
    bf16_t* dkp = static_cast<bf16_t*>(a.dK) + off;
    bf16_t* dvp = static_cast<bf16_t*>(a.dV) + off;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int ch = 16 * ct + 4 * grp;
      bf16x4 vk, vv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vk[i] = bf16_t(dk[ct][i] * a.scale);
        vv[i] = bf16_t(dv[ct][i]);
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
// share query l % 32).  Blocks of kQKeys keys of the KV head are copied
// straight into LDS (global_load_lds_dwordx4, double-buffered, one barrier
// per block) and shared by the waves; each block is taken in two 32-key
// steps, each of them complete:
//   S^T = K Q^T,  dP^T = V dO^T            (32 keys x queries, k = channels)
//   one online pass: m = running maximum of S sl2 (raised only when a
//   step exceeds it; dq and the sum rescaled then), p = 2^(S sl2 - m),
//   dS^T = p (dP^T - D)
//   dQ^T += K^T dS^T                        (channels x queries, k = keys)
// so only one step's scores are held (237 VGPRs at d = 128, no AGPRs: two
// waves per SIMD), and a step with none of the wave's pairs is skipped.  At
// the end dQ = scale dq / l, LSE = m + log2(l), D = <dO, O> (formed from
// the same registers before the pass).  K is read both ways (plain
// rows for the scores, ds_read_b64_tr_b16 for K^T), with the swizzle of
// KvTile.  One launch holds both kinds of tile: the first ntile * B * Hq
// workgroups take the gate=1 rows of their head's gate group, gathered from
// the compacted list (keys [0, i]), heaviest tiles first; the rest take rows
// in token order and write only the gate=0 ones (their keys are the window).
// The long gathered tiles are dispatched first and the short window tiles
// fill the slots that they leave idle.
// ---------------------------------------------------------------------------
constexpr int kQRows = 128;  // query rows per workgroup (4 waves x 32)
constexpr int kQKeys = 64;   // keys per LDS block

template <int D>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_q_mfma_kernel(BwdArgs a) {
  using L = KvTile<D>;
  constexpr int KS = D / 16;
  constexpr int MD = D / 32;
  constexpr int kMat = kQKeys * L::kRowB;  // one staged K or V block
  constexpr int kPerWave = kMat / 1024 / (kBwdThreads / kWave);  // 1 KB direct copies per wave and matrix
  static_assert(kPerWave >= 1 && kMat / 1024 % (kBwdThreads / kWave) == 0, "block copies");
  __shared__ __attribute__((aligned(16))) char lds[2][2 * kMat];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int rl = lane & 31, hf = lane >> 5;
  const int nbh = a.B * a.Hq;
  const int ntile = (a.N + kQRows - 1) / kQRows;
  // workgroups are dealt to the 8 XCDs in turn: give the workgroups of one
  // XCD neighbouring heads (the query heads of a KV head), which read the
  // same keys
  const bool far = int(blockIdx.x) < ntile * nbh;
  const int wg = far ? int(blockIdx.x) : int(blockIdx.x) - ntile * nbh;
  const int jh = wg % nbh;
  const int bh = nbh % 8 == 0 ? (jh % 8) * (nbh / 8) + jh / 8 : jh;
  const int b = bh / a.Hq, h = bh % a.Hq, kvh = h / a.HK, g = h / a.HG;
  const int32_t* list = a.idx + (int64_t(b) * a.G + g) * a.N;
  int tile = wg / nbh;
  int n = 0;
  if (far) {
    n = a.cnt[b * a.G + g];
    tile = ntile - 1 - tile;  // the last gathered tiles hold the longest rows: first
    if (tile * kQRows >= n) return;  // workgroup-uniform, before any barrier
  }
  // this lane's query row and its visible keys [lo, hi]; act: row written here
  const int slot = tile * kQRows + wave * 32 + rl;
  int row, lo, hi;
  bool act;
  if (far) {
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
  if (far) {
    wlo = 0;
    whi = list[min(n, tile * kQRows + kQRows) - 1];
  } else {
    wlo = max(0, tile * kQRows - a.W + 1);
    whi = min(a.N, tile * kQRows + kQRows) - 1;
  }
  const int kb0 = wlo / kQKeys, kb1 = whi / kQKeys;
  const int vlo = wave_min_i(act ? lo : INT_MAX), vhi = wave_max_i(act ? hi : -1);  // this wave's keys
  // keys every active row of the wave sees: [flo, fhi]
  const int flo = wave_max_i(act ? lo : INT_MIN), fhi = wave_min_i(act ? hi : INT_MAX);
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
  // the copies of one key block: copy m covers LDS bytes [1024 m, 1024 m +
  // 1024) of each matrix; lane i writes the 16 bytes at 16 i, which hold
  // chunk slot ^ swz(r) of row r (keys past the end read the last key; their
  // pairs are masked)
  const auto issue_block = [&](char* buf, int kb) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int m = wave * kPerWave + i;
      const int byte = m * 1024 + lane * 16;
      const int r = byte / L::kRowB, c = ((byte % L::kRowB) >> 4) ^ L::swz(r);
      const int64_t src = int64_t(min(kb * kQKeys + r, a.N - 1)) * krs + 8 * c;
      __builtin_amdgcn_global_load_lds(SWI_BWD_GLOBAL(kh + src), SWI_BWD_LOCAL(buf + m * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(SWI_BWD_GLOBAL(vh + src), SWI_BWD_LOCAL(buf + kMat + m * 1024), 16, 0, 0);
    }
  };
  f32x16 dq[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) dq[md] = f32x16{};
  float m = kNegInf, l = 0.f;
  const int tr_r = (lane >> 2) & 3, tr_kq = lane & 3, tr_c16 = (lane >> 4) & 1;
  issue_block(lds[0], kb0);
  // iteration kb: block kb lands in buffer (kb - kb0) % 2 (the wait + barrier
  // at the top make every wave's copies visible and make sure every wave is
  // done with block kb - 1, whose buffer the next copies overwrite)
  for (int kb = kb0; kb <= kb1; ++kb) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kb < kb1) issue_block(lds[(kb + 1 - kb0) & 1], kb + 1);
    const char* kt = lds[(kb - kb0) & 1];
    const char* vt = kt + kMat;
    // the block in two halves of 32 keys, each a full step (scores, softmax
    // update, dS, dQ products): half the score registers of a 64-key step
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int key0 = kb * kQKeys + 32 * mt;
      if (key0 + 31 < vlo || key0 > vhi) continue;  // wave-uniform: none of this wave's pairs here
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(kt + L::pos(32 * mt + rl, 2 * ks + hf));
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(vt + L::pos(32 * mt + rl, 2 * ks + hf));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qreg[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, oreg[ks], dp, 0, 0, 0);
      }
      // element i: key key0 + 8 (i/4) + 4 hf + i%4.  Masking only rewrites
      // the scores, in a wave-uniform branch skipped by steps whose keys
      // every active row sees.
      if (key0 < flo || key0 + 31 > fhi) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 8 * (i >> 2) + 4 * hf + (i & 3);
          if (key < lo || key > hi) s[i] = kNegInf;
        }
      }
      float bmax = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float x = s[i] * a.sl2;
        s[i] = x;
        bmax = fmaxf(bmax, x);
      }
      bmax = fmaxf(bmax, xor32(bmax));
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
      // dS^T of k-steps st = 2 mt + j (slot e: key 16 st + 8 (e/4) + 4 hf + e%4)
      bf16x8 sb[2];
      const float mu = m == kNegInf ? 0.f : m;  // -inf while no key was seen: p = 0 then
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float x = s[i];
        const float p = fast_exp2(x - mu);
        l += p;
        sb[i >> 3][i & 7] = bf16_t(p * (dp[i] - Dv));
      }
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const int c = 4 * md + 2 * tr_c16 + (tr_kq >> 1), cb = (tr_kq & 1) * 8;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int r0 = 16 * (2 * mt + j) + 4 * hf + tr_r, r1 = r0 + 8;
          const s16x4 k0 = lds_tr16(kt + L::pos(r0, c) + cb), k1 = lds_tr16(kt + L::pos(r1, c) + cb);
          const bf16x8 ak = __builtin_bit_cast(bf16x8, __builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7));
          dq[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, sb[j], dq[md], 0, 0, 0);
        }
      }
    }
  }
  const float lt = l + xor32(l);
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
    hipLaunchKernelGGL((bwd_q_mfma_kernel<D>), dim3(unsigned(2 * nq)), dim3(kBwdThreads), 0, s, a);
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
