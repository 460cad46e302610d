// SwiAttn routed decode on gfx950.
//
// SwiAttn report, section 2: during decode the full and window branches read
// one shared KV cache.  The new token of sequence b sits at position L-1
// (L = cache_len[b]); a head routed full reads keys [0, L-1], a head routed
// to the window reads the last min(W, L) keys (weimeta SWA glossary, section
// "详细解释").  The bytes read therefore depend on the gate: 32K keys for a
// full sequence at a 32K cache, W keys otherwise.
//
// Work split (stream-K): the key range of each (sequence, KV head) pair is
// cut into 64-key blocks, the blocks of all pairs are laid end to end, and
// workgroup w of G takes the contiguous share [w*T/G, (w+1)*T/G) of the T
// blocks.  Every workgroup reads the gates and cache lengths itself to find
// T and its share, so no scheduling launch precedes the kernel; the shares
// differ by at most one block.
//
// decode_kernel        single-wave workgroups; each walks its share with the
//                      next block's loads in flight (also across pairs).  A
//                      pair that lies wholly inside one share is finished and
//                      written there; a pair cut by share boundaries leaves a
//                      normalised partial output + log-sum-exp per piece
// decode_merge_kernel  log-sum-exp merge of the pieces of each cut pair
// step_prep_kernel     serving step: routes each sequence's new token,
//                      appends its key and value rows and advances the
//                      length, ahead of the two launches above
// The allocation-free entry point runs the same launches on a fixed
// per-device scratch array instead of a caller workspace.  With a window
// offset o a window head takes the window of position L-1-o.
//
// Global anchors (weimeta SWA glossary, section "SWA 落地的四个常见坑",
// pitfall 1, fix 2): with A > 0 a window head also reads the first
// min(A, L-W) keys of the cache.  A pair with a window head then starts with
// anchor blocks [0, 64 na) (masked to each head's anchors) before its main
// range; the masks keep the two key sets of a head disjoint.
#include <climits>
#include <mutex>

#include "attn_core.hpp"
#include "kernels.hpp"

namespace swi {

constexpr int kDecThreads = 64;  // one wave per workgroup
constexpr int kDecGrid = 1024;   // four single-wave workgroups per CU (bf16: 32 KB LDS each)
// K/V rows carry the non-temporal hint: the cache is read once per step.
constexpr bool kDecStream = true;

struct DecodeArgs {
  const void* q;
  const void* Kc;
  const void* Vc;
  const int32_t* cache_len;
  const uint8_t* gate;
  void* o;
  int32_t* info;    // [0] T; per pair bk: [1+2bk] first block if cut else -1, [2+2bk] block count
  float* part_o;    // [2*grid][HK][D] pieces of cut pairs, slot 2w (first piece of share w) or 2w+1
  float* part_lse;  // [2*grid][HK]
  int B, Lmax, Hq, Hkv, G, W, HK, HG;
  int A;    // global anchor keys of the window branch (0 = none)
  int off;  // window offset of the layer: a window head takes the window of position L-1-off
  float sl2;
};

SWI_DEV int clamp_len(int L, int Lmax) { return L < 1 ? 1 : (L > Lmax ? Lmax : L); }

// Keys [lo, hi] of head h in sequence b: [0, L-1] for a full head; for a
// window head the window of position p = L-1-off, [max(0, p-W+1), p]
// (empty, hi < lo, when p < 0).
SWI_DEV void head_range(const DecodeArgs& a, int b, int h, int L, int& lo, int& hi) {
  if (a.gate[b * a.G + h / a.HG] != 0) {
    lo = 0;
    hi = L - 1;
    return;
  }
  const int p = L - 1 - a.off;
  lo = max(0, p - a.W + 1);
  hi = p;
}

// Keys [lo, hi] read for pair bk = (sequence, KV head): the union of the
// ranges of its query heads (at least one block: a pair whose window heads
// all have an empty window visits one fully masked block, so that its
// output is still written); na anchor blocks precede them when a head of
// the pair is a window head.  Returns the number of 64-key blocks.
SWI_DEV int pair_blocks(const DecodeArgs& a, int bk, int& L, int& lo, int& hi, int& na) {
  const int b = bk / a.Hkv, kvh = bk - b * a.Hkv;
  L = clamp_len(a.cache_len[b], a.Lmax);
  const int g0 = kvh * a.HK / a.HG, g1 = (kvh * a.HK + a.HK - 1) / a.HG;
  bool full = false, win = false;
  for (int gg = g0; gg <= g1; ++gg) {
    const bool f = a.gate[b * a.G + gg] != 0;
    full = full || f;
    win = win || !f;
  }
  const int p = L - 1 - a.off;
  const int wlo = max(0, p - a.W + 1);
  lo = full ? 0 : wlo;
  hi = full ? L - 1 : max(p, wlo);
  na = win ? (min(a.A, wlo) + kBN - 1) / kBN : 0;
  return na + (hi - lo) / kBN + 1;
}

// First block of share w: floor(w*T/G).
SWI_DEV int share_start(int w, int T, int G) { return int(int64_t(w) * T / G); }
// The share that holds block x: the largest w with share_start(w) <= x.
SWI_DEV int share_of(int x, int T, int G) {
  return int(((int64_t(x) + 1) * G + T - 1) / T) - 1;
}

SWI_DEV int lane_of(int v, int j) { return __builtin_amdgcn_readlane(v, j); }

// float32 staging of one 64-key block (one wave, padded layout of the
// float32 core): 16-key quarters through registers, the next quarter's loads
// in flight while the current one is stored (a whole block in registers
// would take 256 VGPRs).
template <int D, bool kStream>
struct DecF32Stage {
  using L = Lds<float, D>;
  static constexpr int CPR = D / 4;                 // 16-byte pieces per row
  static constexpr int QK = 16;                     // keys per quarter
  static constexpr int PER = QK * CPR / kWave;      // pieces per lane and matrix
  static_assert(QK * CPR % kWave == 0, "quarter layout");
  u32x4 kr[2][PER], vr[2][PER];
  SWI_DEV void load(int st, const float* Kb, const float* Vb, int64_t rs, int k0, int kend, int lane) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int u = lane + kWave * j, key = u / CPR, c = u - key * CPR;
      const int kk = clamp_row(k0 + key, kend);
      kr[st][j] = load16<kStream>(Kb + kk * rs + c * 4);
      vr[st][j] = load16<kStream>(Vb + kk * rs + c * 4);
    }
  }
  SWI_DEV void store(int st, char* lds, int q0, int lane) const {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int u = lane + kWave * j, key = q0 + u / CPR, c = u % CPR;
      uint32_t* kp = reinterpret_cast<uint32_t*>(lds + key * L::kKStride) + c * 4;
      uint32_t* vp = reinterpret_cast<uint32_t*>(lds + L::kKBytes + key * L::kVStride) + c * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kp[e] = kr[st][j][e];
        vp[e] = vr[st][j][e];
      }
    }
  }
  SWI_DEV void block(char* lds, const float* Kb, const float* Vb, int64_t rs, int kb, int kend, int lane) {
    load(0, Kb, Vb, rs, kb, kend, lane);
#pragma unroll
    for (int qq = 0; qq < kBN / QK; ++qq) {
      if (qq + 1 < kBN / QK) load((qq + 1) & 1, Kb, Vb, rs, kb + (qq + 1) * QK, kend, lane);
      store(qq & 1, lds, qq * QK, lane);
    }
  }
};

// 64 consecutive pairs, one per lane, with the inclusive prefix sum of their
// block counts (absolute: carry holds the blocks of all earlier pairs).
struct PairWindow {
  int base, L, lo, hi, na, incl;
  SWI_DEV void fill(const DecodeArgs& a, int base_, int carry, int lane, int npairs) {
    base = base_;
    const int bk = base + lane;
    int n = 0;
    L = 1;
    lo = 0;
    hi = 0;
    na = 0;
    if (bk < npairs) n = pair_blocks(a, bk, L, lo, hi, na);
    incl = wave_incl_scan_i(n) + carry;
  }
};

// The blocks [blk0, blk1) of pair bk that fall into share [s, e).  Block n
// of the pair is anchor block n for n < na, else main block n - na.
struct DecSeg {
  int bk, b, kvh, L, lo, na, first, nb, blk0, blk1;
  SWI_DEV void from(const DecodeArgs& a, const PairWindow& win, int j, int s, int e) {
    bk = win.base + j;
    b = bk / a.Hkv;
    kvh = bk - b * a.Hkv;
    L = lane_of(win.L, j);
    lo = lane_of(win.lo, j);
    const int hi = lane_of(win.hi, j);
    na = lane_of(win.na, j);
    const int incl = lane_of(win.incl, j);
    nb = na + (hi - lo) / kBN + 1;
    first = incl - nb;
    blk0 = max(s, first) - first;
    blk1 = min(e, incl) - first;
  }
  SWI_DEV int kb(int n) const { return n < na ? n * kBN : lo + (n - na) * kBN; }
  template <typename T, int D>
  SWI_DEV const T* kbase(const DecodeArgs& a) const {
    return static_cast<const T*>(a.Kc) + (int64_t(b) * a.Lmax * a.Hkv + kvh) * D;
  }
  template <typename T, int D>
  SWI_DEV const T* vbase(const DecodeArgs& a) const {
    return static_cast<const T*>(a.Vc) + (int64_t(b) * a.Lmax * a.Hkv + kvh) * D;
  }
};

// Per-dtype staging of the decode's K/V blocks.  bf16: the swizzled row
// layout of the prefill's DMA path, filled from registers with linear
// 16-byte stores (K and V separately, so the next block's K loads are in
// flight while V is stored), read by the DMA-layout core (V^T through
// transposing LDS reads).  float32: the padded layout of the float32 core,
// staged in 16-key quarters (DecF32Stage).
template <typename T, int D>
struct DecCfg;
template <int D>
struct DecCfg<bf16_t, D> {
  using Core = CoreBF16Dma<D>;
  using Loader = KVRegDma<D, kDecThreads, kDecStream>;
  static constexpr int kLds = LdsDma<D>::kBytes;
  static constexpr bool kSplit = true;
};
template <int D>
struct DecCfg<float, D> {
  using Core = CoreF32<D>;
  using Loader = DecF32Stage<D, kDecStream>;
  static constexpr int kLds = Lds<float, D>::kBytes;
  static constexpr bool kSplit = false;
};

template <typename T, int D>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(DecodeArgs a) {
  using Cfg = DecCfg<T, D>;
  using Core = typename Cfg::Core;
  __shared__ __align__(16) char lds[Cfg::kLds];
  const int lane = threadIdx.x, q = lane & 31, g = lane >> 5;
  const int npairs = a.B * a.Hkv;
  const int G = gridDim.x, w = blockIdx.x;

  // the blocks of all pairs (every workgroup counts them itself)
  int tsum = 0;
  for (int base = 0; base < npairs; base += 4 * kWave) {
    int n[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int bk = base + k * kWave + lane;
      int L, lo, hi, na;
      n[k] = bk < npairs ? pair_blocks(a, bk, L, lo, hi, na) : 0;
    }
    tsum += n[0] + n[1] + n[2] + n[3];
  }
  const int total = wave_sum_i(tsum);
  if (w == 0 && lane == 0) a.info[0] = total;
  const int s = share_start(w, total, G), e = share_start(w + 1, total, G);
  if (s >= e) return;

  // the pair holding block s
  PairWindow win;
  int carry = 0, j = -1;
  for (int base = 0; base < npairs; base += kWave) {
    win.fill(a, base, carry, lane, npairs);
    const uint64_t hit = __ballot(win.incl > s);
    if (hit) {
      j = __builtin_ctzll(hit);
      break;
    }
    carry = lane_of(win.incl, kWave - 1);
  }
  if (j < 0) return;  // unreachable: s < T

  const bool valid = q < a.HK;
  const int64_t rs = int64_t(a.Hkv) * D;
  DecSeg cur;
  cur.from(a, win, j, s, e);
  Core c;
  int lo_h = 0, hi_h = -1, ahi = -1, wmax_lo = 0, wmin_hi = -1, wmin_ahi = -1;
  auto begin = [&]() {
    c.init();
    const int h = cur.kvh * a.HK + q;
    const T* qp = static_cast<const T*>(a.q) + (int64_t(cur.b) * a.Hq + h) * D;
    c.load_q(valid ? qp : nullptr, g);
    lo_h = 0;
    hi_h = -1;
    if (valid) head_range(a, cur.b, h, cur.L, lo_h, hi_h);
    // a window head's anchors [0, ahi] end where its window starts; a full
    // head (lo_h = 0) has none
    ahi = valid ? min(a.A, lo_h) - 1 : -1;
    // anchor blocks every head covers whole need no mask
    wmin_ahi = wave_min_i(valid ? ahi : INT_MAX);
    // heads of one KV head may start and end at different keys (window
    // heads next to full ones): blocks before the latest start or past the
    // earliest end are masked
    wmax_lo = wave_max_i(valid ? lo_h : -1);
    wmin_hi = wave_min_i(valid ? hi_h : INT_MAX);
  };
  begin();
  typename Cfg::Loader ld;
  if constexpr (Cfg::kSplit) ld.load(cur.kbase<T, D>(a), cur.vbase<T, D>(a), rs, cur.kb(cur.blk0), cur.L, lane);
  int n = cur.blk0;
  while (true) {
    // the block after this one, possibly the first block of the next pair
    const bool seg_end = n + 1 >= cur.blk1;
    const bool more = !seg_end || cur.first + cur.blk1 < e;
    DecSeg nx = cur;
    int nn = n + 1;
    if (seg_end && more) {
      if (++j == kWave) {
        win.fill(a, win.base + kWave, lane_of(win.incl, kWave - 1), lane, npairs);
        j = 0;
      }
      nx.from(a, win, j, s, e);
      nn = nx.blk0;
    }
    __syncthreads();
    if constexpr (Cfg::kSplit) {
      // The loads are issued whether or not a next block exists (without
      // one they re-read row 0 of this block: in bounds, 256 bytes), so the
      // load sequence does not depend on `more` and the waits before the V
      // stores count the new K loads instead of waiting for them.
      const T* kbn = more ? nx.kbase<T, D>(a) : cur.kbase<T, D>(a);
      const T* vbn = more ? nx.vbase<T, D>(a) : cur.vbase<T, D>(a);
      const int lkb = more ? nx.kb(nn) : cur.kb(n);
      const int lend = more ? nx.L : lkb + 1;
      ld.store_k(lds, lane);
      ld.load_k(kbn, rs, lkb, lend, lane);
      ld.store_v(lds, lane);
      ld.load_v(vbn, rs, lkb, lend, lane);
      __syncthreads();
    } else {
      ld.block(lds, cur.kbase<T, D>(a), cur.vbase<T, D>(a), rs, cur.kb(n), cur.L, lane);
      __syncthreads();
    }
    const int kb = cur.kb(n);
    const bool anc = n < cur.na;  // wave-uniform
    const bool masked = anc ? kb + kBN - 1 > wmin_ahi : (kb < wmax_lo || kb + kBN - 1 > wmin_hi);
    c.block(lds, kb, masked, anc ? 0 : lo_h, anc ? ahi : hi_h, a.sl2, q, g);
    if (!seg_end) {
      n = nn;
      continue;
    }
    // pair piece finished: write the output, or a partial for the merge
    float lse2;
    const float inv = finish_row(c.m, c.l, lse2);
    const bool whole = cur.blk0 == 0 && cur.blk1 == cur.nb;
    if (whole) {
      T* orow = static_cast<T*>(a.o) + (int64_t(cur.b) * a.Hq + cur.kvh * a.HK + q) * D;
      if (valid) store_row<Core::MD>(orow, c.acc, inv, g);
    } else {
      const int slot = 2 * w + (cur.first + cur.blk0 == s ? 0 : 1);
      if (valid) {
        store_row<Core::MD>(a.part_o + (int64_t(slot) * a.HK + q) * D, c.acc, inv, g);
        if (g == 0) a.part_lse[int64_t(slot) * a.HK + q] = lse2;
      }
    }
    if (cur.blk0 == 0 && lane == 0) {  // the share that starts the pair describes it
      a.info[1 + 2 * cur.bk] = whole ? -1 : cur.first;
      a.info[2 + 2 * cur.bk] = cur.nb;
    }
    if (!more) break;
    cur = nx;
    begin();
    n = nn;
  }
}

// One workgroup per pair cut by share boundaries.  Thread t merges output
// elements 2t, 2t+1 (+512 ...) of the pair's [HK][D] block over its pieces
// in share order (a fixed order, so the result does not depend on timing),
// with the log-sum-exp rule: weights 2^(lse_k - max) on the normalised
// piece outputs.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a, int G) {
  __shared__ int slots[kDecGrid];
  const int bk = blockIdx.x;
  const int first = a.info[1 + 2 * bk];
  if (first < 0) return;
  const int nb = a.info[2 + 2 * bk], total = a.info[0];
  const int w0 = share_of(first, total, G), w1 = share_of(first + nb - 1, total, G);
  const int np = w1 - w0 + 1;
  // piece in share w0: its first or its second slot; later shares start
  // inside the pair, so their piece is their first slot (empty shares,
  // possible when there are fewer blocks than workgroups, hold none)
  for (int k = threadIdx.x; k < np; k += 256) {
    const int w = w0 + k;
    int sl = 2 * w;
    if (k == 0) sl += share_start(w0, total, G) == first ? 0 : 1;
    else if (share_start(w, total, G) == share_start(w + 1, total, G)) sl = -1;
    slots[k] = sl;
  }
  __syncthreads();
  const int b = bk / a.Hkv, kvh = bk - b * a.Hkv;
  T* obase = static_cast<T*>(a.o) + (int64_t(b) * a.Hq + kvh * a.HK) * D;
  // pieces are read in batches of kBatch with all loads in flight; the
  // running maximum is raised once per batch
  constexpr int kBatch = 32;  // a full-cache pair at 32K keys has about 24 pieces
  for (int e0 = 2 * threadIdx.x; e0 < a.HK * D; e0 += 512) {
    const int r = e0 / D;
    float M = kNegInf, Ls = 0.f, o0 = 0.f, o1 = 0.f;
    for (int k0 = 0; k0 < np; k0 += kBatch) {
      float lk[kBatch];
      float2 v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int sl = k0 + j < np ? slots[k0 + j] : -1;
        lk[j] = kNegInf;
        v[j] = make_float2(0.f, 0.f);
        if (sl >= 0) {
          lk[j] = a.part_lse[int64_t(sl) * a.HK + r];
          v[j] = *reinterpret_cast<const float2*>(a.part_o + int64_t(sl) * a.HK * D + e0);
        }
      }
      float mb = M;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) mb = fmaxf(mb, lk[j]);
      if (mb == kNegInf) continue;
      const float sc = M == kNegInf ? 0.f : fast_exp2(M - mb);
      Ls *= sc;
      o0 *= sc;
      o1 *= sc;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const float wt = lk[j] == kNegInf ? 0.f : fast_exp2(lk[j] - mb);
        Ls += wt;
        o0 = fmaf(wt, v[j].x, o0);
        o1 = fmaf(wt, v[j].y, o1);
      }
      M = mb;
    }
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
    Elem<T>::store(obase + e0, o0 * inv);
    Elem<T>::store(obase + e0 + 1, o1 * inv);
  }
}

static size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

bool plan_decode(const DecodeShape& sh, DecodePlan* p) {
  p->HK = sh.Hq / sh.Hkv;
  p->HG = sh.Hq / sh.G;
  const long long npairs = (long long)sh.B * sh.Hkv;
  const long long tmax = npairs * ((sh.Lmax + kBN - 1) / kBN);  // T can not exceed this
  if (tmax > INT_MAX / 4 || npairs > INT_MAX / 4) return false;
  p->grid = int(tmax < kDecGrid ? tmax : kDecGrid);
  size_t off = 0;
  p->off_info = off;
  off = align_up(off + (1 + 2 * size_t(npairs)) * 4);
  p->off_part_o = off;
  off = align_up(off + 2 * size_t(p->grid) * p->HK * sh.d * 4);
  p->off_part_lse = off;
  off = align_up(off + 2 * size_t(p->grid) * p->HK * 4);
  p->bytes = off;
  return true;
}

template <typename T, int D>
static hipError_t run_decode(const DecodeShape& sh, const DecodePlan& p, DecodeArgs& a,
                             hipStream_t s, void* const* ev) {
  hipError_t e;
  if ((e = mark(ev, 0, s)) != hipSuccess) return e;
  hipLaunchKernelGGL((decode_kernel<T, D>), dim3(p.grid), dim3(kDecThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = mark(ev, 1, s)) != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(sh.B * sh.Hkv), dim3(256), 0, s, a, p.grid);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return mark(ev, 2, s);
}

hipError_t launch_decode(const DecodeShape& sh, const DecodePlan& p, const void* q,
                         const void* Kc, const void* Vc, const int32_t* cache_len,
                         const uint8_t* gate, void* o, void* ws, hipStream_t s,
                         void* const* ev) {
  char* w = static_cast<char*>(ws);
  DecodeArgs a;
  a.q = q;
  a.Kc = Kc;
  a.Vc = Vc;
  a.cache_len = cache_len;
  a.gate = gate;
  a.o = o;
  a.info = reinterpret_cast<int32_t*>(w + p.off_info);
  a.part_o = reinterpret_cast<float*>(w + p.off_part_o);
  a.part_lse = reinterpret_cast<float*>(w + p.off_part_lse);
  a.B = sh.B;
  a.Lmax = sh.Lmax;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.G = sh.G;
  a.W = sh.W;
  a.A = sh.A;
  a.off = sh.off;
  a.HK = p.HK;
  a.HG = p.HG;
  a.sl2 = sh.scale * kLog2e;
  if (sh.f32) {
    if (sh.d == 64) return run_decode<float, 64>(sh, p, a, s, ev);
    return run_decode<float, 128>(sh, p, a, s, ev);
  }
  if (sh.d == 64) return run_decode<bf16_t, 64>(sh, p, a, s, ev);
  return run_decode<bf16_t, 128>(sh, p, a, s, ev);
}

// ---------------------------------------------------------------------------
// Fixed scratch of the allocation-free decode entry point: the decode
// workspace (pair table, partial outputs and log-sum-exps of the split-K
// pieces) placed in one file-scope device array instead of caller memory.
// Each GPU that loads the library holds its own copy of the array until the
// process ends.  Host code never passes the array's name to a kernel (on
// the host that name is only a stand-in, not a device address): the device
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and that pointer is used from then on.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

size_t decode_scratch_bytes() { return kScratchBytes; }

hipError_t decode_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Serving step: route the new token of each sequence, append its key and
// value rows at position L = cache_len[b] and advance the length to L + 1,
// in one launch (SwiAttn report, section 2: a router per token; both
// branches read one cache, so every token is appended whatever its gate),
// then the decode.  One workgroup per sequence: wave w computes the logits of
// gate groups w, w + 4, ... with the router's lane order and reduction tree
// (the same logits as swiattn_route), the threads copy the Hkv*d-element
// rows in 16-byte pieces, and one thread stores the new length after a
// barrier (every thread has read the old one before it).  A length below 0
// is taken as 0; a full cache (L >= Lmax) is left as it is.
// ---------------------------------------------------------------------------
constexpr int kStepThreads = 256;

template <typename T>
__global__ __launch_bounds__(kStepThreads) void step_prep_kernel(
    const T* __restrict__ Hn, const T* __restrict__ r, const float* __restrict__ bias,
    uint8_t* __restrict__ gate, int hidden, int G, const uint4* __restrict__ k,
    const uint4* __restrict__ v, uint4* __restrict__ Kc, uint4* __restrict__ Vc,
    int32_t* __restrict__ cache_len, int Lmax, int row16) {
  constexpr int VEC = 16 / Elem<T>::kBytes;  // elements per 16-byte load
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int L = max(cache_len[b], 0);
  const T* row = Hn + int64_t(b) * hidden;
  for (int g = wave; g < G; g += kStepThreads / 64) {
    float acc = 0.f;
    if (hidden % VEC == 0) {
      for (int vv = lane; vv < hidden / VEC; vv += 64) {
        u32x4 hv = *reinterpret_cast<const u32x4*>(row + int64_t(vv) * VEC);
        const T* hp = reinterpret_cast<const T*>(&hv);
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          acc = fmaf(Elem<T>::load(hp + e), Elem<T>::load(r + int64_t(vv * VEC + e) * G + g), acc);
      }
    } else {
      for (int kk = lane; kk < hidden; kk += 64)
        acc = fmaf(Elem<T>::load(row + kk), Elem<T>::load(r + int64_t(kk) * G + g), acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) gate[int64_t(b) * G + g] = acc + bias[g] > 0.f ? 1 : 0;
  }
  if (L < Lmax) {
    const int64_t dst = (int64_t(b) * Lmax + L) * row16;
    const int64_t src = int64_t(b) * row16;
    for (int i = threadIdx.x; i < row16; i += kStepThreads) {
      Kc[dst + i] = k[src + i];
      Vc[dst + i] = v[src + i];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && L < Lmax) cache_len[b] = L + 1;
}

hipError_t launch_decode_step(const DecodeShape& sh, const DecodePlan& p, const void* Hn,
                              const void* r, const float* bias, int hidden, const void* q,
                              const void* k, const void* v, void* Kc, void* Vc, int32_t* cache_len,
                              uint8_t* gate, void* o, void* ws, hipStream_t s) {
  const int row16 = sh.Hkv * sh.d * (sh.f32 ? 4 : 2) / 16;
  auto k4 = static_cast<const uint4*>(k);
  auto v4 = static_cast<const uint4*>(v);
  auto K4 = static_cast<uint4*>(Kc);
  auto V4 = static_cast<uint4*>(Vc);
  if (sh.f32)
    hipLaunchKernelGGL(step_prep_kernel<float>, dim3(sh.B), dim3(kStepThreads), 0, s,
                       static_cast<const float*>(Hn), static_cast<const float*>(r), bias, gate, hidden,
                       sh.G, k4, v4, K4, V4, cache_len, sh.Lmax, row16);
  else
    hipLaunchKernelGGL(step_prep_kernel<bf16_t>, dim3(sh.B), dim3(kStepThreads), 0, s,
                       static_cast<const bf16_t*>(Hn), static_cast<const bf16_t*>(r), bias, gate, hidden,
                       sh.G, k4, v4, K4, V4, cache_len, sh.Lmax, row16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode(sh, p, q, Kc, Vc, cache_len, gate, o, ws, s, nullptr);
}

}  // namespace swi
