// SwiAttn dual-branch prefill on gfx950.
//
// SwiAttn report, section 2 (dual-branch paragraph): the full branch and
// the sliding-window branch share Q, K, V and the output is
// gate * O_FULL + (1 - gate) * O_SWA with a hard 0/1 gate.  The window of
// query i is [i-W+1, i] (weimeta SWA glossary, section "详细解释"), the full
// branch is causal [0, i].
//
// Hard-gate mode (on-device schedule, one attention launch, merge):
//   far_schedule_kernel  cuts the far keys of the gathered gate=1 rows into
//                        work items
//   attn_kernel          far items first: for the gathered rows only, the
//                        far keys [0, i-W] (the full set minus the window)
//                        of one key chunk, written as normalised partials;
//                        then window tiles: the window branch for every
//                        row, written to O with its log-sum-exp (log2)
//   merge_kernel         log-sum-exp merge of window output + far chunks =
//                        O_FULL for the gathered rows, written over their
//                        window output
// The window and far key sets are disjoint and cover [0, i], so the merge is
// the exact full softmax up to rounding.
//
// Global anchors (weimeta SWA glossary, section "SWA 落地的四个常见坑",
// pitfall 1, fix 2): with A > 0 every window-branch query also sees the
// first A keys of its sequence, [0, min(A, i-W+1) - 1].  A window tile then
// walks the anchor blocks before its window blocks (the two masks keep each
// row's key sets disjoint, so a block that falls in both segments is simply
// visited twice with different keys), and the far part of a gate=1 row
// shrinks to [A, i-W].
//
// Per-layer window offsets (weimeta SWA glossary, section
// "两个核心工程参数（W 和步长 S）详解"): with an offset o the window
// of query i is that of query i - o, [max(0, i-o-W+1), i-o] (empty for
// i < o); a gate=1 row still takes all of [0, i], the keys (i-o, i] in its
// window pass (window_row).
//
// Both-branch mode: the same launches with every row taking the full
// branch (no compaction: the far tiles are consecutive positions).  The
// merge then also writes the per-(head, token) squared distance between
// O_FULL and O_SWA, and replaces the window output only where the gate is
// 1; diff_kernel sums the distance over heads (the regulariser paragraph
// of the same section uses this distance).  On request the same pass also
// writes both branch outputs of every row, O_FULL and O_SWA (the router
// gradient's inputs; store_branches and the merge).
#include <atomic>
#include <climits>
#include <type_traits>

#include "attn_core.hpp"
#include "kernels.hpp"

namespace swi {

constexpr int kRows = 128;  // query rows of every tile
constexpr int kTargetItems = 1024;      // far work items aimed for per launch (hard gate)
constexpr int kTargetItemsAll = 4096;   // the same when every row takes the full branch
constexpr int kMinChunkBlocks = 8;  // far chunk is at least 8 x 64 keys
// A hard-gate far chunk is at most kMaxChunkBlocks 64-key blocks (8 MB of
// K and V at d = 128) unless that would need more than kTargetItemsAll
// items: the resident items of an XCD read the same chunk, and longer
// chunks drift apart in that L2 (at gate density 1, 1024 items of about
// 960 blocks each took 5.8 ms against 4.5 ms for the both-branch pass).
constexpr int kMaxChunkBlocks = 256;
constexpr int kSchedThreads = 1024;

struct PrefillArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  const uint8_t* gate;
  const int32_t* idx;
  const int32_t* cnt;
  float* lse_s;     // [B,Hq,N] window-branch normaliser, log2 units
  int32_t* sched;   // far schedule (layout in far_schedule_kernel)
  void* part_o;     // [max_items][kRows][D], input type (normalised far partials)
  float* part_lse;  // [max_items][kRows]
  float* diffp;     // [B,Hq,N] per-head squared distance (both-branch mode)
  float* diff;      // [B,N]
  void* O_full;     // [B,N,Hq,D] both-branch mode, optional: O_FULL of every row
  void* O_swa;      // [B,N,Hq,D] both-branch mode, optional: O_SWA of every row
  int* queue;       // [8] window-tile queue positions (zeroed by the schedule kernel)
  int B, N, Hq, Hkv, G, W;
  int A;    // global anchor keys of the window branch (0 = none)
  int off;  // window offset of the layer: the window of query i is that of query i - off
  int Wf;   // W + off: gate=1 rows take keys [i-off-W+1, i] in the window pass, the far part below
  int HK, HG, hpu, units, tpt_band, tpt_far, band_tiles, far_tiles, max_items;
  int far_grid;  // workgroups of attn_kernel reserved for far items (multiple of 8)
  int band_grid; // workgroups of attn_kernel that work off the window-tile queues
  int cmax;   // width of the per-unit chunk tables
  int all_rows;      // both-branch mode: every row takes the full branch (no idx/cnt)
  int target_items;  // far work items aimed for
  float sl2;  // softmax scale * log2(e)
};

// The rows that take the full branch, per gate group: the compacted gate=1
// positions (hard gate), or every position (both-branch mode).
SWI_DEV int far_count(const PrefillArgs& a, int b, int g) {
  return a.all_rows ? a.N : a.cnt[b * a.G + g];
}
SWI_DEV int far_pos(const PrefillArgs& a, int b, int g, int k) {
  return a.all_rows ? k : a.idx[(int64_t(b) * a.G + g) * a.N + k];
}

// Far-part schedule inside a.sched (int32).  Per (batch, unit) bu the
// gathered rows are cut into nt(bu) active tiles of tpt_far rows; the active
// tiles of all units are laid end to end (active tile x, abase[bu] = first
// one of unit bu).  Tile (bu, t) is cut into chunks of cb 64-key blocks,
// and the items (tile, chunk) are ordered by (unit, chunk, tile), so that
// consecutive items read the same key range of the same KV head: chunk c
// of unit bu holds the tiles from first[bu][c] (the first tile with more
// than c chunks) on, and its items start at off[bu][c], so the item of
// chunk c of tile t is off[bu][c] + t - first[bu][c].
//   [0] items  [1] cb  [2] active tiles  [3] unused
//   item_tile[max_items]   global tile index bu * far_tiles + t of each item
//   item_chunk[max_items]  its chunk
//   meta[nT][4]            per active tile: bu, t, chunks, gathered rows
//   first[nbu][cmax], off[nbu][cmax]
//   abase[nbu + 1], ucnt[nbu], maxc[nbu]  (schedule kernel's own tables when
//                          they do not fit its LDS)
struct SchedView {
  int32_t *item_tile, *item_chunk, *meta, *first, *off, *abase, *ucnt, *maxc;
  SWI_DEV SchedView(const PrefillArgs& a) {
    const int nT = a.B * a.units * a.far_tiles;
    const int nbu = a.B * a.units;
    item_tile = a.sched + 4;
    item_chunk = item_tile + a.max_items;
    meta = item_chunk + a.max_items;
    first = meta + 4 * nT;
    off = first + nbu * a.cmax;
    abase = off + nbu * a.cmax;
    ucnt = abase + nbu + 1;
    maxc = ucnt + nbu;
  }
  // item holding chunk c of tile t of unit bu
  SWI_DEV int item_of(int bu, int t, int c, int cmax) const {
    return off[bu * cmax + c] + (t - first[bu * cmax + c]);
  }
};

// Linear workgroup id -> logical work index so that each of the 8 XCDs (which
// receive workgroups round-robin) runs one contiguous slice of the logical
// order; returns -1 for padding workgroups.
SWI_DEV int xcd_slice(int i, int total) {
  const int per = (total + 7) / 8;
  const int lin = (i & 7) * per + (i >> 3);
  return ((i >> 3) < per && lin < total) ? lin : -1;
}

// Four consecutive values as float, and back.
SWI_DEV f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
SWI_DEV void store4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
SWI_DEV void store4(bf16_t* p, f32x4 v) {
  bf16x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = bf16_t(v[e]);
  *reinterpret_cast<bf16x4*>(p) = o;
}
SWI_DEV f32x4 load4(const bf16_t* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{float(v[0]), float(v[1]), float(v[2]), float(v[3])};
}

// Per-wave bounds used to skip blocks no row of the wave needs and to drop
// the mask inside blocks every row of the wave fully covers.
struct WaveBounds {
  int min_lo, max_hi, max_lo, min_hi;
  // A valid row with an empty range (lo > hi) needs no block but forces the
  // mask everywhere, so it never accumulates keys it does not own.
  SWI_DEV void init(bool valid, int lo, int hi) {
    const bool live = valid && lo <= hi;
    min_lo = wave_min_i(live ? lo : INT_MAX);
    max_hi = wave_max_i(live ? hi : -1);
    max_lo = wave_max_i(valid ? lo : -1);
    min_hi = wave_min_i(valid ? hi : INT_MAX);
  }
  SWI_DEV bool needed(int kb) const { return kb <= max_hi && kb + kBN - 1 >= min_lo; }
  SWI_DEV bool masked(int kb) const { return kb < max_lo || kb + kBN - 1 > min_hi; }
};

// Union of the key intervals of the wave's live rows, for skipping blocks
// and dropping the mask (see WaveBounds).
template <int TPW>
struct TileBounds {
  int min_lo, max_hi;
  WaveBounds wb;
  SWI_DEV void init(const bool (&valid)[TPW], const int (&lo)[TPW], const int (&hi)[TPW]) {
    int a = INT_MAX, b = -1, c = -1, d = INT_MAX;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const bool live = valid[t] && lo[t] <= hi[t];
      a = min(a, live ? lo[t] : INT_MAX);
      b = max(b, live ? hi[t] : -1);
      c = max(c, valid[t] ? lo[t] : -1);
      d = min(d, valid[t] ? hi[t] : INT_MAX);
    }
    min_lo = wave_min_i(a);
    max_hi = wave_max_i(b);
    wb.max_lo = wave_max_i(c);
    wb.min_hi = wave_min_i(d);
  }
  SWI_DEV bool needed(int kb) const { return kb <= max_hi && kb + kBN - 1 >= min_lo; }
  SWI_DEV bool masked(int kb) const { return wb.masked(kb); }
};

// Blocks kb0, kb0+64, ... (nb of them) of one KV head through the core, with
// the global loads of the next two blocks in flight (two register stages,
// used alternately) while a block is computed.
template <typename Core, typename T, int D, int NT, int TPW>
SWI_DEV void block_loop_regs(Core& c, char* lds, const T* Kb, const T* Vb, int64_t rs, int kb0, int nb,
                        int kend, const TileBounds<TPW>& tb, const int (&lo)[TPW],
                        const int (&hi)[TPW], float sl2, int tid, int q, int g) {
  KVLoader<T, D, NT> ld[2];
  ld[0].load(Kb, Vb, rs, kb0, kend, tid);
  if (nb > 1) ld[1].load(Kb, Vb, rs, kb0 + kBN, kend, tid);
  for (int n = 0; n < nb; n += 2) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // stage j holds block n + j
      const int m = n + j;
      if (m >= nb) break;
      const int kb = kb0 + m * kBN;
      __syncthreads();
      ld[j].store(lds, tid);
      __syncthreads();
      if (m + 2 < nb) ld[j].load(Kb, Vb, rs, kb + 2 * kBN, kend, tid);
      if (tb.needed(kb)) c.block(lds, kb, tb.masked(kb), lo, hi, sl2, q, g);
    }
  }
}

// The same with DMA staging (bf16): block m+1 is copied into buffer (m+1)%2
// while block m is computed from the other one.  The wait + barrier at the
// top of each step makes block m's copies (from every wave) visible and
// ensures every wave is done with block m-1, whose buffer the next copy
// then overwrites.
template <typename Core, int D, int NT, int TPW>
SWI_DEV void block_loop_dma(Core& c, char* buf0, char* buf1, const bf16_t* Kb, const bf16_t* Vb,
                            int64_t rs, int kb0, int nb, int kend, const TileBounds<TPW>& tb,
                            const int (&lo)[TPW], const int (&hi)[TPW], float sl2, int tid, int q,
                            int g) {
  using Dma = KVDma<D, NT>;
  Dma::issue(buf0, Kb, Vb, rs, kb0, kend, tid);
  for (int n = 0; n < nb; n += 2) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int m = n + j;
      if (m >= nb) break;
      char* cur = j == 0 ? buf0 : buf1;
      char* nxt = j == 0 ? buf1 : buf0;
      // this wave's copies of block m have landed (the core's LDS reads are
      // invisible to the compiler's wait insertion, so wait explicitly),
      // then every wave's
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (m + 1 < nb) Dma::issue(nxt, Kb, Vb, rs, kb0 + (m + 1) * kBN, kend, tid);
      const int kb = kb0 + m * kBN;
      if (tb.needed(kb)) c.block(cur, kb, tb.masked(kb), lo, hi, sl2, q, g);
    }
  }
}

template <typename Core, typename T, int D, int NT, int TPW>
SWI_DEV void block_loop(Core& c, char* buf0, char* buf1, const T* Kb, const T* Vb, int64_t rs,
                        int kb0, int nb, int kend, const TileBounds<TPW>& tb, const int (&lo)[TPW],
                        const int (&hi)[TPW], float sl2, int tid, int q, int g) {
  if constexpr (TileCfg<T, D>::kDma)
    block_loop_dma<Core, D, NT>(c, buf0, buf1, Kb, Vb, rs, kb0, nb, kend, tb, lo, hi, sl2, tid, q, g);
  else
    block_loop_regs<Core, T, D, NT>(c, buf0, Kb, Vb, rs, kb0, nb, kend, tb, lo, hi, sl2, tid, q, g);
}

// LDS of the window / far work: two DMA buffers (bf16) or one staging
// buffer (float32)
template <typename T, int D>
struct TileLds {
  static constexpr bool kDma = TileCfg<T, D>::kDma;
  static constexpr int kBuf0 = kDma ? LdsDma<D>::kBytes : Lds<T, D>::kBytes;
  static constexpr int kBuf1 = kDma ? LdsDma<D>::kBytes : 16;
};

// Window-pass results of one row that also go to the optional branch
// outputs of both-branch mode: O_SWA of every row, and O_FULL of the rows
// whose window and anchors already hold every key [0, i] (no far part; the
// merge writes O_FULL of the other rows).
template <typename T, int MD>
SWI_DEV void store_branches(const PrefillArgs& a, int b, int tok, int h, const f32x16 (&acc)[MD],
                            float inv, int g) {
  constexpr int D = MD * 32;
  const int64_t row = ((int64_t(b) * a.N + tok) * a.Hq + h) * D;
  if (a.O_swa) store_row<MD>(static_cast<T*>(a.O_swa) + row, acc, inv, g);
  if (a.O_full && tok - a.Wf < a.A) store_row<MD>(static_cast<T*>(a.O_full) + row, acc, inv, g);
}

// Key ranges of one row in the window pass: the window [lo, hi] and the
// anchors [0, ahi].  With a window offset o the window is that of query
// i - o, [max(0, i-o-W+1), i-o] (empty for i < o); a gate=1 row then also
// takes the keys (i-o, i] here, so that its window-pass range [lo, i] and
// its far part [A, lo-1] again cover [0, i] (with the anchors [0, A)).
SWI_DEV void window_row(const PrefillArgs& a, int b, int tok, int h, bool valid, int& lo, int& hi,
                        int& ahi) {
  if (!valid) {
    lo = 0;
    hi = -1;
    ahi = -1;
    return;
  }
  const int p = tok - a.off;
  lo = max(0, p - a.W + 1);
  hi = p;
  if (a.off > 0 && a.gate[(int64_t(b) * a.N + tok) * a.G + h / a.HG] != 0) hi = tok;
  ahi = min(a.A, lo) - 1;  // anchors end where the window starts
}

// Whether a window tile (tokens q0..qlast of KV head kvh) holds a gate=1 row:
// with a window offset its block range then reaches the diagonal.  At most
// 128 (token, gate group) pairs, one ballot per 64; the result is
// wave-uniform.
SWI_DEV bool tile_has_full_row(const PrefillArgs& a, int b, int kvh, int q0, int qlast) {
  const int g0 = kvh * a.HK / a.HG, g1 = (kvh * a.HK + a.HK - 1) / a.HG;
  const int ng = g1 - g0 + 1, n = (qlast - q0 + 1) * ng;
  bool any = false;
  for (int k = threadIdx.x & 63; k < n; k += 64) {
    const int t = q0 + k / ng, g = g0 + k % ng;
    any = any || a.gate[(int64_t(b) * a.N + t) * a.G + g] != 0;
  }
  return __any(any);
}

// Block range of a window tile: the first block holding a window key of
// its first token, through the block holding the last key any row takes
// (at least one block: a tile whose rows all have an empty window visits
// block 0 fully masked).
SWI_DEV void window_blocks(const PrefillArgs& a, int b, int kvh, int q0, int qlast, int& kb0, int& nb) {
  kb0 = (max(0, q0 - a.off - a.W + 1) / kBN) * kBN;
  int last = qlast - a.off;
  if (a.off > 0 && tile_has_full_row(a, b, kvh, q0, qlast)) last = qlast;
  nb = last >= kb0 ? (last - kb0) / kBN + 1 : 1;
}

// ---------------------------------------------------------------------------
// Window branch over every row.  Rows of a tile are tpt_band consecutive
// tokens x the HK query heads of one KV head (128 rows).
// ---------------------------------------------------------------------------
template <typename T, int D>
SWI_DEV void band_tile(const PrefillArgs& a, char* buf0, char* buf1, int lin) {
  using Core = typename TileCfg<T, D>::Core;
  constexpr int NT = TileCfg<T, D>::kWaves * 64;
  constexpr int TPW = Core::TPW;
  const int tile = lin % a.band_tiles;
  const int bk = lin / a.band_tiles;
  const int b = bk / a.Hkv, kvh = bk - b * a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane & 31, g = lane >> 5;
  const int q0 = tile * a.tpt_band;
  const int qlast = min(a.N - 1, q0 + a.tpt_band - 1);
  int tok[TPW], h[TPW], lo[TPW], hi[TPW], alo[TPW], ahi[TPW];
  bool valid[TPW];
  Core c;
  c.init();
  const T* Qp = static_cast<const T*>(a.Q);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int r = wave * (kQR * TPW) + t * kQR + q;
    const int slot = r / a.HK, hh = r - slot * a.HK;
    tok[t] = q0 + slot;
    valid[t] = slot < a.tpt_band && tok[t] < a.N;
    h[t] = kvh * a.HK + hh;
    window_row(a, b, tok[t], h[t], valid[t], lo[t], hi[t], ahi[t]);
    alo[t] = 0;
    c.load_q(t, valid[t] ? Qp + ((int64_t(b) * a.N + tok[t]) * a.Hq + h[t]) * D : nullptr, g);
  }
  TileBounds<TPW> tb;
  tb.init(valid, lo, hi);

  const T* Kb = static_cast<const T*>(a.K) + (int64_t(b) * a.N * a.Hkv + kvh) * D;
  const T* Vb = static_cast<const T*>(a.V) + (int64_t(b) * a.N * a.Hkv + kvh) * D;
  const int64_t rs = int64_t(a.Hkv) * D;
  // anchor blocks first (the last row of the tile has the most anchors)
  const int na = (min(a.A, max(0, qlast - a.off - a.W + 1)) + kBN - 1) / kBN;
  if (na > 0) {
    TileBounds<TPW> tba;
    tba.init(valid, alo, ahi);
    block_loop<Core, T, D, NT>(c, buf0, buf1, Kb, Vb, rs, 0, na, a.N, tba, alo, ahi, a.sl2, tid, q, g);
    __syncthreads();  // every wave is done with the staging buffers
  }
  int kb0, nb;
  window_blocks(a, b, kvh, q0, qlast, kb0, nb);
  block_loop<Core, T, D, NT>(c, buf0, buf1, Kb, Vb, rs, kb0, nb, a.N, tb, lo, hi, a.sl2, tid, q, g);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    float lse2;
    const float inv = finish_row(c.m_of(t), c.l_of(t), lse2);
    if (valid[t]) {
      T* orow = static_cast<T*>(a.O) + ((int64_t(b) * a.N + tok[t]) * a.Hq + h[t]) * D;
      store_row<Core::MD>(orow, c.acc_of(t), inv, g);
      store_branches<T, Core::MD>(a, b, tok[t], h[t], c.acc_of(t), inv, g);
      if (g == 0) a.lse_s[(int64_t(b) * a.Hq + h[t]) * a.N + tok[t]] = lse2;
      if (g == 0 && a.diffp) a.diffp[(int64_t(b) * a.Hq + h[t]) * a.N + tok[t]] = 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// On-device schedule of the far part (one 1024-thread workgroup).
// A far tile is tpt_far consecutive gathered tokens x hpu heads of one unit
// (heads that share both the KV head and the gate group).  Its far keys are
// [0, t_last - W] where t_last is its largest token; the tile is cut into
// chunks of `cb` 64-key blocks, cb chosen so that the launch has about
// target_items chunks in total, with chunks of at most kMaxChunkBlocks
// blocks while that needs no more than kTargetItemsAll items.
// ---------------------------------------------------------------------------
SWI_DEV int block_excl_scan(int v, int* sh, int& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int nw = blockDim.x / 64;
    const int x = lane < nw ? sh[lane] : 0;
    int w = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(w, o, 64);
      if (lane >= o) w += t;
    }
    if (lane < nw) sh[lane] = w - x;
    if (lane == nw - 1) sh[32] = w;
  }
  __syncthreads();
  const int res = sh[wave] + incl - v;
  total = sh[32];
  __syncthreads();
  return res;
}

// The schedule kernel keeps its tables in LDS when they fit (the per-unit
// ones up to kSchedUnits units, the (unit, chunk) ones up to kSchedLds
// entries) and in the workspace otherwise.  Work is spread over the active
// tiles only; each pass issues the position loads of all its tiles before
// using them.
constexpr int kSchedLds = 4096;    // ints per (unit, chunk) table in LDS
constexpr int kSchedUnits = 1024;  // (batch, unit) entries of the per-unit tables in LDS
constexpr int kSchedPer = 4;       // active tiles a thread takes per round

__global__ __launch_bounds__(kSchedThreads) void far_schedule_kernel(PrefillArgs a) {
  __shared__ int scan_sh[33];
  __shared__ long long red[kSchedThreads / 64];
  __shared__ int cb_sh;
  __shared__ int first_sh[kSchedLds], off_sh[kSchedLds];
  __shared__ int abase_sh[kSchedUnits + 1], ucnt_sh[kSchedUnits], maxc_sh[kSchedUnits];
  SchedView sv(a);
  const int tid = threadIdx.x;
  const int nbu = a.B * a.units, TT = a.far_tiles, cmax = a.cmax;
  const int ntab = nbu * cmax;
  const bool u_lds = nbu <= kSchedUnits;
  const bool t_lds = ntab <= kSchedLds;
  int* abase = u_lds ? abase_sh : sv.abase;
  int* ucnt = u_lds ? ucnt_sh : sv.ucnt;
  int* maxc = u_lds ? maxc_sh : sv.maxc;
  int* first = t_lds ? first_sh : sv.first;
  int* off = t_lds ? off_sh : sv.off;
  if (tid < 8) a.queue[tid] = 0;
  // gathered rows and active tiles of each unit, and their prefix
  int NA = 0;
  for (int x0 = 0; x0 < nbu; x0 += kSchedThreads) {
    const int bu = x0 + tid;
    int nt = 0;
    if (bu < nbu) {
      const int b = bu / a.units, u = bu - b * a.units;
      const int c = far_count(a, b, (u * a.hpu) / a.HG);
      ucnt[bu] = c;
      maxc[bu] = 0;
      nt = (c + a.tpt_far - 1) / a.tpt_far;
    }
    int tot;
    const int ex = block_excl_scan(nt, scan_sh, tot);
    if (bu < nbu) abase[bu] = NA + ex;
    NA += tot;
  }
  if (tid == 0) abase[nbu] = NA;
  __syncthreads();
  // unit of active tile x: the last unit whose first active tile is <= x
  const auto unit_of = [&](int x) {
    int lo = 0, hi = nbu - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (abase[mid] <= x) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  // position of the last gathered row of tile (bu, t) (a memory load)
  const auto last_pos = [&](int bu, int t) {
    const int b = bu / a.units, u = bu - b * a.units;
    const int ntok = min(a.tpt_far, ucnt[bu] - t * a.tpt_far);
    return far_pos(a, b, (u * a.hpu) / a.HG, t * a.tpt_far + ntok - 1);
  };
  // 64-key blocks of far keys [A, pos - W - off] (none when empty)
  const auto blocks_of = [&](int pos) {
    const int fh = pos - a.Wf;
    return fh >= a.A ? fh / kBN - a.A / kBN + 1 : 0;
  };
  // pass 1: total blocks, then the chunk size
  long long mine = 0;
  for (int x0 = 0; x0 < NA; x0 += kSchedPer * kSchedThreads) {
    int pos[kSchedPer];
#pragma unroll
    for (int j = 0; j < kSchedPer; ++j) {
      const int x = x0 + j * kSchedThreads + tid;
      pos[j] = -1;
      if (x < NA) {
        const int bu = unit_of(x);
        pos[j] = last_pos(bu, x - abase[bu]);
      }
    }
#pragma unroll
    for (int j = 0; j < kSchedPer; ++j) mine += pos[j] >= 0 ? blocks_of(pos[j]) : 0;
  }
  for (int o = 32; o >= 1; o >>= 1) mine += __shfl_xor(mine, o, 64);
  if ((tid & 63) == 0) red[tid >> 6] = mine;
  __syncthreads();
  if (tid == 0) {
    long long total = 0;
    for (int w = 0; w < kSchedThreads / 64; ++w) total += red[w];
    const auto cdiv = [](long long x, long long y) {
      return x + y - 1 < INT_MAX ? (long long)(unsigned(x + y - 1) / unsigned(y)) : (x + y - 1) / y;
    };
    const long long c = cdiv(total, a.target_items);
    const long long cap = max<long long>(kMaxChunkBlocks, cdiv(total, kTargetItemsAll));
    cb_sh = int(max<long long>(kMinChunkBlocks, min(c, cap)));
  }
  __syncthreads();
  const int cb = cb_sh;
  // pass 2: chunks of every active tile (meta), the first tile holding chunk
  // c (chunks step up at tile t for c in [chunks(t-1), chunks(t))), and the
  // chunks of each unit's last tile
  for (int x0 = 0; x0 < NA; x0 += kSchedPer * kSchedThreads) {
    int pos[kSchedPer], prv[kSchedPer], bus[kSchedPer];
#pragma unroll
    for (int j = 0; j < kSchedPer; ++j) {
      const int x = x0 + j * kSchedThreads + tid;
      pos[j] = prv[j] = -1;
      bus[j] = 0;
      if (x < NA) {
        const int bu = unit_of(x), t = x - abase[bu];
        bus[j] = bu;
        pos[j] = last_pos(bu, t);
        if (t > 0) prv[j] = last_pos(bu, t - 1);
      }
    }
#pragma unroll
    for (int j = 0; j < kSchedPer; ++j) {
      const int x = x0 + j * kSchedThreads + tid;
      if (x >= NA) continue;
      const int bu = bus[j], t = x - abase[bu];
      const int n = (blocks_of(pos[j]) + cb - 1) / cb;
      const int np = prv[j] >= 0 ? (blocks_of(prv[j]) + cb - 1) / cb : 0;
      for (int c = np; c < n; ++c) first[bu * cmax + c] = t;
      if (t == abase[bu + 1] - abase[bu] - 1) maxc[bu] = n;
      int32_t* m = sv.meta + 4 * int64_t(x);
      m[0] = bu;
      m[1] = t;
      m[2] = n;
      m[3] = min(a.tpt_far, ucnt[bu] - t * a.tpt_far);
    }
  }
  __syncthreads();
  // pass 3: first item of each (unit, chunk): an exclusive scan over the flat
  // table of the chunk sizes (tiles from first[bu][c] to the unit's last)
  int items = 0;
  for (int x0 = 0; x0 < ntab; x0 += kSchedThreads) {
    const int x = x0 + tid;
    int val = 0;
    if (x < ntab) {
      const int bu = x / cmax, c = x - bu * cmax;
      if (c < maxc[bu]) val = abase[bu + 1] - abase[bu] - first[x];
    }
    int tot;
    const int ex = block_excl_scan(val, scan_sh, tot);
    if (x < ntab) off[x] = items + ex;
    items += tot;
  }
  __syncthreads();
  // pass 4: the item list
  for (int x = tid; x < NA; x += kSchedThreads) {
    const int32_t* m = sv.meta + 4 * int64_t(x);
    const int bu = m[0], t = m[1], n = m[2];
    for (int c = 0; c < n; ++c) {
      const int it = off[bu * cmax + c] + t - first[bu * cmax + c];
      if (it >= a.max_items) continue;  // cannot happen: the plan's bound
      sv.item_tile[it] = bu * TT + t;
      sv.item_chunk[it] = c;
    }
  }
  // the tables the merge reads, and the counts
  if (t_lds)
    for (int x = tid; x < ntab; x += kSchedThreads) {
      sv.first[x] = first_sh[x];
      sv.off[x] = off_sh[x];
    }
  if (tid == 0) {
    a.sched[0] = min(items, a.max_items);
    a.sched[1] = cb;
    a.sched[2] = NA;
  }
}

// ---------------------------------------------------------------------------
// Far part of the full branch for gathered rows: keys [A, i-W-off] (the full
// set minus the window pass's keys and the anchors).  One workgroup per work item (tile,
// chunk); grid = upper bound, idle workgroups exit at once.
// Every item, also the only chunk of a tile, writes its normalised partial
// output and log-sum-exp; merge_kernel combines them with the window
// result.
// ---------------------------------------------------------------------------
template <typename T, int D>
SWI_DEV void far_item(const PrefillArgs& a, char* buf0, char* buf1, int item) {
  using Core = typename TileCfg<T, D>::Core;
  constexpr int NT = TileCfg<T, D>::kWaves * 64;
  constexpr int TPW = Core::TPW;
  SchedView sv(a);
  const int cb = a.sched[1];
  const int T_ = sv.item_tile[item], ch = sv.item_chunk[item];
  const int per_b = a.units * a.far_tiles;
  const int b = T_ / per_b, rem = T_ - b * per_b;
  const int u = rem / a.far_tiles, t_ = rem - u * a.far_tiles;
  const int g_gate = (u * a.hpu) / a.HG;
  const int kvh = (u * a.hpu) / a.HK;
  const int cnt = far_count(a, b, g_gate);
  const int ntok = min(a.tpt_far, cnt - t_ * a.tpt_far);
  const int far_hi = far_pos(a, b, g_gate, t_ * a.tpt_far + ntok - 1) - a.Wf;
  const int fb = (a.A / kBN) * kBN;  // block holding the first far key A
  const int c0 = fb + ch * cb * kBN;
  const int c1 = min(far_hi + 1, fb + (ch + 1) * cb * kBN);  // keys [c0, c1)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane & 31, g = lane >> 5;
  int r[TPW], tok[TPW], h[TPW], lo[TPW], hi[TPW];
  bool valid[TPW];
  Core c;
  c.init();
  const T* Qp = static_cast<const T*>(a.Q);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    r[t] = wave * (kQR * TPW) + t * kQR + q;
    const int slot = r[t] / a.hpu, hh = r[t] - slot * a.hpu;
    valid[t] = slot < ntok;
    tok[t] = valid[t] ? far_pos(a, b, g_gate, t_ * a.tpt_far + slot) : 0;
    h[t] = u * a.hpu + hh;
    lo[t] = max(c0, a.A);
    hi[t] = valid[t] ? min(tok[t] - a.Wf, c1 - 1) : -1;
    c.load_q(t, valid[t] ? Qp + ((int64_t(b) * a.N + tok[t]) * a.Hq + h[t]) * D : nullptr, g);
  }
  TileBounds<TPW> tb;
  tb.init(valid, lo, hi);
  const T* Kb = static_cast<const T*>(a.K) + (int64_t(b) * a.N * a.Hkv + kvh) * D;
  const T* Vb = static_cast<const T*>(a.V) + (int64_t(b) * a.N * a.Hkv + kvh) * D;
  const int64_t rs = int64_t(a.Hkv) * D;
  block_loop<Core, T, D, NT>(c, buf0, buf1, Kb, Vb, rs, c0, (c1 - c0 + kBN - 1) / kBN, c1, tb, lo, hi,
                             a.sl2, tid, q, g);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    float lse2;
    const float inv = finish_row(c.m_of(t), c.l_of(t), lse2);
    if (!valid[t]) continue;
    T* prow = static_cast<T*>(a.part_o) + (int64_t(item) * kRows + r[t]) * D;
    store_row<Core::MD>(prow, c.acc_of(t), inv, g);
    if (g == 0) a.part_lse[int64_t(item) * kRows + r[t]] = lse2;
  }
}

// ---------------------------------------------------------------------------
// Persistent window workers (DMA path).  The window tiles, ordered by
// (sequence, tile, KV head), are split into 8 queues, queue x holding the
// x-th eighth of them (one token range of every KV head: neighbouring tiles
// of a head share most of their keys in that XCD's L2); a worker
// takes tiles from the queue of its XCD and moves on to the others when it
// runs dry.  Every position of every queue is handed out once (atomic
// counters, zeroed by the schedule kernel that precedes the launch).
// Across tiles the block stream continues without a pipeline restart: the
// next tile id is claimed four blocks before the current tile ends and
// published two blocks before it ends, the copy of its first K/V block is issued during the
// last block of the current tile, and its queries are loaded right after
// that block's score MFMAs.
// ---------------------------------------------------------------------------
struct TileQueue {
  int n, per;
  SWI_DEV int len(int x) const { return min(per, max(0, n - x * per)); }
};
// Claims on the tile queues (one thread).  The counters are shared by
// workgroups on all XCDs, whose L2 caches are not coherent with each other:
// the increments are made at system scope, which performs them past the
// L2s, and their results take a memory round trip.  A claim is therefore
// split: claim() issues the increment on queue x and returns the raw
// position without waiting for it; resolve(), a block or more later (the
// block barriers have drained the increment by then), turns it into a tile,
// or, if queue x ran dry, reads all 8 counters at once (one round trip) and
// claims, in turn, only from queues that still had tiles: a counter only
// grows, so a queue seen dry stays dry and skipping it loses no tile.  (A
// claim on each other queue in turn cost up to seven contended round trips
// at the end of every worker's last tile.)  That path is kept out of line,
// so that it does not weigh on the register allocation of the block loop.
SWI_DEV int claim(int* queue, int x) {
  return __hip_atomic_fetch_add(queue + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __attribute__((noinline)) int steal(int* queue, int n, int per, int x) {
  TileQueue tq;
  tq.n = n;
  tq.per = per;
  int seen[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    seen[k] = __hip_atomic_load(queue + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  for (int k = 1; k < 8; ++k) {
    const int y = (x + k) & 7;
    if (seen[y] >= tq.len(y)) continue;
    const int q = claim(queue, y);
    if (q < tq.len(y)) return y * tq.per + q;
  }
  return -1;
}
SWI_DEV int resolve(int* queue, const TileQueue& tq, int& x, int p) {
  if (p < tq.len(x)) return x * tq.per + p;
  const int lin = steal(queue, tq.n, tq.per, x);
  if (lin >= 0) x = lin / tq.per;
  return lin;
}

// Window tile lin: tpt_band consecutive tokens x the HK heads of one KV head.
// Its blocks: na anchor blocks [0, 64 na), then nb window blocks from kb0.
// kAnch = false compiles the anchor-free stream (na = 0 is a constant).
template <bool kAnch>
struct BandTile {
  int b, kvh, q0, kb0, nb, na;
  SWI_DEV void set(const PrefillArgs& a, int lin) {
    // KV heads fastest: an XCD's resident workers cover one token range of
    // every KV head of the sequence
    kvh = lin % a.Hkv;
    const int bt = lin / a.Hkv;
    b = bt / a.band_tiles;
    const int tile = bt - b * a.band_tiles;
    q0 = tile * a.tpt_band;
    const int qlast = min(a.N - 1, q0 + a.tpt_band - 1);
    window_blocks(a, b, kvh, q0, qlast, kb0, nb);
    na = kAnch ? (min(a.A, max(0, qlast - a.off - a.W + 1)) + kBN - 1) / kBN : 0;
  }
  SWI_DEV int anchors() const { return kAnch ? na : 0; }
  SWI_DEV int total() const { return anchors() + nb; }
  SWI_DEV int kb(int n) const { return n < anchors() ? n * kBN : kb0 + (n - anchors()) * kBN; }
};

template <typename T, int D, bool kAnch>
SWI_DEV void band_worker(const PrefillArgs& a, char* buf0, char* buf1) {
  using Core = typename TileCfg<T, D>::Core;
  constexpr int NT = TileCfg<T, D>::kWaves * 64;
  using Dma = KVDma<D, NT>;
  __shared__ int s_next;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane & 31, g = lane >> 5;
  TileQueue tq;
  tq.n = a.band_tiles * a.B * a.Hkv;
  tq.per = (tq.n + 7) / 8;
  int qx = blockIdx.x & 7;  // workgroups are dealt to the 8 XCDs in turn
  if (tid == 0) s_next = resolve(a.queue, tq, qx, claim(a.queue, qx));
  __syncthreads();
  int lin = __builtin_amdgcn_readfirstlane(s_next);
  if (lin < 0) return;
  // this lane's row inside any tile
  const int r = wave * kQR + q, slot = r / a.HK, hh = r - slot * a.HK;
  const T* Qp = static_cast<const T*>(a.Q);
  const int64_t rs = int64_t(a.Hkv) * D;
  using BandTile = swi::BandTile<kAnch>;
  auto qrow = [&](const BandTile& t) -> const T* {
    const int tok = t.q0 + slot;
    const bool v = slot < a.tpt_band && tok < a.N;
    return v ? Qp + ((int64_t(t.b) * a.N + tok) * a.Hq + t.kvh * a.HK + hh) * D : nullptr;
  };
  auto kv_off = [&](const BandTile& t) { return (int64_t(t.b) * a.N * a.Hkv + t.kvh) * D; };
  BandTile t;
  t.set(a, lin);
  Core c;
  c.init();
  c.load_q(0, qrow(t), g);
  Dma::issue(buf0, static_cast<const T*>(a.K) + kv_off(t), static_cast<const T*>(a.V) + kv_off(t), rs,
             t.kb(0), a.N, tid);
  int s = 0;  // blocks streamed so far: block s sits in buffer s % 2
  int next_raw = 0;  // thread 0: raw position of the pending claim on queue qx
  bool q_pref = false;
  while (true) {
    const int tok = t.q0 + slot;
    const bool valid = slot < a.tpt_band && tok < a.N;
    int lo, hi, ahi;  // window [lo, hi], anchors [0, ahi]
    window_row(a, t.b, tok, t.kvh * a.HK + hh, valid, lo, hi, ahi);
    TileBounds<1> tb, tba;
    {
      const bool v1[1] = {valid};
      const int l1[1] = {lo}, h1[1] = {hi};
      tb.init(v1, l1, h1);
      if (t.anchors() > 0) {
        const int l0[1] = {0}, h0[1] = {ahi};
        tba.init(v1, l0, h0);
      }
    }
    const T* Kb = static_cast<const T*>(a.K) + kv_off(t);
    const T* Vb = static_cast<const T*>(a.V) + kv_off(t);
    // the next tile is claimed at step cl, its id resolved and published at
    // step pub and read one barrier later (the claim is issued only a few
    // blocks before the tile ends: claimed a whole tile ahead, the first
    // workers to start took two tiles each when there are barely more tiles
    // than workers, and the workers that started later found no tile)
    const int nbt = t.total();
    const int pub = nbt >= 2 ? nbt - 2 : 0;
    const int rd = nbt >= 2 ? pub + 1 : 0;
    const int cl = pub >= 2 ? pub - 2 : 0;
    int nlin = -1;
    BandTile nt;
    nt.set(a, 0);
    for (int n = 0; n < nbt; ++n, ++s) {
      char* cur = (s & 1) ? buf1 : buf0;
      char* nxt = (s & 1) ? buf0 : buf1;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (n == cl && tid == 0) next_raw = claim(a.queue, qx);
      if (n == pub && tid == 0) s_next = resolve(a.queue, tq, qx, next_raw);
      if (nbt < 2) __syncthreads();
      if (n == rd) {
        nlin = __builtin_amdgcn_readfirstlane(s_next);
        if (nlin >= 0) nt.set(a, nlin);
      }
      if (n + 1 < nbt)
        Dma::issue(nxt, Kb, Vb, rs, t.kb(n + 1), a.N, tid);
      else if (nlin >= 0)
        Dma::issue(nxt, static_cast<const T*>(a.K) + kv_off(nt), static_cast<const T*>(a.V) + kv_off(nt),
                   rs, nt.kb(0), a.N, tid);
      const int kb = t.kb(n);
      const bool anc = n < t.anchors();  // wave-uniform
      if (!(anc ? tba.needed(kb) : tb.needed(kb))) continue;
      // last block of the tile: the next tile's queries follow its scores
      const bool pre = n + 1 == nbt && nlin >= 0;
      const bool msk = anc ? tba.masked(kb) : tb.masked(kb);
      c.block_hook(cur, kb, msk, anc ? 0 : lo, anc ? ahi : hi, a.sl2, q, g, [&]() {
        if (pre) c.c.load_q(qrow(nt), g);
      });
      q_pref = q_pref || pre;
    }
    // tile finished: output and window normaliser
    float lse2;
    const float inv = finish_row(c.m_of(0), c.l_of(0), lse2);
    if (valid) {
      const int h = t.kvh * a.HK + hh;
      T* orow = static_cast<T*>(a.O) + ((int64_t(t.b) * a.N + tok) * a.Hq + h) * D;
      store_row<Core::MD>(orow, c.acc_of(0), inv, g);
      store_branches<T, Core::MD>(a, t.b, tok, h, c.acc_of(0), inv, g);
      if (g == 0) a.lse_s[(int64_t(t.b) * a.Hq + h) * a.N + tok] = lse2;
      if (g == 0 && a.diffp) a.diffp[(int64_t(t.b) * a.Hq + h) * a.N + tok] = 0.f;
    }
    if (nlin < 0) break;
    lin = nlin;
    t = nt;
    c.init();
    if (!q_pref) c.load_q(0, qrow(t), g);
    q_pref = false;
  }
}

// ---------------------------------------------------------------------------
// Window tiles and far items in one launch.  Workgroups [0, far_grid) take
// far items (an XCD takes a contiguous slice of the (unit, chunk, tile)
// order, so its resident workgroups read the same keys of one KV head);
// the rest take window tiles (consecutive tiles of one KV head share most
// of their window, so they too stay on one XCD's L2).  Workgroups start in
// index order, so the long far items start first and the shorter window
// tiles fill the tail of the launch.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__((TileCfg<T, D>::kWaves * 64), (TileCfg<T, D>::kMinWG)) void attn_kernel(PrefillArgs a) {
  __shared__ __align__(16) char buf0[TileLds<T, D>::kBuf0];
  __shared__ __align__(16) char buf1[TileLds<T, D>::kBuf1];
  if (int(blockIdx.x) < a.far_grid) {
    const int item = xcd_slice(blockIdx.x, a.sched[0]);
    if (item >= 0) far_item<T, D>(a, buf0, buf1, item);
    return;
  }
  if constexpr (TileCfg<T, D>::kDma) {
    if (a.A > 0)
      band_worker<T, D, true>(a, buf0, buf1);
    else
      band_worker<T, D, false>(a, buf0, buf1);
  } else {
    const int lin = xcd_slice(blockIdx.x - a.far_grid, a.band_tiles * a.B * a.Hkv);
    if (lin >= 0) band_tile<T, D>(a, buf0, buf1, lin);
  }
}

// Sum of squared differences of n channels.  Contraction is off so that
// each difference is taken between the two rounded values.
template <int n>
SWI_DEV float sq_distance(const float (&x)[n], const float (&y)[n]) {
#pragma clang fp contract(off)
  float dd = 0.f;
#pragma unroll
  for (int i = 0; i < n; ++i) {
    const float e = x[i] - y[i];
    dd += e * e;
  }
  return dd;
}

// ---------------------------------------------------------------------------
// Merge of the far tiles.  Work units are (active tile, quarter of its
// rows), taken by a fixed grid (tiles without chunks are skipped); the
// schedule's record of the tile and its (unit, chunk) tables give the items
// of its chunks, so a unit needs three rounds of dependent loads (record;
// row positions and item numbers; partials and window output).  8 threads
// share a
// row, each with D/8 consecutive channels, so that many independent loads
// are in flight (one thread per row walking its chunks one after another
// left the kernel bound by load latency).  O_FULL of a row is the
// log-sum-exp weighted sum of its window output and its chunks' partials,
// taken in chunk order.  In both-branch mode every row is merged: the
// per-head squared distance between O_FULL and the window output is
// written, and O_FULL replaces the window output only where the gate is 1.
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = 256;
constexpr int kMergeTPR = 8;  // threads per row
constexpr int kMergeBatch = 4;  // chunks whose loads are in flight together
template <typename T, int D, bool kBoth>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(PrefillArgs a) {
  constexpr int kRowsWG = kMergeThreads / kMergeTPR;  // rows per work unit
  constexpr int kParts = kRows / kRowsWG;
  constexpr int CPT = D / kMergeTPR;  // channels per thread
  SchedView sv(a);
  const int na = a.sched[2];
  const int rr = threadIdx.x / kMergeTPR, c0 = (threadIdx.x % kMergeTPR) * CPT;
  for (int w = blockIdx.x; w < na * kParts; w += gridDim.x) {
    const int32_t* m = sv.meta + 4 * int64_t(w / kParts);
    const int bu = m[0], t = m[1], ni = m[2], ntok = m[3];
    if (ni == 0) continue;
    const int r = (w % kParts) * kRowsWG + rr;
    const int b = bu / a.units, u = bu - b * a.units;
    const int g_gate = (u * a.hpu) / a.HG;
    const int slot = r / a.hpu, hh = r - slot * a.hpu;
    // (the 8 threads of a row take every branch together)
    if (slot >= ntok) continue;
    const int tok = far_pos(a, b, g_gate, t * a.tpt_far + slot);
    if (tok - a.Wf < a.A) continue;  // no far keys: the window pass already holds O_FULL
    const int h = u * a.hpu + hh;
    const float ls = a.lse_s[(int64_t(b) * a.Hq + h) * a.N + tok];
    T* orow = static_cast<T*>(a.O) + ((int64_t(b) * a.N + tok) * a.Hq + h) * D + c0;
    float os[CPT], o[CPT];
#pragma unroll
    for (int i4 = 0; i4 < CPT / 4; ++i4) {
      const f32x4 v = load4(orow + i4 * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) os[i4 * 4 + e] = o[i4 * 4 + e] = v[e];
    }
    // chunks in batches of kMergeBatch with all their loads in flight: the
    // running maximum M starts at the window's normaliser and is raised once
    // per batch (weights 2^(lse - M) on the normalised partial outputs)
    float M = ls, wsum = 1.f;
    for (int k0 = 0; k0 < ni; k0 += kMergeBatch) {
      int it[kMergeBatch];
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) it[j] = k0 + j < ni ? sv.item_of(bu, t, k0 + j, a.cmax) : -1;
      // partials kept in their stored type until they are summed
      using R4 = std::conditional_t<std::is_same_v<T, float>, f32x4, bf16x4>;
      float lk[kMergeBatch];
      R4 pv[kMergeBatch][CPT / 4];
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) {
        lk[j] = kNegInf;
        if (it[j] < 0) continue;
        lk[j] = a.part_lse[int64_t(it[j]) * kRows + r];
        const T* prow = static_cast<const T*>(a.part_o) + (int64_t(it[j]) * kRows + r) * D + c0;
#pragma unroll
        for (int i4 = 0; i4 < CPT / 4; ++i4) pv[j][i4] = *reinterpret_cast<const R4*>(prow + i4 * 4);
      }
      float mb = M;
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) mb = fmaxf(mb, lk[j]);
      const float sc = mb == kNegInf ? 1.f : fast_exp2(M - mb);
      wsum *= sc;
#pragma unroll
      for (int e = 0; e < CPT; ++e) o[e] *= sc;
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) {
        if (it[j] < 0) continue;
        const float wk = lk[j] == kNegInf ? 0.f : fast_exp2(lk[j] - mb);
        wsum += wk;
#pragma unroll
        for (int i4 = 0; i4 < CPT / 4; ++i4)
#pragma unroll
          for (int e = 0; e < 4; ++e) o[i4 * 4 + e] = fmaf(wk, float(pv[j][i4][e]), o[i4 * 4 + e]);
      }
      M = mb;
    }
    const float inv = 1.f / wsum;
#pragma unroll
    for (int e = 0; e < CPT; ++e) o[e] *= inv;
    bool write = true;
    if constexpr (kBoth) {
      // squared distance to the window output, summed over the row's 8
      // threads (lanes 8k .. 8k+7 of the wave) in a fixed order
      float dd = sq_distance<CPT>(o, os);
      dd += __shfl_xor(dd, 1, kMergeTPR);
      dd += __shfl_xor(dd, 2, kMergeTPR);
      dd += __shfl_xor(dd, 4, kMergeTPR);
      if (c0 == 0) a.diffp[(int64_t(b) * a.Hq + h) * a.N + tok] = dd;
      write = a.gate[(int64_t(b) * a.N + tok) * a.G + h / a.HG] != 0;
    }
    if (write) {
#pragma unroll
      for (int i4 = 0; i4 < CPT / 4; ++i4)
        store4(orow + i4 * 4, f32x4{o[i4 * 4], o[i4 * 4 + 1], o[i4 * 4 + 2], o[i4 * 4 + 3]});
    }
    if (kBoth && a.O_full) {
      T* frow = static_cast<T*>(a.O_full) + ((int64_t(b) * a.N + tok) * a.Hq + h) * D + c0;
#pragma unroll
      for (int i4 = 0; i4 < CPT / 4; ++i4)
        store4(frow + i4 * 4, f32x4{o[i4 * 4], o[i4 * 4 + 1], o[i4 * 4 + 2], o[i4 * 4 + 3]});
    }
  }
}

// diff[b,t] = sum over heads (in head order) of the per-head distances
__global__ __launch_bounds__(256) void diff_kernel(PrefillArgs a) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(a.B) * a.N) return;
  const int b = int(i / a.N), t = int(i - int64_t(b) * a.N);
  float s = 0.f;
  for (int h = 0; h < a.Hq; ++h) s += a.diffp[(int64_t(b) * a.Hq + h) * a.N + t];
  a.diff[i] = s;
}

// ---------------------------------------------------------------------------
static size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Compute units of the current device (queried once per device).
static hipError_t compute_units(int* n) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && cache[dev].load() > 0) {
    *n = cache[dev].load();
    return hipSuccess;
  }
  e = hipDeviceGetAttribute(n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (*n < 1) *n = 1;
  if (dev >= 0 && dev < 64) cache[dev].store(*n);
  return hipSuccess;
}

bool plan_prefill(const PrefillShape& sh, PrefillPlan* p) {
  p->HK = sh.Hq / sh.Hkv;
  p->HG = sh.Hq / sh.G;
  p->hpu = p->HK < p->HG ? p->HK : p->HG;
  p->units = sh.Hq / p->hpu;
  p->tpt_band = kRows / p->HK;
  p->tpt_far = kRows / p->hpu;
  p->band_tiles = (sh.N + p->tpt_band - 1) / p->tpt_band;
  p->far_tiles = (sh.N + p->tpt_far - 1) / p->tpt_far;
  const long long nT = (long long)sh.B * p->units * p->far_tiles;
  p->target_items = sh.both_branch ? kTargetItemsAll : kTargetItems;
  // Item bound.  The schedule cuts chunks of cb = max(8, min(c, cap))
  // blocks, c = ceil(total / target), cap = max(kMaxChunkBlocks,
  // ceil(total / kTargetItemsAll)), so total / cb <= kTargetItemsAll, and
  // total / cb <= target while c <= kMaxChunkBlocks; a tile adds at most one
  // partial chunk.  A tile has at most N / 64 + 1 far blocks, so when
  // nT (N / 64 + 1) <= kMaxChunkBlocks target no gate can need more than
  // target + nT items.  The far grid is sized by this bound, and its idle
  // workgroups delay the window workers behind them (about 15 us for 4320
  // of them at N = 4096).
  const long long bmax = sh.N / kBN + 1;
  const long long lim =
      nT * bmax <= (long long)kMaxChunkBlocks * p->target_items ? p->target_items : kTargetItemsAll;
  const long long max_items = lim + nT;
  if (max_items > INT_MAX / kRows) return false;
  p->max_items = int(max_items);
  // chunks per tile <= ceil(ceil(N / 64) / kMinChunkBlocks)
  p->cmax = ((sh.N + kBN - 1) / kBN + kMinChunkBlocks - 1) / kMinChunkBlocks + 1;
  const size_t rowsN = size_t(sh.B) * sh.Hq * sh.N;
  size_t off = 0;
  p->off_lse = off;
  off = align_up(off + rowsN * 4);
  p->off_sched = off;
  const size_t nbu = size_t(sh.B) * p->units;
  const size_t sched_ints = 4 + 2 * size_t(max_items) + 4 * size_t(nT) + 2 * nbu * p->cmax + 3 * nbu + 1;
  off = align_up(off + sched_ints * 4);
  p->off_queue = off;
  off = align_up(off + 8 * 4);
  p->off_part_o = off;
  off = align_up(off + size_t(max_items) * kRows * sh.d * (sh.f32 ? 4 : 2));
  p->off_part_lse = off;
  off = align_up(off + size_t(max_items) * kRows * 4);
  p->off_diffp = 0;
  if (sh.both_branch) {
    p->off_diffp = off;
    off = align_up(off + rowsN * 4);
  }
  p->bytes = off;
  return true;
}

template <typename T, int D>
static hipError_t run_prefill(const PrefillShape& sh, const PrefillPlan& p, PrefillArgs& a,
                              hipStream_t s, void* const* ev) {
  hipError_t e;
#define SWI_TRY(x)                    \
  if ((e = (x)) != hipSuccess) return e;
  SWI_TRY(mark(ev, 0, s));
  hipLaunchKernelGGL(far_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, s, a);
  SWI_TRY(hipGetLastError());
  SWI_TRY(mark(ev, 1, s));
  constexpr int nt = TileCfg<T, D>::kWaves * 64;
  const int band_total = p.band_tiles * sh.B * sh.Hkv;
  int cus = 0;
  SWI_TRY(compute_units(&cus));
  if (TileCfg<T, D>::kDma) {  // resident window workers: kMinWG per CU
    const int workers = TileCfg<T, D>::kMinWG * cus;
    a.band_grid = band_total < workers ? band_total : workers;
  } else {
    a.band_grid = band_total;
  }
  hipLaunchKernelGGL((attn_kernel<T, D>), dim3(a.far_grid + 8 * ((a.band_grid + 7) / 8)), dim3(nt), 0,
                     s, a);
  SWI_TRY(hipGetLastError());
  SWI_TRY(mark(ev, 2, s));
  if (sh.both_branch)
    hipLaunchKernelGGL((merge_kernel<T, D, true>), dim3(8 * cus), dim3(kMergeThreads), 0, s, a);
  else
    hipLaunchKernelGGL((merge_kernel<T, D, false>), dim3(8 * cus), dim3(kMergeThreads), 0, s, a);
  SWI_TRY(hipGetLastError());
  SWI_TRY(mark(ev, 3, s));
  if (sh.both_branch) {
    const long long n = (long long)sh.B * sh.N;
    hipLaunchKernelGGL(diff_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, a);
    SWI_TRY(hipGetLastError());
    SWI_TRY(mark(ev, 4, s));
  }
#undef SWI_TRY
  return hipSuccess;
}

hipError_t launch_prefill(const PrefillShape& sh, const PrefillPlan& p, const void* Q,
                          const void* K, const void* V, const uint8_t* gate, const int32_t* idx,
                          const int32_t* cnt, void* O, float* diff, void* ws, hipStream_t s,
                          void* const* ev, void* O_full, void* O_swa) {
  char* w = static_cast<char*>(ws);
  PrefillArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.gate = gate;
  a.idx = idx;
  a.cnt = cnt;
  a.lse_s = reinterpret_cast<float*>(w + p.off_lse);
  a.sched = reinterpret_cast<int32_t*>(w + p.off_sched);
  a.queue = reinterpret_cast<int*>(w + p.off_queue);
  a.part_o = static_cast<void*>(w + p.off_part_o);
  a.part_lse = reinterpret_cast<float*>(w + p.off_part_lse);
  a.diffp = sh.both_branch ? reinterpret_cast<float*>(w + p.off_diffp) : nullptr;
  a.all_rows = sh.both_branch ? 1 : 0;
  a.target_items = p.target_items;
  a.diff = diff;
  a.O_full = sh.both_branch ? O_full : nullptr;
  a.O_swa = sh.both_branch ? O_swa : nullptr;
  a.B = sh.B;
  a.N = sh.N;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.G = sh.G;
  a.W = sh.W;
  a.A = sh.A;
  a.off = sh.off;
  a.Wf = sh.W + sh.off;
  a.HK = p.HK;
  a.HG = p.HG;
  a.hpu = p.hpu;
  a.units = p.units;
  a.tpt_band = p.tpt_band;
  a.tpt_far = p.tpt_far;
  a.band_tiles = p.band_tiles;
  a.far_tiles = p.far_tiles;
  a.max_items = p.max_items;
  a.far_grid = 8 * ((p.max_items + 7) / 8);
  a.cmax = p.cmax;
  a.sl2 = sh.scale * kLog2e;
  if (sh.f32) {
    if (sh.d == 64) return run_prefill<float, 64>(sh, p, a, s, ev);
    return run_prefill<float, 128>(sh, p, a, s, ev);
  }
  if (sh.d == 64) return run_prefill<bf16_t, 64>(sh, p, a, s, ev);
  return run_prefill<bf16_t, 128>(sh, p, a, s, ev);
}

}  // namespace swi
