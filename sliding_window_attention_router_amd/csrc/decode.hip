// SwiAttn routed decode on gfx950.
//
// SwiAttn report, section 2: during decode the full and window branches read
// one shared KV cache.  The new token of sequence b sits at position L-1
// (L = cache_len[b]); a head routed full reads keys [0, L-1], a head routed
// to the window reads the last min(W, L) keys (weimeta SWA glossary, section
// "详细解释").  The bytes read therefore depend on the gate: 32K keys for a
// full sequence at a 32K cache, W keys otherwise.
//
// decode_schedule_kernel  (one workgroup) turns gates and cache lengths into
//                         a list of (sequence, KV head, key chunk) items
// decode_kernel           persistent single-wave workgroups; each walks its
//                         items' key blocks with the next block's loads in
//                         flight (also across item boundaries) and writes a
//                         normalised partial output + log-sum-exp per item
// decode_merge_kernel     log-sum-exp merge of a sequence's chunks
#include <climits>

#include "attn_core.hpp"
#include "kernels.hpp"

namespace swi {

constexpr int kDecChunk = 256;       // keys per work item (4 blocks of 64)
constexpr int kDecThreads = 64;      // one wave per workgroup
constexpr int kDecSchedThreads = 1024;

struct DecodeArgs {
  const void* q;
  const void* Kc;
  const void* Vc;
  const int32_t* cache_len;
  const uint8_t* gate;
  void* o;
  int32_t* sched;   // [0] total, item_start[nbk] | n_items[nbk] | lo[nbk] | item_bk[max] | item_ch[max]
  float* part_o;    // [max_items][HK][D]
  float* part_lse;  // [max_items][HK]
  int B, Lmax, Hq, Hkv, G, W, HK, HG, max_items;
  float sl2;
};

struct DecSched {
  int32_t *item_start, *n_items, *lo, *item_bk, *item_ch;
  SWI_DEV DecSched(const DecodeArgs& a) {
    const int nbk = a.B * a.Hkv;
    item_start = a.sched + 1;
    n_items = item_start + nbk;
    lo = n_items + nbk;
    item_bk = lo + nbk;
    item_ch = item_bk + a.max_items;
  }
};

SWI_DEV int clamp_len(int L, int Lmax) { return L < 1 ? 1 : (L > Lmax ? Lmax : L); }

// first key of head h's range in sequence b
SWI_DEV int head_lo(const DecodeArgs& a, int b, int h, int L) {
  const bool full = a.gate[b * a.G + h / a.HG] != 0;
  return full ? 0 : max(0, L - a.W);
}

__global__ __launch_bounds__(kDecSchedThreads) void decode_schedule_kernel(DecodeArgs a) {
  __shared__ int sh[kDecSchedThreads / 64 + 1];
  __shared__ int carry_s;
  DecSched sv(a);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nbk = a.B * a.Hkv;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < nbk; base += kDecSchedThreads) {
    const int bk = base + tid;
    int n = 0, lo = 0;
    if (bk < nbk) {
      const int b = bk / a.Hkv, kvh = bk - b * a.Hkv;
      const int L = clamp_len(a.cache_len[b], a.Lmax);
      lo = INT_MAX;
      for (int hh = 0; hh < a.HK; ++hh) lo = min(lo, head_lo(a, b, kvh * a.HK + hh, L));
      n = (L - lo + kDecChunk - 1) / kDecChunk;
    }
    int incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    if (lane == 63) sh[wave] = incl;
    __syncthreads();
    if (wave == 0) {
      const int nw = kDecSchedThreads / 64;
      const int x = lane < nw ? sh[lane] : 0;
      int w = x;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(w, o, 64);
        if (lane >= o) w += t;
      }
      if (lane < nw) sh[lane] = w - x;
      if (lane == nw - 1) sh[nw] = w;
    }
    __syncthreads();
    const int start = carry_s + sh[wave] + incl - n;
    if (bk < nbk) {
      sv.item_start[bk] = start;
      sv.n_items[bk] = n;
      sv.lo[bk] = lo;
      for (int k = 0; k < n; ++k) {
        sv.item_bk[start + k] = bk;
        sv.item_ch[start + k] = k;
      }
    }
    __syncthreads();
    if (tid == 0) carry_s += sh[kDecSchedThreads / 64];
    __syncthreads();
  }
  if (tid == 0) a.sched[0] = carry_s;
}

template <typename T, int D>
struct DecItem {
  int b, kvh, L, c0, c1, nblk;
  SWI_DEV void setup(const DecodeArgs& a, const DecSched& sv, int item) {
    const int bk = sv.item_bk[item], ch = sv.item_ch[item];
    b = bk / a.Hkv;
    kvh = bk - b * a.Hkv;
    L = clamp_len(a.cache_len[b], a.Lmax);
    c0 = sv.lo[bk] + ch * kDecChunk;
    c1 = min(L, c0 + kDecChunk);
    nblk = (c1 - c0 + kBN - 1) / kBN;
  }
  SWI_DEV const T* kbase(const DecodeArgs& a) const {
    return static_cast<const T*>(a.Kc) + (int64_t(b) * a.Lmax * a.Hkv + kvh) * D;
  }
  SWI_DEV const T* vbase(const DecodeArgs& a) const {
    return static_cast<const T*>(a.Vc) + (int64_t(b) * a.Lmax * a.Hkv + kvh) * D;
  }
};

template <typename T, int D>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(DecodeArgs a) {
  using Core = typename CoreSel<T, D>::type;
  __shared__ __align__(16) char lds[Lds<T, D>::kBytes];
  const int total = a.sched[0];
  int item = blockIdx.x;
  if (item >= total) return;
  DecSched sv(a);
  const int lane = threadIdx.x, q = lane & 31, g = lane >> 5;
  const bool valid = q < a.HK;
  const int64_t rs = int64_t(a.Hkv) * D;

  DecItem<T, D> it;
  it.setup(a, sv, item);
  Core c;
  int lo = 0, hi = -1;
  auto begin_item = [&]() {
    c.init();
    const int h = it.kvh * a.HK + q;
    const T* qp = static_cast<const T*>(a.q) + (int64_t(it.b) * a.Hq + h) * D;
    c.load_q(valid ? qp : nullptr, g);
    lo = valid ? max(it.c0, head_lo(a, it.b, h, it.L)) : 0;
    hi = valid ? it.c1 - 1 : -1;
  };
  begin_item();
  KVLoader<T, D, kDecThreads> ld;
  ld.load(it.kbase(a), it.vbase(a), rs, it.c0, it.c1, lane);
  int n = 0;
  while (true) {
    // the block after this one, possibly in the next item
    int nitem = item, nn = n + 1;
    if (nn >= it.nblk) {
      nitem = item + gridDim.x;
      nn = 0;
    }
    __syncthreads();
    ld.store(lds, lane);
    __syncthreads();
    DecItem<T, D> nx = it;
    if (nitem < total) {
      if (nitem != item) nx.setup(a, sv, nitem);
      ld.load(nx.kbase(a), nx.vbase(a), rs, nx.c0 + nn * kBN, nx.c1, lane);
    }
    const int kb = it.c0 + n * kBN;
    // rows of the wave may start later than the item (window heads sharing a
    // KV head with a full head); the block beyond c1 is zero-filled
    const int wmax_lo = wave_max_i(valid ? lo : -1);
    const bool masked = kb < wmax_lo || kb + kBN > it.c1;
    c.block(lds, kb, masked, lo, hi, a.sl2, q, g);
    if (nn == 0) {  // item finished
      float lse2;
      const float inv = finish_row(c.m, c.l, lse2);
      if (valid) {
        float* prow = a.part_o + (int64_t(item) * a.HK + q) * D;
        store_row<Core::MD>(prow, c.acc, inv, g);
        if (g == 0) a.part_lse[int64_t(item) * a.HK + q] = lse2;
      }
      if (nitem >= total) break;
      item = nitem;
      it = nx;
      begin_item();
      n = 0;
    } else {
      n = nn;
    }
  }
}

// One workgroup per (sequence, query head): the four waves take every
// fourth chunk, each keeps its own maximum and weighted sum, and the waves
// are combined through LDS in a fixed order.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  constexpr int PL = D / 64;  // adjacent channels per lane
  __shared__ float sm[4], sl[4];
  __shared__ float so[4][D];
  DecSched sv(a);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = blockIdx.x / a.Hq, h = blockIdx.x - b * a.Hq;
  const int kvh = h / a.HK, r = h - kvh * a.HK;
  const int bk = b * a.Hkv + kvh;
  const int is = sv.item_start[bk], ni = sv.n_items[bk];
  float M = kNegInf;
  for (int k = w + 4 * lane; k < ni; k += 256) M = fmaxf(M, a.part_lse[int64_t(is + k) * a.HK + r]);
  M = wave_max(M);
  float o[PL];
#pragma unroll
  for (int e = 0; e < PL; ++e) o[e] = 0.f;
  float L = 0.f;
  int k = w;
  for (; k + 12 < ni; k += 16) {  // four chunks of this wave per step, loads in flight together
    float lk[4], v[4][PL];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t it = is + k + 4 * j;
      lk[j] = a.part_lse[it * a.HK + r];
#pragma unroll
      for (int e = 0; e < PL; ++e) v[j][e] = a.part_o[(it * a.HK + r) * D + lane * PL + e];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float wt = lk[j] == kNegInf ? 0.f : fast_exp2(lk[j] - M);
      L += wt;
#pragma unroll
      for (int e = 0; e < PL; ++e) o[e] = fmaf(wt, v[j][e], o[e]);
    }
  }
  for (; k < ni; k += 4) {
    const int64_t it = is + k;
    const float lk = a.part_lse[it * a.HK + r];
    const float wt = lk == kNegInf ? 0.f : fast_exp2(lk - M);
    L += wt;
#pragma unroll
    for (int e = 0; e < PL; ++e) o[e] = fmaf(wt, a.part_o[(it * a.HK + r) * D + lane * PL + e], o[e]);
  }
  if (lane == 0) {
    sm[w] = M;
    sl[w] = L;
  }
#pragma unroll
  for (int e = 0; e < PL; ++e) so[w][lane * PL + e] = o[e];
  __syncthreads();
  if (w != 0) return;
  const float Mt = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
  float Lt = 0.f, ot[PL];
#pragma unroll
  for (int e = 0; e < PL; ++e) ot[e] = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float f = sm[j] == kNegInf ? 0.f : fast_exp2(sm[j] - Mt);
    Lt += f * sl[j];
#pragma unroll
    for (int e = 0; e < PL; ++e) ot[e] = fmaf(f, so[j][lane * PL + e], ot[e]);
  }
  const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
  T* orow = static_cast<T*>(a.o) + (int64_t(b) * a.Hq + h) * D;
#pragma unroll
  for (int e = 0; e < PL; ++e) Elem<T>::store(orow + lane * PL + e, ot[e] * inv);
}

static size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

bool plan_decode(const DecodeShape& sh, DecodePlan* p) {
  p->HK = sh.Hq / sh.Hkv;
  p->HG = sh.Hq / sh.G;
  p->chunk = kDecChunk;
  const long long max_items = (long long)sh.B * sh.Hkv * ((sh.Lmax + kDecChunk - 1) / kDecChunk);
  if (max_items > INT_MAX / 64) return false;
  p->max_items = int(max_items);
  p->grid = int(max_items < 1024 ? max_items : 1024);
  const int nbk = sh.B * sh.Hkv;
  size_t off = 0;
  p->off_sched = off;
  off = align_up(off + (1 + 3 * size_t(nbk) + 2 * size_t(max_items)) * 4);
  p->off_part_o = off;
  off = align_up(off + size_t(max_items) * p->HK * sh.d * 4);
  p->off_part_lse = off;
  off = align_up(off + size_t(max_items) * p->HK * 4);
  p->bytes = off;
  return true;
}

template <typename T, int D>
static hipError_t run_decode(const DecodeShape& sh, const DecodePlan& p, DecodeArgs& a,
                             hipStream_t s, void* const* ev) {
  hipError_t e;
  if ((e = mark(ev, 0, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(decode_schedule_kernel, dim3(1), dim3(kDecSchedThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = mark(ev, 1, s)) != hipSuccess) return e;
  hipLaunchKernelGGL((decode_kernel<T, D>), dim3(p.grid), dim3(kDecThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = mark(ev, 2, s)) != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(sh.B * sh.Hq), dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return mark(ev, 3, s);
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
  a.sched = reinterpret_cast<int32_t*>(w + p.off_sched);
  a.part_o = reinterpret_cast<float*>(w + p.off_part_o);
  a.part_lse = reinterpret_cast<float*>(w + p.off_part_lse);
  a.B = sh.B;
  a.Lmax = sh.Lmax;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.G = sh.G;
  a.W = sh.W;
  a.HK = p.HK;
  a.HG = p.HG;
  a.max_items = p.max_items;
  a.sl2 = sh.scale * kLog2e;
  if (sh.f32) {
    if (sh.d == 64) return run_decode<float, 64>(sh, p, a, s, ev);
    return run_decode<float, 128>(sh, p, a, s, ev);
  }
  if (sh.d == 64) return run_decode<bf16_t, 64>(sh, p, a, s, ev);
  return run_decode<bf16_t, 128>(sh, p, a, s, ev);
}

}  // namespace swi
