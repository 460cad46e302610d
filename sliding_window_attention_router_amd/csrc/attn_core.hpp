// Flash-attention building blocks for the SwiAttn kernels on gfx950.
//
// Orientation.  Every wave owns 32 query rows.  Scores are formed
// transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (A = a 32-key slice
// of K from LDS, B = the wave's queries kept in registers), so the 32x32
// accumulator puts one query per lane column: lane l holds query l%32 and 16
// keys.  The softmax state (running max, running sum) of a query therefore
// lives in its two lanes l and l^32, and the only cross-lane step is one xor
// shuffle by 32.  The output is accumulated transposed as well,
// O^T = V^T P^T, which lets P^T come straight from the score accumulators
// (same lane <-> query mapping) and makes the per-query rescale a per-lane
// multiply.  V is staged transposed in LDS so that an A operand (one
// channel, 8 keys) is a single 16-byte LDS read.
//
// The contraction index of an MFMA may be permuted freely as long as A and B
// use the same permutation; the P^T / V^T operands use the permutation that
// the 32x32 accumulator layout hands out (lane group g holds keys
// 8*(i/4) + 4*g + i%4 of each 32-key slice).
//
// float32 inputs use the same structure with v_mfma_f32_32x32x2f32.
#pragma once
#include "common.hpp"

namespace swi {

constexpr int kBN = 64;  // keys per LDS block
constexpr int kMfmaPrio = 1;  // wave issue priority inside MFMA sections
constexpr int kQR = 32;  // query rows per wave

template <typename T, int D>
struct Lds;
template <int D>
struct Lds<bf16_t, D> {
  // K block [kBN][D]: row stride D*2+16 bytes puts consecutive keys 4 banks
  // apart, so 16-byte operand reads of 8 consecutive lanes hit distinct banks.
  static constexpr int kKStride = D * 2 + 16;
  // V block transposed [D][kBN]: row stride kBN*2+16 bytes.  Inside each
  // 16-key group the 4-key quarters are stored in the order 0,2,1,3, so the
  // 8 keys an MFMA lane group needs (quarters g and g+2) are adjacent and
  // one 16-byte read fetches them.
  static constexpr int kVStride = kBN * 2 + 16;
  static constexpr int kKBytes = kBN * kKStride;
  static constexpr int kBytes = kKBytes + D * kVStride;
  // byte offset of 4-key quarter kq (keys 4kq..4kq+3) inside a V^T row
  SWI_DEV static constexpr int vq_offset(int kq) {
    return ((kq & ~3) | ((kq & 1) << 1) | ((kq >> 1) & 1)) * 8;
  }
};
template <int D>
struct Lds<float, D> {
  static constexpr int kKStride = (D + 2) * 4;  // [kBN][D+2] floats
  static constexpr int kVStride = (D + 8) * 4;  // [kBN][D+8] floats, not transposed
  static constexpr int kKBytes = kBN * kKStride;
  static constexpr int kBytes = kKBytes + kBN * kVStride;
};

// ---------------------------------------------------------------------------
// Global -> register -> LDS staging of one block of kBN keys of one KV head.
// Rows at or beyond `kend` are read from row kend-1 instead (branch-free and
// in bounds): every block that reaches past kend is processed with the key
// mask, which gives those keys probability exactly 0, and 0 times a finite
// value adds nothing.
// ---------------------------------------------------------------------------
SWI_DEV int clamp_row(int kk, int kend) { return kk < kend ? kk : kend - 1; }

// kStream: the rows are read once (decode), so the loads carry the
// non-temporal hint and do not displace reusable lines from the caches.
template <bool kStream>
SWI_DEV u32x4 load16(const void* p) {
  const u32x4* v = static_cast<const u32x4*>(p);
  if constexpr (kStream) return __builtin_nontemporal_load(v);
  return *v;
}

template <typename T, int D, int NT, bool kStream = false>
struct KVLoader;

template <int D, int NT, bool kStream>
struct KVLoader<bf16_t, D, NT, kStream> {
  using L = Lds<bf16_t, D>;
  static constexpr int CPR = D / 8;  // 16-byte pieces per row
  static constexpr int KU = kBN * CPR;
  static constexpr int KPER = (KU + NT - 1) / NT;
  static constexpr int VU = (kBN / 4) * CPR;  // pieces of (4 keys x 8 channels)
  static constexpr int VPER = (VU + NT - 1) / NT;
  u32x4 kr[KPER];
  u32x4 vr[VPER][4];

  // K piece u: key u / CPR, channels 8*(u % CPR): 16 consecutive lanes read
  // one 256-byte row.  V piece u: key quarter u % 16 (4 keys), channels
  // 8*(u / 16): the 16 lanes that write one V^T row together cover all its
  // banks.
  //
  // Addressing: the block's first row is wave-uniform (scalar base), each
  // piece adds a fixed per-lane 32-bit byte offset.  Only a block that
  // reaches past kend (wave-uniform test) pays for the clamp.  The streaming
  // (decode) loader keeps the per-row form, which measured faster there.
  SWI_DEV void load(const bf16_t* __restrict__ Kb, const bf16_t* __restrict__ Vb, int64_t rs,
                    int kb, int kend, int tid) {
    const char* kp = reinterpret_cast<const char*>(Kb + int64_t(kb) * rs);
    const char* vp = reinterpret_cast<const char*>(Vb + int64_t(kb) * rs);
    const uint32_t rb = uint32_t(rs) * 2u;  // bytes per row
    const int last = kend - 1 - kb;         // last readable row of the block
    if (!kStream && kb + kBN <= kend) {
      // piece j of lane tid: row tid/CPR + j*NT/CPR, column tid%CPR (K);
      // rows 4*(tid%16) + r, columns tid/16 + j*NT/16 (V).  The j and r
      // parts are uniform and go into the scalar base.
      static_assert(NT % CPR == 0 && NT % 16 == 0, "lane layout");
      const uint32_t k_lane = uint32_t(tid / CPR) * rb + uint32_t(tid % CPR) * 16u;
      const uint32_t v_lane = uint32_t(4 * (tid & 15)) * rb + uint32_t(tid >> 4) * 16u;
#pragma unroll
      for (int j = 0; j < KPER; ++j) {
        if (KU % NT != 0 && tid + NT * j >= KU) continue;
        kr[j] = load16<kStream>(kp + size_t(j * (NT / CPR)) * rb + k_lane);
      }
#pragma unroll
      for (int j = 0; j < VPER; ++j) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (VU % NT != 0 && tid + NT * j >= VU) continue;
          vr[j][r] = load16<kStream>(vp + (size_t(r) * rb + size_t(j * (NT / 16)) * 16u) + v_lane);
        }
      }    } else {
#pragma unroll
      for (int j = 0; j < KPER; ++j) {
        const int u = tid + NT * j;
        const int key = u / CPR, c = u - key * CPR;
        if (KU % NT != 0 && u >= KU) continue;
        const int kk = min(key, last);
        kr[j] = load16<kStream>(kp + (int64_t(kk) * rb + c * 16));
      }
#pragma unroll
      for (int j = 0; j < VPER; ++j) {
        const int u = tid + NT * j;
        const int kq = u & 15, c = u >> 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (VU % NT != 0 && u >= VU) continue;
          const int kk = min(4 * kq + r, last);
          vr[j][r] = load16<kStream>(vp + (int64_t(kk) * rb + c * 16));
        }
      }
    }
  }

  SWI_DEV void store(char* lds, int tid) const {
#pragma unroll
    for (int j = 0; j < KPER; ++j) {
      const int u = tid + NT * j;
      if (KU % NT != 0 && u >= KU) continue;
      const int key = u / CPR, c = u - key * CPR;
      *reinterpret_cast<u32x4*>(lds + key * L::kKStride + c * 16) = kr[j];
    }
    char* vt = lds + L::kKBytes;
#pragma unroll
    for (int j = 0; j < VPER; ++j) {
      const int u = tid + NT * j;
      if (VU % NT != 0 && u >= VU) continue;
      const int kq = u & 15, c = u >> 4;
      const int col = L::vq_offset(kq);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a0 = vr[j][0][e], a1 = vr[j][1][e], a2 = vr[j][2][e], a3 = vr[j][3][e];
        // channel 2e: low halves of the four keys; channel 2e+1: high halves
        u32x2 lo = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
        u32x2 hi = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
        const int ch = c * 8 + 2 * e;
        *reinterpret_cast<u32x2*>(vt + ch * L::kVStride + col) = lo;
        *reinterpret_cast<u32x2*>(vt + (ch + 1) * L::kVStride + col) = hi;
      }
    }
  }
};

template <int D, int NT, bool kStream>
struct KVLoader<float, D, NT, kStream> {
  using L = Lds<float, D>;
  static constexpr int CPR = D / 4;
  static constexpr int KU = kBN * CPR;
  static constexpr int KPER = (KU + NT - 1) / NT;
  u32x4 kr[KPER];
  u32x4 vr[KPER];

  SWI_DEV void load(const float* __restrict__ Kb, const float* __restrict__ Vb, int64_t rs,
                    int kb, int kend, int tid) {
#pragma unroll
    for (int j = 0; j < KPER; ++j) {
      const int u = tid + NT * j;
      const int key = u / CPR, c = u - key * CPR;
      if (KU % NT != 0 && u >= KU) continue;
      const int kk = clamp_row(kb + key, kend);
      kr[j] = load16<kStream>(Kb + kk * rs + c * 4);
      vr[j] = load16<kStream>(Vb + kk * rs + c * 4);
    }
  }
  SWI_DEV void store(char* lds, int tid) const {
#pragma unroll
    for (int j = 0; j < KPER; ++j) {
      const int u = tid + NT * j;
      if (KU % NT != 0 && u >= KU) continue;
      const int key = u / CPR, c = u - key * CPR;
      uint32_t* kp = reinterpret_cast<uint32_t*>(lds + key * L::kKStride) + c * 4;
      uint32_t* vp = reinterpret_cast<uint32_t*>(lds + L::kKBytes + key * L::kVStride) + c * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kp[e] = kr[j][e];
        vp[e] = vr[j][e];
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Online softmax update shared by both cores.  s[mt][i] holds the raw score
// of key kb + 32*mt + 8*(i/4) + 4*g + i%4 for this lane's query.  On return
// s holds the unnormalised probabilities exp2(sl2*s - m), l is updated and
// the accumulators rescaled if m moved.  Keys outside [lo, hi] are dropped
// when `masked` (wave-uniform).
//
// m is the running maximum of sl2*score, kept lazily: it is only raised (and
// the accumulators rescaled) when a block's maximum exceeds it by more than
// kRescale, so a probability is at most 2^kRescale before the final
// normalisation.  The result is the same softmax; only rounding differs.
// ---------------------------------------------------------------------------
constexpr float kRescale = 8.f;

template <int MD, bool kSum = true>
SWI_DEV void online_softmax(f32x16 (&s)[2], f32x16 (&acc)[MD], float& m, float& l, int kb,
                            bool masked, int lo, int hi, float sl2, int g) {
  // Masking only rewrites the scores, in a wave-uniform branch, so masked
  // and unmasked blocks share every other instruction and register.
  if (masked) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = kb + mt * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
        if (j < lo || j > hi) s[mt][i] = kNegInf;
      }
  }
  float mx = kNegInf;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[mt][i]);
  mx = fmaxf(mx, xor32(mx)) * sl2;
  // raise m when the block maximum exceeds it by more than kRescale (and on
  // the first block that has any key); wave-uniform skip otherwise
  const bool raise = mx > m + kRescale;
  if (__any(raise)) {
    // lanes that do not raise keep m (which may still be -inf): alpha 1
    const float alpha = raise ? fast_exp2(m - mx) : 1.f;  // 0 when m was -inf
    if (raise) m = mx;
    l *= alpha;
#pragma unroll
    for (int md = 0; md < MD; ++md) acc[md] *= alpha;
  }
  const float mu = (m == kNegInf) ? 0.f : m;
  float ls = 0.f;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(fmaf(s[mt][i], sl2, -mu));
      s[mt][i] = p;
      if constexpr (kSum) ls += p;
    }
  }
  if constexpr (kSum) l += ls;
}

// ---------------------------------------------------------------------------
// bf16 core
// ---------------------------------------------------------------------------
template <int D>
struct CoreBF16 {
  using T = bf16_t;
  using L = Lds<bf16_t, D>;
  static constexpr int KS = D / 16;  // k-steps of the score product
  static constexpr int MD = D / 32;  // 32-channel tiles of the output
  bf16x8 qreg[KS];
  f32x16 acc[MD];
  float m, l;

  SWI_DEV void init() {
    m = kNegInf;
    l = 0.f;
#pragma unroll
    for (int md = 0; md < MD; ++md) acc[md] = f32x16{};
  }
  // qrow: this lane's query row (nullptr = padding row, zeros)
  SWI_DEV void load_q(const bf16_t* qrow, int g) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[ks] = qrow ? *reinterpret_cast<const bf16x8*>(qrow + ks * 16 + g * 8) : bf16x8{};
  }
  SWI_DEV void block(const char* lds, int kb, bool masked, int lo, int hi, float sl2, int q,
                     int g) {
    f32x16 s[2];
    // Issue priority: a wave raises it for its MFMA sections, so the SIMD's
    // other wave fills the VALU while the matrix pipe stays busy.
    __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = f32x16{};
      const char* kp = lds + (mt * 32 + q) * L::kKStride + g * 16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kp + ks * 32);
        s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], s[mt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    online_softmax<MD>(s, acc, m, l, kb, masked, lo, hi, sl2, g);
    bf16x8 pb[4];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[st][e] = bf16_t(s[st >> 1][(st & 1) * 8 + e]);
    // k-step st covers keys 16st..16st+15; lane group g supplies quarters
    // 4st+g and 4st+g+2, stored adjacently (Lds::vq_offset)
    const char* vt = lds + L::kKBytes;
    __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      const char* vp = vt + (md * 32 + q) * L::kVStride + g * 16;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vp + st * 32);
        acc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st], acc[md], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }
};

// ---------------------------------------------------------------------------
// Direct (DMA) staging for bf16: gfx950's global_load_lds_dwordx4 copies 16
// bytes per lane from global memory straight into LDS (lane i of a wave
// writes bytes [16i, 16i+16) after the wave-uniform destination), so a K/V
// block needs no registers and no LDS store instructions.  Each 1 KB copy
// covers 1024 / (2D) whole rows; the lane -> source mapping is free, which
// is used to XOR-swizzle the 16-byte chunks of every row so that the
// operand reads hit distinct banks (64 banks of 4 bytes: a 128-bit read is
// served 16 lanes at a time, a 64-bit read 32 lanes at a time):
//   K: the 16 lanes of a read take 16 consecutive key rows at one chunk;
//      chunk c of row k is stored at c ^ (k & 15) (d = 128) or
//      c ^ ((k >> 1) & 7) (d = 64, two rows per 256 bytes);
//   V: 32 lanes of a transposing read take 4 rows x 4 chunks; chunk c of
//      row k is stored at c ^ ((k & 3) << 2) (d = 128) or
//      c ^ (((k >> 1) & 1) << 2) (d = 64).
// V^T operands come from ds_read_b64_tr_b16: within each group of 16
// lanes, source lane 4r + k supplies four 16-bit values and destination
// lane 4k + e receives value e of source lanes k, 4 + k, 8 + k, 12 + k (as
// its elements 0..3).  Pointing source lane 4r + k at channels
// [c0 + 4k, c0 + 4k + 4) of key row r therefore gives lane i the channel
// c0 + i for four consecutive keys: one half of an MFMA A operand.
// ---------------------------------------------------------------------------
#define SWI_GLOBAL(p) ((__attribute__((address_space(1))) void*)(p))
#define SWI_LOCAL(p) ((__attribute__((address_space(3))) void*)(p))
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct LdsDma {
  static constexpr int kRowB = 2 * D;  // bytes per key row
  static constexpr int kKBytes = kBN * kRowB;
  static constexpr int kBytes = 2 * kKBytes;  // K block, then V block
  SWI_DEV static constexpr int k_swz(int key) { return D == 128 ? (key & 15) : ((key >> 1) & 7); }
  SWI_DEV static constexpr int v_swz(int key) {
    return D == 128 ? ((key & 3) << 2) : (((key >> 1) & 1) << 2);
  }
  SWI_DEV static constexpr int k_pos(int key, int chunk) {
    return key * kRowB + ((chunk ^ k_swz(key)) << 4);
  }
  SWI_DEV static constexpr int v_pos(int key, int chunk) {
    return kKBytes + key * kRowB + ((chunk ^ v_swz(key)) << 4);
  }
};

template <int D, int NT>
struct KVDma {
  using L = LdsDma<D>;
  static constexpr int kCopies = L::kKBytes / 1024;  // 1 KB copies per matrix
  static constexpr int kPer = kCopies / (NT / 64);   // per wave
  static_assert(kCopies % (NT / 64) == 0, "copies per wave");
  // Copy rows kb .. kb+63 (rows at or past kend read row kend-1) into buf.
  SWI_DEV static void issue(char* buf, const bf16_t* Kb, const bf16_t* Vb, int64_t rs, int kb,
                            int kend, int tid) {
    const int wave = tid >> 6, lane = tid & 63;
    const char* kp = reinterpret_cast<const char*>(Kb + int64_t(kb) * rs);
    const char* vp = reinterpret_cast<const char*>(Vb + int64_t(kb) * rs);
    const uint32_t rb = uint32_t(rs) * 2u;
    const int last = kend - 1 - kb;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int m = wave * kPer + i;
      const int byte = m * 1024 + lane * 16;
      const int row = byte / L::kRowB, p = (byte % L::kRowB) >> 4;
      const uint32_t src = uint32_t(min(row, last)) * rb;
      // one 32-bit lane offset per address: the copies then use the
      // scalar-base + offset form (one VGPR per address instead of two)
      const uint32_t ko = src + uint32_t((p ^ L::k_swz(row)) << 4);
      const uint32_t vo = src + uint32_t((p ^ L::v_swz(row)) << 4);
      __builtin_amdgcn_global_load_lds(SWI_GLOBAL(kp + ko), SWI_LOCAL(buf + m * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(SWI_GLOBAL(vp + vo), SWI_LOCAL(buf + L::kKBytes + m * 1024), 16,
                                       0, 0);
    }
  }
};

// Register-staged loads into the DMA layout (used by decode, which keeps one
// LDS buffer per wave): lane i of copy m loads the 16 bytes that the DMA
// copy above would place at buf + m*1024 + 16i (the same source swizzle),
// and stores them there, so the stores are linear 16-byte writes with no
// transposition.  K and V are loaded and stored separately, so that the
// next block's K loads can be issued before the current block's V is
// stored.  kStream adds the non-temporal hint (rows read once).
template <int D, int NT, bool kStream>
struct KVRegDma {
  using L = LdsDma<D>;
  static constexpr int kCopies = L::kKBytes / 1024;
  static constexpr int kPer = kCopies / (NT / 64);
  static_assert(kCopies % (NT / 64) == 0, "copies per wave");
  u32x4 kr[kPer], vr[kPer];

  template <bool kIsK>
  SWI_DEV static void load_part(u32x4 (&r)[kPer], const bf16_t* __restrict__ base, int64_t rs, int kb,
                                int kend, int tid) {
    const int wave = tid >> 6, lane = tid & 63;
    const char* p0 = reinterpret_cast<const char*>(base + int64_t(kb) * rs);
    const uint32_t rb = uint32_t(rs) * 2u;
    const int last = kend - 1 - kb;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int m = wave * kPer + i;
      const int byte = m * 1024 + lane * 16;
      const int row = byte / L::kRowB, pc = (byte % L::kRowB) >> 4;
      const int sw = kIsK ? L::k_swz(row) : L::v_swz(row);
      r[i] = load16<kStream>(p0 + (int64_t(min(row, last)) * rb + ((pc ^ sw) << 4)));
    }
  }
  SWI_DEV void load_k(const bf16_t* Kb, int64_t rs, int kb, int kend, int tid) {
    load_part<true>(kr, Kb, rs, kb, kend, tid);
  }
  SWI_DEV void load_v(const bf16_t* Vb, int64_t rs, int kb, int kend, int tid) {
    load_part<false>(vr, Vb, rs, kb, kend, tid);
  }
  SWI_DEV void load(const bf16_t* Kb, const bf16_t* Vb, int64_t rs, int kb, int kend, int tid) {
    load_k(Kb, rs, kb, kend, tid);
    load_v(Vb, rs, kb, kend, tid);
  }
  SWI_DEV void store_k(char* lds, int tid) const {
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      *reinterpret_cast<u32x4*>(lds + (wave * kPer + i) * 1024 + lane * 16) = kr[i];
  }
  SWI_DEV void store_v(char* lds, int tid) const {
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      *reinterpret_cast<u32x4*>(lds + L::kKBytes + (wave * kPer + i) * 1024 + lane * 16) = vr[i];
  }
};

// LDS reads of the DMA layout are issued from inline assembly with explicit
// waits.  The compiler cannot tell that the transposing reads touch only
// the buffer that is not being filled, and would otherwise wait for the
// copies of the next block before every read of the current one.  Byte
// address = wave-invariant per-lane part (register) + compile-time offset.
template <int OFF>
SWI_DEV bf16x8 lds_read_b128(uint32_t addr) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int OFF>
SWI_DEV s16x4 lds_read_tr16(uint32_t addr) {
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
// Wait for every outstanding LDS read; tying the operands orders their uses
// after the wait.
template <typename V, int N>
SWI_DEV void lds_wait(V (&v)[N]) {
  static_assert(N == 8, "eight operands per group");
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                 "+v"(v[6]), "+v"(v[7]));
}
// The same, placed after the MFMA chain that produced `after` (an input
// only, to order the wait behind that chain in the instruction stream).
template <typename V, int N>
SWI_DEV void lds_wait_after(V (&v)[N], float after) {
  static_assert(N == 8, "eight operands per group");
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                 "+v"(v[6]), "+v"(v[7])
               : "v"(after));
}
SWI_DEV uint32_t lds_addr(const char* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}

// Called by a core's block() right after its score MFMAs, when the query
// registers are free for the rest of the block (used to start loading the
// next tile's queries).
struct NoHook {
  SWI_DEV void operator()() const {}
};

// bf16 core reading the DMA layout (same arithmetic as CoreBF16).  Operand
// reads run one group of eight ahead of the MFMAs that use them.
template <int D>
struct CoreBF16Dma {
  using T = bf16_t;
  using L = LdsDma<D>;
  static constexpr int KS = D / 16;
  static constexpr int MD = D / 32;
  static_assert(KS == 8 || KS == 4, "head dim 64 or 128");
  bf16x8 qreg[KS];
  f32x16 acc[MD];
  float m, l;

  SWI_DEV void init() {
    m = kNegInf;
    l = 0.f;
#pragma unroll
    for (int md = 0; md < MD; ++md) acc[md] = f32x16{};
  }
  SWI_DEV void load_q(const bf16_t* qrow, int g) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[ks] = qrow ? *reinterpret_cast<const bf16x8*>(qrow + ks * 16 + g * 8) : bf16x8{};
  }

  // K operands of key tile MT: 8 reads (KS = 8) or the KS reads of both tiles
  template <int MT>
  SWI_DEV static void read_k(const uint32_t (&ka)[KS], bf16x8 (&a)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int mt = KS == 8 ? MT : i / KS, ks = i % KS;
      a[i] = [&]() {
        if (mt == 0) return lds_read_b128<0>(ka[ks]);
        return lds_read_b128<32 * L::kRowB>(ka[ks]);
      }();
    }
  }
  // V^T operands of output tile md: st = 0..3, two transposing reads each
  template <int MDI>
  SWI_DEV static void read_v(uint32_t va, s16x4 (&v)[8]) {
    v[0] = lds_read_tr16<L::kKBytes + 0 * L::kRowB>(va);
    v[1] = lds_read_tr16<L::kKBytes + 8 * L::kRowB>(va);
    v[2] = lds_read_tr16<L::kKBytes + 16 * L::kRowB>(va);
    v[3] = lds_read_tr16<L::kKBytes + 24 * L::kRowB>(va);
    v[4] = lds_read_tr16<L::kKBytes + 32 * L::kRowB>(va);
    v[5] = lds_read_tr16<L::kKBytes + 40 * L::kRowB>(va);
    v[6] = lds_read_tr16<L::kKBytes + 48 * L::kRowB>(va);
    v[7] = lds_read_tr16<L::kKBytes + 56 * L::kRowB>(va);
  }

  template <typename F = NoHook>
  SWI_DEV void block(const char* lds, int kb, bool masked, int lo, int hi, float sl2, int q,
                     int g, F&& after_scores = F()) {
    const int lane = threadIdx.x & 63;
    const uint32_t base = lds_addr(lds);
    // per-lane parts of the addresses (key row q of a tile, chunk 2ks+g)
    uint32_t ka[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ka[ks] = base + L::k_pos(q, ks * 2 + g);
    f32x16 s[2];
    s[0] = f32x16{};
    s[1] = f32x16{};
    bf16x8 a0[8], a1[8];
    read_k<0>(ka, a0);
    lds_wait(a0);
    if (KS == 8) read_k<1>(ka, a1);
    __builtin_amdgcn_s_setprio(kMfmaPrio);
    if (KS == 8) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[ks], qreg[ks], s[0], 0, 0, 0);
      lds_wait_after(a1, s[0][0]);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[ks], qreg[ks], s[1], 0, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        s[i / KS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], qreg[i % KS], s[i / KS], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    after_scores();
    online_softmax<MD, false>(s, acc, m, l, kb, masked, lo, hi, sl2, g);
    bf16x8 pb[4];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[st][e] = bf16_t(s[st >> 1][(st & 1) * 8 + e]);
    // row sum of the probabilities as rounded for the P.V product (the
    // normaliser then matches the numerator), two at a time
    {
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      const bf16x2_t one = {bf16_t(1.f), bf16_t(1.f)};
      float l0 = 0.f, l1 = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int e = 0; e < 8; e += 4) {
          l0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{pb[st][e], pb[st][e + 1]}, one, l0, false);
          l1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{pb[st][e + 2], pb[st][e + 3]}, one, l1, false);
        }
      l += l0 + l1;
    }
    // k-step st, lane group g holds keys 16st + 4g + {0..3} (slots 0..3) and
    // 16st + 8 + 4g + {0..3} (slots 4..7) of P^T; the transposing reads
    // fetch V^T to match (source lane 4r + k of each 16-lane group points at
    // key row 4g + r, channels c0 + 4k .. c0 + 4k + 3)
    const int r = (lane >> 2) & 3, k = lane & 3, hh = (lane >> 4) & 1;
    uint32_t va[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md)
      va[md] = base + (L::v_pos(4 * g + r, md * 4 + 2 * hh + (k >> 1)) - L::kKBytes) + (k & 1) * 8;
    s16x4 v0[8], v1[8];
    read_v<0>(va[0], v0);
    __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      s16x4(&cur)[8] = (md & 1) ? v1 : v0;
      s16x4(&nxt)[8] = (md & 1) ? v0 : v1;
      lds_wait(cur);
      if (md + 1 < MD) read_v<0>(va[md + 1], nxt);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(cur[2 * st], cur[2 * st + 1], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st], acc[md], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }
};

// Array interface over a one-tile core (TPW = 1): the window and far kernels
// are written for TPW row tiles per wave.
template <typename C>
struct OneTile {
  using T = typename C::T;
  using L = typename C::L;
  static constexpr int TPW = 1;
  static constexpr int MD = C::MD;
  C c;
  SWI_DEV void init() { c.init(); }
  SWI_DEV void load_q(int, const T* qrow, int g) { c.load_q(qrow, g); }
  SWI_DEV void block(const char* lds, int kb, bool masked, const int (&lo)[1], const int (&hi)[1],
                     float sl2, int q, int g) {
    c.block(lds, kb, masked, lo[0], hi[0], sl2, q, g);
  }
  template <typename F>
  SWI_DEV void block_hook(const char* lds, int kb, bool masked, int lo, int hi, float sl2, int q,
                          int g, F&& after_scores) {
    c.block(lds, kb, masked, lo, hi, sl2, q, g, after_scores);
  }
  SWI_DEV f32x16 (&acc_of(int))[MD] { return c.acc; }
  SWI_DEV float m_of(int) const { return c.m; }
  SWI_DEV float l_of(int) const { return c.l; }
};

// ---------------------------------------------------------------------------
// float32 core (same structure, v_mfma_f32_32x32x2f32)
// ---------------------------------------------------------------------------
template <int D>
struct CoreF32 {
  using T = float;
  using L = Lds<float, D>;
  static constexpr int KS = D / 2;
  static constexpr int MD = D / 32;
  float qreg[KS];
  f32x16 acc[MD];
  float m, l;

  SWI_DEV void init() {
    m = kNegInf;
    l = 0.f;
#pragma unroll
    for (int md = 0; md < MD; ++md) acc[md] = f32x16{};
  }
  SWI_DEV void load_q(const float* qrow, int g) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qreg[ks] = qrow ? qrow[ks * 2 + g] : 0.f;
  }
  SWI_DEV void block(const char* lds, int kb, bool masked, int lo, int hi, float sl2, int q,
                     int g) {
    f32x16 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = f32x16{};
      const float* kp = reinterpret_cast<const float*>(lds + (mt * 32 + q) * L::kKStride) + g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(kp[ks * 2], qreg[ks], s[mt], 0, 0, 0);
    }
    online_softmax<MD>(s, acc, m, l, kb, masked, lo, hi, sl2, g);
    const char* vs = lds + L::kKBytes;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
      for (int st = 0; st < 32; ++st) {
        const int i = st & 15, mt = st >> 4;
        const int key = mt * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
        const float a = *reinterpret_cast<const float*>(vs + key * L::kVStride + (md * 32 + q) * 4);
        acc[md] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[mt][i], acc[md], 0, 0, 0);
      }
    }
  }
};

template <typename T, int D>
struct CoreSel;
template <int D>
struct CoreSel<bf16_t, D> {
  using type = CoreBF16<D>;
};
template <int D>
struct CoreSel<float, D> {
  using type = CoreF32<D>;
};

// Row-tile configuration of the window and far kernels: 128 query rows per
// workgroup, four waves of the one-tile core.
template <typename T, int D>
struct TileCfg;
template <int D>
struct TileCfg<bf16_t, D> {
  using Core = OneTile<CoreBF16Dma<D>>;
  static constexpr bool kDma = true;
  static constexpr int kWaves = 4;
  static constexpr int kMinWG = 2;  // two workgroups per CU: 256 registers per wave
};
template <int D>
struct TileCfg<float, D> {
  using Core = OneTile<CoreF32<D>>;
  static constexpr bool kDma = false;
  static constexpr int kWaves = 4;
  static constexpr int kMinWG = 1;
};

// Total row sum over the lane pair, the log2-domain normaliser, and 1/sum
// (0 for a row that saw no key).
SWI_DEV float finish_row(float m, float l, float& lse2) {
  const float lt = l + xor32(l);
  lse2 = lt > 0.f ? m + fast_log2(lt) : kNegInf;
  return lt > 0.f ? 1.f / lt : 0.f;
}

// Channel held by accumulator element i of output tile md in lane group g.
SWI_DEV constexpr int acc_channel(int md, int i, int g) {
  return md * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
}

// Store this lane's half of an output row: the two lanes of a row swap
// 4-channel groups first (v_permlane32_swap), so that lane g holds channels
// 16g .. 16g + 15 of each 32-channel tile and writes them as two 16-byte
// stores.  Group i4 of a lane holds channels 8 i4 + 4 g .. + 3.  One swap
// of (group k, group k + 2) exchanges the upper half-wave of the first
// operand with the lower half-wave of the second, which leaves in both
// results exactly the pieces the lane stores: lane group 0 keeps its group k
// (first result) and receives group k of lane group 1 (second result); lane
// group 1 receives group k + 2 of lane group 0 (first) and keeps its own
// (second): channels 16 g + 8 k .. + 7 in order, for either group.
template <int MD>
SWI_DEV void store_row(bf16_t* orow, const f32x16 (&acc)[MD], float inv, int g) {
  typedef uint32_t u32x4_ __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int md = 0; md < MD; ++md) {
    uint32_t pk[4][2];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = bf16_t(acc[md][i4 * 4 + e] * inv);
      const auto w = __builtin_bit_cast(u32x2, v);
      pk[i4][0] = w[0];
      pk[i4][1] = w[1];
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const auto r0 = __builtin_amdgcn_permlane32_swap(pk[k][0], pk[k + 2][0], false, false);
      const auto r1 = __builtin_amdgcn_permlane32_swap(pk[k][1], pk[k + 2][1], false, false);
      *reinterpret_cast<u32x4_*>(orow + md * 32 + 16 * g + 8 * k) = u32x4_{r0[0], r1[0], r0[1], r1[1]};
    }
  }
}
template <int MD>
SWI_DEV void store_row(float* orow, const f32x16 (&acc)[MD], float inv, int g) {
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[md][i4 * 4 + e] * inv;
      *reinterpret_cast<f32x4*>(orow + md * 32 + i4 * 8 + g * 4) = v;
    }
}

}  // namespace swi
