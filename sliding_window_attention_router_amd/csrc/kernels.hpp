// Host-side launchers of the SwiAttn kernels (internal to libswiattn.so).
// Arguments have been validated by the C ABI layer before these are called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace swi {

// ---- router -------------------------------------------------------------
hipError_t launch_route(const void* H, const void* r, const float* bias, uint8_t* gate,
                        float* z_out, int B, int N, int hidden, int G, bool f32, hipStream_t s);
hipError_t launch_compact(const uint8_t* gate, int32_t* idx, int32_t* cnt, int B, int N, int G,
                          hipStream_t s);

// ---- adaptive regulariser ----------------------------------------------
hipError_t launch_regularizer(const float* z, const float* nll, const float* diff, float* loss,
                              int B, int N, int G, float gamma_base, float eps, float alpha,
                              hipStream_t s);

// ---- router gradient through the straight-through gate -----------------
size_t router_grad_workspace(int64_t ntok, int hidden, int G);
int router_grad_max_groups();
hipError_t launch_router_grad(const void* dO, const void* Of, const void* Os, const float* z,
                              const void* H, const void* r, float* dz, void* dH, float* dr,
                              float* dbias, int B, int N, int Hq, int d, int hidden, int G, bool f32,
                              void* ws, hipStream_t s);

// ---- attention backward of the hard-gated prefill -----------------------
size_t backward_workspace(int B, int N, int Hq);
hipError_t launch_backward(const void* Q, const void* K, const void* V, const void* O,
                           const void* dO, const uint8_t* gate, const int32_t* idx,
                           const int32_t* cnt, void* dQ, void* dK, void* dV, int B, int N, int Hq,
                           int Hkv, int G, int d, int W, float scale, bool f32, void* ws,
                           hipStream_t s);

// ---- prefill ------------------------------------------------------------
struct PrefillShape {
  int B, N, Hq, Hkv, G, d, W;  // W clamped to N (a longer window sees the same keys)
  int A;    // global anchor keys of the window branch (0 = none)
  int off;  // window offset of the layer (0 = none), clamped to N
  float scale;
  bool f32;
  bool both_branch;
};

// Workspace plan: byte offsets of each buffer inside the caller's workspace.
struct PrefillPlan {
  int HK;         // query heads per KV head
  int HG;         // query heads per gate group
  int hpu;        // heads per far unit: min(HK, HG)
  int units;      // far units per sequence: Hq / hpu
  int tpt_band;   // tokens per window tile: 128 / HK
  int tpt_far;    // gathered tokens per far tile: 128 / hpu
  int band_tiles; // ceil(N / tpt_band)
  int far_tiles;  // per (b, unit): ceil(N / tpt_far)
  int target_items;  // far work items aimed for
  int max_items;  // upper bound on far work items
  int cmax;       // bound on chunks per far tile (+1)
  size_t off_lse, off_sched, off_queue, off_part_o, off_part_lse, off_diffp, bytes;
};

bool plan_prefill(const PrefillShape& sh, PrefillPlan* p);
// ev: optional array of 6 hipEvent_t recorded at stage boundaries (may be null);
// O_full, O_swa: optional branch outputs of both-branch mode (may be null)
hipError_t launch_prefill(const PrefillShape& sh, const PrefillPlan& p, const void* Q,
                          const void* K, const void* V, const uint8_t* gate, const int32_t* idx,
                          const int32_t* cnt, void* O, float* diff, void* ws, hipStream_t s,
                          void* const* ev, void* O_full = nullptr, void* O_swa = nullptr);

// ---- decode -------------------------------------------------------------
struct DecodeShape {
  int B, Lmax, Hq, Hkv, G, d, W;  // W clamped to Lmax
  int A;    // global anchor keys of the window branch (0 = none)
  int off;  // window offset of the layer (0 = none), clamped to Lmax
  float scale;
  bool f32;
};
struct DecodePlan {
  int HK, HG;
  int grid;       // workgroups of the split-K kernel (one share of the key blocks each)
  size_t off_info, off_part_o, off_part_lse, bytes;
};
bool plan_decode(const DecodeShape& sh, DecodePlan* p);
hipError_t launch_decode(const DecodeShape& sh, const DecodePlan& p, const void* q,
                         const void* Kc, const void* Vc, const int32_t* cache_len,
                         const uint8_t* gate, void* o, void* ws, hipStream_t s,
                         void* const* ev);
// Device address (on the current device) and size of the fixed scratch that
// the allocation-free decode uses as its workspace.
hipError_t decode_scratch(void** ptr);
size_t decode_scratch_bytes();
// route of the new tokens (N = 1), append of their K/V rows, decode
hipError_t launch_decode_step(const DecodeShape& sh, const DecodePlan& p, const void* Hn,
                              const void* r, const float* bias, int hidden, const void* q,
                              const void* k, const void* v, void* Kc, void* Vc, int32_t* cache_len,
                              uint8_t* gate, void* o, void* ws, hipStream_t s);

// Record ev[i] on s if present; returns the first error.
inline hipError_t mark(void* const* ev, int i, hipStream_t s) {
  if (!ev || !ev[i]) return hipSuccess;
  return hipEventRecord(static_cast<hipEvent_t>(ev[i]), s);
}

}  // namespace swi
