// C ABI of libswiattn.so: argument validation, workspace planning and
// kernel launches on the caller's stream.  Declarations and the contract of
// each entry point are in include/swiattn.h.
#include "../../include/swiattn.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>

#include "kernels.hpp"

namespace {

bool dtype_ok(swiattn_dtype_t dt) { return dt == SWIATTN_BF16 || dt == SWIATTN_F32; }

// Shared shape checks of prefill and decode.  Returns SWIATTN_OK or an error.
int check_heads(int Hq, int Hkv, int G, int d, int W, float scale) {
  if (Hq < 1 || Hkv < 1 || G < 1 || W < 1) return SWIATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0 || Hq % G != 0) return SWIATTN_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !std::isfinite(scale)) return SWIATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return SWIATTN_ERR_UNSUPPORTED;
  const int HK = Hq / Hkv, HG = Hq / G;
  if (HK > 32) return SWIATTN_ERR_UNSUPPORTED;
  if (HK % HG != 0 && HG % HK != 0) return SWIATTN_ERR_UNSUPPORTED;
  return SWIATTN_OK;
}

int prefill_shape(int B, int N, int Hq, int Hkv, int G, int d, int W, float scale,
                  swiattn_dtype_t dt, unsigned flags, swi::PrefillShape* sh,
                  swi::PrefillPlan* plan) {
  if (B < 1 || N < 1 || !dtype_ok(dt)) return SWIATTN_ERR_INVALID_ARG;
  if (flags & ~SWIATTN_FLAG_BOTH_BRANCH) return SWIATTN_ERR_INVALID_ARG;
  const int rc = check_heads(Hq, Hkv, G, d, W, scale);
  if (rc != SWIATTN_OK) return rc;
  // element offsets are int64 on the device; token counts stay in int32
  if ((long long)B * N > INT_MAX / 2 || (long long)B * Hq > INT_MAX / 2)
    return SWIATTN_ERR_UNSUPPORTED;
  sh->B = B;
  sh->N = N;
  sh->Hq = Hq;
  sh->Hkv = Hkv;
  sh->G = G;
  sh->d = d;
  sh->W = W < N ? W : N;  // a window of N or more keys sees every earlier key
  sh->A = 0;
  sh->off = 0;
  sh->scale = scale;
  sh->f32 = dt == SWIATTN_F32;
  sh->both_branch = (flags & SWIATTN_FLAG_BOTH_BRANCH) != 0;
  if (!swi::plan_prefill(*sh, plan)) return SWIATTN_ERR_UNSUPPORTED;
  return SWIATTN_OK;
}

int decode_shape(int B, int Lmax, int Hq, int Hkv, int G, int d, int W, float scale,
                 swiattn_dtype_t dt, swi::DecodeShape* sh, swi::DecodePlan* plan) {
  if (B < 1 || Lmax < 1 || !dtype_ok(dt)) return SWIATTN_ERR_INVALID_ARG;
  const int rc = check_heads(Hq, Hkv, G, d, W, scale);
  if (rc != SWIATTN_OK) return rc;
  if ((long long)B * Hkv > INT_MAX / 4) return SWIATTN_ERR_UNSUPPORTED;
  sh->B = B;
  sh->Lmax = Lmax;
  sh->Hq = Hq;
  sh->Hkv = Hkv;
  sh->G = G;
  sh->d = d;
  sh->W = W < Lmax ? W : Lmax;
  sh->A = 0;
  sh->off = 0;
  sh->scale = scale;
  sh->f32 = dt == SWIATTN_F32;
  if (!swi::plan_decode(*sh, plan)) return SWIATTN_ERR_UNSUPPORTED;
  return SWIATTN_OK;
}

int hip_rc(hipError_t e) { return e == hipSuccess ? SWIATTN_OK : SWIATTN_ERR_HIP; }

}  // namespace

extern "C" {

int swiattn_route(const void* H, const void* r, const float* bias, uint8_t* gate, float* z_out,
                  int32_t* idx, int32_t* cnt, int B, int N, int hidden, int G,
                  swiattn_dtype_t dtype, swiattn_stream_t stream) {
  if (B < 1 || N < 1 || G < 1 || !dtype_ok(dtype)) return SWIATTN_ERR_INVALID_ARG;
  if (!gate || !idx || !cnt) return SWIATTN_ERR_INVALID_ARG;
  if (H && (!r || !bias || hidden < 1)) return SWIATTN_ERR_INVALID_ARG;
  if ((long long)B * N * G > INT_MAX || (long long)B * G > INT_MAX / 2)
    return SWIATTN_ERR_UNSUPPORTED;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (H) {
    const int rc = hip_rc(swi::launch_route(H, r, bias, gate, z_out, B, N, hidden, G,
                                            dtype == SWIATTN_F32, s));
    if (rc != SWIATTN_OK) return rc;
  }
  return hip_rc(swi::launch_compact(gate, idx, cnt, B, N, G, s));
}

int swiattn_regularizer(const float* z, const float* nll, const float* diff, float* loss, int B,
                        int N, int G, float gamma_base, float eps, float alpha,
                        swiattn_stream_t stream) {
  if (B < 1 || N < 1 || G < 1) return SWIATTN_ERR_INVALID_ARG;
  if (!z || !nll || !diff || !loss) return SWIATTN_ERR_INVALID_ARG;
  // eps > 0 and alpha >= 0 keep the weight's denominator positive for
  // non-negative NLL and distance; NaN fails every comparison
  if (!(eps > 0.f) || !(alpha >= 0.f) || !(gamma_base == gamma_base) ||
      !(eps < 3.4e38f) || !(alpha < 3.4e38f) || !(gamma_base < 3.4e38f && gamma_base > -3.4e38f))
    return SWIATTN_ERR_INVALID_ARG;
  return hip_rc(swi::launch_regularizer(z, nll, diff, loss, B, N, G, gamma_base, eps, alpha,
                                        reinterpret_cast<hipStream_t>(stream)));
}

size_t swiattn_prefill_workspace_size(int B, int N, int Hq, int Hkv, int G, int d, int W,
                                      swiattn_dtype_t dtype, unsigned flags) {
  swi::PrefillShape sh;
  swi::PrefillPlan p;
  if (prefill_shape(B, N, Hq, Hkv, G, d, W, 1.f, dtype, flags, &sh, &p) != SWIATTN_OK) return 0;
  return p.bytes;
}

int swiattn_prefill_offset(const void* Q, const void* K, const void* V, const uint8_t* gate,
                           const int32_t* idx, const int32_t* cnt, void* O, float* diff, int B, int N,
                           int Hq, int Hkv, int G, int d, int W, int anchors, int offset, float scale,
                           swiattn_dtype_t dtype, unsigned flags, void* ws, size_t ws_bytes,
                           swiattn_stream_t stream, const swiattn_events_t* events) {
  swi::PrefillShape sh;
  swi::PrefillPlan p;
  const int rc = prefill_shape(B, N, Hq, Hkv, G, d, W, scale, dtype, flags, &sh, &p);
  if (rc != SWIATTN_OK) return rc;
  if (anchors < 0 || offset < 0) return SWIATTN_ERR_INVALID_ARG;
  if (offset > 0 && sh.both_branch) return SWIATTN_ERR_UNSUPPORTED;
  sh.A = anchors < N ? anchors : N;
  sh.off = offset < N ? offset : N;
  if (!Q || !K || !V || !gate || !O) return SWIATTN_ERR_INVALID_ARG;
  if (sh.both_branch ? !diff : (!idx || !cnt)) return SWIATTN_ERR_INVALID_ARG;
  if (!ws || ws_bytes < p.bytes) return SWIATTN_ERR_WORKSPACE;
  return hip_rc(swi::launch_prefill(sh, p, Q, K, V, gate, idx, cnt, O, diff, ws,
                                    reinterpret_cast<hipStream_t>(stream),
                                    events ? events->ev : nullptr));
}

int swiattn_prefill_branches(const void* Q, const void* K, const void* V, const uint8_t* gate,
                             void* O, float* diff, void* O_full, void* O_swa, int B, int N, int Hq,
                             int Hkv, int G, int d, int W, int anchors, float scale,
                             swiattn_dtype_t dtype, void* ws, size_t ws_bytes, swiattn_stream_t stream,
                             const swiattn_events_t* events) {
  swi::PrefillShape sh;
  swi::PrefillPlan p;
  const int rc = prefill_shape(B, N, Hq, Hkv, G, d, W, scale, dtype, SWIATTN_FLAG_BOTH_BRANCH, &sh, &p);
  if (rc != SWIATTN_OK) return rc;
  if (anchors < 0) return SWIATTN_ERR_INVALID_ARG;
  sh.A = anchors < N ? anchors : N;
  if (!Q || !K || !V || !gate || !O || !diff || !O_full || !O_swa) return SWIATTN_ERR_INVALID_ARG;
  if (!ws || ws_bytes < p.bytes) return SWIATTN_ERR_WORKSPACE;
  return hip_rc(swi::launch_prefill(sh, p, Q, K, V, gate, nullptr, nullptr, O, diff, ws,
                                    reinterpret_cast<hipStream_t>(stream),
                                    events ? events->ev : nullptr, O_full, O_swa));
}

int swiattn_prefill_anchored(const void* Q, const void* K, const void* V, const uint8_t* gate,
                             const int32_t* idx, const int32_t* cnt, void* O, float* diff, int B,
                             int N, int Hq, int Hkv, int G, int d, int W, int anchors,
                             float scale, swiattn_dtype_t dtype, unsigned flags, void* ws,
                             size_t ws_bytes, swiattn_stream_t stream,
                             const swiattn_events_t* events) {
  return swiattn_prefill_offset(Q, K, V, gate, idx, cnt, O, diff, B, N, Hq, Hkv, G, d, W, anchors, 0,
                                scale, dtype, flags, ws, ws_bytes, stream, events);
}

int swiattn_prefill_ex(const void* Q, const void* K, const void* V, const uint8_t* gate,
                       const int32_t* idx, const int32_t* cnt, void* O, float* diff, int B,
                       int N, int Hq, int Hkv, int G, int d, int W, float scale,
                       swiattn_dtype_t dtype, unsigned flags, void* ws, size_t ws_bytes,
                       swiattn_stream_t stream, const swiattn_events_t* events) {
  return swiattn_prefill_anchored(Q, K, V, gate, idx, cnt, O, diff, B, N, Hq, Hkv, G, d, W, 0,
                                  scale, dtype, flags, ws, ws_bytes, stream, events);
}

int swiattn_prefill(const void* Q, const void* K, const void* V, const uint8_t* gate,
                    const int32_t* idx, const int32_t* cnt, void* O, float* diff, int B, int N,
                    int Hq, int Hkv, int G, int d, int W, float scale, swiattn_dtype_t dtype,
                    unsigned flags, void* ws, size_t ws_bytes, swiattn_stream_t stream) {
  return swiattn_prefill_anchored(Q, K, V, gate, idx, cnt, O, diff, B, N, Hq, Hkv, G, d, W, 0,
                                  scale, dtype, flags, ws, ws_bytes, stream, nullptr);
}

size_t swiattn_decode_workspace_size(int B, int Lmax, int Hq, int Hkv, int G, int d, int W,
                                     swiattn_dtype_t dtype) {
  swi::DecodeShape sh;
  swi::DecodePlan p;
  if (decode_shape(B, Lmax, Hq, Hkv, G, d, W, 1.f, dtype, &sh, &p) != SWIATTN_OK) return 0;
  return p.bytes;
}

int swiattn_decode_offset(const void* q, const void* Kc, const void* Vc, const int32_t* cache_len,
                          const uint8_t* gate, void* o, int B, int Lmax, int Hq, int Hkv, int G,
                          int d, int W, int anchors, int offset, float scale, swiattn_dtype_t dtype,
                          void* ws, size_t ws_bytes, swiattn_stream_t stream,
                          const swiattn_events_t* events) {
  swi::DecodeShape sh;
  swi::DecodePlan p;
  const int rc = decode_shape(B, Lmax, Hq, Hkv, G, d, W, scale, dtype, &sh, &p);
  if (rc != SWIATTN_OK) return rc;
  if (anchors < 0 || offset < 0) return SWIATTN_ERR_INVALID_ARG;
  sh.A = anchors < Lmax ? anchors : Lmax;
  sh.off = offset < Lmax ? offset : Lmax;
  if (!q || !Kc || !Vc || !cache_len || !gate || !o) return SWIATTN_ERR_INVALID_ARG;
  if (!ws || ws_bytes < p.bytes) return SWIATTN_ERR_WORKSPACE;
  return hip_rc(swi::launch_decode(sh, p, q, Kc, Vc, cache_len, gate, o, ws,
                                   reinterpret_cast<hipStream_t>(stream),
                                   events ? events->ev : nullptr));
}

int swiattn_decode_anchored(const void* q, const void* Kc, const void* Vc,
                            const int32_t* cache_len, const uint8_t* gate, void* o, int B,
                            int Lmax, int Hq, int Hkv, int G, int d, int W, int anchors,
                            float scale, swiattn_dtype_t dtype, void* ws, size_t ws_bytes,
                            swiattn_stream_t stream, const swiattn_events_t* events) {
  return swiattn_decode_offset(q, Kc, Vc, cache_len, gate, o, B, Lmax, Hq, Hkv, G, d, W, anchors, 0,
                               scale, dtype, ws, ws_bytes, stream, events);
}

int swiattn_decode_ex(const void* q, const void* Kc, const void* Vc, const int32_t* cache_len,
                      const uint8_t* gate, void* o, int B, int Lmax, int Hq, int Hkv, int G,
                      int d, int W, float scale, swiattn_dtype_t dtype, void* ws,
                      size_t ws_bytes, swiattn_stream_t stream, const swiattn_events_t* events) {
  return swiattn_decode_anchored(q, Kc, Vc, cache_len, gate, o, B, Lmax, Hq, Hkv, G, d, W, 0,
                                 scale, dtype, ws, ws_bytes, stream, events);
}

int swiattn_decode(const void* q, const void* Kc, const void* Vc, const int32_t* cache_len,
                   const uint8_t* gate, void* o, int B, int Lmax, int Hq, int Hkv, int G, int d,
                   int W, float scale, swiattn_dtype_t dtype, void* ws, size_t ws_bytes,
                   swiattn_stream_t stream) {
  return swiattn_decode_anchored(q, Kc, Vc, cache_len, gate, o, B, Lmax, Hq, Hkv, G, d, W, 0,
                                 scale, dtype, ws, ws_bytes, stream, nullptr);
}

int swiattn_decode_noalloc(const void* q, const void* Kc, const void* Vc,
                           const int32_t* cache_len, const uint8_t* gate, void* o, int B, int Lmax,
                           int Hq, int Hkv, int G, int d, int W, float scale,
                           swiattn_dtype_t dtype, swiattn_stream_t stream) {
  swi::DecodeShape sh;
  swi::DecodePlan p;
  const int rc = decode_shape(B, Lmax, Hq, Hkv, G, d, W, scale, dtype, &sh, &p);
  if (rc != SWIATTN_OK) return rc;
  if (!q || !Kc || !Vc || !cache_len || !gate || !o) return SWIATTN_ERR_INVALID_ARG;
  // the decode plan must fit the fixed scratch (checked before any HIP call)
  if (p.bytes > swi::decode_scratch_bytes()) return SWIATTN_ERR_TOO_LARGE;
  void* ws = nullptr;
  const int src = hip_rc(swi::decode_scratch(&ws));
  if (src != SWIATTN_OK) return src;
  return hip_rc(swi::launch_decode(sh, p, q, Kc, Vc, cache_len, gate, o, ws,
                                   reinterpret_cast<hipStream_t>(stream), nullptr));
}

size_t swiattn_decode_noalloc_scratch_bytes(void) { return swi::decode_scratch_bytes(); }

int swiattn_decode_step_anchored(const void* Hn, const void* r, const float* bias, const void* q,
                                 const void* k, const void* v, void* Kc, void* Vc,
                                 int32_t* cache_len, uint8_t* gate, void* o, int B, int Lmax,
                                 int hidden, int Hq, int Hkv, int G, int d, int W, int anchors,
                                 float scale, swiattn_dtype_t dtype, void* ws, size_t ws_bytes,
                                 swiattn_stream_t stream) {
  swi::DecodeShape sh;
  swi::DecodePlan p;
  const int rc = decode_shape(B, Lmax, Hq, Hkv, G, d, W, scale, dtype, &sh, &p);
  if (rc != SWIATTN_OK) return rc;
  if (anchors < 0) return SWIATTN_ERR_INVALID_ARG;
  sh.A = anchors < Lmax ? anchors : Lmax;
  if (hidden < 1) return SWIATTN_ERR_INVALID_ARG;
  if (!Hn || !r || !bias || !q || !k || !v || !Kc || !Vc || !cache_len || !gate || !o)
    return SWIATTN_ERR_INVALID_ARG;
  if (!ws || ws_bytes < p.bytes) return SWIATTN_ERR_WORKSPACE;
  return hip_rc(swi::launch_decode_step(sh, p, Hn, r, bias, hidden, q, k, v, Kc, Vc, cache_len,
                                        gate, o, ws, reinterpret_cast<hipStream_t>(stream)));
}

int swiattn_decode_step(const void* Hn, const void* r, const float* bias, const void* q,
                        const void* k, const void* v, void* Kc, void* Vc, int32_t* cache_len,
                        uint8_t* gate, void* o, int B, int Lmax, int hidden, int Hq, int Hkv, int G,
                        int d, int W, float scale, swiattn_dtype_t dtype, void* ws, size_t ws_bytes,
                        swiattn_stream_t stream) {
  return swiattn_decode_step_anchored(Hn, r, bias, q, k, v, Kc, Vc, cache_len, gate, o, B, Lmax,
                                      hidden, Hq, Hkv, G, d, W, 0, scale, dtype, ws, ws_bytes,
                                      stream);
}

size_t swiattn_prefill_backward_workspace_size(int B, int N, int Hq) {
  if (B < 1 || N < 1 || Hq < 1) return 0;
  if ((long long)B * N > INT_MAX / 2 || (long long)B * Hq > INT_MAX / 2) return 0;
  return swi::backward_workspace(B, N, Hq);
}

int swiattn_prefill_backward(const void* Q, const void* K, const void* V, const void* O,
                             const void* dO, const uint8_t* gate, const int32_t* idx,
                             const int32_t* cnt, void* dQ, void* dK, void* dV, int B, int N,
                             int Hq, int Hkv, int G, int d, int W, float scale,
                             swiattn_dtype_t dtype, void* ws, size_t ws_bytes,
                             swiattn_stream_t stream) {
  if (B < 1 || N < 1 || !dtype_ok(dtype)) return SWIATTN_ERR_INVALID_ARG;
  const int rc = check_heads(Hq, Hkv, G, d, W, scale);
  if (rc != SWIATTN_OK) return rc;
  if ((long long)B * N > INT_MAX / 2 || (long long)B * Hq > INT_MAX / 2)
    return SWIATTN_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !O || !dO || !gate || !idx || !cnt || !dQ || !dK || !dV)
    return SWIATTN_ERR_INVALID_ARG;
  if (!ws || ws_bytes < swi::backward_workspace(B, N, Hq)) return SWIATTN_ERR_WORKSPACE;
  return hip_rc(swi::launch_backward(Q, K, V, O, dO, gate, idx, cnt, dQ, dK, dV, B, N, Hq, Hkv, G,
                                     d, W, scale, dtype == SWIATTN_F32, ws,
                                     reinterpret_cast<hipStream_t>(stream)));
}

size_t swiattn_router_backward_workspace_size(int B, int N, int hidden, int G) {
  if (B < 1 || N < 1 || hidden < 1 || G < 1) return 0;
  return swi::router_grad_workspace((int64_t)B * N, hidden, G);
}

int swiattn_router_backward(const void* dO, const void* O_full, const void* O_swa, const float* z,
                            const void* H, const void* r, float* dz, void* dH, float* dr,
                            float* dbias, int B, int N, int Hq, int d, int hidden, int G,
                            swiattn_dtype_t dtype, void* ws, size_t ws_bytes,
                            swiattn_stream_t stream) {
  if (B < 1 || N < 1 || Hq < 1 || hidden < 1 || G < 1 || !dtype_ok(dtype))
    return SWIATTN_ERR_INVALID_ARG;
  if (Hq % G != 0) return SWIATTN_ERR_INVALID_ARG;
  if (!dO || !O_full || !O_swa || !z || !H || !r || !dz || !dH || !dr || !dbias)
    return SWIATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return SWIATTN_ERR_UNSUPPORTED;
  if (hidden % 8 != 0 || G > swi::router_grad_max_groups()) return SWIATTN_ERR_UNSUPPORTED;
  if ((long long)B * N > INT_MAX / 2) return SWIATTN_ERR_UNSUPPORTED;
  const size_t need = swi::router_grad_workspace((int64_t)B * N, hidden, G);
  if (!ws || ws_bytes < need) return SWIATTN_ERR_WORKSPACE;
  return hip_rc(swi::launch_router_grad(dO, O_full, O_swa, z, H, r, dz, dH, dr, dbias, B, N, Hq, d,
                                        hidden, G, dtype == SWIATTN_F32, ws,
                                        reinterpret_cast<hipStream_t>(stream)));
}

const char* swiattn_strerror(int code) {
  switch (code) {
    case SWIATTN_OK: return "ok";
    case SWIATTN_ERR_INVALID_ARG: return "invalid argument";
    case SWIATTN_ERR_UNSUPPORTED: return "unsupported shape or head dimension";
    case SWIATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case SWIATTN_ERR_HIP: return "HIP runtime or launch error";
    case SWIATTN_ERR_TOO_LARGE:
      return "sizes exceed the fixed scratch of the allocation-free entry point";
    default: return "unknown error code";
  }
}

const char* swiattn_version(void) { return "0.1.0"; }

}  // extern "C"
