/*
 * swiattn.h - C ABI of the SwiAttn routed dual-branch attention library
 * (libswiattn.so, HIP for AMD MI355X / gfx950).
 *
 * The method (paper-daily report on SwiAttn, section 2 "方法详解"):
 *   - a per-token router: a linear map of the layer's hidden state gives a
 *     logit z, the soft gate is sigmoid(z), and the forward value of the
 *     straight-through estimator is the hard gate 1[sigmoid(z) > 0.5];
 *   - two attention branches on the same Q, K, V: full causal attention and
 *     sliding-window attention (SWA); the output is
 *     O = gate * O_FULL + (1 - gate) * O_SWA;
 *   - during decode both branches read one shared KV cache;
 *   - the adaptive regulariser uses the per-token squared L2 distance
 *     between the two branch outputs.
 * The SWA key set of query i is the W most recent keys including i itself,
 * [i-W+1, i] clipped at 0 (weimeta glossary "滑窗注意力 Sliding Window
 * Attention 是什么？", section "详细解释" and its W=4 table); the full
 * branch is causal, [0, i] (same glossary, FAQ on W equal to the context
 * length, where the window mask becomes the whole lower triangle).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *     aligned, dense row-major in the layouts given below.  The library
 *     allocates nothing and keeps no state between calls.
 *   - Work is enqueued on `stream` (0 = the default stream) and returns
 *     without synchronising the host.  Faults inside kernels surface at the
 *     caller's next synchronisation.
 *   - The dtype argument selects the storage type of Q/K/V/O (and of H, r
 *     for the router): SWIATTN_BF16 (bfloat16) or SWIATTN_F32 (float32).
 *     Scores, softmax statistics and accumulators are float32 in both cases;
 *     bf16 outputs are rounded to nearest even.
 *   - Head mapping: query head h reads KV head h / (Hq/Hkv) and gate group
 *     h / (Hq/G).  The two group sizes Hq/Hkv and Hq/G must nest (one divides
 *     the other) and Hq/Hkv must be at most 32.
 *   - Supported head dims: d = 64 or 128.
 *   - Return value: SWIATTN_OK (0) or a negative error code.  Argument
 *     errors are detected on the host before anything is enqueued; then no
 *     output is touched.
 */
#ifndef SWIATTN_H
#define SWIATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* swiattn_stream_t; /* same object as hipStream_t */

typedef enum { SWIATTN_BF16 = 0, SWIATTN_F32 = 1 } swiattn_dtype_t;

enum {
  SWIATTN_OK = 0,
  SWIATTN_ERR_INVALID_ARG = -1, /* null pointer, bad size, bad scale      */
  SWIATTN_ERR_UNSUPPORTED = -2, /* d not 64/128, group sizes not nested   */
  SWIATTN_ERR_WORKSPACE = -3,   /* workspace null or smaller than needed  */
  SWIATTN_ERR_HIP = -4,         /* a HIP launch or runtime call failed    */
  SWIATTN_ERR_TOO_LARGE = -5    /* sizes exceed the fixed scratch of
                                   swiattn_decode_noalloc                 */
};

/* Both-branch mode for swiattn_prefill: compute both branches for every
 * token and also write the per-token branch discrepancy `diff`. */
#define SWIATTN_FLAG_BOTH_BRANCH 1u

/*
 * swiattn_route - router logits, hard gate, and compaction of the tokens
 * routed to the full branch.
 * (SwiAttn report, section 2, router paragraph.)
 *
 *   H     [B,N,hidden] dtype   hidden states; may be NULL (see below)
 *   r     [hidden,G]   dtype   router weight (one column per gate group)
 *   bias  [G]          float   router bias
 *   gate  [B,N,G]      uint8   out: 1 = full branch, 0 = window branch.
 *                              When H == NULL it is an INPUT instead and
 *                              only the compaction runs (r, bias unused).
 *   z_out [B,N,G]      float   out, optional (NULL = not written): logits
 *   idx   [B,G,N]      int32   out: ascending token positions with gate=1;
 *                              entries at or beyond cnt are unspecified
 *   cnt   [B,G]        int32   out: number of gate=1 tokens
 *
 * z = sum_k H[b,i,k] r[k,g] + bias[g], accumulated in float32 in a fixed
 * order (bitwise reproducible); gate = (z > 0), which equals
 * sigmoid(z) > 0.5 without rounding a sigmoid.
 * Errors: INVALID_ARG for B,N,hidden,G < 1 or a required NULL pointer.
 */
int swiattn_route(const void* H, const void* r, const float* bias, uint8_t* gate,
                  float* z_out, int32_t* idx, int32_t* cnt, int B, int N, int hidden,
                  int G, swiattn_dtype_t dtype, swiattn_stream_t stream);

/*
 * swiattn_regularizer - adaptive regulariser of one layer, per token.
 * (SwiAttn report, section 2, adaptive regulariser paragraph.)
 *
 *   z     [B,N,G]  float  router logits R(h_t) (swiattn_route's z_out)
 *   nll   [B,N]    float  the token's negative log-likelihood
 *   diff  [B,N]    float  ||o_FULL - o_SWA||^2 of the token (swiattn_prefill's
 *                         both-branch output)
 *   loss  [B,N,G]  float  out: gamma_t * softplus(z) with
 *                         gamma_t = gamma_base / (eps + nll + alpha * diff)
 *
 * The pages use gamma_base = 1e-3, eps = 0.1, alpha = 100.  Every group's
 * logit of a token shares the token's gamma.  Computed in float32;
 * softplus(x) = max(x, 0) + log1p(e^-|x|).  Device pointers, caller-owned;
 * loss must not overlap the inputs.  NLL and diff are expected to be >= 0
 * (the denominator is then at least eps).
 * Errors: INVALID_ARG for B, N, G < 1, a NULL pointer, eps <= 0, alpha < 0
 * or a non-finite parameter.
 */
int swiattn_regularizer(const float* z, const float* nll, const float* diff, float* loss, int B,
                        int N, int G, float gamma_base, float eps, float alpha,
                        swiattn_stream_t stream);

/*
 * swiattn_prefill_workspace_size - bytes of device workspace that
 * swiattn_prefill needs for these sizes (an upper bound over every gate).
 * Returns 0 if the arguments are invalid.
 */
size_t swiattn_prefill_workspace_size(int B, int N, int Hq, int Hkv, int G, int d, int W,
                                      swiattn_dtype_t dtype, unsigned flags);

/*
 * swiattn_prefill - dual-branch attention forward over whole sequences.
 * (SwiAttn report, section 2, dual-branch and regulariser paragraphs.)
 *
 *   Q     [B,N,Hq,d]   dtype   queries (positions already encoded)
 *   K, V  [B,N,Hkv,d]  dtype   keys and values shared by both branches
 *   gate  [B,N,G]      uint8   hard gate (nonzero = full branch)
 *   idx   [B,G,N]      int32   compacted gate=1 positions, ascending, as
 *   cnt   [B,G]        int32   written by swiattn_route; ignored in
 *                              both-branch mode (may be NULL there)
 *   O     [B,N,Hq,d]   dtype   out: gate ? O_FULL : O_SWA, every row written
 *   diff  [B,N]        float   out, both-branch mode only (else may be
 *                              NULL): sum over heads and channels of
 *                              (O_FULL - O_SWA)^2 in float32, with O_SWA
 *                              as stored (rounded to dtype) and O_FULL
 *                              before rounding; exactly 0 for rows i < W
 *   W >= 1 (W >= N makes the two branches identical); scale > 0 is the
 *   softmax scale (1/sqrt(d) for standard attention).
 *   ws, ws_bytes: device workspace of at least
 *   swiattn_prefill_workspace_size(...) bytes, clobbered.
 *
 * Hard-gate mode runs the window branch for every row, the far part
 * [0, i-W] of the full branch only for gathered gate=1 rows, and merges the
 * two key sets by their log-sum-exp.  Both-branch mode runs the same
 * stages with every row taking the far part; its merge also writes the
 * distance and keeps O_SWA where the gate is 0.
 * Errors: INVALID_ARG (sizes < 1, NULL pointers, Hq % Hkv, Hq % G, scale),
 * UNSUPPORTED (d, group nesting, Hq/Hkv > 32), WORKSPACE.
 */
int swiattn_prefill(const void* Q, const void* K, const void* V, const uint8_t* gate,
                    const int32_t* idx, const int32_t* cnt, void* O, float* diff, int B,
                    int N, int Hq, int Hkv, int G, int d, int W, float scale,
                    swiattn_dtype_t dtype, unsigned flags, void* ws, size_t ws_bytes,
                    swiattn_stream_t stream);

/*
 * swiattn_decode_workspace_size - bytes of device workspace for
 * swiattn_decode (upper bound over every gate and cache length).
 * G is the number of gate groups of the call; it does not change the size
 * but is validated with the other head arguments (Hq % G, group nesting),
 * so a size query succeeds exactly when the matching decode call's shapes
 * are accepted.  Returns 0 if the arguments are invalid.
 */
size_t swiattn_decode_workspace_size(int B, int Lmax, int Hq, int Hkv, int G, int d, int W,
                                     swiattn_dtype_t dtype);

/*
 * swiattn_decode - one routed decode step per sequence on a shared KV cache.
 * (SwiAttn report, section 2: both branches share the KV cache in decode.)
 *
 *   q      [B,Hq,d]        dtype  the new token's queries
 *   Kc, Vc [B,Lmax,Hkv,d]  dtype  linear cache; positions 0..L-1 are valid
 *                                 and position L-1 holds the new token
 *   cache_len [B]          int32  L per sequence, 1 <= L <= Lmax (device
 *                                 memory: values outside are clamped)
 *   gate   [B,G]           uint8  hard gate of the new token
 *   o      [B,Hq,d]        dtype  out
 *   The full branch reads keys [0, L-1], the window branch the last
 *   min(W, L) keys.  Work is split into equal shares of 64-key blocks on
 *   the device from the gate and L (no host synchronisation); pieces of a
 *   (sequence, KV head) range cut by share boundaries are merged by
 *   log-sum-exp.
 * Errors: as swiattn_prefill.
 */
int swiattn_decode(const void* q, const void* Kc, const void* Vc, const int32_t* cache_len,
                   const uint8_t* gate, void* o, int B, int Lmax, int Hq, int Hkv, int G,
                   int d, int W, float scale, swiattn_dtype_t dtype, void* ws,
                   size_t ws_bytes, swiattn_stream_t stream);

/*
 * swiattn_decode_noalloc - swiattn_decode without a workspace argument and
 * without any device allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).
 *
 *   Arguments, outputs, arithmetic and errors are those of swiattn_decode;
 *   the split-K workspace lives instead in a fixed scratch array that the
 *   library holds in device memory, one copy per GPU, for the life of the
 *   process: swiattn_decode_noalloc_scratch_bytes() bytes (16 MiB).  Sizes
 *   whose decode workspace (swiattn_decode_workspace_size) exceeds it are
 *   rejected with SWIATTN_ERR_TOO_LARGE before anything is enqueued.  At
 *   Hq/Hkv = 4 and d = 128 the partials take 4 MiB whatever the cache
 *   length, and up to 1.5 million (sequence, KV head) pairs fit.
 *   Every call on one GPU uses that GPU's scratch: calls that overlap in
 *   time on one GPU (other streams, other threads) race and must be
 *   serialised by the caller.  Nothing in the scratch needs to start at
 *   zero; a call overwrites what it reads.  The scratch's device address
 *   is looked up on the first call on each device (hipGetSymbolAddress
 *   with that device current); the call allocates nothing.
 */
int swiattn_decode_noalloc(const void* q, const void* Kc, const void* Vc, const int32_t* cache_len,
                           const uint8_t* gate, void* o, int B, int Lmax, int Hq, int Hkv, int G,
                           int d, int W, float scale, swiattn_dtype_t dtype,
                           swiattn_stream_t stream);

/* Bytes of the fixed scratch used by swiattn_decode_noalloc. */
size_t swiattn_decode_noalloc_scratch_bytes(void);

/*
 * swiattn_decode_step - one serving step: route the new tokens, append
 * their keys and values to the shared cache, decode.
 * (SwiAttn report, section 2: router per token; in decode both branches
 * read one KV cache, so every new token is appended whatever its gate.)
 *
 *   Hn     [B,hidden]      dtype  the new tokens' hidden states (router input)
 *   r      [hidden,G]      dtype  router weight;  bias [G] float
 *   q      [B,Hq,d]        dtype  the new tokens' queries
 *   k, v   [B,Hkv,d]       dtype  the new tokens' keys and values
 *   Kc, Vc [B,Lmax,Hkv,d]  dtype  in/out: linear cache
 *   cache_len [B]          int32  in/out: L per sequence before the step,
 *                                 0 <= L <= Lmax; the new token goes to
 *                                 position L and L becomes L + 1.  A full
 *                                 cache (L = Lmax) is not appended and its
 *                                 sequence decodes over the cache as it is;
 *                                 a value below 0 is taken as 0
 *   gate   [B,G]           uint8  out: the new tokens' hard gate (as
 *                                 swiattn_route with N = 1)
 *   o      [B,Hq,d]        dtype  out: as swiattn_decode after the append
 *   ws, ws_bytes: as swiattn_decode (swiattn_decode_workspace_size).
 * Runs the router and the append (one launch) and then the decode on
 * `stream`, with no host synchronisation.  A sequence whose cache is full
 * must not be stepped: its append is skipped, cache_len stays Lmax and its
 * output is the decode of the new query over the unchanged cache, which
 * does not hold the new token's key (the library cannot report this on the
 * host, since the lengths live on the device; callers check L < Lmax).
 * Errors: as swiattn_decode, plus INVALID_ARG for hidden < 1 or a NULL
 * router or k/v pointer.
 */
int swiattn_decode_step(const void* Hn, const void* r, const float* bias, const void* q,
                        const void* k, const void* v, void* Kc, void* Vc, int32_t* cache_len,
                        uint8_t* gate, void* o, int B, int Lmax, int hidden, int Hq, int Hkv, int G,
                        int d, int W, float scale, swiattn_dtype_t dtype, void* ws, size_t ws_bytes,
                        swiattn_stream_t stream);

/*
 * Stage timing (for profilers and benchmarks).  `events` holds up to six
 * hipEvent_t handles created by the caller (stored as void*; NULL entries
 * are skipped).  The _ex calls behave exactly like the plain ones and in
 * addition record ev[i] on `stream` at stage boundary i:
 *   prefill, hard-gate mode: 0 before the far-part schedule, 1 after it,
 *     2 after the attention kernel (window tiles and far chunks), 3 after
 *     the merge;
 *   prefill, both-branch mode: the same four, and 4 after the per-token
 *     head sum of the distance;
 *   decode: 0 before the split-K kernel, 1 after it, 2 after the merge.
 * Passing events == NULL is the plain call.  Recording failures are
 * reported as SWIATTN_ERR_HIP.
 */
typedef struct {
  void* ev[6];
} swiattn_events_t;

int swiattn_prefill_ex(const void* Q, const void* K, const void* V, const uint8_t* gate,
                       const int32_t* idx, const int32_t* cnt, void* O, float* diff, int B,
                       int N, int Hq, int Hkv, int G, int d, int W, float scale,
                       swiattn_dtype_t dtype, unsigned flags, void* ws, size_t ws_bytes,
                       swiattn_stream_t stream, const swiattn_events_t* events);

int swiattn_decode_ex(const void* q, const void* Kc, const void* Vc, const int32_t* cache_len,
                      const uint8_t* gate, void* o, int B, int Lmax, int Hq, int Hkv, int G,
                      int d, int W, float scale, swiattn_dtype_t dtype, void* ws,
                      size_t ws_bytes, swiattn_stream_t stream, const swiattn_events_t* events);

/*
 * swiattn_prefill_anchored / swiattn_decode_anchored - the same calls with
 * global anchors in the window branch.
 * (weimeta glossary "滑窗注意力 Sliding Window Attention 是什么？", section
 * "SWA 落地的四个常见坑", pitfall 1, fix 2: the keys of the first tokens of
 * the document, 256 there, are listed apart and every query attends to them
 * in addition to its window, outside the sliding.)
 *
 *   anchors  A >= 0: the window-branch key set of query i becomes
 *            [0, min(A, i-W+1) - 1] union [max(0, i-W+1), i], every key
 *            once, in one softmax.  The full branch is unchanged ([0, i]
 *            already holds the anchors).  A = 0 is exactly swiattn_prefill /
 *            swiattn_decode; A >= N (prefill) or A >= Lmax (decode) is
 *            treated as N or Lmax.
 *   Every other argument, the workspace (same size queries: anchors need
 *   no extra space), the outputs and the events are those of
 *   swiattn_prefill_ex / swiattn_decode_ex (events may be NULL).
 *   Prefill: gate=1 rows take the far part [A, i-W] (empty when i-W < A);
 *   in both-branch mode diff is exactly 0 for rows i < W + A.
 *   Decode: a window head of a sequence with L = cache_len reads its anchors
 *   [0, min(A, L-W) - 1] from the same linear cache.
 * Errors: as swiattn_prefill / swiattn_decode, plus INVALID_ARG for A < 0.
 */
int swiattn_prefill_anchored(const void* Q, const void* K, const void* V, const uint8_t* gate,
                             const int32_t* idx, const int32_t* cnt, void* O, float* diff, int B,
                             int N, int Hq, int Hkv, int G, int d, int W, int anchors,
                             float scale, swiattn_dtype_t dtype, unsigned flags, void* ws,
                             size_t ws_bytes, swiattn_stream_t stream,
                             const swiattn_events_t* events);

int swiattn_decode_anchored(const void* q, const void* Kc, const void* Vc,
                            const int32_t* cache_len, const uint8_t* gate, void* o, int B,
                            int Lmax, int Hq, int Hkv, int G, int d, int W, int anchors,
                            float scale, swiattn_dtype_t dtype, void* ws, size_t ws_bytes,
                            swiattn_stream_t stream, const swiattn_events_t* events);

/*
 * swiattn_prefill_branches - both-branch prefill that also returns the two
 * branch outputs of every token, for training.
 * (SwiAttn report, section 2: the layer output is
 * O = sigma * O_FULL + (1 - sigma) * O_SWA, and the straight-through gate
 * passes the gradient <dO, O_FULL - O_SWA> to the router, so a training step
 * needs both branch outputs of every token; swiattn_router_backward takes
 * them.)
 *
 *   Q, K, V, gate, W, anchors, scale, dtype: as swiattn_prefill_anchored in
 *                both-branch mode (idx, cnt are not used)
 *   O      [B,N,Hq,d]  dtype  out: gate ? O_FULL : O_SWA
 *   diff   [B,N]       float  out: as swiattn_prefill's both-branch distance
 *   O_full [B,N,Hq,d]  dtype  out: the full-branch output of every token
 *   O_swa  [B,N,Hq,d]  dtype  out: the window-branch output of every token
 *   ws, ws_bytes: at least swiattn_prefill_workspace_size(...,
 *   SWIATTN_FLAG_BOTH_BRANCH) bytes, clobbered; events as swiattn_prefill_ex
 *   in both-branch mode (may be NULL).
 * One pass: the window tiles write O_SWA (and O_FULL of rows whose window
 * and anchors hold every key [0, i]), the merge writes O_FULL of the other
 * rows.  O, O_FULL and O_SWA hold the same values as the gated output where
 * the gate picks them.  Outputs must not overlap each other or the inputs.
 * Errors: as swiattn_prefill, plus INVALID_ARG for a NULL output.
 */
int swiattn_prefill_branches(const void* Q, const void* K, const void* V, const uint8_t* gate,
                             void* O, float* diff, void* O_full, void* O_swa, int B, int N, int Hq,
                             int Hkv, int G, int d, int W, int anchors, float scale,
                             swiattn_dtype_t dtype, void* ws, size_t ws_bytes, swiattn_stream_t stream,
                             const swiattn_events_t* events);

/*
 * swiattn_prefill_offset / swiattn_decode_offset - the anchored calls with a
 * window offset, for stacked layers whose windows are staggered.
 * (weimeta glossary "滑窗注意力 Sliding Window Attention 是什么？", section
 * "两个核心工程参数（W 和步长 S）详解": the stride S offsets the windows of
 * different layers, e.g. 0, W/4, W/2, 3W/4 in turn, so that together they
 * reach past W; section "SWA 落地的四个常见坑", pitfall 2, fix (2): the
 * windows of layers 0, 1, 2 are [0, W], [W/2, 3W/2], [W, 2W].)
 *
 *   offset  o >= 0: the window branch of query i takes the window and the
 *           anchors of query i - o: keys [max(0, i-o-W+1), i-o] (the W keys
 *           at distances o .. o+W-1 behind the query; the query itself only
 *           for o = 0) and [0, min(A, i-o-W+1) - 1].  A row i < o has no
 *           window key: its window-branch output is 0.  The full branch is
 *           unchanged ([0, i]).  o = 0 is swiattn_prefill_anchored /
 *           swiattn_decode_anchored; o >= N (prefill) or o >= Lmax (decode)
 *           is treated as N or Lmax.
 *   Decode: a window head of a sequence with L = cache_len takes the window
 *   of position L-1-o (output 0 when L <= o).
 *   Every other argument, the workspace (same size queries), the outputs
 *   and the events are those of the anchored calls.
 * Errors: as the anchored calls, plus INVALID_ARG for offset < 0 and
 * UNSUPPORTED for offset > 0 in both-branch mode.
 */
int swiattn_prefill_offset(const void* Q, const void* K, const void* V, const uint8_t* gate,
                           const int32_t* idx, const int32_t* cnt, void* O, float* diff, int B, int N,
                           int Hq, int Hkv, int G, int d, int W, int anchors, int offset, float scale,
                           swiattn_dtype_t dtype, unsigned flags, void* ws, size_t ws_bytes,
                           swiattn_stream_t stream, const swiattn_events_t* events);

int swiattn_decode_offset(const void* q, const void* Kc, const void* Vc, const int32_t* cache_len,
                          const uint8_t* gate, void* o, int B, int Lmax, int Hq, int Hkv, int G,
                          int d, int W, int anchors, int offset, float scale, swiattn_dtype_t dtype,
                          void* ws, size_t ws_bytes, swiattn_stream_t stream,
                          const swiattn_events_t* events);

/* swiattn_decode_step_anchored - swiattn_decode_step whose decode has the
 * global anchors above (the anchors stay in the linear cache like every
 * key); anchors = 0 is swiattn_decode_step.  Same arguments, workspace and
 * errors, plus INVALID_ARG for anchors < 0. */
int swiattn_decode_step_anchored(const void* Hn, const void* r, const float* bias, const void* q,
                                 const void* k, const void* v, void* Kc, void* Vc,
                                 int32_t* cache_len, uint8_t* gate, void* o, int B, int Lmax,
                                 int hidden, int Hq, int Hkv, int G, int d, int W, int anchors,
                                 float scale, swiattn_dtype_t dtype, void* ws, size_t ws_bytes,
                                 swiattn_stream_t stream);

/*
 * swiattn_router_backward - gradient that reaches the router through the
 * straight-through gate.
 * (SwiAttn report, section 2: the hard gate is
 * sigma = 1(soft > 0.5) + soft - sg(soft) with soft = sigmoid(R(H)), so its
 * forward value is the 0/1 decision and its backward derivative the
 * sigmoid's; the layer output is O = sigma * O_FULL + (1 - sigma) * O_SWA.)
 *
 *   dO            [B,N,Hq,d]  dtype  gradient of the loss w.r.t. O
 *   O_full, O_swa [B,N,Hq,d]  dtype  the two branch outputs of the forward
 *                                    (e.g. prefill with the gate all ones /
 *                                    all zeros)
 *   z             [B,N,G]     float  router logits (swiattn_route's z_out)
 *   H             [B,N,hidden] dtype hidden states, r [hidden,G] dtype weight
 *   dz            [B,N,G]     float  out: soft'(z) * sum over the heads of
 *                                    group g and their channels of
 *                                    dO * (O_full - O_swa)
 *   dH            [B,N,hidden] dtype out: sum_g dz r[:,g]
 *   dr            [hidden,G]  float  out: sum over tokens of H dz
 *   dbias         [G]         float  out: sum over tokens of dz
 *   ws, ws_bytes: device workspace of at least
 *   swiattn_router_backward_workspace_size(B, N, hidden, G) bytes, clobbered.
 * Query head h belongs to gate group h / (Hq/G).  Sums are float32 in a fixed
 * order (bitwise reproducible); soft'(z) is evaluated as
 * e^-|z| / (1 + e^-|z|)^2.  The gradients that reach Q, K, V through the
 * two branch outputs are not computed.  Outputs must not overlap inputs.
 * Errors: INVALID_ARG (sizes < 1, Hq % G, NULL pointers), UNSUPPORTED
 * (d not 64/128, hidden not a multiple of 8, G > 64), WORKSPACE.
 */
size_t swiattn_router_backward_workspace_size(int B, int N, int hidden, int G);

int swiattn_router_backward(const void* dO, const void* O_full, const void* O_swa, const float* z,
                            const void* H, const void* r, float* dz, void* dH, float* dr,
                            float* dbias, int B, int N, int Hq, int d, int hidden, int G,
                            swiattn_dtype_t dtype, void* ws, size_t ws_bytes,
                            swiattn_stream_t stream);

/*
 * swiattn_prefill_backward - gradients of L = sum(dO * O) with respect to
 * Q, K, V for the hard-gated prefill.
 * (SwiAttn report, section 2: with a 0/1 forward gate, row i of a head in
 * gate group g is softmax attention over [0, i] (gate 1) or
 * [max(0, i-W+1), i] (gate 0); weimeta glossary "详细解释" for the window.)
 *
 *   Q, dO [B,N,Hq,d], K, V [B,N,Hkv,d], O [B,N,Hq,d]  dtype  the forward's
 *                    inputs, its output (swiattn_prefill) and the output's
 *                    gradient
 *   gate [B,N,G] uint8, idx [B,G,N] / cnt [B,G] int32  the forward's gate
 *                    and its compaction (swiattn_route)
 *   dQ [B,N,Hq,d], dK, dV [B,N,Hkv,d]  dtype  out (K, V gradients summed
 *                    over the query heads of each KV head)
 *   W, scale as swiattn_prefill.  ws, ws_bytes: at least
 *   swiattn_prefill_backward_workspace_size(B, N, Hq) bytes (each row's
 *   log-sum-exp and <dO, O>), clobbered.
 * Only the attention path: the gate's gradient is swiattn_router_backward's.
 * Arithmetic, in a fixed order (bitwise reproducible):
 *   bf16:    every product on the matrix cores (bf16 operands, float32
 *            accumulation).  Scores, softmax and D = <dO, O> are float32;
 *            the probabilities P and dS = P (dP - D) are rounded to bf16
 *            where they become operands of the dV, dQ and dK products.
 *            One launch for dQ (the gathered gate=1 rows first, then the
 *            gate=0 rows; it also writes LSE and D to the workspace), one
 *            for dK and dV (a workgroup per 64 keys of a KV head).
 *   float32: float32 throughout on the vector ALUs, 16 lanes per (row,
 *            query head) for dQ and per (key, KV head) for dK and dV.
 * Outputs must not overlap inputs.
 * Errors: as swiattn_prefill (INVALID_ARG, UNSUPPORTED, WORKSPACE).
 */
size_t swiattn_prefill_backward_workspace_size(int B, int N, int Hq);

int swiattn_prefill_backward(const void* Q, const void* K, const void* V, const void* O,
                             const void* dO, const uint8_t* gate, const int32_t* idx,
                             const int32_t* cnt, void* dQ, void* dK, void* dV, int B, int N,
                             int Hq, int Hkv, int G, int d, int W, float scale,
                             swiattn_dtype_t dtype, void* ws, size_t ws_bytes,
                             swiattn_stream_t stream);

/* Static text for an error code. */
const char* swiattn_strerror(int code);

/* Library version, e.g. "0.1.0". */
const char* swiattn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SWIATTN_H */
