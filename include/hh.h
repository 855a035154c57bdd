/*
 * libhymba_hh -- the Hymba hybrid-head layer on AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every tensor argument is a DEVICE pointer to row-major memory owned
 * by the caller; the library never allocates, frees or keeps a pointer after a
 * call returns.  Work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and the calls return without synchronising.
 *
 * Errors: a call returns HH_OK or an error code and never throws.  Arguments
 * are validated on the host BEFORE anything is enqueued, so on an error no
 * buffer has been touched; hh_last_error() then holds a message (per thread).
 * HH_ERR_HIP reports a failed kernel launch; output buffers may then be
 * partially written, except when the first stage of a call fails (nothing has
 * been enqueued yet).  For tests, the environment variable HH_FAULT_INJECT set
 * to a stage name (e.g. "inproj", "scan", "decode_inproj", "decode_norm")
 * makes that stage report a failed launch on the host without launching.
 *
 * Launch-plan switches read from the environment at each hh_prefill call
 * (every plan computes the same values; the defaults are the fastest measured):
 *   HH_FUSED_NORM=0           bf16 prefills of 1024+ rows run the fusion step
 *                             as its own kernel instead of inside the output
 *                             projection (same result up to bf16 rounding);
 *   HH_CONCURRENT_BRANCHES=1  the SSM branch runs on a library side stream
 *                             beside the input projection and the attention;
 *   HH_ONE_LAUNCH_BRANCHES=1  (bf16) the attention and the scan's last pass
 *                             run in one grid of role-split workgroups.
 * The last two give results identical bit for bit to the default plan.
 *
 * What the layer computes (the method of "Hymba: A Hybrid-head Architecture
 * for Small Language Models", arXiv 2411.13676, and the authors' OpenReview
 * replies on implementation details):
 *   X~ = [R; X]                   meta tokens R prepended          (§2.3, Eq. 4)
 *   P  = X~ W_in^T                one fused input projection       (§2.1)
 *        columns Q | K | V | xs | z | dt | B | C  (K, V absent in a KV-sharing
 *        consumer layer, which reads its producer's K/V)  (reply on cache
 *        optimisation; §2.2 cross-layer KV sharing)
 *   O  = softmax(Q K^T / sqrt(hd)) V per head, grouped-query (head h reads KV
 *        head h / (H/G)), over all meta keys plus the real keys j with
 *        i - W < j <= i (sliding window) or j <= i (global layer)
 *        (§2.1 Eq. 1, §2.2, reply on the "A-shape" mask and the 1/sqrt(d) scale)
 *   u  = SiLU(causal depthwise conv_k(xs) + conv_b)
 *   Delta = softplus(dt + dt_bias)
 *   h_t = exp(Delta_t A) h_{t-1} + Delta_t u_t B_t,  y_t = h_t . C_t,
 *   Y  = y * SiLU(z)                                        (§2.1 Eq. 2)
 *   F  = 1/2 [beta_attn * rmsnorm(O) || beta_ssm * rmsnorm(Y)]
 *   out = F W_out^T                                         (§2.1 Eq. 3)
 * The meta rows depend on nothing but the weights, so their part (meta K/V,
 * SSM state and conv history after the meta rows) is computed once by
 * hh_meta_prefix and reused (§2.3: computed offline, a learned cache
 * initialisation).
 *
 * Storage types: `dtype` (HH_F32 or HH_BF16) is the element type of x, out,
 * meta tokens, W_in, W_out and the K/V buffers and caches.  dt_bias, A,
 * conv_w, conv_b, the betas and the whole SSM state (h and the conv history)
 * are always fp32.  The bf16 path accumulates in fp32 and keeps the SSM input
 * features, Delta, B, C, softmax, norms and the SSM state in fp32.
 *
 * Supported shapes: head_dim 32 or 64 (bf16: 64); n_heads a multiple of
 * n_kv_heads with at most 8 query heads per KV head; d_state 16; d_conv 2..4;
 * d_model, n_heads*head_dim + d_inner and d_inner multiples of 8 (bf16: d_model
 * and n_heads*head_dim + d_inner multiples of 64); d_model, n_heads*head_dim
 * and d_inner at most 16384 (bf16) or 8192 (fp32).  Every one of these limits
 * is checked before any launch (HH_ERR_UNSUPPORTED).
 */
#ifndef HH_H
#define HH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { HH_F32 = 0, HH_BF16 = 1 } hh_dtype;

typedef enum {
  HH_OK = 0,
  HH_ERR_INVALID_ARG = 1,  /* null pointer, bad size, inconsistent shape */
  HH_ERR_UNSUPPORTED = 2,  /* valid but not implemented (e.g. head_dim 128) */
  HH_ERR_WORKSPACE = 3,    /* ws_bytes smaller than the *_workspace_size */
  HH_ERR_HIP = 4           /* a HIP launch failed */
} hh_status;

/* Layer shape.  n_heads = H query heads, n_kv_heads = G query groups,
 * d_inner = D SSM channels, d_state = N, d_conv = k taps, n_meta = m.
 *
 * rope_base: rotary position embedding of Q and K (Hymba paper §3: the
 * model is trained with RoPE and its base is changed for the 8k stage; the
 * pages give neither the base nor the convention).  0 = none.  Otherwise
 * dims i and i + head_dim/2 of every Q and K head form pair i and are turned
 * by the angle pos * rope_base^(-2i/head_dim), (a, b) -> (a cos - b sin,
 * b cos + a sin), right after the input projection, so the meta K/V, the
 * prefill K/V and the cache all hold rotated keys.  pos counts the rows of
 * [R; X]: meta token j is at position j, real position p at n_meta + p (a
 * decode token at real position len[b], or len[b] - 1 for a KV-sharing
 * consumer, likewise).  Must be 0 or a finite value > 1.
 *
 * ssm_heads: the SSM heads' form (the authors' reply on Mamba vs Mamba2: the
 * hybrid head works with either; shapes not given).  0 = Mamba (Eq. 2 as
 * written: Delta per channel, A per channel and state).  S > 0 = Mamba2: the
 * d_inner channels form S heads of P = d_inner / S consecutive channels, each
 * head with one Delta_t (the dt block of w_in has S rows, dt_bias [S]) and
 * one negative scalar A (A [S]); h_t[c,s] = exp(Delta_t[h] A[h]) h_{t-1}[c,s]
 * + Delta_t[h] u_t[c] B_t[s] with h = c / P.  S must divide d_inner and be a
 * multiple of 4. */
typedef struct {
  int32_t d_model, n_heads, n_kv_heads, head_dim;
  int32_t d_inner, d_state, d_conv, n_meta;
  int32_t dtype;   /* hh_dtype */
  float rms_eps;   /* epsilon inside the RMS norm of both branches */
  float rope_base; /* rotary embedding base of Q and K; 0 = none */
  int32_t ssm_heads; /* Mamba2 SSM heads S (see below); 0 = Mamba heads */
} hh_dims;

/* One layer's parameters (all device pointers, read only).
 *   w_in      [n_in, d_model] dtype, rows Q (H*hd) | K (G*hd) | V (G*hd) |
 *             xs (D) | z (D) | dt (D, or S for Mamba2 heads) | B (N) | C (N);
 *             the K and V rows are absent when kv_producer == 0
 *             (n_in = H*hd + 3D + 2N for Mamba heads).
 *   dt_bias   [D] fp32       A [D, N] fp32 (negative)
 *             (Mamba2 heads: dt_bias [S], A [S])
 *   conv_w    [D, k] fp32 (tap k-1 multiplies the current row)   conv_b [D] fp32
 *   beta_attn [H*hd] fp32    beta_ssm [D] fp32
 *   w_out     [d_model, H*hd + D] dtype
 *   kv_producer: 1 = computes and stores K/V; 0 = KV-sharing consumer. */
typedef struct {
  const void *w_in;
  const float *dt_bias;
  const float *A;
  const float *conv_w;
  const float *conv_b;
  const float *beta_attn;
  const float *beta_ssm;
  const void *w_out;
  int32_t kv_producer;
} hh_weights;

/* A layer's meta-token part, shared by every sequence (pinned, read only).
 *   k, v       [G, m, hd] dtype: meta keys/values (a consumer layer passes
 *              its producer's)
 *   h0         [D, N] fp32: SSM state after the m meta rows
 *   conv_tail  [k-1, D] fp32: xs of the last k-1 meta rows (oldest first) */
typedef struct {
  const void *k, *v;
  const float *h0;
  const float *conv_tail;
} hh_meta;

/* K/V of real tokens.
 *   full_k, full_v  [B, G, seqlen, hd] dtype: prefill K/V of every real
 *                   token.  A producer writes them (NULL: kept in the
 *                   workspace only); a consumer reads its producer's here.
 *   cache_k, cache_v [B, G, cap, hd] dtype: decode cache.  Real position p
 *                   lives in slot p % cap when is_ring, else slot p.  Prefill
 *                   by a producer fills the slots of the last min(seqlen, cap)
 *                   positions (ring) or of positions < seqlen (linear); NULL
 *                   skips the cache.
 *   len             [B] int32: real positions held.  Prefill by a producer sets
 *                   it to seqlen (NULL skips).  Decode: a producer appends at
 *                   position len[b] and then increments len[b]; a consumer
 *                   attends up to position len[b]-1 (the token its producer
 *                   appended this step) and writes nothing.
 *                   Prefill into a linear cache needs cap >= seqlen
 *                   (HH_ERR_INVALID_ARG otherwise).  Decoding a sequence whose
 *                   linear cache is full (len[b] >= cap) is a caller error:
 *                   len lives on the device, so it is not checked before the
 *                   launch; the kernels then write no slot and leave len[b]
 *                   unchanged (the sequence's output for that step does not
 *                   include the new token).
 *   cap, is_ring    slots per sequence and head; ring caches need window <= cap. */
typedef struct {
  void *full_k, *full_v;
  void *cache_k, *cache_v;
  int32_t *len;
  int32_t cap;
  int32_t is_ring;
} hh_kv;

/* Per-sequence SSM state.
 *   h     [B, D, N] fp32
 *   conv  [B, k-1, D] fp32: xs of the last k-1 positions, oldest first. */
typedef struct {
  float *h;
  float *conv;
} hh_ssm_state;

/* Library version string, e.g. "libhymba_hh 0.1.0 gfx950". */
const char *hh_version(void);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *hh_last_error(void);

/* Bytes of device workspace hh_meta_prefix needs (0 on invalid dims). */
size_t hh_meta_prefix_workspace_size(const hh_dims *dims, int32_t kv_producer);

/* The meta-token part of one layer (paper §2.3: fixed meta tokens, computed
 * offline).  meta_tokens [m, d_model] dtype.  Writes meta_k/meta_v
 * [G, m, hd] dtype (producer layers only; ignored and may be NULL for a
 * consumer), h0 [D, N] fp32 (state after the meta rows, from a zero state)
 * and conv_tail [k-1, D] fp32 (xs of the last k-1 meta rows; zero rows in
 * front when m < k-1). */
hh_status hh_meta_prefix(const hh_dims *dims, const hh_weights *w,
                         const void *meta_tokens, void *meta_k, void *meta_v,
                         float *h0, float *conv_tail, void *ws, size_t ws_bytes,
                         void *stream);

/* Bytes of device workspace hh_prefill needs (0 on invalid arguments). */
size_t hh_prefill_workspace_size(const hh_dims *dims, int32_t batch,
                                 int32_t seqlen, int32_t kv_producer);

/* Prefill of `seqlen` real tokens per sequence after the meta tokens
 * (paper §2.1 Eqs. 1-3 over X~ of §2.3 Eq. 4).
 *   x      [B, seqlen, d_model] dtype
 *   meta   the layer's hh_meta (its h0 and conv_tail start the SSM branch)
 *   window sliding-window length W >= 1 (ignored when is_global)
 *   out    [B, seqlen, d_model] dtype
 *   kv     see hh_kv (producer writes, consumer reads full_k/full_v)
 *   state  if not NULL: receives h after the last token and the conv history
 *          (either member may be NULL to skip it). */
hh_status hh_prefill(const hh_dims *dims, const hh_weights *w, const void *x,
                     int32_t batch, int32_t seqlen, const hh_meta *meta,
                     int32_t window, int32_t is_global, void *out, hh_kv *kv,
                     hh_ssm_state *state, void *ws, size_t ws_bytes,
                     void *stream);

/* Bytes of device workspace hh_decode_step needs for `batch` sequences whose
 * cache has `cap` slots (0 on invalid arguments). */
size_t hh_decode_workspace_size(const hh_dims *dims, int32_t batch, int32_t cap,
                                int32_t kv_producer);

/* One new token per sequence (generation with the KV cache and SSM state;
 * authors' replies: KV-sharing groups of two consecutive sliding-window layers,
 * meta K/V precomputed and pinned).
 *   x_t    [B, d_model] dtype;  out [B, d_model] dtype
 *   meta   pinned meta K/V of the cache (shared by all sequences)
 *   kv     cache_k/cache_v/len/cap/is_ring used (full_* ignored)
 *   state  h and conv read and updated in place (both required). */
hh_status hh_decode_step(const hh_dims *dims, const hh_weights *w,
                         const void *x_t, int32_t batch, const hh_meta *meta,
                         int32_t window, int32_t is_global, hh_kv *kv,
                         hh_ssm_state *state, void *out, void *ws,
                         size_t ws_bytes, void *stream);

/* hh_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same step with no workspace argument.  Its scratch is a static device
 * array of HH_STATIC_SCRATCH_BYTES inside the library, one per GPU, held until
 * the process ends; the call itself allocates nothing.  Arguments, results
 * and errors as for hh_decode_step, plus HH_ERR_WORKSPACE (before anything
 * is enqueued) when the step needs more scratch than that, i.e. more than
 * hh_decode_workspace_size() reports (32 MiB covers batch 128 at 1.5B widths
 * with caches of up to 32768 slots).  Every call on one GPU shares that GPU's
 * scratch: calls that can overlap on one GPU (different streams or host
 * threads without ordering between them) race and must be serialised by the
 * caller. */
#define HH_STATIC_SCRATCH_BYTES (32u << 20)
hh_status hh_decode_step_noalloc(const hh_dims *dims, const hh_weights *w,
                                 const void *x_t, int32_t batch, const hh_meta *meta,
                                 int32_t window, int32_t is_global, hh_kv *kv,
                                 hh_ssm_state *state, void *out, void *stream);

/* ---- the block around the layer ---------------------------------------
 * One block (Hymba paper, Fig. 4 and the architecture table's MLP width):
 *   x1  = x + layer(g1 * rms(x))            (the layer above, meta rows g1 * rms(R))
 *   out = x1 + W_down (SiLU(W_gate v) * (W_up v)),  v = g2 * rms(x1)
 * with rms(v) = v / sqrt(mean(v^2) + rms_eps) per row, fp32 statistics.
 *   mixer      the layer's weights (hh_weights)
 *   norm1, norm2 [d_model] fp32 gains
 *   w_gate_up  [2 d_ff, d_model] dtype; rows alternate gate, up (row 2i is the
 *              gate of hidden unit i, row 2i+1 its up projection)
 *   w_down     [d_model, d_ff] dtype
 *   d_ff       MLP hidden width: a multiple of 4 (fp32) or 64 (bf16); 5504 at 1.5B */
typedef struct {
  hh_weights mixer;
  const float *norm1, *norm2;
  const void *w_gate_up;
  const void *w_down;
  int32_t d_ff;
} hh_block_weights;

/* Bytes of device workspace hh_block_meta_prefix needs (0 on invalid dims). */
size_t hh_block_meta_prefix_workspace_size(const hh_dims *dims, int32_t kv_producer);

/* hh_meta_prefix of the block's layer, whose meta rows are g1 * rms(R):
 * meta_tokens [m, d_model] dtype are the block's meta inputs R. */
hh_status hh_block_meta_prefix(const hh_dims *dims, const hh_block_weights *w,
                               const void *meta_tokens, void *meta_k, void *meta_v,
                               float *h0, float *conv_tail, void *ws, size_t ws_bytes,
                               void *stream);

/* Bytes of device workspace hh_block_prefill needs (0 on invalid arguments). */
size_t hh_block_prefill_workspace_size(const hh_dims *dims, int32_t d_ff, int32_t batch,
                                       int32_t seqlen, int32_t kv_producer);

/* hh_prefill of one block: arguments as for hh_prefill, x and out the block's
 * input and output [B, seqlen, d_model] dtype (out must not alias x); kv and
 * state are the layer's.  The residual stream is kept in dtype. */
hh_status hh_block_prefill(const hh_dims *dims, const hh_block_weights *w, const void *x,
                           int32_t batch, int32_t seqlen, const hh_meta *meta,
                           int32_t window, int32_t is_global, void *out, hh_kv *kv,
                           hh_ssm_state *state, void *ws, size_t ws_bytes, void *stream);

/* Bytes of device workspace hh_block_decode_step needs (0 on invalid arguments). */
size_t hh_block_decode_workspace_size(const hh_dims *dims, int32_t d_ff, int32_t batch,
                                      int32_t cap, int32_t kv_producer);

/* hh_decode_step of one block: arguments as for hh_decode_step, x_t and out
 * [B, d_model] dtype (out must not alias x_t). */
hh_status hh_block_decode_step(const hh_dims *dims, const hh_block_weights *w,
                               const void *x_t, int32_t batch, const hh_meta *meta,
                               int32_t window, int32_t is_global, hh_kv *kv,
                               hh_ssm_state *state, void *out, void *ws,
                               size_t ws_bytes, void *stream);

/* Workspace regions of hh_prefill, for inspecting intermediate results after
 * a call (test and debugging aid).  Fills offs[HH_WS_COUNT] with byte offsets
 * (SIZE_MAX for a region that is not used) and returns the total size. */
enum {
  HH_WS_Q = 0,   /* [B*n, H*hd] dtype */
  HH_WS_K,       /* [B, G, n, hd] dtype (used when full_k is NULL) */
  HH_WS_V,
  HH_WS_XS,      /* SSM input features, fp32; these three regions hold  */
  HH_WS_Z,       /* [B*n, D] (Delta: [B*n, D or S]) channel-block-major: */
  HH_WS_DELTA,   /* element (r, c) at ((c/64)*B*n + r)*64 + c%64; Delta softplus'd */
  HH_WS_BC,      /* [B*n, 2N] fp32: B then C */
  HH_WS_O,       /* [B*n, H*hd] dtype attention output */
  HH_WS_Y,       /* [B*n, D] dtype gated SSM output */
  HH_WS_F,       /* [B*n, H*hd + D] dtype fused features */
  HH_WS_SCAN,    /* scan chunk carries */
  HH_WS_GEMM,    /* split-K partial sums of the projections (few-row calls) */
  HH_WS_SSQ,     /* fp32 partial row sums of squares of the branch
                    outputs: [B*n, G] (O^2 per row and KV group), then
                    [B*n, ceil(D/64)] (Y^2 per row and 64-channel block).
                    Written by bf16 prefills of 1024+ rows, where the
                    fusion runs inside the output projection: O and Y then
                    hold beta-scaled values and F is not written */
  HH_WS_COUNT
};
size_t hh_prefill_workspace_layout(const hh_dims *dims, int32_t batch,
                                   int32_t seqlen, int32_t kv_producer,
                                   size_t *offs);

/* ---- stage hooks (test aids) -------------------------------------------
 * The prefill's own kernels on caller-given inputs, so each branch can be
 * compared with a plain implementation on its own; hh_prefill runs the same
 * kernels.  Validation and errors as for hh_prefill (nothing is enqueued on
 * an error); all work goes to `stream`.
 *
 * hh_stage_attn: the attention heads of Hymba paper §2.1 Eq. (1) with the
 * meta tokens of §2.3 and the window of §2.2 (real query i sees every meta
 * key and the real keys j with i - window < j <= i, or j <= i when
 * is_global).  q [B*n, H*hd], k and v [B, G, n, hd], meta_k and meta_v
 * [G, n_meta, hd] (NULL when n_meta is 0), o [B*n, H*hd]: dtype, 16-byte
 * aligned, caller-owned.  The rotary embedding, if any, is not applied here
 * (q and k are taken as given). */
hh_status hh_stage_attn(const hh_dims *dims, const void *q, const void *k, const void *v,
                        const void *meta_k, const void *meta_v, int32_t batch,
                        int32_t seqlen, int32_t window, int32_t is_global, void *o,
                        void *stream);

/* hh_stage_ssm: the SSM heads of Eq. (2) from their input features: the
 * causal conv + SiLU on xs, the selective scan from h0 and the gate SiLU(z).
 * Uses w->A, w->conv_w, w->conv_b only.  xs (fp32), z (dtype) and delta (fp32,
 * softplus already applied; D columns, or ssm_heads for Mamba2 heads) are in
 * the channel-block-major layout of the prefill workspace over R = B*n rows:
 * element (r, c) at ((c/64)*R + r)*64 + c%64, whole 64-column blocks.
 * bc [B*n, 2*d_state] fp32 (B_t then C_t).  h0 [D, N] and conv_tail
 * [d_conv-1, D] fp32 start every sequence (NULL: zero).  Outputs: y [B*n, D]
 * dtype, h_out [B, D, N] fp32 and tail_out [B, d_conv-1, D] fp32 (each may be
 * NULL).  ws: at least hh_stage_ssm_workspace_size bytes (chunk carries). */
size_t hh_stage_ssm_workspace_size(const hh_dims *dims, int32_t batch, int32_t seqlen);
hh_status hh_stage_ssm(const hh_dims *dims, const hh_weights *w, const float *xs,
                       const void *z, const float *delta, const float *bc,
                       const float *h0, const float *conv_tail, int32_t batch,
                       int32_t seqlen, void *y, float *h_out, float *tail_out, void *ws,
                       size_t ws_bytes, void *stream);

/* Per-stage GPU timing (measurement aid, off by default).  While enabled on
 * the calling thread, each kernel stage an entry point enqueues (in-proj GEMM,
 * attention, scan, norm/average, out-proj GEMM, decode kernels) is bracketed
 * by HIP events recorded on the caller's stream.  hh_timing_read waits for the
 * recorded events, writes up to max_stages per-stage summaries (launches and
 * summed milliseconds, stages in first-seen order), clears the record and
 * returns the number of stages written, or -1 on a HIP error. */
typedef struct {
  char name[32];
  int32_t launches;
  double total_ms;
} hh_stage_time;
hh_status hh_timing_enable(int32_t on);
int32_t hh_timing_read(hh_stage_time *out, int32_t max_stages);

#ifdef __cplusplus
}
#endif
#endif /* HH_H */
