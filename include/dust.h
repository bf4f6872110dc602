/*
 * dust.h -- C ABI of the MI355X (gfx950) Dust gradient-estimator library.
 *
 * Dust (Q Labs, 2026) estimates the gradient of a Transformer linear layer
 * y_t = W x_t without backprop: every token's layer output gets K independent
 * Gaussian perturbations sigma * a_t^(i); the loss downstream of the layer is
 * recomputed per draw; the reward r_t^(i) is the clean per-token cross-entropy
 * minus the perturbed one; the output-error estimate is
 *     g_hat_t = -(1/(K sigma)) sum_i r_t^(i) a_t^(i)
 * and the weight-gradient estimate is G_W = sum_t g_hat_t x_t^T.
 *   - TL;DR page "Dust: zeroth-order Transformer pretraining without backprop"
 *     (agentlenshq.com), section 1, "activation-space perturbation" and
 *     "credit assignment without backprop" (the equations for g_hat_t, G_W).
 *   - same page, section 1, "reducing interference": the LM head is jittered
 *     on cached logits; the rest of the network stays cached.
 *   - news article on tahou.com, mechanism paragraph: cache the unperturbed
 *     intermediates; head perturbed on cached logits, only the loss recomputed.
 *
 * Conventions for every entry point
 *   - Tensors are caller-owned DEVICE memory, row-major, contiguous, aligned to
 *     at least 16 bytes.  The library keeps no pointer after a call returns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     on it and the call returns at once; outputs are valid once the stream
 *     has completed the work.
 *   - All argument checks run on the host before anything is enqueued.  A
 *     failed check returns DUST_E_INVALID / DUST_E_UNSUPPORTED /
 *     DUST_E_WORKSPACE with a message (dust_last_error) and has no side
 *     effect.  A failed launch returns DUST_E_DEVICE.
 *   - The library allocates no device memory: scratch space comes from the
 *     caller's `workspace`, sized by the matching *_workspace_bytes query.
 *   - Labels are trusted: an out-of-range label never causes an out-of-bounds
 *     access, but the result is then meaningless.  With DUST_DEBUG_CHECKS=1 in
 *     the environment the labels are copied back and checked (synchronising).
 *   - Results are bitwise deterministic run to run (no floating-point atomics).
 *   - State: the library holds no state between calls apart from two kinds of
 *     thread-local data: the error message (dust_last_error) and the profiling
 *     hooks a caller sets with dust_set_stage_event / dust_set_kernel_events
 *     (event handles recorded on the call's stream; cleared by passing NULL).
 *   - Token and draw ids: token_offset is 64-bit in every signature, but the
 *     noise counter holds token and draw ids in one 32-bit Philox word each, so
 *     token_offset + T <= 2^32 and draw_offset + K <= 2^32 (else DUST_E_INVALID).
 *
 * Noise stream (the pages say only "independent Gaussian noise per token";
 * this library fixes one stream so that results are reproducible):
 *   Philox4x32-10 (Salmon et al., SC'11), key = (lo32(seed), hi32(seed)),
 *   counter = (token_offset + t, c >> 2, draw_offset + i, layer), followed by
 *   Box-Muller on each pair of output words:
 *     u1 = ((w[2p] >> 8) + 1) 2^-24, u2 = (w[2p+1] >> 8) 2^-24,
 *     a[4q+2p] = sqrt(-2 ln u1) cos(2 pi u2), a[4q+2p+1] = sqrt(-2 ln u1) sin(2 pi u2).
 *   The noise is regenerated in registers wherever it is needed, never stored.
 *   Because the counters are global, a run split over draws or tokens (the
 *   offsets) reproduces a single run:  K G_W[0,K) = K1 G_W[0,K1) + (K-K1) G_W[K1,K).
 */
#ifndef DUST_H
#define DUST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DUST_ABI_VERSION 2

typedef enum {
    DUST_OK = 0,
    DUST_E_INVALID = 1,      /* bad pointer, size, sigma, offset range ...          */
    DUST_E_UNSUPPORTED = 2,  /* valid but not implemented (e.g. a vocabulary too large) */
    DUST_E_WORKSPACE = 3,    /* workspace missing or smaller than the query says   */
    DUST_E_DEVICE = 4        /* a HIP call failed                                   */
} dust_status;

typedef enum { DUST_F32 = 0, DUST_BF16 = 1 } dust_dtype;

/* ABI version of the loaded library (DUST_ABI_VERSION at build time). */
int dust_abi_version(void);

/* Message of the last failed call on this thread ("" if none).  Valid until
 * the next call into the library on the same thread. */
const char *dust_last_error(void);

/*
 * Profiling hook: while set, `event` (a hipEvent_t) is recorded on the call's
 * stream right after the given stage of every estimator call made from this
 * thread.  stage 0 = after g_hat is ready (the per-token estimator kernels),
 * stage 1 = after the weight-gradient outer product; for dust_estimate_linear
 * also stage 2 = after the downstream GEMM1 (F = LN(x + W2 GELU(.))) and
 * stage 3 = after GEMM2 (logits and their per-tile log-sum-exp) of each row
 * chunk (the last chunk's record wins); for dust_lm_estimate (and dust_lm_step)
 * stage 4 = after the clean forward, 5 = after the head pass, 6 = after the
 * layer-type passes, 7 = after the attention internals (the residual-scalar ES
 * follows).  Pass NULL to clear.  The caller owns the events.  Used to time the
 * stages of one call.
 */
dust_status dust_set_stage_event(int stage, void *event);

/*
 * Profiling hook: while set, each launch of the chosen kernel from this thread records
 * starts[i] before and ends[i] after it on the call's stream, i = 0, 1, ... for the
 * first `capacity` launches (hipEvent_t handles owned by the caller; the arrays are
 * copied).  kernel 0 = the small-LM step's GEMM of change rows (C = A B^T on bf16x3
 * MFMA), 1 = its fused head change, 2 = the main pass of dust_estimate_attn (query, key
 * or value kernel), 3 = dust_estimate_linear's GEMM1 (F = LN(x + W2 GELU(.)): at small
 * sigma the GELU rows and the W2/LayerNorm kernel together, else the single kernel), once
 * per row chunk, 4 = its GEMM2 (the head product and log-sum-exp), once per row chunk,
 * 5 = dust_estimate_head's per-token estimator kernel, 6 = the main product kernel of
 * the bf16-pair outer product (the first pass over whole rounds of output tiles).
 * dust_kernel_event_count(kernel) returns how many launches were recorded since the
 * hook was set (-1 for an unknown kernel).  NULL arrays or capacity <= 0 clear it.
 */
dust_status dust_set_kernel_events(int kernel, void *const *starts, void *const *ends, int capacity);
int dust_kernel_event_count(int kernel);

/*
 * Noise export: the exact Gaussian values (and optionally the raw Philox words)
 * that the estimators use, for draws [draw_offset, draw_offset+K) x tokens
 * [token_offset, token_offset+T) x channels [0, n).
 *   raw   : uint32 [K, T, 4*ceil(n/4)] or NULL -- the Philox output words of
 *           quad q of (draw, token) at [.., .., 4q .. 4q+3].
 *   gauss : float  [K, T, n] or NULL.
 * Requires draw_offset + K <= 2^32 and token_offset + T <= 2^32.
 */
dust_status dust_noise(uint64_t seed, uint32_t layer, uint32_t draw_offset, int64_t K,
                       uint64_t token_offset, int64_t T, int64_t n,
                       uint32_t *raw, float *gauss, void *stream);

/*
 * Noise of one (draw, token): the Gaussian values a[0..n) and, optionally, the raw
 * Philox words behind them, exactly as every estimator draws them for that draw id,
 * token id and layer.  The same stream as dust_noise with K = T = 1.
 *   raw   : uint32 [4*ceil(n/4)] or NULL;  gauss : float [n] or NULL (not both NULL).
 *   token < 2^32 (DUST_E_INVALID otherwise); n >= 1.
 */
dust_status dust_debug_noise(uint64_t seed, uint32_t layer, uint32_t draw, uint64_t token, int64_t n,
                             uint32_t *raw, float *gauss, void *stream);

/*
 * Weight-gradient outer product  grad_w = ghat^T x  =  sum_t ghat_t x_t^T
 * (TL;DR page, section 1, equation for G_W).
 *   ghat   : float [T, n];  x : float [T, d];  grad_w : float [n, d] (overwritten).
 * Workspace: dust_outer_workspace_bytes(T, n, d) bytes (split-K partial sums).
 */
size_t dust_outer_workspace_bytes(int64_t T, int64_t n, int64_t d);
dust_status dust_outer_product(const float *ghat, const float *x, int64_t T, int64_t n, int64_t d,
                               float *grad_w, void *workspace, size_t workspace_bytes, void *stream);

/*
 * LM-head estimator on cached logits (full vocabulary per draw).
 *   logits       : [T, V] cached clean logits z_t = W x_t, fp32 or bf16 bits
 *                  (logits_dtype = DUST_F32 / DUST_BF16).
 *   x            : float [T, d] cached input of the head (the x_t of G_W).
 *   labels       : int32 [T] next-token ids in [0, V).
 *   K >= 1 draws, sigma > 0 finite.
 *   seed, layer  : noise stream; token_offset/draw_offset: global ids of token 0 / draw 0.
 *   grad_w       : OUT float [V, d]  G_W = sum_t g_hat_t x_t^T (overwritten).
 *   ghat         : OUT float [T, V]  g_hat_t, or NULL.
 *   rewards      : OUT float [K, T]  r_t^(i) = CE_clean - CE_perturbed (nats), or NULL.
 * Per draw the perturbed loss is evaluated as log1p(sum_v p_v expm1(sigma a_v)) -
 * sigma a_y with p = softmax(z_t): equal to CE(z + sigma a) - CE(z) in exact
 * arithmetic, without the cancellation of subtracting two losses of order ln V.
 * Supported: V <= 65536.
 */
size_t dust_head_workspace_bytes(int64_t T, int64_t V, int64_t d, int64_t K);
dust_status dust_estimate_head(const void *logits, int logits_dtype, const float *x,
                               const int32_t *labels, int64_t T, int64_t V, int64_t d,
                               int64_t K, float sigma, uint64_t seed, uint32_t layer,
                               uint64_t token_offset, uint32_t draw_offset,
                               float *grad_w, float *ghat, float *rewards,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * dust_estimate_head without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, outputs, checks and kernels as
 * dust_estimate_head; its scratch is a static device array of the library, one per GPU,
 * of dust_head_noalloc_max_bytes() bytes (64 MiB), held from the library's first use of
 * that GPU until the process ends.  The call allocates nothing (no hipMalloc, no
 * allocating library routine).  A shape whose dust_head_workspace_bytes exceeds that
 * size (ignoring the g_hat rows when `ghat` is passed) is rejected with
 * DUST_E_UNSUPPORTED before anything is enqueued.  Calls on one GPU share the array:
 * calls that overlap on one GPU (other streams, other threads) race; serialize them.
 */
dust_status dust_estimate_head_noalloc(const void *logits, int logits_dtype, const float *x,
                                       const int32_t *labels, int64_t T, int64_t V, int64_t d,
                                       int64_t K, float sigma, uint64_t seed, uint32_t layer,
                                       uint64_t token_offset, uint32_t draw_offset,
                                       float *grad_w, float *ghat, float *rewards, void *stream);
size_t dust_head_noalloc_max_bytes(void);

/*
 * Vocabulary-subset LM-head estimator (TL;DR page, section 1, "reducing
 * interference": the head is evaluated on part of the vocabulary per draw).
 * The pages give no subset rule.  Here, per (token, draw), the perturbed set S is
 * a cyclic window of mq = m/4 consecutive channel quads (channels 4q..4q+3 of
 * the nq = ceil(V/4) quads) starting at quad o = (w * nq) >> 32, w = word 0 of
 * Philox4x32-10 on the counter (token_offset + t, 0xFFFFFFFF, draw_offset + i,
 * layer) with the noise key, plus the label y_t.  S carries the same noise a_v as
 * dust_estimate_head; nothing else is perturbed, and
 *   r = CE(z_t) - CE(z_t + sigma a 1_S)
 *   g_hat_t[v] = -(1/(K sigma)) sum_i r a_v 1[v in S_i] / pi_v
 * with pi_v = mq/nq the inclusion probability of a window channel (1 for the
 * label), so the estimate stays unbiased.  Per draw the work is mq quads
 * instead of nq.
 *   m : channels per draw, a positive multiple of 4; when m >= 4 nq the window
 *       is the whole vocabulary and the call is dust_estimate_head's.
 * Other arguments and outputs as dust_estimate_head, with its limits on V
 * (fp32 logits V <= 32768, bf16 V <= 65536; DUST_E_UNSUPPORTED beyond).  Rows
 * of V <= 16384 run in one kernel with the probabilities and running sums of a
 * token in LDS; wider rows in two (the rewards, then the running sums by
 * vocabulary segment), regenerating the window's noise in the second.
 * Workspace: dust_head_subset_workspace_bytes(T, V, d, K) bytes: that of
 * dust_head_workspace_bytes, plus for V > 16384 room for the rewards and the
 * window offsets of every (draw, token), 2 * ceil(4KT / 256) * 256 bytes.
 */
size_t dust_head_subset_workspace_bytes(int64_t T, int64_t V, int64_t d, int64_t K);
dust_status dust_estimate_head_subset(const void *logits, int logits_dtype, const float *x,
                                      const int32_t *labels, int64_t T, int64_t V, int64_t d,
                                      int64_t K, int64_t m, float sigma, uint64_t seed, uint32_t layer,
                                      uint64_t token_offset, uint32_t draw_offset,
                                      float *grad_w, float *ghat, float *rewards,
                                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Interior MLP-linear estimator: W1 of a pre-LN MLP block, with the cached
 * downstream recomputed per draw (TL;DR page, section 1: noise on the output of
 * every linear layer, reward = loss reduction at the token; news article on
 * tahou.com, mechanism paragraph: unperturbed intermediates are cached and
 * only the part the perturbation changes is recomputed).
 * For token t and draw i, with a = a_t^(i):
 *   m   = bf16(GELU_erf(h_t + sigma a))                 (fp32, then round to nearest even)
 *   f   = bf16(LN(x_t + W2 m))                          (LN without affine, eps = ln_eps)
 *   CE  = logsumexp(W_head f) - (W_head f)[y_t]         (fp32 accumulation)
 *   r   = CE(a = 0) - CE(a);  g_hat_t = -(1/(K sigma)) sum_i r a;  G_W1 = sum_t g_hat_t u_t^T.
 *   u      : float [T, d]   input of W1 (u = LN(x), the x_t of G_W1)
 *   h      : float [T, n]   cached W1 output (pre-GELU)
 *   x_res  : float [T, d]   residual stream added after W2
 *   w2     : bf16 bits [d, n];   w_head : bf16 bits [V, d]
 *   labels : int32 [T]
 *   grad_w : OUT float [n, d];  ghat : OUT float [T, n] or NULL;  rewards : OUT float [K, T] or NULL.
 * Supported: d in {256, 512}, n a multiple of 32, V >= 1, V*d < 2^31 and n*d < 2^31
 * (DUST_E_UNSUPPORTED otherwise).
 * Workspace: dust_linear_workspace_bytes(T, d, n, V, K) bytes.
 */
size_t dust_linear_workspace_bytes(int64_t T, int64_t d, int64_t n, int64_t V, int64_t K);
dust_status dust_estimate_linear(const float *u, const float *h, const float *x_res,
                                 const uint16_t *w2, const uint16_t *w_head, const int32_t *labels,
                                 int64_t T, int64_t d, int64_t n, int64_t V, int64_t K,
                                 float sigma, float ln_eps, uint64_t seed, uint32_t layer,
                                 uint64_t token_offset, uint32_t draw_offset,
                                 float *grad_w, float *ghat, float *rewards,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * Attention internals: the estimators of the query, key and value projections.
 * Method: TL;DR page "Dust: zeroth-order Transformer pretraining without backprop",
 * section 1, "credit assignment without backprop" (attention internals are rewarded by
 * the change of the attention output, not the token's loss) and "reducing interference"
 * (only the attention output is recomputed); the tahou.com news article, mechanism
 * paragraph (that change is judged against the error signal); the iitog.ru page,
 * mechanics paragraph (the error at the attention output over current and future
 * tokens).  Reading: causal multi-head attention within sequences of S tokens (token
 * t = b S + s); the chosen projection's output y_t (q_t, k_t or v_t) of every token
 * perturbed by sigma a_t^(i) in the same draw; e_s the error (loss gradient) at the
 * attention output o_s, before W_O:
 *   c_s   = <e_s, o'_s - o_s>
 *   r_t   = -sum_{s >= t, same sequence} c_s     (keys and values: the outputs they move)
 *   r_t   = -c_t                                (queries: only o_t depends on q_t)
 *   g_hat_t = -(1/(K sigma)) sum_i r_t a_t;   G_W = sum_t g_hat_t u_t^T.
 * The output change is formed without subtracting two outputs: for values
 * o'_s - o_s = sigma sum_t P_st a_t (P unchanged); for queries and keys, with delta_st
 * the logit change (sigma <a_s, k_t> / sqrt(dh) or sigma <q_s, a_t> / sqrt(dh)),
 * rho_s = sum_t P_st expm1(delta_st) and mu_s = sum_t P_st expm1(delta_st) <v_t, e_s>:
 * c_s = (mu_s - rho_s <e_s, o_s>) / (1 + rho_s), per head.
 *   proj   : DUST_ATTN_Q, DUST_ATTN_K or DUST_ATTN_V
 *   q, k   : float [T, d]  clean query and key projections (heads of 64 channels: d = 64 H)
 *   v      : float [T, d]  clean value projection (queries and keys only; may be NULL for values)
 *   e      : float [T, d]  error at the attention output (per head, before W_O)
 *   u      : float [T, d]  input of the projection (the u_t of G_W)
 *   grad_w : OUT float [d, d];  ghat : OUT float [T, d] or NULL;  rewards : OUT float [K, T] or NULL.
 * Noise counter: (token, channel/4, draw, layer).  Supported: S a multiple of 64 up to
 * 4096, T a multiple of S, d = 64 H with 1 <= H <= 16 (else DUST_E_UNSUPPORTED).  Stages (dust_set_stage_event): 2 = after the
 * rewards, 0 = after g_hat, 1 = after G_W.
 * Workspace: dust_attn_workspace_bytes(proj, T, S, d, H, K) bytes.
 * dust_estimate_attn_v is dust_estimate_attn with DUST_ATTN_V (no v argument).
 */
typedef enum { DUST_ATTN_Q = 0, DUST_ATTN_K = 1, DUST_ATTN_V = 2 } dust_attn_proj;
size_t dust_attn_workspace_bytes(int proj, int64_t T, int64_t S, int64_t d, int64_t H, int64_t K);
dust_status dust_estimate_attn(int proj, const float *q, const float *k, const float *v, const float *e,
                               const float *u, int64_t T, int64_t S, int64_t d, int64_t H, int64_t K,
                               float sigma, uint64_t seed, uint32_t layer, uint64_t token_offset,
                               uint32_t draw_offset, float *grad_w, float *ghat, float *rewards,
                               void *workspace, size_t workspace_bytes, void *stream);
size_t dust_attn_v_workspace_bytes(int64_t T, int64_t S, int64_t d, int64_t H, int64_t K);
dust_status dust_estimate_attn_v(const float *q, const float *k, const float *e, const float *u,
                                 int64_t T, int64_t S, int64_t d, int64_t H, int64_t K, float sigma,
                                 uint64_t seed, uint32_t layer, uint64_t token_offset,
                                 uint32_t draw_offset, float *grad_w, float *ghat, float *rewards,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * One full Dust update step on a small causal language model.
 * Method: TL;DR page "Dust: zeroth-order Transformer pretraining without backprop",
 * section 1, "reducing interference" (each layer type jittered in a forward pass of
 * its own with its own noise scale; attention internals with only the attention output
 * recomputed; the head on cached logits) and "credit assignment without backprop"
 * (g_hat, G_W); section 2, "pretraining results" (SGD with momentum); iitog.ru page,
 * mechanics paragraph (every weight by the per-token estimator except the 2L residual
 * mixing scalars, which weight-space ES trains).
 *
 * Model (a reading; the pages give no architecture): tokens t = b S + s of B sequences
 * of S tokens; x_0 = E[token] + P[s]; L pre-LN blocks
 *     x <- x + alpha_l W_O attn(LN(x) W_Q^T, LN(x) W_K^T, LN(x) W_V^T)
 *     x <- x + beta_l  W_2 GELU(W_1 LN(x))
 * then LN, logits z = W_head LN(x), cross-entropy against the next-token label.  Causal
 * attention within each sequence, heads of 64 channels (d = 64 H), scale 1/8;
 * exact-erf GELU; LayerNorm without affine, eps = ln_eps; no biases.
 *
 * Parameters: one packed fp32 vector, in this order, weights [out, in] row-major:
 *     E [V, d], P [S, d], then per block l: W_Q [d, d], W_K [d, d], W_V [d, d],
 *     W_O [d, d], W_1 [n, d], W_2 [d, n]; then W_head [V, d]; then the scalars
 *     alpha_0, beta_0, alpha_1, beta_1, ... (2L).
 * dust_lm_param_count gives its length (0 for an invalid config).
 *
 * One step, all estimates at the same parameters:
 *   head   dust_estimate_head on the cached logits (sigma_head, noise layer 2);
 *   emb, o, up, down   one pass per linear type: every point of that type (the embedding
 *          sum x_0; each block's W_O, W_1 or W_2 output) perturbed by sigma a in the same
 *          draw, the rest of the network recomputed, r_t = CE_t - CE'_t (the token's own
 *          loss); noise layer 1 for the embedding, 16 (l + 1) + {3, 4, 5} for o, up, down;
 *          G_E[v] = sum of g_hat over tokens equal to v, G_P[s] = sum over sequences;
 *   q, k, v   dust_estimate_attn per block with the error at the attention output
 *          e_l = g_hat_O,l W_O,l (noise layer 16 (l + 1) + {0, 1, 2});
 *   scalars   antithetic ES with M pairs on the summed loss: member 2j is s + sigma_es eps_j,
 *          member 2j + 1 is s - sigma_es eps_j, eps_j[c] = the noise of (token 0, channel c,
 *          draw j, layer 3); g = (1/(2 M sigma_es)) sum_j (L_2j - L_2j+1) eps_j.
 * Each perturbed forward is evaluated as the change of every activation against the
 * cached clean pass (no difference of two losses is taken), over chunks of draws.
 * Then SGD with momentum: m <- momentum m + G; theta <- theta - lr m (lr_scalar for the
 * 2L scalars).
 *
 * Arguments (device pointers unless stated):
 *   cfg, hp : host structs.   tokens, labels : int32 [B S] ids in [0, V) (trusted: an
 *   out-of-range id is clamped, never read out of bounds).   seed : noise key.
 *   grads   : OUT float [param_count] the estimates G, packed like the parameters.
 *   rewards : OUT float [dust_lm_rewards_count] or NULL: each pass's rewards [K, T] in
 *             the order head, emb, o, up, down, then per block q, k, v; then the 2M
 *             members' summed-loss changes L(member) - L(clean), member 2j then 2j + 1.
 *   ce      : OUT float [T] the clean per-token cross-entropy (dust_lm_forward).
 * Supported: 1 <= H <= 16, S a multiple of 64 up to 4096, n a multiple of 64 up to 65536,
 * 1 <= V <= 32768, 1 <= L <= 32, K >= 1, M >= 1, chunk >= 0; every sigma > 0.
 * Workspace: dust_lm_workspace_bytes(cfg, hp) bytes (the clean cache, the change tensors
 * of one chunk of draws (at most 1 GiB, at least one draw), the rewards and the
 * estimators' own scratch); dust_lm_forward needs the same query's size.
 */
typedef struct {
    int32_t V, d, H, L, n, S, B;
    float ln_eps;
} dust_lm_config;

typedef struct {
    int32_t K, M;
    float sigma_emb, sigma_q, sigma_k, sigma_v, sigma_o, sigma_up, sigma_down, sigma_head, sigma_es;
    float lr, lr_scalar, momentum;
    int32_t chunk; /* most draws (or ES members) per chunk of change tensors; 0: as many as fit in 1 GiB */
} dust_lm_hparams;

size_t dust_lm_param_count(const dust_lm_config *cfg);
size_t dust_lm_rewards_count(const dust_lm_config *cfg, const dust_lm_hparams *hp);
size_t dust_lm_workspace_bytes(const dust_lm_config *cfg, const dust_lm_hparams *hp);
dust_status dust_lm_forward(const dust_lm_config *cfg, const float *params, const int32_t *tokens,
                            const int32_t *labels, float *ce, void *workspace, size_t workspace_bytes,
                            void *stream);
dust_status dust_lm_estimate(const dust_lm_config *cfg, const dust_lm_hparams *hp, const float *params,
                             const int32_t *tokens, const int32_t *labels, uint64_t seed, float *grads,
                             float *rewards, void *workspace, size_t workspace_bytes, void *stream);
/* m <- momentum m + grads; params <- params - lr m (lr_scalar on the last 2L entries). */
dust_status dust_lm_sgd(const dust_lm_config *cfg, const dust_lm_hparams *hp, float *params, float *momentum,
                        const float *grads, void *stream);
/* dust_lm_estimate followed by dust_lm_sgd. */
dust_status dust_lm_step(const dust_lm_config *cfg, const dust_lm_hparams *hp, float *params, float *momentum,
                         const int32_t *tokens, const int32_t *labels, uint64_t seed, float *grads,
                         float *rewards, void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DUST_H */
