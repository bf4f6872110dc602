// Host-side launchers of the Dust kernels (internal; the public surface is
// include/dust.h).  Every launcher assumes its arguments were validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dust {

hipError_t launch_noise_export(uint64_t seed, uint32_t layer, uint32_t draw0, int64_t K, uint32_t tok0,
                               int64_t T, int64_t n, uint32_t* raw, float* gauss, hipStream_t stream);

// ---- LM head on cached logits -------------------------------------------
struct HeadArgs {
    const void* logits;      // [T,V] fp32 or bf16 bits
    const int32_t* labels;   // [T]
    float* ghat;             // [T,V] out, or null
    uint16_t* ghi;           // [T, ldp] bf16 hi/lo pairs of g_hat (token-major, zero past V), or null
    uint16_t* glo;
    int64_t ldp;
    float* rewards;          // [K,T] out or null
    int32_t T, V, K;
    float sigma;
    float smul;              // factor applied to the per-draw sum before log1p
    float gscale;            // -1/(K sigma)
    float coef[8];           // Horner coefficients of expm1(sigma a)/(sigma a), see head.hpp
    uint32_t k0, k1, layer, tok0, draw0;
};

struct HeadPlan {
    int nt;        // threads per workgroup (one workgroup per token)
    int q;         // channel quads per lane
    int pmode;     // 0: probabilities in registers, 1: logit row staged in LDS
    int ql;        // quads per lane whose running sums live in LDS (pmode 1 only)
    int deg;       // 5: polynomial expm1, 0: library expm1
    size_t lds;    // dynamic LDS bytes
    bool ok;
    const char* why;
};

HeadPlan plan_head(int64_t V, int logits_dtype, float sigma);
hipError_t launch_head(const HeadPlan& plan, int logits_dtype, const HeadArgs& args, hipStream_t stream);
// vocabulary-subset estimator (head_subset.hip)
// rows of up to kSubsetLdsMaxV channels run in one pass with the row in LDS;
// wider ones in two (rewards, then accumulation), which need K T floats of
// rewards (unless the caller keeps them) and K T ints of window offsets
constexpr int64_t kSubsetLdsMaxV = 16384;
size_t head_subset_lds_bytes(int64_t V);
size_t head_subset_wide_lds_bytes(int64_t V, int logits_dtype);
int head_subset_qw(int64_t m, int64_t V);
hipError_t launch_head_subset(const HeadPlan& plan, int logits_dtype, const HeadArgs& args, int64_t m,
                              float* rew_ws, int* off_ws, hipStream_t stream);

// ---- grad_w = ghat^T x (fp32 MFMA) --------------------------------------
size_t outer_workspace_bytes(int64_t T, int64_t n, int64_t d);
// Where the bf16 pairs of ghat go in the outer-product workspace when the
// product takes the bf16-pair path (hi == nullptr otherwise): [T.., ld] rows.
struct OuterPairs {
    uint16_t* hi;
    uint16_t* lo;
    int64_t ld;
};
OuterPairs outer_ghat_pairs(int64_t T, int64_t n, int64_t d, void* workspace);
bool outer_uses_pairs(int64_t T, int64_t n, int64_t d);
hipError_t launch_outer(const float* ghat, const float* x, int64_t T, int64_t n, int64_t d, float* grad_w,
                        void* workspace, size_t workspace_bytes, hipStream_t stream, bool pairs_ready = false);

// ---- interior MLP linear ------------------------------------------------
struct MlpArgs {
    const float* u;          // [T,d] input of W1 (the x_t of G_W1)
    const float* h;          // [T,n] cached W1 output
    const float* x_res;      // [T,d] residual stream
    const uint16_t* w2;      // [d,n] bf16
    const uint16_t* w_head;  // [V,d] bf16
    const int32_t* labels;   // [T]
    float* rewards;          // [K,T] out or null
    int32_t T, d, n, V, K;
    float sigma, ln_eps, gscale;
    uint32_t k0, k1, layer, tok0, draw0;
    hipEvent_t stage_event;  // recorded after g_hat, before the outer product (or null)
    hipEvent_t gemm1_event;  // recorded after each chunk's GEMM1 (or null)
    hipEvent_t gemm2_event;  // recorded after each chunk's GEMM2 (or null)
};

struct MlpLayout {
    int64_t chunk;  // rows of recomputed downstream per pass
    int nvt;        // vocabulary tiles
    size_t off_f, off_part, off_zy, off_wnorm, off_ce, off_ghat, off_outer, total;
};

MlpLayout mlp_layout(int64_t T, int64_t d, int64_t n, int64_t V, int64_t K);
hipError_t launch_mlp(const MlpArgs& args, const MlpLayout& layout, unsigned char* workspace, float* ghat_user,
                      float* grad_w, hipStream_t stream);

// attention projection estimators (attn.hip); proj 0 = query, 1 = key, 2 = value
struct AttnVLayout {
    size_t off_lse, off_ob, off_cpart, off_rew, off_ghat, off_outer, total;
};
AttnVLayout attn_layout(int proj, int64_t T, int64_t S, int64_t d, int64_t H, int64_t K);
hipError_t launch_attn_rewards(int proj, const float* q, const float* k, const float* v, const float* e, int64_t T,
                               int64_t S, int64_t d, int64_t H, int64_t K, float sigma, uint64_t seed, uint32_t layer,
                               uint32_t token_offset, uint32_t draw_offset, float* rew, unsigned char* ws,
                               const AttnVLayout& L, hipStream_t stream);
hipError_t launch_attn_v_ghat(int64_t T, int64_t d, int64_t K, float sigma, uint64_t seed, uint32_t layer,
                              uint32_t token_offset, uint32_t draw_offset, const float* rew, float* ghat,
                              hipStream_t stream);

// ---- small causal LM: clean forward and change-propagating forward (lm.hip) ----
// Profiling: while starts is set, each launch of the LM's GEMM kernel records
// starts[count] before and ends[count] after it, for the first `capacity` launches.
struct LaunchEvents {
    hipEvent_t* starts = nullptr;
    hipEvent_t* ends = nullptr;
    int capacity = 0;
    int count = 0;
};
extern thread_local LaunchEvents g_gemm_events;

// Rows of a change tensor are r = i T + t for draw i of the chunk; every size
// assumption (M % 64, K % 16, d = 64 H, S % 64, widths % 4) is checked by the caller.
hipError_t lm_gemm_nt(const float* A, const float* B, float* C, int64_t M, int64_t N, int64_t K, const float* alpha,
                      bool accumulate, hipStream_t s);
hipError_t lm_embed(const float* emb, const float* pos, const int32_t* tok, int T, int S, int d, int V, float* x,
                    hipStream_t s);
hipError_t lm_layernorm(const float* x, int64_t R, int d, float eps, float* u, float* mu, float* rs, hipStream_t s);
// also writes the clean probabilities pc[((b H + h) S + query) S + key] for the key tiles up
// to the query's own (zero after the query)
hipError_t lm_attn_fwd(const float* q, const float* k, const float* v, int T, int S, int H, float* o, float* lse,
                       float* pc, hipStream_t s);
hipError_t lm_gelu(const float* h, int64_t count, float* m, hipStream_t s);
hipError_t lm_residual(const float* x, const float* b, const float* alpha, int64_t count, float* out, hipStream_t s);
hipError_t lm_ce(const float* z, const int32_t* labels, int T, int V, float* lse, float* ce, float* prob, int Vp,
                 hipStream_t s);
// the head's change fused with its loss change (d = 64 or 128): bf16 parts of W_head
// [Vp, d] (Vp = V rounded up to 128, zero rows past V), probabilities [T, Vp];
// part [kc T, nseg] the per-segment sums, then rew = D_z_y - log1p(sum part)
hipError_t lm_split(const float* W, int64_t rows, int64_t rows_p, int K, uint16_t* hi, uint16_t* lo, hipStream_t s);
hipError_t lm_head_delta(const float* du, const uint16_t* whi, const uint16_t* wlo, const float* prob, int d, int kc,
                         int T, int Vp, int vseg, int nseg, float* part, hipStream_t s);
hipError_t lm_head_reward(const float* du, const float* whead, const int32_t* labels, const float* part, int T, int V,
                          int d, int nseg, int64_t rows, float* rew, hipStream_t s);
hipError_t lm_noise_add(float* D, int kc, int T, int w, float sigma, uint32_t k0, uint32_t k1, uint32_t layer,
                        uint32_t draw0, hipStream_t s);
hipError_t lm_layernorm_delta(const float* x, const float* mu, const float* rs, const float* dx, int64_t R, int T,
                              int d, float* du, hipStream_t s);
hipError_t lm_attn_delta(const float* q, const float* k, const float* v, const float* o, const float* pc,
                         const float* dq, const float* dk, const float* dv, int kc, int T, int S, int H, float* dout,
                         hipStream_t s);
hipError_t lm_gelu_delta(const float* h, const float* dh, int64_t per_draw, int64_t count, float* dm, hipStream_t s);
hipError_t lm_residual_delta(float* dx, const float* db, const float* b, const float* scal, int slot, int kc,
                             int64_t per_draw, float es_sigma, uint32_t member0, uint32_t k0, uint32_t k1,
                             uint32_t es_layer, hipStream_t s);
hipError_t lm_ce_delta(const float* z, const float* lse, const float* dz, const int32_t* labels, int kc, int T, int V,
                       float* rew, hipStream_t s);
hipError_t lm_ghat(const float* rew, int K, int T, int w, float scale, uint32_t k0, uint32_t k1, uint32_t layer,
                   float* ghat, hipStream_t s);
hipError_t lm_embed_grads(const float* ghat, const int32_t* tok, int T, int S, int V, int d, float* gemb, float* gpos,
                          hipStream_t s);
hipError_t lm_transpose(const float* W, int R, int C, float* WT, hipStream_t s);
hipError_t lm_member_losses(const float* rew, int members, int T, float* dL, hipStream_t s);
hipError_t lm_es_grad(const float* dL, int M, int nsc, float scale, uint32_t k0, uint32_t k1, uint32_t es_layer,
                      float* g, hipStream_t s);
hipError_t lm_sgd(float* theta, float* mom, const float* G, int64_t count, int64_t scal0, float lr, float lr_scalar,
                  float mu, hipStream_t s);

}  // namespace dust
