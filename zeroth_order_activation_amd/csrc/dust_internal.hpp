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
    int deg;       // 3, 4 or 6: Taylor degree of the polynomial expm1; 0: library expm1
    size_t lds;    // dynamic LDS bytes
    bool ok;
    const char* why;
};

HeadPlan plan_head(int64_t V, int logits_dtype, float sigma);
hipError_t launch_head(const HeadPlan& plan, int logits_dtype, const HeadArgs& args, hipStream_t stream);
// vocabulary-subset estimator (head_subset.hip)
// rows of up to kSubsetLdsMaxV channels run in one pass with the row in LDS;
// wider ones in two (rewards, then accumulation), which pass K T pairs of
// (reward, window offset) through the workspace
constexpr int64_t kSubsetLdsMaxV = 16384;
size_t head_subset_lds_bytes(int64_t V);
int head_subset_qw(int64_t m, int64_t V);
hipError_t launch_head_subset(const HeadPlan& plan, int logits_dtype, const HeadArgs& args, int64_t m,
                              float2* ro_ws, hipStream_t stream);

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
    size_t off_f, off_wt, off_part, off_zy, off_wnorm, off_ce, off_ghat, off_w2f, off_phi, off_m, off_outer, total;
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

}  // namespace dust
