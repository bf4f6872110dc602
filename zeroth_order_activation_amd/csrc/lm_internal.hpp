// Host-side launchers of the small-LM step kernels (lm.hip); internal.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dust {

// ---- small causal LM: clean forward and change-propagating forward (lm.hip) ----

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
// also writes Phi(h) and phi(h) (the normal distribution and density), reused by lm_gelu_delta
hipError_t lm_gelu(const float* h, int64_t count, float* m, float* cdf, float* pdf, hipStream_t s);
hipError_t lm_residual(const float* x, const float* b, const float* alpha, int64_t count, float* out, hipStream_t s);
hipError_t lm_ce(const float* z, const int32_t* labels, int T, int V, float* lse, float* ce, float* prob, int Vp,
                 hipStream_t s);
// the head's change fused with its loss change (d = 64 or 128): bf16 parts of W_head
// [Vp, d] (Vp = V rounded up to 128, zero rows past V), probabilities [T, Vp];
// part [kc T, nseg] the per-segment sums, then rew = D_z_y - log1p(sum part)
// C = A B^T on bf16x3 MFMA for change rows: B given as bf16 parts [N, K]; K % 32 == 0.
// C is [M, N], or with a plane width pw (N % pw == 0) N / pw planes [M, pw] ps floats apart
hipError_t lm_gemm_x3(const float* A, const uint16_t* Bh, const uint16_t* Bl, float* C, int64_t M, int64_t N,
                      int64_t K, hipStream_t s, int64_t pw = 0, int64_t ps = 0);
hipError_t lm_split(const float* W, int64_t rows, int64_t rows_p, int K, uint16_t* hi, uint16_t* lo, hipStream_t s);
// the same parts in MFMA fragment order (16-byte unit ((row / 32) (K / 16) + k / 16) 64 + lane), for the head change
hipError_t lm_split_frag(const float* W, int64_t rows, int64_t rows_p, int K, uint16_t* hi, uint16_t* lo,
                        hipStream_t s);
hipError_t lm_head_delta(const float* du, const uint16_t* whi, const uint16_t* wlo, const float* prob, int d, int kc,
                         int T, int Vp, int vseg, int nseg, float* part, hipStream_t s);
hipError_t lm_head_reward(const float* du, const float* whead, const int32_t* labels, const float* part, int T, int V,
                          int d, int nseg, int64_t rows, float* rew, hipStream_t s);
hipError_t lm_noise_add(float* D, int kc, int T, int w, float sigma, uint32_t k0, uint32_t k1, uint32_t layer,
                        uint32_t draw0, hipStream_t s, bool set = false);  // set: D holds no change yet
hipError_t lm_layernorm_delta(const float* x, const float* mu, const float* rs, const float* dx, int64_t R, int T,
                              int d, float* du, hipStream_t s);
hipError_t lm_attn_delta(const float* q, const float* k, const float* v, const float* o, const float* pc,
                         const float* dq, const float* dk, const float* dv, int kc, int T, int S, int H, float* dout,
                         hipStream_t s);
hipError_t lm_gelu_delta(const float* h, const float* cdf, const float* pdf, const float* dh, int64_t per_draw,
                         int64_t count, float* dm, hipStream_t s);
hipError_t lm_residual_delta(float* dx, const float* db, const float* b, const float* scal, int slot, int kc,
                             int64_t per_draw, float es_sigma, uint32_t member0, uint32_t k0, uint32_t k1,
                             uint32_t es_layer, hipStream_t s);
// the residual change, then the LayerNorm change (x, mu, rs of that LayerNorm) of the updated
// rows into du, in one pass; for d = 64, 128, 256 or 512 (lm_residual_ln_fusable)
bool lm_residual_ln_fusable(int d);
hipError_t lm_residual_ln_delta(float* dx, const float* db, const float* b, const float* scal, int slot, int kc,
                                int T, int d, float es_sigma, uint32_t member0, uint32_t k0, uint32_t k1,
                                uint32_t es_layer, const float* x, const float* mu, const float* rs, float* du,
                                hipStream_t s);
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
