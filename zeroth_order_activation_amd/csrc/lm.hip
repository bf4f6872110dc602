// Kernels of the full Dust step on a small causal LM: the clean forward with
// its cached intermediates, and the change-propagating forward that every
// layer-type pass and the residual-scalar ES pass run over a chunk of draws.
//
// Method: TL;DR page "Dust: zeroth-order Transformer pretraining without
// backprop", section 1, "reducing interference" (each layer type jittered in a
// forward pass of its own, with its own noise scale; the rest cached) and
// "credit assignment without backprop" (reward = the token's loss reduction);
// iitog.ru page, mechanics paragraph (the 2L residual mixing scalars by
// weight-space ES).  The model (pre-LN blocks x <- x + alpha W_O attn(...),
// x <- x + beta W_2 GELU(W_1 LN(x)), final LN, head) is this library's reading.
//
// A perturbed forward is carried as the change D = x' - x of every activation
// relative to the cached clean pass, never as a second forward whose loss is
// subtracted from the clean one:
//   linear      D_y = D_x W^T                                  (exact)
//   LayerNorm   D_u = c rs (1 + f) + (x - mu) rs f,  c = D - mean(D),
//               f = (1 + dv rs^2)^(-1/2) - 1 = expm1(-log1p(dv rs^2) / 2),
//               dv = 2 mean((x - mu) c) + mean(c^2)
//   GELU        D_m = D_h Phi(h + D_h) + h (Phi(h + D_h) - Phi(h)), the
//               difference of Phi by Simpson's rule for |D_h| < 1/4, else by
//               complementary error functions of one sign
//   attention   P' = P e^delta / (1 + rho), rho = sum_t P expm1(delta),
//               D_o = (sum_t P expm1(delta) v_t + sum_t P e^delta D_v_t - rho o) / (1 + rho)
//   CE          D_CE = log1p(sum_v p_v expm1(D_z_v)) - D_z_y
// so every reward keeps fp32 relative accuracy however small it is.
#include <hip/hip_runtime.h>
#include <algorithm>
#include <math.h>
#include <stdint.h>

#include "dust_device.hpp"
#include "dust_internal.hpp"
#include "launch_events.hpp"
#include "lm_internal.hpp"

namespace dust {
namespace {

typedef float lf32x16 __attribute__((ext_vector_type(16)));

// ---- GEMM  C (=|+=) alpha A B^T,  A [M, K], B [N, K] row-major, fp32 MFMA ------------
constexpr int GB = 64, GK = 16;

__global__ void __launch_bounds__(256) lm_gemm_nt_kernel(const float* __restrict__ A, const float* __restrict__ B,
                                                         float* __restrict__ C, int M, int N, int K,
                                                         const float* __restrict__ alpha, int accumulate) {
    __shared__ float As[GK][GB + 4];
    __shared__ float Bs[GK][GB + 4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w & 1, wn = w >> 1;
    const int64_t m0 = (int64_t)blockIdx.x * GB, n0 = (int64_t)blockIdx.y * GB;
    const int lr = tid >> 2, lk = (tid & 3) * 4;  // loader: row of the tile, 4 consecutive k
    const float* ap = A + (m0 + lr) * (int64_t)K + lk;
    const bool bok = n0 + lr < N;
    const float* bp = B + (bok ? (n0 + lr) : 0) * (int64_t)K + lk;
    lf32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    float4 ra = *reinterpret_cast<const float4*>(ap);
    float4 rb = bok ? *reinterpret_cast<const float4*>(bp) : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = 0; k0 < K; k0 += GK) {
        __syncthreads();
        As[lk + 0][lr] = ra.x;
        As[lk + 1][lr] = ra.y;
        As[lk + 2][lr] = ra.z;
        As[lk + 3][lr] = ra.w;
        Bs[lk + 0][lr] = rb.x;
        Bs[lk + 1][lr] = rb.y;
        Bs[lk + 2][lr] = rb.z;
        Bs[lk + 3][lr] = rb.w;
        __syncthreads();
        if (k0 + GK < K) {  // next k-step's operands, in flight during the MFMAs
            ra = *reinterpret_cast<const float4*>(ap + k0 + GK);
            if (bok) rb = *reinterpret_cast<const float4*>(bp + k0 + GK);
        }
#pragma unroll
        for (int kk = 0; kk < GK; kk += 2) {
            const int k = kk + (lane >> 5);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[k][wm * 32 + (lane & 31)], Bs[k][wn * 32 + (lane & 31)],
                                                       acc, 0, 0, 0);
        }
    }
    // D[i][j] of the 32x32 block: lane j + 32 ((i / 4) % 2), register (i % 4) + 4 (i / 8)
    const float al = alpha ? *alpha : 1.0f;
    const int64_t col = n0 + wn * 32 + (lane & 31);
    if (col < N) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = m0 + wm * 32 + (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5);
            float* c = C + row * N + col;
            *c = accumulate ? fmaf(al, acc[r], *c) : al * acc[r];
        }
    }
}

// ---- clean forward ------------------------------------------------------------
__global__ void __launch_bounds__(256) lm_embed_kernel(const float* __restrict__ emb, const float* __restrict__ pos,
                                                       const int32_t* __restrict__ tok, int T, int S, int d, int V,
                                                       float* __restrict__ x) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // float index
    if (i >= (int64_t)T * d) return;
    const int t = (int)(i / d), c = (int)(i % d);
    const int id = min(max(tok[t], 0), V - 1);  // an out-of-range id reads row 0 or V - 1, never outside
    x[i] = emb[(int64_t)id * d + c] + pos[(int64_t)(t % S) * d + c];
}

// One wave per row of d = 64 E channels (E <= 16): lane holds channels lane + 64 e.
constexpr int LNE = 16;

__global__ void __launch_bounds__(256) lm_layernorm_kernel(const float* __restrict__ x, int R, int d, float eps,
                                                           float* __restrict__ u, float* __restrict__ mu,
                                                           float* __restrict__ rs) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63, E = d >> 6;
    if (row >= R) return;
    const float* xr = x + (int64_t)row * d;
    float v[LNE], s = 0.f;
#pragma unroll
    for (int e = 0; e < LNE; ++e)
        if (e < E) {
            v[e] = xr[lane + 64 * e];
            s += v[e];
        }
    const float m = wave_total(s) / (float)d;
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < LNE; ++e)
        if (e < E) q = fmaf(v[e] - m, v[e] - m, q);
    const float r = 1.0f / sqrtf(wave_total(q) / (float)d + eps);
#pragma unroll
    for (int e = 0; e < LNE; ++e)
        if (e < E) u[(int64_t)row * d + lane + 64 * e] = (v[e] - m) * r;
    if (lane == 0) {
        mu[row] = m;
        rs[row] = r;
    }
}

// Causal attention of FQ = 4 queries x one head per workgroup (one wave): the 16 lanes of
// a query split its keys (lane r takes keys r mod 16) and hold all 64 channels, so a dot
// product needs no other lane.  Each lane keeps an online softmax over its keys (running
// maximum, sum and output) and the 16 lanes merge once at the end.  The key and value tiles
// up to the queries' own 64-key tile are staged in LDS, rows padded to 68 floats so that
// the 16 lanes of a query read 16 consecutive rows at one column in distinct banks.  The raw
// logits go to the probability cache during the pass and become probabilities once the
// log-sum-exp is known: each lane rewrites the keys it wrote.
constexpr int FQ = 4;   // queries per workgroup
constexpr int FQL = 16; // lanes per query
constexpr int FKP = 68;

// over the 16 lanes of a row: quad xor 1 and 2, then the half-row and row mirrors
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));
    return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true)));
    return fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true)));
}

__global__ void __launch_bounds__(FQL * FQ) lm_attn_fwd_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                             const float* __restrict__ v, int T, int S, int H,
                                                             float* __restrict__ o, float* __restrict__ lse,
                                                             float* __restrict__ pc) {
    __shared__ __align__(16) float Ks[64][FKP];
    __shared__ __align__(16) float Vs[64][FKP];
    const int nqt = S / FQ, qt = blockIdx.x % nqt, bh = blockIdx.x / nqt, b = bh / H, h = bh % H;
    const int d = 64 * H, ql = threadIdx.x / FQL, r = threadIdx.x % FQL;
    const int query = qt * FQ + ql, q64 = (qt * FQ) / 64;  // the queries' 64-key tile
    const int64_t s0 = (int64_t)b * S, row = s0 + query;
    float qv[64];  // the query scaled by 1/8 (exact)
#pragma unroll
    for (int c4 = 0; c4 < 16; ++c4) {
        const float4 f = *reinterpret_cast<const float4*>(q + row * d + h * 64 + 4 * c4);
        qv[4 * c4] = 0.125f * f.x;
        qv[4 * c4 + 1] = 0.125f * f.y;
        qv[4 * c4 + 2] = 0.125f * f.z;
        qv[4 * c4 + 3] = 0.125f * f.w;
    }
    float m = -INFINITY, s = 0.f, acc[64];
#pragma unroll
    for (int c = 0; c < 64; ++c) acc[c] = 0.f;
    float* prow = pc + ((int64_t)bh * S + query) * S;
    for (int kt = 0; kt <= q64; ++kt) {
        __syncthreads();  // the previous tiles are used up
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {  // 64 rows x 16 float4 of each tile over the 64 lanes
            const int f = threadIdx.x + 64 * jj, rr = f >> 4, c4 = (f & 15) * 4;
            const int64_t src = (s0 + kt * 64 + rr) * d + h * 64 + c4;
            *reinterpret_cast<float4*>(&Ks[rr][c4]) = *reinterpret_cast<const float4*>(k + src);
            *reinterpret_cast<float4*>(&Vs[rr][c4]) = *reinterpret_cast<const float4*>(v + src);
        }
        __syncthreads();
        float dl[64 / FQL], tm = -INFINITY;
#pragma unroll
        for (int i = 0; i < 64 / FQL; ++i) {
            const int j = FQL * i + r, key = kt * 64 + j;
            float dot = 0.f;
#pragma unroll
            for (int c4 = 0; c4 < 16; ++c4) {
                const float4 kk = *reinterpret_cast<const float4*>(&Ks[j][4 * c4]);
                dot = fmaf(qv[4 * c4], kk.x, dot);
                dot = fmaf(qv[4 * c4 + 1], kk.y, dot);
                dot = fmaf(qv[4 * c4 + 2], kk.z, dot);
                dot = fmaf(qv[4 * c4 + 3], kk.w, dot);
            }
            dl[i] = key <= query ? dot : -INFINITY;
            tm = fmaxf(tm, dl[i]);
            prow[key] = dl[i];  // the raw logit, rewritten as a probability below
        }
        const float mn = fmaxf(m, tm), sc = mn == m ? 1.f : __expf(m - mn);
        s *= sc;
#pragma unroll
        for (int c = 0; c < 64; ++c) acc[c] *= sc;
        m = mn;
#pragma unroll
        for (int i = 0; i < 64 / FQL; ++i) {
            const int j = FQL * i + r;
            const float p = dl[i] > -INFINITY ? __expf(dl[i] - m) : 0.f;
            s += p;
#pragma unroll
            for (int c4 = 0; c4 < 16; ++c4) {
                const float4 vv = *reinterpret_cast<const float4*>(&Vs[j][4 * c4]);
                acc[4 * c4] = fmaf(p, vv.x, acc[4 * c4]);
                acc[4 * c4 + 1] = fmaf(p, vv.y, acc[4 * c4 + 1]);
                acc[4 * c4 + 2] = fmaf(p, vv.z, acc[4 * c4 + 2]);
                acc[4 * c4 + 3] = fmaf(p, vv.w, acc[4 * c4 + 3]);
            }
        }
    }
    // merge the query's lanes: lane 0 holds key 0, so the maximum is finite
    const float M = row16_max(m), sc = __expf(m - M);  // 0 for a lane whose keys were all masked
    s = row16_sum(s * sc);
#pragma unroll
    for (int c = 0; c < 64; ++c) acc[c] = row16_sum(acc[c] * sc);
    const float inv = 1.0f / s, l = M + logf(s);
    if (r == 0) {
#pragma unroll
        for (int c4 = 0; c4 < 16; ++c4)
            *reinterpret_cast<float4*>(o + row * d + h * 64 + 4 * c4) =
                make_float4(acc[4 * c4] * inv, acc[4 * c4 + 1] * inv, acc[4 * c4 + 2] * inv, acc[4 * c4 + 3] * inv);
        lse[row * H + h] = l;
    }
    // the probabilities over the key tiles up to the query's own (zero after the query):
    // pc[((b H + h) S + query) S + key]
    for (int kt = 0; kt <= q64; ++kt)
#pragma unroll
        for (int i = 0; i < 64 / FQL; ++i) {
            const int key = kt * 64 + FQL * i + r;
            prow[key] = key <= query ? __expf(prow[key] - l) : 0.f;
        }
}

__device__ __forceinline__ float phi_cdf(float x) { return 0.5f * erfcf(-x * 0.70710678118654752f); }
__device__ __forceinline__ float phi_pdf(float x) { return 0.39894228040143268f * __expf(-0.5f * x * x); }

// m = GELU(h) = h Phi(h); also Phi(h) and phi(h), which the change passes reuse
__global__ void __launch_bounds__(256) lm_gelu_kernel(const float* __restrict__ h, int64_t count,
                                                      float* __restrict__ m, float* __restrict__ cdf,
                                                      float* __restrict__ pdf) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= count) return;
    const float x = h[i], c = phi_cdf(x);
    m[i] = x * c;
    cdf[i] = c;
    pdf[i] = phi_pdf(x);
}

// out = x + alpha b
__global__ void __launch_bounds__(256) lm_residual_kernel(const float* __restrict__ x, const float* __restrict__ b,
                                                          const float* __restrict__ alpha, int64_t count,
                                                          float* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < count) out[i] = fmaf(*alpha, b[i], x[i]);
}

// Per row: lse = log sum exp z, ce = lse - z_label.  One workgroup per row.
__device__ __forceinline__ float block_total(float v, float* red) {
    v = wave_total(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__global__ void __launch_bounds__(256) lm_ce_kernel(const float* __restrict__ z, const int32_t* __restrict__ labels,
                                                    int V, float* __restrict__ lse, float* __restrict__ ce,
                                                    float* __restrict__ prob, int Vp) {
    __shared__ float red[4];
    const int64_t t = blockIdx.x;
    const float* zr = z + t * V;
    float m = -INFINITY;
    for (int j = threadIdx.x; j < V; j += 256) m = fmaxf(m, zr[j]);
    m = block_max(m, red);
    float s = 0.f;
    for (int j = threadIdx.x; j < V; j += 256) s += __expf(zr[j] - m);
    s = block_total(s, red);
    const float l = m + logf(s);
    if (threadIdx.x == 0) {
        lse[t] = l;
        ce[t] = l - zr[min(max(labels[t], 0), V - 1)];
    }
    if (prob)  // softmax row, zero past V up to the padded width Vp
        for (int j = threadIdx.x; j < Vp; j += 256) prob[t * Vp + j] = j < V ? __expf(zr[j] - l) : 0.f;
}

// ---- change-propagating forward (rows r = i T + t for draw i of the chunk) --------
// D[r][c] += sigma a(t, c, draw0 + i, layer)
__global__ void __launch_bounds__(256) lm_noise_add_kernel(float* __restrict__ D, int kc, int T, int w, float sigma,
                                                           uint32_t k0, uint32_t k1, uint32_t layer, uint32_t draw0,
                                                           int set) {
    const int64_t qi = (int64_t)blockIdx.x * 256 + threadIdx.x;  // quad index
    const int nq = w >> 2;
    if (qi >= (int64_t)kc * T * nq) return;
    const int64_t r = qi / nq;
    const int cq = (int)(qi % nq), i = (int)(r / T), t = (int)(r % T);
    const f32x4 a = gauss4((uint32_t)t, (uint32_t)cq, draw0 + (uint32_t)i, layer, k0, k1);
    float4* p = reinterpret_cast<float4*>(D + r * w + 4 * cq);
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);  // set: D holds no change yet (not read)
    if (!set) v = *p;
    v.x = fmaf(sigma, a.v[0], v.x);
    v.y = fmaf(sigma, a.v[1], v.y);
    v.z = fmaf(sigma, a.v[2], v.z);
    v.w = fmaf(sigma, a.v[3], v.w);
    *p = v;
}

__global__ void __launch_bounds__(256) lm_layernorm_delta_kernel(const float* __restrict__ x,
                                                                 const float* __restrict__ mu,
                                                                 const float* __restrict__ rs,
                                                                 const float* __restrict__ dx, int R, int T, int d,
                                                                 float* __restrict__ du) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63, E = d >> 6;
    if (row >= R) return;
    const int t = row % T;
    const float m = mu[t], r = rs[t];
    float xc[LNE], c[LNE], s = 0.f;
#pragma unroll
    for (int e = 0; e < LNE; ++e)
        if (e < E) {
            xc[e] = x[(int64_t)t * d + lane + 64 * e] - m;
            c[e] = dx[(int64_t)row * d + lane + 64 * e];
            s += c[e];
        }
    const float dm = wave_total(s) / (float)d;
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int e = 0; e < LNE; ++e)
        if (e < E) {
            c[e] -= dm;
            s1 = fmaf(xc[e], c[e], s1);
            s2 = fmaf(c[e], c[e], s2);
        }
    const float dv = (2.0f * wave_total(s1) + wave_total(s2)) / (float)d;
    const float f = expm1f(-0.5f * log1pf(dv * r * r));  // rs' / rs - 1
    const float a = r * (1.0f + f), bb = r * f;
#pragma unroll
    for (int e = 0; e < LNE; ++e)
        if (e < E) du[(int64_t)row * d + lane + 64 * e] = fmaf(c[e], a, xc[e] * bb);
}

// The same with 8 channels per lane and LPR = d / 8 lanes per row (d <= 512): several
// rows per wave, float4 accesses, sums over the row's lanes.
template <int LPR>
__device__ __forceinline__ float group_total(float v) {
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <int LPR>
__global__ void __launch_bounds__(256) lm_layernorm_delta8_kernel(const float* __restrict__ x,
                                                                  const float* __restrict__ mu,
                                                                  const float* __restrict__ rs,
                                                                  const float* __restrict__ dx, int64_t R, int T,
                                                                  float* __restrict__ du) {
    constexpr int D = 8 * LPR;
    const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
    if (row >= R) return;  // whole lane groups: the sums below stay within live groups
    const int li = threadIdx.x % LPR, t = (int)(row % T);
    const float m = mu[t], r = rs[t];
    const float* xp = x + (int64_t)t * D + 8 * li;
    const float* dp = dx + row * D + 8 * li;
    const float4 x0 = *reinterpret_cast<const float4*>(xp), x1 = *reinterpret_cast<const float4*>(xp + 4);
    const float4 d0 = *reinterpret_cast<const float4*>(dp), d1 = *reinterpret_cast<const float4*>(dp + 4);
    float xc[8] = {x0.x - m, x0.y - m, x0.z - m, x0.w - m, x1.x - m, x1.y - m, x1.z - m, x1.w - m};
    float c[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += c[e];
    const float dm = group_total<LPR>(s) / (float)D;
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        c[e] -= dm;
        s1 = fmaf(xc[e], c[e], s1);
        s2 = fmaf(c[e], c[e], s2);
    }
    const float dv = (2.0f * group_total<LPR>(s1) + group_total<LPR>(s2)) / (float)D;
    const float f = expm1f(-0.5f * log1pf(dv * r * r));  // rs' / rs - 1
    const float a = r * (1.0f + f), bb = r * f;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = fmaf(c[e], a, xc[e] * bb);
    float* op = du + row * D + 8 * li;
    *reinterpret_cast<float4*>(op) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4*>(op + 4) = make_float4(o[4], o[5], o[6], o[7]);
}

// The residual change (as lm_residual_delta_kernel) of a row, then the LayerNorm change
// of the updated row (as lm_layernorm_delta8_kernel): D_x is read once.
template <int LPR>
__global__ void __launch_bounds__(256) lm_residual_ln_delta8_kernel(float* __restrict__ dx,
                                                                    const float* __restrict__ db,
                                                                    const float* __restrict__ b,
                                                                    const float* __restrict__ scal, int slot,
                                                                    int64_t R, int T, float es_sigma,
                                                                    uint32_t member0, uint32_t k0, uint32_t k1,
                                                                    uint32_t es_layer, const float* __restrict__ x,
                                                                    const float* __restrict__ mu,
                                                                    const float* __restrict__ rs,
                                                                    float* __restrict__ du) {
    constexpr int D = 8 * LPR;
    const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
    if (row >= R) return;  // whole lane groups: the sums below stay within live groups
    const int li = threadIdx.x % LPR;
    const int64_t dr = row / T;
    const int t = (int)(row - dr * T);
    const float al = scal[slot];
    float* dp = dx + row * D + 8 * li;
    const float* bp = db + row * D + 8 * li;
    const float4 d0 = *reinterpret_cast<const float4*>(dp), d1 = *reinterpret_cast<const float4*>(dp + 4);
    const float4 y0 = *reinterpret_cast<const float4*>(bp), y1 = *reinterpret_cast<const float4*>(bp + 4);
    // the token's cached LayerNorm input and statistics, in flight with the change rows
    const float mm = mu[t], r = rs[t];
    const float* xp = x + (int64_t)t * D + 8 * li;
    const float4 x0 = *reinterpret_cast<const float4*>(xp), x1 = *reinterpret_cast<const float4*>(xp + 4);
    const float y[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
    float c[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = fmaf(al, y[e], c[e]);
    if (es_sigma > 0.f) {
        const uint32_t m = member0 + (uint32_t)dr;
        const f32x4 g = gauss4(0u, (uint32_t)(slot >> 2), m >> 1, es_layer, k0, k1);
        const float coef = ((m & 1u) ? -es_sigma : es_sigma) * g.v[slot & 3];
        const float* bb = b + (int64_t)t * D + 8 * li;
        const float4 b0 = *reinterpret_cast<const float4*>(bb), b1 = *reinterpret_cast<const float4*>(bb + 4);
        const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) c[e] = fmaf(coef, bv[e] + y[e], c[e]);
    }
    *reinterpret_cast<float4*>(dp) = make_float4(c[0], c[1], c[2], c[3]);
    *reinterpret_cast<float4*>(dp + 4) = make_float4(c[4], c[5], c[6], c[7]);
    // the LayerNorm change of the updated row
    const float xc[8] = {x0.x - mm, x0.y - mm, x0.z - mm, x0.w - mm, x1.x - mm, x1.y - mm, x1.z - mm, x1.w - mm};
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += c[e];
    const float dm = group_total<LPR>(s) / (float)D;
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        c[e] -= dm;
        s1 = fmaf(xc[e], c[e], s1);
        s2 = fmaf(c[e], c[e], s2);
    }
    const float dv = (2.0f * group_total<LPR>(s1) + group_total<LPR>(s2)) / (float)D;
    const float f = expm1f(-0.5f * log1pf(dv * r * r));  // rs' / rs - 1
    const float a = r * (1.0f + f), bf = r * f;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = fmaf(c[e], a, xc[e] * bf);
    float* op = du + row * D + 8 * li;
    *reinterpret_cast<float4*>(op) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4*>(op + 4) = make_float4(o[4], o[5], o[6], o[7]);
}


__device__ __forceinline__ float expm1_s(float x) {
    if (fabsf(x) < 0.25f)
        return x * fmaf(x, fmaf(x, fmaf(x, fmaf(x, fmaf(x, 1.0f / 720.0f, 1.0f / 120.0f), 1.0f / 24.0f),
                                          1.0f / 6.0f), 0.5f), 1.0f);
    return __expf(x) - 1.0f;
}

// D_m = GELU(h + D_h) - GELU(h) = D_h Phi(h) + (D_h + h) (Phi(h + D_h) - Phi(h)), with the
// cached Phi(h), phi(h) of the clean pass; the difference of Phi by Simpson's rule on the
// density for |D_h| < 1/4 (error below |D_h|^5 max|phi''''| / 2880), else by complementary
// error functions of one sign (no cancellation in either).
// One thread: entry j of the draws' rows for GDD draws (blockIdx.y GDD on): the cached h,
// Phi(h), phi(h) of the entry are read once for all of them
constexpr int GDD = 8;

__device__ __forceinline__ float gelu_change(float h, float c, float q, float e) {
    const float h1 = h + e;
    float dphi;
    if (fabsf(e) < 0.25f) {
        dphi = e * (1.0f / 6.0f) * (q + 4.0f * phi_pdf(h + 0.5f * e) + phi_pdf(h1));
    } else if (h + 0.5f * e > 0.f) {  // upper tail: 1 - Phi by erfc
        dphi = 0.5f * (erfcf(h * 0.70710678118654752f) - erfcf(h1 * 0.70710678118654752f));
    } else {
        dphi = 0.5f * (erfcf(-h1 * 0.70710678118654752f) - erfcf(-h * 0.70710678118654752f));
    }
    return fmaf(e, c, (e + h) * dphi);
}

// Four consecutive entries per thread (per_draw % 4 == 0), their cached h, Phi(h), phi(h)
// read once for GDD draws, every draw's change loaded before any is computed.
__global__ void __launch_bounds__(256) lm_gelu_delta_kernel(const float4* __restrict__ hc,
                                                            const float4* __restrict__ cdf,
                                                            const float4* __restrict__ pdf,
                                                            const float4* __restrict__ dh, int64_t per_draw4,
                                                            int kc, float4* __restrict__ dm) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= per_draw4) return;
    const int d0 = blockIdx.y * GDD, dn = min(GDD, kc - d0);
    float4 e[GDD];
#pragma unroll
    for (int dd = 0; dd < GDD; ++dd)
        if (dd < dn) e[dd] = dh[(int64_t)(d0 + dd) * per_draw4 + j];
    const float4 h = hc[j], c = cdf[j], q = pdf[j];
#pragma unroll
    for (int dd = 0; dd < GDD; ++dd) {
        if (dd >= dn) break;
        float4 r;
        r.x = gelu_change(h.x, c.x, q.x, e[dd].x);
        r.y = gelu_change(h.y, c.y, q.y, e[dd].y);
        r.z = gelu_change(h.z, c.z, q.z, e[dd].z);
        r.w = gelu_change(h.w, c.w, q.w, e[dd].w);
        dm[(int64_t)(d0 + dd) * per_draw4 + j] = r;
    }
}

// dx += alpha db, plus for an ES member (es_sigma > 0) the change of the scalar:
// + s sigma_es eps_{j, slot} (b + db), member m = member0 + i, j = m / 2, s = +1 / -1
// for even / odd m, eps from the noise stream (token 0, channel slot, draw j).
__global__ void __launch_bounds__(256) lm_residual_delta_kernel(float* __restrict__ dx, const float* __restrict__ db,
                                                                const float* __restrict__ b,
                                                                const float* __restrict__ scal, int slot, int kc,
                                                                int64_t per_draw, float es_sigma, uint32_t member0,
                                                                uint32_t k0, uint32_t k1, uint32_t es_layer) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)kc * per_draw) return;
    const float al = scal[slot];
    float v = fmaf(al, db[idx], dx[idx]);
    if (es_sigma > 0.f) {
        const uint32_t m = member0 + (uint32_t)(idx / per_draw);
        const f32x4 g = gauss4(0u, (uint32_t)(slot >> 2), m >> 1, es_layer, k0, k1);
        const float coef = ((m & 1u) ? -es_sigma : es_sigma) * g.v[slot & 3];
        v = fmaf(coef, b[idx % per_draw] + db[idx], v);
    }
    dx[idx] = v;
}

// rew[r] = -(log1p(sum_v p_v expm1(D_z_v)) - D_z_y),  p = exp(z - lse)
__global__ void __launch_bounds__(256) lm_ce_delta_kernel(const float* __restrict__ z, const float* __restrict__ lse,
                                                          const float* __restrict__ dz,
                                                          const int32_t* __restrict__ labels, int T, int V,
                                                          float* __restrict__ rew) {
    __shared__ float red[4];
    const int64_t r = blockIdx.x;
    const int t = (int)(r % T);
    const float* zr = z + (int64_t)t * V;
    const float* dr = dz + r * V;
    const float l = lse[t];
    float s = 0.f;
    for (int j = threadIdx.x; j < V; j += 256) s = fmaf(__expf(zr[j] - l), expm1f(dr[j]), s);
    s = block_total(s, red);
    if (threadIdx.x == 0) rew[r] = dr[min(max(labels[t], 0), V - 1)] - log1pf(s);
}

// g_hat[t][c] = scale sum_i rew[i][t] a(t, c, draw0 + i, layer)
// ghat[t][c] = scale sum_i rew[i][t] a(t, c, i): one workgroup per (token, 32 channel quads);
// its 8 thread groups take draws g, g + 8, ... and their sums are added in a fixed order
// through LDS (noise regenerated)
__global__ void __launch_bounds__(256) lm_ghat_kernel(const float* __restrict__ rew, int K, int T, int w, float scale,
                                                      uint32_t k0, uint32_t k1, uint32_t layer,
                                                      float* __restrict__ ghat) {
    __shared__ float4 part[8][32];
    const int nq = w >> 2, nch = (nq + 31) / 32;
    const int t = blockIdx.x / nch, cq = (blockIdx.x % nch) * 32 + (threadIdx.x & 31), g = threadIdx.x >> 5;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    if (cq < nq)
        for (int i = g; i < K; i += 8) {
            const float r = rew[(int64_t)i * T + t];
            const f32x4 a = gauss4((uint32_t)t, (uint32_t)cq, (uint32_t)i, layer, k0, k1);
            s0 = fmaf(r, a.v[0], s0);
            s1 = fmaf(r, a.v[1], s1);
            s2 = fmaf(r, a.v[2], s2);
            s3 = fmaf(r, a.v[3], s3);
        }
    part[g][threadIdx.x & 31] = make_float4(s0, s1, s2, s3);
    __syncthreads();
    if (threadIdx.x < 32 && cq < nq) {
        float4 v = part[0][threadIdx.x];
        for (int gg = 1; gg < 8; ++gg) {
            const float4 o = part[gg][threadIdx.x];
            v.x += o.x;
            v.y += o.y;
            v.z += o.z;
            v.w += o.w;
        }
        *reinterpret_cast<float4*>(ghat + (int64_t)t * w + 4 * cq) =
            make_float4(v.x * scale, v.y * scale, v.z * scale, v.w * scale);
    }
}

// G_E[v] = sum over the tokens t with id v of g_hat[t], in token order (deterministic);
// G_P[s] = sum over sequences of g_hat at position s.  The embedding gradient takes one
// workgroup per token t: unless an earlier token has t's id (each wave checks 64 ids per
// ballot), it walks the ids from t on, 64 per ballot, and adds the matching rows in token
// order.  Rows no token names keep the zero written before.  Ids outside [0, V) add nothing.
constexpr int ECH = 4;  // channels per thread: d <= 1024

constexpr int EMB_G = 8;  // matching rows gathered per load wait in the embedding gradient

__global__ void __launch_bounds__(256) lm_embed_grad_kernel(const float* __restrict__ ghat,
                                                            const int32_t* __restrict__ tok, int T, int V, int d,
                                                            float* __restrict__ gemb) {
    const int t = blockIdx.x, lane = threadIdx.x & 63;
    const int id = tok[t];
    if (id < 0 || id >= V) return;
    // an earlier token with this id owns the row; 4 chunks of 64 tokens per load wait (the
    // same answer in every wave: the workgroup leaves together)
    for (int u0 = 0; u0 < t; u0 += 256) {
        bool seen = false;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int u = u0 + 64 * q + lane;
            seen |= u < t && tok[u] == id;
        }
        if (__builtin_amdgcn_ballot_w64(seen)) return;
    }
    float acc[ECH];
#pragma unroll
    for (int k = 0; k < ECH; ++k) acc[k] = 0.f;
    for (int u0 = t; u0 < T; u0 += 64) {
        const int u = u0 + lane;
        uint64_t m = __builtin_amdgcn_ballot_w64(u < T && tok[u] == id);
        while (m) {  // matches in increasing token order, up to EMB_G rows loaded per wait
            int rows[EMB_G];
            int nr = 0;
#pragma unroll
            for (int j = 0; j < EMB_G; ++j) {
                rows[j] = m ? u0 + __builtin_ctzll(m) : -1;
                if (m) {
                    m &= m - 1;
                    ++nr;
                }
            }
            float v[EMB_G][ECH];
#pragma unroll
            for (int j = 0; j < EMB_G; ++j)
#pragma unroll
                for (int k = 0; k < ECH; ++k) {
                    const int c = threadIdx.x + 256 * k;
                    v[j][k] = (j < nr && c < d) ? ghat[(int64_t)rows[j] * d + c] : 0.f;
                }
#pragma unroll
            for (int j = 0; j < EMB_G; ++j)
#pragma unroll
                for (int k = 0; k < ECH; ++k)
                    if (j < nr) acc[k] += v[j][k];
        }
    }
#pragma unroll
    for (int k = 0; k < ECH; ++k) {
        const int c = threadIdx.x + 256 * k;
        if (c < d) gemb[(int64_t)id * d + c] = acc[k];
    }
}

__global__ void __launch_bounds__(256) lm_pos_grad_kernel(const float* __restrict__ ghat, int T, int S, int d,
                                                          float* __restrict__ gpos) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)S * d) return;
    float s = 0.f;
    for (int b = 0; b < T / S; ++b) s += ghat[(int64_t)b * S * d + i];
    gpos[i] = s;
}

__global__ void __launch_bounds__(256) lm_transpose_kernel(const float* __restrict__ W, int R, int Cn,
                                                           float* __restrict__ WT) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)R * Cn) return;
    const int r = (int)(i / Cn), c = (int)(i % Cn);
    WT[(int64_t)c * R + r] = W[i];
}

// dL[m] = -sum_t rew[m][t] (the member's summed-loss change), fixed order.
__global__ void __launch_bounds__(256) lm_rowsum_neg_kernel(const float* __restrict__ rew, int T,
                                                            float* __restrict__ out) {
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    float s = 0.f;
    for (int t = threadIdx.x; t < T; t += 256) s += rew[m * T + t];
    s = block_total(s, red);
    if (threadIdx.x == 0) out[m] = -s;
}

// g[c] = scale sum_j (dL[2j] - dL[2j+1]) eps_{j,c}
__global__ void __launch_bounds__(64) lm_es_grad_kernel(const float* __restrict__ dL, int M, int nsc, float scale,
                                                        uint32_t k0, uint32_t k1, uint32_t es_layer,
                                                        float* __restrict__ g) {
    const int c = threadIdx.x;
    if (c >= nsc) return;
    float s = 0.f;
    for (int j = 0; j < M; ++j) {
        const f32x4 e = gauss4(0u, (uint32_t)(c >> 2), (uint32_t)j, es_layer, k0, k1);
        s = fmaf(dL[2 * j] - dL[2 * j + 1], e.v[c & 3], s);
    }
    g[c] = s * scale;
}

__global__ void __launch_bounds__(256) lm_sgd_kernel(float* __restrict__ theta, float* __restrict__ mom,
                                                     const float* __restrict__ G, int64_t count, int64_t scal0,
                                                     float lr, float lr_scalar, float mu) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= count) return;
    const float m = fmaf(mu, mom[i], G[i]);
    mom[i] = m;
    theta[i] = fmaf(-(i >= scal0 ? lr_scalar : lr), m, theta[i]);
}

// ---- head change fused with its loss change (bf16x3 MFMA) -----------------------
typedef float hf32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 hbf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 hbf16x8 __attribute__((ext_vector_type(8)));
typedef float hf32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {  // round to nearest even, a in the low half
    const hf32x2 v = {a, b};
    const hbf16x2 h = __builtin_convertvector(v, hbf16x2);
    uint32_t u;
    __builtin_memcpy(&u, &h, 4);
    return u;
}

// 8 fp32 values as bf16 hi and lo parts: x = hi + lo within 2^-17 |x|
__device__ __forceinline__ void split8(const float4& x0, const float4& x1, uint4& hi, uint4& lo) {
    const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        h[q] = bf16_pair(x[2 * q], x[2 * q + 1]);
        l[q] = bf16_pair(x[2 * q] - __uint_as_float(h[q] << 16), x[2 * q + 1] - __uint_as_float(h[q] & 0xFFFF0000u));
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
}

__device__ __forceinline__ hf32x16 mfma_bf16(const uint4& a, const uint4& b, const hf32x16& c) {
    hbf16x8 av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
}

// hi/lo bf16 parts of a [rows, K] fp32 matrix into [rows_p, K] arrays (rows past `rows` zero)
__global__ void __launch_bounds__(256) lm_split_kernel(const float* __restrict__ W, int64_t rows, int64_t rows_p,
                                                       int K, uint32_t* __restrict__ hi, uint32_t* __restrict__ lo) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // pair index
    if (i >= rows_p * K / 2) return;
    const int64_t row = (2 * i) / K;
    const float a = row < rows ? W[2 * i] : 0.f, b = row < rows ? W[2 * i + 1] : 0.f;
    const uint32_t h = bf16_pair(a, b);
    hi[i] = h;
    lo[i] = bf16_pair(a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xFFFF0000u));
}

// hi/lo bf16 parts of W [rows, K] in MFMA fragment order: 16-byte unit u = ((vb KS + ks) 64 + lane)
// (KS = K / 16) holds channels 16 ks + 8 (lane >> 5) + [0, 8) of row 32 vb + (lane & 31), so a
// wave's fragment load of one 32-row block and channel step reads 1 KB contiguous; rows past
// `rows` are zero
__global__ void __launch_bounds__(256) lm_split_frag_kernel(const float* __restrict__ W, int64_t rows, int64_t rows_p,
                                                            int K, uint4* __restrict__ hi, uint4* __restrict__ lo) {
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int KS = K / 16;
    if (u >= rows_p * K / 8) return;
    const int lane = (int)(u & 63), ks = (int)((u >> 6) % KS);
    const int64_t vb = (u >> 6) / KS, row = vb * 32 + (lane & 31);
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (row < rows) {
        const float* src = W + row * K + 16 * ks + 8 * (lane >> 5);
        a = *reinterpret_cast<const float4*>(src);
        b = *reinterpret_cast<const float4*>(src + 4);
    }
    uint4 h, l;
    split8(a, b, h, l);
    hi[u] = h;
    lo[u] = l;
}

// expm1 of 16 values: the degree-6 Taylor polynomial (relative truncation below 5e-8
// for |x| < 1/4); waves holding a larger |x| take exp(x) - 1 for those values.
__device__ __forceinline__ void expm1_x16(float (&x)[16]) {
    bool big = false;
#pragma unroll
    for (int r = 0; r < 16; ++r) big |= fabsf(x[r]) >= 0.25f;
    float q[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
        q[r] = x[r] * fmaf(x[r], fmaf(x[r], fmaf(x[r], fmaf(x[r], fmaf(x[r], 1.0f / 720.0f, 1.0f / 120.0f),
                                                             1.0f / 24.0f), 1.0f / 6.0f), 0.5f), 1.0f);
    if (__builtin_amdgcn_ballot_w64(big)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) q[r] = fabsf(x[r]) < 0.25f ? q[r] : __expf(x[r]) - 1.0f;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = q[r];
}

// the degree-6 Taylor polynomial of exp(x) - 1 (relative truncation below 5e-8 for |x| < 1/4)
__device__ __forceinline__ float expm1_poly(float x) {
    return x * fmaf(x, fmaf(x, fmaf(x, fmaf(x, fmaf(x, 1.0f / 720.0f, 1.0f / 120.0f), 1.0f / 24.0f), 1.0f / 6.0f),
                        0.5f), 1.0f);
}

// Per row r (draw i, token t) and vocabulary segment: sum_v p_t[v] expm1(D_z[r][v]) with
// D_z = D_u W_head^T formed on bf16x3 MFMA (products within ~3 2^-17 of fp32), as the
// transposed product D_z^T[v][r] so that a lane holds one row (token) and 16 of its
// vocabulary entries: the row's sum accumulates in one register.  One workgroup: a
// block of 64 tokens x one vocabulary segment x a group of HDG draws; the group's D_u
// rows are split into bf16 parts once, into LDS; each wave takes every eighth 32-entry
// vocabulary block of the segment, holds its W_head fragments and the 64 tokens'
// probabilities in registers and runs all the group's rows against them.  Workgroups
// of one (token block, segment) run on one XCD (workgroup id mod 8), sharing its L2.
constexpr int HDG = 4;   // draws per workgroup
constexpr int HW = 8;    // waves per workgroup (two per SIMD)

// slot swizzle of the split D_u rows in LDS (2 KS 16-byte slots per row)
template <int KS>
__device__ __forceinline__ int head_swz(int row) {
    static_assert(KS == 4 || KS == 8, "d = 64 or 128");
    return KS == 8 ? (row & 15) : ((row & 7) ^ ((row >> 3) & 1));
}

// D_z^T block of 32 vocabulary rows (the W_head fragments a lane holds) x the 32 tokens
// of `row`'s half, for draw j of the workgroup's group: hi*lo + lo*hi + hi*hi per 16 channels
template <int KS>
__device__ __forceinline__ hf32x16 head_block(const uint4 (&ahi)[KS], const uint4 (&alo)[KS], const uint4* UH,
                                              const uint4* UL, int j, int row, int hf) {
    hf32x16 c = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int at = (j * 64 + row) * 2 * KS + ((2 * ks + hf) ^ head_swz<KS>(row));
        const uint4 h = UH[at], l = UL[at];
        c = mfma_bf16(alo[ks], h, c);
        c = mfma_bf16(ahi[ks], l, c);
        c = mfma_bf16(ahi[ks], h, c);
    }
    return c;
}

template <int KS>  // d = 16 KS
__global__ void __launch_bounds__(64 * HW) lm_head_delta_kernel(const float* __restrict__ du,
                                                            const uint16_t* __restrict__ whi,
                                                            const uint16_t* __restrict__ wlo,
                                                            const float* __restrict__ prob, int T, int Vp, int vseg,
                                                            int nseg, int kc, float* __restrict__ part) {
    constexpr int D = 16 * KS, UNITS = HDG * 64 * KS * 2;  // 16-byte units of one group's parts
    __shared__ uint4 UH[UNITS];
    __shared__ uint4 UL[UNITS];
    __shared__ float red[HW][HDG][64];
    const int ngr = (kc + HDG - 1) / HDG;
    const int id = blockIdx.x, xcd = id & 7, loc = id >> 3;
    const int pair = xcd + 8 * (loc / ngr), g = loc % ngr;
    if (pair >= (T / 64) * nseg) return;
    const int tb = pair / nseg, sg = pair % nseg, dn = min(HDG, kc - g * HDG);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hf = lane >> 5;
    // unit (j, row, ks, h) = 8 channels 16 ks + 8 h of row `row` of draw j, stored at slot
    // (2 ks + h) ^ head_swz(row) of the row's 2 KS slots: any 8 (and any 16) consecutive rows
    // reading one (ks, h) hit distinct 16-byte bank groups
    // draws past the last one of a short group are zero rows: their changes are 0 and unused
    for (int u = threadIdx.x; u < UNITS; u += 64 * HW) {
        const int h = u & 1, ks = (u >> 1) % KS, row = (u / (2 * KS)) % 64, j = u / (2 * KS * 64);
        uint4 hi = make_uint4(0, 0, 0, 0), lo = hi;
        if (j < dn) {
            const float* a = du + ((int64_t)(g * HDG + j) * T + (int64_t)tb * 64 + row) * D + 16 * ks + 8 * h;
            split8(*reinterpret_cast<const float4*>(a), *reinterpret_cast<const float4*>(a + 4), hi, lo);
        }
        const int at = (j * 64 + row) * 2 * KS + ((2 * ks + h) ^ head_swz<KS>(row));
        UH[at] = hi;
        UL[at] = lo;
    }
    __syncthreads();
    float s[HDG][2];
#pragma unroll
    for (int j = 0; j < HDG; ++j) s[j][0] = s[j][1] = 0.f;
    const int vb = sg * vseg, ve = min(Vp, vb + vseg);
    for (int v0 = vb + 32 * w; v0 < ve; v0 += 32 * HW) {
        uint4 ahi[KS], alo[KS];  // W_head rows v0 + (lane & 31), channels 16 ks + 8 hf + [0, 8)
        // the parts are stored in fragment order: unit ((v0 / 32) KS + ks) 64 + lane
        const uint4* bh = reinterpret_cast<const uint4*>(whi) + (int64_t)(v0 / 32) * KS * 64 + lane;
        const uint4* bl = reinterpret_cast<const uint4*>(wlo) + (int64_t)(v0 / 32) * KS * 64 + lane;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            ahi[ks] = bh[ks * 64];
            alo[ks] = bl[ks * 64];
        }
        float pv[2][16];  // p of this lane's token (column) at the 16 vocabulary rows it holds, per token half
#pragma unroll
        for (int th = 0; th < 2; ++th) {
            const float* pp = prob + ((int64_t)tb * 64 + 32 * th + (lane & 31)) * Vp + v0 + 4 * hf;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float4 q = *reinterpret_cast<const float4*>(pp + 8 * m);
                pv[th][4 * m] = q.x;
                pv[th][4 * m + 1] = q.y;
                pv[th][4 * m + 2] = q.z;
                pv[th][4 * m + 3] = q.w;
            }
        }
        // Fast pass over the (token half, draw) blocks with the polynomial alone, branch-free and
        // software-pipelined: stage b runs block b's MFMA chain beside block b - 1's exp - 1 and
        // sum (scheduling barriers keep two blocks live at most).  A block in which some |D_z|
        // reaches 1/4 is flagged (wave-uniform) and recomputed below.
        float acc[2][HDG];
        uint32_t bad = 0;
        hf32x16 cp = head_block<KS>(ahi, alo, UH, UL, 0, lane & 31, hf);
#pragma unroll
        for (int b = 1; b <= 2 * HDG; ++b) {
            hf32x16 cn;
            if (b < 2 * HDG) cn = head_block<KS>(ahi, alo, UH, UL, b % HDG, 32 * (b / HDG) + (lane & 31), hf);
            const int th = (b - 1) / HDG, j = (b - 1) % HDG;
            float mx = 0.f, a = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                mx = fmaxf(mx, fabsf(cp[r]));
                a = fmaf(pv[th][r], expm1_poly(cp[r]), a);
            }
            acc[th][j] = a;
            bad |= __builtin_amdgcn_ballot_w64(mx >= 0.25f) ? 1u << (b - 1) : 0u;
            __builtin_amdgcn_sched_barrier(0);
            if (b < 2 * HDG) cp = cn;
        }
        if (bad) {  // exact pass for the flagged blocks: exp(x) - 1 where |x| >= 1/4
            for (int b = 0; b < 2 * HDG; ++b) {
                if (!((bad >> b) & 1)) continue;
                const int th = b / HDG, j = b % HDG, row = 32 * th + (lane & 31);
                const hf32x16 c = head_block<KS>(ahi, alo, UH, UL, j, row, hf);
                float a = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float x = c[r];
                    a = fmaf(th ? pv[1][r] : pv[0][r], fabsf(x) < 0.25f ? expm1_poly(x) : __expf(x) - 1.0f, a);
                }
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int jj = 0; jj < HDG; ++jj)
                        if (tt * HDG + jj == b) acc[tt][jj] = a;
            }
        }
#pragma unroll
        for (int th = 0; th < 2; ++th)
#pragma unroll
            for (int j = 0; j < HDG; ++j) s[j][th] += acc[th][j];
    }
    // the two halves of a wave hold the same tokens (different vocabulary rows); then the waves
#pragma unroll
    for (int j = 0; j < HDG; ++j)
#pragma unroll
        for (int th = 0; th < 2; ++th) s[j][th] += __shfl_xor(s[j][th], 32, 64);
    if (hf == 0) {
#pragma unroll
        for (int j = 0; j < HDG; ++j) {
            red[w][j][lane] = s[j][0];
            red[w][j][32 + lane] = s[j][1];
        }
    }
    __syncthreads();
    for (int x = threadIdx.x; x < dn * 64; x += 64 * HW) {
        const int j = x >> 6, q = x & 63;
        float t = 0.f;
#pragma unroll
        for (int ww = 0; ww < HW; ++ww) t += red[ww][j][q];
        part[((int64_t)(g * HDG + j) * T + (int64_t)tb * 64 + q) * nseg + sg] = t;
    }
}

// rew[r] = D_z_y - log1p(sum over segments), D_z_y = <D_u[r], W_head[y_t]> in fp32.
// One wave per row.
__global__ void __launch_bounds__(256) lm_head_reward_kernel(const float* __restrict__ du,
                                                             const float* __restrict__ whead,
                                                             const int32_t* __restrict__ labels,
                                                             const float* __restrict__ part, int T, int V, int d,
                                                             int nseg, int64_t rows, float* __restrict__ rew) {
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    const int lane = threadIdx.x & 63, t = (int)(r % T), y = min(max(labels[t], 0), V - 1);
    float zy = 0.f, ps = 0.f;
    for (int c = lane; c < d; c += 64) zy = fmaf(du[r * d + c], whead[(int64_t)y * d + c], zy);
    for (int j = lane; j < nseg; j += 64) ps += part[r * nseg + j];
    zy = wave_total(zy);
    ps = wave_total(ps);
    if (lane == 0) rew[r] = zy - log1pf(ps);
}

// The same rewards with 16 lanes per row (4 rows per wave) for d = 64 or 128 and at most 16
// segments: CPL channels per lane, sums over the lane group by DPP row operations.
__device__ __forceinline__ float row16_total(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));   // quad: lane ^ 1
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));   // quad: lane ^ 2
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));  // half-row mirror
    return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));  // row mirror
}

template <int CPL>
__global__ void __launch_bounds__(256) lm_head_reward16_kernel(const float* __restrict__ du,
                                                               const float* __restrict__ whead,
                                                               const int32_t* __restrict__ labels,
                                                               const float* __restrict__ part, int T, int V, int nseg,
                                                               int64_t rows, float* __restrict__ rew) {
    constexpr int D = 16 * CPL;
    const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
    if (r >= rows) return;  // whole 16-lane rows: the DPP sums stay within live rows
    const int li = threadIdx.x & 15, t = (int)(r % T), y = min(max(labels[t], 0), V - 1);
    const float* a = du + r * D + CPL * li;
    const float* w = whead + (int64_t)y * D + CPL * li;
    float zy = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; c += 4) {
        const float4 av = *reinterpret_cast<const float4*>(a + c), wv = *reinterpret_cast<const float4*>(w + c);
        zy = fmaf(av.x, wv.x, zy);
        zy = fmaf(av.y, wv.y, zy);
        zy = fmaf(av.z, wv.z, zy);
        zy = fmaf(av.w, wv.w, zy);
    }
    float ps = li < nseg ? part[r * nseg + li] : 0.f;
    zy = row16_total(zy);
    ps = row16_total(ps);
    if (li == 0) rew[r] = zy - log1pf(ps);
}

// ---- change of the attention output (bf16x3 MFMA) ---------------------------------
// One workgroup: draw i, sequence b, head h, 64 queries; wave w takes queries 32 (w >> 1)
// and, of every 64-key tile, keys 32 (w & 1).  Per key tile:
//   delta^T[key][query] = (<k, D_q> + <D_k, q + D_q>) / 8  (one accumulator, 24 MFMAs),
//   w1 = P expm1(delta), w2 = P + w1 with P the cached clean probabilities,
//   acc^T[c][query] += sum_key v[key][c] w1 + D_v[key][c] w2  (24 MFMAs),
// the weights going from the accumulator registers straight into the second product's
// B operand: register r of a lane holds key (r & 3) + 8 (r >> 2) + 4 (lane >> 5), so
// k-step s takes registers 8 s .. 8 s + 7 and v, D_v are read from LDS, transposed to
// [channel][key] bf16 parts, in that key order.  Then
//   D_o = (acc - rho o) / (1 + rho),  rho = sum_key w1,
// the two key halves added through LDS.
constexpr int AVP = 68;  // padded row of the transposed tiles (bf16): 136 bytes, so that the 8-byte
                         // reads of 32 consecutive channels at one key fall in distinct bank pairs

// the transposed tiles, and after the last tile the odd key half's partial sums in the same bytes
union AttnDeltaLds {
    struct {
        uint16_t vth[64][AVP], vtl[64][AVP], dvth[64][AVP], dvtl[64][AVP];
    } t;
    float accx[2][64][33];  // [query block][channel][query]
};

__device__ __forceinline__ uint4 vt_frag(const uint16_t (*t)[AVP], int c, int k0) {
    const uint2 a = *reinterpret_cast<const uint2*>(&t[c][k0]);
    const uint2 b = *reinterpret_cast<const uint2*>(&t[c][k0 + 8]);
    return make_uint4(a.x, a.y, b.x, b.y);
}

__global__ void __launch_bounds__(256) lm_attn_delta_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                            const float* __restrict__ v, const float* __restrict__ o,
                                                            const float* __restrict__ pc,
                                                            const float* __restrict__ dq,
                                                            const float* __restrict__ dk,
                                                            const float* __restrict__ dv, int T, int S, int H,
                                                            float* __restrict__ dout) {
    __shared__ __align__(16) AttnDeltaLds lds;
    __shared__ float rhox[2][32];
    uint16_t(*VTH)[AVP] = lds.t.vth;
    uint16_t(*VTL)[AVP] = lds.t.vtl;
    uint16_t(*DVTH)[AVP] = lds.t.dvth;
    uint16_t(*DVTL)[AVP] = lds.t.dvtl;
    float(*accx)[64][33] = lds.accx;
    const int nqt = S / 64, nbh = (T / S) * H;
    const int qt = blockIdx.x % nqt, bh = (blockIdx.x / nqt) % nbh, i = blockIdx.x / (nqt * nbh);
    const int b = bh / H, h = bh % H, d = 64 * H;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, qb = w >> 1, kb = w & 1, hf = lane >> 5, l31 = lane & 31;
    const int64_t s0 = (int64_t)b * S, drow0 = (int64_t)i * T;
    const int query = qt * 64 + 32 * qb + l31;  // this lane's query (column of both products)
    // B operands over the channels: D_q and q + D_q of this wave's 32 queries
    uint4 dqh[4], dql[4], qqh[4], qql[4];
    {
        const float* pq = q + (s0 + query) * d + h * 64 + 8 * hf;
        const float* pd = dq + (drow0 + s0 + query) * d + h * 64 + 8 * hf;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float4 a0 = *reinterpret_cast<const float4*>(pd + 16 * ks);
            float4 a1 = *reinterpret_cast<const float4*>(pd + 16 * ks + 4);
            const float4 b0 = *reinterpret_cast<const float4*>(pq + 16 * ks);
            const float4 b1 = *reinterpret_cast<const float4*>(pq + 16 * ks + 4);
            split8(a0, a1, dqh[ks], dql[ks]);
            a0 = make_float4(a0.x + b0.x, a0.y + b0.y, a0.z + b0.z, a0.w + b0.w);
            a1 = make_float4(a1.x + b1.x, a1.y + b1.y, a1.z + b1.z, a1.w + b1.w);
            split8(a0, a1, qqh[ks], qql[ks]);
        }
    }
    hf32x16 acc0 = {}, acc1 = {};  // channels 0..31 and 32..63 (rows) x this wave's queries
    float rho = 0.f;
    const float* prow = pc + ((int64_t)bh * S + query) * S;
    for (int kt = 0; kt <= qt; ++kt) {
        __syncthreads();  // the previous tile's transposed values are used up
        // v and D_v of the 64 keys, transposed into bf16 parts: unit = 2 keys x 4 channels.
        // A wave takes 8 key pairs x 8 channel quads (each row read is one 128-byte line), so
        // its transposed 4-byte writes land on 32 distinct banks per half-wave
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int f = threadIdx.x + 256 * u, kp = (f >> 3) & 31, c4 = ((f & 7) + 8 * (f >> 8)) * 4;
            const int64_t r0 = s0 + kt * 64 + 2 * kp;
            const float4 va = *reinterpret_cast<const float4*>(v + r0 * d + h * 64 + c4);
            const float4 vb = *reinterpret_cast<const float4*>(v + (r0 + 1) * d + h * 64 + c4);
            const float4 da = *reinterpret_cast<const float4*>(dv + (drow0 + r0) * d + h * 64 + c4);
            const float4 db = *reinterpret_cast<const float4*>(dv + (drow0 + r0 + 1) * d + h * 64 + c4);
            const float xa[4] = {va.x, va.y, va.z, va.w}, xb[4] = {vb.x, vb.y, vb.z, vb.w};
            const float ya[4] = {da.x, da.y, da.z, da.w}, yb[4] = {db.x, db.y, db.z, db.w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint32_t hv = bf16_pair(xa[m], xb[m]);
                const uint32_t lv = bf16_pair(xa[m] - __uint_as_float(hv << 16), xb[m] - __uint_as_float(hv & 0xFFFF0000u));
                const uint32_t hd = bf16_pair(ya[m], yb[m]);
                const uint32_t ld = bf16_pair(ya[m] - __uint_as_float(hd << 16), yb[m] - __uint_as_float(hd & 0xFFFF0000u));
                *reinterpret_cast<uint32_t*>(&VTH[c4 + m][2 * kp]) = hv;
                *reinterpret_cast<uint32_t*>(&VTL[c4 + m][2 * kp]) = lv;
                *reinterpret_cast<uint32_t*>(&DVTH[c4 + m][2 * kp]) = hd;
                *reinterpret_cast<uint32_t*>(&DVTL[c4 + m][2 * kp]) = ld;
            }
        }
        // logit change of this wave's 32 keys x 32 queries
        const int64_t krow = s0 + kt * 64 + 32 * kb + l31;
        hf32x16 dl = {};
        {
            const float* pk = k + krow * d + h * 64 + 8 * hf;
            const float* pdk = dk + (drow0 + krow) * d + h * 64 + 8 * hf;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                uint4 kh, kl, dh, dlo;
                split8(*reinterpret_cast<const float4*>(pk + 16 * ks), *reinterpret_cast<const float4*>(pk + 16 * ks + 4),
                       kh, kl);
                split8(*reinterpret_cast<const float4*>(pdk + 16 * ks),
                       *reinterpret_cast<const float4*>(pdk + 16 * ks + 4), dh, dlo);
                dl = mfma_bf16(kl, dqh[ks], dl);
                dl = mfma_bf16(kh, dql[ks], dl);
                dl = mfma_bf16(kh, dqh[ks], dl);
                dl = mfma_bf16(dlo, qqh[ks], dl);
                dl = mfma_bf16(dh, qql[ks], dl);
                dl = mfma_bf16(dh, qqh[ks], dl);
            }
        }
        float x[16], pv[16];
#pragma unroll
        for (int m = 0; m < 4; ++m) {  // P of keys 8 m + 4 hf + [0, 4) of this key half
            const float4 pp = *reinterpret_cast<const float4*>(prow + kt * 64 + 32 * kb + 8 * m + 4 * hf);
            pv[4 * m] = pp.x;
            pv[4 * m + 1] = pp.y;
            pv[4 * m + 2] = pp.z;
            pv[4 * m + 3] = pp.w;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = dl[r] * 0.125f;
        expm1_x16(x);
        uint4 w1h[2], w1l[2], w2h[2], w2l[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            uint32_t a[4], al[4], c[4], cl[4];
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
                const int r = 8 * st + 2 * pr;
                const float u0 = pv[r] * x[r], u1 = pv[r + 1] * x[r + 1];  // w1
                const float z0 = pv[r] + u0, z1 = pv[r + 1] + u1;          // w2
                rho += u0 + u1;
                a[pr] = bf16_pair(u0, u1);
                al[pr] = bf16_pair(u0 - __uint_as_float(a[pr] << 16), u1 - __uint_as_float(a[pr] & 0xFFFF0000u));
                c[pr] = bf16_pair(z0, z1);
                cl[pr] = bf16_pair(z0 - __uint_as_float(c[pr] << 16), z1 - __uint_as_float(c[pr] & 0xFFFF0000u));
            }
            w1h[st] = make_uint4(a[0], a[1], a[2], a[3]);
            w1l[st] = make_uint4(al[0], al[1], al[2], al[3]);
            w2h[st] = make_uint4(c[0], c[1], c[2], c[3]);
            w2l[st] = make_uint4(cl[0], cl[1], cl[2], cl[3]);
        }
        __syncthreads();  // transposed tiles written
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int k0 = 32 * kb + 16 * st + 4 * hf;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                const int c = 32 * cb + l31;
                const uint4 vh = vt_frag(VTH, c, k0), vl = vt_frag(VTL, c, k0);
                const uint4 eh = vt_frag(DVTH, c, k0), el = vt_frag(DVTL, c, k0);
                hf32x16& a = cb ? acc1 : acc0;
                a = mfma_bf16(vl, w1h[st], a);
                a = mfma_bf16(vh, w1l[st], a);
                a = mfma_bf16(vh, w1h[st], a);
                a = mfma_bf16(el, w2h[st], a);
                a = mfma_bf16(eh, w2l[st], a);
                a = mfma_bf16(eh, w2h[st], a);
            }
        }
    }
    rho += __shfl_xor(rho, 32, 64);  // the lane pair of a query holds its two key quarters
    __syncthreads();  // the last tile's transposed values are used up: accx takes their bytes
    if (kb == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int cr = (r & 3) + 8 * (r >> 2) + 4 * hf;
            accx[qb][cr][l31] = acc0[r];
            accx[qb][32 + cr][l31] = acc1[r];
        }
        if (hf == 0) rhox[qb][l31] = rho;
    }
    __syncthreads();
    if (kb == 0) {
        const float rt = rho + rhox[qb][l31], inv = 1.0f / (1.0f + rt);
        const int64_t orow = s0 + query;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int m = 0; m < 4; ++m) {  // channels 32 cb + 8 m + 4 hf + [0, 4)
                const int c0 = 32 * cb + 8 * m + 4 * hf;
                const float4 ov = *reinterpret_cast<const float4*>(o + orow * d + h * 64 + c0);
                const hf32x16& a = cb ? acc1 : acc0;
                float4 r4;
                r4.x = (a[4 * m] + accx[qb][c0][l31] - rt * ov.x) * inv;
                r4.y = (a[4 * m + 1] + accx[qb][c0 + 1][l31] - rt * ov.y) * inv;
                r4.z = (a[4 * m + 2] + accx[qb][c0 + 2][l31] - rt * ov.z) * inv;
                r4.w = (a[4 * m + 3] + accx[qb][c0 + 3][l31] - rt * ov.w) * inv;
                *reinterpret_cast<float4*>(dout + (drow0 + orow) * d + h * 64 + c0) = r4;
            }
    }
}

// ---- change rows times a weight on bf16x3 MFMA: C = A B^T ----------------------------
// A [M, K] fp32 (change rows), B [N, K] given as bf16 parts Bh, Bl (the weight split once
// per step).  Workgroup tile 128 rows x 128 columns, 4 waves of 64 x 64 (2 x 2 MFMA
// blocks), over chunks of XK channels.  A chunk's rows are read whole (8 lanes per 128-byte
// row piece), split into bf16 parts once and staged in LDS beside B's parts; the next
// chunk's loads are in flight while this chunk's MFMAs run.  Rows past M are read clamped
// and not stored; columns past N read zero weights and are not stored; K % XK == 0.
constexpr int XT = 128, XK = 32;

// LDS slot of 8-channel piece p of A row `row`: any 8 consecutive rows reading one piece hit
// distinct 16-byte bank groups (rows are 64 bytes, 4 pieces)
__device__ __forceinline__ int x3_slot(int row, int p) { return p ^ ((row >> 1) & 3); }

__global__ void __launch_bounds__(256, 3) lm_gemm_x3_kernel(const float* __restrict__ A, const uint16_t* __restrict__ Bh,
                                                         const uint16_t* __restrict__ Bl, float* __restrict__ C,
                                                         int M, int N, int K, int pw, int64_t ps) {
    __shared__ __align__(16) uint4 AH[XT][XK / 8];      // [row][slot]
    __shared__ __align__(16) uint4 AL[XT][XK / 8];
    __shared__ __align__(16) uint4 SH[XT][XK / 8 + 1];  // [column][8-channel piece], padded
    __shared__ __align__(16) uint4 SL[XT][XK / 8 + 1];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w & 1, wn = w >> 1, hf = lane >> 5;
    const int nx = (N + XT - 1) / XT, loc = blockIdx.x >> 3, rt = (blockIdx.x & 7) + 8 * (loc / nx);
    if ((int64_t)rt * XT >= M) return;
    const int64_t m0 = (int64_t)rt * XT, n0 = (int64_t)(loc % nx) * XT;
    hf32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = hf32x16{};
    // staging roles: A rows (threadIdx >> 3) + 32 u, channels 4 aq + [0, 4) of the chunk;
    // B units f = threadIdx + 256 u: column f / 4, piece f % 4
    constexpr int AU = XT * XK / 4 / 256, BU = XT * (XK / 8) / 256;
    const int aq = threadIdx.x & 7;
    const float* asrc[AU];
#pragma unroll
    for (int u = 0; u < AU; ++u) {
        const int64_t r = min(m0 + (threadIdx.x >> 3) + 32 * u, (int64_t)M - 1);
        asrc[u] = A + r * K + 4 * aq;
    }
    float4 ar[AU];
    uint4 bhr[BU], blr[BU];
    auto load = [&](int k0) {
#pragma unroll
        for (int u = 0; u < AU; ++u) ar[u] = *reinterpret_cast<const float4*>(asrc[u] + k0);
#pragma unroll
        for (int u = 0; u < BU; ++u) {
            const int f = threadIdx.x + 256 * u;
            const int64_t n = n0 + f / (XK / 8);
            bhr[u] = blr[u] = make_uint4(0u, 0u, 0u, 0u);
            if (n < N) {
                bhr[u] = *reinterpret_cast<const uint4*>(Bh + n * K + k0 + 8 * (f % (XK / 8)));
                blr[u] = *reinterpret_cast<const uint4*>(Bl + n * K + k0 + 8 * (f % (XK / 8)));
            }
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int u = 0; u < AU; ++u) {
            const int row = (threadIdx.x >> 3) + 32 * u;
            const float x[4] = {ar[u].x, ar[u].y, ar[u].z, ar[u].w};
            const uint32_t h0 = bf16_pair(x[0], x[1]), h1 = bf16_pair(x[2], x[3]);
            const uint32_t l0 = bf16_pair(x[0] - __uint_as_float(h0 << 16), x[1] - __uint_as_float(h0 & 0xFFFF0000u));
            const uint32_t l1 = bf16_pair(x[2] - __uint_as_float(h1 << 16), x[3] - __uint_as_float(h1 & 0xFFFF0000u));
            const int sl = x3_slot(row, aq >> 1), half = aq & 1;
            reinterpret_cast<uint2*>(&AH[row][sl])[half] = make_uint2(h0, h1);
            reinterpret_cast<uint2*>(&AL[row][sl])[half] = make_uint2(l0, l1);
        }
#pragma unroll
        for (int u = 0; u < BU; ++u) {
            const int f = threadIdx.x + 256 * u;
            SH[f / (XK / 8)][f % (XK / 8)] = bhr[u];
            SL[f / (XK / 8)][f % (XK / 8)] = blr[u];
        }
    };
    load(0);
    store();
    __syncthreads();
    for (int k0 = 0; k0 < K; k0 += XK) {
        const bool more = k0 + XK < K;
        if (more) load(k0 + XK);  // in flight during this chunk's MFMAs
#pragma unroll
        for (int ks = 0; ks < XK / 16; ++ks) {
            uint4 ah[2], al[2], bh[2], bl[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = 64 * wm + 32 * i + (lane & 31), sl = x3_slot(row, 2 * ks + hf);
                ah[i] = AH[row][sl];
                al[i] = AL[row][sl];
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = 64 * wn + 32 * j + (lane & 31);
                bh[j] = SH[col][2 * ks + hf];
                bl[j] = SL[col][2 * ks + hf];
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    acc[i][j] = mfma_bf16(al[i], bh[j], acc[i][j]);
                    acc[i][j] = mfma_bf16(ah[i], bl[j], acc[i][j]);
                    acc[i][j] = mfma_bf16(ah[i], bh[j], acc[i][j]);
                }
        }
        if (more) {
            __syncthreads();  // this chunk's parts are used up
            store();
            __syncthreads();
        }
    }
    // D[row][col]: lane holds column lane & 31 and rows (r & 3) + 8 (r >> 2) + 4 hf; column
    // col goes to plane col / pw (planes of [M, pw], ps floats apart), column col % pw
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int col = (int)n0 + 64 * wn + 32 * j + (lane & 31);
        if (col >= N) continue;
        float* cp = C + (col / pw) * ps + col % pw;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + 64 * wm + 32 * i + (r & 3) + 8 * (r >> 2) + 4 * hf;
                if (row < M) cp[row * pw] = acc[i][j][r];
            }
    }
}

unsigned blocks(int64_t n, int per = 256) { return (unsigned)((n + per - 1) / per); }

}  // namespace

// ---- launchers (arguments validated by the caller) ------------------------------
hipError_t lm_gemm_nt(const float* A, const float* B, float* C, int64_t M, int64_t N, int64_t K, const float* alpha,
                      bool accumulate, hipStream_t s) {
    hipLaunchKernelGGL(lm_gemm_nt_kernel, dim3((unsigned)(M / GB), (unsigned)((N + GB - 1) / GB)), dim3(256), 0, s,
                       A, B, C, (int)M, (int)N, (int)K, alpha, accumulate ? 1 : 0);
    return hipGetLastError();
}

hipError_t lm_embed(const float* emb, const float* pos, const int32_t* tok, int T, int S, int d, int V, float* x,
                    hipStream_t s) {
    hipLaunchKernelGGL(lm_embed_kernel, dim3(blocks((int64_t)T * d)), dim3(256), 0, s, emb, pos, tok, T, S, d, V, x);
    return hipGetLastError();
}

hipError_t lm_layernorm(const float* x, int64_t R, int d, float eps, float* u, float* mu, float* rs, hipStream_t s) {
    hipLaunchKernelGGL(lm_layernorm_kernel, dim3(blocks(R, 4)), dim3(256), 0, s, x, (int)R, d, eps, u, mu, rs);
    return hipGetLastError();
}

hipError_t lm_attn_fwd(const float* q, const float* k, const float* v, int T, int S, int H, float* o, float* lse,
                       float* pc, hipStream_t s) {
    hipLaunchKernelGGL(lm_attn_fwd_kernel, dim3((unsigned)((T / S) * H * (S / FQ))), dim3(FQL * FQ), 0, s, q, k, v, T,
                       S, H, o, lse, pc);
    return hipGetLastError();
}

hipError_t lm_gelu(const float* h, int64_t count, float* m, float* cdf, float* pdf, hipStream_t s) {
    hipLaunchKernelGGL(lm_gelu_kernel, dim3(blocks(count)), dim3(256), 0, s, h, count, m, cdf, pdf);
    return hipGetLastError();
}

hipError_t lm_residual(const float* x, const float* b, const float* alpha, int64_t count, float* out,
                       hipStream_t s) {
    hipLaunchKernelGGL(lm_residual_kernel, dim3(blocks(count)), dim3(256), 0, s, x, b, alpha, count, out);
    return hipGetLastError();
}

hipError_t lm_ce(const float* z, const int32_t* labels, int T, int V, float* lse, float* ce, float* prob, int Vp,
                 hipStream_t s) {
    hipLaunchKernelGGL(lm_ce_kernel, dim3((unsigned)T), dim3(256), 0, s, z, labels, V, lse, ce, prob, Vp);
    return hipGetLastError();
}

hipError_t lm_noise_add(float* D, int kc, int T, int w, float sigma, uint32_t k0, uint32_t k1, uint32_t layer,
                        uint32_t draw0, hipStream_t s, bool set) {
    hipLaunchKernelGGL(lm_noise_add_kernel, dim3(blocks((int64_t)kc * T * (w / 4))), dim3(256), 0, s, D, kc, T, w,
                       sigma, k0, k1, layer, draw0, set ? 1 : 0);
    return hipGetLastError();
}

hipError_t lm_layernorm_delta(const float* x, const float* mu, const float* rs, const float* dx, int64_t R, int T,
                              int d, float* du, hipStream_t s) {
    const int64_t lanes = R * (d / 8);
    switch (d) {
        case 64:
            hipLaunchKernelGGL(lm_layernorm_delta8_kernel<8>, dim3(blocks(lanes)), dim3(256), 0, s, x, mu, rs, dx, R, T,
                               du);
            break;
        case 128:
            hipLaunchKernelGGL(lm_layernorm_delta8_kernel<16>, dim3(blocks(lanes)), dim3(256), 0, s, x, mu, rs, dx, R,
                               T, du);
            break;
        case 256:
            hipLaunchKernelGGL(lm_layernorm_delta8_kernel<32>, dim3(blocks(lanes)), dim3(256), 0, s, x, mu, rs, dx, R,
                               T, du);
            break;
        case 512:
            hipLaunchKernelGGL(lm_layernorm_delta8_kernel<64>, dim3(blocks(lanes)), dim3(256), 0, s, x, mu, rs, dx, R,
                               T, du);
            break;
        default:  // other widths: one wave per row
            hipLaunchKernelGGL(lm_layernorm_delta_kernel, dim3(blocks(R, 4)), dim3(256), 0, s, x, mu, rs, dx, (int)R,
                               T, d, du);
    }
    return hipGetLastError();
}

hipError_t lm_attn_delta(const float* q, const float* k, const float* v, const float* o, const float* pc,
                         const float* dq, const float* dk, const float* dv, int kc, int T, int S, int H, float* dout,
                         hipStream_t s) {
    hipLaunchKernelGGL(lm_attn_delta_kernel, dim3((unsigned)(kc * (T / S) * H * (S / 64))), dim3(256), 0, s, q, k, v,
                       o, pc, dq, dk, dv, T, S, H, dout);
    return hipGetLastError();
}

hipError_t lm_gelu_delta(const float* h, const float* cdf, const float* pdf, const float* dh, int64_t per_draw,
                         int64_t count, float* dm, hipStream_t s) {
    if (per_draw <= 0 || per_draw % 4 != 0 || count % per_draw != 0) return hipErrorInvalidValue;
    const int64_t kc = count / per_draw;
    if (kc == 0) return hipSuccess;
    hipLaunchKernelGGL(lm_gelu_delta_kernel, dim3(blocks(per_draw / 4), (unsigned)((kc + GDD - 1) / GDD)), dim3(256), 0,
                       s, reinterpret_cast<const float4*>(h), reinterpret_cast<const float4*>(cdf),
                       reinterpret_cast<const float4*>(pdf), reinterpret_cast<const float4*>(dh), per_draw / 4, (int)kc,
                       reinterpret_cast<float4*>(dm));
    return hipGetLastError();
}

hipError_t lm_residual_delta(float* dx, const float* db, const float* b, const float* scal, int slot, int kc,
                             int64_t per_draw, float es_sigma, uint32_t member0, uint32_t k0, uint32_t k1,
                             uint32_t es_layer, hipStream_t s) {
    hipLaunchKernelGGL(lm_residual_delta_kernel, dim3(blocks((int64_t)kc * per_draw)), dim3(256), 0, s, dx, db, b,
                       scal, slot, kc, per_draw, es_sigma, member0, k0, k1, es_layer);
    return hipGetLastError();
}

bool lm_residual_ln_fusable(int d) { return d == 64 || d == 128 || d == 256 || d == 512; }

template <int LPR>
static void launch_residual_ln(float* dx, const float* db, const float* b, const float* scal, int slot, int64_t R,
                               int T, float es_sigma, uint32_t member0, uint32_t k0, uint32_t k1, uint32_t es_layer,
                               const float* x, const float* mu, const float* rs, float* du, hipStream_t s) {
    hipLaunchKernelGGL(lm_residual_ln_delta8_kernel<LPR>, dim3(blocks(R * LPR)), dim3(256), 0, s, dx, db, b, scal,
                       slot, R, T, es_sigma, member0, k0, k1, es_layer, x, mu, rs, du);
}

hipError_t lm_residual_ln_delta(float* dx, const float* db, const float* b, const float* scal, int slot, int kc,
                                int T, int d, float es_sigma, uint32_t member0, uint32_t k0, uint32_t k1,
                                uint32_t es_layer, const float* x, const float* mu, const float* rs, float* du,
                                hipStream_t s) {
    const int64_t R = (int64_t)kc * T;
    if (R == 0) return hipSuccess;
    switch (d) {
        case 64: launch_residual_ln<8>(dx, db, b, scal, slot, R, T, es_sigma, member0, k0, k1, es_layer, x, mu, rs, du, s); break;
        case 128: launch_residual_ln<16>(dx, db, b, scal, slot, R, T, es_sigma, member0, k0, k1, es_layer, x, mu, rs, du, s); break;
        case 256: launch_residual_ln<32>(dx, db, b, scal, slot, R, T, es_sigma, member0, k0, k1, es_layer, x, mu, rs, du, s); break;
        case 512: launch_residual_ln<64>(dx, db, b, scal, slot, R, T, es_sigma, member0, k0, k1, es_layer, x, mu, rs, du, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t lm_ce_delta(const float* z, const float* lse, const float* dz, const int32_t* labels, int kc, int T, int V,
                       float* rew, hipStream_t s) {
    hipLaunchKernelGGL(lm_ce_delta_kernel, dim3((unsigned)((int64_t)kc * T)), dim3(256), 0, s, z, lse, dz, labels, T,
                       V, rew);
    return hipGetLastError();
}

hipError_t lm_ghat(const float* rew, int K, int T, int w, float scale, uint32_t k0, uint32_t k1, uint32_t layer,
                   float* ghat, hipStream_t s) {
    hipLaunchKernelGGL(lm_ghat_kernel, dim3((unsigned)((int64_t)T * ((w / 4 + 31) / 32))), dim3(256), 0, s, rew, K, T, w,
                       scale, k0, k1, layer, ghat);
    return hipGetLastError();
}

hipError_t lm_embed_grads(const float* ghat, const int32_t* tok, int T, int S, int V, int d, float* gemb, float* gpos,
                          hipStream_t s) {
    if (d > 256 * ECH) return hipErrorInvalidValue;
    hipError_t e = hipMemsetAsync(gemb, 0, (size_t)V * d * sizeof(float), s);  // rows no token names
    if (e != hipSuccess) return e;
    if (T > 0) hipLaunchKernelGGL(lm_embed_grad_kernel, dim3((unsigned)T), dim3(256), 0, s, ghat, tok, T, V, d, gemb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lm_pos_grad_kernel, dim3(blocks((int64_t)S * d)), dim3(256), 0, s, ghat, T, S, d, gpos);
    return hipGetLastError();
}

hipError_t lm_split_frag(const float* W, int64_t rows, int64_t rows_p, int K, uint16_t* hi, uint16_t* lo,
                        hipStream_t s) {
    if (K % 16 != 0 || rows_p % 32 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(lm_split_frag_kernel, dim3(blocks(rows_p * K / 8)), dim3(256), 0, s, W, rows, rows_p, K,
                       reinterpret_cast<uint4*>(hi), reinterpret_cast<uint4*>(lo));
    return hipGetLastError();
}

hipError_t lm_split(const float* W, int64_t rows, int64_t rows_p, int K, uint16_t* hi, uint16_t* lo, hipStream_t s) {
    hipLaunchKernelGGL(lm_split_kernel, dim3(blocks(rows_p * K / 2)), dim3(256), 0, s, W, rows, rows_p, K,
                       reinterpret_cast<uint32_t*>(hi), reinterpret_cast<uint32_t*>(lo));
    return hipGetLastError();
}

hipError_t lm_head_delta(const float* du, const uint16_t* whi, const uint16_t* wlo, const float* prob, int d, int kc,
                         int T, int Vp, int vseg, int nseg, float* part, hipStream_t s) {
    // W_head's parts are in fragment order over whole 32-row blocks
    if (T % 64 != 0 || Vp % 32 != 0 || vseg % 32 != 0) return hipErrorInvalidValue;
    const int64_t npairs = (int64_t)(T / 64) * nseg, ngr = (kc + HDG - 1) / HDG;
    const dim3 grid((unsigned)(8 * ngr * ((npairs + 7) / 8)));
    bool timed;
    hipError_t e = launch_timer_begin(kTimedLmHead, s, timed);
    if (e != hipSuccess) return e;
    if (d == 64)
        hipLaunchKernelGGL(lm_head_delta_kernel<4>, grid, dim3(64 * HW), 0, s, du, whi, wlo, prob, T, Vp, vseg, nseg,
                           kc, part);
    else
        hipLaunchKernelGGL(lm_head_delta_kernel<8>, grid, dim3(64 * HW), 0, s, du, whi, wlo, prob, T, Vp, vseg, nseg,
                           kc, part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_timer_end(kTimedLmHead, s, timed);
}

hipError_t lm_head_reward(const float* du, const float* whead, const int32_t* labels, const float* part, int T, int V,
                          int d, int nseg, int64_t rows, float* rew, hipStream_t s) {
    if (nseg <= 16 && (d == 64 || d == 128)) {
        if (d == 64)
            hipLaunchKernelGGL(lm_head_reward16_kernel<4>, dim3(blocks(rows, 16)), dim3(256), 0, s, du, whead, labels,
                               part, T, V, nseg, rows, rew);
        else
            hipLaunchKernelGGL(lm_head_reward16_kernel<8>, dim3(blocks(rows, 16)), dim3(256), 0, s, du, whead, labels,
                               part, T, V, nseg, rows, rew);
    } else {
        hipLaunchKernelGGL(lm_head_reward_kernel, dim3(blocks(rows, 4)), dim3(256), 0, s, du, whead, labels, part, T, V,
                           d, nseg, rows, rew);
    }
    return hipGetLastError();
}

hipError_t lm_gemm_x3(const float* A, const uint16_t* Bh, const uint16_t* Bl, float* C, int64_t M, int64_t N,
                      int64_t K, hipStream_t s, int64_t pw, int64_t ps) {
    if (pw <= 0) pw = N;
    if (N % pw != 0) return hipErrorInvalidValue;
    bool timed;
    hipError_t e = launch_timer_begin(kTimedLmGemm, s, timed);
    if (e != hipSuccess) return e;
    const int64_t nx = (N + XT - 1) / XT, ny = (M + XT - 1) / XT;
    hipLaunchKernelGGL(lm_gemm_x3_kernel, dim3((unsigned)(8 * nx * ((ny + 7) / 8))),
                       dim3(256), 0, s, A, Bh, Bl, C, (int)M, (int)N, (int)K, (int)pw, ps);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_timer_end(kTimedLmGemm, s, timed);
}

hipError_t lm_transpose(const float* W, int R, int C, float* WT, hipStream_t s) {
    hipLaunchKernelGGL(lm_transpose_kernel, dim3(blocks((int64_t)R * C)), dim3(256), 0, s, W, R, C, WT);
    return hipGetLastError();
}

hipError_t lm_member_losses(const float* rew, int members, int T, float* dL, hipStream_t s) {
    hipLaunchKernelGGL(lm_rowsum_neg_kernel, dim3((unsigned)members), dim3(256), 0, s, rew, T, dL);
    return hipGetLastError();
}

hipError_t lm_es_grad(const float* dL, int M, int nsc, float scale, uint32_t k0, uint32_t k1, uint32_t es_layer,
                      float* g, hipStream_t s) {
    hipLaunchKernelGGL(lm_es_grad_kernel, dim3(1), dim3(64), 0, s, dL, M, nsc, scale, k0, k1, es_layer, g);
    return hipGetLastError();
}

hipError_t lm_sgd(float* theta, float* mom, const float* G, int64_t count, int64_t scal0, float lr, float lr_scalar,
                  float mu, hipStream_t s) {
    hipLaunchKernelGGL(lm_sgd_kernel, dim3(blocks(count)), dim3(256), 0, s, theta, mom, G, count, scal0, lr,
                       lr_scalar, mu);
    return hipGetLastError();
}

}  // namespace dust
