// Attention internals: the value-projection estimator.
//
// Method (TL;DR page "Dust: zeroth-order Transformer pretraining without
// backprop", section 1, "credit assignment without backprop": attention
// internals are rewarded by the change of the attention output instead of the
// token's loss; news article, mechanism paragraph: that change is judged
// against the error signal; iitog.ru page, mechanics paragraph: the error at
// the attention output over the current and future tokens).  Reading: with
// e_s the error at the attention output of token s and every token's value
// v_t perturbed by sigma a_t in the same draw,
//     r_t = -sum_{s >= t, same sequence} <e_s, o'_s - o_s>,
//     g_hat_t = -(1/(K sigma)) sum_i r_t^(i) a_t^(i),   G_WV = sum_t g_hat_t u_t^T.
// Only the values move, so o'_s - o_s = sigma sum_{t <= s} P_st a_t exactly,
// P the clean causal attention probabilities, and per head
//     c_s = <e_s, o'_s - o_s> = sigma sum_{t <= s} P_st <e_s, a_t>,
// no difference of two outputs is formed (no cancellation).
//
// Kernels (heads of 64 channels, sequences of whole 64-token tiles):
//   attn_stats_kernel per (sequence, head, query tile): log-sum-exp of the
//                     clean scaled logits of each query (and <e, o>);
//   attn_v_kernel     per (sequence, head, key tile) and chunk of 8 draws: the
//                     key tile's noise for the chunk is generated once into LDS; for every
//                     query tile at or after it the transposed logits
//                     K Q^T / sqrt(64) are recomputed, P = exp(L - lse), and
//                     per draw G^T = A E^T on MFMA, then per query the column
//                     sum of P (.) G^T: the partial c of this key tile;
//   attn_k_kernel, attn_q_kernel: the same for keys and queries (two sums);
//   attn_csum(_k)_kernel per (draw, token): c_s from the partials;
//   attn_suffix_scan_kernel per (draw, sequence): r_t = -sigma sum_{s >= t} c_s
//                     by a reverse block scan;
//   attn_reduce_kernel per token: g_hat from the rewards, noise regenerated.
// Products of two fp32 operands run on bf16 MFMA with both operands split into
// pairs v = hi + lo and the three products lo.hi + hi.lo + hi.hi accumulated in
// fp32 (each within about 3 2^-17 of fp32).
#include <algorithm>

#include "dust_device.hpp"
#include "dust_internal.hpp"
#include "launch_events.hpp"

namespace dust {

namespace {
typedef __bf16 abf16x2_t __attribute__((ext_vector_type(2)));
typedef float af32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 abf16x8_t __attribute__((ext_vector_type(8)));
typedef float af32x16_t __attribute__((ext_vector_type(16)));

constexpr int AT = 64;    // tokens per query / key tile
constexpr int ADH = 64;   // channels per head
constexpr int ANT = 256;  // lanes of the statistics pass: 4 waves of 32 keys x 32 queries
constexpr int VNT = 512;  // lanes of the main pass: two groups of 4 waves on alternate query tiles
constexpr int ADC = 8;    // draws whose key-tile noise sits in LDS at once
constexpr int ASMAX = 4096;  // longest sequence
constexpr float kAL2e = kLog2eF;

__device__ __forceinline__ uint32_t pack2(float a, float b) {  // two floats -> bf16 pair (RNE), a low
    const af32x2_t v = {a, b};
    const abf16x2_t h = __builtin_convertvector(v, abf16x2_t);
    uint32_t u;
    __builtin_memcpy(&u, &h, 4);
    return u;
}

// 8 consecutive fp32 values as bf16 hi and lo parts (x = hi + lo + O(2^-17 |x|)).
__device__ __forceinline__ void split8(const float4& x0, const float4& x1, uint4& hi, uint4& lo) {
    const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        h[p] = pack2(x[2 * p], x[2 * p + 1]);
        l[p] = pack2(x[2 * p] - __uint_as_float(h[p] << 16), x[2 * p + 1] - __uint_as_float(h[p] & 0xFFFF0000u));
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
}

__device__ __forceinline__ af32x16_t mfma(const uint4& a, const uint4& b, const af32x16_t& c) {
    abf16x8_t av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
}

// Fragments of one 32-row x 64-channel block of a row-major fp32 matrix: lane l
// holds row (l & 31), channels 16 ks + 8 (l >> 5) + [0, 8) for ks = 0..3.
__device__ __forceinline__ void load_frags(const float* __restrict__ M, int64_t ld, int64_t row, int ch0,
                                           uint4 (&hi)[4], uint4 (&lo)[4]) {
    const int lane = threadIdx.x & 63;
    const float* p = M + row * ld + ch0 + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const float4 a = *reinterpret_cast<const float4*>(p + 16 * ks);
        const float4 b = *reinterpret_cast<const float4*>(p + 16 * ks + 4);
        split8(a, b, hi[ks], lo[ks]);
    }
}

// 32 x 32 block of A B^T over 64 channels from split fragments (three products).
__device__ __forceinline__ af32x16_t prod_x3(const uint4 (&ahi)[4], const uint4 (&alo)[4], const uint4 (&bhi)[4],
                                             const uint4 (&blo)[4]) {
    af32x16_t acc = {};
    af32x16_t acc2 = {};  // two chains, so no MFMA waits on the one just issued
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        acc = mfma(alo[ks], bhi[ks], acc);
        acc2 = mfma(ahi[ks], blo[ks], acc2);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma(ahi[ks], bhi[ks], acc);
    return acc + acc2;
}

// Row of the D layout (the A operand's row) held by register r of a lane.
__device__ __forceinline__ int drow(int r, int lane) { return (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5); }

// LDS layout of a 64-key x 64-channel bf16 tile: row = key, 8 pieces of 8
// channels, piece p of row r at p ^ ((r >> 1) & 7) (fragment reads of 16
// consecutive rows touch all banks once).
__device__ __forceinline__ int aswz(int row, int piece) { return row * 64 + ((piece ^ ((row >> 1) & 7)) << 3); }
}  // namespace

struct AttnKArgs {
    const float* q;  // [T,d]
    const float* k;  // [T,d]
    const float* v;  // [T,d] (query and key projections only)
    const float* e;  // [T,d] error at the attention output
    float* ob;       // [T,H] <e_s, o_s> per head (query and key projections only)
    float sdelta;    // sigma / sqrt(dh): the logit change per unit of <a, q> or <k, a>
    float* lse2;     // [T,H] log2-sum-exp2 of the clean scaled logits (log2 e / sqrt(dh) q.k)
    float* cpart;    // [KC][nkt][H][2][T] partial c per (draw, key tile, head, key half, query)
    int dper;        // draws per workgroup along y (a multiple of ADC): workgroup y takes [y dper, (y+1) dper)
    int T, S, d, H;
    uint32_t k0, k1, layer, tok0, draw0;
};

// expm1(s D) for the 16 logit-change inputs D of a lane, x = s D.  The common
// case is the degree-4 Taylor polynomial with s folded into its coefficients
// (s, s^2/2, s^3/6, s^4/24: four operations per value, no separate product s D;
// truncation below 1.3e-7 relative for |x| < 1/16).  Only in a wave where some
// lane holds |D| >= dlim = (1/16)/s do those values take the degree-6 polynomial
// (truncation below 5e-8 relative for |x| < 1/4) or, beyond, exp(x) - 1, where
// no cancellation arises.  At sigma = 1e-2 logit changes are about 1e-2, so that
// branch practically never runs; the degree-6 form for every value had cost
// a third more vector instructions per draw.
struct Expm1Coef {
    float c1, c2, c3, c4, dlim;
};

__host__ __device__ inline Expm1Coef expm1_coef(float s) {
    Expm1Coef c;
    c.c1 = s;
    c.c2 = s * s * 0.5f;
    c.c3 = s * s * s * (1.0f / 6.0f);
    c.c4 = s * s * s * s * (1.0f / 24.0f);
    c.dlim = s > 0.f ? 0.0625f / s : __builtin_huge_valf();
    return c;
}

__device__ __forceinline__ void expm1_16s(float (&D)[16], const Expm1Coef& cf) {
    bool big = false;
#pragma unroll
    for (int r = 0; r < 16; ++r) big |= fabsf(D[r]) >= cf.dlim;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = D[r] * fmaf(D[r], fmaf(D[r], fmaf(D[r], cf.c4, cf.c3), cf.c2), cf.c1);
    if (__builtin_amdgcn_ballot_w64(big)) {  // wave-uniform, rare at small sigma
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float x = D[r] * cf.c1;
            const float q6 = x * fmaf(x, fmaf(x, fmaf(x, fmaf(x, fmaf(x, 1.0f / 720.0f, 1.0f / 120.0f), 1.0f / 24.0f),
                                                      1.0f / 6.0f), 0.5f), 1.0f);
            const float alt = fabsf(x) < 0.25f ? q6 : __expf(x) - 1.0f;
            p[r] = fabsf(D[r]) >= cf.dlim ? alt : p[r];
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) D[r] = p[r];
}

// ---- clean statistics -------------------------------------------------------
// Per (sequence, head, query tile): log2-sum-exp2 of the scaled logits and, with
// OB, <e_s, o_s> = sum_t P_st <v_t, e_s> (needed by the query and key projections).
template <bool OB>
__global__ void __launch_bounds__(ANT) attn_stats_kernel(AttnKArgs A) {
    __shared__ float4 sh[2][AT];
    const int nqt = A.S / AT;
    const int qt = blockIdx.x % nqt, bh = blockIdx.x / nqt, b = bh / A.H, h = bh % A.H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, kh = w >> 1, qh = w & 1;
    const int64_t s0 = (int64_t)b * A.S;  // first token of the sequence
    const float sl2 = kAL2e * 0.125f;     // log2 e / sqrt(64)
    uint4 qhi[4], qlo[4], ehi[4], elo[4];
    load_frags(A.q, A.d, s0 + qt * AT + qh * 32 + (lane & 31), h * ADH, qhi, qlo);
    if (OB) load_frags(A.e, A.d, s0 + qt * AT + qh * 32 + (lane & 31), h * ADH, ehi, elo);
    const int query = qt * AT + qh * 32 + (lane & 31);
    float m = -__builtin_inff(), s = 0.f, o = 0.f;
    for (int kt = 0; kt <= qt; ++kt) {
        uint4 khi[4], klo[4];
        load_frags(A.k, A.d, s0 + kt * AT + kh * 32 + (lane & 31), h * ADH, khi, klo);
        const af32x16_t L = prod_x3(khi, klo, qhi, qlo);  // [key][query]
        af32x16_t W = {};
        if (OB) {
            uint4 vhi[4], vlo[4];
            load_frags(A.v, A.d, s0 + kt * AT + kh * 32 + (lane & 31), h * ADH, vhi, vlo);
            W = prod_x3(vhi, vlo, ehi, elo);  // [key][query]: <v_key, e_query>
        }
        float x[16];
        float mt = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kt * AT + kh * 32 + drow(r, lane);
            x[r] = key <= query ? L[r] * sl2 : -__builtin_inff();
            mt = fmaxf(mt, x[r]);
        }
        const float mn = fmaxf(m, mt);
        if (mn == -__builtin_inff()) continue;  // every key of this lane so far lies after its query
        float st = 0.f, ot = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pr = __builtin_amdgcn_exp2f(x[r] - mn);
            st += pr;
            if (OB) ot = fmaf(pr, W[r], ot);
        }
        const float f = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - mn);
        s = s * f + st;
        o = o * f + ot;
        m = mn;
    }
    // merge the two lanes of a query (lane, lane ^ 32), then the two key halves
    const float mo = __shfl_xor(m, 32, 64), so = __shfl_xor(s, 32, 64), oo = __shfl_xor(o, 32, 64);
    const float mm = fmaxf(m, mo);
    const float f0 = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - mm);
    const float f1 = mo == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mo - mm);
    if (lane < 32) sh[kh][qh * 32 + lane] = make_float4(mm, s * f0 + so * f1, o * f0 + oo * f1, 0.f);
    __syncthreads();
    if (tid < AT) {
        const float4 p0 = sh[0][tid], p1 = sh[1][tid];
        const float M = fmaxf(p0.x, p1.x);
        const float g0 = p0.y > 0.f ? __builtin_amdgcn_exp2f(p0.x - M) : 0.f;
        const float g1 = p1.y > 0.f ? __builtin_amdgcn_exp2f(p1.x - M) : 0.f;
        const float S2 = p0.y * g0 + p1.y * g1;
        const int64_t tok = s0 + qt * AT + tid;
        A.lse2[tok * A.H + h] = M + __builtin_amdgcn_logf(S2);  // log2 of sum exp2
        if (OB) A.ob[tok * A.H + h] = (p0.z * g0 + p1.z * g1) / S2;
    }
}

// Noise of 64 tokens (rows) x the 64 channels of head h for one draw, as bf16
// hi/lo parts in the swizzled LDS layout; NTH lanes, 1024 / NTH quads each.
template <int NTH>
__device__ __forceinline__ void gen_tile(uint16_t* nh, uint16_t* nl, uint32_t tok_row0, int h, uint32_t draw,
                                         const AttnKArgs& A) {
#pragma unroll
    for (int j = 0; j < 1024 / NTH; ++j) {
        const int qi = (int)threadIdx.x + j * NTH;
        const int row = qi >> 4, cq = qi & 15;  // channel quad within the head
        const f32x4 g = gauss4(tok_row0 + (uint32_t)row, (uint32_t)(h * (ADH / 4) + cq), draw, A.layer, A.k0, A.k1);
        const uint32_t h0 = pack2(g.v[0], g.v[1]), h1 = pack2(g.v[2], g.v[3]);
        const uint32_t l0 = pack2(g.v[0] - __uint_as_float(h0 << 16), g.v[1] - __uint_as_float(h0 & 0xFFFF0000u));
        const uint32_t l1 = pack2(g.v[2] - __uint_as_float(h1 << 16), g.v[3] - __uint_as_float(h1 & 0xFFFF0000u));
        const int off = aswz(row, cq >> 1) + 4 * (cq & 1);
        *reinterpret_cast<uint2*>(nh + off) = make_uint2(h0, h1);
        *reinterpret_cast<uint2*>(nl + off) = make_uint2(l0, l1);
    }
}

__device__ __forceinline__ void read_tile_frags(const uint16_t* nh, const uint16_t* nl, int row, uint4 (&hi)[4],
                                                uint4 (&lo)[4]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int off = aswz(row, 2 * ks + (lane >> 5));
        hi[ks] = *reinterpret_cast<const uint4*>(nh + off);
        lo[ks] = *reinterpret_cast<const uint4*>(nl + off);
    }
}

// One accumulator chain of the three products A B^T (hi/lo pairs).
__device__ __forceinline__ af32x16_t prod_x3c(const uint4 (&ahi)[4], const uint4 (&alo)[4], const uint4 (&bhi)[4],
                                              const uint4 (&blo)[4]) {
    af32x16_t g = {};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) g = mfma(alo[ks], bhi[ks], g);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) g = mfma(ahi[ks], blo[ks], g);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) g = mfma(ahi[ks], bhi[ks], g);
    return g;
}

// ---- per-draw partial output changes ------------------------------------------
__global__ void __launch_bounds__(VNT, 1) attn_v_kernel(AttnKArgs A, int i0, int kc) {
    __shared__ __align__(16) uint16_t NH[ADC][AT * ADH];  // noise tile, bf16 hi parts
    __shared__ __align__(16) uint16_t NL[ADC][AT * ADH];  // and lo parts
    const int nqt = A.S / AT, nbh = (A.T / A.S) * A.H;
    // key tiles with the most query tiles after them first
    const int kt = blockIdx.x / nbh, bh = blockIdx.x % nbh, b = bh / A.H, h = bh % A.H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, kh = (w >> 1) & 1, qh = w & 1, grp = w >> 2;
    const int64_t s0 = (int64_t)b * A.S;
    const int nkt = nqt;
    const float sl2 = kAL2e * 0.125f;
    uint4 khi[4], klo[4];  // this wave's 32 keys
    load_frags(A.k, A.d, s0 + kt * AT + kh * 32 + (lane & 31), h * ADH, khi, klo);

    for (int d0 = (int)blockIdx.y * A.dper; d0 < kc && d0 < ((int)blockIdx.y + 1) * A.dper; d0 += ADC) {
        const int dn = min(ADC, kc - d0);
        __syncthreads();  // the previous chunk's noise fully used
        // noise of the 64 keys x 64 channels for dn draws: 1024 quads per draw
        for (int dd = 0; dd < dn; ++dd) {
            const uint32_t draw = A.draw0 + (uint32_t)(i0 + d0 + dd);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int qi = tid + j * VNT;
                const int key = qi >> 4, cq = qi & 15;  // channel quad within the head
                const uint32_t tok = A.tok0 + (uint32_t)(s0 + kt * AT + key);
                const f32x4 g = gauss4(tok, (uint32_t)(h * (ADH / 4) + cq), draw, A.layer, A.k0, A.k1);
                const uint32_t h0 = pack2(g.v[0], g.v[1]), h1 = pack2(g.v[2], g.v[3]);
                const uint32_t l0 = pack2(g.v[0] - __uint_as_float(h0 << 16), g.v[1] - __uint_as_float(h0 & 0xFFFF0000u));
                const uint32_t l1 = pack2(g.v[2] - __uint_as_float(h1 << 16), g.v[3] - __uint_as_float(h1 & 0xFFFF0000u));
                const int off = aswz(key, cq >> 1) + 4 * (cq & 1);
                *reinterpret_cast<uint2*>(&NH[dd][off]) = make_uint2(h0, h1);
                *reinterpret_cast<uint2*>(&NL[dd][off]) = make_uint2(l0, l1);
            }
        }
        __syncthreads();
        // query tiles kt + grp, kt + grp + 2, ...: the two wave groups share the
        // noise tile and run without barriers
        for (int qt = kt + grp; qt < nqt; qt += 2) {
            const int64_t qrow = s0 + qt * AT + qh * 32 + (lane & 31);
            const int query = qt * AT + qh * 32 + (lane & 31);
            uint4 qhi[4], qlo[4], ehi[4], elo[4];
            load_frags(A.q, A.d, qrow, h * ADH, qhi, qlo);
            load_frags(A.e, A.d, qrow, h * ADH, ehi, elo);
            const float l2q = A.lse2[qrow * A.H + h];
            const af32x16_t L = prod_x3(khi, klo, qhi, qlo);  // [key][query]
            float P[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kt * AT + kh * 32 + drow(r, lane);
                P[r] = key <= query ? __builtin_amdgcn_exp2f(fmaf(L[r], sl2, -l2q)) : 0.f;
            }
            float cacc[ADC];
#pragma unroll
            for (int dd = 0; dd < ADC; ++dd) {
                if (dd < dn) {
                    uint4 ahi[4], alo[4];
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const int off = aswz(kh * 32 + (lane & 31), 2 * ks + (lane >> 5));
                        ahi[ks] = *reinterpret_cast<const uint4*>(&NH[dd][off]);
                        alo[ks] = *reinterpret_cast<const uint4*>(&NL[dd][off]);
                    }
                    af32x16_t g = {};  // [key][query]: <a_key, e_query>, one accumulator chain
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) g = mfma(alo[ks], ehi[ks], g);
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) g = mfma(ahi[ks], elo[ks], g);
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) g = mfma(ahi[ks], ehi[ks], g);
                    float c = 0.f;
#pragma unroll
                    for (int r = 0; r < 16; ++r) c = fmaf(P[r], g[r], c);
                    cacc[dd] = c;
                }
            }
            // the two lanes of a query (lane, lane ^ 32) hold the two halves of its 32 keys
#pragma unroll
            for (int dd = 0; dd < ADC; ++dd)
                if (dd < dn) cacc[dd] += __shfl_xor(cacc[dd], 32, 64);
            if (lane < 32) {
#pragma unroll
                for (int dd = 0; dd < ADC; ++dd)
                    if (dd < dn)
                        A.cpart[((((int64_t)(d0 + dd) * nkt + kt) * A.H + h) * 2 + kh) * A.T + s0 + qt * AT +
                                qh * 32 + lane] = cacc[dd];
            }
        }
    }
}

// ---- key projection: per-draw partial sums of the softmax change ---------------
// With k'_t = k_t + sigma a_t, the logit of (s, t) moves by delta_st = sigma
// <q_s, a_t> / 8 (times log2 e for exp2) and, per head,
//     o'_s - o_s = sum_t (P'_st - P_st) v_t,  P'_st = P_st e^delta_st / (1 + rho_s),
//     rho_s = sum_t P_st expm1(delta_st),
// so c_s = <e_s, o'_s - o_s> = (mu_s - rho_s <e_s, o_s>) / (1 + rho_s) with
// mu_s = sum_t P_st expm1(delta_st) <v_t, e_s>: two sums over the keys, formed
// per key tile (partials rho, mu) like the value projection's c.
__global__ void __launch_bounds__(VNT, 1) attn_k_kernel(AttnKArgs A, int kc) {
    __shared__ __align__(16) uint16_t NH[ADC][AT * ADH];
    __shared__ __align__(16) uint16_t NL[ADC][AT * ADH];
    const int nqt = A.S / AT, nbh = (A.T / A.S) * A.H;
    const int kt = blockIdx.x / nbh, bh = blockIdx.x % nbh, b = bh / A.H, h = bh % A.H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, kh = (w >> 1) & 1, qh = w & 1, grp = w >> 2;
    const int64_t s0 = (int64_t)b * A.S;
    const int nkt = nqt;
    const float sl2 = kAL2e * 0.125f;
    const Expm1Coef cf = expm1_coef(A.sdelta);
    uint4 khi[4], klo[4], vhi[4], vlo[4];  // this wave's 32 keys
    load_frags(A.k, A.d, s0 + kt * AT + kh * 32 + (lane & 31), h * ADH, khi, klo);
    load_frags(A.v, A.d, s0 + kt * AT + kh * 32 + (lane & 31), h * ADH, vhi, vlo);
    for (int d0 = (int)blockIdx.y * A.dper; d0 < kc && d0 < ((int)blockIdx.y + 1) * A.dper; d0 += ADC) {
        const int dn = min(ADC, kc - d0);
        __syncthreads();  // the previous chunk's noise fully used
        for (int dd = 0; dd < dn; ++dd)
            gen_tile<VNT>(NH[dd], NL[dd], A.tok0 + (uint32_t)(s0 + kt * AT), h, A.draw0 + (uint32_t)(d0 + dd), A);
        __syncthreads();
        for (int qt = kt + grp; qt < nqt; qt += 2) {
            const int64_t qrow = s0 + qt * AT + qh * 32 + (lane & 31);
            const int query = qt * AT + qh * 32 + (lane & 31);
            uint4 qhi[4], qlo[4];
            load_frags(A.q, A.d, qrow, h * ADH, qhi, qlo);
            float P[16], PW[16];
            {
                uint4 ehi[4], elo[4];
                load_frags(A.e, A.d, qrow, h * ADH, ehi, elo);
                const float l2q = A.lse2[qrow * A.H + h];
                const af32x16_t L = prod_x3c(khi, klo, qhi, qlo);  // [key][query]
                const af32x16_t W = prod_x3c(vhi, vlo, ehi, elo);  // [key][query]: <v_key, e_query>
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kt * AT + kh * 32 + drow(r, lane);
                    P[r] = key <= query ? __builtin_amdgcn_exp2f(fmaf(L[r], sl2, -l2q)) : 0.f;
                    PW[r] = P[r] * W[r];
                }
            }
            float rho[ADC], mu[ADC];
#pragma unroll
            for (int dd = 0; dd < ADC; ++dd) {
                if (dd < dn) {
                    uint4 ahi[4], alo[4];
                    read_tile_frags(NH[dd], NL[dd], kh * 32 + (lane & 31), ahi, alo);
                    const af32x16_t D = prod_x3c(ahi, alo, qhi, qlo);  // [key][query]: <a_key, q_query>
                    float x[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) x[r] = D[r];
                    expm1_16s(x, cf);
                    float rr = 0.f, mm = 0.f;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        rr = fmaf(P[r], x[r], rr);
                        mm = fmaf(PW[r], x[r], mm);
                    }
                    rho[dd] = rr;
                    mu[dd] = mm;
                }
            }
#pragma unroll
            for (int dd = 0; dd < ADC; ++dd)
                if (dd < dn) {
                    rho[dd] += __shfl_xor(rho[dd], 32, 64);
                    mu[dd] += __shfl_xor(mu[dd], 32, 64);
                }
            if (lane < 32) {
#pragma unroll
                for (int dd = 0; dd < ADC; ++dd)
                    if (dd < dn) {
                        float* pp = A.cpart + (((((int64_t)(d0 + dd) * nkt + kt) * A.H + h) * 2 + kh) * 2) * A.T +
                                    s0 + qt * AT + qh * 32 + lane;
                        pp[0] = rho[dd];
                        pp[A.T] = mu[dd];
                    }
            }
        }
    }
}

// ---- query projection: every sum stays in one workgroup ----------------------------
// With q'_s = q_s + sigma a_s only the row of query s moves: delta_st = sigma
// <a_s, k_t> / 8, and c_s = (mu_s - rho_s <e_s, o_s>) / (1 + rho_s) as for the keys,
// the sums over the keys of query s, all in the query tile's workgroup: two wave
// groups on alternate key tiles, merged through LDS at the end.  The reward is the
// current token's own, r_s = -c_s, summed over the heads (per-head values go to
// the partial buffer [draw][head][token]).
__global__ void __launch_bounds__(VNT, 1) attn_q_kernel(AttnKArgs A, int kc) {
    __shared__ __align__(16) uint16_t NH[ADC][AT * ADH];
    __shared__ __align__(16) uint16_t NL[ADC][AT * ADH];
    __shared__ float2 red[4][ADC][32 * 2];  // [group, key half][draw][query of the half * 2 + half]
    const int nqt = A.S / AT, nbh = (A.T / A.S) * A.H;
    // query tiles with the most key tiles first
    const int qt = nqt - 1 - blockIdx.x / nbh, bh = blockIdx.x % nbh, b = bh / A.H, h = bh % A.H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, kh = (w >> 1) & 1, qh = w & 1, grp = w >> 2;
    const int64_t s0 = (int64_t)b * A.S;
    const float sl2 = kAL2e * 0.125f;
    const Expm1Coef cf = expm1_coef(A.sdelta);
    const int64_t qrow = s0 + qt * AT + qh * 32 + (lane & 31);
    const int query = qt * AT + qh * 32 + (lane & 31);
    uint4 qhi[4], qlo[4], ehi[4], elo[4];  // this wave's 32 queries
    load_frags(A.q, A.d, qrow, h * ADH, qhi, qlo);
    load_frags(A.e, A.d, qrow, h * ADH, ehi, elo);
    const float l2q = A.lse2[qrow * A.H + h];
    for (int d0 = (int)blockIdx.y * A.dper; d0 < kc && d0 < ((int)blockIdx.y + 1) * A.dper; d0 += ADC) {
        const int dn = min(ADC, kc - d0);
        __syncthreads();  // the previous chunk's noise and sums fully used
        for (int dd = 0; dd < dn; ++dd)
            gen_tile<VNT>(NH[dd], NL[dd], A.tok0 + (uint32_t)(s0 + qt * AT), h, A.draw0 + (uint32_t)(d0 + dd), A);
        __syncthreads();
        float rho[ADC], mu[ADC];
#pragma unroll
        for (int dd = 0; dd < ADC; ++dd) rho[dd] = mu[dd] = 0.f;
        for (int kt = grp; kt <= qt; kt += 2) {
            uint4 khi[4], klo[4], vhi[4], vlo[4];
            load_frags(A.k, A.d, s0 + kt * AT + kh * 32 + (lane & 31), h * ADH, khi, klo);
            load_frags(A.v, A.d, s0 + kt * AT + kh * 32 + (lane & 31), h * ADH, vhi, vlo);
            const af32x16_t L = prod_x3c(khi, klo, qhi, qlo);  // [key][query]
            const af32x16_t W = prod_x3c(vhi, vlo, ehi, elo);  // [key][query]: <v_key, e_query>
            float P[16], PW[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kt * AT + kh * 32 + drow(r, lane);
                P[r] = key <= query ? __builtin_amdgcn_exp2f(fmaf(L[r], sl2, -l2q)) : 0.f;
                PW[r] = P[r] * W[r];
            }
#pragma unroll
            for (int dd = 0; dd < ADC; ++dd) {
                if (dd < dn) {
                    uint4 ahi[4], alo[4];  // this wave's queries' noise
                    read_tile_frags(NH[dd], NL[dd], qh * 32 + (lane & 31), ahi, alo);
                    const af32x16_t D = prod_x3c(khi, klo, ahi, alo);  // [key][query]: <k_key, a_query>
                    float x[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) x[r] = D[r];
                    expm1_16s(x, cf);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        rho[dd] = fmaf(P[r], x[r], rho[dd]);
                        mu[dd] = fmaf(PW[r], x[r], mu[dd]);
                    }
                }
            }
        }
#pragma unroll
        for (int dd = 0; dd < ADC; ++dd)
            if (dd < dn) {
                rho[dd] += __shfl_xor(rho[dd], 32, 64);
                mu[dd] += __shfl_xor(mu[dd], 32, 64);
            }
        if (lane < 32) {
#pragma unroll
            for (int dd = 0; dd < ADC; ++dd)
                if (dd < dn) red[grp * 2 + kh][dd][lane * 2 + qh] = make_float2(rho[dd], mu[dd]);
        }
        __syncthreads();
        for (int x = tid; x < dn * AT; x += VNT) {
            const int dd = x / AT, qq = x % AT;  // query qq of the tile
            const int slot = (qq & 31) * 2 + (qq >> 5);
            float rr = 0.f, mm = 0.f;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                rr += red[g4][dd][slot].x;
                mm += red[g4][dd][slot].y;
            }
            const int64_t tok = s0 + qt * AT + qq;
            const float c = (mm - rr * A.ob[tok * A.H + h]) / (1.0f + rr);
            A.cpart[((int64_t)(d0 + dd) * A.H + h) * A.T + tok] = -c;
        }
    }
}

// ---- key projection: c_t from the partial sums (one thread per draw and token) -----
// c = sum over heads of (mu - rho <e, o>) / (1 + rho), rho and mu summed over the key
// tiles up to the token's own and the key halves; written to rew[(i0 + dd) T + t] for
// the suffix scan.
// One workgroup per (draw, 64 consecutive tokens), one wave per head (H <= 16):
// the lanes read consecutive tokens (coalesced), and each head's term meets the
// others in LDS, added in head order.  One thread per (draw, token) looping over
// heads and key tiles kept too few loads in flight: 75 us per 16 draws.
constexpr int kCsumMaxH = 16;
__global__ void __launch_bounds__(64 * kCsumMaxH) attn_csum_k_kernel(const float* __restrict__ cpart,
                                                                   const float* __restrict__ ob, int T, int S,
                                                                   int H, int i0, float* __restrict__ rew) {
    __shared__ float sh[kCsumMaxH][64];
    const int lane = threadIdx.x & 63, h = threadIdx.x >> 6;
    const int64_t x0 = (int64_t)blockIdx.x * 64;   // T is a multiple of 64
    const int64_t dd = x0 / T, t = x0 % T + lane;
    const int s = (int)(t % S), nkt = S / AT;      // s / AT: the same for the 64 tokens
    float rr = 0.f, mm = 0.f;
    for (int kt = 0; kt <= s / AT; ++kt)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            const float* pp = cpart + ((((dd * nkt + kt) * H + h) * 2 + kh) * 2) * T + t;
            rr += pp[0];
            mm += pp[T];
        }
    sh[h][lane] = (mm - rr * ob[t * H + h]) / (1.0f + rr);
    __syncthreads();
    if (h == 0) {
        float c = 0.f;
        for (int g = 0; g < H; ++g) c += sh[g][lane];
        rew[(i0 + dd) * T + t] = c;
    }
}

// ---- in place: rew_t = -scale sum_{s >= t, same sequence} c_s (one workgroup per
// draw and sequence) ----------------------------------------------------------------
__global__ void __launch_bounds__(256) attn_suffix_scan_kernel(float* __restrict__ rew, int T, int S, int i0,
                                                               float scale) {
    __shared__ float cs[ASMAX];
    __shared__ float sh[256];
    const int nb = T / S;
    const int dd = blockIdx.x / nb, b = blockIdx.x % nb, tid = threadIdx.x;
    const int per = (S + 255) / 256;  // consecutive tokens per lane
    float* row = rew + (int64_t)(i0 + dd) * T + (int64_t)b * S;
    for (int s = tid; s < S; s += 256) cs[s] = row[s];
    __syncthreads();
    float tot = 0.f;  // suffix sums within this lane's tokens, in place
    for (int j = per - 1; j >= 0; --j) {
        const int s = tid * per + j;
        if (s < S) {
            tot += cs[s];
            cs[s] = tot;
        }
    }
    sh[tid] = tot;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {  // inclusive suffix scan of the lane totals
        const float v = tid + off < 256 ? sh[tid + off] : 0.f;
        __syncthreads();
        sh[tid] += v;
        __syncthreads();
    }
    const float after = tid + 1 < 256 ? sh[tid + 1] : 0.f;
    for (int j = 0; j < per; ++j) {
        const int s = tid * per + j;
        if (s < S) row[s] = -scale * (cs[s] + after);
    }
}

// ---- query projection: r_t = -sum over the heads of c_t --------------------------
__global__ void __launch_bounds__(256) attn_heads_q_kernel(const float* __restrict__ cpart, int T, int H, int i0,
                                                           int kc, float* __restrict__ rew) {
    const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (x >= (int64_t)kc * T) return;
    const int64_t dd = x / T, t = x % T;
    float r = 0.f;
    for (int h = 0; h < H; ++h) r += cpart[(dd * H + h) * T + t];
    rew[(i0 + dd) * T + t] = r;
}

// ---- value projection: c_t = sum over heads, key tiles and key halves of the
// partials, written to rew[(i0 + dd) T + t] for the suffix scan.  Laid out as the
// key projection's sum: one workgroup per (draw, 64 tokens), one wave per head.
__global__ void __launch_bounds__(64 * kCsumMaxH) attn_csum_kernel(const float* __restrict__ cpart, int T, int S,
                                                                 int H, int i0, float* __restrict__ rew) {
    __shared__ float sh[kCsumMaxH][64];
    const int lane = threadIdx.x & 63, h = threadIdx.x >> 6;
    const int64_t x0 = (int64_t)blockIdx.x * 64;
    const int64_t dd = x0 / T, t = x0 % T + lane;
    const int s = (int)(t % S), nkt = S / AT;
    float c = 0.f;
    for (int kt = 0; kt <= s / AT; ++kt) {
        const float* pp = cpart + (((dd * nkt + kt) * H + h) * 2) * T + t;
        c += pp[0] + pp[T];
    }
    sh[h][lane] = c;
    __syncthreads();
    if (h == 0) {
        float tot = 0.f;
        for (int g = 0; g < H; ++g) tot += sh[g][lane];
        rew[(i0 + dd) * T + t] = tot;
    }
}

// ---- g_hat_t = -(1/(K sigma)) sum_i r_t^(i) a_t^(i) ------------------------------
// One workgroup of ART threads per token.  With fewer than ART channel quads, the draws are
// spread over G = ART / (d / 4) thread groups (group g takes draws g, g + G, ...) and the
// groups' sums are added in a fixed order through LDS.
constexpr int ART = 256;
__global__ void __launch_bounds__(ART) attn_reduce_kernel(AttnKArgs A, int K, const float* __restrict__ rew,
                                                          float gscale, float* __restrict__ ghat) {
    __shared__ float4 part[ART];
    const int t = blockIdx.x;
    const int nqd = A.d / 4;
    const uint32_t tok = A.tok0 + (uint32_t)t;
    if (nqd < ART) {
        const int G = ART / nqd, g = threadIdx.x / nqd, qd = threadIdx.x % nqd;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        if (g < G)
            for (int i = g; i < K; i += G) {
                const float r = rew[(int64_t)i * A.T + t];
                const f32x4 gg = gauss4(tok, (uint32_t)qd, A.draw0 + (uint32_t)i, A.layer, A.k0, A.k1);
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[c] = fmaf(r, gg.v[c], acc[c]);
            }
        part[threadIdx.x] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        __syncthreads();
        if (threadIdx.x < nqd) {
            float4 s4 = part[threadIdx.x];
            for (int gg = 1; gg < G; ++gg) {
                const float4 o = part[gg * nqd + threadIdx.x];
                s4.x += o.x;
                s4.y += o.y;
                s4.z += o.z;
                s4.w += o.w;
            }
            *reinterpret_cast<float4*>(ghat + (int64_t)t * A.d + 4 * threadIdx.x) =
                make_float4(s4.x * gscale, s4.y * gscale, s4.z * gscale, s4.w * gscale);
        }
        return;
    }
    for (int qd = threadIdx.x; qd < nqd; qd += ART) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < K; ++i) {
            const float r = rew[(int64_t)i * A.T + t];
            const f32x4 g = gauss4(tok, (uint32_t)qd, A.draw0 + (uint32_t)i, A.layer, A.k0, A.k1);
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = fmaf(r, g.v[c], acc[c]);
        }
        *reinterpret_cast<float4*>(ghat + (int64_t)t * A.d + 4 * qd) =
            make_float4(acc[0] * gscale, acc[1] * gscale, acc[2] * gscale, acc[3] * gscale);
    }
}

// Partial-buffer floats per draw: per (key tile, head, key half) one c (values)
// or the two sums rho, mu (keys); per head one c (queries).
static int64_t attn_part_per_draw(int proj, int64_t T, int64_t S, int64_t H) {
    const int64_t nkt = S / AT;
    return proj == 2 ? nkt * H * 2 * T : proj == 1 ? nkt * H * 4 * T : H * T;
}

// Draws per pass of the partial buffer (kept to about 256 MB).
static int attn_kc(int proj, int64_t T, int64_t S, int64_t H, int64_t K) {
    const int64_t per_draw = attn_part_per_draw(proj, T, S, H) * 4;
    int64_t kc = ((int64_t)256 << 20) / (per_draw > 0 ? per_draw : 1);
    kc = kc < 1 ? 1 : kc > 64 ? 64 : kc;
    return (int)(K < kc ? K : kc);
}

static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

AttnVLayout attn_layout(int proj, int64_t T, int64_t S, int64_t d, int64_t H, int64_t K) {
    AttnVLayout L{};
    size_t off = 0;
    L.off_lse = off;   off += al256((size_t)T * H * 4);
    L.off_ob = off;    off += proj == 2 ? 0 : al256((size_t)T * H * 4);
    L.off_cpart = off; off += al256((size_t)attn_kc(proj, T, S, H, K) * attn_part_per_draw(proj, T, S, H) * 4);
    L.off_rew = off;   off += al256((size_t)K * T * 4);
    L.off_ghat = off;  off += al256((size_t)T * d * 4);
    L.off_outer = off; off += outer_workspace_bytes(T, d, d);
    L.total = off;
    return L;
}

hipError_t launch_attn_rewards(int proj, const float* q, const float* k, const float* v, const float* e, int64_t T,
                               int64_t S, int64_t d, int64_t H, int64_t K, float sigma, uint64_t seed, uint32_t layer,
                               uint32_t token_offset, uint32_t draw_offset, float* rew, unsigned char* ws,
                               const AttnVLayout& L, hipStream_t stream) {
    const int64_t nkt = S / AT, nb = T / S;
    const int kcmax = attn_kc(proj, T, S, H, K);
    AttnKArgs A{};
    A.q = q; A.k = k; A.v = v; A.e = e;
    A.lse2 = reinterpret_cast<float*>(ws + L.off_lse);
    A.ob = proj == 2 ? nullptr : reinterpret_cast<float*>(ws + L.off_ob);
    A.cpart = reinterpret_cast<float*>(ws + L.off_cpart);
    A.T = (int)T; A.S = (int)S; A.d = (int)d; A.H = (int)H;
    A.k0 = (uint32_t)seed; A.k1 = (uint32_t)(seed >> 32);
    A.layer = layer; A.tok0 = token_offset; A.draw0 = draw_offset;
    A.sdelta = sigma * 0.125f;
    const unsigned grid = (unsigned)(nb * H * nkt);
    if (proj == 2) hipLaunchKernelGGL(attn_stats_kernel<false>, dim3(grid), dim3(ANT), 0, stream, A);
    else hipLaunchKernelGGL(attn_stats_kernel<true>, dim3(grid), dim3(ANT), 0, stream, A);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    for (int64_t i0 = 0; i0 < K; i0 += kcmax) {
        const int kc = (int)(K - i0 < kcmax ? K - i0 : kcmax);
        AttnKArgs Ai = A;
        Ai.draw0 = draw_offset + (uint32_t)i0;
        bool timed;
        if ((err = launch_timer_begin(kTimedAttnMain, stream, timed)) != hipSuccess) return err;
        // one workgroup per (sequence, head, tile) and range of draws: the draws are split
        // across workgroups only as far as needed for about two workgroups per CU (each
        // workgroup recomputes its tiles' clean products per chunk of ADC draws anyway)
        const int nch = (kc + ADC - 1) / ADC;
        const int ny = (int)std::min<int64_t>(nch, std::max<int64_t>(1, (512 + grid - 1) / grid));
        Ai.dper = ((nch + ny - 1) / ny) * ADC;
        const dim3 g2(grid, (unsigned)((kc + Ai.dper - 1) / Ai.dper));
        if (proj == 2)
            hipLaunchKernelGGL(attn_v_kernel, g2, dim3(VNT), 0, stream, Ai, 0, kc);
        else if (proj == 1)
            hipLaunchKernelGGL(attn_k_kernel, g2, dim3(VNT), 0, stream, Ai, kc);
        else
            hipLaunchKernelGGL(attn_q_kernel, g2, dim3(VNT), 0, stream, Ai, kc);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        if ((err = launch_timer_end(kTimedAttnMain, stream, timed)) != hipSuccess) return err;
        const unsigned nblk = (unsigned)(kc * T / 64);   // one workgroup per (draw, 64 tokens)
        if (proj == 2) {
            hipLaunchKernelGGL(attn_csum_kernel, dim3(nblk), dim3((unsigned)(64 * H)), 0, stream, A.cpart, (int)T,
                               (int)S, (int)H, (int)i0, rew);
            if ((err = hipGetLastError()) != hipSuccess) return err;
            hipLaunchKernelGGL(attn_suffix_scan_kernel, dim3((unsigned)(kc * nb)), dim3(256), 0, stream, rew, (int)T,
                               (int)S, (int)i0, sigma);
        } else if (proj == 1) {
            hipLaunchKernelGGL(attn_csum_k_kernel, dim3(nblk), dim3((unsigned)(64 * H)), 0, stream, A.cpart, A.ob,
                               (int)T, (int)S, (int)H, (int)i0, rew);
            if ((err = hipGetLastError()) != hipSuccess) return err;
            hipLaunchKernelGGL(attn_suffix_scan_kernel, dim3((unsigned)(kc * nb)), dim3(256), 0, stream, rew, (int)T,
                               (int)S, (int)i0, 1.0f);
        } else {
            hipLaunchKernelGGL(attn_heads_q_kernel, dim3((unsigned)((kc * T + 255) / 256)), dim3(256), 0, stream,
                               A.cpart, (int)T, (int)H, (int)i0, kc, rew);
        }
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
}

hipError_t launch_attn_v_ghat(int64_t T, int64_t d, int64_t K, float sigma, uint64_t seed, uint32_t layer,
                              uint32_t token_offset, uint32_t draw_offset, const float* rew, float* ghat,
                              hipStream_t stream) {
    AttnKArgs A{};
    A.T = (int)T; A.d = (int)d;
    A.k0 = (uint32_t)seed; A.k1 = (uint32_t)(seed >> 32);
    A.layer = layer; A.tok0 = token_offset; A.draw0 = draw_offset;
    hipLaunchKernelGGL(attn_reduce_kernel, dim3((unsigned)T), dim3(ART), 0, stream, A, (int)K, rew,
                       -1.0f / ((float)K * sigma), ghat);
    return hipGetLastError();
}

}  // namespace dust
