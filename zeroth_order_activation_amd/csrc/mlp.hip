// Interior MLP-linear estimator: W1 of a pre-LN MLP block is perturbed and
// the cached downstream is recomputed per draw.
//
// Method: TL;DR page "Dust: zeroth-order Transformer pretraining without
// backprop", section 1 ("activation-space perturbation", "credit assignment
// without backprop"): noise sigma*a on the output h_t = W1 u_t of the linear
// layer, independently per token and draw; reward = reduction of that token's
// LM loss; g_hat_t = -(1/(K sigma)) sum_i r a; G_W1 = sum_t g_hat_t u_t^T.
// News article (tahou.com), mechanism paragraph: the unperturbed
// intermediates are cached and only what the perturbation changes is
// recomputed -- here GELU -> W2 -> residual -> LayerNorm -> LM head -> CE.
//
// Every (token, draw) pair is one row of the recomputed downstream.  Rows are
// numbered globally: g < T are the clean rows (a = 0, giving CE0), g = T(1+i)+t
// is draw i of token t.  Rows are processed in chunks; per chunk:
//   gemm1   F[g] = bf16(LN(x_t + W2 bf16(GELU(h_t + sigma a))))      (MFMA bf16)
//           small sigma: GELU rows (vector ALU) then W2 + LayerNorm (MFMA);
//           larger sigma: one kernel with the library erf
//   gemm2   per (vocab tile, row): max and sum-exp of z = W_head F[g], and the
//           label logit z[y_t]                                       (MFMA bf16)
//   combine CE[g] = log-sum-exp over the tiles - z[y_t]
// then once: reduce (noise regenerated) -> g_hat, and the outer product.
//
// Both GEMMs compute the transposed product D[feature][row] = W . X^T: the
// weight rows are the MFMA A operand and the token-rows the B operand, so each
// lane ends up holding many features of few rows, and the per-row reductions
// of the epilogues (LayerNorm over d, log-sum-exp over V) stay mostly in-lane.
//
// v_mfma_f32_32x32x16_bf16 operand layout (checked on the device): A[i][k] in
// lane i + 32*(k/8) element k%8; B[k][j] in lane j + 32*(k/8) element k%8;
// D[i][j] in lane j + 32*((i/4)%2), register (i%4) + 4*(i/8).
#include <algorithm>

#include "dust_device.hpp"
#include "dust_internal.hpp"
#include "launch_events.hpp"

namespace dust {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, const f32x16_t& c) {
    bf16x8_t av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
}

// Row of the D layout held by register r of a lane (within a 32x32 block).
__device__ __forceinline__ int drow(int r, int lane) { return (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5); }

// Tiled layout of the bf16 LayerNorm output F (and of the repacked W_head): tiles
// of 256 rows, each split into 32-feature slabs of 256 x 32 contiguous elements
// (16 KB), so that one k-step of the head GEMM reads each operand as one
// contiguous 16 KB block.  The row count is padded to a whole tile.
constexpr int FT_ROWS = 256, FT_KS = 32;
__device__ __forceinline__ int64_t ftile_off(int64_t row, int f, int D) {
    return ((row / FT_ROWS) * (D / FT_KS) + f / FT_KS) * (FT_ROWS * FT_KS) + (row % FT_ROWS) * FT_KS + f % FT_KS;
}

// GELU(x) = x Phi(x) (exact erf form), as the fp32 value whose bf16 rounding
// (nearest even) is taken next.  That decision only depends on the fp32
// evaluation when the value is not within a few ulps of a bf16 tie; in that
// rare case (~2^-11 of inputs) the GELU is re-evaluated in fp64 and rounded to
// fp32 once, so the decision is the one the correctly rounded value takes.
__device__ __forceinline__ float gelu_f32(float x) {
    float g = 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
    const int low = (int)(__float_as_uint(g) & 0xFFFFu);
    if (__builtin_expect(abs(low - 0x8000) <= 16, 0)) {
        const double xd = (double)x;
        g = (float)(0.5 * xd * (1.0 + erf(xd * 0.70710678118654752440)));
    }
    return g;
}

// ---------------------------------------------------------------------------
// gemm1: F = bf16(LN(x + W2 . bf16(GELU(h + sigma a))))
// Workgroup: 64 token-rows x all D features in 16 waves (4 per SIMD); wave w
// owns 32 features (and, for D = 256, one half of the rows).  The B operand
// (64 rows x 64 channels per k-step) is generated in the prologue -- one
// channel quad per thread -- into a double-buffered, XOR-swizzled LDS slab;
// W2 fragments are read straight from global memory (W2 is small and stays in
// L2; each k-step's fragments are loaded before the generation that hides
// their latency, and h a whole k-step ahead).  The MFMA accumulator restarts
// every G1_FLUSH k-steps (512 channels) and is added into an fp32 running
// total kept in LDS: summing the 2048 products in groups of about sqrt(n)
// roughly halves the fp32 accumulation error of W2 m (and with it the rate of
// bf16 rounding decisions of the LayerNorm output that it could flip), while
// the registers stay within the 128 that 4 waves per SIMD allow.
// ---------------------------------------------------------------------------
constexpr int G1_ROWS = 64;
constexpr int G1_KS = 64;     // channels per k-step
constexpr int G1_FLUSH = 8;   // k-steps (512 channels) per accumulator restart
constexpr int G1_WAVES = 16;
constexpr int G1_NT = 64 * G1_WAVES;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats to a pair of bf16 (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    const bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
    uint32_t u;
    __builtin_memcpy(&u, &b, 4);
    return u;
}

// LDS tile of 128-byte rows (64 bf16 = eight 16-byte pieces), with piece p of
// row r stored at piece p ^ ((r >> 1) & 7).  Sixteen lanes reading the same
// piece of sixteen consecutive rows (an MFMA fragment), and sixteen lanes
// writing the eight pieces of two consecutive rows, then both touch all 64
// banks exactly once.
__device__ __forceinline__ int swz(int row, int piece) { return row * 64 + ((piece ^ ((row >> 1) & 7)) << 3); }

template <int D>
__global__ void __launch_bounds__(G1_NT, 1) mlp_gemm1_kernel(MlpArgs A, int64_t g0, int64_t nrows, uint16_t* __restrict__ F) {
    constexpr int FG = D / 32;                   // 32-feature groups (16 or 8)
    constexpr int RG = G1_WAVES / FG;            // row groups (1 or 2)
    constexpr int RB = G1_ROWS / 32 / RG;        // 32-row MFMA blocks per wave (2 or 1)
    constexpr int NV = RB * 16;                  // accumulator values per lane
    __shared__ __align__(16) uint16_t Bs[2][G1_ROWS * G1_KS];
    __shared__ __align__(16) float4 tot[NV / 4][G1_NT];   // running totals, lane-interleaved

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int fg = w % FG, rg = w / FG;
    const int64_t rbase = (int64_t)blockIdx.x * G1_ROWS;  // chunk-local row of row 0
    const int n = A.n;
    const int T = A.T;

    // generation mapping: one channel quad per thread per k-step
    const int gen_row = tid >> 4, gen_q = tid & 15;
    const int64_t gen_lr = rbase + gen_row;
    const bool gen_valid = gen_lr < nrows;
    const int64_t gen_g = g0 + (gen_valid ? gen_lr : 0);
    const bool gen_clean = gen_g < T;
    const int64_t gen_t = gen_g % T;
    const uint32_t gen_draw = gen_clean ? 0u : A.draw0 + (uint32_t)(gen_g / T - 1);
    const float* hrow = A.h + gen_t * n;

    // h of the slab after next is loaded a whole k-step ahead of its use (it
    // streams from beyond L2, and one quad per thread leaves little to
    // overlap).  Loads and arithmetic are unconditional -- lanes past the rows
    // or channels read a clamped, valid address and are zeroed at the end -- so
    // no branch separates a load from its use.
    const float sig_eff = gen_clean ? 0.f : A.sigma;
    const bool gen_any = gen_valid;
    auto load_h = [&](int ks) -> float4 {
        const int c0 = ks * G1_KS + 4 * gen_q;
        return *reinterpret_cast<const float4*>(hrow + (c0 < n ? c0 : n - 4));
    };
    auto generate = [&](int ks, const float4& h4) -> uint2 {
        const int c0 = ks * G1_KS + 4 * gen_q;
        const f32x4 g = gauss4(A.tok0 + (uint32_t)gen_t, (uint32_t)(c0 >> 2), gen_draw, A.layer, A.k0, A.k1);
        const float hv[4] = {fmaf(sig_eff, g.v[0], h4.x), fmaf(sig_eff, g.v[1], h4.y), fmaf(sig_eff, g.v[2], h4.z),
                             fmaf(sig_eff, g.v[3], h4.w)};
        const bool ok = gen_any && c0 < n;
        float gv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) gv[c] = ok ? gelu_f32(hv[c]) : 0.f;
        return make_uint2(pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3]));
    };
    auto store_slab = [&](int buf, uint2 v) {
        *reinterpret_cast<uint2*>(&Bs[buf][swz(gen_row, gen_q >> 1) + 4 * (gen_q & 1)]) = v;
    };

    const f32x16_t zero = {};
    f32x16_t acc[RB];
    // each thread owns its column of the total: no atomics needed
    auto flush = [&]() {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                float4 o = tot[rb * 4 + r4][tid];
                o.x += acc[rb][4 * r4]; o.y += acc[rb][4 * r4 + 1];
                o.z += acc[rb][4 * r4 + 2]; o.w += acc[rb][4 * r4 + 3];
                tot[rb * 4 + r4][tid] = o;
            }
    };
    const int f = fg * 32 + (lane & 31);           // W2 row of this lane's A fragments
    const uint16_t* w2row = A.w2 + (int64_t)f * n;
    const int row0 = rg * RB * 32;                 // first LDS row of this wave
    const int nks = (n + G1_KS - 1) / G1_KS;

    // One k-step: fetch this k-step's W2 fragments and the h of the slab after
    // next, generate slab ks + 1 on the VALU (covering both loads), then -- after
    // adding the accumulator into the LDS total when a group of G1_FLUSH k-steps
    // has ended (the MFMAs that produced it are long done) -- read slab ks
    // (buffer ks & 1) and issue the MFMAs.
    // KQ: 16-channel sub-steps in this k-step (4, or 2 for a last k-step of 32).
    // hc holds h of slab ks + 1 (loaded a k-step earlier); hl receives h of slab
    // ks + 2.  The caller alternates the two, so no register copy waits on a load.
    auto kstep = [&](int ks, auto kq, const float4& hc, float4& hl) {
        constexpr int KQ = decltype(kq)::value;
        const int buf = ks & 1;
        uint4 af[KQ];
#pragma unroll
        for (int kk = 0; kk < KQ; ++kk)
            af[kk] = *reinterpret_cast<const uint4*>(w2row + ks * G1_KS + kk * 16 + 8 * (lane >> 5));
        hl = load_h(ks + 2 < nks ? ks + 2 : ks);
        uint2 nxt = make_uint2(0, 0);
        if (ks + 1 < nks) nxt = generate(ks + 1, hc);
        if (ks > 0 && ks % G1_FLUSH == 0) {  // uniform
            flush();
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) acc[rb] = zero;
        }
#pragma unroll
        for (int kk = 0; kk < KQ; ++kk) {
            const int piece = kk * 2 + (lane >> 5);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const uint4 bfr = *reinterpret_cast<const uint4*>(&Bs[buf][swz(row0 + rb * 32 + (lane & 31), piece)]);
                acc[rb] = mfma32(af[kk], bfr, acc[rb]);
            }
        }
        if (ks + 1 < nks) store_slab(buf ^ 1, nxt);
        __syncthreads();
    };
    using Q4 = std::integral_constant<int, 4>;
    using Q2 = std::integral_constant<int, 2>;

#pragma unroll
    for (int r4 = 0; r4 < NV / 4; ++r4) tot[r4][tid] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = zero;
    float4 ha = load_h(0), hb;
    store_slab(0, generate(0, ha));
    ha = load_h(1 < nks ? 1 : 0);
    __syncthreads();
    const int nfull = n / G1_KS;  // k-steps of 64 channels; then one of 32 if n % 64 != 0
    int ks = 0;
    for (; ks + 2 <= nfull; ks += 2) {
        kstep(ks, Q4{}, ha, hb);
        kstep(ks + 1, Q4{}, hb, ha);
    }
    if (ks < nfull) {
        kstep(ks, Q4{}, ha, hb);
        if (nfull < nks) kstep(ks + 1, Q2{}, hb, ha);
    } else if (nfull < nks) {
        kstep(ks, Q2{}, ha, hb);
    }
    flush();

    // ---- epilogue: residual add, LayerNorm over D, bf16 ---------------------
    // lane holds rows j = row0 + rb*32 + lane%32; for each, features
    // fg*32 + drow(r, lane).  y = x + o, the LayerNorm statistics and the
    // normalised value are computed in fp64 and rounded to fp32 once before the
    // bf16 rounding: an fp32 y would carry half an ulp of y into (y - mean),
    // which for entries near the mean decides their bf16 rounding far more often
    // than the accumulation error of o does.  The reduction buffer reuses the slabs.
    double* red = reinterpret_cast<double*>(&Bs[0][0]);   // [G1_WAVES][G1_ROWS]
    double y[RB][16];
    double s[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int lr = row0 + rb * 32 + (lane & 31);
        const int64_t row = rbase + lr;
        const int64_t t = (g0 + (row < nrows ? row : 0)) % T;
        s[rb] = 0.0;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const float4 o = tot[rb * 4 + r4][tid];
            const int ff = fg * 32 + 8 * r4 + 4 * (lane >> 5);
            const float4 xv = *reinterpret_cast<const float4*>(A.x_res + t * D + ff);
            y[rb][4 * r4 + 0] = (double)o.x + (double)xv.x;
            y[rb][4 * r4 + 1] = (double)o.y + (double)xv.y;
            y[rb][4 * r4 + 2] = (double)o.z + (double)xv.z;
            y[rb][4 * r4 + 3] = (double)o.w + (double)xv.w;
#pragma unroll
            for (int c = 0; c < 4; ++c) s[rb] += y[rb][4 * r4 + c];
        }
        s[rb] += __shfl_xor(s[rb], 32, 64);
    }
    // the slabs are free once every wave has passed the loop's last barrier
    auto row_total = [&](int lr) {
        const int g = lr / (RB * 32);  // row group of that row
        double v = 0.0;
#pragma unroll
        for (int k = 0; k < FG; ++k) v += red[(g * FG + k) * G1_ROWS + lr];
        return v;
    };
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
        if (lane < 32) red[w * G1_ROWS + row0 + rb * 32 + lane] = s[rb];
    __syncthreads();
    double mean[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) mean[rb] = row_total(row0 + rb * 32 + (lane & 31)) * (1.0 / D);
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        double v = 0.0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const double dv = y[rb][r] - mean[rb];
            v = fma(dv, dv, v);
        }
        v += __shfl_xor(v, 32, 64);
        if (lane < 32) red[w * G1_ROWS + row0 + rb * 32 + lane] = v;
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int lr = row0 + rb * 32 + (lane & 31);
        const int64_t row = rbase + lr;
        const double var = row_total(lr) * (1.0 / D);
        const double rstd = 1.0 / sqrt(var + (double)A.ln_eps);
        if (row >= nrows) continue;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int ff = fg * 32 + 8 * r4 + 4 * (lane >> 5);
            float o[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) o[c] = (float)((y[rb][4 * r4 + c] - mean[rb]) * rstd);
            *reinterpret_cast<uint2*>(F + ftile_off(row, ff, D)) =
                make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        }
    }
}

// ---------------------------------------------------------------------------
// gemm1, Taylor form (small sigma).  The same F = bf16(LN(x + W2 bf16(GELU(h~))))
// with h~ = h + sigma a, for the draw rows, but GELU(h~) = h~ Phi(h~) is formed
// from the token's cached Phi(h), phi(h) (computed once per call, in fp64, by
// mlp_phi_kernel) through the exact identity
//     Phi(h + delta) - Phi(h) = phi(h) I(h, delta),  I = int_0^delta exp(-h s - s^2/2) ds,
// with I by its Taylor series to delta^5:
//     I = delta (1 + delta (e1 + delta (e2 + delta (e3 + delta e4)))),
//     e1 = -h/2, e2 = (h^2 - 1)/6, e3 = -h (h^2 - 3)/24, e4 = (h^4 - 6 h^2 + 3)/120.
// The host takes this form when |delta| <= sigma sqrt(48 ln 2) <= 1/16; then for
// h >= -3.5 the dropped delta^6 term is below one fp32 ulp of Phi(h~) and the
// fp32 value of GELU(h~) is within 3 ulps of the exact one.  Entries within 8 ulps
// of a bf16 tie, and entries with h < -3.5 (Phi small), are re-evaluated in fp64
// as 0.5 h~ (1 + erf(h~/sqrt 2)), so every bf16 decision is the one the exactly
// rounded GELU takes.  Per entry this costs about a dozen VALU operations where
// the library erf costs about forty.
//
// The form runs as two kernels per chunk of rows: mlp_gelu_rows_kernel writes
// M = bf16(GELU(h~)) for every row of the chunk (one wave per token and 256
// channels, the token's cached h, Phi(h), phi(h) and series coefficients held in
// registers across its draws, two draws' Philox chains side by side), then
// mlp_w2ln_kernel forms F = bf16(LN(x + W2 M)) on MFMA.  W2 is read in MFMA
// fragment order (mlp_w2frag_kernel), one contiguous 1 KB per wave and fragment.
// ---------------------------------------------------------------------------
constexpr float GT_FAR = -3.5f;   // h below this: fp64 evaluation
constexpr double GT_MAX_DELTA = 0.0625;

bool mlp_taylor_ok(float sigma) { return (double)sigma * 5.7683 <= GT_MAX_DELTA; }

// Phi(h), phi(h) of every cached entry, in fp64, rounded to fp32 once.
__global__ void __launch_bounds__(256) mlp_phi_kernel(const float* __restrict__ h, int64_t count,
                                                      float* __restrict__ Pt, float* __restrict__ pt) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= count) return;
    const double x = (double)h[i];
    Pt[i] = (float)(0.5 * erfc(-x * 0.70710678118654752440));
    pt[i] = (float)(exp(-0.5 * x * x) * 0.39894228040143267794);
}

// W2 [D][n] bf16 -> fragment order [D/32][n/16][64 lanes][8]: lane l of the A
// fragment of feature block fb, sub-step s holds W2[32 fb + l%32][16 s + 8 (l/32) .. +8].
__global__ void __launch_bounds__(256) mlp_w2frag_kernel(const uint16_t* __restrict__ w2, int D, int n,
                                                         uint16_t* __restrict__ w2f) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one 16-byte piece
    const int nsub = n / 16;
    if (i >= (int64_t)(D / 32) * nsub * 64) return;
    const int lane = (int)(i & 63);
    const int64_t fs = i >> 6;
    const int s = (int)(fs % nsub), fb = (int)(fs / nsub);
    const int f = fb * 32 + (lane & 31);
    const int c = s * 16 + 8 * (lane >> 5);
    *reinterpret_cast<uint4*>(w2f + i * 8) = *reinterpret_cast<const uint4*>(w2 + (int64_t)f * n + c);
}

// GELU of one entry in fp64, rounded to fp32 once (the rare exact path).
__device__ __attribute__((noinline)) float gelu_exact(float x) {
    const double xd = (double)x;
    return (float)(0.5 * xd * (1.0 + erf(xd * 0.70710678118654752440)));
}

// ---- kernel A: M = bf16(GELU(h + sigma a)) of the draw rows -----------------
// One wave per (token, 256-channel block): lane l holds channel quad l of the
// block, its cached h, Phi(h), phi(h) and the series coefficients, and makes the
// quad for every draw slot of the launch, two draws at a time (token, draw and
// layer are uniform across the wave, so the first Philox rounds stay scalar).  Each
// draw's 512 bytes of the wave are one contiguous store into row (slot T + t) of M.
constexpr int GA_NT = 256;
__global__ void __launch_bounds__(GA_NT) mlp_gelu_rows_kernel(MlpArgs A, float sig_u, const float* __restrict__ Pt,
                                                             const float* __restrict__ pt, int64_t g0, int first_slot,
                                                             int nslots, uint16_t* __restrict__ M) {
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * (GA_NT / 64) + (threadIdx.x >> 6);
    const int T = A.T, n = A.n;
    const int ncb = (n + 255) / 256;
    if (wid >= (int64_t)T * ncb) return;
    const int t = (int)(wid / ncb), cb = (int)(wid % ncb);
    const int c0 = cb * 256 + 4 * lane;
    const bool live = c0 < n;
    const int cc = live ? c0 : n - 4;
    const float4 h4 = *reinterpret_cast<const float4*>(A.h + (int64_t)t * n + cc);
    const float4 P4 = *reinterpret_cast<const float4*>(Pt + (int64_t)t * n + cc);
    const float4 p4 = *reinterpret_cast<const float4*>(pt + (int64_t)t * n + cc);
    const float gh[4] = {h4.x, h4.y, h4.z, h4.w};
    const float gP[4] = {P4.x, P4.y, P4.z, P4.w};
    const float gp[4] = {p4.x, p4.y, p4.z, p4.w};
    float e1[4], e2[4], e3[4], e4[4];
    uint32_t far_mask = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float x = gh[c], x2 = x * x;
        e1[c] = -0.5f * x;
        e2[c] = fmaf(x2, 1.0f / 6.0f, -1.0f / 6.0f);
        e3[c] = x * fmaf(x2, -1.0f / 24.0f, 3.0f / 24.0f);
        e4[c] = fmaf(x2, fmaf(x2, 1.0f / 120.0f, -6.0f / 120.0f), 3.0f / 120.0f);
        far_mask |= (x < GT_FAR ? 1u : 0u) << c;
    }
    const uint32_t tok = A.tok0 + (uint32_t)t;
    const uint32_t q = (uint32_t)(c0 >> 2);
    const int64_t slot_g0 = g0 / T + first_slot;   // g / T of launch slot 0
    uint16_t* mrow0 = M + ((int64_t)first_slot * T + t) * n + cc;
    auto gelu4 = [&](const f32x4& a, float (&v)[4], bool& slow) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float ht = fmaf(sig_u, a.v[c], gh[c]);   // the noise is drawn divided by sqrt(2 ln 2)
            const float dl = ht - gh[c];
            float tt = fmaf(dl, e4[c], e3[c]);
            tt = fmaf(dl, tt, e2[c]);
            tt = fmaf(dl, tt, e1[c]);
            tt = fmaf(dl, tt, 1.0f);
            const float Pn = fmaf(gp[c], dl * tt, gP[c]);
            v[c] = ht * Pn;
            // within 8 fp32 ulps of a bf16 tie (the low half of the bits in [0x7FF8, 0x8007])
            slow |= ((__float_as_uint(v[c]) + 8u) & 0xFFF0u) == 0x8000u;
        }
    };
    auto fix4 = [&](const f32x4& a, float (&v)[4]) {   // the rare fp64 path
#pragma unroll 1
        for (int c = 0; c < 4; ++c) {
            float ve = 0.f, ae = 0.f, he = 0.f;
#pragma unroll
            for (int c2 = 0; c2 < 4; ++c2)   // select without dynamic register indexing
                if (c2 == c) { ve = v[c2]; ae = a.v[c2]; he = gh[c2]; }
            if (((__float_as_uint(ve) + 8u) & 0xFFF0u) == 0x8000u || ((far_mask >> c) & 1u)) {
                ve = gelu_exact(fmaf(sig_u, ae, he));
#pragma unroll
                for (int c2 = 0; c2 < 4; ++c2)
                    if (c2 == c) v[c2] = ve;
            }
        }
    };
    auto store = [&](int s, const float (&v)[4]) {
        if (live)
            *reinterpret_cast<uint2*>(mrow0 + (int64_t)s * T * n) =
                make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    };
#pragma unroll 1
    for (int s = 0; s < nslots; s += 2) {
        const bool two = s + 1 < nslots;   // uniform
        const uint32_t d0 = A.draw0 + (uint32_t)(slot_g0 + s - 1);
        const f32x4 a0 = gauss4_unscaled_uniform(tok, q, d0, A.layer, A.k0, A.k1);
        const f32x4 a1 = gauss4_unscaled_uniform(tok, q, d0 + 1u, A.layer, A.k0, A.k1);
        float v0[4], v1[4];
        bool slow0 = far_mask != 0, slow1 = far_mask != 0;
        gelu4(a0, v0, slow0);
        gelu4(a1, v1, slow1);
        if (__builtin_amdgcn_ballot_w64(slow0 || slow1)) {
            if (slow0) fix4(a0, v0);
            if (slow1) fix4(a1, v1);
        }
        store(s, v0);
        if (two) store(s + 1, v1);
    }
}

// ---- kernel B: F = bf16(LN(x + W2 M)) for 64 consecutive chunk rows ----------
// 8 waves (2 per SIMD); wave c owns features [c D/8, (c+1) D/8) of the 64 rows.
// M moves by direct global->LDS loads into a 4-stage ring of 64 x 128-channel
// slabs (row r's 16-byte piece p stored at p ^ (r & 15), the swizzle applied on
// the global side since a direct load puts lane l at slot l), three k-steps in
// flight; W2 fragments come in fragment order straight from global memory two
// sub-steps ahead.  The accumulator is added into an fp32 running total in
// registers every 128 channels (groups of 128 of the 2048 products: about half
// the rounding error of one chain, which shows in the bf16 decisions of f); the
// residual and the LayerNorm are formed in fp64.
// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt at
// their maxima, i.e. not waited for)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

constexpr int GB_ROWS = 64;
constexpr int GB_KS = 128;
constexpr int GB_NT = 512;
constexpr int GB_STAGES = 4;

// FAST (n a multiple of 512: whole groups of four full k-steps): every k-step has
// the same shape with no branches -- the W2 fragment and M slab loads past the end
// re-read the last valid ones -- so the compiler tracks the outstanding loads
// exactly and waits for a W2 fragment alone, not for the M slab loads issued after
// it (at a branch join it waits for everything).
template <int D, bool FAST>
__global__ void __launch_bounds__(GB_NT, 1) mlp_w2ln_kernel(MlpArgs A, const uint16_t* __restrict__ w2f,
                                                           const uint16_t* __restrict__ M, int64_t g0, int64_t nrows,
                                                           uint16_t* __restrict__ F) {
    constexpr int FB = D / 256;                 // 32-feature blocks per wave (2 or 1)
    // the four ring stages as separate LDS objects: the compiler can then tell that
    // reads of one stage do not alias direct loads still in flight into another,
    // and does not drain those loads before each read
    __shared__ __align__(16) uint16_t Ms0[GB_ROWS * GB_KS], Ms1[GB_ROWS * GB_KS], Ms2[GB_ROWS * GB_KS],
        Ms3[GB_ROWS * GB_KS];
    __shared__ double red[2][8][GB_ROWS];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int T = A.T, n = A.n;
    const int64_t r0 = (int64_t)blockIdx.x * GB_ROWS;
    const int nks = (n + GB_KS - 1) / GB_KS;   // the last k-step may hold 32..96 channels
    const int nsub_total = n / 16;

    // direct loads: each k-step's slab is 64 rows x 16 pieces = 1024 pieces, two
    // per lane; lane slot s = 64 (2 w + j) + lane holds row s/16, stored piece
    // s%16, i.e. logical piece (s%16) ^ (row & 15) of that row (rows past the
    // chunk read zero, channels past n re-read valid ones; both are masked).
    // The loads go through a buffer resource over this block's rows (bytes past the
    // chunk's last row read as zero) rather than through global addresses: the
    // compiler counts a global load into LDS as a possible flat access and then
    // waits for every outstanding load before any use of a loaded register.
    const int vrows = (int)min<int64_t>(GB_ROWS, nrows - r0);
    const __amdgpu_buffer_rsrc_t mres =
        __builtin_amdgcn_make_buffer_rsrc((void*)(M + r0 * n), (short)0, vrows * n * 2, 0x00020000);
    int rowoff[2], soff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int slot = 64 * (2 * w + j) + lane;
        rowoff[j] = (slot >> 4) * n;
        soff[j] = 64 * (2 * w + j) * 8;   // element offset of this wave's 64 slots
    }

    // B fragment of sub-step s, row block rb: row 32 rb + lane%32, logical piece
    // 2 s + lane/32 at stored piece 2 (s ^ m) + c (m = (lane & 15) >> 1,
    // c = (lane/32) ^ (lane & 1)); row block 1 is 8 KB further
    const int rd_base = (lane & 31) * (GB_KS * 2) + (((lane >> 5) ^ (lane & 1)) << 4);
    const int mk = (lane & 15) >> 1;
    const int fbase = w * (32 * FB);
    const uint4* w2fw = reinterpret_cast<const uint4*>(w2f) + ((int64_t)(fbase / 32) * nsub_total) * 64 + lane;
    auto load_a = [&](int sub, uint4 (&af)[FB]) {
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) af[fb] = w2fw[((int64_t)fb * nsub_total + sub) * 64];
    };
    const f32x16_t zero = {};
    f32x16_t acc[FB][2];
    float tot[FB][2][16];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            acc[fb][rb] = zero;
#pragma unroll
            for (int r = 0; r < 16; ++r) tot[fb][rb][r] = 0.f;
        }
    // M slab loads: piece p of k-step ks; past n a piece re-reads the row's
    // first piece of the k-step (its channels are never multiplied)
    auto issue_ks = [&](int ks, uint16_t* dst) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int slot = 64 * (2 * w + j) + lane;
            const int piece = (slot & 15) ^ ((slot >> 4) & 15);
            const int c = ks * GB_KS + 8 * piece;
            const int voff = 2 * (rowoff[j] + (c < n ? c : ks * GB_KS));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(mres, (__attribute__((address_space(3))) void*)(dst + soff[j]), 16,
                                                     voff, 0, 0, 0);
        }
    };
    // W2 fragments are loaded PF sub-steps ahead of their MFMAs (one L2 round trip
    // takes about as long as PF sub-steps of MFMAs).  Order of the vector-memory
    // operations: fragments of sub-steps 0 .. PF-1, slabs 0, 1, 2; then per
    // iteration ks: the fragments of sub-steps 8 ks + PF .. 8 ks + PF + 7 (8 FB
    // loads when they all exist), then slab ks + 3 (2 loads).  Slab ks has landed
    // once at most the operations issued after it are outstanding: 4 (ks = 0),
    // 8 FB + 4 (ks = 1), 16 FB + 4 (ks >= 2), when all of those were issued;
    // otherwise the wait is for everything.
    constexpr int PF = 4;
    uint4 fr[PF][FB];
#pragma unroll
    for (int k = 0; k < PF; ++k)
        if (k < nsub_total) load_a(k, fr[k]);
    if (0 < nks) issue_ks(0, Ms0);
    if (1 < nks) issue_ks(1, Ms1);
    if (2 < nks) issue_ks(2, Ms2);
    // k-step ks on stage `cur`; the slab of ks + 3 goes into `nxt` (the stage read
    // by k-step ks - 1, which every wave has finished at this k-step's barrier)
    auto kstep = [&](int ks, const uint16_t* cur, uint16_t* nxt) {
        if (ks == 0 && nks >= 3) __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
        else if (ks == 1 && nks >= 4) __builtin_amdgcn_s_waitcnt(vmcnt_imm(8 * FB + 4));
        else if (ks >= 2 && ks + 2 < nks) __builtin_amdgcn_s_waitcnt(vmcnt_imm(16 * FB + 4));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        // a barrier without the full memory wait that __syncthreads adds (which
        // would drain the later slabs' loads as well); the memory clobber keeps
        // the compiler from moving LDS accesses across it
        asm volatile("s_barrier" ::: "memory");
        const unsigned char* slab = reinterpret_cast<const unsigned char*>(cur);
        const int nsub = min(GB_KS, n - ks * GB_KS) / 16;
#pragma unroll
        for (int s = 0; s < GB_KS / 16; ++s) {
            if (s < nsub) {
                const int g = ks * (GB_KS / 16) + s;
                const int off = rd_base + (((s ^ mk) & 7) << 5);
                uint4 bfr[2];
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
                    bfr[rb] = *reinterpret_cast<const uint4*>(slab + off + rb * 32 * GB_KS * 2);
#pragma unroll
                for (int fb = 0; fb < FB; ++fb)
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) acc[fb][rb] = mfma32(fr[s % PF][fb], bfr[rb], acc[fb][rb]);
                if (g + PF < nsub_total) load_a(g + PF, fr[s % PF]);
            }
        }
        if (ks + GB_STAGES - 1 < nks) issue_ks(ks + GB_STAGES - 1, nxt);
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) tot[fb][rb][r] += acc[fb][rb][r];
                acc[fb][rb] = zero;
            }
    };
    if (FAST) {
        // Branch-free k-steps: every one issues the same 8 FB + 2 loads (the
        // fragments PF sub-steps ahead and slab ks + 3, both clamped to the last
        // ones), so the waits are exact.  K-step ks reads the first sub-step of
        // slab ks + 1 during its last sub-step (the fragments of the next sub-step
        // are always read while the current one's MFMAs issue), so it starts once
        // slab ks + 1 has landed: then at most the 8 FB + 2 loads of k-step ks - 1
        // (the 2 of slab 2 before k-step 0) are outstanding.
        uint4 bq[2][2];
        auto read_b = [&](const uint16_t* st, int s, uint4 (&b)[2]) {
            const unsigned char* slab = reinterpret_cast<const unsigned char*>(st);
            const int off = rd_base + (((s ^ mk) & 7) << 5);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) b[rb] = *reinterpret_cast<const uint4*>(slab + off + rb * 32 * GB_KS * 2);
        };
        auto kfast = [&](int ks, const uint16_t* cur, const uint16_t* nx1, uint16_t* nxt, bool first) {
            if (first) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2));
            else __builtin_amdgcn_s_waitcnt(vmcnt_imm(8 * FB + 2));
            asm volatile("s_barrier" ::: "memory");
#pragma unroll
            for (int s = 0; s < GB_KS / 16; ++s) {
                const int g = ks * (GB_KS / 16) + s;
                if (s + 1 < GB_KS / 16) read_b(cur, s + 1, bq[(s + 1) & 1]);
                else read_b(nx1, 0, bq[0]);
#pragma unroll
                for (int fb = 0; fb < FB; ++fb)
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) acc[fb][rb] = mfma32(fr[s % PF][fb], bq[s & 1][rb], acc[fb][rb]);
                load_a(min(g + PF, nsub_total - 1), fr[s % PF]);
            }
            issue_ks(min(ks + GB_STAGES - 1, nks - 1), nxt);
#pragma unroll
            for (int fb = 0; fb < FB; ++fb)
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) tot[fb][rb][r] += acc[fb][rb][r];
                    acc[fb][rb] = zero;
                }
        };
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));   // slab 0
        asm volatile("s_barrier" ::: "memory");
        read_b(Ms0, 0, bq[0]);
        kfast(0, Ms0, Ms1, Ms3, true);
        kfast(1, Ms1, Ms2, Ms0, false);
        kfast(2, Ms2, Ms3, Ms1, false);
        kfast(3, Ms3, Ms0, Ms2, false);
        for (int ks = 4; ks < nks; ks += GB_STAGES) {
            kfast(ks, Ms0, Ms1, Ms3, false);
            kfast(ks + 1, Ms1, Ms2, Ms0, false);
            kfast(ks + 2, Ms2, Ms3, Ms1, false);
            kfast(ks + 3, Ms3, Ms0, Ms2, false);
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // the loads past the end
    } else {
        for (int ks = 0; ks < nks; ks += GB_STAGES) {
            kstep(ks, Ms0, Ms3);
            if (ks + 1 < nks) kstep(ks + 1, Ms1, Ms0);
            if (ks + 2 < nks) kstep(ks + 2, Ms2, Ms1);
            if (ks + 3 < nks) kstep(ks + 3, Ms3, Ms2);
        }
    }
    __syncthreads();   // the epilogue reuses nothing of the ring, but every wave leaves the loop together

    // ---- epilogue: residual add, LayerNorm over D, bf16 (fp64) ---------------
    // lane holds rows 32 rb + lane%32 and features fbase + 32 fb + drow(r, lane).
    // The residual values are loaded once, into the registers the accumulators
    // held.  One pass takes the shifted sums S1 = sum (y - c), S2 = sum (y - c)^2
    // with c = x[row][0] (the same for every lane of the row): mean = c + S1 / D
    // and var = S2 / D - (S1 / D)^2, without cancellation as c lies within the
    // row's values.
    float xv[FB][2][16];
    double csh[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int64_t row = min(r0 + rb * 32 + (lane & 31), nrows - 1);
        const float* xrow = A.x_res + ((g0 + row) % T) * D;
        csh[rb] = (double)xrow[0];
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float4 q = *reinterpret_cast<const float4*>(xrow + fbase + fb * 32 + 8 * r4 + 4 * (lane >> 5));
                xv[fb][rb][4 * r4 + 0] = q.x;
                xv[fb][rb][4 * r4 + 1] = q.y;
                xv[fb][rb][4 * r4 + 2] = q.z;
                xv[fb][rb][4 * r4 + 3] = q.w;
            }
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        double s1 = 0.0, s2 = 0.0;
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const double dv = ((double)tot[fb][rb][r] + (double)xv[fb][rb][r]) - csh[rb];
                s1 += dv;
                s2 = fma(dv, dv, s2);
            }
        s1 += __shfl_xor(s1, 32, 64);
        s2 += __shfl_xor(s2, 32, 64);
        if (lane < 32) {
            red[0][w][rb * 32 + lane] = s1;
            red[1][w][rb * 32 + lane] = s2;
        }
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int64_t row = r0 + rb * 32 + (lane & 31);
        double s1 = 0.0, s2 = 0.0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            s1 += red[0][k][rb * 32 + (lane & 31)];
            s2 += red[1][k][rb * 32 + (lane & 31)];
        }
        const double m1 = s1 * (1.0 / D);
        const double mean = csh[rb] + m1;
        const double rstd = 1.0 / sqrt(fma(-m1, m1, s2 * (1.0 / D)) + (double)A.ln_eps);
        if (row >= nrows) continue;
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int ff = fbase + fb * 32 + 8 * r4 + 4 * (lane >> 5);
                float o[4];
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    o[c] = (float)((((double)tot[fb][rb][4 * r4 + c] + (double)xv[fb][rb][4 * r4 + c]) - mean) * rstd);
                *reinterpret_cast<uint2*>(F + ftile_off(row, ff, D)) =
                    make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
            }
    }
}

// ---------------------------------------------------------------------------
// gemm2: per (vocab tile of 256, row): partial log-sum-exp of z = W_head F
// and the label logit.  Workgroup tile 256 vocab x 256 rows, 8 waves of
// 128 vocab x 64 rows (4 x 2 MFMA blocks, 128 accumulators).  Both operands go
// from global memory straight into a four-stage LDS ring in 32-wide k-steps
// (buffer loads into LDS, three k-steps in flight ahead of the one computed);
// each wave reads the fragments of the next 16-channel sub-step while the
// current sub-step's MFMAs issue.  A 128 x 128 wave tile would read a third
// less LDS per MFMA, but its 256 accumulators leave one wave per SIMD.
// ---------------------------------------------------------------------------
constexpr int G2_TV = FT_ROWS, G2_TR = FT_ROWS, G2_KS = FT_KS, G2_STAGES = 4;
constexpr int G2_VB = 4, G2_RB = 2;   // MFMA blocks per wave (vocab, rows): 128 x 64
constexpr int G2_WAVES = 8;           // 2 vocab halves x 4 row quarters
constexpr int G2_NT = 64 * G2_WAVES;
constexpr int G2_WR = G2_RB * 32;     // rows per wave
// Fixed log-sum-exp offset: |z_v| <= |f| |w_v| (Cauchy-Schwarz) and the bf16
// LayerNorm output has |f| <= sqrt(d) (1 + 2^-9).  When C = sqrt(d) 1.004
// max_v |w_v| <= 40, every term exp(z - C) lies in [e^-80, 1]: no overflow,
// no underflow, so the running maximum (and its second pass) can be skipped.
constexpr float G2_FIXED_MAX = 40.0f;

// LDS element offset of 16-byte piece `piece` (0..3) of tile row `row` in a
// 32-channel k-step slab: rows are 64 bytes apart and the piece is XORed with
// (row / 4) % 4, so the 16 lanes of one row-group read 16 distinct 16-byte bank
// groups.
__device__ __forceinline__ int swz32(int row, int piece) { return row * 32 + ((piece ^ ((row >> 2) & 3)) << 3); }

// W_head [V][d] -> tiled layout (ftile_off), rows past V zero.
__global__ void __launch_bounds__(256) mlp_wtile_kernel(const uint16_t* __restrict__ w, int V, int D, int nvt,
                                                        uint16_t* __restrict__ wt) {
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 16-byte piece of the tiled array
    if (p >= (int64_t)nvt * FT_ROWS * D / 8) return;
    const int64_t e = p * 8;
    const int64_t slab = e / (FT_ROWS * FT_KS);
    const int within = (int)(e % (FT_ROWS * FT_KS));
    const int nks = D / FT_KS;
    const int v = (int)(slab / nks) * FT_ROWS + within / FT_KS;
    const int f = (int)(slab % nks) * FT_KS + within % FT_KS;
    uint4 q = make_uint4(0u, 0u, 0u, 0u);
    if (v < V) q = *reinterpret_cast<const uint4*>(w + (int64_t)v * D + f);
    *reinterpret_cast<uint4*>(wt + e) = q;
}


// Largest row norm of W_head, as an fp32 upper bound (one workgroup per 256
// rows, then a single-block maximum).
__global__ void __launch_bounds__(256) mlp_wnorm_kernel(const uint16_t* __restrict__ w, int V, int D,
                                                        float* __restrict__ blockmax) {
    const int v = blockIdx.x * 256 + threadIdx.x;
    float s = 0.f;
    if (v < V) {
        const uint16_t* row = w + (int64_t)v * D;
        for (int k = 0; k < D; k += 8) {
            const uint4 q = *reinterpret_cast<const uint4*>(row + k);
            const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = __uint_as_float(u[e] << 16), b = __uint_as_float(u[e] & 0xFFFF0000u);
                s = fmaf(a, a, fmaf(b, b, s));
            }
        }
    }
    __shared__ float sh[4];
    s = wave_max(s);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) blockmax[blockIdx.x] = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}

__global__ void __launch_bounds__(256) mlp_wnorm_final_kernel(const float* __restrict__ blockmax, int nb, int D,
                                                              float* __restrict__ offset) {
    float m = 0.f;
    for (int i = threadIdx.x; i < nb; i += 256) m = fmaxf(m, blockmax[i]);
    __shared__ float sh[4];
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        const float mx = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
        // sqrt rounded up generously; the 1.004 covers |f| growth by bf16 rounding
        offset[0] = sqrtf((float)D * mx) * 1.004f * (1.0f + 1e-5f);
    }
}

__global__ void __launch_bounds__(G2_NT, 1) mlp_gemm2_kernel(MlpArgs A, int64_t g0, int64_t nrows, int64_t nrt, int nvt,
                                                            const uint16_t* __restrict__ Wt,
                                                            const uint16_t* __restrict__ F, float2* __restrict__ part,
                                                            float* __restrict__ zy, const float* __restrict__ offset) {
    // the ring stages as separate LDS objects: reads of one provably do not
    // alias loads in flight into another
    __shared__ __align__(16) uint16_t As0[G2_TV * G2_KS], As1[G2_TV * G2_KS], As2[G2_TV * G2_KS], As3[G2_TV * G2_KS];
    __shared__ __align__(16) uint16_t Bs0[G2_TR * G2_KS], Bs1[G2_TR * G2_KS], Bs2[G2_TR * G2_KS], Bs3[G2_TR * G2_KS];
    __shared__ float2 red[2][G2_TR];

    // the wave index as a scalar: the LDS destinations of the loads into LDS (M0)
    // then come from scalar arithmetic, not from a read of the first lane per load
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wv = w & 1, wr = w >> 1;
    // XCD-aware order (workgroup b runs on XCD b % 8).  With a vocabulary tile
    // count that is a multiple of 4, the vocabulary is split into 4 groups; XCDs
    // 2g and 2g + 1 take group g, alternating over the row tiles, and on one XCD
    // the group's tiles of a row tile run back to back.  Each F tile then leaves
    // HBM 4 times (once per group) and each XCD keeps a quarter of W_head in its
    // L2.  Otherwise: vocabulary tile fastest.
    int vt;
    int64_t rt;
    if ((nvt & 3) == 0) {
        const int x = blockIdx.x & 7, gv = nvt >> 2;
        const int64_t i = blockIdx.x >> 3;
        rt = 2 * (i / gv) + (x & 1);
        vt = (x >> 1) * gv + (int)(i % gv);
        if (rt >= nrt) return;   // the odd row tile's empty twin (whole workgroup)
    } else {
        vt = blockIdx.x % nvt;
        rt = blockIdx.x / nvt;
    }
    const int v0 = vt * G2_TV;
    const int64_t r0 = rt * G2_TR;
    const int D = A.d, V = A.V;

    // Both operands are in the tiled layout: the k-step slab of a tile is 256 rows
    // x 64 bytes, contiguous.  Each slab is 1024 pieces of 16 bytes, two per lane.
    // A load into LDS puts lane l of a wave at LDS slot base + l, so the swizzle
    // is applied on the global side: slot s = 4 row + p' holds logical piece
    // p' ^ ((row >> 2) & 3) of that row.  The W_head tiles are zero past V; the
    // rows of the last F tile past the chunk hold stale values, which only reach
    // those rows' outputs, discarded below.
    constexpr int NL = G2_TV * 4 / G2_NT;   // loads per lane per operand and k-step
    const __amdgpu_buffer_rsrc_t ares =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Wt + (int64_t)vt * G2_TV * D), (short)0, G2_TV * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t bres =
        __builtin_amdgcn_make_buffer_rsrc((void*)(F + rt * G2_TR * D), (short)0, G2_TR * D * 2, 0x00020000);
    int voff[NL];   // byte offsets of this lane's pieces within a slab (same for both operands)
#pragma unroll
    for (int jj = 0; jj < NL; ++jj) {
        const int slot = (jj * G2_WAVES + w) * 64 + lane;
        const int row = slot >> 2, piece = (slot & 3) ^ ((row >> 2) & 3);
        voff[jj] = row * (G2_KS * 2) + 16 * piece;
    }
    auto issue_ks = [&](int ks, uint16_t* as, uint16_t* bs) {
#pragma unroll
        for (int jj = 0; jj < NL; ++jj) {
            const int base = (jj * G2_WAVES + w) * 64 * 8;  // element offset of this wave's 64 slots
            const int off = voff[jj] + ks * (G2_TV * G2_KS * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ares, (__attribute__((address_space(3))) void*)(as + base), 16, off,
                                                     0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(bres, (__attribute__((address_space(3))) void*)(bs + base), 16, off,
                                                     0, 0, 0);
        }
    };

    f32x16_t acc[G2_VB][G2_RB];
#pragma unroll
    for (int i = 0; i < G2_VB; ++i)
#pragma unroll
        for (int j = 0; j < G2_RB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    auto read_frags = [&](const uint16_t* as, const uint16_t* bs, int kk, uint4 (&a)[G2_VB], uint4 (&b)[G2_RB]) {
        const int piece = kk * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < G2_VB; ++i)
            a[i] = *reinterpret_cast<const uint4*>(&as[swz32(wv * 128 + i * 32 + (lane & 31), piece)]);
#pragma unroll
        for (int j = 0; j < G2_RB; ++j)
            b[j] = *reinterpret_cast<const uint4*>(&bs[swz32(wr * G2_WR + j * 32 + (lane & 31), piece)]);
    };
    // k-step ks works on stage ks % 4 (its second sub-step; the first one's
    // fragments were read during k-step ks - 1) and reads the first sub-step of
    // slab ks + 1 from stage (ks + 1) % 4, so it starts once slab ks + 1 has
    // landed: only the 2 NL loads of slab ks + 2 may be outstanding.  Past its
    // barrier every wave has finished k-step ks - 1, so stage (ks + 3) % 4 takes
    // slab ks + 3 (clamped to the last one: every k-step issues the same loads).
    const int nks = D / G2_KS;   // a multiple of 4: D is 256 or 512
    uint4 af[2][G2_VB], bfr[2][G2_RB];
    auto kstep = [&](int ks, const uint16_t* as, const uint16_t* bs, const uint16_t* as1, const uint16_t* bs1,
                     uint16_t* as_n, uint16_t* bs_n) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NL));
        // a barrier without the full memory wait that __syncthreads adds; the
        // memory clobber keeps LDS accesses on their side of it
        asm volatile("s_barrier" ::: "memory");
        issue_ks(min(ks + G2_STAGES - 1, nks - 1), as_n, bs_n);
        read_frags(as, bs, 1, af[1], bfr[1]);
#pragma unroll
        for (int i = 0; i < G2_VB; ++i)
#pragma unroll
            for (int j = 0; j < G2_RB; ++j) acc[i][j] = mfma32(af[0][i], bfr[0][j], acc[i][j]);
        read_frags(as1, bs1, 0, af[0], bfr[0]);   // past the last k-step: a stage of valid data, unused
#pragma unroll
        for (int i = 0; i < G2_VB; ++i)
#pragma unroll
            for (int j = 0; j < G2_RB; ++j) acc[i][j] = mfma32(af[1][i], bfr[1][j], acc[i][j]);
        // each sub-step's MFMAs interleaved with the fragment reads of the next
        // one, the loads spread between MFMAs (a wave issues in order: a burst of
        // loads waiting for the address unit would hold back the MFMAs behind it)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int q = 0; q < G2_VB + G2_RB; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
#pragma unroll
            for (int q = 0; q < NL; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, G2_VB * G2_RB - (G2_VB + G2_RB) - NL, 0);
        }
    };

    issue_ks(0, As0, Bs0);
    issue_ks(1, As1, Bs1);
    issue_ks(2, As2, Bs2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * NL));   // slab 0
    asm volatile("s_barrier" ::: "memory");
    read_frags(As0, Bs0, 0, af[0], bfr[0]);
    for (int ks = 0; ks < nks; ks += G2_STAGES) {
        kstep(ks, As0, Bs0, As1, Bs1, As3, Bs3);
        kstep(ks + 1, As1, Bs1, As2, Bs2, As0, Bs0);
        kstep(ks + 2, As2, Bs2, As3, Bs3, As1, Bs1);
        kstep(ks + 3, As3, Bs3, As0, Bs0, As2, Bs2);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // the clamped loads past the end

    // ---- epilogue: per row, log-sum-exp over this tile's vocabulary ---------
    // lane holds rows j = wr*G2_WR + rb*32 + lane%32, vocab v0 + wv*128 + vb*32 + drow(r, lane)
    const bool full = v0 + G2_TV <= V;  // uniform: no vocabulary bound to test
    const float C = offset[0];
    const bool fixed = C <= G2_FIXED_MAX;  // uniform
#pragma unroll
    for (int rb = 0; rb < G2_RB; ++rb) {
        const int lrow = wr * G2_WR + rb * 32 + (lane & 31);
        const int64_t row = r0 + lrow;
        if (!full) {  // last vocabulary tile: columns past V do not count
#pragma unroll
            for (int vb = 0; vb < G2_VB; ++vb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (v0 + wv * 128 + vb * 32 + drow(r, lane) >= V) acc[vb][rb][r] = -__builtin_inff();
        }
        // label logit first (the fixed-offset path below overwrites nothing, but
        // keep the capture next to the accumulators it reads)
        if (row < nrows) {
            const int64_t t = (g0 + row) % A.T;
            const int ii = A.labels[t] - (v0 + wv * 128);
            const bool mine = ii >= 0 && ii < 128 && (((ii >> 2) & 1) == (lane >> 5));
            if (__builtin_amdgcn_ballot_w64(mine)) {
                if (mine) {
                    const int vb = ii >> 5, i2 = ii & 31;
                    const int rr = (i2 & 3) + 4 * (i2 >> 3);
                    float val = 0.f;
#pragma unroll
                    for (int b = 0; b < G2_VB; ++b)
#pragma unroll
                        for (int r = 0; r < 16; ++r) val = (b == vb && r == rr) ? acc[b][rb][r] : val;
                    zy[row] = val;
                }
            }
        }
        float m;
        if (fixed) {
            m = C;
        } else {
            float m0 = -__builtin_inff(), m1 = -__builtin_inff();
#pragma unroll
            for (int vb = 0; vb < G2_VB; ++vb)
#pragma unroll
                for (int r = 0; r < 16; r += 4) {
                    m0 = fmaxf(m0, fmaxf(acc[vb][rb][r], acc[vb][rb][r + 1]));
                    m1 = fmaxf(m1, fmaxf(acc[vb][rb][r + 2], acc[vb][rb][r + 3]));
                }
            m = fmaxf(m0, m1);
            m = fmaxf(m, __shfl_xor(m, 32, 64));
        }
        const float ml2 = m * kLog2eF;
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int vb = 0; vb < G2_VB; ++vb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s4[r & 3] += __builtin_amdgcn_exp2f(fmaf(acc[vb][rb][r], kLog2eF, -ml2));
        float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        s += __shfl_xor(s, 32, 64);
        if (lane < 32) red[wv][lrow] = make_float2(m, s);
    }
    __syncthreads();
    for (int lr = tid; lr < G2_TR; lr += G2_NT) {
        const int64_t row = r0 + lr;
        if (row < nrows) {
            const float2 a = red[0][lr], b = red[1][lr];
            const float m = fmaxf(a.x, b.x);
            float s = 0.f;
            if (a.y > 0.f) s += a.y * __builtin_amdgcn_exp2f((a.x - m) * kLog2eF);
            if (b.y > 0.f) s += b.y * __builtin_amdgcn_exp2f((b.x - m) * kLog2eF);
            part[(int64_t)vt * nrows + row] = make_float2(m, s);
        }
    }
}

// CE[g0 + row] = max + log(sum) - z_y, combining the vocabulary tiles in order.
__global__ void __launch_bounds__(256) mlp_combine_kernel(int64_t g0, int64_t nrows, int nvt,
                                                          const float2* __restrict__ part,
                                                          const float* __restrict__ zy, float* __restrict__ ce) {
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (row >= nrows) return;
    float m = -__builtin_inff();
    for (int vt = 0; vt < nvt; ++vt) m = fmaxf(m, part[(int64_t)vt * nrows + row].x);
    float s = 0.f;
    for (int vt = 0; vt < nvt; ++vt) {
        const float2 p = part[(int64_t)vt * nrows + row];
        if (p.y > 0.f) s += p.y * __builtin_amdgcn_exp2f((p.x - m) * kLog2eF);
    }
    ce[g0 + row] = m + __logf(s) - zy[row];
}

// g_hat_t = -(1/(K sigma)) sum_i (CE0_t - CE_{t,i}) a_{t,i}, noise regenerated.
// One workgroup per token (token, draw and layer are then uniform, which keeps
// the first Philox rounds on the scalar unit); each thread owns channel quads.
__global__ void __launch_bounds__(256) mlp_reduce_kernel(MlpArgs A, const float* __restrict__ ce, float* __restrict__ ghat) {
    const int t = blockIdx.x;
    const int nq = A.n >> 2;
    const float c0 = ce[t];
    const uint32_t tok = A.tok0 + (uint32_t)t;
    const float scale = A.gscale * kSqrt2Ln2;  // the noise below is drawn divided by sqrt(2 ln 2)
    for (int q = threadIdx.x; q < nq; q += 256) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < A.K; ++i) {
            const float r = c0 - ce[(int64_t)A.T * (i + 1) + t];
            const f32x4 g = gauss4_unscaled_uniform(tok, (uint32_t)q, A.draw0 + (uint32_t)i, A.layer, A.k0, A.k1);
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = fmaf(r, g.v[c], acc[c]);
        }
        *reinterpret_cast<float4*>(ghat + (int64_t)t * A.n + 4 * q) =
            make_float4(acc[0] * scale, acc[1] * scale, acc[2] * scale, acc[3] * scale);
    }
    if (threadIdx.x == 0 && A.rewards)
        for (int i = 0; i < A.K; ++i) A.rewards[(int64_t)i * A.T + t] = c0 - ce[(int64_t)A.T * (i + 1) + t];
}

// ---------------------------------------------------------------------------
// The GELU operand M of one chunk (bf16 rows of n) is kept to at most 2 GiB and F
// (bf16 rows of d) to 512 MiB; a chunk is a whole number of token blocks.  A block
// of T rows whose M exceeds 1 GiB runs the chunk through mlp_gemm1_kernel instead
// (no M is stored).
static bool mlp_m_path(int64_t T, int64_t n) { return T * n * 2 <= ((int64_t)1 << 30); }

size_t mlp_chunk_rows(int64_t T, int64_t K, int64_t d, int64_t n) {
    const int64_t total = T * (K + 1);
    int64_t cap = ((int64_t)512 << 20) / (2 * d);
    if (mlp_m_path(T, n)) cap = std::min<int64_t>(cap, ((int64_t)2 << 30) / (2 * n));
    cap = cap / T * T;
    if (cap < T) cap = T;
    return (size_t)(total < cap ? total : cap);
}

static size_t al256(size_t v) { return (v + 255) / 256 * 256; }

MlpLayout mlp_layout(int64_t T, int64_t d, int64_t n, int64_t V, int64_t K) {
    MlpLayout L{};
    L.chunk = (int64_t)mlp_chunk_rows(T, K, d, n);
    L.nvt = (int)((V + G2_TV - 1) / G2_TV);
    size_t off = 0;
    L.off_f = off;    off += al256((size_t)((L.chunk + FT_ROWS - 1) / FT_ROWS) * FT_ROWS * d * 2);
    L.off_wt = off;   off += al256((size_t)L.nvt * G2_TV * d * 2);
    L.off_part = off; off += al256((size_t)L.chunk * L.nvt * sizeof(float2));
    L.off_zy = off;   off += al256((size_t)L.chunk * sizeof(float));
    L.off_wnorm = off; off += al256((size_t)((V + 255) / 256 + 1) * sizeof(float));
    L.off_ce = off;   off += al256((size_t)T * (K + 1) * sizeof(float));
    L.off_ghat = off; off += al256((size_t)T * n * sizeof(float));
    L.off_w2f = off;  off += al256((size_t)d * n * 2);
    L.off_phi = off;  off += 2 * al256((size_t)T * n * sizeof(float));
    L.off_m = off;    off += mlp_m_path(T, n) ? al256((size_t)L.chunk * n * 2) : 0;
    L.off_outer = off;
    off += outer_workspace_bytes(T, n, d);
    L.total = off;
    return L;
}

hipError_t launch_mlp(const MlpArgs& A, const MlpLayout& L, unsigned char* ws, float* ghat_user, float* grad_w,
                      hipStream_t stream) {
    uint16_t* F = reinterpret_cast<uint16_t*>(ws + L.off_f);
    float2* part = reinterpret_cast<float2*>(ws + L.off_part);
    float* zy = reinterpret_cast<float*>(ws + L.off_zy);
    float* wnorm = reinterpret_cast<float*>(ws + L.off_wnorm);
    const int nwb = (A.V + 255) / 256;
    float* offset = wnorm + nwb;
    float* ce = reinterpret_cast<float*>(ws + L.off_ce);
    float* ghat = ghat_user ? ghat_user : reinterpret_cast<float*>(ws + L.off_ghat);
    const int64_t total = (int64_t)A.T * (A.K + 1);
    hipError_t e = hipSuccess;
    hipLaunchKernelGGL(mlp_wnorm_kernel, dim3((unsigned)nwb), dim3(256), 0, stream, A.w_head, A.V, A.d, wnorm);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(mlp_wnorm_final_kernel, dim3(1), dim3(256), 0, stream, wnorm, nwb, A.d, offset);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    uint16_t* Wt = reinterpret_cast<uint16_t*>(ws + L.off_wt);
    const int64_t wpieces = (int64_t)L.nvt * G2_TV * A.d / 8;
    hipLaunchKernelGGL(mlp_wtile_kernel, dim3((unsigned)((wpieces + 255) / 256)), dim3(256), 0, stream, A.w_head, A.V,
                       A.d, L.nvt, Wt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // small sigma: M = bf16(GELU(h + sigma a)) of every row from the cached Phi(h),
    // phi(h) by the series (mlp_gelu_rows_kernel), then F = bf16(LN(x + W2 M)) on
    // MFMA (mlp_w2ln_kernel); larger sigma (or an M block beyond 1 GiB): both in
    // mlp_gemm1_kernel with the library erf
    const bool taylor = mlp_taylor_ok(A.sigma) && mlp_m_path(A.T, A.n);
    const uint16_t* w2f = reinterpret_cast<const uint16_t*>(ws + L.off_w2f);
    float* Pt = reinterpret_cast<float*>(ws + L.off_phi);
    float* pt = reinterpret_cast<float*>(ws + L.off_phi + al256((size_t)A.T * A.n * sizeof(float)));
    uint16_t* M = reinterpret_cast<uint16_t*>(ws + L.off_m);
    const float sig_u = (float)((double)A.sigma * (double)kSqrt2Ln2);
    if (taylor) {
        const int64_t cnt = (int64_t)A.T * A.n;
        hipLaunchKernelGGL(mlp_phi_kernel, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, stream, A.h, cnt, Pt,
                           pt);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int64_t pieces = (int64_t)(A.d / 32) * (A.n / 16) * 64;
        hipLaunchKernelGGL(mlp_w2frag_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, stream, A.w2, A.d,
                           A.n, const_cast<uint16_t*>(w2f));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    auto gemm1_direct = [&](int64_t g0, int64_t nrows) {
        const unsigned b1 = (unsigned)((nrows + G1_ROWS - 1) / G1_ROWS);
        if (A.d == 512)
            hipLaunchKernelGGL(mlp_gemm1_kernel<512>, dim3(b1), dim3(G1_NT), 0, stream, A, g0, nrows, F);
        else
            hipLaunchKernelGGL(mlp_gemm1_kernel<256>, dim3(b1), dim3(G1_NT), 0, stream, A, g0, nrows, F);
        return hipGetLastError();
    };
    // the GELU rows of slots [first_slot, first_slot + nslots) of the chunk at g0;
    // the clean slot (zero noise) with s = 0
    auto gelu_rows = [&](int64_t g0, int first_slot, int nslots, float s) {
        const int64_t waves = (int64_t)A.T * ((A.n + 255) / 256);
        hipLaunchKernelGGL(mlp_gelu_rows_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(GA_NT), 0, stream, A, s, Pt, pt,
                           g0, first_slot, nslots, M);
        return hipGetLastError();
    };
    auto w2ln = [&](int64_t g0, int64_t nrows) {
        const unsigned b = (unsigned)((nrows + GB_ROWS - 1) / GB_ROWS);
        const bool fast = A.n % (GB_STAGES * GB_KS) == 0;
        if (A.d == 512 && fast)
            hipLaunchKernelGGL((mlp_w2ln_kernel<512, true>), dim3(b), dim3(GB_NT), 0, stream, A, w2f, M, g0, nrows, F);
        else if (A.d == 512)
            hipLaunchKernelGGL((mlp_w2ln_kernel<512, false>), dim3(b), dim3(GB_NT), 0, stream, A, w2f, M, g0, nrows, F);
        else if (fast)
            hipLaunchKernelGGL((mlp_w2ln_kernel<256, true>), dim3(b), dim3(GB_NT), 0, stream, A, w2f, M, g0, nrows, F);
        else
            hipLaunchKernelGGL((mlp_w2ln_kernel<256, false>), dim3(b), dim3(GB_NT), 0, stream, A, w2f, M, g0, nrows, F);
        return hipGetLastError();
    };
    for (int64_t g0 = 0; g0 < total; g0 += L.chunk) {
        const int64_t nrows = (total - g0) < L.chunk ? (total - g0) : L.chunk;
        bool timed = false;
        if ((e = launch_timer_begin(kTimedMlpGemm1, stream, timed)) != hipSuccess) return e;
        if (!taylor) {
            if ((e = gemm1_direct(g0, nrows)) != hipSuccess) return e;
        } else {
            // a chunk is a whole number of slots of T rows; slot 0 of the first is the clean rows
            const int first = g0 == 0 ? 1 : 0;
            const int nslots = (int)(nrows / A.T) - first;
            if (first && (e = gelu_rows(0, 0, 1, 0.0f)) != hipSuccess) return e;
            if (nslots > 0 && (e = gelu_rows(g0, first, nslots, sig_u)) != hipSuccess) return e;
            if ((e = w2ln(g0, nrows)) != hipSuccess) return e;
        }
        if ((e = launch_timer_end(kTimedMlpGemm1, stream, timed)) != hipSuccess) return e;
        if (A.gemm1_event && (e = hipEventRecord(A.gemm1_event, stream)) != hipSuccess) return e;
        const int64_t nrt = (nrows + G2_TR - 1) / G2_TR;
        if ((e = launch_timer_begin(kTimedMlpGemm2, stream, timed)) != hipSuccess) return e;
        const int64_t nb2 = (L.nvt & 3) == 0 ? 2 * L.nvt * ((nrt + 1) / 2) : nrt * L.nvt;
        hipLaunchKernelGGL(mlp_gemm2_kernel, dim3((unsigned)nb2), dim3(G2_NT), 0, stream, A, g0, nrows, nrt, L.nvt, Wt,
                           F, part, zy, offset);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = launch_timer_end(kTimedMlpGemm2, stream, timed)) != hipSuccess) return e;
        if (A.gemm2_event && (e = hipEventRecord(A.gemm2_event, stream)) != hipSuccess) return e;
        hipLaunchKernelGGL(mlp_combine_kernel, dim3((unsigned)((nrows + 255) / 256)), dim3(256), 0, stream, g0, nrows,
                           L.nvt, part, zy, ce);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(mlp_reduce_kernel, dim3((unsigned)A.T), dim3(256), 0, stream, A, ce, ghat);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (A.stage_event && (e = hipEventRecord(A.stage_event, stream)) != hipSuccess) return e;
    return launch_outer(ghat, A.u, A.T, A.n, A.d, grad_w, ws + L.off_outer, L.total - L.off_outer, stream);
}

}  // namespace dust
