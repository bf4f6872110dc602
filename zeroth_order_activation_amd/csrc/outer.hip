// Weight-gradient outer product  grad_w = ghat^T x = sum_t ghat_t x_t^T
// (TL;DR page, section 1, equation for G_W).
//
// Two paths.  Small products use the fp32 MFMA directly (below).  Large ones
// (>= 4 GFLOP) split both fp32 operands into bf16 pairs v = hi + lo (hi =
// bf16(v), lo = bf16(v - hi), so |v - hi - lo| <= 2^-17 |v|) and accumulate
// hi*hi + hi*lo + lo*hi on the bf16 MFMA in fp32: each product is then within
// about 3 * 2^-17 of the fp32 product, at 3/16 of the fp32-MFMA time.  The bf16
// MFMA wants 8 consecutive tokens per lane, so a transpose pass first writes
// the pairs token-contiguous ([column][token], token count padded to 64).
//
// The contraction runs over tokens, which is the row index of both operands,
// so a [BK x BM] slab of ghat and a [BK x BN] slab of x are each contiguous
// row pieces: both are staged through LDS exactly as they lie in memory and
// read back as MFMA operands with no transpose.  v_mfma_f32_32x32x2_f32
// takes A[i][k] from lane i + 32k and B[k][j] from lane j + 32k, i.e. one LDS
// row segment of 32 floats per half-wave.  Token ranges are split over
// workgroups when the output has too few tiles to fill the 256 CUs; partial
// sums then go to the workspace and are added in a fixed order (no atomics,
// bitwise deterministic).
#include "dust_device.hpp"
#include "dust_internal.hpp"

namespace dust {

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {
constexpr int BM = 128, BN = 128, BK = 16, NTH = 256;

constexpr int XM = 128, XN = 128, XK = 32;  // bf16x3 tiles; 64-byte LDS rows, xor-swizzled pieces

// piece p (16 bytes) of LDS row r lives at piece p ^ ((r >> 2) & 3): conflict-free
// for both the coalesced row writes and the MFMA fragment reads.
__device__ __forceinline__ int xswz(int row, int piece) { return row * XK + ((piece ^ ((row >> 2) & 3)) << 3); }
constexpr double kSplitMinFlop = 4e9;

struct OuterPlan {
    bool x3;         // bf16x3 path
    int splits;
    int64_t tchunk;  // tokens per split
    int64_t Tp;      // padded token count of the transposed pairs (x3)
    size_t off_ah, off_al, off_bh, off_bl, off_part, total;
};

OuterPlan plan_outer(int64_t T, int64_t n, int64_t d) {
    OuterPlan p{};
    p.x3 = 2.0 * (double)T * (double)n * (double)d >= kSplitMinFlop;
    const int64_t bm = p.x3 ? XM : BM, bn = p.x3 ? XN : BN, bk = p.x3 ? 64 : BK;
    p.Tp = p.x3 ? (T + 63) / 64 * 64 : T;
    const int64_t tiles = ((n + bm - 1) / bm) * ((d + bn - 1) / bn);
    int64_t s = (512 + tiles - 1) / tiles;
    const int64_t smax = (p.Tp + 255) / 256;  // at least 256 tokens per split
    if (s > smax) s = smax;
    if (s < 1) s = 1;
    int64_t chunk = (p.Tp + s - 1) / s;
    chunk = (chunk + bk - 1) / bk * bk;
    s = (p.Tp + chunk - 1) / chunk;
    p.splits = (int)s;
    p.tchunk = chunk;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) / 256 * 256; return o; };
    if (p.x3) {
        p.off_ah = take((size_t)n * p.Tp * 2);
        p.off_al = take((size_t)n * p.Tp * 2);
        p.off_bh = take((size_t)d * p.Tp * 2);
        p.off_bl = take((size_t)d * p.Tp * 2);
    }
    p.off_part = take(p.splits > 1 ? (size_t)p.splits * n * d * sizeof(float) : 0);
    p.total = off;
    return p;
}

__device__ __forceinline__ void load_slab(const float* __restrict__ P, int64_t ld, int64_t t, int64_t te,
                                          int64_t c, int64_t cols, bool vec, float (&r)[4]) {
    if (t < te && vec && c + 3 < cols) {
        const float4 v = *reinterpret_cast<const float4*>(P + t * ld + c);
        r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = (t < te && c + e < cols) ? P[t * ld + c + e] : 0.f;
    }
}
}  // namespace

__global__ void __launch_bounds__(NTH) outer_f32_kernel(const float* __restrict__ G, const float* __restrict__ X,
                                                        int64_t T, int64_t M, int64_t N, int64_t tchunk,
                                                        float* __restrict__ out) {
    __shared__ __align__(16) float As[BK][BM];
    __shared__ __align__(16) float Bs[BK][BN];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w & 1, wn = w >> 1;
    const int64_t m0 = (int64_t)blockIdx.x * BM, n0 = (int64_t)blockIdx.y * BN;
    const int64_t tb = (int64_t)blockIdx.z * tchunk;
    const int64_t te = (tb + tchunk < T) ? tb + tchunk : T;
    const bool vecA = (M & 3) == 0, vecB = (N & 3) == 0;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    for (int64_t kb = tb; kb < te; kb += BK) {
        float ra[2][4], rb[2][4];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int f = tid + r * NTH;
            const int row = f >> 5, c4 = (f & 31) * 4;
            load_slab(G, M, kb + row, te, m0 + c4, M, vecA, ra[r]);
            load_slab(X, N, kb + row, te, n0 + c4, N, vecB, rb[r]);
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int f = tid + r * NTH;
            const int row = f >> 5, c4 = (f & 31) * 4;
            *reinterpret_cast<float4*>(&As[row][c4]) = make_float4(ra[r][0], ra[r][1], ra[r][2], ra[r][3]);
            *reinterpret_cast<float4*>(&Bs[row][c4]) = make_float4(rb[r][0], rb[r][1], rb[r][2], rb[r][3]);
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; kk += 2) {
            const int k = kk + (lane >> 5);
            const float a0 = As[k][wm * 64 + (lane & 31)];
            const float a1 = As[k][wm * 64 + 32 + (lane & 31)];
            const float b0 = Bs[k][wn * 64 + (lane & 31)];
            const float b1 = Bs[k][wn * 64 + 32 + (lane & 31)];
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
        }
    }

    // D[i][j] of a 32x32 block sits in lane j + 32*((i/4)%2), register (i%4) + 4*(i/8).
    float* o = out + (int64_t)blockIdx.z * M * N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * 64 + i * 32 + (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5);
                const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
                if (row < M && col < N) o[row * N + col] = acc[i][j][r];
            }
}

__global__ void __launch_bounds__(256) sum_splits_kernel(const float* __restrict__ part, int splits, int64_t count,
                                                         float* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= count) return;
    float s = part[i];
    for (int k = 1; k < splits; ++k) s += part[(int64_t)k * count + i];
    out[i] = s;
}

// ---------------------------------------------------------------------------
// bf16x3 path
// ---------------------------------------------------------------------------
// src [rows, cols] fp32 -> hi, lo [cols, Tp] bf16 (rows >= nrows read as 0).
// 64 x 64 tiles through LDS: coalesced 256-byte row reads, 128-byte row writes.
__global__ void __launch_bounds__(256) split_transpose_kernel(const float* __restrict__ src, int64_t nrows, int64_t ncols,
                                                              int64_t Tp, uint16_t* __restrict__ hi,
                                                              uint16_t* __restrict__ lo) {
    constexpr int TS = 64, LS = TS + 8;
    __shared__ __align__(16) uint16_t th[TS * LS];
    __shared__ __align__(16) uint16_t tl[TS * LS];
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * TS, c0 = (int64_t)blockIdx.y * TS;
    const bool vec = (ncols & 3) == 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = tid / 16 + 16 * r;
        const int col = 4 * (tid % 16);
        const int64_t t = t0 + row, c = c0 + col;
        float v[4];
        if (t < nrows && vec && c + 3 < ncols) {
            const float4 f = *reinterpret_cast<const float4*>(src + t * ncols + c);
            v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (t < nrows && c + e < ncols) ? src[t * ncols + c + e] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint16_t h = f32_to_bf16_rne(v[e]);
            th[(col + e) * LS + row] = h;
            tl[(col + e) * LS + row] = f32_to_bf16_rne(v[e] - bf16_to_f32(h));
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int idx = tid + 256 * r;  // 64 columns x 8 pieces of 8 tokens
        const int col = idx >> 3, piece = idx & 7;
        const int64_t c = c0 + col;
        if (c >= ncols) continue;
        const uint4 vh = *reinterpret_cast<const uint4*>(&th[col * LS + 8 * piece]);
        const uint4 vl = *reinterpret_cast<const uint4*>(&tl[col * LS + 8 * piece]);
        *reinterpret_cast<uint4*>(hi + c * Tp + t0 + 8 * piece) = vh;
        *reinterpret_cast<uint4*>(lo + c * Tp + t0 + 8 * piece) = vl;
    }
}

typedef __bf16 bf16x8_o __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma_bf16(const uint4& a, const uint4& b, const f32x16& c) {
    bf16x8_o av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
}

// out[m][n] = sum_k Ah[m][k] Bh[n][k] + Ah Bl + Al Bh over k in this split.
// 128 x 128 tiles, 4 waves of 64 x 64; 32-token k-steps staged through LDS
// (register prefetch of the next step).  v_mfma_f32_32x32x16_bf16: A[i][k] in
// lane i + 32*(k/8), B[k][j] in lane j + 32*(k/8), 8 consecutive k per lane.
__global__ void __launch_bounds__(256) outer_bf16x3_kernel(const uint16_t* __restrict__ Ah, const uint16_t* __restrict__ Al,
                                                           const uint16_t* __restrict__ Bh, const uint16_t* __restrict__ Bl,
                                                           int64_t M, int64_t N, int64_t Tp, int64_t tchunk,
                                                           float* __restrict__ out) {
    __shared__ __align__(16) uint16_t S[4][XM * XK];  // Ah, Al, Bh, Bl
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w & 1, wn = w >> 1;
    // XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs, so
    // block b runs on XCD b % 8.  All N-tiles of one M-tile go to the same XCD
    // (consecutive blocks of that XCD), whose L2 then serves the shared ghat
    // slabs to all of them instead of each refetching from HBM.
    const int64_t nmt = (M + XM - 1) / XM, nnt = (N + XN - 1) / XN;
    const int64_t b = blockIdx.x, xcd = b % 8, sq = b / 8;
    const int64_t mt = (sq / nnt) * 8 + xcd, nt = sq % nnt;
    if (mt >= nmt) return;
    const int64_t m0 = mt * XM, n0 = nt * XN;
    const int64_t kb0 = (int64_t)blockIdx.z * tchunk;
    const int64_t ke = (kb0 + tchunk < Tp) ? kb0 + tchunk : Tp;
    const uint16_t* src[4] = {Ah, Al, Bh, Bl};

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // loads: per operand 128 rows x 32 tokens = 512 pieces of 16 bytes -> 2 per thread
    auto load = [&](int64_t kb, uint4 (&reg)[4][2]) {
#pragma unroll
        for (int o = 0; o < 4; ++o)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int pi = tid + 256 * jj;
                const int row = pi >> 2, piece = pi & 3;
                const int64_t grow = (o < 2 ? m0 : n0) + row;
                const int64_t lim = o < 2 ? M : N;
                reg[o][jj] = grow < lim ? *reinterpret_cast<const uint4*>(src[o] + grow * Tp + kb + 8 * piece)
                                        : make_uint4(0, 0, 0, 0);
            }
    };
    uint4 reg[4][2];
    load(kb0, reg);
    for (int64_t kb = kb0; kb < ke; kb += XK) {
        __syncthreads();
#pragma unroll
        for (int o = 0; o < 4; ++o)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int pi = tid + 256 * jj;
                const int row = pi >> 2, piece = pi & 3;
                *reinterpret_cast<uint4*>(&S[o][xswz(row, piece)]) = reg[o][jj];
            }
        __syncthreads();
        if (kb + XK < ke) load(kb + XK, reg);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            uint4 ah[2], al[2], bh[2], bl[2];
            const int piece = kk * 2 + (lane >> 5);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ra = xswz(wm * 64 + i * 32 + (lane & 31), piece);
                const int rb = xswz(wn * 64 + i * 32 + (lane & 31), piece);
                ah[i] = *reinterpret_cast<const uint4*>(&S[0][ra]);
                al[i] = *reinterpret_cast<const uint4*>(&S[1][ra]);
                bh[i] = *reinterpret_cast<const uint4*>(&S[2][rb]);
                bl[i] = *reinterpret_cast<const uint4*>(&S[3][rb]);
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
    }

    float* o = out + (int64_t)blockIdx.z * M * N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * 64 + i * 32 + (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5);
                const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
                if (row < M && col < N) o[row * N + col] = acc[i][j][r];
            }
}

size_t outer_workspace_bytes(int64_t T, int64_t n, int64_t d) { return plan_outer(T, n, d).total; }

hipError_t launch_outer(const float* ghat, const float* x, int64_t T, int64_t n, int64_t d, float* grad_w,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const OuterPlan p = plan_outer(T, n, d);
    if (p.total > 0 && (workspace == nullptr || workspace_bytes < p.total)) return hipErrorInvalidValue;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    float* part = p.splits > 1 ? reinterpret_cast<float*>(ws + p.off_part) : grad_w;
    hipError_t e;
    if (p.x3) {
        uint16_t* ah = reinterpret_cast<uint16_t*>(ws + p.off_ah);
        uint16_t* al = reinterpret_cast<uint16_t*>(ws + p.off_al);
        uint16_t* bh = reinterpret_cast<uint16_t*>(ws + p.off_bh);
        uint16_t* bl = reinterpret_cast<uint16_t*>(ws + p.off_bl);
        hipLaunchKernelGGL(split_transpose_kernel, dim3((unsigned)(p.Tp / 64), (unsigned)((n + 63) / 64)), dim3(256), 0,
                           stream, ghat, T, n, p.Tp, ah, al);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(split_transpose_kernel, dim3((unsigned)(p.Tp / 64), (unsigned)((d + 63) / 64)), dim3(256), 0,
                           stream, x, T, d, p.Tp, bh, bl);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int64_t nmt8 = ((n + XM - 1) / XM + 7) / 8 * 8;  // M-tiles rounded up to whole XCD groups
        const dim3 grid((unsigned)(nmt8 * ((d + XN - 1) / XN)), 1, (unsigned)p.splits);
        hipLaunchKernelGGL(outer_bf16x3_kernel, grid, dim3(256), 0, stream, ah, al, bh, bl, n, d, p.Tp, p.tchunk, part);
    } else {
        const dim3 grid((unsigned)((n + BM - 1) / BM), (unsigned)((d + BN - 1) / BN), (unsigned)p.splits);
        hipLaunchKernelGGL(outer_f32_kernel, grid, dim3(NTH), 0, stream, ghat, x, T, n, d, p.tchunk, part);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.splits == 1) return hipSuccess;
    const int64_t count = n * d;
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream, part, p.splits,
                       count, grad_w);
    return hipGetLastError();
}

}  // namespace dust
