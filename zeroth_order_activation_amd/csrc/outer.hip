// Weight-gradient outer product  grad_w = ghat^T x = sum_t ghat_t x_t^T
// (TL;DR page, section 1, equation for G_W).
//
// Two paths.  Small products use the fp32 MFMA directly (below).  Large ones
// (>= 4 GFLOP) split both fp32 operands into bf16 pairs v = hi + lo (hi =
// bf16(v), lo = bf16(v - hi), so |v - hi - lo| <= 2^-17 |v|) and accumulate
// lo*hi + hi*lo + hi*hi on the bf16 MFMA in fp32: each product is then within
// about 3 * 2^-17 of the fp32 product, at 3/16 of the fp32-MFMA time.  The
// pairs keep the operands' own token-major layout ([token][column], row pitch
// padded to whole 256-column tiles, token count to whole 32-token k-steps,
// padding zero); the bf16 MFMA wants 8 consecutive tokens per lane, which the
// transposing LDS read (ds_read_b64_tr_b16) delivers from a token-major tile.
//
// fp32 path: the contraction runs over tokens, which is the row index of both
// operands, so a [BK x BM] slab of ghat and a [BK x BN] slab of x are each
// contiguous row pieces: both are staged through LDS exactly as they lie in
// memory and read back as MFMA operands with no transpose.
// v_mfma_f32_32x32x2_f32 takes A[i][k] from lane i + 32k and B[k][j] from lane
// j + 32k, i.e. one LDS row segment of 32 floats per half-wave.
//
// Token ranges are split over workgroups when the output has too few tiles to
// fill the 256 CUs; partial sums then go to the workspace and are added in a
// fixed order (no atomics, bitwise deterministic).
#include <algorithm>

#include "dust_device.hpp"
#include "dust_internal.hpp"
#include "launch_events.hpp"

namespace dust {

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {
constexpr int BM = 128, BN = 128, BK = 16, NTH = 256;

// bf16x3 tiles: 256 x 256 outputs per workgroup (8 waves of 128 x 64), 32-token
// k-steps.  LDS rows are 256 columns (32 pieces of 16 bytes, 512 bytes: every
// row starts on the same bank); piece p of row r is stored at piece
// p ^ (4 (r & 3)).  Half a wave of transposing reads touches four consecutive
// rows (r & 3 = 0..3) at the same four pieces, which the swizzle moves into
// four different quarters of the 64 banks.
constexpr int YT = 256, YK = 32, YWAVES = 8, YNT = 64 * YWAVES;
__device__ __forceinline__ int yswz(int row, int piece) { return row * YT + ((piece ^ ((row & 3) << 2)) << 3); }
// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (expcnt and lgkmcnt left unconstrained)
constexpr int vmcnt_imm_o(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr double kSplitMinFlop = 4e9;

struct OuterPlan {
    bool x3;         // bf16x3 path
    int splits;
    int64_t tchunk;  // tokens per split
    // bf16x3, one split: when the tiles leave a last round of workgroups mostly idle, the
    // main launch takes the M-tiles [0, mA) (whole rounds) and the rest run as a second
    // launch with their token range split tsplits ways (partial sums, then summed)
    int64_t mA;
    int tsplits;
    int64_t tchunk_t;
    int64_t Tp;      // padded token count of the pairs (x3)
    int64_t Mp, Np;  // padded row pitches of the ghat and x pairs (x3)
    size_t off_ah, off_al, off_bh, off_bl, off_part, off_tail, total;
};

constexpr int64_t kOuterCUs = 256;  // workgroups of the bf16x3 kernel resident at once (one per CU)

OuterPlan plan_outer(int64_t T, int64_t n, int64_t d) {
    OuterPlan p{};
    p.x3 = 2.0 * (double)T * (double)n * (double)d >= kSplitMinFlop;
    const int64_t bm = p.x3 ? YT : BM, bn = p.x3 ? YT : BN, bk = p.x3 ? YK : BK;
    p.Tp = p.x3 ? (T + YK - 1) / YK * YK : T;
    p.Mp = p.x3 ? (n + YT - 1) / YT * YT : n;
    p.Np = p.x3 ? (d + YT - 1) / YT * YT : d;
    const int64_t tiles = ((n + bm - 1) / bm) * ((d + bn - 1) / bn);
    int64_t s = (512 + tiles - 1) / tiles;
    // at least 256 tokens per split; 64 when the output has few tiles (short inputs)
    const int64_t minsplit = tiles < 64 ? 64 : 256;
    const int64_t smax = (p.Tp + minsplit - 1) / minsplit;
    if (s > smax) s = smax;
    if (s < 1) s = 1;
    int64_t chunk = (p.Tp + s - 1) / s;
    chunk = (chunk + bk - 1) / bk * bk;
    s = (p.Tp + chunk - 1) / chunk;
    p.splits = (int)s;
    p.tchunk = chunk;
    const int64_t nmt = (n + bm - 1) / bm, nnt = (d + bn - 1) / bn;
    p.mA = nmt;
    p.tsplits = 1;
    p.tchunk_t = p.Tp;
    if (p.x3 && p.splits == 1 && tiles > kOuterCUs && tiles % kOuterCUs != 0 &&
        tiles % kOuterCUs <= kOuterCUs / 2) {
        const int64_t mA = (tiles / kOuterCUs) * kOuterCUs / nnt / 8 * 8;  // whole rounds, whole XCD groups
        const int64_t tail = (nmt - mA) * nnt;
        int64_t ts = std::min<int64_t>((kOuterCUs + tail - 1) / tail, (p.Tp + 255) / 256);
        if (mA > 0 && ts > 1) {
            int64_t tc = ((p.Tp + ts - 1) / ts + YK - 1) / YK * YK;
            ts = (p.Tp + tc - 1) / tc;
            p.mA = mA;
            p.tsplits = (int)ts;
            p.tchunk_t = tc;
        }
    }
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) / 256 * 256; return o; };
    if (p.x3) {
        p.off_ah = take((size_t)p.Mp * p.Tp * 2);
        p.off_al = take((size_t)p.Mp * p.Tp * 2);
        p.off_bh = take((size_t)p.Np * p.Tp * 2);
        p.off_bl = take((size_t)p.Np * p.Tp * 2);
    }
    p.off_part = take(p.splits > 1 ? (size_t)p.splits * n * d * sizeof(float) : 0);
    p.off_tail = take(p.tsplits > 1 ? (size_t)p.tsplits * (n - p.mA * bm) * d * sizeof(float) : 0);
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
typedef __bf16 bf16x2_o __attribute__((ext_vector_type(2)));
typedef float f32x2_o __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16_pair(float a, float b) {  // round to nearest even, a low
    const f32x2_o v = {a, b};
    const bf16x2_o h = __builtin_convertvector(v, bf16x2_o);
    uint32_t u;
    __builtin_memcpy(&u, &h, 4);
    return u;
}

// src [rows, cols] fp32 -> hi, lo [Tp, ldp] bf16, same (token-major) layout,
// zero past rows x cols.  One thread per 8 columns: 16-byte stores.
__global__ void __launch_bounds__(256) split_pairs_kernel(const float* __restrict__ src, int64_t nrows, int64_t ncols,
                                                          int64_t Tp, int64_t ldp, uint16_t* __restrict__ hi,
                                                          uint16_t* __restrict__ lo) {
    const int64_t per_row = ldp / 8;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= Tp * per_row) return;
    const int64_t t = i / per_row, c = (i % per_row) * 8;
    float v[8];
    if (t < nrows && c + 8 <= ncols && (ncols & 3) == 0) {
        const float4 a = *reinterpret_cast<const float4*>(src + t * ncols + c);
        const float4 b = *reinterpret_cast<const float4*>(src + t * ncols + c + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (t < nrows && c + e < ncols) ? src[t * ncols + c + e] : 0.f;
    }
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = pack_bf16_pair(v[2 * e], v[2 * e + 1]);
        const float h0 = __uint_as_float(h[e] << 16), h1 = __uint_as_float(h[e] & 0xFFFF0000u);
        l[e] = pack_bf16_pair(v[2 * e] - h0, v[2 * e + 1] - h1);
    }
    *reinterpret_cast<uint4*>(hi + t * ldp + c) = make_uint4(h[0], h[1], h[2], h[3]);
    *reinterpret_cast<uint4*>(lo + t * ldp + c) = make_uint4(l[0], l[1], l[2], l[3]);
}

typedef __bf16 bf16x8_o __attribute__((ext_vector_type(8)));
typedef short i16x4_o __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma_bf16(const uint4& a, const uint4& b, const f32x16& c) {
    bf16x8_o av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
}

// MFMA fragment of a token-major LDS tile: 32 columns from c0, tokens
// 16 kk .. 16 kk + 15.  v_mfma_f32_32x32x16_bf16 wants column (lane % 32),
// tokens 8 (lane / 32) .. + 7 in each lane.  The transposing read gives lane
// 4a + b of a 16-lane group element b of the 8-byte chunks read by lanes a,
// 4 + a, 8 + a, 12 + a (checked on the device); so lane 4e + a of group g
// points at token row 8 (g / 2) + e (+ 16 kk, + 4 for the second read),
// columns c0 + 16 (g % 2) + 4a.  Every term but c0 is either a per-lane
// constant or a compile-time offset, so each column block needs one lane
// offset (tr_lane_off) and the reads use immediate offsets.
__device__ __forceinline__ int tr_lane_off(int c0, int lane) {
    const int g = lane >> 4, e = (lane >> 2) & 3, a = lane & 3;
    const int col = c0 + 16 * (g & 1) + 4 * a;
    return yswz(8 * (g >> 1) + e, col >> 3) + (col & 7);  // rows 8(g/2)+e: (row & 3) = e
}
__device__ __forceinline__ uint4 tr_frag(const uint16_t* p) {  // p = tile + lane offset + 16 kk rows
    uint32_t u[4];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const i16x4_o v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_o*)(p + 4 * r * YT));
        __builtin_memcpy(&u[2 * r], &v, 8);
    }
    return make_uint4(u[0], u[1], u[2], u[3]);
}

// out[m][n] = sum_k Ah[k][m] Bh[k][n] + Ah Bl + Al Bh over the tokens k of this
// split.  256 x 256 tiles, 8 waves of 128 (m) x 64 (n).  The four [16 x 256] pair
// tiles of each 16-token k-step go straight from global memory into a four-stage
// LDS ring (buffer loads into LDS; the swizzle is applied on the global side,
// since such a load puts lane l at slot base + l), three k-steps ahead; the
// fragments of k-step ks + 1 are read while k-step ks's MFMAs issue.
constexpr int YK2 = 16, PL2 = YK2 * YT;   // tokens per k-step; elements of one plane of a stage

struct PairFrags {
    uint4 ah[4], al[4], bh[2], bl[2];
};

__global__ void __launch_bounds__(YNT, 1) outer_x3_kernel(const uint16_t* __restrict__ Ah, const uint16_t* __restrict__ Al,
                                                         const uint16_t* __restrict__ Bh, const uint16_t* __restrict__ Bl,
                                                         int64_t M, int64_t N, int64_t Mp, int64_t Np, int64_t Tp,
                                                         int64_t tchunk, float* __restrict__ out, int64_t mt0,
                                                         int64_t zs, int64_t orow0) {
    // the ring stages as separate LDS objects ([plane][token][column], 32 KB each):
    // reads of one provably do not alias loads in flight into another
    __shared__ __align__(16) uint16_t S0[4 * PL2], S1[4 * PL2], S2[4 * PL2], S3[4 * PL2];
    // the wave index as a scalar: the loads into LDS take M0 from scalar arithmetic
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w & 1, wn = w >> 1;
    // XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs, so
    // block b runs on XCD b % 8.  All N-tiles of one M-tile go to the same XCD
    // (consecutive blocks of that XCD), whose L2 then serves the shared ghat
    // tiles to all of them instead of each refetching from HBM.
    const int64_t nmt = (M + YT - 1) / YT, nnt = (N + YT - 1) / YT;
    const int64_t b = blockIdx.x, xcd = b % 8, sq = b / 8;
    const int64_t mt = mt0 + (sq / nnt) * 8 + xcd, nt = sq % nnt;  // M-tiles from mt0 on
    if (mt >= nmt) return;
    const int64_t m0 = mt * YT, n0 = nt * YT;
    const int64_t kb0 = (int64_t)blockIdx.z * tchunk;
    const int64_t ke = (kb0 + tchunk < Tp) ? kb0 + tchunk : Tp;
    const int nks = (int)((ke - kb0) / YK2);   // tchunk and Tp are whole 32-token steps

    // one load per lane and plane: wave w fills rows 2w, 2w + 1 of the plane; slot
    // p' of a row holds logical piece p' ^ 4 (row & 3)
    constexpr int NL = 4;
    const int lrow = 2 * w + (lane >> 5);
    const int lpiece = (lane & 31) ^ ((lrow & 3) << 2);
    const int dsto = w * 64 * 8;   // element offset of this wave's 64 slots in a plane
    auto issue_ks = [&](int ks, uint16_t* dst) {
        const int64_t kb = kb0 + (int64_t)ks * YK2;
#pragma unroll
        for (int pl = 0; pl < 4; ++pl) {
            const uint16_t* base = pl == 0 ? Ah : pl == 1 ? Al : pl == 2 ? Bh : Bl;
            const int64_t ld = pl < 2 ? Mp : Np;
            const int64_t c0 = pl < 2 ? m0 : n0;
            // a resource over this k-step's rows of the plane (offsets stay 32-bit)
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(base + kb * ld + c0), (short)0, (int)(YK2 * ld * 2), 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (__attribute__((address_space(3))) void*)(dst + pl * PL2 + dsto), 16,
                (int)(lrow * ld * 2 + lpiece * 16), 0, 0, 0);
        }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    int oa[4], ob[2];  // lane offsets of the A and B column blocks
#pragma unroll
    for (int i = 0; i < 4; ++i) oa[i] = tr_lane_off(wm * 128 + 32 * i, lane);
#pragma unroll
    for (int j = 0; j < 2; ++j) ob[j] = tr_lane_off(wn * 64 + 32 * j, lane);
    auto read_frags = [&](const uint16_t* t, PairFrags& f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f.ah[i] = tr_frag(t + oa[i]);
            f.al[i] = tr_frag(t + PL2 + oa[i]);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            f.bh[j] = tr_frag(t + 2 * PL2 + ob[j]);
            f.bl[j] = tr_frag(t + 3 * PL2 + ob[j]);
        }
    };
    // k-step ks: MFMAs on the fragments of slab ks (read during k-step ks - 1),
    // while the fragments of slab ks + 1 are read from its stage; it starts once
    // slab ks + 1 has landed (only the NL loads of slab ks + 2 outstanding).  Past
    // its barrier every wave has finished k-step ks - 1, so the stage of slab
    // ks - 1 takes slab ks + 3 (clamped to the last one: every k-step issues the
    // same loads).
    auto kstep = [&](int ks, const uint16_t* nx1, uint16_t* wr, PairFrags& cur, PairFrags& nxt) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm_o(NL));
        asm volatile("s_barrier" ::: "memory");
        issue_ks(min(ks + 3, nks - 1), wr);
        read_frags(nx1, nxt);   // past the last k-step: a stage of valid data, unused
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                acc[i][j] = mfma_bf16(cur.al[i], cur.bh[j], acc[i][j]);
                acc[i][j] = mfma_bf16(cur.ah[i], cur.bl[j], acc[i][j]);
                acc[i][j] = mfma_bf16(cur.ah[i], cur.bh[j], acc[i][j]);
            }
        // the loads first, then one fragment read between consecutive MFMAs
        __builtin_amdgcn_sched_group_barrier(0x020, NL, 0);
#pragma unroll
        for (int q = 0; q < 24; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };

    PairFrags fa, fb;
    issue_ks(0, S0);
    issue_ks(min(1, nks - 1), S1);
    issue_ks(min(2, nks - 1), S2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm_o(2 * NL));   // slab 0
    asm volatile("s_barrier" ::: "memory");
    read_frags(S0, fa);
    for (int ks = 0; ks < nks; ks += 4) {
        kstep(ks, S1, S3, fa, fb);
        if (ks + 1 < nks) kstep(ks + 1, S2, S0, fb, fa);
        if (ks + 2 < nks) kstep(ks + 2, S3, S1, fa, fb);
        if (ks + 3 < nks) kstep(ks + 3, S0, S2, fb, fa);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm_o(0));   // the clamped loads past the end

    // split z writes plane z (zs floats apart) of rows orow0 on
    float* o = out + (int64_t)blockIdx.z * zs - orow0 * N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * 128 + i * 32 + (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5);
                const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
                if (row < M && col < N) o[row * N + col] = acc[i][j][r];
            }
}

// zero rows [r0, r1) of two [*, ld] bf16 planes (token padding of pairs written elsewhere)
__global__ void __launch_bounds__(256) zero_rows_kernel(uint16_t* __restrict__ a, uint16_t* __restrict__ b, int64_t r0,
                                                        int64_t r1, int64_t ld) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 8 elements each
    const int64_t n8 = (r1 - r0) * ld / 8;
    if (i >= n8) return;
    const int64_t off = r0 * ld + 8 * i;
    *reinterpret_cast<uint4*>(a + off) = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(b + off) = make_uint4(0, 0, 0, 0);
}

size_t outer_workspace_bytes(int64_t T, int64_t n, int64_t d) { return plan_outer(T, n, d).total; }

bool outer_uses_pairs(int64_t T, int64_t n, int64_t d) { return plan_outer(T, n, d).x3; }

OuterPairs outer_ghat_pairs(int64_t T, int64_t n, int64_t d, void* workspace) {
    const OuterPlan p = plan_outer(T, n, d);
    OuterPairs r{nullptr, nullptr, 0};
    if (!p.x3 || workspace == nullptr) return r;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    r.hi = reinterpret_cast<uint16_t*>(ws + p.off_ah);
    r.lo = reinterpret_cast<uint16_t*>(ws + p.off_al);
    r.ld = p.Mp;
    return r;
}

hipError_t launch_outer(const float* ghat, const float* x, int64_t T, int64_t n, int64_t d, float* grad_w,
                        void* workspace, size_t workspace_bytes, hipStream_t stream, bool pairs_ready) {
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
        const int64_t ga = p.Tp * p.Mp / 8, gb = p.Tp * p.Np / 8;
        if (!pairs_ready) {
            hipLaunchKernelGGL(split_pairs_kernel, dim3((unsigned)((ga + 255) / 256)), dim3(256), 0, stream, ghat, T, n,
                               p.Tp, p.Mp, ah, al);
        } else if (p.Tp > T) {  // rows 0..T-1 (all Mp columns) came from the estimator
            const int64_t z8 = (p.Tp - T) * p.Mp / 8;
            hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)((z8 + 255) / 256)), dim3(256), 0, stream, ah, al, T, p.Tp,
                               p.Mp);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(split_pairs_kernel, dim3((unsigned)((gb + 255) / 256)), dim3(256), 0, stream, x, T, d, p.Tp,
                           p.Np, bh, bl);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int64_t nnt = (d + YT - 1) / YT, nmt = (n + YT - 1) / YT;
        const int64_t nmt8 = (p.mA + 7) / 8 * 8;  // M-tiles rounded up to whole XCD groups
        const dim3 grid((unsigned)(nmt8 * nnt), 1, (unsigned)p.splits);
        bool timed = false;
        if ((e = launch_timer_begin(kTimedOuter, stream, timed)) != hipSuccess) return e;
        hipLaunchKernelGGL(outer_x3_kernel, grid, dim3(YNT), 0, stream, ah, al, bh, bl, std::min(n, p.mA * YT), d, p.Mp,
                           p.Np, p.Tp, p.tchunk, part, (int64_t)0, n * d, (int64_t)0);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = launch_timer_end(kTimedOuter, stream, timed)) != hipSuccess) return e;
        if (p.mA < nmt) {  // the last round's M-tiles, their tokens split
            float* tpart = reinterpret_cast<float*>(ws + p.off_tail);
            const int64_t rows = n - p.mA * YT, tcount = rows * d;
            const dim3 gt((unsigned)((nmt - p.mA + 7) / 8 * 8 * nnt), 1, (unsigned)p.tsplits);
            hipLaunchKernelGGL(outer_x3_kernel, gt, dim3(YNT), 0, stream, ah, al, bh, bl, n, d, p.Mp, p.Np, p.Tp,
                               p.tchunk_t, tpart, p.mA, tcount, p.mA * YT);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((tcount + 255) / 256)), dim3(256), 0, stream, tpart,
                               p.tsplits, tcount, grad_w + p.mA * YT * d);
        }
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
