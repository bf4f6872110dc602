// Weight-gradient outer product  grad_w = ghat^T x = sum_t ghat_t x_t^T
// (TL;DR page, section 1, equation for G_W), as an fp32 MFMA GEMM.
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

struct OuterPlan {
    int splits;
    int64_t tchunk;
};

OuterPlan plan_outer(int64_t T, int64_t n, int64_t d) {
    const int64_t tiles = ((n + BM - 1) / BM) * ((d + BN - 1) / BN);
    int64_t s = (512 + tiles - 1) / tiles;
    const int64_t smax = (T + 255) / 256;  // at least 256 tokens per split
    if (s > smax) s = smax;
    if (s < 1) s = 1;
    int64_t chunk = (T + s - 1) / s;
    chunk = (chunk + BK - 1) / BK * BK;
    s = (T + chunk - 1) / chunk;
    return {(int)s, chunk};
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

size_t outer_workspace_bytes(int64_t T, int64_t n, int64_t d) {
    const OuterPlan p = plan_outer(T, n, d);
    return p.splits > 1 ? (size_t)p.splits * (size_t)n * (size_t)d * sizeof(float) : 0;
}

hipError_t launch_outer(const float* ghat, const float* x, int64_t T, int64_t n, int64_t d, float* grad_w,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const OuterPlan p = plan_outer(T, n, d);
    const dim3 grid((unsigned)((n + BM - 1) / BM), (unsigned)((d + BN - 1) / BN), (unsigned)p.splits);
    if (p.splits == 1) {
        hipLaunchKernelGGL(outer_f32_kernel, grid, dim3(NTH), 0, stream, ghat, x, T, n, d, p.tchunk, grad_w);
        return hipGetLastError();
    }
    if (workspace == nullptr || workspace_bytes < outer_workspace_bytes(T, n, d)) return hipErrorInvalidValue;
    float* part = static_cast<float*>(workspace);
    hipLaunchKernelGGL(outer_f32_kernel, grid, dim3(NTH), 0, stream, ghat, x, T, n, d, p.tchunk, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t count = n * d;
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream, part,
                       p.splits, count, grad_w);
    return hipGetLastError();
}

}  // namespace dust
