// Noise export: the exact Gaussian values (and raw Philox words) the
// estimators regenerate in registers, written out for inspection and tests.
#include "dust_device.hpp"
#include "dust_internal.hpp"

namespace dust {

// One thread per (draw, token, channel quad).
__global__ void __launch_bounds__(256) noise_export_kernel(uint32_t k0, uint32_t k1, uint32_t layer,
                                                           uint32_t draw0, uint32_t tok0, int64_t T,
                                                           int64_t n, int64_t rows, uint32_t* raw,
                                                           float* gauss) {
    const int64_t nq = (n + 3) >> 2;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= rows * nq) return;
    const int64_t row = gid / nq;  // row = i * T + t
    const uint32_t q = (uint32_t)(gid - row * nq);
    const uint32_t i = (uint32_t)(row / T);
    const uint32_t t = (uint32_t)(row - (int64_t)i * T);
    const u32x4 w = philox4x32_10(tok0 + t, q, draw0 + i, layer, k0, k1);
    if (raw) {
        uint32_t* o = raw + row * (4 * nq) + 4 * (int64_t)q;
        o[0] = w.x; o[1] = w.y; o[2] = w.z; o[3] = w.w;
    }
    if (gauss) {
        float a[4];
        box_muller(w.x, w.y, a[0], a[1]);
        box_muller(w.z, w.w, a[2], a[3]);
        float* o = gauss + row * n + 4 * (int64_t)q;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (4 * (int64_t)q + c < n) o[c] = a[c];
    }
}

hipError_t launch_noise_export(uint64_t seed, uint32_t layer, uint32_t draw0, int64_t K, uint32_t tok0,
                               int64_t T, int64_t n, uint32_t* raw, float* gauss, hipStream_t stream) {
    const int64_t nq = (n + 3) >> 2;
    const int64_t rows = K * T;
    const int64_t total = rows * nq;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(noise_export_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint32_t)seed,
                       (uint32_t)(seed >> 32), layer, draw0, tok0, T, n, rows, raw, gauss);
    return hipGetLastError();
}

}  // namespace dust
