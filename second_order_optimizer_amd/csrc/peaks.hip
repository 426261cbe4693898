// Machine-peak probes for measurement tools: the matrix-core issue rate with
// no memory traffic (fp32 v_mfma_f32_32x32x2f32, fp64 v_mfma_f64_16x16x4f64
// and bf16 v_mfma_f32_32x32x16_bf16, the instructions the optimizer's
// products run on) and a plain device copy.
// They hold none of the method's arithmetic; measured peaks sit beside the
// published ones when kernel rates are reported as fractions of a peak.
#include "../../include/shampoo.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kPeakIters = 4096;   // MFMA steps per wave
constexpr int kPeakAcc = 8;        // independent accumulators per wave
constexpr int kPeakGrid = 256 * 8; // 8 workgroups of 4 waves per CU: 8 waves per SIMD

typedef float pf16 __attribute__((ext_vector_type(16)));
typedef double pd4 __attribute__((ext_vector_type(4)));
typedef float pv4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_peak_mfma_f32(float* out, float seed) {
    pf16 acc[kPeakAcc];
#pragma unroll
    for (int i = 0; i < kPeakAcc; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
    const float a = seed * (1.0f + 1e-7f * (threadIdx.x & 63));
    const float b = seed;
    for (int it = 0; it < kPeakIters; ++it) {
#pragma unroll
        for (int i = 0; i < kPeakAcc; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[i], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kPeakAcc; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[i][v];
    // one store per wave, so the products are not dead code
    if ((threadIdx.x & 63) == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

__global__ __launch_bounds__(256) void k_peak_mfma_f64(double* out, double seed) {
    pd4 acc[kPeakAcc];
#pragma unroll
    for (int i = 0; i < kPeakAcc; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][v] = 0.0;
    const double a = seed * (1.0 + 1e-15 * (threadIdx.x & 63));
    const double b = seed;
    for (int it = 0; it < kPeakIters; ++it) {
#pragma unroll
        for (int i = 0; i < kPeakAcc; ++i)
            acc[i] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[i], 0, 0, 0);
    }
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < kPeakAcc; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) s += acc[i][v];
    if ((threadIdx.x & 63) == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

typedef __bf16 pb8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void k_peak_mfma_bf16(float* out, float seed) {
    pf16 acc[kPeakAcc];
#pragma unroll
    for (int i = 0; i < kPeakAcc; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
    pb8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(seed * (1.0f + 0.01f * ((threadIdx.x + e) & 7)));
        b[e] = (__bf16)seed;
    }
    for (int it = 0; it < kPeakIters; ++it) {
#pragma unroll
        for (int i = 0; i < kPeakAcc; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kPeakAcc; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[i][v];
    if ((threadIdx.x & 63) == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

// dst[i] = src[i] over n 16-byte elements, grid-stride, each thread issuing
// U loads before their stores; NT: nontemporal loads and stores.
template <int U, bool NT>
__global__ __launch_bounds__(256) void k_peak_copy(const pv4* __restrict__ src,
                                                   pv4* __restrict__ dst, int64_t n) {
    const int64_t span = (int64_t)256 * U;
    for (int64_t b = (int64_t)blockIdx.x * span; b < n; b += (int64_t)gridDim.x * span) {
        pv4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = b + 256 * u + threadIdx.x;
            if (i < n) x[u] = NT ? __builtin_nontemporal_load(src + i) : src[i];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = b + 256 * u + threadIdx.x;
            if (i < n) {
                if (NT) __builtin_nontemporal_store(x[u], dst + i);
                else dst[i] = x[u];
            }
        }
    }
}

int hip_ok(hipError_t e) { return e == hipSuccess ? SHAMPOO_OK : SHAMPOO_E_HIP; }

// Median of three timed launches of `launch` (one untimed warm-up first).
template <typename F>
int time_launches(F&& launch, hipStream_t s, float* ms_out) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    int rc = hip_ok(hipEventCreate(&e0));
    if (!rc) rc = hip_ok(hipEventCreate(&e1));
    float ms[3] = {0.f, 0.f, 0.f};
    if (!rc) {
        launch();
        rc = hip_ok(hipGetLastError());
    }
    for (int r = 0; r < 3 && !rc; ++r) {
        rc = hip_ok(hipEventRecord(e0, s));
        if (!rc) {
            launch();
            rc = hip_ok(hipGetLastError());
        }
        if (!rc) rc = hip_ok(hipEventRecord(e1, s));
        if (!rc) rc = hip_ok(hipEventSynchronize(e1));
        if (!rc) rc = hip_ok(hipEventElapsedTime(&ms[r], e0, e1));
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (rc) return rc;
    // median of three
    float a = ms[0], b = ms[1], c = ms[2];
    if (a > b) { float t = a; a = b; b = t; }
    if (b > c) { float t = b; b = c; c = t; }
    if (a > b) { float t = a; a = b; b = t; }
    *ms_out = b;
    return SHAMPOO_OK;
}

}  // namespace

extern "C" int shampoo_measure_peaks(shampoo_peaks* out, void* scratch, size_t scratch_bytes,
                                     void* stream) {
    if (!out || !scratch) return SHAMPOO_E_ARG;
    if ((reinterpret_cast<uintptr_t>(scratch) & 255) != 0) return SHAMPOO_E_ARG;
    // the copy moves half the buffer into the other half; the MFMA probes
    // write one value per wave into its start
    const size_t half = (scratch_bytes / 2) & ~size_t(255);
    const size_t need_mfma = size_t(kPeakGrid) * 4 * sizeof(double);
    if (half < (size_t(1) << 20) || scratch_bytes < need_mfma) return SHAMPOO_E_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float ms = 0.f;
    int rc = time_launches(
        [&] {
            k_peak_mfma_f32<<<kPeakGrid, 256, 0, s>>>(static_cast<float*>(scratch), 0.5f);
        },
        s, &ms);
    if (rc) return rc;
    // flops per v_mfma_f32_32x32x2f32: 32 x 32 x 2 multiply-adds
    const double waves = double(kPeakGrid) * 4;
    out->mfma_f32_tflops = waves * kPeakIters * kPeakAcc * (2.0 * 32 * 32 * 2) / (ms * 1e-3) / 1e12;
    rc = time_launches(
        [&] {
            k_peak_mfma_f64<<<kPeakGrid, 256, 0, s>>>(static_cast<double*>(scratch), 0.5);
        },
        s, &ms);
    if (rc) return rc;
    out->mfma_f64_tflops = waves * kPeakIters * kPeakAcc * (2.0 * 16 * 16 * 4) / (ms * 1e-3) / 1e12;
    rc = time_launches(
        [&] {
            k_peak_mfma_bf16<<<kPeakGrid, 256, 0, s>>>(static_cast<float*>(scratch), 0.5f);
        },
        s, &ms);
    if (rc) return rc;
    out->mfma_bf16_tflops = waves * kPeakIters * kPeakAcc * (2.0 * 32 * 32 * 16) / (ms * 1e-3) / 1e12;
    const int64_t n4 = (int64_t)(half / sizeof(pv4));
    const pv4* src = static_cast<const pv4*>(scratch);
    pv4* dst = reinterpret_cast<pv4*>(static_cast<unsigned char*>(scratch) + half);
    // the best of a few copy shapes (loads in flight per thread, workgroups
    // per CU, nontemporal or not)
    double best = 0.0;
    for (int v = 0; v < 4; ++v) {
        rc = time_launches(
            [&] {
                if (v == 0) k_peak_copy<4, false><<<256 * 8, 256, 0, s>>>(src, dst, n4);
                else if (v == 1) k_peak_copy<8, false><<<256 * 16, 256, 0, s>>>(src, dst, n4);
                else if (v == 2) k_peak_copy<16, true><<<256 * 8, 256, 0, s>>>(src, dst, n4);
                else k_peak_copy<1, false><<<256 * 32, 256, 0, s>>>(src, dst, n4);
            },
            s, &ms);
        if (rc) return rc;
        const double gbs = 2.0 * double(n4) * sizeof(pv4) / (ms * 1e-3) / 1e9;
        if (gbs > best) best = gbs;
    }
    out->copy_gbs = best;
    out->copy_bytes = (int64_t)n4 * (int64_t)sizeof(pv4);
    return SHAMPOO_OK;
}
