// calib.hip -- attainable-peak measurement kernels (streaming copy, fp16 matrix-core loop) for
// the benchmark's same-run reference figures.  Not part of the GDN computation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdn_calib.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr size_t kUnit = 16 * kThreads * 8;  // bytes must be a multiple of this

// grid-stride copy of n 16-byte units, NF loads in flight per thread (n a multiple of
// kThreads * NF); NT: stores that do not keep the lines in the caches
template <int NF, bool NT>
__global__ void __launch_bounds__(kThreads) copy_kernel(const f32x4 *src, f32x4 *dst, size_t n) {
    const size_t step = static_cast<size_t>(gridDim.x) * kThreads * NF;
    for (size_t base = static_cast<size_t>(blockIdx.x) * kThreads * NF + threadIdx.x; base < n;
         base += step) {
        f32x4 v[NF];
#pragma unroll
        for (int j = 0; j < NF; ++j) v[j] = src[base + j * kThreads];
#pragma unroll
        for (int j = 0; j < NF; ++j) {
            if constexpr (NT)
                __builtin_nontemporal_store(v[j], &dst[base + j * kThreads]);
            else
                dst[base + j * kThreads] = v[j];
        }
    }
}

// each workgroup copies one contiguous slice of n / gridDim.x units (a multiple of
// kThreads * 8), 8 loads in flight per thread, walking it front to back
__global__ void __launch_bounds__(kThreads) slice_copy_kernel(const f32x4 *__restrict__ src,
                                                              f32x4 *__restrict__ dst, size_t n) {
    const size_t per = n / gridDim.x, lo = static_cast<size_t>(blockIdx.x) * per;
    for (size_t base = lo + threadIdx.x; base < lo + per; base += kThreads * 8) {
        f32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = src[base + j * kThreads];
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[base + j * kThreads] = v[j];
    }
}

// 8 independent accumulation chains per wavefront keep the matrix core's pipeline full
__global__ void __launch_bounds__(kThreads) mfma_kernel(float *__restrict__ out, int iters) {
    const int lane = threadIdx.x & 63;
    f16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {  // small exact values: the sums stay far from overflow
        a[e] = static_cast<_Float16>(static_cast<float>((lane + e) & 7) * (1.f / 1024.f));
        b[e] = static_cast<_Float16>(static_cast<float>((lane * 3 + e) & 7) * (1.f / 1024.f));
    }
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = s;
}

// The same loop with a clock record and a choice of product shape.  FORM 0: 16x16x32 fp16
// (16384 flops per instruction), FORM 1: 32x32x16 fp16 (32768).  Wavefront 0 of every
// workgroup writes clk[2b] = shader-clock cycles and clk[2b + 1] = constant-rate wall-clock
// ticks over its loop, so that cycles / ticks x the wall-clock rate is the engine clock the
// products actually ran at.
template <int FORM>
__global__ void __launch_bounds__(kThreads) mfma_clock_kernel(float *__restrict__ out,
                                                              unsigned long long *__restrict__ clk,
                                                              int iters) {
    const int lane = threadIdx.x & 63;
    f16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = static_cast<_Float16>(static_cast<float>((lane + e) & 7) * (1.f / 1024.f));
        b[e] = static_cast<_Float16>(static_cast<float>((lane * 3 + e) & 7) * (1.f / 1024.f));
    }
    float s = 0.f;
    const unsigned long long c0 = clock64(), w0 = wall_clock64();
    if constexpr (FORM == 0) {
        f32x4 acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    } else {
        f32x16 acc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) s += acc[j][e];
    }
    const unsigned long long c1 = clock64(), w1 = wall_clock64();
    out[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        clk[2 * static_cast<size_t>(blockIdx.x)] = c1 - c0;
        clk[2 * static_cast<size_t>(blockIdx.x) + 1] = w1 - w0;
    }
}

}  // namespace

extern "C" {

int gdn_calib_copy(const void *src, void *dst, size_t bytes, int blocks, int variant,
                   void *stream) {
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    // variant 3 updates in place (src == dst), every other variant needs disjoint buffers
    const bool overlap = s < d + bytes && d < s + bytes;
    if (src == nullptr || dst == nullptr || blocks <= 0 || bytes == 0 || bytes % kUnit != 0 ||
        s % 16 != 0 || d % 16 != 0 || variant < 0 || variant > 4 ||
        (variant == 3 ? s != d : overlap) ||
        (variant == 4 && bytes % (kUnit * static_cast<size_t>(blocks)) != 0))
        return 1;
    if (variant == 4) {
        hipLaunchKernelGGL(slice_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                           0, static_cast<hipStream_t>(stream), static_cast<const f32x4 *>(src),
                           static_cast<f32x4 *>(dst), bytes / 16);
        return hipGetLastError() == hipSuccess ? 0 : 3;
    }
    auto kern = variant == 0 ? copy_kernel<4, false>
                : variant == 2 ? copy_kernel<8, true> : copy_kernel<8, false>;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const f32x4 *>(src),
                       static_cast<f32x4 *>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

int gdn_calib_mfma(float *out, int blocks, int iters, void *stream) {
    if (out == nullptr || blocks <= 0 || iters < 1 || iters > (1 << 20)) return 1;
    hipLaunchKernelGGL(mfma_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), out, iters);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

int gdn_calib_mfma_clock(float *out, unsigned long long *clk, int blocks, int iters, int form,
                         void *stream) {
    if (out == nullptr || clk == nullptr || blocks <= 0 || iters < 1 || iters > (1 << 20) ||
        (form != 0 && form != 1))
        return 1;
    auto kern = form == 0 ? mfma_clock_kernel<0> : mfma_clock_kernel<1>;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), out, clk, iters);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

int gdn_calib_wall_clock_khz(void) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return -1;
    return khz;
}

}  // extern "C"
