// ssd_probe.hip -- measurements of the machine (include/ssd_probe.h): the dense bf16 MFMA
// rate the chip reaches and its shader clock, alone or beside another kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_probe.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void stamp(uint64_t* out) {
    out[0] = __builtin_amdgcn_s_memtime();
    out[1] = __builtin_amdgcn_s_memrealtime();
}

// Four independent accumulator chains per wave, operands in registers; small operands
// (2^-8 each) keep the sums far from overflow for any iteration count allowed.
__global__ void __launch_bounds__(256) mfma_rate_kernel(int64_t iters, uint64_t* stamps) {
    uint64_t t[4];
    stamp(t);
    const float v = 0.00390625f * (float)(1 + (threadIdx.x & 3));
    bf16x8 a, b;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        a[q] = (__bf16)v;
        b[q] = (__bf16)(v * 0.5f);
    }
    f32x16 c0 = f32x16{}, c1 = f32x16{}, c2 = f32x16{}, c3 = f32x16{};
    for (int64_t i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
    __syncthreads();
    stamp(t + 2);
    uint64_t* o = stamps + 4 * (int64_t)blockIdx.x;
    if (threadIdx.x == 0) {
        o[0] = t[0];
        o[1] = t[1];
        o[2] = t[2];
        o[3] = t[3];
    }
    // (every product is positive, so this never stores; it keeps the products alive)
    if (s < 0.f) o[0] = 0;
}

__global__ void __launch_bounds__(64) clock_kernel(int64_t spins, uint64_t* stamps) {
    uint64_t t[4];
    stamp(t);
    for (int64_t i = 0; i < spins; ++i) __builtin_amdgcn_s_sleep(1);
    stamp(t + 2);
    if (threadIdx.x == 0) {
        uint64_t* o = stamps + 4 * (int64_t)blockIdx.x;
        o[0] = t[0];
        o[1] = t[1];
        o[2] = t[2];
        o[3] = t[3];
    }
}

}  // namespace

extern "C" int ssd_probe_mfma_bf16(int64_t iters, int blocks, uint64_t* stamps, void* stream) {
    if (iters < 1 || iters > ((int64_t)1 << 30) || blocks < 1 || blocks > 65536 || !stamps) return -1;
    hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                       stamps);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int ssd_probe_clock(int64_t spins, int blocks, uint64_t* stamps, void* stream) {
    if (spins < 1 || spins > ((int64_t)1 << 24) || blocks < 1 || blocks > 65536 || !stamps) return -1;
    hipLaunchKernelGGL(clock_kernel, dim3((unsigned)blocks), dim3(64), 0, static_cast<hipStream_t>(stream), spins,
                       stamps);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int ssd_probe_device(int* compute_units, int* max_clock_khz) {
    if (!compute_units || !max_clock_khz) return -1;
    if (hipDeviceGetAttribute(compute_units, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess) return -4;
    if (hipDeviceGetAttribute(max_clock_khz, hipDeviceAttributeClockRate, 0) != hipSuccess) return -4;
    return 0;
}
