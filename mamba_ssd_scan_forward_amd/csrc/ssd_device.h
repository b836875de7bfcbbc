// ssd_device.h -- gfx950 building blocks for the SSD kernels: MFMA tiles, operand
// fragments and their loads from LDS and global memory.
//
// Every contraction in the SSD forward is built from one 32 x 32 output tile
// held by a 64-lane wavefront, advanced 16 along the contraction index per
// step:
//   bf16: one v_mfma_f32_32x32x16_bf16 per step;
//   f32 : eight v_mfma_f32_32x32x2_f32 per step.
// Fragment layouts (lane = 0..63, lr = lane % 32, lg = lane / 32):
//   A operand  (M x K): lane holds A[lr][8*lg + q],      q = 0..7
//   B operand  (K x N): lane holds B[8*lg + q][lr],      q = 0..7
//   accumulator (M x N): element i of a lane is D[8*(i/4) + 4*lg + (i%4)][lr]
// For f32 the eight K values of a fragment are fed to eight K=2 instructions,
// the q-th instruction taking element q of both operands; A and B use the same
// K order, so the sum over K is unchanged.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define SSD_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Buffer resources: 32-bit byte offsets against a base and a size; a load whose bytes
// fall outside [0, size) returns zeros.  Predicated loads pass kOutOfRange.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;   // gfx9 raw buffer, no swizzle

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
// A value the optimizer must treat as unknown at this point: offsets derived from it are
// recomputed where they are used instead of being hoisted out of a loop and held in
// (or spilled from) registers for its whole length.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}
__device__ __forceinline__ float ldb_f32(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

template <typename T> struct Elem;

template <> struct Elem<__bf16> {
    typedef bf16x8 frag;
    static constexpr int bytes = 2;
    __device__ static __forceinline__ frag zero() {
        u32x4 z = {0u, 0u, 0u, 0u};
        return __builtin_bit_cast(frag, z);
    }
    __device__ static __forceinline__ f32x16 mma(f32x16 acc, frag a, frag b) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
    // 8 contiguous elements from global memory (16-byte aligned).
    __device__ static __forceinline__ frag ldg8(const __bf16* p) {
        return __builtin_bit_cast(frag, *reinterpret_cast<const u32x4*>(p));
    }
    // 8 contiguous elements through a buffer resource (zeros out of range).  The whole
    // vector is cast at once: casting single elements of the loaded vector has been
    // seen to shrink the load.
    __device__ static __forceinline__ frag ldb8(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(frag, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
    }
    // the same with a uniform byte offset in a scalar register; only for loads that are
    // known to be in range (the scalar offset takes no part in the range check)
    __device__ static __forceinline__ frag ldb8(rsrc_t r, uint32_t voff, uint32_t soff) {
        return __builtin_bit_cast(frag, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
    }
    // 8 contiguous elements from LDS.
    __device__ static __forceinline__ frag lds8(const __bf16* p) {
        return __builtin_bit_cast(frag, *reinterpret_cast<const u32x4*>(p));
    }
    __device__ static __forceinline__ float to_f(__bf16 v) { return (float)v; }
    __device__ static __forceinline__ __bf16 from_f(float v) { return (__bf16)v; }
    // 4 values -> 4 consecutive elements (8 bytes).
    __device__ static __forceinline__ void st4(__bf16* p, float a, float b, float c, float d) {
        bf16x4 v = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
        *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, v);
    }
};

template <> struct Elem<float> {
    typedef f32x8 frag;
    static constexpr int bytes = 4;
    __device__ static __forceinline__ frag zero() {
        frag z = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        return z;
    }
    __device__ static __forceinline__ f32x16 mma(f32x16 acc, frag a, frag b) {
#pragma unroll
        for (int q = 0; q < 8; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[q], b[q], acc, 0, 0, 0);
        return acc;
    }
    __device__ static __forceinline__ frag ldg8(const float* p) {
        const f32x4* v = reinterpret_cast<const f32x4*>(p);
        f32x4 lo = v[0], hi = v[1];
        frag r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return r;
    }
    __device__ static __forceinline__ frag ldb8(rsrc_t r, uint32_t off) {
        const f32x4 lo = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
        const f32x4 hi = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 16), 0, 0));
        frag v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return v;
    }
    __device__ static __forceinline__ frag lds8(const float* p) { return ldg8(p); }
    __device__ static __forceinline__ float to_f(float v) { return v; }
    __device__ static __forceinline__ float from_f(float v) { return v; }
    __device__ static __forceinline__ void st4(float* p, float a, float b, float c, float d) {
        f32x4 v = {a, b, c, d};
        *reinterpret_cast<f32x4*>(p) = v;
    }
};

// Column fragment of a row-major LDS matrix M (row stride `stride` elements):
// the lane receives M[r0 + 8*lg + q][c0 + lr], q = 0..7.  This is the operand
// shape of both "A = M^T" (rows of M along K) and "B = M" (rows of M along K).
// bf16 uses two ds_read_b64_tr_b16: inside each group of 16 lanes, lane i
// reads 4 consecutive elements of row (i / 4) at column 4 * (i % 4) of a 4 x 16
// block and the hardware hands lane j the j-th column of that block.
template <typename T> __device__ __forceinline__ typename Elem<T>::frag
lds_col(const T* M, int stride, int r0, int c0, int lane);

template <> __device__ __forceinline__ bf16x8
lds_col<__bf16>(const __bf16* M, int stride, int r0, int c0, int lane) {
    const int row = r0 + 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const __bf16* p0 = M + row * stride + col;
    const __bf16* p1 = p0 + 4 * stride;
    bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SSD_LDS bf16x4*)(SSD_LDS __bf16*)p0);
    bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SSD_LDS bf16x4*)(SSD_LDS __bf16*)p1);
    bf16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return r;
}

template <> __device__ __forceinline__ f32x8
lds_col<float>(const float* M, int stride, int r0, int c0, int lane) {
    const float* p = M + (r0 + 8 * (lane >> 5)) * stride + c0 + (lane & 31);
    f32x8 r;
#pragma unroll
    for (int q = 0; q < 8; ++q) r[q] = p[q * stride];
    return r;
}

// Row-major LDS matrices of W columns.  bf16: rows are not padded; the 16-byte units
// of a row are XOR-swizzled by the row index so that the four rows read together by
// a transposing load fall in different banks.  f32: rows padded by 16 bytes.
template <typename T, int W> struct LdsMat;

template <int W> struct LdsMat<__bf16, W> {
    static constexpr int stride = W;
    static constexpr int rows_bytes(int rows) { return rows * W * 2; }
    __device__ static __forceinline__ int swz(int r) {
        return W >= 64 ? 2 * (r & 3) : 2 * ((r >> 1) & 1);
    }
    // element (r, c) with c % 4 == 0: start of a 4- or 8-element piece inside a unit
    __device__ static __forceinline__ int idx(int r, int c) {
        return r * W + ((((c >> 3) ^ swz(r)) << 3) | (c & 7));
    }
};

template <int W> struct LdsMat<float, W> {
    static constexpr int stride = W + 4;
    static constexpr int rows_bytes(int rows) { return rows * (W + 4) * 4; }
    __device__ static __forceinline__ int idx(int r, int c) { return r * (W + 4) + c; }
};

// Column fragment of an LDS matrix M (layout LdsMat<T, W>): the lane receives
// M[r0 + 8*lg + q][c0 + lr], q = 0..7.  This is the operand shape of both "A = M^T"
// (rows of M along K) and "B = M" (rows of M along K).
// bf16 uses two ds_read_b64_tr_b16: inside each group of 16 lanes, lane i reads 4
// consecutive elements of row (i / 4) at column 4 * (i % 4) of a 4 x 16 block and the
// hardware hands lane j the j-th column of that block.
template <typename T, int W> struct LdsCol;

template <int W> struct LdsCol<__bf16, W> {
    __device__ static __forceinline__ bf16x8 get(const __bf16* M, int r0, int c0, int lane) {
        typedef LdsMat<__bf16, W> L;
        const int row = r0 + 8 * (lane >> 5) + ((lane & 15) >> 2);
        const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const __bf16* p0 = M + L::idx(row, col);
        const __bf16* p1 = M + L::idx(row + 4, col);
        bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SSD_LDS bf16x4*)(SSD_LDS __bf16*)p0);
        bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SSD_LDS bf16x4*)(SSD_LDS __bf16*)p1);
        bf16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return r;
    }
};

template <int W> struct LdsCol<float, W> {
    __device__ static __forceinline__ f32x8 get(const float* M, int r0, int c0, int lane) {
        typedef LdsMat<float, W> L;
        const float* p = M + L::idx(r0 + 8 * (lane >> 5), c0 + (lane & 31));
        f32x8 r;
#pragma unroll
        for (int q = 0; q < 8; ++q) r[q] = p[q * L::stride];
        return r;
    }
};

// Element 16*ks + 8*lg + q of a 32-wide row, as a (row, column) index inside a
// 32 x 32 tile: the K position of fragment element q at K-step ks.
__device__ __forceinline__ int frag_k(int ks, int lane, int q) { return 16 * ks + 8 * (lane >> 5) + q; }

// Row of accumulator element i (column is lane % 32).
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

}  // namespace ssd
