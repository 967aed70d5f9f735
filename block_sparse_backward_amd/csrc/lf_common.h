// Shared device helpers of the LazyFlash HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lf {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- element access -------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Eight consecutive elements as floats (16-byte aligned source).
__device__ __forceinline__ void load8(const bf16* p, float (&x)[8]) {
    u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[2 * j] = __uint_as_float(r[j] << 16);
        x[2 * j + 1] = __uint_as_float(r[j] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) { x[j] = a[j]; x[4 + j] = b[j]; }
}

// Round-to-nearest-even float -> bf16 (hardware convert on gfx950).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }

// ---- MFMA ------------------------------------------------------------------
// 32x32x16 bf16 -> f32.  Lane l holds A row (l % 32) with k = 8*(l/32) + 0..7,
// B column (l % 32) with the same k, and C column (l % 32) with rows
// 8*a + 4*(l/32) + b at register 4*a + b.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---- LDS --------------------------------------------------------------------
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposing 8-byte LDS read.  Within each group of 16 lanes, lane i receives
// element (i & 3) of the 8 bytes fetched by lanes 4*e + (i >> 2), e = 0..3.
// So if lane j of the group fetches row (r0 + (j >> 2)), columns c0 + 4*(j & 3)
// .. +3 of a row-major 16-bit matrix, lane i receives column c0 + i of rows
// r0 .. r0 + 3.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* lds_ptr) {
    auto p = (lds_i16x4*)((__attribute__((address_space(3))) char*)(lds_ptr));
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
    return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---- buffer resources ------------------------------------------------------
// Raw buffer over [base, base + bytes): 32-bit lane offsets plus a uniform
// scalar offset address it, and accesses past the end read 0 / are dropped.
constexpr int kBufferConfig = 0x00020000;  // raw 32-bit dword format (gfx9 family)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufferConfig);
}
typedef __attribute__((address_space(3))) void lds_void;

// ---- misc -------------------------------------------------------------------
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace lf
