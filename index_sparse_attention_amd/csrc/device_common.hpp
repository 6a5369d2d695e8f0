// Device helpers for gfx950 (CDNA4): bf16 MFMA wrappers, packing, loads.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace isattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// D = A(32x16) * B(16x32) + C, fp32 accumulate.  Lane l: A row l%32 and B
// column l%32, eight k-slots 8*(l/32)..+7; C/D register i holds row
// 8*(i/4) + 4*(l/32) + i%4 of column l%32.
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D = A(16x32) * B(32x16) + C.  Lane l: A row l%16 and B column l%16, k-slots
// 8*(l/16)..+7; C/D register i holds row 4*(l/16) + i of column l%16.
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp32 pair -> packed bf16 pair, round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t x = {lo, hi};
    bf16x2_t y = __builtin_convertvector(x, bf16x2_t);
    return __builtin_bit_cast(uint32_t, y);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t w) { return __builtin_bit_cast(bf16x8_t, w); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Hardware fp32 atomic add (global_atomic_add_f32, no return value).
__device__ __forceinline__ void atomic_add_f32(float* p, float v) { unsafeAtomicAdd(p, v); }

__device__ __forceinline__ u32x4_t lds_read128(const uint16_t* p) {
    return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ u32x2_t lds_read64(const uint16_t* p) {
    return *reinterpret_cast<const u32x2_t*>(p);
}

__device__ __forceinline__ u32x4_t gload128(const uint16_t* p) {
    return *reinterpret_cast<const u32x4_t*>(p);
}

}  // namespace isattn
