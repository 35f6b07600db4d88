// Shared device helpers for the gfx950 kernels of the encoder pass.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // BF16 bit pattern in memory

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define LAYA_DEV __device__ __forceinline__

// BF16 -> float32 is exact: the 16 bits become the high half of the word.
LAYA_DEV float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
LAYA_DEV float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
LAYA_DEV float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> BF16 bits, round to nearest even; NaN stays a quiet NaN.
LAYA_DEV uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

LAYA_DEV uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Wave-wide (64 lanes) butterfly sums / maxima.
LAYA_DEV float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Reduction across the 16 lanes that share (lane / 16), i.e. xor 1, 2, 4, 8.
LAYA_DEV float group16_sum(float v) {
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}
LAYA_DEV float group16_max(float v) {
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// 16-byte global load / store helpers.
LAYA_DEV u32x4_t ld16(const void *p) { return *reinterpret_cast<const u32x4_t *>(p); }
LAYA_DEV void st16(void *p, u32x4_t v) { *reinterpret_cast<u32x4_t *>(p) = v; }

LAYA_DEV bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
