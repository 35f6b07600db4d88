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

// float32 -> BF16, round to nearest even (NaN stays NaN), with the gfx950
// conversion instruction v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
LAYA_DEV uint32_t cvt_pk_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
LAYA_DEV uint32_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
LAYA_DEV uint32_t pack_bf16x2(float lo, float hi) { return cvt_pk_bf16(lo, hi); }

// Sum over a 64-lane wave, the same value in every lane.  DPP moves within
// each 16-lane row (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row half
// mirror, row mirror: pairs, quads, eights, rows), then the four row sums are
// read into scalar registers and added as (r0 + r1) + (r2 + r3).  No LDS
// round trip: a lane shuffle through ds_bpermute costs a full LDS latency per
// step, and the row statistics sit on every row's critical path.
template <int CTRL>
LAYA_DEV float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, 0xF, 0xF, false));
}
LAYA_DEV float lane_f32(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
LAYA_DEV float wave_sum(float v) {
    v += dpp_f32<0xB1>(v);
    v += dpp_f32<0x4E>(v);
    v += dpp_f32<0x141>(v);
    v += dpp_f32<0x140>(v);
    return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
}

// 16-byte global load / store helpers.
LAYA_DEV u32x4_t ld16(const void *p) { return *reinterpret_cast<const u32x4_t *>(p); }
LAYA_DEV void st16(void *p, u32x4_t v) { *reinterpret_cast<u32x4_t *>(p) = v; }

// LayerNorm of one row held by one 64-lane wave, shared by every kernel that
// ends in a LayerNorm so they round alike: lane L holds the 8 values of
// chunks L, L + 64, ... (v[c] for chunk lane + 64 c < nch) and `sum`, their
// running sum in chunk order.  Mean and biased variance in float32 (two
// passes over the registers, DPP and readlane sums over the wave), then
// n = bf16((v - mean) * rs * gamma) with rs = 1 / sqrt(var + eps), one
// division per row.  gamma is loaded before the reductions, so its latency
// overlaps them.
template <int MAXC>
LAYA_DEV void layernorm_row_store(const float (&v)[MAXC][8], float sum, int lane, int nch,
                                  int hidden, float eps, const float *__restrict__ gamma,
                                  uint16_t *__restrict__ n_row) {
    const float inv_h = 1.0f / (float)hidden;
    f32x4_t gv[MAXC][2];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + c * 64;
        if (ch < nch) {
            gv[c][0] = *reinterpret_cast<const f32x4_t *>(gamma + ch * 8);
            gv[c][1] = *reinterpret_cast<const f32x4_t *>(gamma + ch * 8 + 4);
        }
    }
    const float mean = wave_sum(sum) * inv_h;
    float sq = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        if (lane + c * 64 < nch) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = v[c][e] - mean;
                sq += d * d;
            }
        }
    }
    const float var = wave_sum(sq) * inv_h;
    const float rs = 1.0f / sqrtf(var + eps);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + c * 64;
        if (ch < nch) {
            const f32x4_t g0 = gv[c][0];
            const f32x4_t g1 = gv[c][1];
            float g[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
            u32x4_t o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float lo = ((v[c][2 * q] - mean) * rs) * g[2 * q];
                const float hi = ((v[c][2 * q + 1] - mean) * rs) * g[2 * q + 1];
                o[q] = pack_bf16x2(lo, hi);
            }
            st16(n_row + ch * 8, o);
        }
    }
}

LAYA_DEV bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// ---------------------------------------------------------------------------
// Direct HBM -> LDS loads and the waits around them.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void *lds_ptr_t;

// Last word of a buffer resource on CDNA: raw byte addressing (stride 0),
// 32-bit data format, no swizzle.
constexpr int kBufferWord3 = 0x00020000;

// 16 bytes per lane from base + voff + soff (bytes) into LDS: lane L writes
// dst + 16 L (dst is the wave's 1 KB block).  The buffer resource covers
// `bytes` bytes from base; the hardware drops accesses past its end.  These
// are buffer loads rather than global ones because LLVM's wait-count pass
// also counts a global load into LDS as an LDS access, which would force
// every wait on an LDS read behind it to lgkmcnt(0).
LAYA_DEV void dma16(const void *base, uint32_t bytes, lds_ptr_t dst, uint32_t voff,
                    uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                          kBufferWord3),
        dst, 16, voff, soff, 0, 0);
}

// s_waitcnt on vmcnt only (expcnt and lgkmcnt left at their maxima).
template <int N>
LAYA_DEV void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt on lgkmcnt only.
template <int N>
LAYA_DEV void wait_lgkmcnt() {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));
}

// Workgroup barrier for load rings.  __syncthreads() also waits for every
// outstanding global load (its release fence counts the in-flight DMA loads
// of later stages), which would drain the ring; a wave reaching this barrier
// has already waited (vmcnt) for the loads it publishes, and LDS reads are
// complete once the instructions that use them have run, so a bare
// s_barrier suffices.  The empty asm statements keep the compiler from
// moving LDS accesses across it.
LAYA_DEV void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Dispatch index -> work index such that the live work items [0, live) are
// spread evenly over the 8 XCDs as contiguous ranges (dispatch index d runs
// on XCD d % 8, and each XCD has its own L2).  Returns -1 past `live`.
LAYA_DEV int xcd_contiguous(int d, int live) {
    if (d >= live) return -1;
    const int x = d & 7, j = d >> 3;
    const int q = live >> 3, r = live & 7;
    return x * q + min(x, r) + j;
}
