// Memory-bound kernels of the encoder pass: weight generation, embedding
// gather, row gather, fused residual + LayerNorm, and RoPE.
#include "kernels.h"

namespace laya {

// ---------------------------------------------------------------------------
// Weight generator.  There is no checkpoint, so each weight element is drawn
// from a counter: three SplitMix64 outputs (Steele, Lea and Flood, OOPSLA
// 2014) of key (tensor_id << 40 | 3*idx + j), their twelve 16-bit fields
// summed (Irwin-Hall(12): mean 0, variance ~1 after centring and scaling by
// 2^-16, exact in float32), times 0.02, rounded to BF16.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t splitmix_at(uint64_t seed, uint64_t key) {
    uint64_t z = seed + (key + 1ull) * 0x9e3779b97f4a7c15ull;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

__global__ void init_weights_kernel(bf16_t *dst, uint64_t n, uint64_t seed, uint32_t tid) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        uint32_t s = 0;
#pragma unroll
        for (uint32_t j = 0; j < 3; ++j) {
            uint64_t r = splitmix_at(seed, ((uint64_t)tid << 40) | (3ull * i + j));
            s += (uint32_t)(r & 0xffffu) + (uint32_t)((r >> 16) & 0xffffu) +
                 (uint32_t)((r >> 32) & 0xffffu) + (uint32_t)(r >> 48);
        }
        float z = ((float)s - 393210.0f) * (1.0f / 65536.0f);
        dst[i] = (bf16_t)f32_to_bf16(0.02f * z);
    }
}

hipError_t launch_init_weights(hipStream_t s, bf16_t *dst, uint64_t n, uint64_t seed,
                               uint32_t tensor_id) {
    if (n == 0) return hipSuccess;
    uint64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(init_weights_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, dst, n,
                       seed, tensor_id);
    return hipGetLastError();
}

__global__ void fill_f32_kernel(float *dst, int32_t n, float value) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = value;
}

hipError_t launch_fill_f32(hipStream_t s, float *dst, int32_t n, float value) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, dst, n, value);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Embedding gather: out[t] = emb[ids[t]], 16 bytes per thread (bit-exact).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gather_kernel(const bf16_t *__restrict__ emb,
                                                     const int32_t *__restrict__ ids,
                                                     const int32_t *count_dev, int32_t count_max,
                                                     int32_t chunks, bf16_t *__restrict__ out) {
    const int32_t T = count_dev ? *count_dev : count_max;
    const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
    const uint32_t t = gid / (uint32_t)chunks;
    const uint32_t c = gid - t * (uint32_t)chunks;
    if ((int32_t)t >= T) return;
    const uint32_t id = (uint32_t)ids[t];
    const uint32_t hid = (uint32_t)chunks * 8u;
    st16(out + t * hid + c * 8u, ld16(emb + id * hid + c * 8u));
}

hipError_t launch_gather(hipStream_t s, const bf16_t *emb, const int32_t *ids,
                         const int32_t *count_dev, int32_t count_max, int32_t hidden,
                         bf16_t *out) {
    if (count_max <= 0) return hipSuccess;
    const int32_t chunks = hidden / 8;
    const int64_t threads = (int64_t)count_max * chunks;
    hipLaunchKernelGGL(gather_kernel, dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, s,
                       emb, ids, count_dev, count_max, chunks, out);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void gather_rows_kernel(const bf16_t *__restrict__ src,
                                                          int32_t ld_src,
                                                          const int32_t *__restrict__ idx,
                                                          int32_t n, int32_t chunks,
                                                          bf16_t *__restrict__ dst,
                                                          int32_t ld_dst) {
    const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
    const uint32_t r = gid / (uint32_t)chunks;
    const uint32_t c = gid - r * (uint32_t)chunks;
    if ((int32_t)r >= n) return;
    const uint32_t srow = (uint32_t)idx[r];
    st16(dst + r * (uint32_t)ld_dst + c * 8u, ld16(src + srow * (uint32_t)ld_src + c * 8u));
}

hipError_t launch_gather_rows(hipStream_t s, const bf16_t *src, int32_t ld_src,
                              const int32_t *idx, int32_t n, int32_t cols, bf16_t *dst,
                              int32_t ld_dst) {
    if (n <= 0) return hipSuccess;
    const int32_t chunks = cols / 8;
    const int64_t threads = (int64_t)n * chunks;
    hipLaunchKernelGGL(gather_rows_kernel, dim3((uint32_t)((threads + 255) / 256)), dim3(256),
                       0, s, src, ld_src, idx, n, chunks, dst, ld_dst);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused residual add + LayerNorm, one 64-lane wave per row, 4 rows per block.
//   x <- bf16(x + r)  (when r != nullptr; written back)
//   n <- bf16((x - mean) / sqrt(var + eps) * gamma)
// mean and biased variance in float32 (two passes over the row held in
// registers).  Each lane holds up to MAXC 16-byte chunks of the row.
// ---------------------------------------------------------------------------
template <int MAXC>
__global__ __launch_bounds__(256) void layernorm_kernel(bf16_t *__restrict__ x,
                                                        const bf16_t *__restrict__ r,
                                                        bf16_t *__restrict__ n,
                                                        const float *__restrict__ gamma,
                                                        const int32_t *count_dev,
                                                        int32_t count_max, int32_t hidden,
                                                        float eps) {
    const int32_t T = count_dev ? *count_dev : count_max;
    const int32_t row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= T) return;
    const int nch = hidden >> 3;
    bf16_t *xr = x + (uint32_t)row * (uint32_t)hidden;
    float v[MAXC][8];
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + c * 64;
        if (ch < nch) {
            u32x4_t a = ld16(xr + ch * 8);
            if (r != nullptr) {
                u32x4_t b = ld16(r + (uint32_t)row * (uint32_t)hidden + ch * 8);
                u32x4_t o;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float lo = bf16_to_f32(f32_to_bf16(bf16lo(a[q]) + bf16lo(b[q])));
                    float hi = bf16_to_f32(f32_to_bf16(bf16hi(a[q]) + bf16hi(b[q])));
                    v[c][2 * q] = lo;
                    v[c][2 * q + 1] = hi;
                    o[q] = pack_bf16x2(lo, hi);
                }
                st16(xr + ch * 8, o);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v[c][2 * q] = bf16lo(a[q]);
                    v[c][2 * q + 1] = bf16hi(a[q]);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) sum += v[c][e];
        }
    }
    layernorm_row_store<MAXC>(v, sum, lane, nch, hidden, eps, gamma,
                              n + (uint32_t)row * (uint32_t)hidden);
}

hipError_t launch_layernorm(hipStream_t s, bf16_t *x, const bf16_t *r, bf16_t *n,
                            const float *gamma, const int32_t *count_dev, int32_t count_max,
                            int32_t hidden, float eps) {
    if (count_max <= 0) return hipSuccess;
    const dim3 grid((count_max + 3) / 4), block(256);
    const int maxc = (hidden / 8 + 63) / 64;
    switch (maxc) {
        case 1:
            hipLaunchKernelGGL(layernorm_kernel<1>, grid, block, 0, s, x, r, n, gamma,
                               count_dev, count_max, hidden, eps);
            break;
        case 2:
            hipLaunchKernelGGL(layernorm_kernel<2>, grid, block, 0, s, x, r, n, gamma,
                               count_dev, count_max, hidden, eps);
            break;
        case 3:
        case 4:
            hipLaunchKernelGGL(layernorm_kernel<4>, grid, block, 0, s, x, r, n, gamma,
                               count_dev, count_max, hidden, eps);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RoPE in place.  One thread per (row, rotated head, group of 8 pairs), with
// 32-bit index arithmetic throughout: pairs (i, i+32) of a 64-wide head are
// rotated by the BF16 table entries of the row's position,
//   v[i] <- bf16(x c - y s),  v[i+32] <- bf16(y c + x s),
// where both products of BF16 values are exact in float32, so each output has
// a single float32 rounding before the BF16 one.  Columns past the rotated
// heads (the V block) are never touched.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rope_kernel(bf16_t *__restrict__ buf, int32_t ld,
                                                   int32_t n_rot, const int32_t *count_dev,
                                                   int32_t rows_max,
                                                   const int32_t *__restrict__ pos,
                                                   const bf16_t *__restrict__ cos_tab,
                                                   const bf16_t *__restrict__ sin_tab) {
    const int32_t rows = count_dev ? *count_dev : rows_max;
    const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
    const uint32_t per_row = (uint32_t)n_rot * 4u;
    const uint32_t row = gid / per_row;
    const uint32_t rem = gid - row * per_row;
    const uint32_t head = rem >> 2, grp = rem & 3u;
    if ((int32_t)row >= rows) return;
    const uint32_t p = (uint32_t)pos[row];
    bf16_t *hp = buf + row * (uint32_t)ld + head * 64u + grp * 8u;
    const u32x4_t xv = ld16(hp);
    const u32x4_t yv = ld16(hp + 32);
    const u32x4_t cv = ld16(cos_tab + p * 32u + grp * 8u);
    const u32x4_t sv = ld16(sin_tab + p * 32u + grp * 8u);
    u32x4_t xo, yo;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float x0 = bf16lo(xv[q]), x1 = bf16hi(xv[q]);
        const float y0 = bf16lo(yv[q]), y1 = bf16hi(yv[q]);
        const float c0 = bf16lo(cv[q]), c1 = bf16hi(cv[q]);
        const float s0 = bf16lo(sv[q]), s1 = bf16hi(sv[q]);
        // fmaf(x, c, -(y*s)): y*s is exact, so this is the correctly rounded x*c - y*s.
        xo[q] = pack_bf16x2(fmaf(x0, c0, -(y0 * s0)), fmaf(x1, c1, -(y1 * s1)));
        yo[q] = pack_bf16x2(fmaf(y0, c0, x0 * s0), fmaf(y1, c1, x1 * s1));
    }
    st16(hp, xo);
    st16(hp + 32, yo);
}

// RoPE in the pages' original launch geometry, kept as the reference arm of
// the RoPE comparison ("perf(model): exact Metal speed-ups of the forward
// pass": the rotary kernel it replaced found every element's coordinates by
// 64-bit integer division, a software routine on the GPU).  One thread
// per rotation pair over a flat 64-bit index, split back into (row, head,
// pair) with 64-bit division and remainder; the same arithmetic per pair as
// rope_kernel, so the two give bitwise equal results.
__global__ __launch_bounds__(256) void rope_original_kernel(
    bf16_t *__restrict__ buf, int32_t ld, int32_t n_rot, const int32_t *count_dev,
    int32_t rows_max, const int32_t *__restrict__ pos, const bf16_t *__restrict__ cos_tab,
    const bf16_t *__restrict__ sin_tab) {
    const uint64_t rows = (uint64_t)(count_dev ? *count_dev : rows_max);
    const uint64_t idx = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t per_row = (uint64_t)n_rot * 32u;
    const uint64_t row = idx / per_row;
    const uint64_t rem = idx % per_row;
    const uint64_t head = rem / 32u, i = rem % 32u;
    if (row >= rows) return;
    const uint64_t p = (uint64_t)pos[row];
    bf16_t *hp = buf + row * (uint64_t)ld + head * 64u + i;
    const float x = bf16_to_f32(hp[0]), y = bf16_to_f32(hp[32]);
    const float c = bf16_to_f32(cos_tab[p * 32u + i]), sn = bf16_to_f32(sin_tab[p * 32u + i]);
    // both products of BF16 values are exact in float32
    hp[0] = (bf16_t)f32_to_bf16(fmaf(x, c, -(y * sn)));
    hp[32] = (bf16_t)f32_to_bf16(fmaf(y, c, x * sn));
}

hipError_t launch_rope_original(hipStream_t s, bf16_t *buf, int32_t ld, int32_t n_heads_rot,
                                const int32_t *count_dev, int32_t rows_max, const int32_t *pos,
                                const bf16_t *cos_tab, const bf16_t *sin_tab) {
    if (rows_max <= 0) return hipSuccess;
    const int64_t threads = (int64_t)rows_max * n_heads_rot * 32;
    hipLaunchKernelGGL(rope_original_kernel, dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0,
                       s, buf, ld, n_heads_rot, count_dev, rows_max, pos, cos_tab, sin_tab);
    return hipGetLastError();
}

hipError_t launch_rope(hipStream_t s, bf16_t *buf, int32_t ld, int32_t n_heads_rot,
                       const int32_t *count_dev, int32_t rows_max, const int32_t *pos,
                       const bf16_t *cos_tab, const bf16_t *sin_tab) {
    if (rows_max <= 0) return hipSuccess;
    const int64_t threads = (int64_t)rows_max * n_heads_rot * 4;
    hipLaunchKernelGGL(rope_kernel, dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, s,
                       buf, ld, n_heads_rot, count_dev, rows_max, pos, cos_tab, sin_tab);
    return hipGetLastError();
}

}  // namespace laya
