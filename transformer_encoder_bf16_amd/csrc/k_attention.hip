// Masked bidirectional attention for packed rows on gfx950 matrix cores,
// flash style: scores and the running softmax stay on chip, K/V tiles are
// staged through LDS, and the output is written token-major ([token][head *
// 64 + d]) so the output projection reads it with no transpose (the strided
// attention output of "perf(model): exact Metal speed-ups of the forward
// pass").  A work item (AttnBlock) is up to 64 queries of one batch row; the
// key-padding mask is the row's length and, on local layers, a query at
// position p sees key j iff |p - j| <= half_window.  The same kernel serves
// the marker-row subset: its queries are an arbitrary list of rows of the
// query buffer, each with its own position, while keys are the whole row
// (a single query row applies the mask like any other, which the pages' Metal
// single-query kernel did not).
//
// Per workgroup: one block x one head, four waves of 16 queries.  For each
// 64-key tile: S = Q K^T with MFMA 16x16x32 (queries as rows), scale,
// mask, online softmax in float32 (max subtracted, exp2 domain), then
// O += P V with MFMA 16x16x32 reading V from a transposed LDS copy.  The
// matrix cores take BF16 operands, so the float32 P is split into a BF16 head
// and a BF16 tail (p = hi + lo to about 16 significant bits) and both halves
// are multiplied with V: rounding P to BF16 alone would perturb every output
// by up to 2^-9 relative, a first-order departure from float32 softmax.
#include "kernels.h"

namespace laya {

namespace {

constexpr int KT = 64;          // keys per tile
constexpr int LDK = 64;         // K tile row length (swizzled 16-byte chunks)
constexpr int LDV = 64 + 8;     // transposed V row length (padded)
constexpr int LDP = 64 + 8;     // P row length (padded)

__device__ __forceinline__ int kswz(int key, int chunk) {
    return key * LDK + ((chunk ^ ((key >> 1) & 7)) << 3);
}

__global__ __launch_bounds__(256) void attention_kernel(
    const bf16_t *__restrict__ q, int32_t ldq, const bf16_t *__restrict__ k,
    const bf16_t *__restrict__ v, int32_t ldkv, bf16_t *__restrict__ o, int32_t ldo,
    const AttnBlock *__restrict__ blocks, const int32_t *nblk_dev, int32_t nblk_max,
    const int32_t *__restrict__ qpos, int32_t half_window) {
    const int32_t nblk = nblk_dev ? *nblk_dev : nblk_max;
    const int32_t bi = blockIdx.x;
    if (bi >= nblk) return;
    const AttnBlock blk = blocks[bi];
    const int h = blockIdx.y;

    __shared__ __attribute__((aligned(16))) bf16_t sK[KT * LDK];
    __shared__ __attribute__((aligned(16))) bf16_t sVt[64 * LDV];
    __shared__ __attribute__((aligned(16))) bf16_t sP[4][2][16 * LDP];  // [wave][hi, lo]

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, c16 = lane & 15;

    // Q fragments: MFMA A rows are queries w*16 + c16 (clamped to a valid row).
    const int qa = w * 16 + c16;
    const int32_t qrow_a = blk.q_first + (qa < blk.q_count ? qa : 0);
    const bf16_t *qp = q + (size_t)qrow_a * ldq + h * 64;
    const bf16x8_t qf0 = as_bf16x8(ld16(qp + g * 8));
    const bf16x8_t qf1 = as_bf16x8(ld16(qp + 32 + g * 8));

    // Accumulator rows held by this lane: queries w*16 + g*4 + i.
    int32_t qp_r[4];
    bool qv_r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int qi = w * 16 + g * 4 + i;
        qv_r[i] = qi < blk.q_count;
        qp_r[i] = qpos[blk.q_first + (qv_r[i] ? qi : 0)];
    }

    const float sl2 = 0.125f * 1.44269504088896341f;  // 1/sqrt(64) * log2(e)
    float m[4], l[4];
    f32x4_t oacc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m[i] = -INFINITY;
        l[i] = 0.f;
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) oacc[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const bf16_t *kbase = k + (size_t)blk.kt0 * ldkv + h * 64;
    const bf16_t *vbase = v + (size_t)blk.kt0 * ldkv + h * 64;

    for (int32_t kb = blk.k_lo; kb < blk.k_hi; kb += KT) {
        __syncthreads();  // the previous tile's readers are done
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int idx = tid + 256 * it;
            const int key = idx >> 3, ch = idx & 7;
            const int32_t kj = kb + key;
            u32x4_t kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
            if (kj < blk.k_hi) {
                kv = ld16(kbase + (size_t)kj * ldkv + ch * 8);
                vv = ld16(vbase + (size_t)kj * ldkv + ch * 8);
            }
            *reinterpret_cast<u32x4_t *>(&sK[kswz(key, ch)]) = kv;
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                sVt[(ch * 8 + 2 * qd) * LDV + key] = (bf16_t)(vv[qd] & 0xffffu);
                sVt[(ch * 8 + 2 * qd + 1) * LDV + key] = (bf16_t)(vv[qd] >> 16);
            }
        }
        __syncthreads();

        // S = Q K^T: four 16-key blocks, each two MFMAs over d = 0..31, 32..63.
        f32x4_t s[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int key = b * 16 + c16;
            const bf16x8_t k0 = *reinterpret_cast<const bf16x8_t *>(&sK[kswz(key, g)]);
            const bf16x8_t k1 = *reinterpret_cast<const bf16x8_t *>(&sK[kswz(key, 4 + g)]);
            f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf0, k0, z, 0, 0, 0);
            s[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf1, k1, z, 0, 0, 0);
        }

        // Mask + scale; lane holds S[query g*4+i][key b*16 + c16].
        float mx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            mx[i] = -INFINITY;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int32_t kj = kb + b * 16 + c16;
                const int32_t dpos = qp_r[i] - kj;
                const bool ok = (kj < blk.k_hi) &&
                                (half_window < 0 || (dpos <= half_window && -dpos <= half_window));
                const float t = ok ? s[b][i] * sl2 : -INFINITY;
                s[b][i] = t;
                mx[i] = fmaxf(mx[i], t);
            }
            mx[i] = group16_max(mx[i]);
        }

        bf16_t *pw = sP[w][0];
        bf16_t *pwl = sP[w][1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float mnew = fmaxf(m[i], mx[i]);
            const float alpha = (mnew == -INFINITY) ? 1.f : exp2f(m[i] - mnew);
            float rs = 0.f;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float t = s[b][i];
                const float p = (t == -INFINITY) ? 0.f : exp2f(t - mnew);
                const uint32_t ph = f32_to_bf16(p);
                const uint32_t pl = f32_to_bf16(p - bf16_to_f32(ph));  // p - hi is exact
                rs += p;
                pw[(g * 4 + i) * LDP + b * 16 + c16] = (bf16_t)ph;
                pwl[(g * 4 + i) * LDP + b * 16 + c16] = (bf16_t)pl;
            }
            l[i] = l[i] * alpha + group16_sum(rs);
            m[i] = mnew;
#pragma unroll
            for (int d = 0; d < 4; ++d) oacc[d][i] *= alpha;
        }
        __syncthreads();  // P visible to the whole wave (and V tile still valid)

        // O += (P_hi + P_lo) V: A = P [16 queries][keys], B = V [keys][d] from V^T.
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x8_t pa =
                *reinterpret_cast<const bf16x8_t *>(&pw[c16 * LDP + ks * 32 + g * 8]);
            const bf16x8_t pal =
                *reinterpret_cast<const bf16x8_t *>(&pwl[c16 * LDP + ks * 32 + g * 8]);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const bf16x8_t vb = *reinterpret_cast<const bf16x8_t *>(
                    &sVt[(d * 16 + c16) * LDV + ks * 32 + g * 8]);
                oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, oacc[d], 0, 0, 0);
                oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pal, vb, oacc[d], 0, 0, 0);
            }
        }
    }

    // O / l, stored as BF16 at [q row][h*64 + d]; lane holds O[query g*4+i][d*16 + c16].
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (!qv_r[i]) continue;
        const int32_t orow = blk.q_first + w * 16 + g * 4 + i;
        bf16_t *op = o + (size_t)orow * ldo + h * 64;
#pragma unroll
        for (int d = 0; d < 4; ++d) op[d * 16 + c16] = (bf16_t)f32_to_bf16(oacc[d][i] / l[i]);
    }
}

}  // namespace

hipError_t launch_attention(hipStream_t s, const bf16_t *q, int32_t ldq, const bf16_t *k,
                            const bf16_t *v, int32_t ldkv, bf16_t *o, int32_t ldo,
                            const AttnBlock *blocks, const int32_t *nblk_dev,
                            int32_t nblk_max, const int32_t *qpos, int32_t n_heads,
                            int32_t half_window) {
    if (nblk_max <= 0) return hipSuccess;
    hipLaunchKernelGGL(attention_kernel, dim3(nblk_max, n_heads), dim3(256), 0, s, q, ldq, k, v,
                       ldkv, o, ldo, blocks, nblk_dev, nblk_max, qpos, half_window);
    return hipGetLastError();
}

}  // namespace laya
