// Masked bidirectional attention for packed rows on gfx950 matrix cores,
// flash style: scores and the running softmax stay on chip, K and V tiles
// are staged through LDS, and the output is written token-major ([token][head
// * 64 + d]) so the output projection reads it with no transpose (the
// strided attention output of "perf(model): exact Metal speed-ups of the
// forward pass").  A work item (AttnBlock) is up to 64 queries of one batch
// row; the key-padding mask is the row's length and, on local layers, a query
// at position p sees key j iff |p - j| <= half_window.  The same kernel
// serves the marker-row subset: its queries are an arbitrary list of rows of
// the query buffer, each with its own position, while keys are the whole row
// (a single query row applies the mask like any other, which the pages'
// Metal single-query kernel did not).
//
// Layout of the work, per workgroup (one block x one head, 4 waves of 16
// queries), per 64-key tile:
//   - S^T = K Q^T with v_mfma_f32_16x16x32_bf16: keys are the MFMA rows and
//     queries the columns, so each lane ends up with 16 scores of ONE query
//     (lane l: query l%16, keys 8*(l/16)+0..7 of each 32-key half);
//   - online softmax in float32, exp2 domain: each tile's maximum is
//     reduced over the 4 lanes of a query with the gfx950 lane swaps
//     (v_permlane16_swap, v_permlane32_swap: plain VALU moves, no LDS round
//     trip), and the reference maximum that the weights are taken against
//     moves only when a score passes it by more than 2^8, so the
//     accumulators are rarely rescaled; tiles inside every window of the
//     wave skip the mask;
//   - O^T += V^T P^T: P^T is the MFMA B operand, whose lane layout (query
//     l%16, 8 consecutive k slots per lane) is exactly the lane's own scores
//     once the K rows of S^T are fed in the matching order, so P never leaves
//     the registers.  V^T comes from the transposed V that the QKV GEMM
//     writes (each row's keys start at a 64-aligned column).  The row sum is
//     the same product with an all-ones A operand.
// The matrix cores take BF16 operands, so the float32 P is split into a BF16
// head and a BF16 tail (p = hi + lo to about 16 significant bits) and both
// halves are multiplied with V: rounding P to BF16 alone would perturb every
// output by up to 2^-9 relative, a first-order departure from float32
// softmax (measured ~2e-3 nRMS; fp16 P, 2^-12, still ~8e-4 and 1.6x the
// first layer's error against the oracle).
//
// K and V^T tiles go HBM -> LDS with buffer loads (no VGPR staging) into two
// buffers: the next tile's loads are in flight while this tile is computed,
// with one barrier per tile.
#include "kernels.h"

namespace laya {

namespace {

constexpr int KT = 64;                 // keys per tile
constexpr int TILE_ELEMS = 64 * 64;    // one 64 x 64 BF16 tile
constexpr int BUF_ELEMS = 2 * TILE_ELEMS;  // K tile, then V^T tile

// Physical 16-byte chunk of logical chunk c in row r of a 128-byte-row tile.
// Two rows share one 256-byte sweep of the 64 banks; the XOR spreads the 16
// rows that one ds_read_b128 quarter-wave reads over all 16 chunk slots.
// K tile rows are read 16 at a time as keys {0..3, 8..11, 16..19, 24..27}
// (+ 4 e + 32 ks), V^T tile rows as 16 consecutive rows.
__device__ __forceinline__ int kchunk(int r, int c) {
    return c ^ (((r >> 1) & 1) | ((r >> 2) & 6));
}
__device__ __forceinline__ int vchunk(int r, int c) { return c ^ ((r >> 1) & 7); }

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void attention_kernel(
    AttnParams p) {
    const int32_t nblk = p.nblk_dev ? *p.nblk_dev : p.nblk_max;
    // (block, head) work index: the blocks of one head are consecutive, and
    // contiguous ranges go to one XCD, so a row's K/V tiles are fetched into
    // one L2 for all of its blocks.
    const int u = xcd_contiguous(blockIdx.y * gridDim.x + blockIdx.x, nblk * p.n_heads);
    if (u < 0) return;
    const int h = u / nblk;
    const AttnBlock blk = p.blocks[u - h * nblk];

    __shared__ __attribute__((aligned(16))) bf16_t smem[2 * BUF_ELEMS];

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, c16 = lane & 15;

    // This lane's query (MFMA column c16 of wave w), clamped to a valid row.
    const int qi = w * 16 + c16;
    const bool qvalid = qi < blk.q_count;
    const int32_t qrow = blk.q_first + (qvalid ? qi : 0);
    const bf16_t *qp = p.q + (size_t)qrow * p.ldq + h * 64;
    const bf16x8_t qb0 = as_bf16x8(ld16(qp + 8 * g));       // dims 8g..8g+7
    const bf16x8_t qb1 = as_bf16x8(ld16(qp + 32 + 8 * g));  // dims 32+8g..
    const int32_t my_pos = p.qpos[qrow];

    // DMA sources.  Each wave loads 1 KB blocks jj = w and w + 4 of each tile
    // (rows 8 jj .. 8 jj + 7); lane L fills physical chunk L % 8 of row
    // 8 jj + L / 8 with the logical chunk the swizzle puts there.
    const int dr = lane >> 3, dpc = lane & 7;
    uint32_t koff[2], voff[2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int r = 8 * (w + 4 * it) + dr;
        koff[it] = (uint32_t)(((blk.kt0 + r) * p.ldk + h * 64 + kchunk(r, dpc) * 8) * 2);
        voff[it] = (uint32_t)(((h * 64 + r) * p.ldvt + blk.vcol0 + vchunk(r, dpc) * 8) * 2);
    }
    const int w_u = __builtin_amdgcn_readfirstlane(w);
    auto issue = [&](int32_t kb, int buf) {
        bf16_t *base = smem + buf * BUF_ELEMS;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int jj = w_u + 4 * it;
            // the tile offset goes into the per-lane offset, which is what the
            // buffer's range check covers
            dma16(p.k, p.k_bytes, (lds_ptr_t)(base + jj * 512),
                  koff[it] + (uint32_t)(kb * p.ldk * 2), 0);
            dma16(p.vt, p.vt_bytes, (lds_ptr_t)(base + TILE_ELEMS + jj * 512),
                  voff[it] + (uint32_t)(kb * 2), 0);
        }
    };

    // Keys this lane's query may see: [q_lo, q_hi) (row end and window), and
    // the keys every query of the wave sees, [w_lo, w_hi): tiles inside that
    // range need no mask.
    const int32_t q_lo = p.half_window < 0 ? 0 : max(0, my_pos - p.half_window);
    const int32_t q_hi =
        p.half_window < 0 ? blk.k_hi : min(blk.k_hi, my_pos + p.half_window + 1);
    const uint32_t q_span = (uint32_t)(q_hi - q_lo);
    // Reduced over each 16-lane row (one lane per query) by DPP moves:
    // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row half mirror, row mirror.
    // All 64 lanes are active here (invalid queries are clamped, not
    // masked off), so no DPP source lane is disabled.
    int32_t w_lo = q_lo, w_hi = q_hi;
    w_lo = max(w_lo, __builtin_amdgcn_update_dpp(0, w_lo, 0xB1, 0xF, 0xF, false));
    w_hi = min(w_hi, __builtin_amdgcn_update_dpp(0, w_hi, 0xB1, 0xF, 0xF, false));
    w_lo = max(w_lo, __builtin_amdgcn_update_dpp(0, w_lo, 0x4E, 0xF, 0xF, false));
    w_hi = min(w_hi, __builtin_amdgcn_update_dpp(0, w_hi, 0x4E, 0xF, 0xF, false));
    w_lo = max(w_lo, __builtin_amdgcn_update_dpp(0, w_lo, 0x141, 0xF, 0xF, false));
    w_hi = min(w_hi, __builtin_amdgcn_update_dpp(0, w_hi, 0x141, 0xF, 0xF, false));
    w_lo = max(w_lo, __builtin_amdgcn_update_dpp(0, w_lo, 0x140, 0xF, 0xF, false));
    w_hi = min(w_hi, __builtin_amdgcn_update_dpp(0, w_hi, 0x140, 0xF, 0xF, false));
    w_lo = __builtin_amdgcn_readfirstlane(w_lo);
    w_hi = __builtin_amdgcn_readfirstlane(w_hi);

    const float sl2 = 0.125f * 1.44269504088896341f;  // 1/sqrt(64) * log2(e)
    float m = -INFINITY;  // reference maximum, raw score units
    f32x4_t oacc[4];       // O^T rows 16 dblk + 4 g + i, column c16
#pragma unroll
    for (int d = 0; d < 4; ++d) oacc[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t lacc = {0.f, 0.f, 0.f, 0.f};  // running row sum (all 4 elements)
    const bf16x8_t ones = as_bf16x8(u32x4_t{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});

    int buf = 0;
    if (blk.k_lo < blk.k_hi) issue(blk.k_lo, 0);
    for (int32_t kb = blk.k_lo; kb < blk.k_hi; kb += KT, buf ^= 1) {
        wait_vmcnt<0>();  // this wave's loads of the tile (and the Q loads)
        if (kb + KT > blk.k_hi) {
            // Keys past the row's end may hold anything (other rows, stale
            // memory): their P is 0, and their V is zeroed here, in the rows
            // this wave loaded, so that 0 * V stays 0.
            bf16_t *sVw = smem + buf * BUF_ELEMS + TILE_ELEMS;
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int r = 8 * (w + 4 * it) + dr;
                const int left = blk.k_hi - kb - 8 * vchunk(r, dpc);  // valid keys in the chunk
                if (left < 8) {
                    u32x4_t *cp = reinterpret_cast<u32x4_t *>(&sVw[r * 64 + dpc * 8]);
                    u32x4_t v = *cp;
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd)
                        v[qd] &= (2 * qd < left ? 0x0000ffffu : 0u) |
                                 (2 * qd + 1 < left ? 0xffff0000u : 0u);
                    *cp = v;
                }
            }
            wait_lgkmcnt<0>();
        }
        ring_barrier();  // every wave's loads landed; the other buffer is free
        if (kb + KT < blk.k_hi) issue(kb + KT, buf ^ 1);
        const bf16_t *sK = smem + buf * BUF_ELEMS;
        const bf16_t *sV = sK + TILE_ELEMS;

        // S^T: block b = 2 ks + e covers keys 32 ks + 8 (m/4) + 4 e + m%4 for
        // MFMA row m, so output row 4g + i of block b is key 32 ks + 8 g + 4 e + i.
        f32x4_t s[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int r = 32 * (b >> 1) + 8 * (c16 >> 2) + 4 * (b & 1) + (c16 & 3);
            const bf16x8_t k0 =
                *reinterpret_cast<const bf16x8_t *>(&sK[r * 64 + kchunk(r, g) * 8]);
            const bf16x8_t k1 =
                *reinterpret_cast<const bf16x8_t *>(&sK[r * 64 + kchunk(r, 4 + g) * 8]);
            f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qb0, z, 0, 0, 0);
            s[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qb1, z, 0, 0, 0);
        }

        // mask, only on tiles that are not inside every window of the wave;
        // s[b][i] is key kb + 32 (b/2) + 8 g + 4 (b%2) + i
        if (!(kb >= w_lo && kb + KT <= w_hi)) {
            const int32_t base = kb + 8 * g - q_lo;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t rel = (uint32_t)(base + 32 * (b >> 1) + 4 * (b & 1) + i);
                    s[b][i] = rel < q_span ? s[b][i] : -INFINITY;
                }
        }
        // this tile's maximum in raw score units (the scale is positive),
        // reduced over the 4 lanes of a query (rows of 16 lanes swapped
        // pairwise, then the two halves of the wave).  Two chains of
        // max(max(a, b), c), which the compiler fuses into three-input
        // v_max3_f32: 8 instructions for the 16 scores instead of 12.
        float mx = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
        mx = fmaxf(fmaxf(mx, s[0][3]), s[1][0]);
        mx = fmaxf(fmaxf(mx, s[1][1]), s[1][2]);
        mx = fmaxf(fmaxf(mx, s[1][3]), s[2][0]);
        float my = fmaxf(fmaxf(s[2][1], s[2][2]), s[2][3]);
        my = fmaxf(fmaxf(my, s[3][0]), s[3][1]);
        my = fmaxf(fmaxf(my, s[3][2]), s[3][3]);
        mx = fmaxf(mx, my);
        {
            const uint32_t xb = __float_as_uint(mx);
            const auto r16 = __builtin_amdgcn_permlane16_swap(xb, xb, false, false);
            mx = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
            const uint32_t yb = __float_as_uint(mx);
            const auto r32 = __builtin_amdgcn_permlane32_swap(yb, yb, false, false);
            mx = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
        }
        // The reference maximum m follows the scores lazily: it moves only
        // when a score exceeds it by more than 8 after scaling (2^8 in the
        // weights), or at the first unmasked keys, so rescaling the
        // accumulators is rare and the weights stay at most 2^8.  The
        // normalisation by the row sum makes the result independent of m.
        float alpha = 1.f;
        if (mx * sl2 > fmaf(m, sl2, 8.f)) {
            if (m != -INFINITY) alpha = __builtin_amdgcn_exp2f((m - mx) * sl2);
            m = mx;
        }
        const float neg = m == -INFINITY ? 0.f : -m * sl2;
        // P = 2^(s * scale - m * scale), split into BF16 hi + lo and packed
        // as the B operand of each 32-key half: slot 4 e + i <- block 2 ks + e,
        // element i (masked keys: 2^-inf = 0).
        u32x4_t ph[2], pl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int b0 = 2 * ks + (qd >> 1), i0 = 2 * (qd & 1);
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[b0][i0], sl2, neg));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[b0][i0 + 1], sl2, neg));
                const uint32_t hi = cvt_pk_bf16(p0, p1);
                ph[ks][qd] = hi;
                pl[ks][qd] = cvt_pk_bf16(p0 - bf16lo(hi), p1 - bf16hi(hi));  // exact tails
            }
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {  // the reference moved for some query
#pragma unroll
            for (int d = 0; d < 4; ++d) oacc[d] *= alpha;
            lacc *= alpha;
        }

        // O^T[d][q] += V^T[d][keys] (P_hi + P_lo)^T[keys][q]; V^T row
        // 16 dblk + c16, keys 32 ks + 8 g .. + 7 (logical chunk 4 ks + g).  The
        // row sum is the same product with an all-ones A operand, so every
        // lane gets its query's sum of exactly the weights that multiply V.
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x8_t phb = as_bf16x8(ph[ks]), plb = as_bf16x8(pl[ks]);
            bf16x8_t vb[4];
#pragma unroll
            for (int dblk = 0; dblk < 4; ++dblk) {
                const int r = 16 * dblk + c16;
                vb[dblk] = *reinterpret_cast<const bf16x8_t *>(
                    &sV[r * 64 + vchunk(r, 4 * ks + g) * 8]);
            }
            // independent accumulators between dependent MFMAs
#pragma unroll
            for (int dblk = 0; dblk < 4; ++dblk)
                oacc[dblk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb[dblk], phb, oacc[dblk], 0, 0, 0);
            lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, phb, lacc, 0, 0, 0);
#pragma unroll
            for (int dblk = 0; dblk < 4; ++dblk)
                oacc[dblk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb[dblk], plb, oacc[dblk], 0, 0, 0);
            lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, plb, lacc, 0, 0, 0);
        }
    }

    // O / l stored as BF16 at [q row][h*64 + 16 dblk + 4 g + i]
    const float lsum = lacc[0];
    if (!qvalid) return;
    bf16_t *op = p.o + (size_t)qrow * p.ldo + h * 64 + 4 * g;
#pragma unroll
    for (int dblk = 0; dblk < 4; ++dblk) {
        const f32x4_t v = oacc[dblk];
        *reinterpret_cast<u32x2_t *>(op + 16 * dblk) =
            u32x2_t{pack_bf16x2(v[0] / lsum, v[1] / lsum), pack_bf16x2(v[2] / lsum, v[3] / lsum)};
    }
}

}  // namespace

hipError_t launch_attention(hipStream_t s, const AttnParams &p) {
    if (p.nblk_max <= 0) return hipSuccess;
    hipLaunchKernelGGL(attention_kernel, dim3(p.nblk_max, p.n_heads), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace laya
