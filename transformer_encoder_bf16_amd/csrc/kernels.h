// Internal launch functions of the gfx950 kernels.  Every launch queues on
// the given stream and returns the launch status; none synchronises.
//
// Row counts: where a kernel takes (count_dev, count_max), it processes
// *count_dev rows when count_dev != nullptr (read on the device, so a captured
// graph serves any count <= count_max) and count_max rows otherwise.  Grids
// are always sized for count_max; surplus workgroups exit at once.
#pragma once

#include "common.h"

namespace laya {

// Attention work item: up to 64 queries of one batch row, one head per
// workgroup.  Keys of the row are tokens kt0 .. kt0+klen-1 (positions
// 0..klen-1) of the K buffer and columns vcol0 .. vcol0+klen-1 of the
// transposed V; the block only visits key positions [k_lo, k_hi), k_lo a
// multiple of 64.  Queries are rows q_first .. q_first+q_count-1 of the
// query/output buffers, with positions qpos[q_first + i].
struct AttnBlock {
    int32_t kt0, klen, k_lo, k_hi, q_first, q_count, vcol0, pad;
};
static_assert(sizeof(AttnBlock) == 32, "AttnBlock is 8 int32");

constexpr int kAttnQueries = 64;  // queries per block

hipError_t launch_init_weights(hipStream_t s, bf16_t *dst, uint64_t n, uint64_t seed,
                               uint32_t tensor_id);

hipError_t launch_fill_f32(hipStream_t s, float *dst, int32_t n, float value);

hipError_t launch_gather(hipStream_t s, const bf16_t *emb, const int32_t *ids,
                         const int32_t *count_dev, int32_t count_max, int32_t hidden,
                         bf16_t *out);

// dst[r][0:cols] = src[idx[r]][0:cols] for r < n (bit-exact).
hipError_t launch_gather_rows(hipStream_t s, const bf16_t *src, int32_t ld_src,
                              const int32_t *idx, int32_t n, int32_t cols, bf16_t *dst,
                              int32_t ld_dst);

hipError_t launch_layernorm(hipStream_t s, bf16_t *x, const bf16_t *r, bf16_t *n,
                            const float *gamma, const int32_t *count_dev, int32_t count_max,
                            int32_t hidden, float eps);

// GEMM tile configuration and K split.  Every output element is one MFMA
// chain per K range, the ranges summed in order, so a result depends only on
// `splits` (never on the tile shape).
constexpr int kGemmConfigs = 12;
constexpr int kPingPongConfig = 9;
struct GemmPlan {
    int config;  // 0 XS 32x64, 1 XSG 64x64, 2 S 128x64, 3 M 128x128, 4 L 256x128, 5 XL 256x256,
                 // 6 M2 128x128 with a 2-stage ring (two workgroups per CU),
                 // 7 XS2 32x64 and 8 XSG2 64x64 (two computing waves each, deep
                 // rings; XS2 with two more waves that only load),
                 // 9 P 256x256 with two wave groups in ping-pong (whole K),
                 // 10 Q3 192x256 (three heads, twelve waves, three per SIMD),
                 // 11 W2 256x192 (eight waves of 64x96); whole K for 4..6, 9..11
    int splits;  // K ranges (>= 1)
};
// plan for a GEMM of up to M_max rows (its K split and tile shape; the split
// thresholds are 64, 256, 1024 and 2048 rows); plan_gemm_tiles: the best
// whole-K tile shape for M rows.
GemmPlan plan_gemm(int32_t M_max, int32_t N, int32_t K, int epilogue);
GemmPlan plan_gemm_tiles(int32_t M, int32_t N, int32_t K, int epilogue);
int gemm_max_splits(int config);
// float32 partial-tile bytes a plan needs (0 when splits == 1)
size_t gemm_workspace_bytes(const GemmPlan &g, int32_t M_max, int32_t N, int epilogue);
// The library's own split-K scratch on the current device (for callers that
// cannot allocate): its size, and its device address (looked up once per
// device; every call on one device shares it).
size_t gemm_static_scratch_bytes();
hipError_t gemm_static_scratch(float **ptr);

// Epilogue 2 (QKV projection): output columns [0, rope_cols) are heads of
// 64 that are rotated (RoPE, rotate-half pairs (i, i+32), c/s = tab[pos][i])
// after rounding to BF16, exactly as the standalone RoPE kernel does;
// columns [vt_col0, N) are stored transposed, column f of token t at
// vt[(f - vt_col0) * ldvt + vt_tok[t]]; columns in between are stored plain.
// rope_cols and vt_col0 are multiples of 64.
struct QkvEpilogue {
    const int32_t *pos;               // position of each output row (token)
    const bf16_t *cos_tab, *sin_tab;  // [positions][32]
    int32_t rope_cols;
    int32_t vt_col0;
    bf16_t *vt;
    int32_t ldvt;
    const int32_t *vt_tok;  // vt column of each output row
};

// C = bf16(A W^T), epilogue 0 plain, 1 GeGLU (W has 2N rows), 2 QKV (`qe`),
// 3 bias then GELU.  `bias` ([N], BF16, optional for 0 and 2, required for 3,
// not allowed for 1): y = bf16(bf16(A W^T) + bias).  With plan.splits > 1,
// `partial` is required and two kernels are queued.  `res` (epilogue 0, whole
// K, any tile shape but the ping-pong one; 16-byte aligned, row stride ldc, may
// be C): C = bf16(res + y), the residual add, bitwise as launch_layernorm's.
hipError_t launch_gemm(hipStream_t s, const bf16_t *A, int32_t lda, const bf16_t *W,
                       int32_t ldw, bf16_t *C, int32_t ldc, const int32_t *M_dev,
                       int32_t M_max, int32_t N, int32_t K, int epilogue, const GemmPlan &plan,
                       float *partial, const QkvEpilogue *qe = nullptr,
                       const bf16_t *bias = nullptr, const bf16_t *res = nullptr);

// A projection onto the hidden width (N <= 1024) followed by the residual add
// and LayerNorm: x <- bf16(x + bf16(A W^T) [+ bias, rounded again]),
// n <- bf16(LN(x) * gamma).  Bitwise the same as launch_gemm with this plan
// (C = r) followed by launch_layernorm(x, r, n).  With a K split
// (plan.splits >= 2) the reduce launch does the residual add and the
// LayerNorm, one launch fewer; with whole K (plan.splits == 1) the GEMM's
// store does the residual add into x and launch_layernorm(x, nullptr, n)
// follows, so the LayerNorm reads one input instead of two.
hipError_t launch_gemm_layernorm(hipStream_t s, const bf16_t *A, int32_t lda, const bf16_t *W,
                                 int32_t ldw, const int32_t *M_dev, int32_t M_max, int32_t N,
                                 int32_t K, const GemmPlan &plan, float *partial,
                                 const bf16_t *bias, bf16_t *x, bf16_t *n, const float *gamma,
                                 float eps);

hipError_t launch_rope(hipStream_t s, bf16_t *buf, int32_t ld, int32_t n_heads_rot,
                       const int32_t *count_dev, int32_t rows_max, const int32_t *pos,
                       const bf16_t *cos_tab, const bf16_t *sin_tab);
// The same rotation in the original launch geometry (one thread per pair,
// 64-bit index division); bitwise equal to launch_rope.
hipError_t launch_rope_original(hipStream_t s, bf16_t *buf, int32_t ld, int32_t n_heads_rot,
                                const int32_t *count_dev, int32_t rows_max, const int32_t *pos,
                                const bf16_t *cos_tab, const bf16_t *sin_tab);

// Attention over packed rows.  q [rows][ldq] (head h at columns h*64..),
// k [rows][ldk] likewise, vt [n_heads*64][ldvt] (row h*64+d holds
// dimension d of head h for every key column), o [rows][ldo]; all BF16.  k_bytes / vt_bytes
// bound what the kernel may read from k / vt (reads past them give zero).
struct AttnParams {
    const bf16_t *q;
    int32_t ldq;
    const bf16_t *k;
    int32_t ldk;
    uint32_t k_bytes;
    const bf16_t *vt;
    int32_t ldvt;
    uint32_t vt_bytes;
    bf16_t *o;
    int32_t ldo;
    const AttnBlock *blocks;
    const int32_t *nblk_dev;
    int32_t nblk_max;
    const int32_t *qpos;
    int32_t n_heads;
    int32_t half_window;  // -1: global
};
hipError_t launch_attention(hipStream_t s, const AttnParams &p);

}  // namespace laya
