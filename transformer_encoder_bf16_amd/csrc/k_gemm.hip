// BF16 GEMMs of the encoder pass on gfx950 matrix cores: C = bf16(A W^T)
// with float32 accumulation (the QKV, output-projection, GeGLU-up and down
// projections, which take most of the pass's time: 72-74% of traced kernel
// time on the pages' Hopper build, "[Performance]: Optimize native Rust/CUDA
// Laya inference #66", section Implementation priorities, which also asks
// for small-shape tiles that keep accumulation and BF16 rounding).
//
// A: activations [M tokens][K], W: weights [N][K] (nn.Linear layout), both
// K-contiguous.  The weight tile is the MFMA "A" operand (rows = output
// features) and the token tile the "B" operand (columns = tokens), so each
// lane of a 32x32 accumulator holds four consecutive output features of one
// token.
//
// One kernel template, several tile shapes (BW weight rows x BT tokens, K
// steps of BK, waves in a WW x WT grid):
//   - operands move HBM -> LDS with buffer_load_dwordx4 ... lds (no VGPR
//     staging) into a STAGES-deep ring; each wave waits for its own loads
//     with an explicit vmcnt and a bare barrier publishes the stage;
//   - the 16-byte chunks of an LDS row are XOR-swizzled with the row's place
//     in a 256-byte sweep of the 64 banks (measured: no bank conflicts),
//     realised by choosing each lane's source address, since the DMA writes
//     lanes contiguously;
//   - fragment reads for the next 16-wide K step are issued before the
//     MFMAs of the current one (two register buffers);
//   - every output element is one chain of v_mfma_f32_32x32x16_bf16 over its
//     K range, in K order, whatever the tile shape or K step: results do not
//     depend on the tile shape or on where a token sits in its tile;
//   - the output tile is assembled in LDS and written with 16-byte stores
//     along whole row segments.
//
// Split-K (few tokens and a long K, where a whole-K chain of few tiles
// would be a long serial wait on loads; at short K the second launch costs
// more than the split saves): the K range is cut
// into S contiguous pieces (multiples of 64); one launch writes each piece's
// float32 partial tile, a second launch adds the partials in piece order
// 0..S-1 and runs the epilogue.  The sum order is fixed, so results are
// deterministic.  Two launches rather than a last-arriving workgroup: on a
// multi-XCD part a device-scope fence writes back the XCD's whole L2, which
// cost tens of microseconds when every workgroup issued one.  A projection
// onto the hidden width is always followed by the residual add and a
// LayerNorm: there the split launch writes its partials row-major and the
// second launch is the fused reduce + residual + LayerNorm
// (splitk_layernorm_kernel), so the split costs no extra launch.
//
// GeGLU epilogue (epilogue 1): the first BW/2 rows of the weight tile are
// rows n0.. of W (the GELU half), the last BW/2 rows are rows N+n0.. (the
// gate half); each wave holds matching u and g fragments (on 32-row tiles,
// accumulator rows r and r + 16 of one fragment), so h = bf16(GELU(u) * g)
// is formed from unrounded float32 u and g.
//
// QKV epilogue (epilogue 2): RoPE on the Q and K heads in registers and the
// V columns stored transposed for attention (see QkvEpilogue); a 32-row tile
// takes half a head, dimensions 16p..16p+15 and their rotation partners.
//
// Bias: with a bias vector, a product is rounded to BF16, the bias added and
// the sum rounded again, y = bf16(bf16(A W^T) + b) (a biased dense layer as
// the matmul followed by x + b in the model's precision); epilogue 3 then
// takes GELU of that BF16 value, h = bf16(GELU(y)).
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "kernels.h"

// Diagnostic build (LAYA_GEMM_PHASES, a separate library next to the product
// one): every whole-K workgroup of gemm_kernel records the shader clock when
// its tile is known, when its ring is first full, when its main loop ends,
// before and after the barrier ahead of its stores, and at its end, plus the
// 100 MHz real-time clock at its start and end and its tile, into
// gemm_phases[workgroup][10] (first 65536 workgroups of a launch).
#ifdef LAYA_GEMM_PHASES
namespace {
constexpr int kPhaseWorkgroups = 65536;
__device__ unsigned long long gemm_phases[kPhaseWorkgroups * 10];
}  // namespace
#define LAYA_PHASE(var) (var) = __builtin_readcyclecounter()
#else
#define LAYA_PHASE(var) (void)0
#endif

// Split-K partials of the allocation-free GEMM entry point: device memory the
// library holds for the life of the process on each GPU it runs on, shared by
// every such call on that GPU.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
static __device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

namespace laya {

namespace {

constexpr int KMULT = 64;  // K and every split piece are multiples of 64
constexpr int kMaxSplits = 8;  // K ranges of a split launch

// Physical 16-byte chunk of logical chunk `c` in stage row `r` (rows of BK
// bf16): XOR with the row's index among the rows that share one 256-byte
// sweep of the banks, so 16 consecutive rows at one logical chunk are spread
// over all banks.  The map is an involution.
template <int BK>
__device__ __forceinline__ int pchunk(int r, int c) {
    constexpr int CH = BK / 8;
    constexpr int SH = BK == 64 ? 1 : 2;
    return c ^ ((r >> SH) & (CH - 1));
}
template <int BK>
__device__ __forceinline__ int swz(int r, int c) {
    return r * BK + (pchunk<BK>(r, c) << 3);
}

// erfc(x) by the Chebyshev fit of Numerical Recipes in C (2nd ed., section
// 6.2, routine erfcc): for z = |x| and t = 1 / (1 + z/2),
// erfc(z) = t exp(-z^2 + P(t)) with a degree-9 polynomial P, fractional error
// below 1.2e-7 everywhere; erfc(-z) = 2 - erfc(z).  About 15 instructions,
// against several times that for the multi-range library erfcf, which
// dominated the GeGLU epilogue.  In float32 the exponent's rounding adds a
// relative error of about 1e-7 * z^2, still far below the BF16 rounding of
// the output.
__device__ __forceinline__ float erfc_cheb(float x) {
    const float z = fabsf(x);
    const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));
    float q = 0.17087277f;
    q = fmaf(q, t, -0.82215223f);
    q = fmaf(q, t, 1.48851587f);
    q = fmaf(q, t, -1.13520398f);
    q = fmaf(q, t, 0.27886807f);
    q = fmaf(q, t, -0.18628806f);
    q = fmaf(q, t, 0.09678418f);
    q = fmaf(q, t, 0.37409196f);
    q = fmaf(q, t, 1.00002368f);
    q = fmaf(q, t, -1.26551223f);
    const float r = t * __expf(fmaf(-z, z, q));
    return x >= 0.f ? r : 2.f - r;
}

// GELU(z) = z Phi(z) = 0.5 z erfc(-z / sqrt 2).  erfc keeps full relative
// accuracy in the negative tail, where 1 + erf(z / sqrt 2) would cancel.
__device__ __forceinline__ float gelu_erf(float z) {
    return 0.5f * z * erfc_cheb(-z * 0.70710678118654752f);
}

// Which tile a workgroup computes; false for a workgroup with no live tile.
// The grid is sized for the largest row count and only the first `live_by`
// token tiles hold rows.  Workgroups are handed to the 8 XCDs in turn
// (dispatch index i goes to XCD i % 8) and each XCD has its own L2, so the
// live dispatch indices are first spread evenly over the XCDs as contiguous
// ranges of tiles; each range is walked in groups of 4 token tiles (all
// weight tiles of a group before the next group), so the tiles resident on
// one XCD share a few activation panels and a few weight panels.
__device__ __forceinline__ bool tile_order(int live_by, int &bx, int &by) {
    const int nbx = gridDim.x;
    const int b = xcd_contiguous(by * nbx + bx, nbx * live_by);
    if (b < 0) return false;
    constexpr int GT = 4;
    const int group = b / (GT * nbx);
    const int first = group * GT;
    const int gsize = min(live_by - first, GT);
    const int idx = b - group * GT * nbx;
    bx = idx / gsize;
    by = first + idx % gsize;
    return true;
}

// Two-dimensional split of the tile grid over the 8 XCDs: XCD x takes the
// block of weight tiles xk = x % xw and token tiles xt = x / xw (xw * xt
// ranges = 8 blocks), so its L2 fetches 1/xw of the weights and xw/8 of the
// activations instead of all of the weights; inside the block the tiles go
// in groups of 4 token tiles as above.  The j-th workgroup dispatched to XCD
// x takes the j-th tile of the block; the host pads the grid so that every
// XCD has a slot for each tile of the largest block, whichever split the
// live token count selects.
//
// The split (xw weight ranges, 1 = the 1-D order) minimises the rows one XCD
// reads, weight rows / xw + token rows * xw / 8, among the splits whose
// largest block needs no more rounds of the XCD's 32 CUs (occ workgroups
// each) than the even 1-D share: a block a few tiles over a round doubles
// the time of the whole launch.
__device__ __forceinline__ int pick_xw(int nbx, int live_by, int bw, int bt, int occ) {
    const int slots = 32 * occ;
    const int r1 = ((nbx * live_by + 7) / 8 + slots - 1) / slots;
    int best = 1;
    int64_t cost = (int64_t)nbx * bw * 8 + (int64_t)live_by * bt;
    for (int xw = 2; xw <= 8; xw *= 2) {
        const int xtn = 8 / xw;
        const int bmax = ((live_by + xtn - 1) / xtn) * ((nbx + xw - 1) / xw);
        if ((bmax + slots - 1) / slots > r1) continue;
        const int64_t c = (int64_t)nbx * bw * 8 / xw + (int64_t)live_by * bt * xw;
        if (c < cost) {
            cost = c;
            best = xw;
        }
    }
    return best;
}

__device__ __forceinline__ bool tile_order_2d(int live_by, int xw, int &bx, int &by) {
    const int nbx = gridDim.x;
    const int d = blockIdx.y * nbx + blockIdx.x;
    const int xtn = 8 / xw;
    const int x = d & 7, j = d >> 3;
    const int xt = x / xw, xk = x % xw;
    const int t_lo = xt * live_by / xtn, t_hi = (xt + 1) * live_by / xtn;
    const int w_lo = xk * nbx / xw, w_hi = (xk + 1) * nbx / xw;
    const int nt = t_hi - t_lo, nw = w_hi - w_lo;
    if (j >= nt * nw) return false;
    constexpr int GT = 4;
    const int group = j / (GT * nw);
    const int first = group * GT;
    const int gsize = min(nt - first, GT);
    const int idx = j - group * GT * nw;
    bx = w_lo + idx / gsize;
    by = t_lo + first + idx % gsize;
    return true;
}

// XW extra waves only move operands: they issue their share of the ring's
// loads and meet the barriers, but read no fragments and run no MFMAs (more
// loads in flight per CU for the small tiles, whose one or two computing
// waves cannot issue them fast enough).
template <int BW_, int BT_, int WW_, int WT_, int BK_, int STAGES_, int XW_ = 0>
struct Cfg {
    static constexpr int BW = BW_, BT = BT_, WW = WW_, WT = WT_, BK = BK_, STAGES = STAGES_;
    static constexpr int XW = XW_;
    static constexpr int NWAVE_C = WW * WT;                 // waves that compute
    static constexpr int NWAVE = NWAVE_C + XW, NTHR = NWAVE * 64;  // waves that load
    static constexpr int RW = BW / WW, RT = BT / WT;  // rows / tokens per wave
    static constexpr int FA = RW / 32, FB = RT / 32;  // 32x32 fragments per wave
    static constexpr int STAGE_ELEMS = (BW + BT) * BK;
    // workgroups per CU that the ring's LDS allows (at most 2 used)
    static constexpr int OCC = (160 * 1024) / (STAGES * STAGE_ELEMS * 2) >= 2 ? 2 : 1;
    static constexpr int CH = BK / 8;                      // 16-byte chunks per row
    static constexpr int RPL = 64 / CH;                    // rows per 1 KB DMA load
    static constexpr int BLOCKS = (BW + BT) / RPL;         // 1 KB DMA loads per stage
    // DMA loads per wave per stage: LOADS_MIN for every wave, one more for
    // the first BLOCKS % NWAVE waves (token rows only)
    static constexpr int LOADS = (BLOCKS + NWAVE - 1) / NWAVE, LOADS_MIN = BLOCKS / NWAVE;
    static constexpr int WLOADS = BW / RPL / NWAVE;        // the first WLOADS are weight rows
    static_assert(BK == 32 || BK == 64, "K step");
    static_assert((BW / RPL) % NWAVE == 0 && BT % RPL == 0, "weight loads split evenly");
    static_assert(RW % 32 == 0 && RT % 32 == 0, "32x32 fragments");
    static_assert(STAGES >= 2 && (STAGES - 1) * LOADS < 64, "vmcnt range");
    static_assert(STAGES * STAGE_ELEMS * 2 <= 160 * 1024, "LDS");
    static_assert(FA + FB <= 15, "lgkmcnt range");
};

// XOR mask of the output staging's 16-byte chunk swizzle for rows of n
// chunks: the largest power of two dividing n, minus one, so a chunk stays
// inside its row (all of it for power-of-two rows).
constexpr int chunk_swizzle(int n) { return (n & -n) - 1; }

struct GemmParams {
    const bf16_t *A;
    int32_t lda;
    const bf16_t *W;
    int32_t ldw;
    bf16_t *C;
    int32_t ldc;
    const int32_t *M_dev;
    int32_t M_max, N, K;
    int32_t splits;
    float *partial;      // [tiles][splits][BW*BT] (splits > 1)
    QkvEpilogue qe;      // epilogue 2 only
    const bf16_t *bias;  // [N] or null (epilogues 0 and 2; required by 3)
    int32_t split2d;     // whole K: 1 if the grid is padded for the 2-D XCD split
    const bf16_t *res;   // whole K, epilogues 0 and 4, or null: C = bf16(res + y), with
                         // C's row stride (the residual add; res may be C itself)
};

// MODE 0: whole K, C written.  MODE 1: one K range per blockIdx.z, its
// float32 partial tile written to p.partial.  MODE 2: the partials of each
// tile summed in range order, then the epilogue (a second launch, so the
// partials are visible without any cross-XCD fence).  MODE 3: as MODE 1, but
// the partials are written row-major, [range][M_max][N], through LDS, for the
// fused reduce + LayerNorm kernel, which reads whole token rows.
enum { kWholeK = 0, kPartial = 1, kReduce = 2, kPartialRows = 3 };

template <class G, int EPI, int MODE>
__global__ __launch_bounds__(G::NTHR) void gemm_kernel(GemmParams p) {
    constexpr int BW = G::BW, BT = G::BT, FA = G::FA, FB = G::FB, STAGES = G::STAGES;
    constexpr int BK = G::BK, CH = G::CH, RPL = G::RPL;
    // GeGLU / QKV pair rows (u with g, dimension i with i + 32): in paired
    // fragments, or, on 32-row tiles, within one fragment (rows r and r + 16)
    constexpr bool HALF = G::RW == 32 && G::WW == 1 && (EPI == 1 || EPI == 2);
    static_assert(EPI == 0 || EPI >= 3 || FA % 2 == 0 || HALF, "GeGLU / QKV need paired rows");
    static_assert(EPI != 2 || G::RW % 64 == 0 || HALF, "QKV epilogue: whole or half heads");
    const int32_t M = p.M_dev ? *p.M_dev : p.M_max;
    int bx = blockIdx.x, by = blockIdx.y;
    if (MODE == kWholeK) {
        const int live_by = (M + BT - 1) / BT;
        const int xw = p.split2d ? pick_xw(gridDim.x, live_by, BW, BT, G::OCC) : 1;
        if (!(xw > 1 ? tile_order_2d(live_by, xw, bx, by) : tile_order(live_by, bx, by)))
            return;
    }
    const int32_t t0 = by * BT;
    if (t0 >= M) return;
    constexpr int BN = EPI == 1 ? BW / 2 : BW;  // output features per tile
    const int32_t n0 = bx * BN;
    const int split = blockIdx.z;
    const int N = p.N;
    [[maybe_unused]] uint64_t ph[6] = {0, 0, 0, 0, 0, 0};
    [[maybe_unused]] uint64_t ph_r0 = 0;
    LAYA_PHASE(ph[0]);
#ifdef LAYA_GEMM_PHASES
    ph_r0 = wall_clock64();
#endif
    // the phase record of this workgroup (diagnostic build, whole K)
    [[maybe_unused]] auto phase_store = [&]() {
#ifdef LAYA_GEMM_PHASES
        LAYA_PHASE(ph[5]);
        const int wg = blockIdx.y * gridDim.x + blockIdx.x;
        if (MODE == kWholeK && threadIdx.x == 0 && wg < kPhaseWorkgroups) {
            unsigned long long *d = gemm_phases + (size_t)wg * 10;
            for (int i = 0; i < 6; ++i) d[i] = ph[i];
            d[6] = ph_r0;
            d[7] = wall_clock64();
            d[8] = ((uint64_t)(uint32_t)bx << 32) | (uint32_t)by;
            d[9] = 1;
        }
#endif
    };

    // The residual add of the whole-K plain epilogues (p.res): this thread's
    // 16-byte chunks of res, in the store's order.  Where they fit in 32
    // registers they are loaded before the main loop, whose waits cover them,
    // so their latency hides behind it; otherwise at the epilogue.
    constexpr bool RES = MODE == kWholeK && (EPI == 0 || EPI == 4);
    constexpr int RCH = BN / 8;  // 16-byte chunks per tile row
    constexpr int RNIT = RES ? (BT * RCH + G::NTHR - 1) / G::NTHR : 1;
    constexpr bool RES_EARLY = RES && RNIT <= 8;
    [[maybe_unused]] u32x4_t rv[RNIT];
    [[maybe_unused]] auto res_chunk = [&](int i, int &tl, int &c, int32_t &tok, int32_t &f) {
        const int idx = (int)threadIdx.x + i * G::NTHR;
        tl = idx / RCH;
        c = idx % RCH;
        tok = t0 + tl;
        f = n0 + 8 * c;
        return idx < BT * RCH && tok < M && f < min(N, n0 + BN);
    };
    [[maybe_unused]] auto res_load = [&]() {
#pragma unroll
        for (int i = 0; i < RNIT; ++i) {
            int tl, c;
            int32_t tok, f;
            if (res_chunk(i, tl, c, tok, f)) rv[i] = ld16(p.res + (size_t)tok * p.ldc + f);
        }
    };
    if constexpr (RES_EARLY)
        if (p.res) res_load();

    __shared__ __attribute__((aligned(16))) bf16_t smem[STAGES * G::STAGE_ELEMS];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const bool compute = G::XW == 0 || wave < G::NWAVE_C;  // else a loading-only wave
    const int wr = wave / G::WT;  // wave row (weight rows)
    const int wc = wave % G::WT;  // wave column (tokens)

    // K range of this split, in 64-wide pieces, then in BK steps
    const int np_all = p.K / KMULT;
    const int pb = (int)((int64_t)split * np_all / p.splits);
    const int pe = (int)((int64_t)(split + 1) * np_all / p.splits);
    const int kbase = pb * KMULT;
    const int nk = (pe - pb) * (KMULT / BK);

    // Per-lane DMA sources.  Load j of a wave covers LDS block
    // jj = j * NWAVE + wave (1 KB: stage rows RPL*jj .. RPL*jj+RPL-1; weight
    // rows come first, then tokens, and loads j < WLOADS are exactly the
    // weight ones).  Lane L writes physical chunk L % CH of row RPL*jj + L/CH,
    // so it fetches the logical chunk that the swizzle stores there.
    // The loads are buffer loads into LDS: a per-lane 32-bit byte offset from
    // the W or A base, the K step's byte offset in a scalar register, and a
    // resource whose size is the operand's extent, so the hardware drops any
    // access past it.  (Buffer rather than global loads: the waitcnt pass
    // counts a global load into LDS as an LDS access too, which would force
    // every wait on the fragment reads to lgkmcnt(0).)
    const int rr = lane / CH, pc = lane % CH;
    const uint32_t w_rows = EPI == 1 ? 2u * (uint32_t)N : (uint32_t)N;
    const uint32_t w_bytes = ((w_rows - 1) * (uint32_t)p.ldw + (uint32_t)p.K) * 2u;
    const uint32_t a_bytes = (((uint32_t)p.M_max - 1) * (uint32_t)p.lda + (uint32_t)p.K) * 2u;
    uint32_t off[G::LOADS];
#pragma unroll
    for (int j = 0; j < G::LOADS; ++j) {
        const int jj = j * G::NWAVE + wave;
        if (j >= G::LOADS_MIN && jj >= G::BLOCKS) {  // past the stage's last block: no load
            off[j] = a_bytes;
            continue;
        }
        const int r = RPL * jj + rr;      // stage row
        const int c = pchunk<BK>(r, pc);  // logical chunk stored at physical chunk pc
        if (j < G::WLOADS) {
            int grow;
            if (EPI == 1) {
                const int half = BW / 2;
                int f = n0 + (r % half);
                if (f >= N) f = N - 1;  // clamp: rows past N are computed, never stored
                grow = (r < half) ? f : N + f;
            } else if (EPI == 2 && HALF) {
                // half a head: dimensions 16p .. 16p+15, then 32+16p .. 32+16p+15
                const int p16 = (bx & 1) * 16;
                grow = (bx >> 1) * 64 + (r < 16 ? p16 + r : 32 + p16 + (r - 16));
            } else {
                grow = n0 + r;
                if (grow >= N) grow = N - 1;
            }
            off[j] = (uint32_t)(grow * p.ldw + kbase + c * 8) * 2u;
        } else {
            // token rows past the live count are never stored: their lanes
            // take an offset past the resource's end, so the hardware fetches
            // nothing and their stage rows read as zero
            const int trow = t0 + (r - BW);
            off[j] = trow < M ? (uint32_t)(trow * p.lda + kbase + c * 8) * 2u : a_bytes;
        }
    }
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto issue = [&](int kt, int stage) {
        bf16_t *base = smem + stage * G::STAGE_ELEMS + wave_u * 512;
        const int k0b = kt * BK * 2;
#pragma unroll
        for (int j = 0; j < G::LOADS; ++j) {
            if (j >= G::LOADS_MIN && j * G::NWAVE + wave_u >= G::BLOCKS) continue;
            if (j < G::WLOADS)
                dma16(p.W, w_bytes, (lds_ptr_t)(base + j * G::NWAVE * 512), off[j], k0b);
            else
                dma16(p.A, a_bytes, (lds_ptr_t)(base + j * G::NWAVE * 512), off[j], k0b);
        }
    };

    f32x16_t acc[FA][FB];
#pragma unroll
    for (int a = 0; a < FA; ++a)
#pragma unroll
        for (int b = 0; b < FB; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

    // stage-row base of each A (weight) fragment
    int wrow[FA];
#pragma unroll
    for (int a = 0; a < FA; ++a) {
        if (EPI == 1 && !HALF)
            wrow[a] = (a < FA / 2) ? (wr * (G::RW / 2) + 32 * a)
                                   : (BW / 2 + wr * (G::RW / 2) + 32 * (a - FA / 2));
        else
            wrow[a] = wr * G::RW + 32 * a;
    }
    const int l32 = lane & 31, lhi = lane >> 5;

    // Software pipeline.  Fragments are double-buffered in registers: the
    // LDS reads of step s+1 are issued before the MFMAs of step s, so the
    // matrix cores hide the LDS latency.  At the last step of a stage the
    // wave waits for the next stage's loads, meets the others at the
    // barrier, refills the stage it has finished reading, and issues the
    // next stage's first reads before its last MFMAs of this stage.
    constexpr int NS = BK / 16;  // MFMA steps per stage (2 or 4)
    static_assert(NS % 2 == 0, "fragment buffers alternate per step");
    bf16x8_t fw[2][FA], fa[2][FB];
    auto read_frags = [&](int stage, int s, int buf) {
        const bf16_t *sw = smem + stage * G::STAGE_ELEMS;
        const bf16_t *sa = sw + BW * BK;
        const int ch = 2 * s + lhi;
#pragma unroll
        for (int a = 0; a < FA; ++a)
            fw[buf][a] = *reinterpret_cast<const bf16x8_t *>(&sw[swz<BK>(wrow[a] + l32, ch)]);
#pragma unroll
        for (int b = 0; b < FB; ++b)
            fa[buf][b] = *reinterpret_cast<const bf16x8_t *>(
                &sa[swz<BK>(wc * G::RT + 32 * b + l32, ch)]);
    };
    auto mfmas = [&](int buf) {
#pragma unroll
        for (int a = 0; a < FA; ++a)
#pragma unroll
            for (int b = 0; b < FB; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[buf][a], fa[buf][b],
                                                                    acc[a][b], 0, 0, 0);
    };

    // Half-head QKV tiles (short calls): the lane's token position is loaded
    // ahead of the ring's first loads and its rotation-table entries right
    // after them, so their latency hides behind the main loop (whose waits,
    // counted in order, then cover them as well).
    constexpr bool QKV_HALF = EPI == 2 && HALF;
    [[maybe_unused]] u32x2_t hcos[2] = {}, hsin[2] = {};
    [[maybe_unused]] uint32_t hps = 0;
    [[maybe_unused]] bool half_rope = false;
    [[maybe_unused]] auto half_tables = [&]() {
#pragma unroll
        for (int g4 = 0; g4 < 2; ++g4) {
            const int j = (bx & 1) * 16 + 8 * g4 + 4 * lhi;  // pair index of element 4*g4
            hcos[g4] = *reinterpret_cast<const u32x2_t *>(p.qe.cos_tab + hps + j);
            hsin[g4] = *reinterpret_cast<const u32x2_t *>(p.qe.sin_tab + hps + j);
        }
    };
    if constexpr (QKV_HALF) {
        half_rope = compute && (bx >> 1) * 64 < p.qe.rope_cols;
        if (half_rope) {
            const int32_t tok = t0 + wc * G::RT + l32;
            hps = (uint32_t)p.qe.pos[tok < M ? tok : M - 1] * 32u;
        }
        if constexpr (MODE == kReduce)
            if (half_rope) half_tables();
    }

    if constexpr (MODE != kReduce) {
    // prologue: every stage of the ring in flight, then stage 0 published
  #pragma unroll
      for (int st = 0; st < STAGES; ++st)
          if (st < nk) issue(st, st);
      if constexpr (QKV_HALF)
          if (half_rope) half_tables();
      if (nk >= STAGES)
          wait_vmcnt<(STAGES - 1) * G::LOADS_MIN>();
      else
          wait_vmcnt<0>();
      // The output, bias, residual, partial and QKV table pointers are needed
      // only after the main loop (or just before it), but left to itself the
      // compiler may issue their scalar loads just before the loop.
      // Scalar and LDS loads share one wait counter and the scalar ones can
      // return out of order, so a scalar load still in flight at the loop's
      // entry turns the loop's first fragment wait into a wait for every LDS
      // read.  Using the pointers here puts their loads under the wait below.
      asm volatile("" ::"s"(p.C), "s"(p.bias), "s"(p.res), "s"(p.partial));
      if constexpr (EPI == 2)
          asm volatile("" ::"s"(p.qe.pos), "s"(p.qe.cos_tab), "s"(p.qe.sin_tab), "s"(p.qe.vt),
                       "s"(p.qe.vt_tok));
      wait_lgkmcnt<0>();  // no scalar loads left in flight, so
                                           // the loop's LDS reads can be waited on in order
      ring_barrier();
      LAYA_PHASE(ph[1]);
      if (!compute) {
          // the same waits, barriers and refills as the computing waves
          for (int i = 0; i < nk; ++i) {
              if (i + STAGES <= nk)
                  wait_vmcnt<(STAGES - 2) * G::LOADS_MIN>();
              else
                  wait_vmcnt<0>();
              ring_barrier();
              if (i + STAGES < nk) issue(i + STAGES, i % STAGES);
          }
      } else {
      if (nk > 0) read_frags(0, 0, 0);
  
      for (int i = 0; i < nk; ++i) {
          const int stage = i % STAGES;
  #pragma unroll
          for (int s = 0; s < NS; ++s) {
              if (s + 1 < NS) {
                  read_frags(stage, s + 1, (s + 1) & 1);
              } else {
                  // outstanding loads after stage i+1: stages i+2 .. min(i+STAGES-1, nk-1)
                  if (i + STAGES <= nk)
                      wait_vmcnt<(STAGES - 2) * G::LOADS_MIN>();
                  else
                      wait_vmcnt<0>();
                  wait_lgkmcnt<0>();  // this stage fully read
                  ring_barrier();
                  if (i + STAGES < nk) issue(i + STAGES, stage);
                  // next stage's first fragments (after the last stage: an unused
                  // read of a valid stage, kept so the loop body has no branch
                  // around LDS reads and their waits stay exact)
                  read_frags((i + 1) % STAGES, 0, 0);
              }
              // the fragments of step s are complete once at most the reads of
              // step s+1 remain in flight
              wait_lgkmcnt<G::FA + G::FB>();
              __builtin_amdgcn_sched_barrier(0);
              mfmas(s & 1);
              __builtin_amdgcn_sched_barrier(0);
          }
      }
      }
    }

    if constexpr (MODE == kPartialRows) {
        // the float32 tile in LDS as [token][feature] (16-byte chunks
        // XOR-swizzled by token), then 16-byte stores along the rows of
        // p.partial + split * M_max * N
        constexpr int NC4 = BW / 4;  // 16-byte chunks per tile row
        static_assert(BT * BW * 4 <= STAGES * G::STAGE_ELEMS * 2, "float32 tile fits the ring");
        __syncthreads();  // every wave is done with the ring
        float *sP = reinterpret_cast<float *>(smem);
        if (compute)
#pragma unroll
        for (int a = 0; a < FA; ++a)
#pragma unroll
            for (int b = 0; b < FB; ++b) {
                const int tl = wc * G::RT + 32 * b + l32;
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int c = (wrow[a] + 8 * g4 + 4 * lhi) >> 2;
                    *reinterpret_cast<f32x4_t *>(&sP[tl * BW + ((c ^ (tl & chunk_swizzle(NC4))) << 2)]) =
                        f32x4_t{acc[a][b][4 * g4], acc[a][b][4 * g4 + 1], acc[a][b][4 * g4 + 2],
                                acc[a][b][4 * g4 + 3]};
                }
            }
        __syncthreads();
        float *dst = p.partial + (size_t)split * p.M_max * N;
#pragma unroll 4
        for (int idx = tid; idx < BT * NC4; idx += G::NTHR) {
            const int tl = idx / NC4, c = idx % NC4;
            const int32_t tok = t0 + tl, f = n0 + 4 * c;
            if (tok < M && f < N)
                *reinterpret_cast<f32x4_t *>(dst + (size_t)tok * N + f) =
                    *reinterpret_cast<const f32x4_t *>(&sP[tl * BW + ((c ^ (tl & chunk_swizzle(NC4))) << 2)]);
        }
        return;
    }
    // Partial tiles: [tile][split][wave][a][b][e4][lane][4] float32, so each
    // lane moves 16 contiguous bytes.
    const int tile = blockIdx.y * gridDim.x + blockIdx.x;
    if constexpr (MODE == kPartial) {
        float *mine = p.partial + ((size_t)tile * p.splits + split) * (BW * BT);
        if (compute)
#pragma unroll
        for (int a = 0; a < FA; ++a)
#pragma unroll
            for (int b = 0; b < FB; ++b)
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int blk = ((wave * FA + a) * FB + b) * 4 + e4;
                    const f32x4_t v = {acc[a][b][4 * e4], acc[a][b][4 * e4 + 1],
                                       acc[a][b][4 * e4 + 2], acc[a][b][4 * e4 + 3]};
                    *reinterpret_cast<f32x4_t *>(mine + (size_t)blk * 256 + lane * 4) = v;
                }
        return;
    }
    if constexpr (MODE == kReduce) {
      if (compute) {
        // sum of the K ranges' partials, in range order; each range's whole
        // share of the tile is loaded before it is added, so a wave has all
        // of its loads for one range in flight at once
        const float *base = p.partial + (size_t)tile * p.splits * (BW * BT) + lane * 4;
        auto part = [&](int sp, int a, int b, int e4) {
            const int blk = ((wave * FA + a) * FB + b) * 4 + e4;
            return *reinterpret_cast<const f32x4_t *>(base + (size_t)sp * (BW * BT) +
                                                     (size_t)blk * 256);
        };
        f32x4_t sum[FA][FB][4];
#pragma unroll
        for (int a = 0; a < FA; ++a)
#pragma unroll
            for (int b = 0; b < FB; ++b)
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) sum[a][b][e4] = part(0, a, b, e4);
        for (int sp = 1; sp < p.splits; ++sp) {
            f32x4_t t[FA][FB][4];
#pragma unroll
            for (int a = 0; a < FA; ++a)
#pragma unroll
                for (int b = 0; b < FB; ++b)
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4) t[a][b][e4] = part(sp, a, b, e4);
#pragma unroll
            for (int a = 0; a < FA; ++a)
#pragma unroll
                for (int b = 0; b < FB; ++b)
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4) sum[a][b][e4] += t[a][b][e4];
        }
#pragma unroll
        for (int a = 0; a < FA; ++a)
#pragma unroll
            for (int b = 0; b < FB; ++b)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[a][b][e] = sum[a][b][e / 4][e % 4];
      }
    }

    // Epilogue.  Accumulator element e of lane l in a 32x32 block holds
    // row (weight row) 8*(e/4) + 4*(l/32) + e%4 and column (token) l%32, so a
    // lane has 4 consecutive output features of one token.  The BF16 output
    // tile is first assembled in LDS ([token][feature], 16-byte chunks
    // XOR-swizzled by token), then written with 16-byte stores along whole
    // row segments: direct stores would touch 32 token rows per instruction.
    // Columns bound for the transposed V (epilogue 2) are stored directly.
    LAYA_PHASE(ph[2]);
    constexpr int NCH = BN / 8;  // 16-byte chunks per tile row
    static_assert(BT * BN * 2 <= STAGES * G::STAGE_ELEMS * 2, "output tile fits the ring");
    __syncthreads();  // every wave is done with the ring
    bf16_t *sC = smem;
    auto put4 = [&](int tl, int fl, uint32_t lo, uint32_t hi) {
        const int c = fl >> 3;
        *reinterpret_cast<u32x2_t *>(
            &sC[tl * BN + ((c ^ (tl & chunk_swizzle(NCH))) << 3) + (fl & 4)]) = u32x2_t{lo, hi};
    };
    auto bf16r = [](float v) { return bf16_to_f32(f32_to_bf16(v)); };
    // four consecutive bias values (f a multiple of 4; the bias is 8-byte aligned)
    auto bias4 = [&](int32_t f, float (&bv)[4]) {
        const u32x2_t w = *reinterpret_cast<const u32x2_t *>(p.bias + f);
        bv[0] = bf16lo(w[0]);
        bv[1] = bf16hi(w[0]);
        bv[2] = bf16lo(w[1]);
        bv[3] = bf16hi(w[1]);
    };
    // QKV tiles of whole heads: each lane's rotation-table entries (they
    // depend only on the token's position and the pair index, so one load
    // serves all of the wave's heads) and V^T columns, all loaded before any
    // is used, so the epilogue waits on memory once.
    constexpr bool QKV_FULL = EPI == 2 && !HALF;
    [[maybe_unused]] u32x2_t rcos[QKV_FULL ? FB : 1][4], rsin[QKV_FULL ? FB : 1][4];
    [[maybe_unused]] int32_t vtcol[QKV_FULL ? FB : 1];
    if constexpr (QKV_FULL) {
        const QkvEpilogue &q = p.qe;
        bool rope = false, vt = false;  // the same for every lane of the wave
#pragma unroll
        for (int a = 0; a < FA; a += 2) {
            const int32_t f0 = n0 + wrow[a];
            if (f0 < N) {
                rope = rope || f0 < q.rope_cols;
                vt = vt || (f0 >= q.vt_col0 && f0 >= q.rope_cols);
            }
        }
        if (compute)
#pragma unroll
            for (int b = 0; b < FB; ++b) {
                const int32_t tok = t0 + wc * G::RT + 32 * b + l32;
                const int32_t tc = tok < M ? tok : M - 1;
                if (rope) {
                    const uint32_t ps = (uint32_t)q.pos[tc] * 32u;
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int j = 8 * g4 + 4 * lhi;
                        rcos[b][g4] = *reinterpret_cast<const u32x2_t *>(q.cos_tab + ps + j);
                        rsin[b][g4] = *reinterpret_cast<const u32x2_t *>(q.sin_tab + ps + j);
                    }
                }
                if (vt) vtcol[b] = q.vt_tok[tc];
            }
    }
    if (compute)
#pragma unroll
    for (int b = 0; b < FB; ++b) {
        const int tl = wc * G::RT + 32 * b + l32;  // token within the tile
        const int32_t tok = t0 + tl;
        if constexpr (EPI == 1 && HALF) {
            // tile rows 0..15 are u, rows 16..31 the matching g: accumulator
            // element 4 g4 + e (row 8 g4 + 4 lhi + e) pairs with 4 (g4 + 2) + e
#pragma unroll
            for (int g4 = 0; g4 < 2; ++g4) {
                float h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    h[e] = gelu_erf(acc[0][b][4 * g4 + e]) * acc[0][b][4 * (g4 + 2) + e];
                put4(tl, 8 * g4 + 4 * lhi, pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
            }
        } else if constexpr (EPI == 1) {
#pragma unroll
            for (int a = 0; a < FA / 2; ++a)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int fl = wr * (G::RW / 2) + 32 * a + 8 * g4 + 4 * lhi;
                    float h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        h[e] = gelu_erf(acc[a][b][4 * g4 + e]) * acc[a + FA / 2][b][4 * g4 + e];
                    put4(tl, fl, pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
                }
        } else if constexpr (EPI == 2 && HALF) {
            // Half a head per tile: accumulator element 4 g4 + e (g4 < 2) is
            // dimension 16p + 8 g4 + 4 lhi + e, element 4 (g4 + 2) + e the
            // dimension 32 above it, so each rotation pair is in one lane.  The
            // staged tile holds the 16 low dimensions, then the 16 high ones.
            // (Rotation tables preloaded above; the bias, head variant only,
            // a compile-time case.)
            const QkvEpilogue &q = p.qe;
            const int32_t hcol = (bx >> 1) * 64;  // first column of the head
            const int p16 = (bx & 1) * 16;
            auto tile = [&](auto bias_tag) {
                constexpr bool HB = decltype(bias_tag)::value;
                if (hcol < q.rope_cols) {
#pragma unroll
                    for (int g4 = 0; g4 < 2; ++g4) {
                        const int j = p16 + 8 * g4 + 4 * lhi;  // pair index of element 4*g4
                        const u32x2_t cv = hcos[g4], sv = hsin[g4];
                        float xo[4], yo[4], bx4[4] = {0, 0, 0, 0}, by4[4] = {0, 0, 0, 0};
                        if constexpr (HB) {
                            bias4(hcol + j, bx4);
                            bias4(hcol + 32 + j, by4);
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float x = bf16r(acc[0][b][4 * g4 + e]);
                            float y = bf16r(acc[0][b][4 * (g4 + 2) + e]);
                            if constexpr (HB) {
                                x = bf16r(x + bx4[e]);
                                y = bf16r(y + by4[e]);
                            }
                            const float c = (e & 1) ? bf16hi(cv[e >> 1]) : bf16lo(cv[e >> 1]);
                            const float sn = (e & 1) ? bf16hi(sv[e >> 1]) : bf16lo(sv[e >> 1]);
                            // both products of BF16 values are exact in float32
                            xo[e] = fmaf(x, c, -(y * sn));
                            yo[e] = fmaf(y, c, x * sn);
                        }
                        put4(tl, 8 * g4 + 4 * lhi, pack_bf16x2(xo[0], xo[1]),
                             pack_bf16x2(xo[2], xo[3]));
                        put4(tl, 16 + 8 * g4 + 4 * lhi, pack_bf16x2(yo[0], yo[1]),
                             pack_bf16x2(yo[2], yo[3]));
                    }
                } else if (hcol >= q.vt_col0) {
                    if (tok < M) {
                        bf16_t *vcol = q.vt + q.vt_tok[tok];
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                            for (int g = 0; g < 2; ++g) {
                                const int32_t f4 = hcol + 32 * h2 + p16 + 8 * g + 4 * lhi;
                                float bv[4] = {0, 0, 0, 0};
                                if constexpr (HB) bias4(f4, bv);
                                bf16_t *dst = vcol + (size_t)(f4 - q.vt_col0) * q.ldvt;
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    float v = acc[0][b][4 * (g + 2 * h2) + e];
                                    if constexpr (HB) v = bf16r(v) + bv[e];
                                    dst[(size_t)e * q.ldvt] = (bf16_t)f32_to_bf16(v);
                                }
                            }
                    }
                } else {
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                        for (int g4 = 0; g4 < 2; ++g4) {
                            float v[4], bv[4] = {0, 0, 0, 0};
                            if constexpr (HB) bias4(hcol + 32 * h2 + p16 + 8 * g4 + 4 * lhi, bv);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                v[e] = acc[0][b][4 * (g4 + 2 * h2) + e];
                                if constexpr (HB) v[e] = bf16r(v[e]) + bv[e];
                            }
                            put4(tl, 16 * h2 + 8 * g4 + 4 * lhi, pack_bf16x2(v[0], v[1]),
                                 pack_bf16x2(v[2], v[3]));
                        }
                }
            };
            if (p.bias)
                tile(std::true_type{});
            else
                tile(std::false_type{});
        } else if constexpr (EPI == 2) {
            // Fragments a (dims 0..31 of a head) and a+1 (dims 32..63) sit in
            // the same lanes, so the rotation pairs (i, i+32) are in registers.
            // The table entries and V^T columns come preloaded (below the
            // main loop); the bias, present only in the head variant, is a
            // compile-time case, so the encoder's tiles carry no per-element
            // branch and no load between their stores.
            const QkvEpilogue &q = p.qe;
            auto tile = [&](auto bias_tag) {
                constexpr bool HB = decltype(bias_tag)::value;
#pragma unroll
                for (int a = 0; a < FA; a += 2) {
                    const int32_t f0 = n0 + wrow[a];  // first column of the head
                    if (f0 >= N) continue;
                    if (f0 < q.rope_cols) {
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            const int j = 8 * g4 + 4 * lhi;  // pair index of element 4*g4
                            const u32x2_t cv = rcos[b][g4], sv = rsin[b][g4];
                            float xo[4], yo[4], bx[4] = {0, 0, 0, 0}, by[4] = {0, 0, 0, 0};
                            if constexpr (HB) {
                                bias4(f0 + j, bx);
                                bias4(f0 + 32 + j, by);
                            }
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                float x = bf16r(acc[a][b][4 * g4 + e]);
                                float y = bf16r(acc[a + 1][b][4 * g4 + e]);
                                if constexpr (HB) {
                                    x = bf16r(x + bx[e]);
                                    y = bf16r(y + by[e]);
                                }
                                const float c = (e & 1) ? bf16hi(cv[e >> 1]) : bf16lo(cv[e >> 1]);
                                const float sn = (e & 1) ? bf16hi(sv[e >> 1]) : bf16lo(sv[e >> 1]);
                                // both products of BF16 values are exact in float32
                                xo[e] = fmaf(x, c, -(y * sn));
                                yo[e] = fmaf(y, c, x * sn);
                            }
                            put4(tl, wrow[a] + j, pack_bf16x2(xo[0], xo[1]),
                                 pack_bf16x2(xo[2], xo[3]));
                            put4(tl, wrow[a] + 32 + j, pack_bf16x2(yo[0], yo[1]),
                                 pack_bf16x2(yo[2], yo[3]));
                        }
                    } else if (f0 >= q.vt_col0) {
                        // transposed: row f - vt_col0 of vt holds this token at
                        // column vtcol[b] (32 lanes write 32 consecutive tokens)
                        if (tok < M) {
#pragma unroll
                            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                                for (int g = 0; g < 4; ++g) {
                                    const int32_t f4 = f0 + 32 * h2 + 8 * g + 4 * lhi;
                                    float bv[4] = {0, 0, 0, 0};
                                    if constexpr (HB) bias4(f4, bv);
                                    bf16_t *dst =
                                        q.vt + (size_t)(f4 - q.vt_col0) * q.ldvt + vtcol[b];
#pragma unroll
                                    for (int e = 0; e < 4; ++e) {
                                        float v = acc[a + h2][b][4 * g + e];
                                        if constexpr (HB) v = bf16r(v) + bv[e];
                                        dst[(size_t)e * q.ldvt] = (bf16_t)f32_to_bf16(v);
                                    }
                                }
                        }
                    } else {
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                            for (int g4 = 0; g4 < 4; ++g4) {
                                const int fl = wrow[a] + 32 * h2 + 8 * g4 + 4 * lhi;
                                float v[4], bv[4] = {0, 0, 0, 0};
                                if constexpr (HB) bias4(n0 + fl, bv);
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    v[e] = acc[a + h2][b][4 * g4 + e];
                                    if constexpr (HB) v[e] = bf16r(v[e]) + bv[e];
                                }
                                put4(tl, fl, pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                            }
                    }
                }
            };
            if (p.bias)
                tile(std::true_type{});
            else
                tile(std::false_type{});
        } else {
            // epilogue 0 (plain), 4 (plain + bias) and 3 (bias, then GELU)
            constexpr bool has_bias = EPI == 3 || EPI == 4;
#pragma unroll
            for (int a = 0; a < FA; ++a)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int fl = wrow[a] + 8 * g4 + 4 * lhi;
                    float v[4], bv[4];
                    // columns past N (clamped weight rows) are never stored; N is
                    // a multiple of 64, so a group of 4 is wholly in or out
                    if constexpr (has_bias) bias4(min(n0 + fl, N - 4), bv);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[e] = acc[a][b][4 * g4 + e];
                        if constexpr (has_bias) {
                            v[e] = bf16r(v[e]) + bv[e];
                            if constexpr (EPI == 3) v[e] = gelu_erf(bf16r(v[e]));
                        }
                    }
                    put4(tl, fl, pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                }
        }
    }
    // columns this tile writes to C: [n0, min(N, n0 + BN), and below vt_col0)
    int32_t n_end = min(N, n0 + BN);
    if constexpr (EPI == 2) n_end = min(n_end, max(p.qe.vt_col0, n0));
    if constexpr (EPI == 2 && HALF) n_end = min(N, p.qe.vt_col0);
    if constexpr (MODE == kWholeK && (EPI == 0 || EPI == 4)) {
        if (p.res) {
            // the residual add of the projections onto the hidden width:
            // C = bf16(res + y), y the BF16 output staged above, summed in
            // float32 and rounded once, as the LayerNorm's residual add does.
            // (Chunks not loaded early are loaded before the barrier, so their
            // latency overlaps the other waves' staging.)
            if constexpr (!RES_EARLY) res_load();
            LAYA_PHASE(ph[3]);
            __syncthreads();
            LAYA_PHASE(ph[4]);
#pragma unroll
            for (int i = 0; i < RNIT; ++i) {
                int tl, c;
                int32_t tok, f;
                if (res_chunk(i, tl, c, tok, f)) {
                    const u32x4_t y =
                        *reinterpret_cast<const u32x4_t *>(&sC[tl * BN + ((c ^ (tl & chunk_swizzle(NCH))) << 3)]);
                    u32x4_t o;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        o[q] = pack_bf16x2(bf16lo(rv[i][q]) + bf16lo(y[q]),
                                           bf16hi(rv[i][q]) + bf16hi(y[q]));
                    st16(p.C + (size_t)tok * p.ldc + f, o);
                }
            }
            phase_store();
            return;
        }
    }
    LAYA_PHASE(ph[3]);
    __syncthreads();
    LAYA_PHASE(ph[4]);
#pragma unroll 4
    for (int idx = tid; idx < BT * NCH; idx += G::NTHR) {
        const int tl = idx / NCH, c = idx % NCH;
        // half-head tiles: chunks 0, 1 are dimensions 16p.., chunks 2, 3 are 32+16p..
        const int32_t f = (EPI == 2 && HALF)
                              ? (bx >> 1) * 64 + (bx & 1) * 16 + (c < 2 ? 8 * c : 32 + 8 * (c - 2))
                              : n0 + 8 * c;
        const int32_t tok = t0 + tl;
        if (tok < M && f < n_end)
            st16(p.C + (size_t)tok * p.ldc + f,
                 *reinterpret_cast<const u32x4_t *>(&sC[tl * BN + ((c ^ (tl & chunk_swizzle(NCH))) << 3)]));
    }
    phase_store();
}

// Split-K reduce fused with the residual add and LayerNorm that follow a
// projection onto the hidden width (the output and down projections), one
// 64-lane wave per token row:
//   f = bf16(sum of the K ranges' float32 partials, in range order)
//       (with a bias: f = bf16(f + bias), as the biased epilogue rounds),
//   x <- bf16(x + f),  n <- bf16(LN(x) * gamma).
// The partials are the row-major ones of the split launch (MODE 3); the sums,
// roundings and the LayerNorm are those of the reduce launch and of the
// LayerNorm kernel, in the same order, so the results are bitwise theirs
// with one launch fewer.
template <int MAXC>
__global__ __launch_bounds__(64) void splitk_layernorm_kernel(
    const float *__restrict__ partial, int32_t splits, const bf16_t *__restrict__ bias,
    bf16_t *__restrict__ x, bf16_t *__restrict__ n, const float *__restrict__ gamma,
    const int32_t *count_dev, int32_t count_max, int32_t hidden, float eps) {
    const int32_t T = count_dev ? *count_dev : count_max;
    const int32_t row = blockIdx.x;
    const int lane = threadIdx.x;
    if (row >= T) return;
    const int nch = hidden >> 3;
    const size_t range_el = (size_t)count_max * hidden;  // floats per K range
    bf16_t *xr = x + (size_t)row * hidden;
    // every partial of the row's chunks is loaded before any is added, so the
    // loads are in flight together (a load-add chain would wait on each)
    f32x4_t pt[MAXC][kMaxSplits][2];
    u32x4_t xa[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + c * 64;
        if (ch < nch) {
            const float *pp = partial + (size_t)row * hidden + ch * 8;
#pragma unroll
            for (int sp = 0; sp < kMaxSplits; ++sp) {
                if (sp < splits) {
                    pt[c][sp][0] = *reinterpret_cast<const f32x4_t *>(pp);
                    pt[c][sp][1] = *reinterpret_cast<const f32x4_t *>(pp + 4);
                }
                pp += range_el;
            }
            xa[c] = ld16(xr + ch * 8);
        }
    }
    float v[MAXC][8];
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + c * 64;
        if (ch < nch) {
            f32x4_t s0 = pt[c][0][0], s1 = pt[c][0][1];
#pragma unroll
            for (int sp = 1; sp < kMaxSplits; ++sp) {
                if (sp < splits) {
                    s0 += pt[c][sp][0];
                    s1 += pt[c][sp][1];
                }
            }
            float f[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = bf16_to_f32(f32_to_bf16(f[e]));
            if (bias != nullptr) {
                const u32x4_t bw4 = ld16(bias + ch * 8);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    f[2 * q] = bf16_to_f32(f32_to_bf16(f[2 * q] + bf16lo(bw4[q])));
                    f[2 * q + 1] = bf16_to_f32(f32_to_bf16(f[2 * q + 1] + bf16hi(bw4[q])));
                }
            }
            u32x4_t o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float lo = bf16_to_f32(f32_to_bf16(bf16lo(xa[c][q]) + f[2 * q]));
                const float hi = bf16_to_f32(f32_to_bf16(bf16hi(xa[c][q]) + f[2 * q + 1]));
                v[c][2 * q] = lo;
                v[c][2 * q + 1] = hi;
                o[q] = pack_bf16x2(lo, hi);
            }
            st16(xr + ch * 8, o);
#pragma unroll
            for (int e = 0; e < 8; ++e) sum += v[c][e];
        }
    }
    layernorm_row_store<MAXC>(v, sum, lane, nch, hidden, eps, gamma, n + (size_t)row * hidden);
}

// ---------------------------------------------------------------------------
// 256 x 256 tiles for the large projections: two wave groups in ping-pong.
//
// One workgroup of 8 waves per compute unit, two per SIMD.  The waves form
// two groups of four (one wave of each group per SIMD) that take turns: while
// one group multiplies (16 MFMAs per wave on fragments already in registers),
// the other reads the fragments of its next K step from LDS and issues its
// share of the global -> LDS loads, and a workgroup barrier ends every phase.
// Each SIMD's matrix core thus always has one wave with MFMAs to issue; in the
// lock-step kernel above both waves of a SIMD wait at the same barrier and the
// matrix core idles there.
//
// K steps of 32 in a 4-slot ring (128 KB): the loads of step k + 3 are issued
// while step k is read, 5 to 6 phases before they are needed.  Group 0 loads
// the weight half of every step and group 1 the token half; a wave waits
// (vmcnt) for its own loads of a step before the barrier that precedes the
// step's first reader.  The remaining 32 KB of LDS gives each wave a private
// 4 KB area in which its output fragments are transposed to token rows, so
// the epilogue needs no workgroup barrier and writes 64-byte row segments.
//
// Each wave owns 128 weight rows x 64 tokens (4 x 2 fragments of 32 x 32);
// every output element is one chain of v_mfma_f32_32x32x16_bf16 over K in
// order, as in the other tile shapes, so the results are bitwise theirs.
// ---------------------------------------------------------------------------
namespace pp {
constexpr int BW = 256, BT = 256, BK = 32, SLOTS = 4;
constexpr int SLOT = (BW + BT) * BK;  // bf16 elements per ring slot (32 KB)
constexpr int FA = 4, FB = 2;         // fragments per wave (weight rows, tokens)
constexpr int D = 4;                  // loads (1 KB each) per wave per half step
constexpr int SCR = 2048;             // bf16 elements of scratch per wave (4 KB)
}  // namespace pp

// scratch chunk swizzle of a 32 x 32 BF16 fragment stored as [token][feature]
__device__ __forceinline__ int pp_sc(int tok, int chunk) {
    return tok * 32 + ((chunk ^ (tok & 3)) << 3);
}

template <int EPI>
__global__ __launch_bounds__(512) void gemm_pp_kernel(GemmParams p) {
    using namespace pp;
    const int32_t M = p.M_dev ? *p.M_dev : p.M_max;
    int bx = blockIdx.x, by = blockIdx.y;
    {
        const int live_by = (M + BT - 1) / BT;
        const int xw = p.split2d ? pick_xw(gridDim.x, live_by, BW, BT, 1) : 1;
        if (!(xw > 1 ? tile_order_2d(live_by, xw, bx, by) : tile_order(live_by, bx, by))) return;
    }
    const int32_t t0 = by * BT;
    if (t0 >= M) return;
    constexpr int BN = EPI == 1 ? BW / 2 : BW;  // output features per tile
    const int32_t n0 = bx * BN;
    const int N = p.N;

    __shared__ __attribute__((aligned(16))) bf16_t ring[SLOTS * SLOT];
    __shared__ __attribute__((aligned(16))) bf16_t scratch[8 * SCR];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int grp = wave >> 2, q = wave & 3;
    const int grp_u = __builtin_amdgcn_readfirstlane(grp);
    const int q_u = __builtin_amdgcn_readfirstlane(q);
    const int nk = p.K / BK;

    // Loads: group 0 fills the weight rows of a step, group 1 the token rows;
    // wave q covers 1 KB blocks q + 4 j (16 rows of 64 bytes each), lane L
    // physical chunk L % 4 of row 16 (q + 4 j) + L / 4.
    const uint32_t w_rows = EPI == 1 ? 2u * (uint32_t)N : (uint32_t)N;
    const uint32_t w_bytes = ((w_rows - 1) * (uint32_t)p.ldw + (uint32_t)p.K) * 2u;
    const uint32_t a_bytes = (((uint32_t)p.M_max - 1) * (uint32_t)p.lda + (uint32_t)p.K) * 2u;
    const bf16_t *src = grp_u == 0 ? p.W : p.A;
    const uint32_t src_bytes = grp_u == 0 ? w_bytes : a_bytes;
    uint32_t off[D];
#pragma unroll
    for (int j = 0; j < D; ++j) {
        const int r = 16 * (q + 4 * j) + (lane >> 2);  // row within the operand's 256
        const int c = pchunk<BK>(r, lane & 3);
        if (grp == 0) {
            int grow;
            if (EPI == 1) {
                int f = n0 + (r & 127);
                if (f >= N) f = N - 1;  // clamp: rows past N are computed, never stored
                grow = r < 128 ? f : N + f;
            } else {
                grow = n0 + r;
                if (grow >= N) grow = N - 1;
            }
            off[j] = (uint32_t)(grow * p.ldw + c * 8) * 2u;
        } else {
            const int trow = t0 + r;
            off[j] = trow < M ? (uint32_t)(trow * p.lda + c * 8) * 2u : a_bytes;
        }
    }
    auto issue = [&](int k) {
        bf16_t *base = ring + (k & (SLOTS - 1)) * SLOT + grp_u * (BW * BK) + q_u * 512;
#pragma unroll
        for (int j = 0; j < D; ++j)
            dma16(src, src_bytes, (lds_ptr_t)(base + j * 4 * 512), off[j], (uint32_t)(k * BK * 2));
    };

    // stage-row base of each weight fragment of this wave, and of its tokens
    int wrow[FA];
#pragma unroll
    for (int a = 0; a < FA; ++a)
        wrow[a] = EPI == 1 ? (a < 2 ? 64 * grp + 32 * a : 128 + 64 * grp + 32 * (a - 2))
                           : 128 * grp + 32 * a;
    const int tcol = 64 * q;
    const int l32 = lane & 31, lhi = lane >> 5;

    f32x16_t acc[FA][FB];
#pragma unroll
    for (int a = 0; a < FA; ++a)
#pragma unroll
        for (int b = 0; b < FB; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;
    bf16x8_t fw[2][FA], fa[2][FB];

    // prologue: steps 0..2 in flight, step 0 published
#pragma unroll
    for (int k = 0; k < 3; ++k)
        if (k < nk) issue(k);
    if (nk >= 3)
        wait_vmcnt<2 * D>();
    else if (nk == 2)
        wait_vmcnt<D>();
    else
        wait_vmcnt<0>();
    wait_lgkmcnt<0>();
    ring_barrier();

    // Phases, each ended by a workgroup barrier: in phase 2k group 0 reads
    // step k and group 1 multiplies step k - 1; in phase 2k + 1 group 0
    // multiplies step k and group 1 reads step k.  So both groups run the same
    // loop, read(k) then multiply(k), group 1 one phase behind (an extra
    // barrier before its loop, group 0's after).  A group that reads step k
    // also issues its half of step k + 3, into the slot of step k - 1, which
    // both groups have read by then.
    //
    // Before the barrier that ends a phase, each wave waits for its own loads
    // of the step read in the next phase, (phase + 1) / 2; `later` counts its
    // loads issued after those (steps are issued in order, D loads each).
    auto wait_later = [&](int later) {
        if (later >= 3)
            wait_vmcnt<3 * D>();
        else if (later == 2)
            wait_vmcnt<2 * D>();
        else if (later == 1)
            wait_vmcnt<D>();
        else
            wait_vmcnt<0>();
    };
    auto read_step = [&](int k) {
        const bf16_t *sw = ring + (k & (SLOTS - 1)) * SLOT;
        const bf16_t *sa = sw + BW * BK;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int ch = 2 * s + lhi;
#pragma unroll
            for (int a = 0; a < FA; ++a)
                fw[s][a] = *reinterpret_cast<const bf16x8_t *>(&sw[swz<BK>(wrow[a] + l32, ch)]);
#pragma unroll
            for (int b = 0; b < FB; ++b)
                fa[s][b] = *reinterpret_cast<const bf16x8_t *>(&sa[swz<BK>(tcol + 32 * b + l32, ch)]);
        }
    };
    auto multiply = [&]() {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int a = 0; a < FA; ++a)
#pragma unroll
                for (int b = 0; b < FB; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[s][a], fa[s][b],
                                                                        acc[a][b], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    if (grp_u == 1) {
        // phase 0: group 1 has nothing to multiply yet; step 0 must be visible
        // for its read in phase 1
        wait_later(min(2, nk - 1));
        ring_barrier();
    }
    for (int k = 0; k < nk; ++k) {
        read_step(k);
        if (k + 3 < nk) issue(k + 3);
        // next phase: group 0 multiplies (group 1 reads step k): step k needed
        // from group 0's loads; group 1's next phase reads step k + 1
        if (grp_u == 0)
            wait_later(min(3, nk - 1 - k));
        else if (k + 1 < nk)
            wait_later(min(2, nk - 2 - k));
        wait_lgkmcnt<0>();
        ring_barrier();
        multiply();
        // next phase reads step k + 1 (group 0) or is group 1's read of k + 1
        if (k + 1 < nk) wait_later(min(2, nk - 2 - k));
        ring_barrier();
    }
    if (grp_u == 0) ring_barrier();  // group 1's last multiply

    // Epilogue.  Accumulator element 4 g + e of lane l holds weight row
    // 8 g + 4 (l / 32) + e and token l % 32 of its fragment.  Each output
    // fragment goes through this wave's scratch as [token][feature] and is
    // stored as 16-byte pieces, four lanes per 64-byte token row segment.
    bf16_t *scr = scratch + wave * SCR;
    auto bf16r = [](float v) { return bf16_to_f32(f32_to_bf16(v)); };
    auto bias4 = [&](int32_t f, float (&bv)[4]) {
        const u32x2_t w = *reinterpret_cast<const u32x2_t *>(p.bias + f);
        bv[0] = bf16lo(w[0]);
        bv[1] = bf16hi(w[0]);
        bv[2] = bf16lo(w[1]);
        bv[3] = bf16hi(w[1]);
    };
    int buf = 0;
    // one 32 x 32 output fragment: values h[g][e] (feature 8 g + 4 lhi + e of
    // token l32), first column col0 of C, token tiles' first row trow0
    auto store_frag = [&](const float (&h)[4][4], int32_t col0, int32_t trow0) {
        bf16_t *s = scr + buf * 1024;
        buf ^= 1;
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *reinterpret_cast<u32x2_t *>(&s[pp_sc(l32, g) + 4 * lhi]) =
                u32x2_t{pack_bf16x2(h[g][0], h[g][1]), pack_bf16x2(h[g][2], h[g][3])};
        wait_lgkmcnt<0>();
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int tl = 16 * r + (lane >> 2), c = lane & 3;
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(&s[pp_sc(tl, c)]);
            const int32_t tok = trow0 + tl;
            if (tok < M) st16(p.C + (size_t)tok * p.ldc + col0 + 8 * c, v);
        }
    };
#pragma unroll
    for (int b = 0; b < FB; ++b) {
        const int32_t trow0 = t0 + tcol + 32 * b;
        const int32_t tok = trow0 + l32;
        if constexpr (EPI == 1) {
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const int32_t col0 = n0 + 64 * grp + 32 * a;
                if (col0 >= N) continue;
                float h[4][4];
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        h[g][e] = gelu_erf(acc[a][b][4 * g + e]) * acc[a + 2][b][4 * g + e];
                store_frag(h, col0, trow0);
            }
        } else if constexpr (EPI == 2) {
            const QkvEpilogue &qe = p.qe;
#pragma unroll
            for (int a = 0; a < FA; a += 2) {
                const int32_t f0 = n0 + wrow[a];  // first column of the head
                if (f0 >= N) continue;
                if (f0 < qe.rope_cols) {
                    const uint32_t ps = (uint32_t)qe.pos[tok < M ? tok : M - 1] * 32u;
                    float xo[4][4], yo[4][4];
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int j = 8 * g + 4 * lhi;  // pair index of element 4 g
                        const u32x2_t cv = *reinterpret_cast<const u32x2_t *>(qe.cos_tab + ps + j);
                        const u32x2_t sv = *reinterpret_cast<const u32x2_t *>(qe.sin_tab + ps + j);
                        float bxv[4] = {0, 0, 0, 0}, byv[4] = {0, 0, 0, 0};
                        if (p.bias) {
                            bias4(f0 + j, bxv);
                            bias4(f0 + 32 + j, byv);
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float x = bf16r(acc[a][b][4 * g + e]);
                            float y = bf16r(acc[a + 1][b][4 * g + e]);
                            if (p.bias) {
                                x = bf16r(x + bxv[e]);
                                y = bf16r(y + byv[e]);
                            }
                            const float c = (e & 1) ? bf16hi(cv[e >> 1]) : bf16lo(cv[e >> 1]);
                            const float sn = (e & 1) ? bf16hi(sv[e >> 1]) : bf16lo(sv[e >> 1]);
                            // both products of BF16 values are exact in float32
                            xo[g][e] = fmaf(x, c, -(y * sn));
                            yo[g][e] = fmaf(y, c, x * sn);
                        }
                    }
                    store_frag(xo, f0, trow0);
                    store_frag(yo, f0 + 32, trow0);
                } else if (f0 >= qe.vt_col0) {
                    // transposed: row f - vt_col0 of vt holds this token at
                    // column vt_tok[tok] (32 lanes write 32 consecutive tokens)
                    if (tok < M) {
                        bf16_t *vcol = qe.vt + qe.vt_tok[tok];
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                            for (int g = 0; g < 4; ++g) {
                                const int32_t f4 = f0 + 32 * h2 + 8 * g + 4 * lhi;
                                float bv[4] = {0, 0, 0, 0};
                                if (p.bias) bias4(f4, bv);
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    float v = acc[a + h2][b][4 * g + e];
                                    if (p.bias) v = bf16r(v) + bv[e];
                                    vcol[(size_t)(f4 + e - qe.vt_col0) * qe.ldvt] =
                                        (bf16_t)f32_to_bf16(v);
                                }
                            }
                    }
                } else {
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        float v[4][4];
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            float bv[4] = {0, 0, 0, 0};
                            if (p.bias) bias4(f0 + 32 * h2 + 8 * g + 4 * lhi, bv);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                v[g][e] = acc[a + h2][b][4 * g + e];
                                if (p.bias) v[g][e] = bf16r(v[g][e]) + bv[e];
                            }
                        }
                        store_frag(v, f0 + 32 * h2, trow0);
                    }
                }
            }
        } else {
            // epilogue 0 (plain), 4 (plain + bias) and 3 (bias, then GELU)
            constexpr bool has_bias = EPI == 3 || EPI == 4;
#pragma unroll
            for (int a = 0; a < FA; ++a) {
                const int32_t col0 = n0 + wrow[a];
                if (col0 >= N) continue;
                float v[4][4];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float bv[4];
                    if constexpr (has_bias) bias4(col0 + 8 * g + 4 * lhi, bv);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[g][e] = acc[a][b][4 * g + e];
                        if constexpr (has_bias) {
                            v[g][e] = bf16r(v[g][e]) + bv[e];
                            if constexpr (EPI == 3) v[g][e] = gelu_erf(bf16r(v[g][e]));
                        }
                    }
                }
                store_frag(v, col0, trow0);
            }
        }
    }
}

// Tile configurations: weight rows x tokens, wave grid, K step, stages.
using CfgXS = Cfg<32, 64, 1, 1, 64, 6>;    // small M, 1 wave (plain only)
using CfgXSG = Cfg<64, 64, 1, 1, 64, 4>;   // small M, 1 wave (GeGLU-capable)
using CfgS = Cfg<128, 64, 2, 2, 64, 4>;    // 4 waves of 64 rows x 32 tokens
using CfgM = Cfg<128, 128, 2, 4, 64, 4>;   // 8 waves of 64 x 32 (two per SIMD)
using CfgL = Cfg<256, 128, 2, 4, 64, 3>;   // 8 waves of 128 x 32
using CfgXL = Cfg<256, 256, 2, 4, 64, 2>;  // 8 waves of 128 x 64
using CfgM2 = Cfg<128, 128, 2, 2, 64, 2>;   // M with a 2-stage ring: 64 KB, two per CU
using CfgXS2 = Cfg<32, 64, 1, 2, 64, 13, 2>;  // small M, 2 waves of 32 x 32 + 2 loading, deep ring
using CfgXSG2 = Cfg<64, 64, 1, 2, 64, 8>;  // small M, 2 waves of 64 x 32, deep ring
// 3 heads x 256 tokens: twelve waves of 64 x 64, three per SIMD (16 x 16 tiles
// cover the QKV projection of 4096 tokens in one round of the 256 CUs)
using CfgQ3 = Cfg<192, 256, 3, 4, 64, 2>;
using CfgW2 = Cfg<256, 192, 4, 2, 64, 2>;  // 8 waves of 64 x 96

struct CfgInfo {
    int bw, bt;
};
constexpr CfgInfo kCfgs[kGemmConfigs] = {{CfgXS::BW, CfgXS::BT}, {CfgXSG::BW, CfgXSG::BT},
                                         {CfgS::BW, CfgS::BT},   {CfgM::BW, CfgM::BT},
                                         {CfgL::BW, CfgL::BT},   {CfgXL::BW, CfgXL::BT},
                                         {CfgM2::BW, CfgM2::BT}, {CfgXS2::BW, CfgXS2::BT},
                                         {CfgXSG2::BW, CfgXSG2::BT}, {pp::BW, pp::BT},
                                         {CfgQ3::BW, CfgQ3::BT}, {CfgW2::BW, CfgW2::BT}};

// Whole-K grids of at least 512 tiles may take the 2-D XCD split (on smaller
// grids it gained nothing and the padding cost a little): the grid rows
// that give every XCD a slot per tile of the largest block of any split
// (blocks only shrink with fewer live tokens).
int grid_rows_2d(int nbx, int nby) {
    int gy = nby;
    for (int xw = 2; xw <= 8; xw *= 2) {
        const int xtn = 8 / xw;
        const int64_t bmax = (int64_t)((nby + xtn - 1) / xtn) * ((nbx + xw - 1) / xw);
        gy = (int)std::max<int64_t>(gy, (8 * bmax + nbx - 1) / nbx);
    }
    return gy;
}

template <class G, int MODE>
hipError_t launch_mode(hipStream_t s, GemmParams p, int epilogue) {
    const int bn = epilogue == 1 ? G::BW / 2 : G::BW;
    const int nbx = (p.N + bn - 1) / bn, nby = (p.M_max + G::BT - 1) / G::BT;
    p.split2d = MODE == kWholeK && nbx * nby >= 512;
    const int gy = p.split2d ? grid_rows_2d(nbx, nby) : nby;
    const dim3 grid(nbx, gy, (MODE == kPartial || MODE == kPartialRows) ? p.splits : 1);
    // partial tiles are the same for the plain and bias epilogues (the bias
    // is applied by the reduce launch)
    if constexpr (MODE == kPartialRows) {
        hipLaunchKernelGGL((gemm_kernel<G, 0, kPartialRows>), grid, dim3(G::NTHR), 0, s, p);
    } else if (epilogue == 0 || (MODE == kPartial && epilogue == 3)) {
        if (MODE != kPartial && p.bias)
            hipLaunchKernelGGL((gemm_kernel<G, 4, MODE>), grid, dim3(G::NTHR), 0, s, p);
        else
            hipLaunchKernelGGL((gemm_kernel<G, 0, MODE>), grid, dim3(G::NTHR), 0, s, p);
    } else if (epilogue == 3) {
        hipLaunchKernelGGL((gemm_kernel<G, 3, MODE>), grid, dim3(G::NTHR), 0, s, p);
    } else if constexpr ((G::FA % 2 == 0 && G::RW % 64 == 0) || (G::RW == 32 && G::WW == 1)) {
        if (epilogue == 1)
            hipLaunchKernelGGL((gemm_kernel<G, 1, MODE>), grid, dim3(G::NTHR), 0, s, p);
        else
            hipLaunchKernelGGL((gemm_kernel<G, 2, MODE>), grid, dim3(G::NTHR), 0, s, p);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Small tiles take split K (partials, then a reduce launch); the large ones
// never do (K is always whole).
template <class G>
hipError_t launch_small(hipStream_t s, const GemmParams &p, int epilogue) {
    if (p.splits == 1) return launch_mode<G, kWholeK>(s, p, epilogue);
    const hipError_t e = launch_mode<G, kPartial>(s, p, epilogue);
    return e != hipSuccess ? e : launch_mode<G, kReduce>(s, p, epilogue);
}
template <class G>
hipError_t launch_large(hipStream_t s, const GemmParams &p, int epilogue) {
    return p.splits > 1 ? hipErrorInvalidValue : launch_mode<G, kWholeK>(s, p, epilogue);
}

// The ping-pong 256 x 256 tiles: whole K only.
hipError_t launch_pp(hipStream_t s, GemmParams p, int epilogue) {
    if (p.splits != 1 || p.K % pp::BK != 0) return hipErrorInvalidValue;
    const int bn = epilogue == 1 ? pp::BW / 2 : pp::BW;
    const int nbx = (p.N + bn - 1) / bn, nby = (p.M_max + pp::BT - 1) / pp::BT;
    p.split2d = nbx * nby >= 512;
    const dim3 grid(nbx, p.split2d ? grid_rows_2d(nbx, nby) : nby);
    const dim3 block(512);
    switch (epilogue) {
        case 0:
            if (p.bias)
                hipLaunchKernelGGL(gemm_pp_kernel<4>, grid, block, 0, s, p);
            else
                hipLaunchKernelGGL(gemm_pp_kernel<0>, grid, block, 0, s, p);
            break;
        case 1: hipLaunchKernelGGL(gemm_pp_kernel<1>, grid, block, 0, s, p); break;
        case 2: hipLaunchKernelGGL(gemm_pp_kernel<2>, grid, block, 0, s, p); break;
        case 3: hipLaunchKernelGGL(gemm_pp_kernel<3>, grid, block, 0, s, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// The split launch's partials, then the fused reduce + residual + LayerNorm.
template <class G>
hipError_t launch_split_layernorm(hipStream_t s, const GemmParams &p, bf16_t *x, bf16_t *n,
                                  const float *gamma, float eps) {
    const hipError_t e = launch_mode<G, kPartialRows>(s, p, 0);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(splitk_layernorm_kernel<2>, dim3(p.M_max), dim3(64), 0, s, p.partial,
                       p.splits, p.bias, x, n, gamma, p.M_dev, p.M_max, p.N, eps);
    return hipGetLastError();
}

}  // namespace

int gemm_max_splits(int config) {
    return (config <= 3 || config == 7 || config == 8) ? kMaxSplits : 1;
}

// The fastest whole-K tile shape for the pass's four projections at hidden
// 1024 and GeGLU width 2624, measured on MI355X over 257..8192 tokens with
// the weights streamed from HBM (every shape gives the same bits, so only
// time decides).  Most switch points are where the faster shape's grid would
// need one more round of the 256 CUs (two workgroups per CU for the 2-stage
// 128x128 tile); between 3072 and 4608 tokens the up projection's 192x256 and
// 256x192 shapes are within a few percent of each other, and the table
// follows the measurement.  Other shapes use the estimate below.
struct MeasuredTiles {
    int32_t N, K, epilogue, n;
    int32_t t_last[12];
    int8_t config[12];
};
constexpr MeasuredTiles kMeasuredTiles[] = {
    // QKV: 128x64 while 24 x T/64 tiles fit one round, then 128x128, the
    // two-per-CU 128x128, 192x256 (16 x T/256 tiles: one round up to 4096
    // tokens), 256x256, and 192x256 again
    {3072, 1024, 2, 6, {640, 1280, 2688, 4096, 5376, 1 << 30}, {2, 3, 6, 10, 5, 10}},
    // GeGLU up (64, 96 or 128 output features per tile); 192x256 and 256x192
    // fit one round up to 2304 tokens and two up to 4608
    {2624, 1024, 1, 12, {384, 768, 1536, 2304, 3072, 3584, 4352, 4608, 4736, 6144, 7936, 1 << 30},
     {2, 3, 6, 10, 5, 10, 11, 10, 6, 5, 6, 5}},
    // output projection (whole K above 1024 tokens)
    {1024, 1024, 0, 3, {2048, 4096, 1 << 30}, {2, 3, 6}},
    // down projection (whole K above 2048 tokens)
    {1024, 2624, 0, 2, {4096, 1 << 30}, {3, 6}},
};

GemmPlan plan_gemm_tiles(int32_t M, int32_t N, int32_t K, int epilogue) {
    for (const MeasuredTiles &m : kMeasuredTiles)
        if (m.N == N && m.K == K && m.epilogue == epilogue)
            for (int i = 0; i < m.n; ++i)
                if (M <= m.t_last[i]) return GemmPlan{m.config[i], 1};
    // Otherwise the tile shape with the least estimated time: the tiles the
    // busiest of the 256 compute units gets, times the per-tile cost, with
    // each shape's relative per-CU throughput (measured on the pass's shapes,
    // weights streamed from HBM).  The 2-stage 128x128 shape fits two workgroups per
    // CU, which hide each other's waits, but its shallow ring cannot cover
    // HBM latency on its own: it pays only where every CU runs a long queue
    // of tiles (at least 4).
    const int64_t nw = epilogue == 1 ? 2LL * N : N;
    const int cand[5] = {2, 3, 4, 5, 6};
    const double eff[5] = {0.45, 0.70, 0.85, 1.0, 1.0};
    GemmPlan g{3, 1};
    double best = 1e30;
    for (int i = 0; i < 5; ++i) {
        const CfgInfo &c = kCfgs[cand[i]];
        const int64_t tiles = ((nw + c.bw - 1) / c.bw) * ((M + c.bt - 1) / c.bt);
        const int64_t per_cu = (tiles + 255) / 256;
        const double e = (cand[i] == 6 && per_cu < 4) ? 0.50 : eff[i];
        const double t = (double)per_cu * c.bw * c.bt / e;
        if (t < best) {
            best = t;
            g.config = cand[i];
        }
    }
    return g;
}

GemmPlan plan_gemm(int32_t M_max, int32_t N, int32_t K, int epilogue) {
    const int64_t nw = epilogue == 1 ? 2LL * N : N;  // weight rows read
    const int np = K / KMULT;                   // 64-wide K pieces
    GemmPlan g{};
    if (M_max <= 256 && K <= 1024 && epilogue == 0 && N <= 1024) {
        // the output projection of a short call: four K ranges on 32-row
        // tiles; the split's reduce launch also takes the residual add and
        // the LayerNorm that follow (launch_gemm_layernorm), so the split
        // costs no extra launch
        g.config = 7;
        g.splits = std::min(4, np);
    } else if (M_max <= 256 && K <= 1024) {
        // few tokens, short K: whole K in one launch.  A K split spreads the
        // weight stream over more workgroups but costs a second launch,
        // which at these sizes takes longer than the split saves (measured
        // in the pass: 1x48 1.79 -> 1.59 ms, 4x64 2.07 -> 1.71 ms).
        // (the plain epilogue on 32-row tiles, three times as many workgroups:
        // 1x187 1.77 -> 1.71 ms; the 128-row tiles stay for the others, whose
        // 64-row alternative was slower in the pass.)  Up to 64 tokens the
        // two-wave deep-ring tiles keep more of the weight stream in flight.
        g.config = M_max <= 64 ? 7 : (epilogue == 0 ? 0 : 2);
        g.splits = 1;
    } else if (M_max <= 64) {
        // small M, long K: stream the weights with many narrow tiles; split K
        // until about 2 workgroups per CU
        g.config = (epilogue == 1 || epilogue == 2) ? 1 : 7;
        const int64_t tiles = (nw + kCfgs[g.config].bw - 1) / kCfgs[g.config].bw;
        int s = 1;
        while (s < 8 && tiles * s * 2 <= 512 && np / (s * 2) >= 2) s *= 2;
        g.splits = s;
    } else if (M_max <= 256) {
        g.config = 2;
        const int64_t tiles = ((nw + 127) / 128) * ((M_max + 63) / 64);
        int s = 1;
        while (s < 4 && tiles * s * 2 <= 512 && np / (s * 2) >= 4) s *= 2;
        g.splits = s;
    } else if (epilogue == 0 && N <= 1024 && M_max <= 1024) {
        // output and down projections up to 1024 rows: whole-K grids hold
        // only 64-128 tiles; up to 4 K ranges on the 128x64 tile, reduced by
        // the fused residual + LayerNorm launch (1x464 2.047 -> 1.703 ms; at
        // 1496 and 1856 rows the split was slower)
        g.config = 2;
        const int64_t tiles = ((nw + 127) / 128) * ((M_max + 63) / 64);
        int s = 1;
        while (s < 4 && tiles * s * 2 <= 512 && np / (s * 2) >= 4) s *= 2;
        g.splits = s;
    } else if (epilogue == 0 && N <= 1024 && K > 1024 && M_max <= 2048) {
        // the down projection up to 2048 rows: 96-116 whole-K 128x128 tiles
        // of 41 K steps leave most CUs idle; two K ranges, reduced by the
        // fused residual + LayerNorm launch (8x187 2.741 -> 2.729 ms, 4x464
        // 3.185 -> 3.174 ms; four ranges, or splitting the output projection
        // too, were slower)
        g.config = 3;
        g.splits = 2;
    } else {
        g = plan_gemm_tiles(M_max, N, K, epilogue);
    }
    return g;
}

size_t gemm_workspace_bytes(const GemmPlan &g, int32_t M_max, int32_t N, int epilogue) {
    if (g.splits <= 1) return 0;
    const CfgInfo &c = kCfgs[g.config];
    const int bn = epilogue == 1 ? c.bw / 2 : c.bw;
    const size_t tiles = (size_t)((N + bn - 1) / bn) * ((M_max + c.bt - 1) / c.bt);
    return tiles * g.splits * c.bw * c.bt * 4;
}

size_t gemm_static_scratch_bytes() { return kStaticScratchBytes; }

// The address of this device's copy of `scratch`, looked up once per device
// with that device current (the array's name is only a host-side stand-in;
// kernels must get the device address).
hipError_t gemm_static_scratch(float **ptr) {
    static std::mutex mu;
    static float *addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = static_cast<float *>(p);
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_gemm(hipStream_t s, const bf16_t *A, int32_t lda, const bf16_t *W,
                       int32_t ldw, bf16_t *C, int32_t ldc, const int32_t *M_dev,
                       int32_t M_max, int32_t N, int32_t K, int epilogue, const GemmPlan &plan,
                       float *partial, const QkvEpilogue *qe, const bf16_t *bias,
                       const bf16_t *res) {
    if (M_max <= 0 || N <= 0) return hipSuccess;
    // the residual add: whole K, plain (or plain + bias) epilogue, one of the
    // one-kernel tile shapes
    if (res && (epilogue != 0 || plan.splits != 1 || plan.config == kPingPongConfig ||
                reinterpret_cast<uintptr_t>(res) % 16 != 0 || ldc % 8 != 0))
        return hipErrorInvalidValue;
    if (epilogue < 0 || epilogue > 3 || (epilogue == 3 && !bias) || (epilogue == 1 && bias) ||
        reinterpret_cast<uintptr_t>(bias) % 8 != 0)
        return hipErrorInvalidValue;
    if (epilogue == 2 && (!qe || qe->rope_cols % 64 || qe->vt_col0 % 64 ||
                          qe->rope_cols > qe->vt_col0 || (qe->rope_cols > 0 && !qe->pos) ||
                          (qe->vt_col0 < N && (!qe->vt || !qe->vt_tok))))
        return hipErrorInvalidValue;
    if (K % KMULT != 0 || N % 64 != 0 || plan.config < 0 || plan.config >= kGemmConfigs ||
        plan.splits < 1 || plan.splits > K / KMULT || plan.splits > gemm_max_splits(plan.config))
        return hipErrorInvalidValue;
    if (plan.splits > 1 && !partial) return hipErrorInvalidValue;
    GemmParams p{A, lda, W, ldw, C, ldc, M_dev, M_max, N, K, plan.splits, partial,
                 epilogue == 2 ? *qe : QkvEpilogue{}, bias, 0, res};
    switch (plan.config) {
        case 0: return launch_small<CfgXS>(s, p, epilogue);
        case 1: return launch_small<CfgXSG>(s, p, epilogue);
        case 2: return launch_small<CfgS>(s, p, epilogue);
        case 3: return launch_small<CfgM>(s, p, epilogue);
        case 4: return launch_large<CfgL>(s, p, epilogue);
        case 5: return launch_large<CfgXL>(s, p, epilogue);
        case 6: return launch_large<CfgM2>(s, p, epilogue);
        case 7: return launch_small<CfgXS2>(s, p, epilogue);
        case 8: return launch_small<CfgXSG2>(s, p, epilogue);
        case 10: return launch_large<CfgQ3>(s, p, epilogue);
        case 11: return launch_large<CfgW2>(s, p, epilogue);
        default: return launch_pp(s, p, epilogue);
    }
}

hipError_t launch_gemm_layernorm(hipStream_t s, const bf16_t *A, int32_t lda, const bf16_t *W,
                                 int32_t ldw, const int32_t *M_dev, int32_t M_max, int32_t N,
                                 int32_t K, const GemmPlan &plan, float *partial,
                                 const bf16_t *bias, bf16_t *x, bf16_t *n, const float *gamma,
                                 float eps) {
    if (M_max <= 0) return hipSuccess;
    if (plan.splits == 1) {
        // whole K: the GEMM's store does the residual add into x, then the
        // LayerNorm of x (no second input)
        if (!x || !n || !gamma || N % 64 != 0 || N > 1024) return hipErrorInvalidValue;
        const hipError_t e =
            launch_gemm(s, A, lda, W, ldw, x, N, M_dev, M_max, N, K, 0, plan, nullptr, nullptr,
                        bias, x);
        return e != hipSuccess ? e : launch_layernorm(s, x, nullptr, n, gamma, M_dev, M_max, N, eps);
    }
    // one wave per row holds 16 values per lane: widths up to 1024, multiples of 64
    if (N % 64 != 0 || N > 1024 || K % KMULT != 0 || plan.splits < 2 ||
        plan.splits > K / KMULT || plan.splits > gemm_max_splits(plan.config) || !partial ||
        !x || !n || !gamma || reinterpret_cast<uintptr_t>(bias) % 16 != 0)
        return hipErrorInvalidValue;
    GemmParams p{A, lda, W, ldw, nullptr, 0, M_dev, M_max, N, K, plan.splits, partial,
                 QkvEpilogue{}, bias, 0, nullptr};
    switch (plan.config) {
        case 0: return launch_split_layernorm<CfgXS>(s, p, x, n, gamma, eps);
        case 1: return launch_split_layernorm<CfgXSG>(s, p, x, n, gamma, eps);
        case 2: return launch_split_layernorm<CfgS>(s, p, x, n, gamma, eps);
        case 3: return launch_split_layernorm<CfgM>(s, p, x, n, gamma, eps);
        case 7: return launch_split_layernorm<CfgXS2>(s, p, x, n, gamma, eps);
        case 8: return launch_split_layernorm<CfgXSG2>(s, p, x, n, gamma, eps);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace laya

#ifdef LAYA_GEMM_PHASES
// Host access to the diagnostic build's phase records (not part of the
// product library's interface): copy out the first `bytes` bytes, or clear
// them all.
extern "C" int laya_gemm_phases_read(void *dst, size_t bytes) {
    return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(gemm_phases), bytes, 0,
                                    hipMemcpyDeviceToHost);
}
extern "C" int laya_gemm_phases_clear() {
    void *ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(gemm_phases));
    if (e == hipSuccess) e = hipMemset(ptr, 0, sizeof(unsigned long long) * kPhaseWorkgroups * 10);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    return (int)e;
}
#endif
