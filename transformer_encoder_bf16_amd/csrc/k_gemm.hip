// BF16 GEMMs of the encoder pass on gfx950 matrix cores: C = bf16(A W^T)
// with float32 accumulation (the QKV, output-projection, GeGLU-up and down
// projections, which take most of the pass's time: 72-74% of traced kernel
// time on the pages' Hopper build, "[Performance]: Optimize native Rust/CUDA
// Laya inference #66", section Implementation priorities).
//
// A: activations [M tokens][K], W: weights [N][K] (nn.Linear layout), both
// K-contiguous.  The weight tile is the MFMA "A" operand (rows = output
// features) and the token tile the "B" operand (columns = tokens), so each
// lane of a 32x32 accumulator ends up holding four consecutive output
// features of one token and stores them with one 8-byte write.
//
// Block tile: 128 weight rows x 128 tokens x 64 K, four waves in a 2x2
// arrangement, each wave 64 weight rows x 64 tokens = 2x2 MFMA 32x32x16
// blocks.  Tiles are staged global -> registers -> LDS, double-buffered, one
// barrier per K step.  LDS rows are 128 bytes; the eight 16-byte chunks of
// row r are XOR-swizzled with (r >> 1) & 7 so that the 16 lanes of one
// ds_read_b128 phase hit distinct banks.
//
// GeGLU epilogue (epilogue 1): the weight tile's first 64 rows are rows
// n0..n0+63 of W (the GELU half) and the last 64 rows are rows N+n0..N+n0+63
// (the gate half), so u and g of the same output feature sit in the same
// lane and register: h = bf16(GELU(u) * g) with u, g unrounded float32.
#include "kernels.h"

namespace laya {

namespace {

constexpr int BW = 128;  // weight rows per block tile
constexpr int BT = 128;  // tokens per block tile
constexpr int BK = 64;   // K per step
constexpr int ROWB = BK * 2;  // bytes per LDS row

__device__ __forceinline__ int swz(int row, int chunk) {
    return row * BK + ((chunk ^ ((row >> 1) & 7)) << 3);
}

// GELU(z) = z Phi(z) = 0.5 z erfc(-z / sqrt 2).  erfc keeps full relative
// accuracy in the negative tail, where 1 + erf(z / sqrt 2) would cancel.
__device__ __forceinline__ float gelu_erf(float z) {
    return 0.5f * z * erfcf(-z * 0.70710678118654752f);
}

template <int EPI>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(
    const bf16_t *__restrict__ A, int32_t lda, const bf16_t *__restrict__ W, int32_t ldw,
    bf16_t *__restrict__ C, int32_t ldc, const int32_t *M_dev, int32_t M_max, int32_t N,
    int32_t K) {
    const int32_t M = M_dev ? *M_dev : M_max;
    const int32_t t0 = blockIdx.y * BT;
    if (t0 >= M) return;
    // output features covered by this block
    constexpr int BN = EPI ? BW / 2 : BW;
    const int32_t n0 = blockIdx.x * BN;

    __shared__ __attribute__((aligned(16))) bf16_t sW[2][BW * BK];
    __shared__ __attribute__((aligned(16))) bf16_t sA[2][BT * BK];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wr = wave >> 1;  // wave row (weight rows)
    const int wc = wave & 1;   // wave column (tokens)

    // Global -> register staging: each thread moves 4 chunks of W and 4 of A.
    // chunk id q = tid + 256*i: row = q >> 3, chunk = q & 7.
    int w_src_row[4];
    bool w_ok[4];
    bool a_ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = (tid + 256 * i) >> 3;
        int wrow;
        if (EPI) {
            wrow = (row < 64) ? (n0 + row) : (N + n0 + row - 64);
            w_ok[i] = (n0 + (row & 63)) < N;
        } else {
            wrow = n0 + row;
            w_ok[i] = wrow < N;
        }
        w_src_row[i] = wrow;
        a_ok[i] = (t0 + row) < M;
    }
    const int chunk_l = tid & 7;

    u32x4_t rw[4], ra[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (tid + 256 * i) >> 3;
            rw[i] = w_ok[i] ? ld16(W + (size_t)w_src_row[i] * ldw + k0 + chunk_l * 8)
                            : u32x4_t{0, 0, 0, 0};
            ra[i] = a_ok[i] ? ld16(A + (size_t)(t0 + row) * lda + k0 + chunk_l * 8)
                            : u32x4_t{0, 0, 0, 0};
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (tid + 256 * i) >> 3;
            *reinterpret_cast<u32x4_t *>(&sW[buf][swz(row, chunk_l)]) = rw[i];
            *reinterpret_cast<u32x4_t *>(&sA[buf][swz(row, chunk_l)]) = ra[i];
        }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

    // Weight-row base of each of the wave's two A fragments within the tile.
    int wbase[2];
    if (EPI) {
        wbase[0] = wr * 32;       // GELU half
        wbase[1] = 64 + wr * 32;  // gate half
    } else {
        wbase[0] = wr * 64;
        wbase[1] = wr * 64 + 32;
    }
    const int tbase = wc * 64;
    const int l32 = lane & 31, lhi = lane >> 5;

    const int nk = K / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const int ch = 2 * s + lhi;
            bf16x8_t fw[2], fa[2];
#pragma unroll
            for (int a = 0; a < 2; ++a)
                fw[a] = *reinterpret_cast<const bf16x8_t *>(&sW[cur][swz(wbase[a] + l32, ch)]);
#pragma unroll
            for (int b = 0; b < 2; ++b)
                fa[b] = *reinterpret_cast<const bf16x8_t *>(&sA[cur][swz(tbase + 32 * b + l32, ch)]);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[a], fa[b], acc[a][b],
                                                                        0, 0, 0);
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  Accumulator element e of lane l in a 32x32 block holds
    // row (weight row) 8*(e/4) + 4*(l/32) + e%4 and column (token) l%32.
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int32_t tok = t0 + tbase + 32 * b + l32;
        if (tok >= M) continue;
        bf16_t *crow = C + (size_t)tok * ldc;
        if (EPI) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int32_t f = n0 + wr * 32 + 8 * g4 + 4 * lhi;
                if (f >= N) continue;
                float h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    h[e] = gelu_erf(acc[0][b][4 * g4 + e]) * acc[1][b][4 * g4 + e];
                u32x2_t pk = {pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
                *reinterpret_cast<u32x2_t *>(crow + f) = pk;
            }
        } else {
#pragma unroll
            for (int a = 0; a < 2; ++a) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int32_t f = n0 + wbase[a] + 8 * g4 + 4 * lhi;
                    if (f >= N) continue;
                    const f32x16_t &v = acc[a][b];
                    u32x2_t pk = {pack_bf16x2(v[4 * g4], v[4 * g4 + 1]),
                                  pack_bf16x2(v[4 * g4 + 2], v[4 * g4 + 3])};
                    *reinterpret_cast<u32x2_t *>(crow + f) = pk;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm(hipStream_t s, const bf16_t *A, int32_t lda, const bf16_t *W,
                       int32_t ldw, bf16_t *C, int32_t ldc, const int32_t *M_dev,
                       int32_t M_max, int32_t N, int32_t K, int epilogue) {
    if (M_max <= 0 || N <= 0) return hipSuccess;
    if (K % BK != 0 || N % 64 != 0) return hipErrorInvalidValue;
    const int bn = epilogue ? BW / 2 : BW;
    const dim3 grid((N + bn - 1) / bn, (M_max + BT - 1) / BT);
    if (epilogue)
        hipLaunchKernelGGL(gemm_bf16_kernel<1>, grid, dim3(256), 0, s, A, lda, W, ldw, C, ldc,
                           M_dev, M_max, N, K);
    else
        hipLaunchKernelGGL(gemm_bf16_kernel<0>, grid, dim3(256), 0, s, A, lda, W, ldw, C, ldc,
                           M_dev, M_max, N, K);
    return hipGetLastError();
}

}  // namespace laya
