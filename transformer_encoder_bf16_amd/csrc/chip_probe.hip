// Chip probes for the roofline: what the matrix cores, the LDS and one
// workgroup's HBM -> LDS stream deliver on this GPU, measured with HIP events
// over back-to-back launches.  A standalone program (no library calls); it
// prints one JSON object per measurement.  Every access stays inside its
// buffer: the LDS probe indexes a 64 KB array modulo its size, and the
// stream probe's buffer resources cover exactly the bytes it reads.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((address_space(3))) void *lds_ptr;

#define CHECK(x)                                                                  \
    do {                                                                          \
        hipError_t e_ = (x);                                                      \
        if (e_ != hipSuccess) {                                                   \
            std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));  \
            std::exit(1);                                                         \
        }                                                                         \
    } while (0)

// Four independent chains of v_mfma_f32_32x32x16_bf16 per wave, no memory.
__global__ __launch_bounds__(256) void mfma_loop(float *out, int iters) {
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(threadIdx.x * 0.001f);
        b[i] = (__bf16)(i * 0.5f);
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float s = 0.f;
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    if (s == 1234.5f) out[blockIdx.x] = s;  // keeps the chains live
}

// ds_read_b128 over a 64 KB array: consecutive lanes read consecutive
// 16-byte chunks (no bank conflicts); the index wraps inside the array.
__global__ __launch_bounds__(512) void lds_read(unsigned *out, int iters) {
    __shared__ u32x4 buf[4096];
    for (int i = threadIdx.x; i < 4096; i += 512) buf[i] = u32x4{(unsigned)i, 1u, 2u, 3u};
    __syncthreads();
    u32x4 acc = {0, 0, 0, 0};
    int idx = threadIdx.x & 4095;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc ^= buf[(idx + j * 512) & 4095];
        idx = (idx + 64) & 4095;
    }
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x12345678u) out[blockIdx.x] = 1;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8));
}

// One workgroup of NW waves streams `bytes` contiguous bytes into an LDS ring
// with buffer loads (16 bytes per lane, 1 KB per wave-load), keeping 16 loads
// per wave in flight.
template <int NW>
__global__ __launch_bounds__(NW * 64) void dma_stream(const unsigned char *src, uint32_t bytes,
                                                      unsigned *out) {
    __shared__ __attribute__((aligned(16))) unsigned char ring[NW * 8 * 1024];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const unsigned char *base = src + (size_t)blockIdx.x * bytes;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char *>(base), (short)0,
                                                      (int)bytes, 0x00020000);
    const int nload = (int)(bytes / (1024u * NW));
    for (int j = 0; j < nload; ++j) {
        const uint32_t voff = (uint32_t)((j * NW + w) * 1024 + lane * 16);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(ring + ((j & 7) * NW + wu) * 1024),
                                                 16, voff, 0, 0, 0);
        if (j >= 16) wait_vmcnt<16>();
    }
    wait_vmcnt<0>();
    __syncthreads();
    if (threadIdx.x == 0 && ring[5] == 0x7f && ring[900] == 0x3e) out[blockIdx.x] = 1;
}

template <class F>
double us_per_launch(F launch, int reps) {
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    launch(0);
    CHECK(hipEventRecord(e0));
    for (int r = 0; r < reps; ++r) launch(r + 1);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    CHECK(hipEventDestroy(e0));
    CHECK(hipEventDestroy(e1));
    return ms * 1e3 / reps;
}

}  // namespace

int main() {
    hipDeviceProp_t prop;
    CHECK(hipGetDeviceProperties(&prop, 0));
    const int cus = prop.multiProcessorCount;
    float *fout;
    unsigned *uout;
    CHECK(hipMalloc(&fout, 1 << 20));
    CHECK(hipMalloc(&uout, 1 << 20));
    std::printf("{\"probe\": \"device\", \"name\": \"%s\", \"arch\": \"%s\", \"cus\": %d}\n", prop.name,
                prop.gcnArchName, cus);

    // matrix cores: 1, 2, 4 and 8 four-wave workgroups per CU
    for (int per_cu = 1; per_cu <= 8; per_cu *= 2) {
        const int iters = 20000, grid = cus * per_cu;
        const double us = us_per_launch(
            [&](int) { hipLaunchKernelGGL(mfma_loop, dim3(grid), dim3(256), 0, 0, fout, iters); }, 3);
        const double flop = (double)grid * 4 * iters * 4 * 32768.0;
        std::printf("{\"probe\": \"mfma_bf16_32x32x16\", \"workgroups_per_cu\": %d, \"us\": %.1f, "
                    "\"tflops\": %.1f}\n", per_cu, us, flop / us / 1e6);
    }
    // LDS reads: 1 and 2 workgroups of 512 threads per CU
    for (int per_cu = 1; per_cu <= 2; ++per_cu) {
        const int iters = 2000, grid = cus * per_cu;
        const double us = us_per_launch(
            [&](int) { hipLaunchKernelGGL(lds_read, dim3(grid), dim3(512), 0, 0, uout, iters); }, 3);
        const double bytes = (double)grid * 512 * iters * 8 * 16;
        std::printf("{\"probe\": \"lds_read_b128\", \"workgroups_per_cu\": %d, \"us\": %.1f, "
                    "\"tb_per_s\": %.1f, \"bytes_per_clk_per_cu_at_2.1ghz\": %.1f}\n",
                    per_cu, us, bytes / us / 1e6, bytes / (us * 1e-6) / cus / 2.1e9);
    }
    // one workgroup's HBM -> LDS stream, 16 workgroups (so HBM is far from
    // its limit), rotated over 1 GiB so every launch reads cold data
    {
        const size_t total = size_t(1) << 30;
        unsigned char *src;
        CHECK(hipMalloc(&src, total));
        CHECK(hipMemset(src, 1, total));
        const int grid = 16;
        const double empty = us_per_launch(
            [&](int) { hipLaunchKernelGGL(dma_stream<8>, dim3(grid), dim3(512), 0, 0, src, 0u, uout); }, 8);
        for (uint32_t kb : {256u, 512u}) {
            const uint32_t bytes = kb * 1024u;
            const size_t span = (size_t)grid * bytes;
            const int nslot = (int)(total / span);
            const double us8 = us_per_launch([&](int r) {
                hipLaunchKernelGGL(dma_stream<8>, dim3(grid), dim3(512), 0, 0,
                                   src + (size_t)(r % nslot) * span, bytes, uout);
            }, 8);
            const double us16 = us_per_launch([&](int r) {
                hipLaunchKernelGGL(dma_stream<16>, dim3(grid), dim3(1024), 0, 0,
                                   src + (size_t)(r % nslot) * span, bytes, uout);
            }, 8);
            std::printf("{\"probe\": \"one_workgroup_stream\", \"kb_per_workgroup\": %u, "
                        "\"empty_launch_us\": %.2f, \"us_8_waves\": %.2f, \"us_16_waves\": %.2f, "
                        "\"gb_per_s_per_workgroup_8_waves\": %.0f, \"gb_per_s_per_workgroup_16_waves\": %.0f}\n",
                        kb, empty, us8, us16, bytes / (us8 - empty) / 1e3, bytes / (us16 - empty) / 1e3);
        }
        CHECK(hipFree(src));
    }
    CHECK(hipDeviceSynchronize());
    CHECK(hipFree(fout));
    CHECK(hipFree(uout));
    return 0;
}
