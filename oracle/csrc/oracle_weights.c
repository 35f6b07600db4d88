/*
 * CPU oracle: counter-based weight generator and byte digest.
 *
 * TEST INFRASTRUCTURE ONLY.  This file belongs to the CPU oracle: only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it.  It shares no code with the HIP library.
 *
 * The pages load a trained checkpoint ("English 421M", page "[Performance]:
 * Optimize native Rust/CUDA Laya inference #66", section Recorded baseline
 * and environment).  No checkpoint exists here, so the weights are synthetic
 * BF16 values of roughly N(0, 0.02^2), drawn per element from a counter so
 * that any element can be regenerated on its own:
 *
 *   key   = (tensor_id << 40) | (3 * idx + j)          j = 0, 1, 2
 *   r_j   = the (key + 1)-th output of SplitMix64 started at state `seed`
 *           (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *           generators", OOPSLA 2014): mix64(seed + (key + 1) * GOLDEN)
 *   u_0..u_11 = the four 16-bit fields of r_0, r_1, r_2 (low field first)
 *   z     = (sum u_k - 393210) / 65536      Irwin-Hall(12), mean 0, var ~ 1;
 *                                           every step is exact in float32
 *   w     = bf16_rne(0.02f * z)
 *
 * idx is the element's index in nn.Linear [out][in] order.
 */
#include <stdint.h>
#include <stddef.h>

static const uint64_t GOLDEN = 0x9e3779b97f4a7c15ULL;

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

/* The (key + 1)-th output of a SplitMix64 generator whose state starts at seed. */
uint64_t oracle_splitmix64_at(uint64_t seed, uint64_t key) {
    return mix64(seed + (key + 1) * GOLDEN);
}

/* float32 -> bfloat16 bits, round to nearest even, NaN kept quiet. */
static inline uint16_t f32_to_bf16_bits(float f) {
    union { float f; uint32_t u; } v;
    v.f = f;
    if ((v.u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((v.u >> 16) | 0x0040u);
    uint32_t lsb = (v.u >> 16) & 1u;
    return (uint16_t)((v.u + 0x7fffu + lsb) >> 16);
}

/* Irwin-Hall(12) draw z for element idx of tensor tensor_id (exact float32). */
float oracle_irwin_hall(uint64_t seed, uint32_t tensor_id, uint64_t idx) {
    uint32_t s = 0;
    for (uint64_t j = 0; j < 3; ++j) {
        uint64_t key = ((uint64_t)tensor_id << 40) | (3u * idx + j);
        uint64_t r = oracle_splitmix64_at(seed, key);
        s += (uint32_t)(r & 0xffffu) + (uint32_t)((r >> 16) & 0xffffu) +
             (uint32_t)((r >> 32) & 0xffffu) + (uint32_t)((r >> 48) & 0xffffu);
    }
    return ((float)s - 393210.0f) / 65536.0f;
}

/* Fill out[0..n) with the BF16 bits of tensor tensor_id. */
void oracle_weights_bf16(uint64_t seed, uint32_t tensor_id, uint64_t n, uint16_t *out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        float z = oracle_irwin_hall(seed, tensor_id, (uint64_t)i);
        out[i] = f32_to_bf16_bits(0.02f * z);
    }
}

/* FNV-1a, 64-bit, over n bytes. */
uint64_t oracle_fnv1a64(const uint8_t *p, uint64_t n) {
    uint64_t h = 14695981039346656037ULL;
    for (uint64_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= 1099511628211ULL;
    }
    return h;
}
