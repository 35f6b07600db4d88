// Host engine of the encoder pass: the C ABI of include/laya_encoder.h.
//
// The engine keeps the weights resident on the device, together with the
// rotary tables, one activation workspace sized for max_batch x max_seq
// tokens, pinned staging memory for the per-run index upload, and a cache of
// per-shape hipGraphs (the executor design of page "Laya native CUDA worker",
// section Prepare the checkpoint and bundle, and of "[RFC]: Native Laya
// inference with Rust and CUDA #14", section Design: a shape seen for the
// first time gets its buffers, two warm-up passes and a synchronous capture).
// A run packs the valid tokens of all rows on the host and moves the packed
// indices to the device in a single copy whose host source the caller may
// free on return (the upload batching asked for in "[Performance]: Optimize
// native Rust/CUDA Laya inference #66", section Implementation priorities),
// then queues the layer schedule: gather; per layer LayerNorm(+residual),
// QKV GEMM, RoPE, attention, output GEMM, LayerNorm(+residual), GeGLU-up
// GEMM, down GEMM; final LayerNorms.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <tuple>
#include <vector>

#include "kernels.h"
#include "laya_encoder.h"

using laya::AttnBlock;

namespace {

thread_local std::string g_last_error;

int set_global_error(int code, const std::string &msg) {
    g_last_error = msg;
    return code;
}

// ---------------------------------------------------------------------------
// Rotary tables: cos/sin of p * theta^(-2i/d) in double, rounded once to BF16
// (nearest, ties to even) straight from the double's bit pattern.
// ---------------------------------------------------------------------------
uint16_t double_to_bf16_rne(double x) {
    uint64_t u;
    std::memcpy(&u, &x, 8);
    const uint64_t sign = u >> 63;
    const int e = (int)((u >> 52) & 0x7ff);
    const uint64_t mant = u & ((1ull << 52) - 1);
    if (e == 0 && mant == 0) return (uint16_t)(sign << 15);
    if (e == 0x7ff) return (uint16_t)((sign << 15) | 0x7f80u | (mant ? 0x40u : 0u));
    const int eb = e - 1023 + 127;  // BF16 biased exponent
    if (eb <= 0 || eb >= 255) {
        // outside the normal BF16 range: go through float (not reached by tables)
        float f = (float)x;
        uint32_t b;
        std::memcpy(&b, &f, 4);
        return (uint16_t)((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
    }
    // keep the top 7 mantissa bits; the 45 dropped bits decide the rounding
    uint64_t keep = mant >> 45;
    const uint64_t rest = mant & ((1ull << 45) - 1);
    const uint64_t half = 1ull << 44;
    uint32_t bits = ((uint32_t)eb << 7) | (uint32_t)keep;
    if (rest > half || (rest == half && (keep & 1))) bits += 1;  // may carry into exponent
    return (uint16_t)((sign << 15) | bits);
}

void build_rope_table(double theta, int max_pos, int head_dim, uint16_t *c, uint16_t *s) {
    const int half = head_dim / 2;
    for (int i = 0; i < half; ++i) {
        const double inv_freq = std::pow(theta, -2.0 * (double)i / (double)head_dim);
        for (int p = 0; p < max_pos; ++p) {
            const double ang = (double)p * inv_freq;
            c[p * half + i] = double_to_bf16_rne(std::cos(ang));
            s[p * half + i] = double_to_bf16_rne(std::sin(ang));
        }
    }
}

// ---------------------------------------------------------------------------
// Attention work list: blocks of <= 64 queries of one row.  Full pass: each
// row's tokens in chunks of 64.  Marker pass: runs of consecutive marker
// entries from the same row, chunked at 64.  Key range per block: the whole
// row on global layers; [min pos - hw, max pos + hw] clipped to the row on
// local layers (one list per window width is built).  The first key is
// rounded down to a multiple of the 64-key tile, so every query meets its keys
// in the same tiles whichever block it sits in: a query's result is then
// bitwise the same in the full pass and in the marker pass (extra fully
// masked keys leave the online softmax exactly unchanged).
// ---------------------------------------------------------------------------
int align_down(int k) { return k - k % 64; }

// Heaviest blocks first (most key tiles), ties in list order.  The kernel
// runs as long as its busiest compute unit, and workgroups are handed out
// in dispatch order, breadth first over the CUs: with the longest chains
// dispatched first each CU gets one heavy block per round, instead of some
// CUs drawing several of a 16x512 batch's 512-key rows.  Blocks are
// independent, so the order changes no result.
void heaviest_first(AttnBlock *blocks, int n) {
    std::stable_sort(blocks, blocks + n, [](const AttnBlock &a, const AttnBlock &b) {
        return a.k_hi - a.k_lo > b.k_hi - b.k_lo;
    });
}

void build_blocks_full(const int32_t *row_off, const int32_t *vcol0, int B, int half_window,
                       AttnBlock *out, int *n_out) {
    int n = 0;
    for (int b = 0; b < B; ++b) {
        const int kt0 = row_off[b], len = row_off[b + 1] - row_off[b];
        for (int i0 = 0; i0 < len; i0 += laya::kAttnQueries) {
            const int cnt = std::min(laya::kAttnQueries, len - i0);
            AttnBlock a{};
            a.kt0 = kt0;
            a.klen = len;
            a.vcol0 = vcol0[b];
            if (half_window < 0) {
                a.k_lo = 0;
                a.k_hi = len;
            } else {
                a.k_lo = align_down(std::max(0, i0 - half_window));
                a.k_hi = std::min(len, i0 + cnt - 1 + half_window + 1);
            }
            a.q_first = kt0 + i0;
            a.q_count = cnt;
            out[n++] = a;
        }
    }
    heaviest_first(out, n);
    *n_out = n;
}

// q_row[r] = row of query r, q_pos[r] = its position.
void build_blocks_list(const int32_t *row_off, const int32_t *vcol0, const int32_t *q_row,
                       const int32_t *q_pos, int n_q, int half_window, AttnBlock *out,
                       int *n_out) {
    int n = 0;
    int r = 0;
    while (r < n_q) {
        const int row = q_row[r];
        int e = r;
        while (e < n_q && q_row[e] == row && e - r < laya::kAttnQueries) ++e;
        int pmin = q_pos[r], pmax = q_pos[r];
        for (int j = r; j < e; ++j) {
            pmin = std::min(pmin, q_pos[j]);
            pmax = std::max(pmax, q_pos[j]);
        }
        const int len = row_off[row + 1] - row_off[row];
        AttnBlock a{};
        a.kt0 = row_off[row];
        a.klen = len;
        a.vcol0 = vcol0[row];
        if (half_window < 0) {
            a.k_lo = 0;
            a.k_hi = len;
        } else {
            a.k_lo = align_down(std::max(0, pmin - half_window));
            a.k_hi = std::min(len, pmax + half_window + 1);
        }
        a.q_first = r;
        a.q_count = e - r;
        out[n++] = a;
        r = e;
    }
    heaviest_first(out, n);
    *n_out = n;
}

int config_check(const laya_config *c, std::string *why) {
    if (!c) {
        *why = "config is NULL";
        return LAYA_E_INVALID;
    }
    if (c->abi_version != LAYA_ABI_VERSION) {
        *why = "abi_version mismatch";
        return LAYA_E_ABI;
    }
    if (c->vocab <= 0 || c->hidden <= 0 || c->n_heads <= 0 || c->head_dim <= 0 || c->ffn <= 0 ||
        c->n_enc_layers <= 0 || c->n_dec_layers <= 0 || c->global_every <= 0 || c->window < 0 ||
        c->max_batch <= 0 || c->max_seq <= 0 || c->max_markers < 0 || !(c->ln_eps > 0.f) ||
        c->max_graphs <= 0 || c->workspace_budget_mib <= 0 || c->dec_head < 0 || c->dec_head > 1 ||
        !(c->theta_global > 1.f) || !(c->theta_local > 1.f)) {
        *why = "non-positive size or parameter in config";
        return LAYA_E_INVALID;
    }
    if (c->n_heads * c->head_dim != c->hidden) {
        *why = "hidden != n_heads * head_dim";
        return LAYA_E_INVALID;
    }
    if (c->head_dim != 64) {
        *why = "head_dim must be 64";
        return LAYA_E_UNSUPPORTED;
    }
    // one 64-lane wave holds a whole row in the fused split reduce + LayerNorm
    // that follows the output and down projections (16 values per lane)
    if (c->hidden % 128 != 0 || c->hidden > 1024) {
        *why = "hidden must be a multiple of 128 and <= 1024";
        return LAYA_E_UNSUPPORTED;
    }
    if (c->ffn % 64 != 0) {
        *why = "ffn must be a multiple of 64";
        return LAYA_E_UNSUPPORTED;
    }
    if (c->window % 2 != 0) {
        *why = "window must be even";
        return LAYA_E_UNSUPPORTED;
    }
    if (c->max_batch > 16 || c->max_seq > 512 || c->max_markers > 2048) {
        *why = "limits above 16 rows x 512 tokens / 2048 markers";
        return LAYA_E_UNSUPPORTED;
    }
    if ((int64_t)c->vocab * c->hidden >= (1ll << 31)) {
        *why = "embedding too large for 32-bit indexing";
        return LAYA_E_UNSUPPORTED;
    }
    return LAYA_OK;
}

int run_args_check(const laya_config *c, const int32_t *ids, const int32_t *lengths, int32_t B,
                   int32_t S, const int32_t *markers, int32_t R, std::string *why) {
    if (B < 0 || S < 0 || R < 0) {
        *why = "negative B, S or R";
        return LAYA_E_INVALID;
    }
    if (B > c->max_batch) {
        *why = "B exceeds max_batch";
        return LAYA_E_INVALID;
    }
    if (S > c->max_seq) {
        *why = "S exceeds max_seq";
        return LAYA_E_INVALID;
    }
    if (R > c->max_markers) {
        *why = "R exceeds max_markers";
        return LAYA_E_INVALID;
    }
    if (B == 0) {
        if (R != 0) {
            *why = "markers given for an empty batch";
            return LAYA_E_INVALID;
        }
        return LAYA_OK;
    }
    if (!ids || !lengths) {
        *why = "token_ids or lengths is NULL";
        return LAYA_E_INVALID;
    }
    if (S == 0) {
        *why = "S == 0 with B > 0";
        return LAYA_E_INVALID;
    }
    for (int b = 0; b < B; ++b) {
        if (lengths[b] < 1 || lengths[b] > S) {
            *why = "length of row " + std::to_string(b) + " outside [1, S]";
            return LAYA_E_INVALID;
        }
        for (int p = 0; p < lengths[b]; ++p) {
            const int32_t id = ids[(int64_t)b * S + p];
            if (id < 0 || id >= c->vocab) {
                *why = "token id out of range at row " + std::to_string(b) + ", position " +
                       std::to_string(p);
                return LAYA_E_INVALID;
            }
        }
    }
    if (R > 0) {
        if (!markers) {
            *why = "markers is NULL with R > 0";
            return LAYA_E_INVALID;
        }
        for (int r = 0; r < R; ++r) {
            const int32_t row = markers[2 * r], pos = markers[2 * r + 1];
            if (row < 0 || row >= B || pos < 0 || pos >= lengths[row]) {
                *why = "marker " + std::to_string(r) + " outside its row";
                return LAYA_E_INVALID;
            }
        }
    }
    return LAYA_OK;
}

struct GraphEntry {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    int launches = 0;
    uint64_t last_used = 0;  // LRU tick
};

// Offsets (in int32) of the per-run index upload for shape key (B, S, R).
struct MetaLayout {
    int64_t hdr, row_off, blk_g, blk_l, blk_sub, mrk_tok, mrk_pos, pos, vtok, ids, total;
    int nblk_full_max, nblk_sub_max;
    static int64_t up8(int64_t v) { return (v + 7) & ~int64_t(7); }
    MetaLayout(int B, int S, int R) {
        nblk_full_max = B * ((S + laya::kAttnQueries - 1) / laya::kAttnQueries);
        nblk_sub_max = R;
        int64_t o = 0;
        hdr = o;
        o += 8;
        row_off = o;
        o = up8(o + B + 1);
        blk_g = o;
        o += (int64_t)nblk_full_max * 8;
        blk_l = o;
        o += (int64_t)nblk_full_max * 8;
        blk_sub = o;
        o += (int64_t)nblk_sub_max * 8;
        mrk_tok = o;
        o = up8(o + R);
        mrk_pos = o;
        o = up8(o + R);
        pos = o;
        o = up8(o + (int64_t)B * S);
        vtok = o;
        o = up8(o + (int64_t)B * S);
        ids = o;
        o = up8(o + (int64_t)B * S);
        total = o;
    }
};

// header fields
enum { H_T = 0, H_B = 1, H_R = 2, H_NBLK = 3, H_NBLK_L = 4, H_NBLK_SUB = 5 };

}  // namespace

struct laya_encoder {
    laya_config cfg{};
    int device = 0;
    bool poisoned = false;
    std::string err;
    laya_stats stats{};

    // weights
    void *wmem = nullptr;
    size_t wbytes = 0;
    bf16_t *emb = nullptr;
    std::vector<bf16_t *> wqkv, wo, wi, wo2;
    // biases of the head variant's decision layers (null elsewhere)
    std::vector<bf16_t *> bqkv, bo, b1, b2;
    struct TensorView {
        bf16_t *dev;
        int32_t rows, cols;
    };
    std::vector<TensorView> tensors;  // by tensor id
    float *gamma_ones = nullptr;
    bf16_t *cos_g = nullptr, *sin_g = nullptr, *cos_l = nullptr, *sin_l = nullptr;

    // workspace
    void *ws = nullptr;
    size_t ws_bytes = 0;
    int64_t tcap = 0;
    bf16_t *xa = nullptr, *xb = nullptr, *nrm = nullptr, *qkv = nullptr, *att = nullptr,
           *hid = nullptr, *out = nullptr;
    bf16_t *x_sub = nullptr, *n_sub = nullptr, *q_sub = nullptr;
    bf16_t *vt = nullptr;  // transposed V [n_heads*64][ldvt], rows start 64-aligned
    int32_t ldvt = 0;
    float *gemm_partial = nullptr;    // split-K partial tiles
    int32_t *meta_dev = nullptr;
    int32_t *meta_host = nullptr;
    int64_t meta_cap = 0;
    hipEvent_t upload_done = nullptr;
    bool upload_pending = false;
    hipStream_t cap_stream = nullptr;

    // GEMM plan range of each token count (see plan_ranges)
    std::vector<int16_t> plan_id;                 // [T], 1 <= T <= tcap
    std::vector<std::pair<int, int>> plan_range;  // [id] -> (first T, last T)

    std::map<std::tuple<int, int, int, int, int>, GraphEntry> graphs;  // (B, S, R, variant, plan)
    uint64_t graph_tick = 0;

    // per-layer captures
    void *cap_mem = nullptr;
    size_t cap_bytes = 0;
    std::vector<std::string> cap_names;
    std::vector<int32_t> cap_rows;
    std::vector<bf16_t *> cap_ptrs;
    bool have_caps = false;

    // indices currently in meta_dev (for LAYA_RUN_RESIDENT)
    bool have_upload = false;
    int up_B = 0, up_S = 0, up_R = 0, up_T = 0;

    int launches = 0;
};

namespace {

int fail(laya_encoder *e, int code, const std::string &msg) {
    if (e) {
        e->err = msg;
        if (code == LAYA_E_DEVICE) e->poisoned = true;
    }
    g_last_error = msg;
    return code;
}

#define HIPCHK(expr)                                                                      \
    do {                                                                                  \
        hipError_t _e = (expr);                                                           \
        if (_e != hipSuccess)                                                             \
            return fail(enc, LAYA_E_DEVICE,                                               \
                        std::string(#expr) + ": " + hipGetErrorString(_e));               \
    } while (0)

// Everything a recorded schedule needs about the run shape.
struct RunShape {
    int B, S, R;
    int T;  // actual tokens (host value; used only for captures in eager mode)
    bool capture_layers;
    // RoPE: 0 in the QKV projection's epilogue, 1 by its own kernel after the
    // projection, 2 by its own kernel in the original launch geometry
    int rope_variant = 0;
    bool rope_standalone() const { return rope_variant != 0; }
    // host-side algorithmic counts, used only when profiling
    double pairs_global = 0, pairs_local = 0, pairs_subset = 0;
};

// Op classes of the per-launch profile (laya_encoder_profile).
enum OpKind {
    OP_GATHER, OP_LAYERNORM, OP_QKV, OP_ROPE, OP_ATTENTION, OP_OUT_PROJ, OP_UP_GEGLU, OP_DOWN,
    OP_ROW_GATHER, OP_KV, OP_Q, OP_UP_GELU, OP_OUT_PROJ_LN, OP_DOWN_LN, OP_ROPE_ORIGINAL, OP_COUNT
};
const char *const kOpNames[OP_COUNT] = {
    "gather", "layernorm", "qkv_gemm", "rope", "attention", "out_proj_gemm",
    "up_geglu_gemm", "down_gemm", "row_gather", "kv_gemm", "q_gemm", "up_gelu_gemm",
    "out_proj_gemm_layernorm", "down_gemm_layernorm", "rope_original"};

struct ProfRec {
    int op;
    double flops, bytes;
};

struct Profiler {
    std::vector<hipEvent_t> ev;  // two per launch
    std::vector<ProfRec> recs;
    size_t n = 0;
};

int layer_count(const laya_config &c) { return c.n_enc_layers + c.n_dec_layers; }

// GEMM plans of one pass.  Every plan (tile shape and K split) follows the
// live token count T alone, never the padded B*S, so the same rows padded to
// a wider S add in the same order and give bitwise the same states.  The
// marker layer's GEMMs over R rows keep the K split of the matching
// full-pass GEMM (so marker rows are bitwise the full pass's rows) and choose
// their own tile shape.
struct PassPlans {
    laya::GemmPlan qkv, o, up, down;              // over the T packed tokens
    laya::GemmPlan kv_sub, q_sub, o_sub, up_sub, down_sub;  // marker layer
    // head variant: the decision layers' 4H-wide FFN (bias + GELU, then bias)
    laya::GemmPlan up4, down4, up4_sub, down4_sub;
};

laya::GemmPlan subset_plan(const laya::GemmPlan &full, int R, int N, int K, int epi) {
    laya::GemmPlan g;
    g.splits = full.splits;
    if (R <= 64)
        g.config = 7;
    else if (R <= 256 || full.splits > 1)
        g.config = 2;  // split-capable
    else
        g.config = laya::plan_gemm(R, N, K, epi).config;  // R > 256: K is whole anyway
    return g;
}

// Plan segments of the live token count T.  The GEMM planner, evaluated at
// exactly T, is piecewise constant in T; a segment is a maximal run of
// counts whose projections (QKV, output, up, down, and the head's two) all
// get the same tile shape and K split.  A pass over T tokens therefore uses
// the plans for exactly T, one captured graph of a (B, S, R) serves one
// segment, and the plan depends on T alone, never on the padded B*S.  The
// segment ends are computed once per model width, FFN width, head variant
// and token capacity.
std::vector<int> compute_segment_ends(const laya_config &c) {
    const int H = c.hidden, F = c.ffn, tcap = c.max_batch * c.max_seq;
    auto key_at = [&](int T) {
        std::array<int, 12> k{};
        const laya::GemmPlan g[6] = {laya::plan_gemm(T, 3 * H, H, 2), laya::plan_gemm(T, H, H, 0),
                                     laya::plan_gemm(T, F, H, 1), laya::plan_gemm(T, H, F, 0),
                                     c.dec_head ? laya::plan_gemm(T, 4 * H, H, 3) : laya::GemmPlan{},
                                     c.dec_head ? laya::plan_gemm(T, H, 4 * H, 0) : laya::GemmPlan{}};
        for (int i = 0; i < 6; ++i) {
            k[2 * i] = g[i].config;
            k[2 * i + 1] = g[i].splits;
        }
        return k;
    };
    std::vector<int> ends;
    std::array<int, 12> prev = key_at(1);
    for (int T = 2; T <= tcap; ++T) {
        const std::array<int, 12> k = key_at(T);
        if (k != prev) ends.push_back(T - 1);
        prev = k;
    }
    ends.push_back(tcap);
    return ends;
}

const std::vector<int> &plan_segment_ends(const laya_config &c) {
    static std::mutex mu;
    static std::map<std::array<int, 4>, std::vector<int>> cache;
    const std::array<int, 4> key = {c.hidden, c.ffn, c.dec_head, c.max_batch * c.max_seq};
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it == cache.end()) it = cache.emplace(key, compute_segment_ends(c)).first;
    return it->second;
}

std::pair<int, int> plan_segment(const laya_config &c, int T) {
    const std::vector<int> &ends = plan_segment_ends(c);
    const auto it = std::lower_bound(ends.begin(), ends.end(), T);
    const int hi = it == ends.end() ? ends.back() : *it;
    const int lo = it == ends.begin() ? 1 : *(it - 1) + 1;
    return {lo, hi};
}

PassPlans make_plans(const laya_config &c, int T, int R) {
    const int H = c.hidden, F = c.ffn;
    const std::pair<int, int> b = plan_segment(c, T);
    auto plan = [&](int N, int K, int epi) { return laya::plan_gemm(b.second, N, K, epi); };
    PassPlans p{};
    p.qkv = plan(3 * H, H, 2);
    p.o = plan(H, H, 0);
    p.up = plan(F, H, 1);
    p.down = plan(H, F, 0);
    if (c.dec_head) {
        p.up4 = plan(4 * H, H, 3);
        p.down4 = plan(H, 4 * H, 0);
    }
    if (R > 0) {
        p.kv_sub = plan(2 * H, H, 2);
        p.kv_sub.splits = p.qkv.splits;
        if (p.kv_sub.splits > laya::gemm_max_splits(p.kv_sub.config)) p.kv_sub.config = 2;
        p.q_sub = subset_plan(p.qkv, R, H, H, 2);
        p.o_sub = subset_plan(p.o, R, H, H, 0);
        p.up_sub = subset_plan(p.up, R, F, H, 1);
        p.down_sub = subset_plan(p.down, R, H, F, 0);
        if (c.dec_head) {
            p.up4_sub = subset_plan(p.up4, R, 4 * H, H, 3);
            p.down4_sub = subset_plan(p.down4, R, H, 4 * H, 0);
        }
    }
    return p;
}

bool same_plan(const laya::GemmPlan &a, const laya::GemmPlan &b) {
    return a.config == b.config && a.splits == b.splits;
}
// full-pass plans (R = 0) equal: the marker layer's plans follow from them and R
bool same_full_plans(const PassPlans &a, const PassPlans &b) {
    return same_plan(a.qkv, b.qkv) && same_plan(a.o, b.o) && same_plan(a.up, b.up) &&
           same_plan(a.down, b.down) && same_plan(a.up4, b.up4) && same_plan(a.down4, b.down4);
}

// A captured graph serves one plan segment of its (B, S, R); its GEMM grids
// are sized for the segment's largest count (or B*S if smaller).
struct PlanRanges {
    std::vector<int16_t> id;                 // [T] for 1 <= T <= tcap
    std::vector<std::pair<int, int>> range;  // [id] -> (first T, last T)
};

PlanRanges plan_ranges(const laya_config &c) {
    const int tcap = c.max_batch * c.max_seq;
    PlanRanges r;
    r.id.assign((size_t)tcap + 1, 0);
    for (int T = 1; T <= tcap; ++T) {
        const std::pair<int, int> b = plan_segment(c, T);
        if (r.range.empty() || r.range.back() != b) r.range.push_back(b);
        r.id[T] = (int16_t)(r.range.size() - 1);
    }
    return r;
}

// Why a planned launch could not run, or "" (checked for every plan a handle
// can use when its configuration is validated): the fused split reduce +
// LayerNorm holds a row of at most 1024 values and runs on the split-capable
// tile shapes; a split must fit the shape's range limit and K; the paired
// epilogues (GeGLU, QKV) need shapes with paired weight rows.
std::string plan_problem(const laya::GemmPlan &g, int N, int K, int epi, bool fused) {
    if (g.config < 0 || g.config >= laya::kGemmConfigs) return "tile shape out of range";
    if (g.splits < 1 || g.splits > K / 64 || g.splits > laya::gemm_max_splits(g.config))
        return "K split not supported by the tile shape";
    if ((epi == 1 || epi == 2) && g.config == 0) return "paired epilogue on the 32x64 plain tile";
    if (fused && (N > 1024 || N % 64 != 0)) return "fused reduce + LayerNorm wider than 1024";
    if (fused && g.config > 3 && g.config != 7 && g.config != 8)
        return "fused reduce + LayerNorm on a whole-K tile shape";
    return "";
}

std::string plans_problem(const laya_config &c, const PassPlans &p, int R) {
    const int H = c.hidden, F = c.ffn;
    struct Item {
        const laya::GemmPlan *g;
        int N, K, epi;
        bool fused_if_split;
        const char *what;
    };
    std::vector<Item> items = {{&p.qkv, 3 * H, H, 2, false, "QKV"}, {&p.o, H, H, 0, true, "output"},
                               {&p.up, F, H, 1, false, "up"},       {&p.down, H, F, 0, true, "down"}};
    if (c.dec_head) {
        items.push_back({&p.up4, 4 * H, H, 3, false, "head up"});
        items.push_back({&p.down4, H, 4 * H, 0, true, "head down"});
    }
    if (R > 0) {
        items.push_back({&p.kv_sub, 2 * H, H, 2, false, "marker K/V"});
        items.push_back({&p.q_sub, H, H, 2, false, "marker Q"});
        items.push_back({&p.o_sub, H, H, 0, true, "marker output"});
        items.push_back({&p.up_sub, F, H, 1, false, "marker up"});
        items.push_back({&p.down_sub, H, F, 0, true, "marker down"});
        if (c.dec_head) {
            items.push_back({&p.up4_sub, 4 * H, H, 3, false, "marker head up"});
            items.push_back({&p.down4_sub, H, 4 * H, 0, true, "marker head down"});
        }
    }
    for (const Item &it : items) {
        const std::string why =
            plan_problem(*it.g, it.N, it.K, it.epi, it.fused_if_split && it.g->splits > 1);
        if (!why.empty()) return std::string(it.what) + " GEMM: " + why;
    }
    return "";
}

// Largest split-K partial buffer (bytes) over every shape the handle accepts,
// and the first planned launch that could not run ("" if none).
void gemm_scratch_bound(const laya_config &c, const PlanRanges &pr, size_t *bytes,
                        std::string *problem) {
    const int H = c.hidden, F = c.ffn;
    size_t b = 0;
    auto acc = [&](const laya::GemmPlan &g, int M, int N, int epi) {
        b = std::max(b, laya::gemm_workspace_bytes(g, M, N, epi));
    };
    problem->clear();
    for (const auto &rg : pr.range) {
        const int T = rg.second;  // grids are sized for the range's largest count
        const PassPlans p = make_plans(c, T, 0);
        acc(p.qkv, T, 3 * H, 2);
        acc(p.o, T, H, 0);
        acc(p.up, T, F, 1);
        acc(p.down, T, H, 0);
        if (c.dec_head) {
            acc(p.up4, T, 4 * H, 3);
            acc(p.down4, T, H, 0);
        }
        if (problem->empty()) *problem = plans_problem(c, p, 0);
        for (int R = 1; R <= c.max_markers; ++R) {
            const PassPlans q = make_plans(c, T, R);
            acc(q.kv_sub, T, 2 * H, 2);
            acc(q.q_sub, R, H, 2);
            acc(q.o_sub, R, H, 0);
            acc(q.up_sub, R, F, 1);
            acc(q.down_sub, R, H, 0);
            if (c.dec_head) {
                acc(q.up4_sub, R, 4 * H, 3);
                acc(q.down4_sub, R, H, 0);
            }
            if (problem->empty()) *problem = plans_problem(c, q, R);
        }
    }
    *bytes = b;
}

// Queue the whole pass on stream s.  Reads T, the row layout and the
// attention work lists from the device copy of the index upload.
int record(laya_encoder *enc, hipStream_t s, const RunShape &rs, Profiler *prof = nullptr) {
    const laya_config &c = enc->cfg;
    const int H = c.hidden, F = c.ffn, nh = c.n_heads;
    const int NL = layer_count(c);
    const int Tmax = rs.B * rs.S;
    const MetaLayout ml(rs.B, rs.S, rs.R);
    const int32_t *md = enc->meta_dev;
    const int32_t *T_dev = md + ml.hdr + H_T;
    const int32_t *ids = md + ml.ids;
    const int32_t *pos = md + ml.pos;
    const int32_t *vtok = md + ml.vtok;
    const AttnBlock *blk_g = reinterpret_cast<const AttnBlock *>(md + ml.blk_g);
    const AttnBlock *blk_l = reinterpret_cast<const AttnBlock *>(md + ml.blk_l);
    const AttnBlock *blk_s = reinterpret_cast<const AttnBlock *>(md + ml.blk_sub);
    const int32_t *nblk_g = md + ml.hdr + H_NBLK;
    const int32_t *nblk_l = md + ml.hdr + H_NBLK_L;
    const int32_t *nblk_s = md + ml.hdr + H_NBLK_SUB;
    const int32_t *mrk_tok = md + ml.mrk_tok;
    const int32_t *mrk_pos = md + ml.mrk_pos;
    const int hw = c.window / 2;
    // the standalone RoPE launch of the chosen variant
    auto rope = rs.rope_variant == 2 ? laya::launch_rope_original : laya::launch_rope;
    const int rope_op = rs.rope_variant == 2 ? OP_ROPE_ORIGINAL : OP_ROPE;
    // plans follow the live count; GEMM grids cover the largest count of its
    // plan range (kernels read the live count from the device)
    const int T_run = std::max(1, rs.T);
    const PassPlans plans = make_plans(c, T_run, rs.R);
    const int Mg = std::min(Tmax, enc->plan_range[enc->plan_id[T_run]].second);
    float *gp = enc->gemm_partial;
    enc->launches = 0;

    size_t ci = 0;
    auto cap = [&](const char *name, const bf16_t *src, int rows) -> int {
        if (!rs.capture_layers) return LAYA_OK;
        if (ci >= enc->cap_ptrs.size()) return fail(enc, LAYA_E_INVALID, "capture overflow");
        enc->cap_names[ci] = name;
        enc->cap_rows[ci] = rows;
        HIPCHK(hipMemcpyAsync(enc->cap_ptrs[ci], src, (size_t)rows * H * 2,
                              hipMemcpyDeviceToDevice, s));
        ++ci;
        return LAYA_OK;
    };
    // Every launch goes through L_OP: op class, algorithmic FLOPs and HBM
    // bytes (for the profile), and the launch itself.
#define L_OP(op, fl, by, expr)                                                        \
    do {                                                                              \
        if (prof) {                                                                   \
            if (prof->n >= prof->recs.size())                                         \
                return fail(enc, LAYA_E_INVALID, "profile event pool too small");     \
            prof->recs[prof->n] = ProfRec{(op), (fl), (by)};                          \
            HIPCHK(hipEventRecord(prof->ev[2 * prof->n], s));                         \
        }                                                                             \
        hipError_t _e = (expr);                                                       \
        ++enc->launches;                                                              \
        if (_e != hipSuccess)                                                         \
            return fail(enc, LAYA_E_DEVICE, std::string(#expr) + ": " + hipGetErrorString(_e)); \
        if (prof) {                                                                   \
            HIPCHK(hipEventRecord(prof->ev[2 * prof->n + 1], s));                     \
            ++prof->n;                                                                \
        }                                                                             \
    } while (0)
#define C_CHK(expr)                      \
    do {                                 \
        int _r = (expr);                 \
        if (_r != LAYA_OK) return _r;    \
    } while (0)

    const double T = rs.T, R = rs.R, b2 = 2.0;
    auto gemm_fl = [](double M, double N, double K) { return 2.0 * M * N * K; };
    auto gemm_by = [&](double M, double Nw, double N, double K) {
        return b2 * (M * K + Nw * K + M * N);
    };
    const double ln_by = 2 * T * H * b2;
    // a projection onto H whose split reduce also does the residual and the
    // LayerNorm: reads A, W and x, writes x and n (f is never stored)
    auto proj_ln_by = [&](double M, double K) { return b2 * (M * K + H * K + 3 * M * H); };
    const double attn_fl_per_pair = 4.0 * c.head_dim * nh;

    // bytes the attention kernel may read from a K column block of row
    // stride ld (the workspace holds tcap token rows), and from V^T
    auto k_bytes = [&](int ld) {
        return (uint32_t)(((size_t)(enc->tcap - 1) * ld + H) * 2);
    };
    const uint32_t vt_bytes = (uint32_t)((size_t)H * enc->ldvt * 2);

    bf16_t *xr = enc->xa, *xalt = enc->xb;
    L_OP(OP_GATHER, 0, 2 * T * H * b2 + 4 * T,
         laya::launch_gather(s, enc->emb, ids, T_dev, Tmax, H, xr));
    C_CHK(cap("emb", xr, rs.T));
    bool prev = false;      // xr holds the previous layer's output (residual added)
    bool ln_ready = false;  // ... and its down projection's reduce made the next LayerNorm
    char name[32];
    for (int L = 0; L < NL; ++L) {
        const bool is_enc = L < c.n_enc_layers;
        const bool glob = !is_enc || (L % c.global_every) == 0;
        const bf16_t *ctab = glob ? enc->cos_g : enc->cos_l;
        const bf16_t *stab = glob ? enc->sin_g : enc->sin_l;
        const int half = glob ? -1 : hw;
        const AttnBlock *blk = glob ? blk_g : blk_l;
        const int32_t *nblk = glob ? nblk_g : nblk_l;
        const bool subset = (L == NL - 1) && rs.R > 0;
        const bf16_t *Wqkv = enc->wqkv[L], *Wo = enc->wo[L], *Wi = enc->wi[L],
                     *Wo2 = enc->wo2[L];
        const float *g1 = enc->gamma_ones;
        // head variant: biased projections and a 4H-wide GELU FFN (W_i, W_o2
        // then hold W_1 [4H][H] and W_2 [H][4H])
        const bool head = c.dec_head && !is_enc;
        const bf16_t *Bqkv = enc->bqkv[L], *Bo = enc->bo[L], *B1 = enc->b1[L], *B2 = enc->b2[L];
        const int FW = head ? 4 * H : F;  // width of the FFN's inner activation
        // up + activation and down projection (M rows, T_dev or Mmax rows when
        // T_dev is null), with the residual add into x_res.  With a K split
        // the down projection's reduce launch also does the LayerNorm that
        // follows, into n_next (*fused set); with whole K the GEMM's store
        // adds f to x_res and the LayerNorm is left to the caller.
        auto ffn = [&](const bf16_t *n_in, const int32_t *M_dev, int Mmax, double Mf,
                       const laya::GemmPlan &pu, const laya::GemmPlan &pd, bf16_t *x_res,
                       bf16_t *n_next, bool *fused) -> int {
            if (head) {
                L_OP(OP_UP_GELU, gemm_fl(Mf, FW, H), gemm_by(Mf, FW, FW, H) + FW * b2,
                     laya::launch_gemm(s, n_in, H, Wi, H, enc->hid, FW, M_dev, Mmax, FW, H, 3,
                                       pu, gp, nullptr, B1));
            } else {
                L_OP(OP_UP_GEGLU, gemm_fl(Mf, 2 * F, H), gemm_by(Mf, 2 * F, F, H),
                     laya::launch_gemm(s, n_in, H, Wi, H, enc->hid, F, M_dev, Mmax, F, H, 1,
                                       pu, gp));
            }
            const bf16_t *Bd = head ? B2 : nullptr;
            const double bias_by = head ? H * b2 : 0.0;
            *fused = pd.splits > 1;
            if (*fused)
                L_OP(OP_DOWN_LN, gemm_fl(Mf, H, FW), proj_ln_by(Mf, FW) + bias_by,
                     laya::launch_gemm_layernorm(s, enc->hid, FW, Wo2, FW, M_dev, Mmax, H, FW,
                                                 pd, gp, Bd, x_res, n_next, g1, c.ln_eps));
            else
                L_OP(OP_DOWN, gemm_fl(Mf, H, FW), gemm_by(Mf, H, H, FW) + bias_by + Mf * H * b2,
                     laya::launch_gemm(s, enc->hid, FW, Wo2, FW, x_res, H, M_dev, Mmax, H, FW, 0,
                                       pd, gp, nullptr, Bd, x_res));
            return LAYA_OK;
        };
        // output projection followed by x += a, n_out = LN(x)
        auto attn_out = [&](const int32_t *M_dev, int Mmax, double Mf, const laya::GemmPlan &po,
                            bf16_t *x_res, bf16_t *n_out) -> int {
            if (po.splits > 1) {
                L_OP(OP_OUT_PROJ_LN, gemm_fl(Mf, H, H), proj_ln_by(Mf, H) + (Bo ? H * b2 : 0.0),
                     laya::launch_gemm_layernorm(s, enc->att, H, Wo, H, M_dev, Mmax, H, H, po, gp,
                                                 Bo, x_res, n_out, g1, c.ln_eps));
            } else {
                // the GEMM's store adds the projection to x_res; the LayerNorm
                // then reads x_res alone
                L_OP(OP_OUT_PROJ, gemm_fl(Mf, H, H), gemm_by(Mf, H, H, H) + Mf * H * b2,
                     laya::launch_gemm(s, enc->att, H, Wo, H, x_res, H, M_dev, Mmax, H, H, 0, po,
                                       gp, nullptr, Bo, x_res));
                L_OP(OP_LAYERNORM, 0, 2 * Mf * H * b2,
                     laya::launch_layernorm(s, x_res, nullptr, n_out, g1, M_dev, Mmax, H,
                                            c.ln_eps));
            }
            return LAYA_OK;
        };

        // attention sublayer: n = LN(x), unless the previous layer's down
        // projection already produced it
        if (!ln_ready)
            L_OP(OP_LAYERNORM, 0, ln_by,
                 laya::launch_layernorm(s, xr, nullptr, enc->nrm, g1, T_dev, Tmax, H, c.ln_eps));
        if (prev) {
            std::snprintf(name, sizeof name, (L - 1) < c.n_enc_layers ? "enc%02d" : "dec%d",
                          (L - 1) < c.n_enc_layers ? L - 1 : L - 1 - c.n_enc_layers);
            C_CHK(cap(name, xr, rs.T));
        }
        prev = ln_ready = false;
        if (!subset) {
            // Q, K rotated in the epilogue (or by the RoPE kernel after it); V
            // stored transposed for attention
            const int rope_cols = rs.rope_standalone() ? 0 : 2 * H;
            const laya::QkvEpilogue qe{pos, ctab, stab, rope_cols, 2 * H, enc->vt, enc->ldvt, vtok};
            L_OP(OP_QKV, gemm_fl(T, 3 * H, H), gemm_by(T, 3 * H, 3 * H, H),
                 laya::launch_gemm(s, enc->nrm, H, Wqkv, H, enc->qkv, 3 * H, T_dev, Mg, 3 * H,
                                   H, 2, plans.qkv, gp, &qe, Bqkv));
            if (rs.rope_standalone())
                L_OP(rope_op, 0, 2 * T * 2 * H * b2,
                     rope(s, enc->qkv, 3 * H, 2 * nh, T_dev, Tmax, pos, ctab, stab));
            const laya::AttnParams ap{enc->qkv, 3 * H, enc->qkv + H, 3 * H, k_bytes(3 * H),
                                      enc->vt, enc->ldvt, vt_bytes, enc->att, H, blk, nblk,
                                      ml.nblk_full_max, pos, nh, half};
            L_OP(OP_ATTENTION, attn_fl_per_pair * (glob ? rs.pairs_global : rs.pairs_local),
                 4 * T * H * b2, laya::launch_attention(s, ap));
            C_CHK(attn_out(T_dev, Mg, T, plans.o, xr, enc->nrm));
            // the LayerNorm after this layer: the next layer's attention norm,
            // the encoder's final norm, or the closing norm
            bf16_t *n_next = L == NL - 1 ? enc->out
                                         : (L == c.n_enc_layers - 1 ? xalt : enc->nrm);
            bool fused = false;
            C_CHK(ffn(enc->nrm, T_dev, Mg, T, head ? plans.up4 : plans.up,
                      head ? plans.down4 : plans.down, xr, n_next, &fused));
            prev = true;
            ln_ready = fused;
            if (L == c.n_enc_layers - 1) {
                // the encoder's final LayerNorm output becomes the decision stream
                if (!fused)
                    L_OP(OP_LAYERNORM, 0, ln_by,
                         laya::launch_layernorm(s, xr, nullptr, xalt, g1, T_dev, Tmax, H,
                                                c.ln_eps));
                std::snprintf(name, sizeof name, "enc%02d", L);
                C_CHK(cap(name, xr, rs.T));
                C_CHK(cap("enc_final", xalt, rs.T));
                std::swap(xr, xalt);
                prev = ln_ready = false;
            }
        } else {
            // keys/values for every token, queries only for the marker rows
            const int Ri = rs.R;
            const laya::QkvEpilogue qe_kv{pos,      ctab,          stab,
                                          rs.rope_standalone() ? 0 : H, H, enc->vt,
                                          enc->ldvt, vtok};
            L_OP(OP_KV, gemm_fl(T, 2 * H, H), gemm_by(T, 2 * H, 2 * H, H),
                 laya::launch_gemm(s, enc->nrm, H, Wqkv + (size_t)H * H, H, enc->qkv, 2 * H,
                                   T_dev, Mg, 2 * H, H, 2, plans.kv_sub, gp, &qe_kv,
                                   Bqkv ? Bqkv + H : nullptr));
            if (rs.rope_standalone())
                L_OP(rope_op, 0, 2 * T * H * b2,
                     rope(s, enc->qkv, 2 * H, nh, T_dev, Tmax, pos, ctab, stab));
            L_OP(OP_ROW_GATHER, 0, 2 * R * H * b2,
                 laya::launch_gather_rows(s, enc->nrm, H, mrk_tok, Ri, H, enc->n_sub, H));
            L_OP(OP_ROW_GATHER, 0, 2 * R * H * b2,
                 laya::launch_gather_rows(s, xr, H, mrk_tok, Ri, H, enc->x_sub, H));
            const laya::QkvEpilogue qe_q{mrk_pos, ctab, stab, rs.rope_standalone() ? 0 : H, H,
                                         nullptr, 0, nullptr};
            L_OP(OP_Q, gemm_fl(R, H, H), gemm_by(R, H, H, H),
                 laya::launch_gemm(s, enc->n_sub, H, Wqkv, H, enc->q_sub, H, nullptr, Ri, H, H,
                                   2, plans.q_sub, gp, &qe_q, Bqkv));
            if (rs.rope_standalone())
                L_OP(rope_op, 0, 2 * R * H * b2,
                     rope(s, enc->q_sub, H, nh, nullptr, Ri, mrk_pos, ctab, stab));
            const laya::AttnParams ap{enc->q_sub, H, enc->qkv, 2 * H, k_bytes(2 * H),
                                      enc->vt, enc->ldvt, vt_bytes, enc->att, H, blk_s, nblk_s,
                                      ml.nblk_sub_max, mrk_pos, nh, half};
            L_OP(OP_ATTENTION, attn_fl_per_pair * rs.pairs_subset, (2 * R + 2 * T) * H * b2,
                 laya::launch_attention(s, ap));
            C_CHK(attn_out(nullptr, Ri, R, plans.o_sub, enc->x_sub, enc->n_sub));
            bool fused = false;
            C_CHK(ffn(enc->n_sub, nullptr, Ri, R, head ? plans.up4_sub : plans.up_sub,
                      head ? plans.down4_sub : plans.down_sub, enc->x_sub, enc->out, &fused));
            if (!fused)
                L_OP(OP_LAYERNORM, 0, 2 * R * H * b2,
                     laya::launch_layernorm(s, enc->x_sub, nullptr, enc->out, g1, nullptr, Ri, H,
                                            c.ln_eps));
            std::snprintf(name, sizeof name, L < c.n_enc_layers ? "enc%02d" : "dec%d",
                          L < c.n_enc_layers ? L : L - c.n_enc_layers);
            C_CHK(cap(name, enc->x_sub, Ri));
            C_CHK(cap("out", enc->out, Ri));
            return LAYA_OK;
        }
    }
    // closing LayerNorm over the decision stream (already done by a fused down
    // projection)
    if (!ln_ready)
        L_OP(OP_LAYERNORM, 0, ln_by,
             laya::launch_layernorm(s, xr, nullptr, enc->out, enc->gamma_ones, T_dev, Tmax, H,
                                    c.ln_eps));
    if (prev) {
        std::snprintf(name, sizeof name, (NL - 1) < c.n_enc_layers ? "enc%02d" : "dec%d",
                      (NL - 1) < c.n_enc_layers ? NL - 1 : NL - 1 - c.n_enc_layers);
        C_CHK(cap(name, xr, rs.T));
    }
    C_CHK(cap("out", enc->out, rs.T));
    return LAYA_OK;
#undef L_OP
#undef C_CHK
}

int ensure_captures(laya_encoder *enc) {
    const laya_config &c = enc->cfg;
    const size_t n = (size_t)layer_count(c) + 4;
    const size_t per = (size_t)enc->tcap * c.hidden * 2;
    if (enc->cap_mem) return LAYA_OK;
    void *p = nullptr;
    if (hipMalloc(&p, n * per) != hipSuccess)
        return fail(enc, LAYA_E_NOMEM, "capture buffers: hipMalloc failed");
    enc->cap_mem = p;
    enc->cap_bytes = n * per;
    enc->cap_ptrs.resize(n);
    enc->cap_names.assign(n, "");
    enc->cap_rows.assign(n, 0);
    for (size_t i = 0; i < n; ++i)
        enc->cap_ptrs[i] = reinterpret_cast<bf16_t *>(static_cast<char *>(p) + i * per);
    return LAYA_OK;
}

}  // namespace

// ============================================================================
// C ABI
// ============================================================================
extern "C" {

int laya_abi_version(void) { return LAYA_ABI_VERSION; }

void laya_config_init(laya_config *c) {
    if (!c) return;
    c->abi_version = LAYA_ABI_VERSION;
    c->vocab = 50368;
    c->hidden = 1024;
    c->n_heads = 16;
    c->head_dim = 64;
    c->ffn = 2624;
    c->n_enc_layers = 28;
    c->n_dec_layers = 2;
    c->global_every = 3;
    c->window = 128;
    c->theta_global = 160000.0f;
    c->theta_local = 10000.0f;
    c->ln_eps = 1e-5f;
    c->max_batch = 16;
    c->max_seq = 512;
    c->max_markers = 2048;
    c->max_graphs = 4;
    c->workspace_budget_mib = 512;
    c->dec_head = 0;
}

const char *laya_last_error(void) { return g_last_error.c_str(); }

int laya_validate_config(const laya_config *cfg) {
    std::string why;
    int rc = config_check(cfg, &why);
    if (rc == LAYA_OK) {
        size_t bytes = 0;
        gemm_scratch_bound(*cfg, plan_ranges(*cfg), &bytes, &why);
        if (!why.empty()) {
            why = "unsupported plan: " + why;
            rc = LAYA_E_UNSUPPORTED;
        }
    }
    if (rc != LAYA_OK) g_last_error = why;
    return rc;
}

int laya_pass_plans(const laya_config *cfg, int32_t T, int32_t R, int32_t *t_first,
                    int32_t *t_last, laya_gemm_plan *out, int32_t cap, int32_t *n_out) {
    std::string why;
    int rc = config_check(cfg, &why);
    if (rc != LAYA_OK) return set_global_error(rc, why);
    const int tcap = cfg->max_batch * cfg->max_seq;
    if (T < 1 || T > tcap || R < 0 || R > cfg->max_markers || !t_first || !t_last || !n_out ||
        cap < 0 || (cap > 0 && !out))
        return set_global_error(LAYA_E_INVALID, "laya_pass_plans: bad arguments");
    const PassPlans p = make_plans(*cfg, T, R);
    const std::pair<int, int> b = plan_segment(*cfg, T);
    *t_first = b.first;
    *t_last = b.second;
    std::vector<std::pair<const laya::GemmPlan *, int>> list = {
        {&p.qkv, 0}, {&p.o, 1}, {&p.up, 0}, {&p.down, 1}};
    if (cfg->dec_head) {
        list.push_back({&p.up4, 0});
        list.push_back({&p.down4, 1});
    }
    if (R > 0) {
        list.push_back({&p.kv_sub, 0});
        list.push_back({&p.q_sub, 0});
        list.push_back({&p.o_sub, 1});
        list.push_back({&p.up_sub, 0});
        list.push_back({&p.down_sub, 1});
        if (cfg->dec_head) {
            list.push_back({&p.up4_sub, 0});
            list.push_back({&p.down4_sub, 1});
        }
    }
    int n = 0;
    for (const auto &it : list) {
        if (n >= cap) break;
        out[n].config = it.first->config;
        out[n].splits = it.first->splits;
        out[n].fused = it.second && it.first->splits > 1 ? 1 : 0;
        ++n;
    }
    *n_out = (int32_t)list.size();
    return LAYA_OK;
}

int laya_plan_gemm(int32_t M, int32_t N, int32_t K, int32_t epilogue, laya_gemm_plan *out) {
    if (M < 1 || N < 1 || K < 1 || K % 64 != 0 || epilogue < 0 || epilogue > 3 || !out)
        return set_global_error(LAYA_E_INVALID, "laya_plan_gemm: bad arguments");
    const laya::GemmPlan g = laya::plan_gemm(M, N, K, epilogue);
    out->config = g.config;
    out->splits = g.splits;
    out->fused = 0;
    return LAYA_OK;
}

int laya_validate_run_args(const laya_config *cfg, const int32_t *ids, const int32_t *lengths,
                           int32_t B, int32_t S, const int32_t *markers, int32_t R) {
    std::string why;
    int rc = config_check(cfg, &why);
    if (rc == LAYA_OK) rc = run_args_check(cfg, ids, lengths, B, S, markers, R, &why);
    if (rc != LAYA_OK) g_last_error = why;
    return rc;
}

int laya_rope_table(float theta, int32_t max_pos, int32_t head_dim, uint16_t *cos_bits,
                    uint16_t *sin_bits) {
    if (!(theta > 1.f) || max_pos <= 0 || head_dim <= 0 || head_dim % 2 || !cos_bits ||
        !sin_bits)
        return set_global_error(LAYA_E_INVALID, "laya_rope_table: bad arguments");
    build_rope_table((double)theta, max_pos, head_dim, cos_bits, sin_bits);
    return LAYA_OK;
}

int laya_encoder_create(const laya_config *cfg, uint64_t seed, int device, laya_encoder **out) {
    auto t_start = std::chrono::steady_clock::now();
    if (!out) return set_global_error(LAYA_E_INVALID, "out is NULL");
    *out = nullptr;
    std::string why;
    int rc = config_check(cfg, &why);
    if (rc != LAYA_OK) return set_global_error(rc, why);

    laya_encoder *enc = new (std::nothrow) laya_encoder();
    if (!enc) return set_global_error(LAYA_E_NOMEM, "host allocation failed");
    enc->cfg = *cfg;
    enc->device = device;
    auto bail = [&](int code) {
        laya_encoder_destroy(enc);
        return code;
    };
    const laya_config &c = *cfg;
    const int H = c.hidden, F = c.ffn, NL = layer_count(c);

    if (hipSetDevice(device) != hipSuccess)
        return bail(set_global_error(LAYA_E_DEVICE, "hipSetDevice failed"));

    // --- weights: one allocation, 256-byte aligned tensors -----------------
    auto al = [](size_t v) { return (v + 255) & ~size_t(255); };
    std::vector<std::pair<size_t, size_t>> tensors;  // (offset, elements)
    size_t off = 0;
    auto add = [&](size_t elems) {
        tensors.push_back({off, elems});
        off += al(elems * 2);
    };
    // (offset, rows, cols) in tensor-id order
    std::vector<std::array<int64_t, 2>> shapes;
    shapes.push_back({c.vocab, H});
    for (int L = 0; L < NL; ++L) {
        const bool head = c.dec_head && L >= c.n_enc_layers;
        shapes.push_back({3 * H, H});
        shapes.push_back({H, H});
        shapes.push_back({head ? 4 * H : 2 * F, H});
        shapes.push_back({H, head ? 4 * H : F});
    }
    if (c.dec_head)
        for (int d = 0; d < c.n_dec_layers; ++d) {
            shapes.push_back({1, 3 * H});
            shapes.push_back({1, H});
            shapes.push_back({1, 4 * H});
            shapes.push_back({1, H});
        }
    for (auto &sh : shapes) add((size_t)sh[0] * sh[1]);
    const size_t gamma_off = off;
    off += al((size_t)H * 4);
    const size_t tab_off = off;
    const size_t tab_elems = (size_t)c.max_seq * (c.head_dim / 2);
    off += 4 * al(tab_elems * 2);
    enc->wbytes = off;
    if (hipMalloc(&enc->wmem, off) != hipSuccess)
        return bail(set_global_error(LAYA_E_NOMEM, "weights: hipMalloc failed"));
    char *wb = static_cast<char *>(enc->wmem);
    for (size_t t = 0; t < tensors.size(); ++t)
        enc->tensors.push_back({reinterpret_cast<bf16_t *>(wb + tensors[t].first),
                                (int32_t)shapes[t][0], (int32_t)shapes[t][1]});
    enc->emb = enc->tensors[0].dev;
    for (int L = 0; L < NL; ++L) {
        enc->wqkv.push_back(enc->tensors[1 + 4 * L].dev);
        enc->wo.push_back(enc->tensors[2 + 4 * L].dev);
        enc->wi.push_back(enc->tensors[3 + 4 * L].dev);
        enc->wo2.push_back(enc->tensors[4 + 4 * L].dev);
        const bool head = c.dec_head && L >= c.n_enc_layers;
        const int bt = 1 + 4 * NL + 4 * (L - c.n_enc_layers);
        enc->bqkv.push_back(head ? enc->tensors[bt + 0].dev : nullptr);
        enc->bo.push_back(head ? enc->tensors[bt + 1].dev : nullptr);
        enc->b1.push_back(head ? enc->tensors[bt + 2].dev : nullptr);
        enc->b2.push_back(head ? enc->tensors[bt + 3].dev : nullptr);
    }
    enc->gamma_ones = reinterpret_cast<float *>(wb + gamma_off);
    enc->cos_g = reinterpret_cast<bf16_t *>(wb + tab_off);
    enc->sin_g = reinterpret_cast<bf16_t *>(wb + tab_off + al(tab_elems * 2));
    enc->cos_l = reinterpret_cast<bf16_t *>(wb + tab_off + 2 * al(tab_elems * 2));
    enc->sin_l = reinterpret_cast<bf16_t *>(wb + tab_off + 3 * al(tab_elems * 2));

    hipStream_t s = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess)
        return bail(set_global_error(LAYA_E_DEVICE, "hipStreamCreate failed"));
    enc->cap_stream = s;
    for (size_t t = 0; t < tensors.size(); ++t) {
        if (laya::launch_init_weights(s, reinterpret_cast<bf16_t *>(wb + tensors[t].first),
                                      tensors[t].second, seed, (uint32_t)t) != hipSuccess)
            return bail(set_global_error(LAYA_E_DEVICE, "weight init launch failed"));
    }
    if (laya::launch_fill_f32(s, enc->gamma_ones, H, 1.0f) != hipSuccess)
        return bail(set_global_error(LAYA_E_DEVICE, "gamma fill failed"));
    {
        std::vector<uint16_t> tc(tab_elems), ts(tab_elems);
        build_rope_table(c.theta_global, c.max_seq, c.head_dim, tc.data(), ts.data());
        if (hipMemcpyAsync(enc->cos_g, tc.data(), tab_elems * 2, hipMemcpyHostToDevice, s) ||
            hipMemcpyAsync(enc->sin_g, ts.data(), tab_elems * 2, hipMemcpyHostToDevice, s) ||
            hipStreamSynchronize(s))
            return bail(set_global_error(LAYA_E_DEVICE, "rope table upload failed"));
        build_rope_table(c.theta_local, c.max_seq, c.head_dim, tc.data(), ts.data());
        if (hipMemcpyAsync(enc->cos_l, tc.data(), tab_elems * 2, hipMemcpyHostToDevice, s) ||
            hipMemcpyAsync(enc->sin_l, ts.data(), tab_elems * 2, hipMemcpyHostToDevice, s) ||
            hipStreamSynchronize(s))
            return bail(set_global_error(LAYA_E_DEVICE, "rope table upload failed"));
    }

    // --- workspace for max_batch x max_seq tokens ---------------------------
    const int64_t tcap = (int64_t)c.max_batch * c.max_seq;
    const int64_t rcap = std::max(1, c.max_markers);
    enc->tcap = tcap;
    // every row's V^T columns start at a multiple of 64
    const int32_t ldvt = (int32_t)(tcap + 64LL * c.max_batch);
    enc->ldvt = ldvt;
    size_t wsz = 0;
    std::vector<std::pair<bf16_t **, size_t>> bufs = {
        {&enc->xa, (size_t)tcap * H},      {&enc->xb, (size_t)tcap * H},
        {&enc->nrm, (size_t)tcap * H},     {&enc->qkv, (size_t)tcap * 3 * H},
        {&enc->att, (size_t)tcap * H},
        {&enc->hid, (size_t)tcap * (c.dec_head ? std::max(F, 4 * H) : F)},
        {&enc->out, (size_t)tcap * H},
        {&enc->x_sub, (size_t)rcap * H},   {&enc->n_sub, (size_t)rcap * H},
        {&enc->q_sub, (size_t)rcap * H},   {&enc->vt, (size_t)H * ldvt}};
    for (auto &b : bufs) wsz += al(b.second * 2);
    const MetaLayout mlmax(c.max_batch, c.max_seq, c.max_markers);
    enc->meta_cap = mlmax.total;
    const size_t meta_off = wsz;
    wsz += al((size_t)enc->meta_cap * 4);
    size_t gp_bytes = 0;
    {
        const PlanRanges pr = plan_ranges(c);
        enc->plan_id = pr.id;
        enc->plan_range = pr.range;
        std::string problem;
        gemm_scratch_bound(c, pr, &gp_bytes, &problem);
        if (!problem.empty())
            return bail(set_global_error(LAYA_E_UNSUPPORTED, "unsupported plan: " + problem));
    }
    const size_t gp_off = wsz;
    wsz += al(gp_bytes);
    enc->ws_bytes = wsz;
    if (wsz > (size_t)c.workspace_budget_mib << 20)
        return bail(set_global_error(LAYA_E_NOMEM, "workspace of " + std::to_string(wsz >> 20) +
                                                       " MiB exceeds workspace_budget_mib"));
    if (hipMalloc(&enc->ws, wsz) != hipSuccess)
        return bail(set_global_error(LAYA_E_NOMEM, "workspace: hipMalloc failed"));
    if (hipMemsetAsync(enc->ws, 0, wsz, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess)
        return bail(set_global_error(LAYA_E_DEVICE, "workspace clear failed"));
    {
        char *p = static_cast<char *>(enc->ws);
        size_t o = 0;
        for (auto &b : bufs) {
            *b.first = reinterpret_cast<bf16_t *>(p + o);
            o += al(b.second * 2);
        }
        enc->meta_dev = reinterpret_cast<int32_t *>(p + meta_off);
        enc->gemm_partial = gp_bytes ? reinterpret_cast<float *>(p + gp_off) : nullptr;
    }
    if (hipHostMalloc((void **)&enc->meta_host, (size_t)enc->meta_cap * 4, hipHostMallocDefault) !=
        hipSuccess)
        return bail(set_global_error(LAYA_E_NOMEM, "pinned staging: hipHostMalloc failed"));
    if (hipEventCreateWithFlags(&enc->upload_done, hipEventDisableTiming) != hipSuccess)
        return bail(set_global_error(LAYA_E_DEVICE, "hipEventCreate failed"));
    if (hipStreamSynchronize(s) != hipSuccess)
        return bail(set_global_error(LAYA_E_DEVICE, "weight generation failed"));

    enc->stats.weight_bytes = (int64_t)enc->wbytes;
    enc->stats.workspace_bytes = (int64_t)enc->ws_bytes;
    enc->stats.create_ms =
        std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t_start)
            .count();
    *out = enc;
    return LAYA_OK;
}

int laya_encoder_destroy(laya_encoder *enc) {
    if (!enc) return LAYA_OK;
    hipSetDevice(enc->device);
    if (enc->cap_stream) hipStreamSynchronize(enc->cap_stream);
    hipDeviceSynchronize();
    for (auto &kv : enc->graphs) {
        if (kv.second.exec) hipGraphExecDestroy(kv.second.exec);
        if (kv.second.graph) hipGraphDestroy(kv.second.graph);
    }
    if (enc->upload_done) hipEventDestroy(enc->upload_done);
    if (enc->meta_host) hipHostFree(enc->meta_host);
    if (enc->cap_mem) hipFree(enc->cap_mem);
    if (enc->ws) hipFree(enc->ws);
    if (enc->wmem) hipFree(enc->wmem);
    if (enc->cap_stream) hipStreamDestroy(enc->cap_stream);
    delete enc;
    return LAYA_OK;
}

const char *laya_encoder_last_error(const laya_encoder *enc) {
    return enc ? enc->err.c_str() : g_last_error.c_str();
}

int laya_encoder_run(laya_encoder *enc, void *stream, const int32_t *ids,
                     const int32_t *lengths, int32_t B, int32_t S, const int32_t *markers,
                     int32_t R, uint32_t flags, laya_output *out) {
    if (!enc) return set_global_error(LAYA_E_INVALID, "handle is NULL");
    if (enc->poisoned) return fail(enc, LAYA_E_POISONED, "handle poisoned by an earlier device failure");
    if (!out) return fail(enc, LAYA_E_INVALID, "out is NULL");
    if (flags & ~(LAYA_RUN_EAGER | LAYA_RUN_CAPTURE_LAYERS | LAYA_RUN_RESIDENT |
                  LAYA_RUN_ROPE_STANDALONE | LAYA_RUN_ROPE_ORIGINAL))
        return fail(enc, LAYA_E_INVALID, "unknown run flags");
    if ((flags & LAYA_RUN_ROPE_STANDALONE) && (flags & LAYA_RUN_ROPE_ORIGINAL))
        return fail(enc, LAYA_E_INVALID, "two RoPE variants requested");
    const bool resident = (flags & LAYA_RUN_RESIDENT) != 0;
    std::string why;
    int rc = LAYA_OK;
    if (resident) {
        if (!enc->have_upload || B != enc->up_B || S != enc->up_S || R != enc->up_R)
            return fail(enc, LAYA_E_INVALID,
                        "LAYA_RUN_RESIDENT: no previous upload with this (B, S, R)");
    } else {
        rc = run_args_check(&enc->cfg, ids, lengths, B, S, markers, R, &why);
        if (rc != LAYA_OK) return fail(enc, rc, why);
    }
    out->hidden = nullptr;
    out->rows = 0;
    out->dim = enc->cfg.hidden;
    out->row_off = nullptr;
    enc->have_caps = false;
    if (B == 0) return LAYA_OK;

    hipStream_t s = static_cast<hipStream_t>(stream);
    HIPCHK(hipSetDevice(enc->device));
    const MetaLayout ml(B, S, R);
    const laya_config &c = enc->cfg;
    int T = enc->up_T;
    if (!resident) {

    // --- pack into pinned staging (wait for the previous upload to drain) ---
    if (enc->upload_pending) {
        HIPCHK(hipEventSynchronize(enc->upload_done));
        enc->upload_pending = false;
    }
    int32_t *mh = enc->meta_host;
    T = 0;
    mh[ml.row_off] = 0;
    std::vector<int32_t> vcol0(B);
    int32_t vcol = 0;
    for (int b = 0; b < B; ++b) {
        vcol0[b] = vcol;
        for (int p = 0; p < lengths[b]; ++p) {
            mh[ml.ids + T] = ids[(int64_t)b * S + p];
            mh[ml.pos + T] = p;
            mh[ml.vtok + T] = vcol + p;
            ++T;
        }
        mh[ml.row_off + b + 1] = T;
        vcol += (lengths[b] + 63) / 64 * 64;
    }
    int nbg = 0, nbl = 0, nbs = 0;
    build_blocks_full(mh + ml.row_off, vcol0.data(), B, -1,
                      reinterpret_cast<AttnBlock *>(mh + ml.blk_g), &nbg);
    build_blocks_full(mh + ml.row_off, vcol0.data(), B, c.window / 2,
                      reinterpret_cast<AttnBlock *>(mh + ml.blk_l), &nbl);
    if (R > 0) {
        std::vector<int32_t> qrow(R);
        for (int r = 0; r < R; ++r) {
            qrow[r] = markers[2 * r];
            mh[ml.mrk_pos + r] = markers[2 * r + 1];
            mh[ml.mrk_tok + r] = mh[ml.row_off + markers[2 * r]] + markers[2 * r + 1];
        }
        // the marker pass's attention runs on the last layer, which is global
        // unless the model has no decision layers and its last encoder layer is local
        const int Llast = layer_count(c) - 1;
        const bool glob = Llast >= c.n_enc_layers || (Llast % c.global_every) == 0;
        build_blocks_list(mh + ml.row_off, vcol0.data(), qrow.data(), mh + ml.mrk_pos, R,
                          glob ? -1 : c.window / 2,
                          reinterpret_cast<AttnBlock *>(mh + ml.blk_sub), &nbs);
    }
    mh[ml.hdr + H_T] = T;
    mh[ml.hdr + H_B] = B;
    mh[ml.hdr + H_R] = R;
    mh[ml.hdr + H_NBLK] = nbg;
    mh[ml.hdr + H_NBLK_L] = nbl;
    mh[ml.hdr + H_NBLK_SUB] = nbs;
    const int64_t span = ml.ids + T;
    HIPCHK(hipMemcpyAsync(enc->meta_dev, mh, (size_t)span * 4, hipMemcpyHostToDevice, s));
    HIPCHK(hipEventRecord(enc->upload_done, s));
    enc->upload_pending = true;
    enc->have_upload = true;
    enc->up_B = B;
    enc->up_S = S;
    enc->up_R = R;
    enc->up_T = T;
    }  // !resident

    const bool capture = (flags & LAYA_RUN_CAPTURE_LAYERS) != 0;
    const bool eager = capture || (flags & LAYA_RUN_EAGER) != 0;
    const int rope_var = (flags & LAYA_RUN_ROPE_ORIGINAL) ? 2 : (flags & LAYA_RUN_ROPE_STANDALONE) ? 1 : 0;
    RunShape rs{B, S, R, T, capture};
    rs.rope_variant = rope_var;
    if (capture) {
        int r2 = ensure_captures(enc);
        if (r2 != LAYA_OK) return r2;
    }

    if (eager) {
        int r2 = record(enc, s, rs);
        if (r2 != LAYA_OK) return r2;
        enc->stats.launches_last_run = enc->launches;
        enc->have_caps = capture;
    } else {
        auto key = std::make_tuple((int)B, (int)S, (int)R, rope_var,
                                   (int)enc->plan_id[std::max(1, T)]);
        auto it = enc->graphs.find(key);
        if (it == enc->graphs.end()) {
            // LRU: make room for the new shape (every graph shares the one
            // workspace, so the cache bounds graph objects, not memory)
            while ((int)enc->graphs.size() >= c.max_graphs) {
                auto lru = enc->graphs.begin();
                for (auto g = enc->graphs.begin(); g != enc->graphs.end(); ++g)
                    if (g->second.last_used < lru->second.last_used) lru = g;
                HIPCHK(hipStreamSynchronize(s));  // a replay of it may still be queued
                if (lru->second.exec) hipGraphExecDestroy(lru->second.exec);
                if (lru->second.graph) hipGraphDestroy(lru->second.graph);
                enc->graphs.erase(lru);
                ++enc->stats.graph_evictions;
            }
            auto t0 = std::chrono::steady_clock::now();
            RunShape warm{B, S, R, T, false};
            warm.rope_variant = rope_var;
            for (int w = 0; w < 2; ++w) {
                int r2 = record(enc, s, warm);
                if (r2 != LAYA_OK) return r2;
            }
            HIPCHK(hipStreamSynchronize(s));
            GraphEntry ge;
            HIPCHK(hipStreamBeginCapture(enc->cap_stream, hipStreamCaptureModeThreadLocal));
            int r2 = record(enc, enc->cap_stream, warm);
            hipGraph_t g = nullptr;
            hipError_t ec = hipStreamEndCapture(enc->cap_stream, &g);
            if (r2 != LAYA_OK) {
                if (g) hipGraphDestroy(g);
                return r2;
            }
            if (ec != hipSuccess)
                return fail(enc, LAYA_E_DEVICE, std::string("hipStreamEndCapture: ") + hipGetErrorString(ec));
            ge.graph = g;
            ge.launches = enc->launches;
            hipError_t ei = hipGraphInstantiate(&ge.exec, g, nullptr, nullptr, 0);
            if (ei != hipSuccess) {
                hipGraphDestroy(g);
                return fail(enc, LAYA_E_DEVICE, std::string("hipGraphInstantiate: ") + hipGetErrorString(ei));
            }
            it = enc->graphs.emplace(key, ge).first;
            enc->stats.last_capture_ms =
                std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0)
                    .count();
            enc->stats.graphs_cached = (int32_t)enc->graphs.size();
        }
        it->second.last_used = ++enc->graph_tick;
        enc->stats.graphs_cached = (int32_t)enc->graphs.size();
        HIPCHK(hipGraphLaunch(it->second.exec, s));
        enc->stats.launches_last_run = it->second.launches;
    }

    out->hidden = enc->out;
    out->rows = R > 0 ? R : T;
    out->dim = c.hidden;
    out->row_off = R > 0 ? nullptr : enc->meta_dev + ml.row_off;
    return LAYA_OK;
}

int laya_encoder_layer_output(laya_encoder *enc, int32_t index, laya_output *out, char *name,
                              size_t cap) {
    if (!enc || !out) return set_global_error(LAYA_E_INVALID, "NULL argument");
    if (!enc->have_caps) return fail(enc, LAYA_E_INVALID, "last run did not capture layers");
    if (index < 0 || (size_t)index >= enc->cap_ptrs.size() || enc->cap_names[index].empty())
        return fail(enc, LAYA_E_INVALID, "layer index out of range");
    out->hidden = enc->cap_ptrs[index];
    out->rows = enc->cap_rows[index];
    out->dim = enc->cfg.hidden;
    out->row_off = nullptr;
    if (name && cap) {
        std::strncpy(name, enc->cap_names[index].c_str(), cap - 1);
        name[cap - 1] = 0;
    }
    return LAYA_OK;
}

int laya_encoder_weight(laya_encoder *enc, int32_t tid, const void **dev, int32_t *rows,
                        int32_t *cols) {
    if (!enc || !dev || !rows || !cols) return set_global_error(LAYA_E_INVALID, "NULL argument");
    if (tid < 0 || tid >= (int32_t)enc->tensors.size())
        return fail(enc, LAYA_E_INVALID, "tensor id out of range");
    *dev = enc->tensors[tid].dev;
    *rows = enc->tensors[tid].rows;
    *cols = enc->tensors[tid].cols;
    return LAYA_OK;
}

int laya_encoder_weight_digest(laya_encoder *enc, int32_t tid, uint64_t *fnv) {
    if (!enc || !fnv) return set_global_error(LAYA_E_INVALID, "NULL argument");
    if (enc->poisoned) return fail(enc, LAYA_E_POISONED, "handle poisoned");
    const void *dev;
    int32_t rows, cols;
    int rc = laya_encoder_weight(enc, tid, &dev, &rows, &cols);
    if (rc != LAYA_OK) return rc;
    std::vector<uint8_t> hbuf((size_t)rows * cols * 2);
    HIPCHK(hipSetDevice(enc->device));
    HIPCHK(hipMemcpy(hbuf.data(), dev, hbuf.size(), hipMemcpyDeviceToHost));
    uint64_t h = 14695981039346656037ull;
    for (uint8_t byte : hbuf) {
        h ^= byte;
        h *= 1099511628211ull;
    }
    *fnv = h;
    return LAYA_OK;
}

int laya_encoder_stats(const laya_encoder *enc, laya_stats *st) {
    if (!enc || !st) return set_global_error(LAYA_E_INVALID, "NULL argument");
    *st = enc->stats;
    return LAYA_OK;
}

int laya_encoder_fill_workspace(laya_encoder *enc, void *stream, uint8_t byte) {
    if (!enc) return set_global_error(LAYA_E_INVALID, "handle is NULL");
    if (enc->poisoned) return fail(enc, LAYA_E_POISONED, "handle poisoned by an earlier device failure");
    hipStream_t s = static_cast<hipStream_t>(stream);
    HIPCHK(hipSetDevice(enc->device));
    if (enc->upload_pending) {
        HIPCHK(hipEventSynchronize(enc->upload_done));
        enc->upload_pending = false;
    }
    HIPCHK(hipMemsetAsync(enc->ws, byte, enc->ws_bytes, s));
    HIPCHK(hipStreamSynchronize(s));
    enc->have_upload = false;  // the index upload is gone with the rest
    return LAYA_OK;
}

int laya_encoder_config(const laya_encoder *enc, laya_config *out) {
    if (!enc || !out) return set_global_error(LAYA_E_INVALID, "NULL argument");
    *out = enc->cfg;
    return LAYA_OK;
}

int laya_encoder_health(const laya_encoder *enc) {
    if (!enc) return set_global_error(LAYA_E_INVALID, "handle is NULL");
    return enc->poisoned ? LAYA_E_POISONED : LAYA_OK;
}

int laya_encoder_inject_failure(laya_encoder *enc) {
    if (!enc) return set_global_error(LAYA_E_INVALID, "handle is NULL");
    enc->poisoned = true;
    enc->err = "injected failure";
    return LAYA_OK;
}

int laya_memcpy(void *dst, const void *src, size_t bytes, int32_t kind, void *stream) {
    if (bytes == 0) return LAYA_OK;
    if (!dst || !src || kind < 0 || kind > 2)
        return set_global_error(LAYA_E_INVALID, "laya_memcpy: bad arguments");
    const hipMemcpyKind k = kind == 0 ? hipMemcpyDeviceToHost
                            : kind == 1 ? hipMemcpyHostToDevice
                                        : hipMemcpyDeviceToDevice;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(dst, src, bytes, k, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess)
        return set_global_error(LAYA_E_DEVICE, std::string("laya_memcpy: ") + hipGetErrorString(e));
    return LAYA_OK;
}

int laya_encoder_profile(laya_encoder *enc, void *stream, const int32_t *ids,
                         const int32_t *lengths, int32_t B, int32_t S, const int32_t *markers,
                         int32_t R, uint32_t flags, laya_op_time *out, int32_t cap,
                         int32_t *n_out, double *total_ms) {
    if (!enc || !out || !n_out || cap < 0) return set_global_error(LAYA_E_INVALID, "NULL argument");
    if (enc->poisoned) return fail(enc, LAYA_E_POISONED, "handle poisoned");
    if (flags & ~(LAYA_RUN_ROPE_STANDALONE | LAYA_RUN_ROPE_ORIGINAL))
        return fail(enc, LAYA_E_INVALID, "laya_encoder_profile: only RoPE variant flags");
    laya_output o;
    // upload the indices (and validate) with an ordinary eager run first
    int rc = laya_encoder_run(enc, stream, ids, lengths, B, S, markers, R,
                              LAYA_RUN_EAGER | flags, &o);
    if (rc != LAYA_OK) return rc;
    *n_out = 0;
    if (total_ms) *total_ms = 0;
    if (B == 0) return LAYA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const laya_config &c = enc->cfg;
    RunShape rs{B, S, R, enc->up_T, false};
    rs.rope_variant = (flags & LAYA_RUN_ROPE_ORIGINAL) ? 2 : (flags & LAYA_RUN_ROPE_STANDALONE) ? 1 : 0;
    const int hw = c.window / 2;
    for (int b = 0; b < B; ++b) {
        const double len = lengths[b];
        rs.pairs_global += len * len;
        for (int i = 0; i < lengths[b]; ++i)
            rs.pairs_local += std::min(lengths[b] - 1, i + hw) - std::max(0, i - hw) + 1;
    }
    for (int r = 0; r < R; ++r) rs.pairs_subset += lengths[markers[2 * r]];
    Profiler prof;
    const size_t n_launch = (size_t)layer_count(c) * 16 + 16;
    prof.recs.resize(n_launch);
    prof.ev.assign(2 * n_launch, nullptr);
    int result = LAYA_OK;
    for (auto &e : prof.ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            result = fail(enc, LAYA_E_DEVICE, "hipEventCreate failed");
            break;
        }
    }
    if (result == LAYA_OK) result = record(enc, s, rs, &prof);
    if (result == LAYA_OK && hipStreamSynchronize(s) != hipSuccess)
        result = fail(enc, LAYA_E_DEVICE, "hipStreamSynchronize failed");
    if (result == LAYA_OK) {
        std::vector<laya_op_time> agg(OP_COUNT);
        for (int k = 0; k < OP_COUNT; ++k) {
            std::memset(&agg[k], 0, sizeof(laya_op_time));
            std::strncpy(agg[k].name, kOpNames[k], sizeof(agg[k].name) - 1);
        }
        double tot = 0;
        for (size_t i = 0; i < prof.n; ++i) {
            float ms = 0;
            if (hipEventElapsedTime(&ms, prof.ev[2 * i], prof.ev[2 * i + 1]) != hipSuccess) {
                result = fail(enc, LAYA_E_DEVICE, "hipEventElapsedTime failed");
                break;
            }
            laya_op_time &a = agg[prof.recs[i].op];
            a.calls += 1;
            a.total_ms += ms;
            a.flops += prof.recs[i].flops;
            a.bytes += prof.recs[i].bytes;
            tot += ms;
        }
        if (prof.n >= 2 && total_ms) {
            float span = 0;
            if (hipEventElapsedTime(&span, prof.ev[0], prof.ev[2 * prof.n - 1]) == hipSuccess)
                *total_ms = span;
        }
        int n = 0;
        for (int k = 0; k < OP_COUNT && result == LAYA_OK; ++k)
            if (agg[k].calls > 0 && n < cap) out[n++] = agg[k];
        *n_out = n;
    }
    for (auto &e : prof.ev)
        if (e) hipEventDestroy(e);
    return result;
}

// ---------------------------------------------------------------------------
// single-step entry points
// ---------------------------------------------------------------------------
#define OPCHK(expr)                                                                       \
    do {                                                                                  \
        hipError_t _e = (expr);                                                           \
        if (_e != hipSuccess)                                                             \
            return set_global_error(LAYA_E_DEVICE, std::string(#expr) + ": " +            \
                                                       hipGetErrorString(_e));            \
    } while (0)

int laya_op_gather(void *stream, const void *emb, int32_t vocab, int32_t hidden,
                   const int32_t *ids, int32_t T, void *out) {
    if (T < 0 || vocab <= 0 || hidden <= 0 || hidden % 8 || (T > 0 && (!emb || !ids || !out)))
        return set_global_error(LAYA_E_INVALID, "laya_op_gather: bad arguments");
    OPCHK(laya::launch_gather(static_cast<hipStream_t>(stream), static_cast<const bf16_t *>(emb),
                              ids, nullptr, T, hidden, static_cast<bf16_t *>(out)));
    return LAYA_OK;
}

int laya_op_layernorm(void *stream, void *x, const void *r, void *n, const float *gamma,
                      int32_t T, int32_t hidden, float eps) {
    if (T < 0 || hidden <= 0 || hidden % 8 || hidden > 2048 || !(eps > 0.f) ||
        (T > 0 && (!x || !n || !gamma)) || n == x || (r && n == r))
        return set_global_error(LAYA_E_INVALID, "laya_op_layernorm: bad arguments");
    OPCHK(laya::launch_layernorm(static_cast<hipStream_t>(stream), static_cast<bf16_t *>(x),
                                 static_cast<const bf16_t *>(r), static_cast<bf16_t *>(n), gamma,
                                 nullptr, T, hidden, eps));
    return LAYA_OK;
}

namespace {
// One GEMM launch on caller buffers; split-K scratch is allocated for the
// call and freed after it completes.
int op_gemm_launch(const char *who, hipStream_t s, const void *A, int32_t lda, const void *W,
                   int32_t ldw, void *C, int32_t ldc, int32_t M, int32_t N, int32_t K,
                   int32_t epilogue, int32_t config, int32_t splits,
                   const laya::QkvEpilogue *qe, const void *bias) {
    laya::GemmPlan plan = laya::plan_gemm(M, N, K, epilogue);
    if (config >= 0) plan = laya::GemmPlan{config, splits < 1 ? 1 : splits};
    if (plan.splits > K / 64 || plan.splits > laya::gemm_max_splits(plan.config) ||
        ((epilogue == 1 || epilogue == 2) && plan.config == 0))
        return set_global_error(LAYA_E_INVALID, std::string(who) + ": unsupported config/splits");
    const size_t pb = laya::gemm_workspace_bytes(plan, M, N, epilogue);
    void *scratch = nullptr;
    if (pb && hipMalloc(&scratch, pb) != hipSuccess)
        return set_global_error(LAYA_E_NOMEM, std::string(who) + ": scratch hipMalloc failed");
    hipError_t e = laya::launch_gemm(s, static_cast<const bf16_t *>(A), lda,
                                     static_cast<const bf16_t *>(W), ldw,
                                     static_cast<bf16_t *>(C), ldc, nullptr, M, N, K, epilogue,
                                     plan, static_cast<float *>(scratch), qe,
                                     static_cast<const bf16_t *>(bias));
    if (pb) {
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        hipFree(scratch);
    }
    if (e != hipSuccess)
        return set_global_error(LAYA_E_DEVICE, std::string(who) + ": " + hipGetErrorString(e));
    return LAYA_OK;
}

bool gemm_args_ok(const void *A, int32_t lda, const void *W, int32_t ldw, const void *C,
                  int32_t ldc, int32_t M, int32_t N, int32_t K, int32_t config) {
    return !(M < 0 || N <= 0 || K <= 0 || K % 64 || N % 64 || lda % 8 || ldw % 8 || ldc % 8 ||
             lda < K || ldw < K || ldc < N || (M > 0 && (!A || !W || !C)) || config < -1 ||
             config >= laya::kGemmConfigs);
}
}  // namespace

int laya_op_gemm(void *stream, const void *A, int32_t lda, const void *W, int32_t ldw, void *C,
                 int32_t ldc, int32_t M, int32_t N, int32_t K, int32_t epilogue, int32_t config,
                 int32_t splits, const void *bias) {
    if (!gemm_args_ok(A, lda, W, ldw, C, ldc, M, N, K, config) ||
        (epilogue != 0 && epilogue != 1 && epilogue != 3) || (epilogue == 1 && bias) ||
        (epilogue == 3 && M > 0 && !bias))
        return set_global_error(LAYA_E_INVALID, "laya_op_gemm: bad arguments");
    if (M == 0) return LAYA_OK;
    return op_gemm_launch("laya_op_gemm", static_cast<hipStream_t>(stream), A, lda, W, ldw, C,
                          ldc, M, N, K, epilogue, config, splits, nullptr, bias);
}

int laya_op_gemm_noalloc(void *stream, const void *A, int32_t lda, const void *W, int32_t ldw,
                         void *C, int32_t ldc, int32_t M, int32_t N, int32_t K, int32_t epilogue,
                         int32_t config, int32_t splits, const void *bias) {
    if (!gemm_args_ok(A, lda, W, ldw, C, ldc, M, N, K, config) ||
        (epilogue != 0 && epilogue != 1 && epilogue != 3) || (epilogue == 1 && bias) ||
        (epilogue == 3 && M > 0 && !bias))
        return set_global_error(LAYA_E_INVALID, "laya_op_gemm_noalloc: bad arguments");
    if (M == 0) return LAYA_OK;
    laya::GemmPlan plan = laya::plan_gemm(M, N, K, epilogue);
    if (config >= 0) plan = laya::GemmPlan{config, splits < 1 ? 1 : splits};
    if (plan.splits > K / 64 || plan.splits > laya::gemm_max_splits(plan.config) ||
        ((epilogue == 1 || epilogue == 2) && plan.config == 0))
        return set_global_error(LAYA_E_INVALID, "laya_op_gemm_noalloc: unsupported config/splits");
    const size_t pb = laya::gemm_workspace_bytes(plan, M, N, epilogue);
    if (pb > laya::gemm_static_scratch_bytes())
        return set_global_error(
            LAYA_E_INVALID, "laya_op_gemm_noalloc: the K split needs " + std::to_string(pb) +
                                " bytes of scratch, more than the library's " +
                                std::to_string(laya::gemm_static_scratch_bytes()));
    float *scratch = nullptr;
    if (pb) OPCHK(laya::gemm_static_scratch(&scratch));
    OPCHK(laya::launch_gemm(static_cast<hipStream_t>(stream), static_cast<const bf16_t *>(A), lda,
                            static_cast<const bf16_t *>(W), ldw, static_cast<bf16_t *>(C), ldc,
                            nullptr, M, N, K, epilogue, plan, scratch, nullptr,
                            static_cast<const bf16_t *>(bias)));
    return LAYA_OK;
}

int laya_op_gemm_layernorm(void *stream, const void *A, int32_t lda, const void *W, int32_t ldw,
                           void *x, void *n, const float *gamma, int32_t M, int32_t N, int32_t K,
                           int32_t config, int32_t splits, const void *bias, float eps) {
    // whole K (splits == 1): any one-kernel tile shape; a K split: the small shapes
    const bool whole = splits == 1;
    if (!gemm_args_ok(A, lda, W, ldw, x, N, M, N, K, config) || N > 1024 || !(eps > 0.f) ||
        config < 0 ||
        (whole ? config == laya::kPingPongConfig
               : ((config > 3 && config < 7) || splits < 2 || splits > K / 64 ||
                  splits > laya::gemm_max_splits(config))) ||
        (M > 0 && (!n || !gamma || n == x)) || reinterpret_cast<uintptr_t>(bias) % 16 != 0)
        return set_global_error(LAYA_E_INVALID, "laya_op_gemm_layernorm: bad arguments");
    if (M == 0) return LAYA_OK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const laya::GemmPlan plan{config, splits};
    void *scratch = nullptr;
    if (!whole && hipMalloc(&scratch, laya::gemm_workspace_bytes(plan, M, N, 0)) != hipSuccess)
        return set_global_error(LAYA_E_NOMEM, "laya_op_gemm_layernorm: scratch hipMalloc failed");
    hipError_t e = laya::launch_gemm_layernorm(
        s, static_cast<const bf16_t *>(A), lda, static_cast<const bf16_t *>(W), ldw, nullptr, M, N,
        K, plan, static_cast<float *>(scratch), static_cast<const bf16_t *>(bias),
        static_cast<bf16_t *>(x), static_cast<bf16_t *>(n), gamma, eps);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (scratch) hipFree(scratch);
    if (e != hipSuccess)
        return set_global_error(LAYA_E_DEVICE,
                                std::string("laya_op_gemm_layernorm: ") + hipGetErrorString(e));
    return LAYA_OK;
}

int laya_op_gemm_qkv(void *stream, const void *A, int32_t lda, const void *W, int32_t ldw,
                     void *C, int32_t ldc, int32_t M, int32_t N, int32_t K, const int32_t *pos,
                     const void *cos_tab, const void *sin_tab, int32_t rope_cols, void *vt,
                     int32_t ldvt, const int32_t *vt_tok, int32_t vt_col0, int32_t config,
                     int32_t splits, const void *bias) {
    if (!gemm_args_ok(A, lda, W, ldw, C, ldc, M, N, K, config) || rope_cols < 0 ||
        rope_cols % 64 || vt_col0 % 64 || rope_cols > vt_col0 || vt_col0 > N ||
        (M > 0 && rope_cols > 0 && (!pos || !cos_tab || !sin_tab)) ||
        (M > 0 && vt_col0 < N && (!vt || !vt_tok || ldvt <= 0)))
        return set_global_error(LAYA_E_INVALID, "laya_op_gemm_qkv: bad arguments");
    if (M == 0) return LAYA_OK;
    const laya::QkvEpilogue qe{pos, static_cast<const bf16_t *>(cos_tab),
                               static_cast<const bf16_t *>(sin_tab), rope_cols, vt_col0,
                               static_cast<bf16_t *>(vt), ldvt, vt_tok};
    return op_gemm_launch("laya_op_gemm_qkv", static_cast<hipStream_t>(stream), A, lda, W, ldw,
                          C, ldc, M, N, K, 2, config, splits, &qe, bias);
}

int laya_op_rope(void *stream, void *buf, int32_t ld, int32_t n_heads_rot, int32_t rows,
                 const int32_t *pos, const void *cos_tab, const void *sin_tab, int32_t max_pos) {
    if (rows < 0 || n_heads_rot <= 0 || ld % 8 || ld < n_heads_rot * 64 || max_pos <= 0 ||
        (rows > 0 && (!buf || !pos || !cos_tab || !sin_tab)))
        return set_global_error(LAYA_E_INVALID, "laya_op_rope: bad arguments");
    OPCHK(laya::launch_rope(static_cast<hipStream_t>(stream), static_cast<bf16_t *>(buf), ld,
                            n_heads_rot, nullptr, rows, pos, static_cast<const bf16_t *>(cos_tab),
                            static_cast<const bf16_t *>(sin_tab)));
    return LAYA_OK;
}

int laya_op_rope_original(void *stream, void *buf, int32_t ld, int32_t n_heads_rot, int32_t rows,
                          const int32_t *pos, const void *cos_tab, const void *sin_tab,
                          int32_t max_pos) {
    if (rows < 0 || n_heads_rot <= 0 || ld % 8 || ld < n_heads_rot * 64 || max_pos <= 0 ||
        (rows > 0 && (!buf || !pos || !cos_tab || !sin_tab)))
        return set_global_error(LAYA_E_INVALID, "laya_op_rope_original: bad arguments");
    OPCHK(laya::launch_rope_original(static_cast<hipStream_t>(stream), static_cast<bf16_t *>(buf),
                                     ld, n_heads_rot, nullptr, rows, pos,
                                     static_cast<const bf16_t *>(cos_tab),
                                     static_cast<const bf16_t *>(sin_tab)));
    return LAYA_OK;
}

int laya_op_attention(void *stream, const void *q, int32_t ldq, const void *k, int32_t ldk,
                      const void *vt, int32_t ldvt, const int32_t *vt_col0, void *o, int32_t ldo,
                      int32_t n_heads, const int32_t *row_off, int32_t B, const int32_t *q_tok,
                      int32_t n_q, int32_t half_window) {
    if (B < 0 || n_heads <= 0 || ldq % 8 || ldk % 8 || ldo % 8 || ldvt % 8 ||
        ldq < n_heads * 64 || ldk < n_heads * 64 || ldo < n_heads * 64 || ldvt <= 0 || !row_off ||
        (B > 0 && !vt_col0))
        return set_global_error(LAYA_E_INVALID, "laya_op_attention: bad arguments");
    if (row_off[0] != 0)
        return set_global_error(LAYA_E_INVALID, "laya_op_attention: row_off[0] != 0");
    for (int b = 0; b < B; ++b) {
        if (row_off[b + 1] <= row_off[b])
            return set_global_error(LAYA_E_INVALID, "laya_op_attention: empty or decreasing row");
        if (vt_col0[b] < 0 || vt_col0[b] % 8 ||
            (int64_t)vt_col0[b] + (row_off[b + 1] - row_off[b]) > ldvt)
            return set_global_error(LAYA_E_INVALID, "laya_op_attention: bad vt_col0");
    }
    const int T = B ? row_off[B] : 0;
    if (T == 0) return LAYA_OK;
    if (!q || !k || !vt || !o)
        return set_global_error(LAYA_E_INVALID, "laya_op_attention: NULL buffer");
    if (((int64_t)(T - 1) * ldk + n_heads * 64) * 2 > INT32_MAX ||
        (int64_t)n_heads * 64 * ldvt * 2 > INT32_MAX)
        return set_global_error(LAYA_E_UNSUPPORTED, "laya_op_attention: buffers over 2 GiB");
    std::vector<int32_t> qpos;
    std::vector<AttnBlock> blocks;
    int nb = 0;
    if (!q_tok) {
        qpos.resize(T);
        for (int b = 0; b < B; ++b)
            for (int t = row_off[b]; t < row_off[b + 1]; ++t) qpos[t] = t - row_off[b];
        blocks.resize((size_t)B * (512 / laya::kAttnQueries + T / laya::kAttnQueries + 1));
        build_blocks_full(row_off, vt_col0, B, half_window, blocks.data(), &nb);
    } else {
        if (n_q <= 0) return LAYA_OK;
        qpos.resize(n_q);
        std::vector<int32_t> qrow(n_q);
        for (int r = 0; r < n_q; ++r) {
            const int t = q_tok[r];
            if (t < 0 || t >= T)
                return set_global_error(LAYA_E_INVALID, "laya_op_attention: q_tok out of range");
            const int b = (int)(std::upper_bound(row_off, row_off + B + 1, t) - row_off) - 1;
            qrow[r] = b;
            qpos[r] = t - row_off[b];
        }
        blocks.resize(n_q);
        build_blocks_list(row_off, vt_col0, qrow.data(), qpos.data(), n_q, half_window,
                          blocks.data(), &nb);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    void *dmem = nullptr;
    const size_t bbytes = (size_t)nb * sizeof(AttnBlock);
    OPCHK(hipMalloc(&dmem, bbytes + qpos.size() * 4));
    hipError_t e = hipMemcpyAsync(dmem, blocks.data(), bbytes, hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(static_cast<char *>(dmem) + bbytes, qpos.data(), qpos.size() * 4,
                           hipMemcpyHostToDevice, s);
    if (e == hipSuccess) {
        const laya::AttnParams ap{
            static_cast<const bf16_t *>(q), ldq, static_cast<const bf16_t *>(k), ldk,
            (uint32_t)(((int64_t)(T - 1) * ldk + n_heads * 64) * 2),
            static_cast<const bf16_t *>(vt), ldvt, (uint32_t)((int64_t)n_heads * 64 * ldvt * 2),
            static_cast<bf16_t *>(o), ldo, static_cast<const AttnBlock *>(dmem), nullptr, nb,
            reinterpret_cast<const int32_t *>(static_cast<char *>(dmem) + bbytes), n_heads,
            half_window};
        e = laya::launch_attention(s, ap);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    hipFree(dmem);
    if (e != hipSuccess)
        return set_global_error(LAYA_E_DEVICE, std::string("laya_op_attention: ") + hipGetErrorString(e));
    return LAYA_OK;
}

}  // extern "C"
