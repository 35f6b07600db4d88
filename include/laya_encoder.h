/*
 * laya_encoder.h -- C ABI of the MI355X (gfx950) BF16 encoder forward pass.
 *
 * What the library computes: the forward pass of an encoder-only transformer
 * (a token embedding, then the encoder stack of 28 layers, then the two
 * decision layers), in BF16, with the final hidden states kept in device
 * memory for the scorer that consumes them (page "Run Laya encoder and
 * decision layers on CUDA", section Purpose).  Each layer is pre-LayerNorm (no bias) with rotary position
 * embedding, bidirectional attention that is global on every 3rd encoder
 * layer and a 128-token sliding window otherwise, and a GeGLU FFN; the QKV
 * projection, the rotation and attention are distinct steps ("[RFC]: Native
 * Laya inference with Rust and CUDA #14", section Design).  Optionally the last decision layer runs only
 * for a list of marker rows, with keys and values still computed for every
 * token (page "perf(model): exact Metal speed-ups of the forward pass").
 *
 * Conventions (the "ops.h"-style C ABI of the RFC's build discussion: an ABI
 * version query, int return codes, device work placed on a stream the caller
 * passes in so that the caller can capture it into a graph, resolved handles
 * reused):
 *   - every function returns LAYA_OK (0) or a negative LAYA_E_* code;
 *   - `stream` arguments are hipStream_t values passed as void* (NULL = the
 *     null stream); all device work is queued on that stream and nothing
 *     synchronises the host unless a function says so;
 *   - pointers documented "host" are ordinary host memory and are only read
 *     during the call; pointers documented "device" are device memory on the
 *     handle's device;
 *   - BF16 tensors are row-major arrays of 16-bit bfloat16 values;
 *   - validation happens before any device call: an invalid argument returns
 *     LAYA_E_INVALID (or LAYA_E_UNSUPPORTED) and touches no device state;
 *   - a HIP failure returns LAYA_E_DEVICE and poisons the handle: every later
 *     call on it returns LAYA_E_POISONED; laya_encoder_destroy still works.
 * Limits follow the worker's input limits: at most 16 rows ("questions"),
 * 512 tokens per row and 2048 markers (page "Laya native CUDA worker",
 * section Start and check).
 */
#ifndef LAYA_ENCODER_H
#define LAYA_ENCODER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LAYA_ABI_VERSION 6

#define LAYA_OK 0
#define LAYA_E_INVALID -1     /* bad ids, lengths, markers, sizes, NULL pointers */
#define LAYA_E_UNSUPPORTED -2 /* configuration outside the kernels' supported shapes */
#define LAYA_E_NOMEM -3       /* device or host allocation failed */
#define LAYA_E_DEVICE -4      /* a HIP call failed; the handle is poisoned */
#define LAYA_E_POISONED -5    /* the handle saw a device failure earlier */
#define LAYA_E_ABI -6         /* laya_config.abi_version != LAYA_ABI_VERSION */
#define LAYA_E_BUSY -7        /* request queue full */
#define LAYA_E_TIMEOUT -8     /* request deadline passed before it could run */
#define LAYA_E_CANCELLED -9   /* request dropped because its queue was destroyed */

/* laya_encoder_run flags */
#define LAYA_RUN_EAGER 1u          /* launch kernels directly instead of replaying a graph */
#define LAYA_RUN_CAPTURE_LAYERS 2u /* keep every layer's output (implies eager) */
#define LAYA_RUN_RESIDENT 4u       /* rerun on the indices already uploaded by the previous
                                      run of the same (B, S, R): no packing, no upload;
                                      token_ids/lengths/markers are not read */
#define LAYA_RUN_ROPE_STANDALONE 8u /* RoPE by its own kernel after the QKV projection
                                      instead of in the projection's epilogue (the
                                      pages' step order: projection, rotation, attention) */
#define LAYA_RUN_ROPE_ORIGINAL 16u /* RoPE by its own kernel in the original launch
                                      geometry (one thread per rotation pair, 64-bit index
                                      division), the reference arm of the RoPE comparison of
                                      "[Performance]: Optimize native Rust/CUDA Laya
                                      inference #66", section Starting evidence.  All three
                                      variants give bitwise equal outputs; each has its own
                                      graphs; at most one of the two flags may be set */

/* Model and limit configuration.  laya_config_init() fills the 421M-parameter
 * shape: vocab 50368, hidden 1024, 16 heads of 64, GeGLU inner width 2624,
 * 28 encoder layers then 2 decision layers, global attention on encoder layers with
 * l % 3 == 0 (RoPE theta 160000), a 128-token window elsewhere (theta 10000),
 * LayerNorm eps 1e-5, limits 16 rows x 512 tokens, 2048 markers. */
typedef struct laya_config {
    int32_t abi_version;   /* must be LAYA_ABI_VERSION */
    int32_t vocab;
    int32_t hidden;        /* n_heads * head_dim; multiple of 128, <= 1024 */
    int32_t n_heads;
    int32_t head_dim;      /* must be 64 */
    int32_t ffn;           /* GeGLU inner width F: W_i has 2F rows, W_o2 has F columns; multiple of 64 */
    int32_t n_enc_layers;
    int32_t n_dec_layers;  /* >= 1 */
    int32_t global_every;  /* encoder layer l is global iff l % global_every == 0 */
    int32_t window;        /* local layers see keys with |i - j| <= window / 2; even */
    float theta_global;
    float theta_local;
    float ln_eps;
    int32_t max_batch;     /* <= 16 */
    int32_t max_seq;       /* <= 512; also the number of rotary-table positions */
    int32_t max_markers;   /* <= 2048 */
    int32_t max_graphs;    /* captured graphs kept (LRU over shape keys), >= 1; 4 by default */
    int32_t workspace_budget_mib; /* create fails with LAYA_E_NOMEM if the workspace needs more;
                                     512 by default */
    int32_t dec_head;      /* 0 (default): decision layers are encoder-shaped.  1: the biased
                              head variant of the decision layers (page "perf(model): exact
                              Metal speed-ups of the forward pass": every projection adds a
                              bias, y = bf16(bf16(x W^T) + b), and the FFN is 4*hidden wide
                              with plain GELU, h = bf16(GELU(y1)), f = y2) */
} laya_config;

/* Device-resident result of a run.  Owned by the handle; valid until the next
 * laya_encoder_run with the same (B, S, R) shape, or laya_encoder_destroy. */
typedef struct laya_output {
    const void *hidden;     /* device BF16 [rows][dim] */
    int32_t rows;           /* T = sum of lengths (full run) or R (marker run) */
    int32_t dim;            /* hidden */
    const int32_t *row_off; /* device int32 [B + 1]: row b's tokens are rows row_off[b] ..
                               row_off[b+1]-1 (full run); NULL for a marker run */
} laya_output;

typedef struct laya_stats {
    double create_ms;        /* weights generated, tables built, workspace allocated */
    double last_capture_ms;  /* last graph miss: 2 eager warmups + capture + instantiate */
    int32_t graphs_cached;   /* instantiated graphs held by the handle (<= max_graphs) */
    int32_t graph_evictions; /* graphs destroyed to make room for a new shape */
    int32_t launches_last_run; /* kernel launches of the last eager run (or captured graph) */
    int64_t weight_bytes;    /* device bytes of resident weights */
    int64_t workspace_bytes; /* device bytes of the activation workspace */
} laya_stats;

typedef struct laya_encoder laya_encoder;

/* Returns LAYA_ABI_VERSION. */
int laya_abi_version(void);

/* Fills *cfg with the model shape and limits listed above.  Host only. */
void laya_config_init(laya_config *cfg);

/* Checks a configuration without touching the device.  Returns LAYA_OK,
 * LAYA_E_ABI, LAYA_E_INVALID (non-positive or inconsistent sizes) or
 * LAYA_E_UNSUPPORTED (head_dim != 64, hidden not a multiple of 128 or above
 * 1024, ffn not a multiple of 64, limits above 16 x 512 / 2048, or a shape
 * for which some planned GEMM launch would be unsupported). */
int laya_validate_config(const laya_config *cfg);

/* Host-only diagnostic: the GEMM plans of a pass over T live tokens and R
 * marker rows.  A plan is a tile shape (laya_op_gemm's `config`) and a number
 * of K ranges; every plan is the planner's choice for exactly T
 * (laya_plan_gemm), never for the padded B x S, so padding never changes a
 * result.  Plans are piecewise constant in T: *t_first and *t_last bound the
 * maximal run of token counts that share this pass's plans, and one captured
 * graph of a (B, S, R) serves exactly such a run.  out (host,
 * `cap` entries) receives the plans in the order QKV, output, up, down, then
 * (dec_head) head up, head down, then (R > 0) the marker layer's K/V, Q,
 * output, up, down (and head up, head down); *n_out is the full count.
 * fused = 1 marks a split projection whose reduce launch also does the
 * residual add and the next LayerNorm.  Returns LAYA_E_INVALID for T outside
 * [1, max_batch x max_seq] or R outside [0, max_markers]. */
typedef struct laya_gemm_plan {
    int32_t config;
    int32_t splits;
    int32_t fused;
} laya_gemm_plan;

int laya_pass_plans(const laya_config *cfg, int32_t T, int32_t R, int32_t *t_first,
                    int32_t *t_last, laya_gemm_plan *out, int32_t cap, int32_t *n_out);

/* Host-only diagnostic: the plan that laya_op_gemm (config -1) uses for an
 * M x N x K product with the given epilogue (0 plain, 1 GeGLU, 2 QKV, 3 bias
 * then GELU): the planner evaluated at exactly M rows.  A pass over T live
 * tokens uses exactly these plans for its projections; laya_pass_plans
 * reports them with the run of token counts that share them.  out->fused is
 * 0.  Returns LAYA_E_INVALID for M, N or K below 1, K not a multiple of 64,
 * an unknown epilogue, or a null out. */
int laya_plan_gemm(int32_t M, int32_t N, int32_t K, int32_t epilogue, laya_gemm_plan *out);

/* Checks run arguments without touching the device (the host half of
 * laya_encoder_run's validation; the worker's input limits, and the refusal
 * of invalid input before any model work, of page "Laya native CUDA worker",
 * section Start and check).  token_ids: host int32 [B][S] row-major,
 * right-padded, each valid id in [0, vocab); lengths: host int32 [B], each in
 * [1, S]; markers: host int32 [R][2] (row, position) pairs with position <
 * lengths[row], or NULL when R == 0.  B == 0 is valid (empty batch).  Limits:
 * B <= max_batch, S <= max_seq, R <= max_markers.  Returns LAYA_OK or
 * LAYA_E_INVALID. */
int laya_validate_run_args(const laya_config *cfg, const int32_t *token_ids,
                           const int32_t *lengths, int32_t B, int32_t S,
                           const int32_t *markers, int32_t R);

/* Creates a handle on HIP device `device`: validates cfg, allocates the
 * weights (vocab x hidden embedding plus four matrices per layer, all BF16)
 * and fills them on the device from weight_seed with the counter-based
 * generator below, builds the four rotary tables, and allocates the
 * activation workspace for max_batch x max_seq tokens.  Synchronous.
 *
 * Weight generator (there is no checkpoint; the pages load "English 421M",
 * page "[Performance]: Optimize native Rust/CUDA Laya inference #66", section
 * Recorded baseline and environment): element idx (nn.Linear [out][in]
 * order) of tensor tensor_id takes three SplitMix64 outputs
 *   r_j = mix64(seed + ((tensor_id << 40 | 3*idx + j) + 1) * 0x9e3779b97f4a7c15)
 * sums their twelve 16-bit fields s, and stores bf16_rne(0.02f * ((s - 393210)
 * / 65536.0f)).  Tensor ids: 0 embedding [vocab][hidden]; for layer L
 * (encoder layers first, then decision layers) 1+4L W_qkv [3*hidden][hidden]
 * with rows [Q | K | V], 2+4L W_o [hidden][hidden], 3+4L W_i [2*ffn][hidden]
 * with rows [GELU half | gate half], 4+4L W_o2 [hidden][ffn].  Every
 * LayerNorm gain is 1; there are no biases.  With dec_head = 1 the decision
 * layers' 3+4L is W_1 [4*hidden][hidden] and 4+4L is W_2 [hidden][4*hidden],
 * and after every weight tensor come decision layer d's biases (NL = all
 * layers): 1+4NL+4d b_qkv [3*hidden], +1 b_o [hidden], +2 b_1 [4*hidden],
 * +3 b_2 [hidden], drawn by the same generator (laya_encoder_weight reports
 * a bias as 1 row).
 *
 * Rotary tables (BF16-rounded tables exported once and then fixed, page
 * "Laya native CUDA worker", section Prepare the checkpoint and bundle; one
 * table for the global layers and one for the local ones, page
 * "[Performance]: Optimize native Rust/CUDA Laya inference #66", section
 * Starting evidence): cos and sin of p * theta^(-2i/head_dim), p < max_seq,
 * i < head_dim/2, evaluated in double and rounded once to BF16.
 *
 * On success *out owns all device memory it allocated.  Errors: LAYA_E_ABI,
 * LAYA_E_INVALID, LAYA_E_UNSUPPORTED, LAYA_E_NOMEM, LAYA_E_DEVICE (no handle is
 * returned; laya_last_error() explains). */
int laya_encoder_create(const laya_config *cfg, uint64_t weight_seed, int device,
                        laya_encoder **out);

/* Runs the forward pass on B right-padded rows of S token ids.
 *
 * Inputs (host, read before the call returns, so the caller may free them
 * at once): token_ids int32 [B][S], lengths int32 [B], markers int32 [R][2]
 * or NULL.  They are validated as laya_validate_run_args does, packed into
 * pinned staging memory and uploaded with one asynchronous copy on `stream`
 * (the host waits only if the previous run's upload from the same staging
 * memory is still in flight).  Padded positions are never computed: valid
 * tokens of all rows are packed and each query sees only its own row's keys.
 *
 * R == 0: the full pass; out->hidden is [T][hidden], T = sum(lengths), rows in
 * batch order, out->row_off the device row offsets.
 * R > 0: the last decision layer computes keys/values for every token but
 * queries, attention, output projection and FFN only for the R marker rows;
 * out->hidden is [R][hidden] in marker-list order (duplicates allowed).
 *
 * Without LAYA_RUN_EAGER the launch sequence for the shape key (B, S, R, the
 * RoPE variant flag, and the run of live token counts T whose GEMM plans are
 * equal, see laya_pass_plans) is captured once into a hipGraph (two eager
 * warmups, then capture; the cost is reported by laya_encoder_stats) and
 * replayed on `stream` afterwards; the kernels read T and the row layout
 * from device memory, so one graph serves every length pattern of its key.  Eager and graph runs give bitwise equal
 * outputs.  B == 0 returns LAYA_OK with out->rows == 0 and launches nothing.
 *
 * With LAYA_RUN_RESIDENT the pass reruns on the device copy of the previous
 * run's indices (same B, S, R; LAYA_E_INVALID otherwise): inputs already in
 * device memory, nothing crosses the host link (the reused-workspace reruns
 * with no readback in between of page "Run Laya encoder and decision layers
 * on CUDA", section Test Plan).
 *
 * The caller synchronises `stream` before reading out->hidden, and must not
 * run the same handle concurrently on two streams. */
int laya_encoder_run(laya_encoder *enc, void *stream, const int32_t *token_ids,
                     const int32_t *lengths, int32_t B, int32_t S,
                     const int32_t *markers, int32_t R, uint32_t flags,
                     laya_output *out);

/* Frees every resource of the handle (waits for its device work): the
 * resident weights and the shape workspaces the executor owns (page "Laya
 * native CUDA worker", section Prepare the checkpoint and bundle) and the
 * cached graphs ("[RFC]: Native Laya inference with Rust and CUDA #14",
 * section Design).  NULL is a no-op.  Works on a poisoned handle, which a
 * native failure leaves stopped but still to be released (the same page's
 * section Start and check). */
int laya_encoder_destroy(laya_encoder *enc);

/* Message of the last failure on this handle ("" if none): the text behind
 * the error classes of page "Laya native CUDA worker", section Start and
 * check (invalid input, unsupported shape, a native failure that stops the
 * executor).  The string is owned by the handle. */
const char *laya_encoder_last_error(const laya_encoder *enc);

/* Message of the last failure in this thread that had no handle to attach
 * to (laya_encoder_create, laya_validate_*, laya_op_*): a refused
 * configuration at startup, which the pages check before anything is loaded
 * (page "Run Laya encoder and decision layers on CUDA", section Purpose). */
const char *laya_last_error(void);

/* The per-layer hidden states that the pages compare against their
 * reference, intermediate states as well as final ones (page "Run Laya
 * encoder and decision layers on CUDA", section Test Plan; the comparison at
 * "encoder27" of "[Performance]: Optimize native Rust/CUDA Laya inference
 * #66", section Starting evidence).
 * After a run with LAYA_RUN_CAPTURE_LAYERS: layer output `index` (0 = "emb",
 * then "enc00".."enc<n_enc-1>" (residual stream after each encoder layer),
 * "enc_final", "dec0".., and "out"), as a device BF16 [rows][hidden] view
 * owned by the handle and valid until the next run.  name_out (host, may be
 * NULL) receives the NUL-terminated name.  Returns LAYA_E_INVALID for an
 * index out of range or when the last run did not capture. */
int laya_encoder_layer_output(laya_encoder *enc, int32_t index, laya_output *out,
                              char *name_out, size_t name_cap);

/* FNV-1a-64 over the BF16 bytes (little-endian, logical [out][in] order) of
 * weight tensor `tensor_id` (numbering as in laya_encoder_create): the
 * weight-parity check of the pages, here between the library and the
 * oracle's independent generator ("[RFC]: Native Laya inference with Rust
 * and CUDA #14", section Implementation and checks; frozen checkpoint hashes,
 * "[Performance]: Optimize native Rust/CUDA Laya inference #66", section
 * Validation and acceptance).  Copies the tensor to the host; synchronous;
 * diagnostic only. */
int laya_encoder_weight_digest(laya_encoder *enc, int32_t tensor_id, uint64_t *fnv64);

/* Device pointer (BF16, [rows][cols]) and shape of weight or bias tensor `tensor_id`;
 * diagnostic only. */
int laya_encoder_weight(laya_encoder *enc, int32_t tensor_id, const void **dev,
                        int32_t *rows, int32_t *cols);

/* Copies the handle's counters into *stats (host only): creation time, the
 * cost of the last graph capture and the graph cache's state, reported apart
 * from replay latency as "[Performance]: Optimize native Rust/CUDA Laya
 * inference #66", section Implementation priorities, asks (first-shape and
 * capture costs measured separately), with the LRU of captured shapes of
 * "[RFC]: Native Laya inference with Rust and CUDA #14", section Design.
 * LAYA_E_INVALID for NULL arguments. */
int laya_encoder_stats(const laya_encoder *enc, laya_stats *stats);

/* Diagnostic: fill every byte of the handle's workspace (activations,
 * transposed V, split-K partials, index upload) with `byte` (0xFF makes every
 * BF16 and float32 value a NaN), on `stream`, then synchronise.  A run after
 * it must give bitwise the same output as before: no kernel may depend on
 * stale workspace contents (the key-padding rows of a batch, the tiles past a
 * row's end, the partial tiles of a previous call).  Captured graphs stay
 * valid; the next non-resident run uploads its indices again.  Returns
 * LAYA_E_INVALID for a NULL handle and LAYA_E_DEVICE on a HIP failure. */
int laya_encoder_fill_workspace(laya_encoder *enc, void *stream, uint8_t byte);

/* The handle's configuration (as given to laya_encoder_create).  Host only. */
int laya_encoder_config(const laya_encoder *enc, laya_config *out);

/* LAYA_OK while the handle can run, LAYA_E_POISONED after a device failure
 * (the docs page's health check: a native failure stops this executor,
 * "Laya native CUDA worker", section Start and check).  Host only. */
int laya_encoder_health(const laya_encoder *enc);

/* Diagnostic for testing failure handling: marks the handle as if a device
 * call had failed (every later call returns LAYA_E_POISONED, health reports
 * it); nothing runs on the device. */
int laya_encoder_inject_failure(laya_encoder *enc);

/* ---------------------------------------------------------------------------
 * Serial request queue (the docs page's serving model, "Laya native CUDA
 * worker", section Architecture: one GPU worker runs complete requests one
 * at a time, in order; the queue holds a bounded number of requests and
 * refuses more; a deadline counts queueing and upload; no cross-request
 * batching).  The queue owns a worker thread with its own HIP stream; while
 * a queue exists, the caller must not run the handle directly.
 * ------------------------------------------------------------------------- */
typedef struct laya_queue laya_queue;

/* capacity: requests waiting (not counting the one running), >= 1 (the
 * pages use 32); deadline_ms > 0: a request that has not started within
 * deadline_ms of its submission fails with LAYA_E_TIMEOUT (the pages use
 * 30000).  LAYA_E_INVALID for bad arguments, LAYA_E_POISONED if the handle
 * already failed, LAYA_E_DEVICE if the worker's stream cannot be made. */
int laya_queue_create(laya_encoder *enc, int32_t capacity, double deadline_ms,
                      laya_queue **out);

/* Validates and copies the request (host arrays as for laya_encoder_run; the
 * caller may free them on return) and queues it.  out_host: caller-owned host
 * memory of out_cap bytes that receives the BF16 hidden states ([T or R]
 * [hidden]); it must stay valid until laya_queue_wait returns for the ticket.
 * Returns LAYA_E_INVALID (bad request or out_cap too small), LAYA_E_BUSY
 * (capacity requests already waiting), LAYA_E_POISONED (the executor has
 * stopped); *ticket identifies the request otherwise. */
int laya_queue_submit(laya_queue *q, const int32_t *token_ids, const int32_t *lengths,
                      int32_t B, int32_t S, const int32_t *markers, int32_t R, void *out_host,
                      size_t out_cap, uint64_t *ticket);

/* Blocks until the request is done and returns its status: LAYA_OK (out_host
 * filled, *rows set), LAYA_E_TIMEOUT, LAYA_E_POISONED (the executor stopped
 * before or while it ran), LAYA_E_DEVICE (it failed on the device; the
 * executor stops), LAYA_E_CANCELLED.  *latency_ms (optional): submission to
 * completion.  A ticket can be waited for once; LAYA_E_INVALID otherwise. */
int laya_queue_wait(laya_queue *q, uint64_t ticket, int32_t *rows, double *latency_ms);

/* LAYA_OK while the worker can serve, LAYA_E_POISONED once it has stopped. */
int laya_queue_health(const laya_queue *q);

/* Stops the worker after the running request; requests still waiting fail
 * with LAYA_E_CANCELLED.  Waits on the worker thread.  No laya_queue_wait may
 * be in progress on another thread when it is called. */
int laya_queue_destroy(laya_queue *q);

/* Per-op time of one eager pass (the pages' per-op share table of the
 * "profile_forward" tool, page "perf(model): exact Metal speed-ups of the
 * forward pass"): the same launches as laya_encoder_run, each bracketed by
 * HIP events on `stream`, aggregated by op class.  flops and bytes are the
 * algorithmic work of the class's launches (GEMMs 2*M*N*K; attention
 * 4*64*heads per visible (query, key) pair; bytes = the tensors each launch
 * must read and write once, in BF16).  Arguments as laya_encoder_run (flags:
 * only LAYA_RUN_ROPE_STANDALONE or LAYA_RUN_ROPE_ORIGINAL, to time a RoPE
 * variant);
 * synchronous; out receives up to `cap` classes, *n_out how many, *total_ms
 * (may be NULL) the event span of the whole pass.  Diagnostic only. */
typedef struct laya_op_time {
    char name[24];
    int32_t calls;
    double total_ms;
    double flops;
    double bytes;
} laya_op_time;

int laya_encoder_profile(laya_encoder *enc, void *stream, const int32_t *token_ids,
                         const int32_t *lengths, int32_t B, int32_t S,
                         const int32_t *markers, int32_t R, uint32_t flags, laya_op_time *out,
                         int32_t cap, int32_t *n_out, double *total_ms);

/* Rotary table of laya_encoder_create, on the host: cos_bits/sin_bits receive
 * max_pos * head_dim/2 BF16 bit patterns ([p][i] row-major).  Host only. */
int laya_rope_table(float theta, int32_t max_pos, int32_t head_dim,
                    uint16_t *cos_bits, uint16_t *sin_bits);

/* Copies `bytes` between host and device memory on `stream` and waits for
 * the copy.  kind: 0 device->host, 1 host->device, 2 device->device. */
int laya_memcpy(void *dst, const void *src, size_t bytes, int32_t kind, void *stream);

/* ----------------------------------------------------------------------------
 * Single-step entry points.  Each queues one step of the pass on `stream`,
 * on device buffers the caller owns; they are the same kernels the handle
 * launches.  Return LAYA_E_INVALID for inconsistent sizes or NULL pointers.
 * ------------------------------------------------------------------------- */

/* Embedding gather: out[t][:] = emb[ids[t]][:] for t < T (bit-exact copy).
 * emb device BF16 [vocab][hidden]; ids device int32 [T], each < vocab;
 * out device BF16 [T][hidden]. */
int laya_op_gather(void *stream, const void *emb, int32_t vocab, int32_t hidden,
                   const int32_t *ids, int32_t T, void *out);

/* Fused residual add + LayerNorm over T rows of `hidden` values:
 *   if r != NULL:  x[t] <- bf16(x[t] + r[t])   (written back to x)
 *   n[t] <- bf16((x[t] - mean) / sqrt(var + eps) * gamma)
 * with mean and biased variance of row t in float32, no bias; the division is
 * a multiply by the row's float32 1 / sqrt(var + eps).  x, r, n device
 * BF16 [T][hidden] (n must not alias x or r); gamma device float32 [hidden]. */
int laya_op_layernorm(void *stream, void *x, const void *r, void *n, const float *gamma,
                      int32_t T, int32_t hidden, float eps);

/* C[m][n] = bf16(sum_k A[m][k] * W[n][k]) for m < M, n < N (float32
 * accumulation; nn.Linear without bias).  epilogue 0: plain.  epilogue 1
 * (GeGLU): W has 2N rows; with u = A W[0:N]^T and g = A W[N:2N]^T in float32,
 * C = bf16(GELU(u) * g), GELU(z) = 0.5 z (1 + erf(z / sqrt 2)).  A device BF16
 * [M][lda], W device BF16 [N or 2N][ldw], C device BF16 [M][ldc]; K a multiple
 * of 64, N a multiple of 64, lda/ldw/ldc multiples of 8 (16-byte rows).
 * config -1 picks the tile shape and K split the pass itself would use for M
 * rows; config 0..11 (tile shapes 32x64, 64x64, 128x64, 128x128, 256x128,
 * 256x256, 128x128 with a shallower ring that fits two per compute unit,
 * 32x64 and 64x64 for short calls, two computing waves with deep rings,
 * 256x256 with two wave groups alternating between multiplying and loading,
 * 192x256 with twelve waves, and 256x192; weight rows x tokens) with
 * `splits` K ranges forces one (split K only on shapes 0..3, 7 and 8; GeGLU
 * not on shape 0).  Each output is the sum, in
 * order, of one MFMA chain per K range, so results depend only on `splits`.
 * With splits > 1 the call allocates its scratch and synchronises the
 * stream.
 *
 * bias (device BF16 [N], or NULL): the biased dense layer of the decision
 * head ("perf(model): exact Metal speed-ups of the forward pass"), the BF16
 * product plus the bias in BF16: epilogue 0 with a bias gives
 * C = bf16(bf16(A W^T) + bias); epilogue 3 (bias required) gives
 * C = bf16(GELU(bf16(bf16(A W^T) + bias))), the head's FFN input layer.
 * Epilogue 1 takes no bias. */
int laya_op_gemm(void *stream, const void *A, int32_t lda, const void *W, int32_t ldw,
                 void *C, int32_t ldc, int32_t M, int32_t N, int32_t K, int32_t epilogue,
                 int32_t config, int32_t splits, const void *bias);

/* laya_op_gemm for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * arguments, plan choice, results and errors as laya_op_gemm, bitwise, but
 * the split-K partials (splits > 1) go to a buffer the library holds for the
 * life of the process on each GPU it runs on (16 MiB; the bytes a plan needs
 * are 4 x tiles x splits x tile area), the call allocates and frees nothing,
 * and it does not synchronise: it only queues the launches on `stream`.
 * LAYA_E_INVALID, before any device work, when the split needs more than the
 * buffer.  Every call on one GPU shares that buffer, which keeps the last
 * call's contents (nothing in it needs clearing: each call writes every
 * partial it reads): calls that may overlap on one GPU, on different streams
 * or from different threads, race; the caller orders them. */
int laya_op_gemm_noalloc(void *stream, const void *A, int32_t lda, const void *W, int32_t ldw,
                         void *C, int32_t ldc, int32_t M, int32_t N, int32_t K, int32_t epilogue,
                         int32_t config, int32_t splits, const void *bias);

/* A projection onto the hidden width followed by the residual add and the
 * LayerNorm of the next sublayer (pre-norm stack, "[RFC]: Native Laya
 * inference with Rust and CUDA #14", section Design; fused residual and
 * LayerNorm as asked for short requests in "[Performance]: Optimize native
 * Rust/CUDA Laya inference #66", section Implementation priorities):
 *   f = bf16(A W^T) (with a bias: bf16(bf16(A W^T) + bias)),
 *   x <- bf16(x + f),  n <- bf16((x - mean) / sqrt(var + eps) * gamma),
 * bitwise laya_op_gemm(config, splits) into r followed by
 * laya_op_layernorm(x, r, n).  With `splits` >= 2 K ranges on tile shape
 * `config` (0..3, 7, 8) the split's reduce launch does the residual and the
 * LayerNorm; with splits == 1 (whole K, any tile shape but 9) the GEMM's
 * store does the residual add into x and a LayerNorm launch reading x alone
 * follows.  A device BF16 [M][lda], W device BF16 [N][ldw] (N <= 1024, a
 * multiple of 64), x device BF16 [M][N] (updated in place, 16-byte aligned),
 * n device BF16 [M][N] (not aliasing x), gamma device float32 [N], bias
 * device BF16 [N] 16-byte aligned or NULL.  The call allocates its scratch
 * (a K split only) and synchronises the stream; LAYA_E_INVALID for any other
 * argument. */
int laya_op_gemm_layernorm(void *stream, const void *A, int32_t lda, const void *W, int32_t ldw,
                           void *x, void *n, const float *gamma, int32_t M, int32_t N, int32_t K,
                           int32_t config, int32_t splits, const void *bias, float eps);

/* RoPE in place on `n_heads_rot` consecutive 64-wide heads starting at column
 * 0 of each of `rows` rows of buf (device BF16, row stride ld): with
 * (x, y) = (v[i], v[i+32]) and (c, s) = table[pos[row]][i],
 *   v[i] <- bf16(fl32(x c - y s)),  v[i+32] <- bf16(fl32(y c + x s)).
 * Columns beyond the rotated heads (the V block) are not read or written.
 * pos device int32 [rows], each < max_pos; cos_tab/sin_tab device BF16
 * [max_pos][32]. */
int laya_op_rope(void *stream, void *buf, int32_t ld, int32_t n_heads_rot, int32_t rows,
                 const int32_t *pos, const void *cos_tab, const void *sin_tab,
                 int32_t max_pos);

/* laya_op_rope in the original launch geometry of the pages' rotary kernel
 * (page "perf(model): exact Metal speed-ups of the forward pass": the kernel it
 * replaced derived each element's coordinates by 64-bit integer division):
 * one thread per rotation pair, its (row, head, pair) recovered from a flat
 * 64-bit index.  Arguments, result and errors as laya_op_rope, bitwise. */
int laya_op_rope_original(void *stream, void *buf, int32_t ld, int32_t n_heads_rot,
                          int32_t rows, const int32_t *pos, const void *cos_tab,
                          const void *sin_tab, int32_t max_pos);

/* The QKV projection with its two consumers' layouts fused into the epilogue
 * (the QKV projection that feeds the rotation and attention steps of "[RFC]: Native Laya
 * inference with Rust and CUDA #14", section Design; RoPE fused as the
 * optimised variant of "[Performance]: Optimize native Rust/CUDA Laya
 * inference #66", section Implementation priorities).  Computes
 * z = bf16(A W^T) as laya_op_gemm epilogue 0 (same plan rules, same bits),
 * then per output column f (heads of 64 columns):
 *   f < rope_cols:           RoPE of the head exactly as laya_op_rope, at
 *                            position pos[m] (device int32 [M]);
 *   rope_cols <= f < vt_col0: stored plain in C;
 *   f >= vt_col0:            stored transposed, vt[(f - vt_col0) * ldvt +
 *                            vt_tok[m]] (vt device BF16, vt_tok device int32
 *                            [M]); C is not written for these columns.
 * rope_cols and vt_col0 are multiples of 64 with rope_cols <= vt_col0 <= N.
 * cos_tab/sin_tab device BF16 [positions][32].  Not on tile shape 0.  With a
 * bias (device BF16 [N], or NULL) z = bf16(bf16(A W^T) + bias) before the
 * rotation and the transposed store, as laya_op_gemm. */
int laya_op_gemm_qkv(void *stream, const void *A, int32_t lda, const void *W, int32_t ldw,
                     void *C, int32_t ldc, int32_t M, int32_t N, int32_t K, const int32_t *pos,
                     const void *cos_tab, const void *sin_tab, int32_t rope_cols, void *vt,
                     int32_t ldvt, const int32_t *vt_tok, int32_t vt_col0, int32_t config,
                     int32_t splits, const void *bias);

/* Attention with a key-padding row and an optional sliding window, for a
 * packed batch (flash attention over the native QKV buffer, "[RFC]: Native
 * Laya inference with Rust and CUDA #14", section Design; single query rows
 * honour the padding mask, "perf(model): exact Metal speed-ups of the
 * forward pass").  Keys of row b are tokens row_off[b] .. row_off[b+1]-1 of
 * k (device BF16, row stride ldk, head h at columns 64h..64h+63); its values
 * are columns vt_col0[b] .. vt_col0[b] + len_b - 1 of vt (device BF16
 * [n_heads*64][ldvt], row 64h + d = dimension d of head h), the layout that
 * laya_op_gemm_qkv writes.  vt_col0 host int32 [B], each a multiple of 8 with
 * vt_col0[b] + len_b <= ldvt.
 * Queries: if q_tok == NULL, every token t is a query, at q row t;
 * otherwise q row r is the query of token q_tok[r] (host int32 [n_q],
 * grouped so that queries of one row are consecutive).  Query of token t in
 * row b at position p sees key j of the same row iff half_window < 0 or
 * |p - j| <= half_window; scores (q . k) / 8 in float32, softmax in float32
 * (the weights enter the products with v as a BF16 head plus a BF16 tail,
 * numerator and denominator alike), o = sum p v / sum p stored as BF16 at
 * o row r (device BF16, row stride ldo).
 * row_off host int32 [B + 1].  Index metadata is built on the host and
 * uploaded into a buffer this call allocates and frees (diagnostic entry;
 * synchronises the stream). */
int laya_op_attention(void *stream, const void *q, int32_t ldq, const void *k, int32_t ldk,
                      const void *vt, int32_t ldvt, const int32_t *vt_col0, void *o, int32_t ldo,
                      int32_t n_heads, const int32_t *row_off, int32_t B, const int32_t *q_tok,
                      int32_t n_q, int32_t half_window);

#ifdef __cplusplus
}
#endif

#endif /* LAYA_ENCODER_H */
