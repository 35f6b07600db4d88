// Serial request queue over one encoder handle: the serving model of the
// docs page ("Laya native CUDA worker", section Architecture).
//   - One worker thread runs complete requests one at a time, in submission
//     order, on its own HIP stream (default priority); there is no
//     cross-request batching.
//   - The queue holds at most `capacity` waiting requests (32 on the page);
//     a submission beyond that is refused (the page's HTTP 503).
//   - A deadline (30 s on the page) counts queueing and upload: a request
//     that has not started within it fails with LAYA_E_TIMEOUT.
//   - A native failure stops the executor: the failing request reports it,
//     every request still waiting fails with LAYA_E_POISONED, later
//     submissions are refused, and the health query reports it (the page's
//     500, then health 503).
// The worker only uses the public C ABI of the encoder.
#include <chrono>
#include <condition_variable>
#include <cstring>
#include <deque>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include <hip/hip_runtime.h>

#include "laya_encoder.h"

namespace {

using Clock = std::chrono::steady_clock;

constexpr int kPending = 1;  // status of a request not finished yet (never a LAYA code)

struct Request {
    uint64_t ticket = 0;
    std::vector<int32_t> ids, lengths, markers;
    int32_t B = 0, S = 0, R = 0;
    void *out = nullptr;
    size_t out_cap = 0;
    Clock::time_point submitted;
    int status = kPending;
    int32_t rows = 0;
    double latency_ms = 0;
};

}  // namespace

struct laya_queue {
    laya_encoder *enc = nullptr;
    int32_t capacity = 0;
    double deadline_ms = 0;
    hipStream_t stream = nullptr;
    mutable std::mutex mu;
    std::condition_variable work_cv, done_cv;
    std::deque<std::shared_ptr<Request>> waiting;
    std::map<uint64_t, std::shared_ptr<Request>> live;  // submitted, not yet collected
    uint64_t next_ticket = 1;
    bool stopping = false;
    bool stopped = false;  // the executor failed
    std::thread worker;
};

namespace {

double ms_since(Clock::time_point t) {
    return std::chrono::duration<double, std::milli>(Clock::now() - t).count();
}

// Runs one request on the worker's stream; returns its LAYA status.
int execute(laya_queue *q, Request &r) {
    laya_output out{};
    int rc = laya_encoder_run(q->enc, q->stream, r.ids.data(), r.lengths.data(), r.B, r.S,
                              r.R ? r.markers.data() : nullptr, r.R, 0, &out);
    if (rc != LAYA_OK) return rc;
    const size_t bytes = (size_t)out.rows * (size_t)out.dim * 2;
    if (bytes > r.out_cap) return LAYA_E_INVALID;  // checked at submission already
    if (bytes > 0) {
        if (hipMemcpyAsync(r.out, out.hidden, bytes, hipMemcpyDeviceToHost, q->stream) !=
            hipSuccess)
            return LAYA_E_DEVICE;
    }
    if (hipStreamSynchronize(q->stream) != hipSuccess) return LAYA_E_DEVICE;
    r.rows = out.rows;
    return LAYA_OK;
}

void worker_main(laya_queue *q, int device) {
    hipSetDevice(device);
    for (;;) {
        std::shared_ptr<Request> r;
        {
            std::unique_lock<std::mutex> lk(q->mu);
            q->work_cv.wait(lk, [&] { return q->stopping || !q->waiting.empty(); });
            if (q->stopping) {
                for (auto &w : q->waiting) w->status = LAYA_E_CANCELLED;
                q->waiting.clear();
                q->done_cv.notify_all();
                return;
            }
            r = q->waiting.front();
            q->waiting.pop_front();
        }
        int status;
        if (ms_since(r->submitted) > q->deadline_ms)
            status = LAYA_E_TIMEOUT;
        else if (laya_encoder_health(q->enc) != LAYA_OK)
            status = LAYA_E_POISONED;
        else
            status = execute(q, *r);
        std::lock_guard<std::mutex> lk(q->mu);
        r->status = status;
        r->latency_ms = ms_since(r->submitted);
        if (status == LAYA_E_DEVICE || status == LAYA_E_POISONED ||
            laya_encoder_health(q->enc) != LAYA_OK) {
            // the executor stops: nothing waiting will run
            q->stopped = true;
            for (auto &w : q->waiting) {
                w->status = LAYA_E_POISONED;
                w->latency_ms = ms_since(w->submitted);
            }
            q->waiting.clear();
        }
        q->done_cv.notify_all();
    }
}

}  // namespace

extern "C" {

int laya_queue_create(laya_encoder *enc, int32_t capacity, double deadline_ms,
                      laya_queue **out) {
    if (!enc || !out || capacity < 1 || !(deadline_ms > 0)) return LAYA_E_INVALID;
    *out = nullptr;
    if (laya_encoder_health(enc) != LAYA_OK) return LAYA_E_POISONED;
    auto q = std::make_unique<laya_queue>();
    q->enc = enc;
    q->capacity = capacity;
    q->deadline_ms = deadline_ms;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return LAYA_E_DEVICE;
    if (hipStreamCreateWithFlags(&q->stream, hipStreamNonBlocking) != hipSuccess)
        return LAYA_E_DEVICE;
    laya_queue *raw = q.get();
    raw->worker = std::thread(worker_main, raw, device);
    *out = q.release();
    return LAYA_OK;
}

int laya_queue_submit(laya_queue *q, const int32_t *token_ids, const int32_t *lengths,
                      int32_t B, int32_t S, const int32_t *markers, int32_t R, void *out_host,
                      size_t out_cap, uint64_t *ticket) {
    if (!q || !ticket) return LAYA_E_INVALID;
    // the whole request is checked against the handle's limits before it is
    // queued (host only)
    laya_config cfg;
    if (laya_encoder_config(q->enc, &cfg) != LAYA_OK) return LAYA_E_INVALID;
    const int vr = laya_validate_run_args(&cfg, token_ids, lengths, B, S, markers, R);
    if (vr != LAYA_OK) return vr;
    int64_t rows = R;
    if (R == 0)
        for (int b = 0; b < B; ++b) rows += lengths[b];
    if ((rows > 0 && !out_host) || (size_t)rows * (size_t)cfg.hidden * 2 > out_cap)
        return LAYA_E_INVALID;
    auto r = std::make_shared<Request>();
    r->B = B;
    r->S = S;
    r->R = R;
    r->ids.assign(token_ids, token_ids + (size_t)B * S);
    r->lengths.assign(lengths, lengths + B);
    if (R > 0) r->markers.assign(markers, markers + 2 * (size_t)R);
    r->out = out_host;
    r->out_cap = out_cap;
    std::lock_guard<std::mutex> lk(q->mu);
    if (q->stopped || laya_encoder_health(q->enc) != LAYA_OK) return LAYA_E_POISONED;
    if (q->stopping) return LAYA_E_CANCELLED;
    if ((int32_t)q->waiting.size() >= q->capacity) return LAYA_E_BUSY;
    r->ticket = q->next_ticket++;
    r->submitted = Clock::now();
    q->waiting.push_back(r);
    q->live[r->ticket] = r;
    *ticket = r->ticket;
    q->work_cv.notify_one();
    return LAYA_OK;
}

int laya_queue_wait(laya_queue *q, uint64_t ticket, int32_t *rows, double *latency_ms) {
    if (!q) return LAYA_E_INVALID;
    std::unique_lock<std::mutex> lk(q->mu);
    auto it = q->live.find(ticket);
    if (it == q->live.end()) return LAYA_E_INVALID;
    std::shared_ptr<Request> r = it->second;
    q->done_cv.wait(lk, [&] { return r->status != kPending; });
    q->live.erase(ticket);
    if (rows) *rows = r->rows;
    if (latency_ms) *latency_ms = r->latency_ms;
    return r->status;
}

int laya_queue_health(const laya_queue *q) {
    if (!q) return LAYA_E_INVALID;
    std::lock_guard<std::mutex> lk(q->mu);
    return (q->stopped || laya_encoder_health(q->enc) != LAYA_OK) ? LAYA_E_POISONED : LAYA_OK;
}

int laya_queue_destroy(laya_queue *q) {
    if (!q) return LAYA_OK;
    {
        std::lock_guard<std::mutex> lk(q->mu);
        q->stopping = true;
    }
    q->work_cv.notify_all();
    if (q->worker.joinable()) q->worker.join();
    {
        // anything still waiting after the worker left (it cancels on exit)
        std::lock_guard<std::mutex> lk(q->mu);
        for (auto &w : q->waiting) w->status = LAYA_E_CANCELLED;
        q->waiting.clear();
    }
    q->done_cv.notify_all();
    if (q->stream) hipStreamDestroy(q->stream);
    delete q;
    return LAYA_OK;
}

}  // extern "C"
