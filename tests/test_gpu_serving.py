"""Serving lifecycle on the GPU: the graph cache's LRU bound, the workspace
budget, the serial request queue (order, bitwise results, refusal when
full, deadline), and the stop-on-failure health state ("Laya native CUDA
worker", section Architecture; "Run Laya encoder and decision layers on
CUDA", section Implementation).  Failures are forced from the host
(laya_encoder_inject_failure); nothing here faults the GPU."""
import numpy as np
import pytest

from tests.gpu_helpers import ensure_built
from transformer_encoder_bf16_amd.inputs import MODEL, WEIGHT_SEED, WORKLOADS, make_batch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def binding():
    ensure_built()
    import torch
    torch.cuda.init()
    torch.cuda.set_device(0)
    from transformer_encoder_bf16_amd import binding as b
    return b


def _sync():
    import torch
    torch.cuda.synchronize()


def _bits(binding, enc, batch, flags=0):
    out = enc.run(batch.ids, batch.lengths, markers=batch.markers, flags=flags)
    _sync()
    return enc.hidden_bits(out)


def test_graph_cache_is_lru_bounded(binding):
    cfg = dict(MODEL, max_graphs=2)
    names = ["short_1", "short_3", "long_3"]
    batches = [make_batch(MODEL, WORKLOADS[n]) for n in names]
    with binding.Encoder(cfg, seed=WEIGHT_SEED, device=0) as enc:
        first = [_bits(binding, enc, b) for b in batches]
        st = enc.stats()
        assert st["graphs_cached"] == 2 and st["graph_evictions"] == 1
        # short_1 was evicted: it is captured again and gives the same bits
        again = _bits(binding, enc, batches[0])
        st = enc.stats()
        assert st["graphs_cached"] == 2 and st["graph_evictions"] == 2
        assert np.array_equal(again, first[0])
        # the most recent shape is still cached (no new eviction)
        assert np.array_equal(_bits(binding, enc, batches[0]), first[0])
        assert enc.stats()["graph_evictions"] == 2


def test_workspace_budget_is_enforced(binding):
    with pytest.raises(binding.LayaError) as ei:
        binding.Encoder(dict(MODEL, workspace_budget_mib=64), seed=WEIGHT_SEED, device=0)
    assert ei.value.code == binding.LAYA_E_NOMEM


@pytest.fixture(scope="module")
def enc(binding):
    e = binding.Encoder(MODEL, seed=WEIGHT_SEED, device=0)
    yield e
    e.close()


def test_queue_runs_requests_in_order_with_direct_run_results(binding, enc):
    batches = [make_batch(MODEL, WORKLOADS[n]) for n in WORKLOADS]
    direct = [_bits(binding, enc, b, binding.RUN_EAGER) for b in batches]
    with binding.Queue(enc, capacity=32, deadline_ms=30000.0) as q:
        assert q.health() == binding.LAYA_OK
        tickets = [q.submit(b.ids, b.lengths, markers=b.markers) for b in batches]
        lat = []
        for t, want in zip(tickets, direct):
            rc, got, ms = q.wait(t)
            assert rc == binding.LAYA_OK
            assert np.array_equal(got, want)
            lat.append(ms)
        # one worker, in submission order: each waited at least as long as the one before
        assert all(b >= a for a, b in zip(lat, lat[1:]))
        # an invalid request is refused at submission and does not stop the queue
        bad = batches[0].ids.copy()
        bad[0, 0] = MODEL["vocab"]
        with pytest.raises(binding.LayaError) as ei:
            q.submit(bad, batches[0].lengths)
        assert ei.value.code == binding.LAYA_E_INVALID
        assert q.health() == binding.LAYA_OK


def test_queue_refuses_when_full(binding, enc):
    b = make_batch(MODEL, WORKLOADS["mixed_16"])
    with binding.Queue(enc, capacity=2, deadline_ms=30000.0) as q:
        accepted, busy = [], 0
        for _ in range(12):
            try:
                accepted.append(q.submit(b.ids, b.lengths))
            except binding.LayaError as e:
                assert e.code == binding.LAYA_E_BUSY
                busy += 1
        assert busy >= 1 and len(accepted) >= 2
        for t in accepted:
            assert q.wait(t)[0] == binding.LAYA_OK


def test_queue_deadline_counts_queueing(binding, enc):
    b = make_batch(MODEL, WORKLOADS["short_1"])
    with binding.Queue(enc, capacity=4, deadline_ms=1e-6) as q:
        t = q.submit(b.ids, b.lengths)
        rc, out, _ = q.wait(t)
        assert rc == binding.LAYA_E_TIMEOUT and out is None
        assert q.health() == binding.LAYA_OK  # a timeout does not stop the executor


def test_queue_destroy_with_requests_waiting(binding, enc):
    b = make_batch(MODEL, WORKLOADS["mixed_16"])
    q = binding.Queue(enc, capacity=32, deadline_ms=30000.0)
    for _ in range(6):
        q.submit(b.ids, b.lengths)
    q.close()  # returns after the running request; the rest are cancelled
    # the handle is usable directly again
    s = make_batch(MODEL, WORKLOADS["short_1"])
    assert _bits(binding, enc, s).shape == (48, MODEL["hidden"])


def test_failure_stops_the_executor(binding):
    b = make_batch(MODEL, WORKLOADS["short_1"])
    with binding.Encoder(MODEL, seed=WEIGHT_SEED, device=0) as e:
        assert e.health() == binding.LAYA_OK
        with binding.Queue(e, capacity=4, deadline_ms=30000.0) as q:
            t = q.submit(b.ids, b.lengths)
            assert q.wait(t)[0] == binding.LAYA_OK
            e.inject_failure()
            assert e.health() == binding.LAYA_E_POISONED
            assert q.health() == binding.LAYA_E_POISONED
            with pytest.raises(binding.LayaError) as ei:
                q.submit(b.ids, b.lengths)
            assert ei.value.code == binding.LAYA_E_POISONED
        with pytest.raises(binding.LayaError) as ei:
            e.run(b.ids, b.lengths)
        assert ei.value.code == binding.LAYA_E_POISONED
