"""The biased decision-head variant (laya_config.dec_head = 1) against the
CPU oracle (GPU only).

Variant of "perf(model): exact Metal speed-ups of the forward pass": every
projection of the two decision layers adds a bias to its BF16 product in
BF16, and their FFN is 4*hidden wide with plain GELU.  The same bars as the
default model: per layer on the GPU's own inputs within the pages' nRMS
0.005, end to end within 1.1x the oracle's float32-vs-float64 spread, graph
replay bitwise equal to eager, marker rows bitwise equal to the full pass's
rows, and no dependence on stale workspace contents.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import bits_of, ensure_built, report
from transformer_encoder_bf16_amd.inputs import (MODEL, TINY, WEIGHT_SEED, WORKLOADS, make_batch,
                                                 random_batch)

pytestmark = pytest.mark.gpu

NRMS_LIMIT = 5e-3
FLOOR_FACTOR = 1.1
TINY_NRMS_LIMIT = 1e-2
HEAD = dict(MODEL, dec_head=1)
TINY_HEAD = dict(TINY, dec_head=1)


@pytest.fixture(scope="module")
def binding():
    ensure_built()
    import torch
    torch.cuda.init()
    from transformer_encoder_bf16_amd import binding as b
    return b


@pytest.fixture(scope="module")
def enc(binding):
    e = binding.Encoder(HEAD, seed=WEIGHT_SEED)
    yield e
    e.close()


@pytest.fixture(scope="module")
def weights():
    return oracle.Weights(HEAD, WEIGHT_SEED)


@pytest.fixture(scope="module")
def orc(weights):
    return oracle.Oracle(HEAD, weights)


@pytest.fixture(scope="module")
def orc64(weights):
    return oracle.Oracle(HEAD, weights, accumulate="float64")


def _sync():
    import torch
    torch.cuda.synchronize()


def _run_bits(enc, batch, flags=0, markers=None):
    out = enc.run(batch.ids, batch.lengths, markers=markers, flags=flags)
    _sync()
    return enc.hidden_bits(out), out


def test_tiny_head_model_every_layer(binding):
    w = oracle.Weights(TINY_HEAD, 3)
    o = oracle.Oracle(TINY_HEAD, w)
    with binding.Encoder(TINY_HEAD, seed=3) as e:
        for tid, name, _ in oracle.tensor_shapes(TINY_HEAD):
            assert e.weight_digest(tid) == w.digest(name), (tid, name)
        for seed, markers in ((9, None), (10, np.array([[0, 0], [2, 5], [3, 1]], np.int32))):
            batch = random_batch(TINY_HEAD, 4, 40, seed=seed, len_lo=6)
            e.run(batch.ids, batch.lengths, markers=markers, flags=binding.RUN_CAPTURE_LAYERS)
            _sync()
            got = e.layer_outputs()
            want = o.forward(batch.ids, batch.lengths, markers=markers, capture=True)["layers"]
            assert [n for n, _ in got] == [n for n, _ in want]
            errs = {name: oracle.nrms(a, b_) for (name, a), (_, b_) in zip(got, want)}
            lw = o.forward_layerwise(batch.ids, batch.lengths, dict(got), markers=markers)
            per_layer = {n: oracle.nrms(dict(got)[n], y) for n, y in lw.items()}
            report("tiny_head_model", {"markers": markers is not None,
                                       "end_to_end_nrms": errs, "per_layer_nrms": per_layer})
            for name, err in errs.items():
                assert err < TINY_NRMS_LIMIT, name
            for name, err in per_layer.items():
                assert err < NRMS_LIMIT, name


def test_head_tensor_digests(enc):
    n_enc, n_dec = HEAD["n_enc_layers"], HEAD["n_dec_layers"]
    tids = dict((name, (tid, shape)) for tid, name, shape in oracle.tensor_shapes(HEAD))
    for L in range(n_enc - 1, n_enc + n_dec):
        names = ["wqkv", "wo", "wi", "wo2"] if L < n_enc else [
            "wqkv", "wo", "w1", "w2", "bqkv", "bo", "b1", "b2"]
        for n in names:
            tid, shape = tids[f"L{L}.{n}"]
            want = oracle.fnv1a64(oracle.tensor_bits(WEIGHT_SEED, tid, shape))
            assert enc.weight_digest(tid) == want, (L, n)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["short_1", "short_3", "marker_subset", "long_3", "mixed_16"])
def test_head_workload_matches_oracle(binding, enc, orc, orc64, name):
    _check_head(binding, enc, orc, orc64, make_batch(HEAD, WORKLOADS[name]), name)


# A short call with markers: the biased output and 4H-wide down projections run
# split with the bias in the fused reduce + LayerNorm, in the full pass and in
# the marker layer alike.
@pytest.mark.timeout(900)
def test_head_short_call_with_markers(binding, enc, orc, orc64):
    batch = random_batch(HEAD, 1, 48, seed=91, len_lo=48, markers_per_row=12)
    _check_head(binding, enc, orc, orc64, batch, "1x48+markers")


def _check_head(binding, enc, orc, orc64, batch, name):
    markers = batch.markers
    print(f"[head {name}] B={batch.B} S={batch.S} T={batch.T}", flush=True)
    enc.run(batch.ids, batch.lengths, markers=markers, flags=binding.RUN_CAPTURE_LAYERS)
    _sync()
    got = enc.layer_outputs()
    caps = dict(got)
    assert [n for n, _ in got] == orc.layer_names()
    lw = orc.forward_layerwise(batch.ids, batch.lengths, caps, markers=markers)
    per_layer = {n: oracle.nrms(caps[n], y) for n, y in lw.items()}
    ref = orc.forward(batch.ids, batch.lengths, markers=markers, capture=True)
    e2e = {n: oracle.nrms(caps[n], y) for n, y in ref["layers"]}
    ref64 = orc64.forward(batch.ids, batch.lengths, markers=markers)["out"]
    floor = oracle.nrms(ref64, ref["out"])
    print(f"[head {name}] per-layer worst {max(per_layer.values()):.3g}, final "
          f"{e2e['out']:.3g} (floor {floor:.3g})", flush=True)
    report("head_workload", {"workload": name, "per_layer_nrms": per_layer,
                             "end_to_end_nrms": e2e, "oracle_f32_vs_f64_final_nrms": floor})
    for n, e in per_layer.items():
        assert e <= NRMS_LIMIT, (n, e)
    assert e2e["out"] <= FLOOR_FACTOR * floor, (e2e["out"], floor)

    eager, _ = _run_bits(enc, batch, binding.RUN_EAGER, markers)
    assert np.array_equal(eager, bits_of(caps["out"]))
    g1, _ = _run_bits(enc, batch, 0, markers)
    assert np.array_equal(g1, eager)
    alone, _ = _run_bits(enc, batch, binding.RUN_EAGER | binding.RUN_ROPE_STANDALONE, markers)
    assert np.array_equal(alone, eager)
    if markers is not None:
        full, _ = _run_bits(enc, batch, binding.RUN_EAGER)
        rows = ref["row_off"][markers[:, 0]] + markers[:, 1]
        assert np.array_equal(eager, full[rows])


def test_head_nan_poisoned_workspace_changes_nothing(binding, enc):
    batch = make_batch(HEAD, WORKLOADS["marker_subset"])
    for markers in (None, batch.markers):
        clean, _ = _run_bits(enc, batch, binding.RUN_EAGER, markers)
        enc.fill_workspace(0xFF)
        again, _ = _run_bits(enc, batch, binding.RUN_EAGER, markers)
        assert np.array_equal(again, clean)
        enc.fill_workspace(0xFF)
        graph, _ = _run_bits(enc, batch, 0, markers)
        assert np.array_equal(graph, clean)


def test_head_and_default_share_the_encoder(binding, enc):
    """The variant changes only the decision layers: the encoder's final
    LayerNorm output is bitwise that of the default model."""
    batch = make_batch(MODEL, WORKLOADS["short_3"])
    enc.run(batch.ids, batch.lengths, flags=binding.RUN_CAPTURE_LAYERS)
    _sync()
    head_enc = bits_of(dict(enc.layer_outputs())["enc_final"])
    with binding.Encoder(MODEL, seed=WEIGHT_SEED) as d:
        d.run(batch.ids, batch.lengths, flags=binding.RUN_CAPTURE_LAYERS)
        _sync()
        base = dict(d.layer_outputs())
        assert np.array_equal(bits_of(base["enc_final"]), head_enc)
        assert not np.array_equal(bits_of(base["out"]),
                                  bits_of(dict(enc.layer_outputs())["out"]))
