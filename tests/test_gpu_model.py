"""Whole-pass parity of the HIP path against the CPU oracle (GPU only).

The pages' parity limit is nRMS <= 0.005 ("[Performance]: Optimize native
Rust/CUDA Laya inference #66", section Starting evidence).  Two readings of
it are checked for every workload:

* per layer: each layer of the oracle is fed the GPU's own input to that
  layer and its output must be within nRMS 0.005 of the GPU's output (this is
  where a wrong kernel shows);
* end to end: the GPU's final hidden states against the oracle's.  In this
  BF16 pass a single rounding decision that comes out differently (any
  change of float32 summation order does that) grows until the two runs'
  rounding noise is decorrelated; the oracle against itself with a float64
  accumulator ends ~1.4% apart.  The GPU must stay within 1.1x of that floor,
  measured in the same test.  Up to 512 tokens the floor is the largest
  distance among three valid orders (float32, float64, and 16-deep K pieces
  added in order): a single token's distance is a noisy sample, 0.016 to
  0.027 among those orders at 1 token.  The pages' absolute 0.005 is NOT met end to end
  (final nRMS ~0.014 on every workload); test_end_to_end_absolute_limit
  records that as an expected failure, and every report says whether a
  batch met it.

The embedding must be bit-exact, graph replay must equal the eager run bit
for bit, repeated runs must be bitwise repeatable, and the invariants the
pages check hold bitwise: reversed row order, changed padding, and marker
rows equal to the same rows of the full pass.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import bits_of, ensure_built, report
from transformer_encoder_bf16_amd.inputs import (ALL_WORKLOADS, MODEL, TINY, WEIGHT_SEED, WORKLOADS, Batch,
                                                 make_batch, random_batch)

pytestmark = pytest.mark.gpu

NRMS_LIMIT = 5e-3
FLOOR_FACTOR = 1.1
# Token counts up to which the end-to-end floor also takes the 16-deep K-piece
# order (its oracle is slower, and above this the single spread is steady)
SMALL_T = 512


@pytest.fixture(scope="module")
def binding():
    ensure_built()
    import torch
    torch.cuda.init()
    from transformer_encoder_bf16_amd import binding as b
    return b


@pytest.fixture(scope="module")
def enc(binding):
    e = binding.Encoder(MODEL, seed=WEIGHT_SEED)
    yield e
    e.close()


@pytest.fixture(scope="module")
def weights():
    return oracle.Weights(MODEL, WEIGHT_SEED)


@pytest.fixture(scope="module")
def orc(weights):
    return oracle.Oracle(MODEL, weights)


@pytest.fixture(scope="module")
def orc64(weights):
    return oracle.Oracle(MODEL, weights, accumulate="float64")


def _sync():
    import torch
    torch.cuda.synchronize()


def test_weight_digests_match_oracle(enc):
    n_layers = MODEL["n_enc_layers"] + MODEL["n_dec_layers"]
    shapes = dict((tid, shape) for tid, _, shape in oracle.tensor_shapes(MODEL))
    for tid in [0, 1, 2, 3, 4, 4 * n_layers - 3, 4 * n_layers - 2, 4 * n_layers - 1, 4 * n_layers]:
        want = oracle.fnv1a64(oracle.tensor_bits(WEIGHT_SEED, tid, shapes[tid]))
        assert enc.weight_digest(tid) == want, tid


# The 128-wide, 5-layer test model amplifies perturbations several times per
# layer (float32 orderings alone move it by ~1e-3), so its bound is looser;
# it checks structure (layer order, digests, exact embedding), the 421M model
# checks the pages' limit.
TINY_NRMS_LIMIT = 1e-2


def test_tiny_model_every_layer(binding):
    w = oracle.Weights(TINY, 3)
    o = oracle.Oracle(TINY, w)
    with binding.Encoder(TINY, seed=3) as e:
        for tid, _, shape in oracle.tensor_shapes(TINY):
            assert e.weight_digest(tid) == w.digest(_), tid
        batch = random_batch(TINY, 4, 40, seed=9, len_lo=1)
        e.run(batch.ids, batch.lengths, flags=binding.RUN_CAPTURE_LAYERS)
        _sync()
        got = e.layer_outputs()
        want = o.forward(batch.ids, batch.lengths, capture=True)["layers"]
        assert [n for n, _ in got] == [n for n, _ in want]
        assert np.array_equal(bits_of(got[0][1]), bits_of(want[0][1]))
        errs = {name: oracle.nrms(a, b_) for (name, a), (_, b_) in zip(got, want)}
        lw = o.forward_layerwise(batch.ids, batch.lengths, dict(got))
        per_layer = {n: oracle.nrms(dict(got)[n], y) for n, y in lw.items()}
        report("tiny_model", {"end_to_end_nrms": errs, "per_layer_nrms": per_layer})
        for name, e in errs.items():
            assert e < TINY_NRMS_LIMIT, name
        for name, e in per_layer.items():
            assert e < NRMS_LIMIT, name


def _run_bits(binding, enc, batch, flags=0, markers=None):
    out = enc.run(batch.ids, batch.lengths, markers=markers, flags=flags)
    _sync()
    return enc.hidden_bits(out), out


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(ALL_WORKLOADS))
def test_workload_matches_oracle(binding, enc, orc, orc64, name):
    _check_batch(binding, enc, orc, orc64, make_batch(MODEL, ALL_WORKLOADS[name]), name)


# Token counts around where the GEMM plans change (split output and down
# projections with the fused residual + LayerNorm up to 256 and 1024 tokens,
# the split down projection up to 2048, whole K above, and tile shapes in
# between), one with markers so the marker layer's fused splits run too.
@pytest.mark.timeout(900)
@pytest.mark.parametrize("B,S,lo,mpr", [(1, 65, 65, 0), (1, 257, 257, 0), (2, 512, 400, 0),
                                        (5, 205, 150, 3), (9, 228, 180, 0)])
def test_plan_boundaries_match_oracle(binding, enc, orc, orc64, B, S, lo, mpr):
    batch = random_batch(MODEL, B, S, seed=B * 1000 + S, len_lo=lo, markers_per_row=mpr)
    _check_batch(binding, enc, orc, orc64, batch, f"{B}x{S}")


# Short calls with markers: the full pass's last layer runs the 32-row tiles
# and the split projections with the fused residual + LayerNorm over all
# tokens, the marker layer the same K ranges over the marker rows on other
# tiles; marker rows must equal the full pass's rows bit for bit.
@pytest.mark.timeout(900)
@pytest.mark.parametrize("B,S,lo,mpr", [(1, 48, 48, 12), (4, 16, 5, 4)])
def test_short_call_markers_match_full_rows(binding, enc, orc, orc64, B, S, lo, mpr):
    batch = random_batch(MODEL, B, S, seed=77 + B, len_lo=lo, markers_per_row=mpr)
    _check_batch(binding, enc, orc, orc64, batch, f"{B}x{S}+markers")


def _check_batch(binding, enc, orc, orc64, batch, name):
    markers = batch.markers
    print(f"[{name}] B={batch.B} S={batch.S} T={batch.T} R={0 if markers is None else len(markers)}",
          flush=True)
    # eager with per-layer capture
    enc.run(batch.ids, batch.lengths, markers=markers, flags=binding.RUN_CAPTURE_LAYERS)
    _sync()
    got_layers = enc.layer_outputs()
    caps = dict(got_layers)
    assert [n for n, _ in got_layers] == orc.layer_names()
    for lname, a in got_layers:
        assert np.isfinite(a).all(), lname

    # per layer, on the GPU's own inputs
    lw = orc.forward_layerwise(batch.ids, batch.lengths, caps, markers=markers)
    per_layer = {n: oracle.nrms(caps[n], y) for n, y in lw.items()}
    worst = max(per_layer, key=per_layer.get)
    print(f"[{name}] per-layer worst {worst} {per_layer[worst]:.3g}", flush=True)

    # end to end, and the oracle's own spread under a float64 accumulator
    ref = orc.forward(batch.ids, batch.lengths, markers=markers, capture=True)
    ref_layers = ref["layers"]
    assert np.array_equal(bits_of(caps["emb"]), bits_of(ref_layers[0][1]))  # embedding
    e2e = {n: oracle.nrms(caps[n], y) for n, y in ref_layers}
    ref64 = orc64.forward(batch.ids, batch.lengths, markers=markers)["out"]
    spreads = {"f32_vs_f64": oracle.nrms(ref64, ref["out"])}
    if batch.T <= SMALL_T:
        # one token's 1024 values give a noisy estimate of the spread, so
        # small calls take the largest distance among three valid orders
        r16 = oracle.Oracle(MODEL, orc.w, accumulate="chunk16").forward(
            batch.ids, batch.lengths, markers=markers)["out"]
        spreads["f32_vs_chunk16"] = oracle.nrms(r16, ref["out"])
        spreads["chunk16_vs_f64"] = oracle.nrms(r16, ref64)
    floor = max(spreads.values())
    final = e2e["out"]
    final64 = oracle.nrms(caps["out"], ref64)
    max_abs = float(np.abs(caps["out"] - ref["out"]).max())
    print(f"[{name}] end-to-end final nRMS {final:.3g} (oracle float32 vs float64 accumulation: "
          f"{floor:.3g}; GPU vs the float64 oracle {final64:.3g}), max_abs {max_abs:.3g}",
          flush=True)
    report("workload", {"workload": name, "T": batch.T, "per_layer_nrms": per_layer,
                        "end_to_end_nrms": e2e, "final_nrms": final, "max_abs": max_abs,
                        "oracle_f32_vs_f64_final_nrms": spreads["f32_vs_f64"],
                        "oracle_spreads": spreads, "floor": floor,
                        "final_nrms_vs_f64_oracle": final64,
                        "final_over_floor": final / floor if floor else None,
                        "end_to_end_within_0.005": bool(final <= NRMS_LIMIT)})
    for n, e in per_layer.items():
        assert e <= NRMS_LIMIT, (n, e)
    assert final <= FLOOR_FACTOR * floor, (final, floor)

    # eager (no capture), graph replay, repeat: all bitwise equal
    eager, _ = _run_bits(binding, enc, batch, binding.RUN_EAGER, markers)
    assert np.array_equal(eager, bits_of(caps["out"]))
    g1, out = _run_bits(binding, enc, batch, 0, markers)
    g2, _ = _run_bits(binding, enc, batch, 0, markers)
    assert np.array_equal(g1, eager)
    assert np.array_equal(g2, eager)
    st = enc.stats()
    assert st["graphs_cached"] >= 1 and st["last_capture_ms"] > 0

    if markers is not None:
        full, fout = _run_bits(binding, enc, batch, binding.RUN_EAGER)
        rows = ref["row_off"][markers[:, 0]] + markers[:, 1]
        bitwise = bool(np.array_equal(eager, full[rows]))
        to_f = lambda u: (u.astype(np.uint32) << 16).view(np.float32)
        e = oracle.nrms(to_f(eager), to_f(full[rows]))
        report("marker_subset_vs_full", {"rows": int(len(rows)), "bitwise": bitwise, "nrms": e})
        assert bitwise, e


def _batch_of(B, S, lengths, seed, markers=None):
    """A batch with the given row lengths (ids drawn as in the workloads)."""
    b = random_batch(MODEL, B, S, seed=seed)
    lengths = np.asarray(lengths, np.int32)
    ids = b.ids.copy()
    for r in range(B):
        ids[r, lengths[r]:] = 0
    mk = None if markers is None else np.asarray(markers, np.int32).reshape(-1, 2)
    return Batch(ids=ids, lengths=lengths, markers=mk)


# Degenerate shapes: a single token, single-token rows beside a full one,
# many tiny rows, every token a marker, and markers out of order with
# duplicates (the output follows the list).
DEGENERATE = {
    "1x1": (1, 1, [1], None),
    "3x512_1_512_2": (3, 512, [1, 512, 2], None),
    "16x8_tiny_rows": (16, 8, [1, 2, 3, 4, 5, 6, 7, 8, 8, 7, 6, 5, 4, 3, 2, 1], None),
    "2x20_all_markers": (2, 20, [20, 13], [(r, p) for r, n in ((0, 20), (1, 13)) for p in range(n)]),
    "4x30_markers_unordered": (4, 30, [30, 1, 17, 5],
                               [(2, 16), (0, 3), (1, 0), (0, 3), (3, 4), (2, 0), (0, 29), (3, 0)]),
}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(DEGENERATE))
def test_degenerate_shapes_match_oracle(binding, enc, orc, orc64, name):
    B, S, lengths, markers = DEGENERATE[name]
    _check_batch(binding, enc, orc, orc64, _batch_of(B, S, lengths, 7 + B * S, markers), name)


@pytest.mark.xfail(strict=True, reason=(
    "the pages' nRMS <= 0.005 is not met end to end: the BF16 pass is chaotic, any "
    "change of float32 summation order (the oracle's own float64 accumulation "
    "included) ends ~0.014 apart at the output; see the floor-relative checks"))
def test_end_to_end_absolute_limit(binding, enc, orc):
    """The pages' limit read as an absolute end-to-end bound on the final
    hidden states of the 1x48 call.  Expected to fail (strict): if it ever
    passes, the parity claims must be revisited."""
    batch = make_batch(MODEL, WORKLOADS["short_1"])
    out = enc.run(batch.ids, batch.lengths, flags=binding.RUN_EAGER)
    _sync()
    got = (enc.hidden_bits(out).astype(np.uint32) << 16).view(np.float32)
    final = oracle.nrms(got, orc.forward(batch.ids, batch.lengths)["out"])
    print(f"[short_1] end-to-end final nRMS {final:.4g} against the absolute 0.005", flush=True)
    assert final <= NRMS_LIMIT, final


def test_reversed_rows_and_padding_are_bitwise_invariant(binding, enc):
    batch = make_batch(MODEL, WORKLOADS["short_3"])
    base, out = _run_bits(binding, enc, batch, binding.RUN_EAGER)
    ro = np.concatenate([[0], np.cumsum(batch.lengths)])
    # reversed request order
    rev = type(batch)(ids=batch.ids[::-1].copy(), lengths=batch.lengths[::-1].copy())
    rbits, _ = _run_bits(binding, enc, rev, binding.RUN_EAGER)
    rro = np.concatenate([[0], np.cumsum(rev.lengths)])
    for b in range(batch.B):
        r = batch.B - 1 - b
        assert np.array_equal(base[ro[b]:ro[b + 1]], rbits[rro[r]:rro[r + 1]])
    # different padding ids, same padded width: bitwise
    ids2 = batch.ids.copy()
    for b in range(batch.B):
        ids2[b, batch.lengths[b]:] = 7 + b
    pad = type(batch)(ids=ids2, lengths=batch.lengths.copy())
    pbits, _ = _run_bits(binding, enc, pad, binding.RUN_EAGER)
    assert np.array_equal(base, pbits)
    gbits, _ = _run_bits(binding, enc, pad, 0)
    assert np.array_equal(base, gbits)
    # the same rows padded to a wider S (4x64 -> 4x96 and 4x512, where B*S
    # crosses several GEMM plan thresholds): plans follow the live token count
    # only, so every valid output is bitwise the same, eager and graph
    for width in (96, 512):
        ids3 = np.full((batch.B, width), 7, np.int32)
        for b in range(batch.B):
            ids3[b, :batch.lengths[b]] = batch.ids[b, :batch.lengths[b]]
        wide = type(batch)(ids=ids3, lengths=batch.lengths.copy())
        wbits, _ = _run_bits(binding, enc, wide, binding.RUN_EAGER)
        wgraph, _ = _run_bits(binding, enc, wide, 0)
        report("wider_padding", {"S": [batch.S, width],
                                 "bitwise": bool(np.array_equal(base, wbits))})
        assert np.array_equal(base, wbits), width
        assert np.array_equal(base, wgraph), width


def test_one_graph_serves_every_length_pattern(binding, enc):
    """Two length patterns of one (B, S) whose token counts fall in the same
    plan segment (a run of counts with equal GEMM plans) replay one graph; a
    third pattern in another segment gets its own graph; every replay equals
    its eager run bitwise."""
    wl = WORKLOADS["short_3"]
    b1 = make_batch(MODEL, wl)
    b2 = random_batch(MODEL, wl.B, wl.S, seed=99, len_lo=wl.len_lo)
    assert binding.pass_plans(MODEL, b1.T)[:2] == binding.pass_plans(MODEL, b2.T)[:2]
    e1, _ = _run_bits(binding, enc, b1, binding.RUN_EAGER)
    e2, _ = _run_bits(binding, enc, b2, binding.RUN_EAGER)
    g1, _ = _run_bits(binding, enc, b1, 0)
    n_graphs = enc.stats()["graphs_cached"]
    g2, _ = _run_bits(binding, enc, b2, 0)
    assert enc.stats()["graphs_cached"] == n_graphs
    assert np.array_equal(g1, e1) and np.array_equal(g2, e2)
    # 4 rows of 8..16 tokens: T <= 64, another plan segment of the same (B, S)
    b3 = random_batch(MODEL, wl.B, wl.S, seed=98, len_lo=8, len_hi=16)
    assert b3.T <= 64 < b1.T
    e3, _ = _run_bits(binding, enc, b3, binding.RUN_EAGER)
    g3, _ = _run_bits(binding, enc, b3, 0)
    assert np.array_equal(g3, e3)


def test_empty_batch_and_invalid_args(binding, enc):
    out = enc.run(np.zeros((0, 8), np.int32), np.zeros(0, np.int32))
    assert out.rows == 0
    batch = make_batch(MODEL, WORKLOADS["short_1"])
    bad = batch.ids.copy()
    bad[0, 3] = MODEL["vocab"] + 5
    with pytest.raises(binding.LayaError) as ei:
        enc.run(bad, batch.lengths)
    assert ei.value.code == binding.LAYA_E_INVALID
    # the handle is still usable and deterministic
    a, _ = _run_bits(binding, enc, batch, binding.RUN_EAGER)
    b_, _ = _run_bits(binding, enc, batch, binding.RUN_EAGER)
    assert np.array_equal(a, b_)


def test_configs_in_reverse_order_are_bitwise_equal(binding, enc):
    """The five configs run in order, then in reverse order on the same handle
    (reused workspace and graphs): every output is bitwise the same."""
    batches = {n: make_batch(MODEL, WORKLOADS[n]) for n in WORKLOADS}
    first = {n: _run_bits(binding, enc, b, 0, b.markers)[0] for n, b in batches.items()}
    for n in reversed(list(batches)):
        b = batches[n]
        again, _ = _run_bits(binding, enc, b, 0, b.markers)
        assert np.array_equal(again, first[n]), n


@pytest.mark.parametrize("name", ["short_1", "short_3", "long_3", "marker_subset"])
def test_nan_poisoned_workspace_changes_nothing(binding, enc, name):
    """Every workspace byte set to 0xFF (NaN in every BF16 and float32 slot)
    before an eager run and before a graph replay: the outputs are bitwise
    those of a clean run, so no kernel reads stale workspace contents."""
    batch = make_batch(MODEL, WORKLOADS[name])
    clean, _ = _run_bits(binding, enc, batch, binding.RUN_EAGER, batch.markers)
    enc.fill_workspace(0xFF)
    eager, _ = _run_bits(binding, enc, batch, binding.RUN_EAGER, batch.markers)
    assert np.array_equal(eager, clean)
    graph_clean, _ = _run_bits(binding, enc, batch, 0, batch.markers)
    enc.fill_workspace(0xFF)
    graph, _ = _run_bits(binding, enc, batch, 0, batch.markers)
    assert np.array_equal(graph, graph_clean) and np.array_equal(graph, clean)


@pytest.mark.parametrize("name", ["short_1", "long_3", "marker_subset"])
def test_rope_variants_are_bitwise_equal(binding, enc, name):
    """RoPE in the QKV projection's epilogue (the default), by its own kernel
    after the projection, and by its own kernel in the original launch
    geometry give bitwise equal outputs, eager and graph."""
    batch = make_batch(MODEL, WORKLOADS[name])
    fused, _ = _run_bits(binding, enc, batch, binding.RUN_EAGER, batch.markers)
    fused_g, _ = _run_bits(binding, enc, batch, 0, batch.markers)
    assert np.array_equal(fused_g, fused)
    for flag in (binding.RUN_ROPE_STANDALONE, binding.RUN_ROPE_ORIGINAL):
        alone, _ = _run_bits(binding, enc, batch, binding.RUN_EAGER | flag, batch.markers)
        alone_g, _ = _run_bits(binding, enc, batch, flag, batch.markers)
        assert np.array_equal(fused, alone), flag
        assert np.array_equal(alone_g, alone), flag


def test_unknown_run_flags_are_rejected(binding, enc):
    batch = make_batch(MODEL, WORKLOADS["short_1"])
    for flags in (64, binding.RUN_ROPE_STANDALONE | binding.RUN_ROPE_ORIGINAL):
        with pytest.raises(binding.LayaError) as ei:
            enc.run(batch.ids, batch.lengths, flags=flags)
        assert ei.value.code == binding.LAYA_E_INVALID


@pytest.mark.timeout(900)
def test_maximum_batch_and_markers_match_oracle(binding, enc, orc, orc64):
    """The handle's limits: 16 rows of 512 tokens (T = 8192, every row full)
    and 2048 marker rows (128 per row).  Per layer within the pages' 0.005 on
    the GPU's own inputs, end to end within 1.1x the oracle's float32/float64
    spread, graph equal to eager, marker rows bitwise equal to the full
    pass's rows."""
    batch = random_batch(MODEL, 16, 512, seed=77, len_lo=512, markers_per_row=128)
    mk = batch.markers
    assert batch.T == 8192 and len(mk) == 2048
    print("[max] B=16 S=512 T=8192 R=2048", flush=True)
    enc.run(batch.ids, batch.lengths, flags=binding.RUN_CAPTURE_LAYERS)
    _sync()
    caps = dict(enc.layer_outputs())
    lw = orc.forward_layerwise(batch.ids, batch.lengths, caps)
    per_layer = {n: oracle.nrms(caps[n], y) for n, y in lw.items()}
    ref = orc.forward(batch.ids, batch.lengths)
    final = oracle.nrms(caps["out"], ref["out"])
    floor = oracle.nrms(orc64.forward(batch.ids, batch.lengths)["out"], ref["out"])
    print(f"[max] per-layer worst {max(per_layer.values()):.3g}, final {final:.3g} "
          f"(floor {floor:.3g})", flush=True)
    report("maximum_batch", {"per_layer_nrms": per_layer, "final_nrms": final,
                             "oracle_f32_vs_f64_final_nrms": floor})
    for n, e in per_layer.items():
        assert e <= NRMS_LIMIT, (n, e)
    assert final <= FLOOR_FACTOR * floor, (final, floor)
    eager, _ = _run_bits(binding, enc, batch, binding.RUN_EAGER)
    graph, _ = _run_bits(binding, enc, batch, 0)
    assert np.array_equal(eager, bits_of(caps["out"])) and np.array_equal(graph, eager)
    sub_e, _ = _run_bits(binding, enc, batch, binding.RUN_EAGER, mk)
    sub_g, _ = _run_bits(binding, enc, batch, 0, mk)
    rows = ref["row_off"][mk[:, 0]] + mk[:, 1]
    assert np.array_equal(sub_e, eager[rows]) and np.array_equal(sub_g, sub_e)
