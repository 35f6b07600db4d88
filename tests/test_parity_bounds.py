"""What the parity bounds of the GPU tests can and cannot catch (CPU, oracle only).

The whole-pass GPU tests hold every layer, fed the GPU's own input, to the
pages' nRMS <= 0.005 ("[Performance]: Optimize native Rust/CUDA Laya
inference #66", section Starting evidence).  Here mistakes of the size a
kernel could make are planted in the oracle and run through the same
per-layer check, against the correct oracle, on the 1x48 workload of a
reduced-depth model (4 encoder + 2 decision layers of the full width, so the
whole file runs in about a minute):

* caught per layer: LayerNorm eps 1e-6 instead of 1e-5, and BF16 stores
  truncated instead of rounded to nearest in the QKV or the output
  projection;
* not caught per layer: the tanh approximation of GELU and truncated stores
  in the down projection stay under 0.005.  They are caught by the
  element-wise kernel checks instead (the GELU epilogue against float64 GELU
  on every BF16 value in [-12, 12]; every GEMM within one BF16 ulp of the
  oracle with under 2% of its outputs not bitwise equal), which is checked
  here on the same mistakes;
* a valid reordering of the float32 sums (16-deep K pieces, as a chain of
  matrix-core steps adds them) passes the per-layer check, while a bound
  relative to the oracle's own float32-vs-float64 spread would reject it (the
  spread underestimates other valid orders' rounding error by up to ~12x at
  some layers), so that floor is not used per layer.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import model as omodel
from tests.gpu_helpers import bf16_close
from transformer_encoder_bf16_amd.inputs import MODEL, WEIGHT_SEED, WORKLOADS, make_batch

LIMIT = 5e-3
CFG = dict(MODEL, n_enc_layers=4)


@pytest.fixture(scope="module")
def setup():
    w = oracle.Weights(CFG, WEIGHT_SEED)
    batch = make_batch(CFG, WORKLOADS["short_1"])
    return w, batch, oracle.Oracle(CFG, w)


def _per_layer(good, batch, caps):
    lw = good.forward_layerwise(batch.ids, batch.lengths, caps)
    return {n: oracle.nrms(caps[n], y) for n, y in lw.items()}


def _caps(o, batch):
    return dict(o.forward(batch.ids, batch.lengths, capture=True)["layers"])


def _trunc(y):
    return (np.ascontiguousarray(y, np.float32).view(np.uint32) &
            np.uint32(0xFFFF0000)).view(np.float32)


def _gelu_tanh(u):
    u = np.asarray(u, np.float64)
    return (0.5 * u * (1 + np.tanh(math.sqrt(2 / math.pi) * (u + 0.044715 * u ** 3)))
            ).astype(np.float32)


class _TruncatedStores(oracle.Oracle):
    """BF16 stores of one projection truncated instead of rounded (the
    product is truncated before the oracle's own rounding, which then keeps
    it): which = 'qkv', 'out' or 'down'."""

    def __init__(self, cfg, w, which):
        super().__init__(cfg, w)
        H, F = cfg["hidden"], cfg["ffn"]
        self.sel = {"qkv": (3 * H, H), "out": (H, H), "down": (H, F)}[which]

    def lin(self, a, w):
        y = super().lin(a, w)
        return _trunc(y) if tuple(w.shape) == self.sel else y


@pytest.mark.parametrize("mistake", ["ln_eps", "qkv_truncated", "out_truncated"])
def test_per_layer_limit_catches(setup, mistake):
    w, batch, good = setup
    if mistake == "ln_eps":
        bad = oracle.Oracle(dict(CFG, ln_eps=1e-6), w)
    else:
        bad = _TruncatedStores(CFG, w, mistake.split("_")[0])
    worst = max(_per_layer(good, batch, _caps(bad, batch)).values())
    assert worst > LIMIT, worst


def test_per_layer_limit_misses_gelu_and_down_truncation(setup, monkeypatch):
    w, batch, good = setup
    down = max(_per_layer(good, batch, _caps(_TruncatedStores(CFG, w, "down"), batch)).values())
    monkeypatch.setattr(omodel, "gelu", _gelu_tanh)
    caps = _caps(oracle.Oracle(CFG, w), batch)
    monkeypatch.undo()
    gelu = max(_per_layer(good, batch, caps).values())
    assert 0 < gelu < LIMIT and 0 < down < LIMIT, (gelu, down)


def test_kernel_checks_catch_what_the_layer_check_misses():
    # GEMM outputs truncated instead of rounded: half the outputs are off by
    # one ulp, far above the 2% of non-bitwise outputs the GEMM tests allow
    rng = np.random.default_rng(3)
    a = oracle.bf16_round(rng.standard_normal((96, 512)).astype(np.float32))
    wt = oracle.bf16_round((0.03 * rng.standard_normal((256, 512))).astype(np.float32))
    prod = oracle.linear(a, wt)
    bad, frac = bf16_close(_trunc(prod), oracle.bf16_round(prod))
    assert frac > 0.3, frac
    # tanh GELU against the exact GELU on the BF16 grid of [-12, 12] that the
    # epilogue test walks: many values differ after BF16 rounding
    z = oracle.bf16_bits_to_f32(np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16))
    z = z[np.isfinite(z) & (np.abs(z) <= 12)]
    exact = oracle.bf16_round(oracle.gelu(z))
    approx = oracle.bf16_round(_gelu_tanh(z))
    assert (exact != approx).sum() > 100


def test_valid_reordering_passes_but_the_float64_floor_would_not(setup):
    w, batch, good = setup
    caps = _caps(oracle.Oracle(CFG, w, accumulate="chunk16"), batch)
    per_layer = _per_layer(good, batch, caps)
    assert max(per_layer.values()) < LIMIT, per_layer
    good64 = oracle.Oracle(CFG, w, accumulate="float64")
    l32 = good.forward_layerwise(batch.ids, batch.lengths, caps)
    l64 = good64.forward_layerwise(batch.ids, batch.lengths, caps)
    ratio = {n: oracle.nrms(caps[n], l64[n]) / oracle.nrms(l32[n], l64[n])
             for n in l32 if oracle.nrms(l32[n], l64[n]) > 0}
    assert max(ratio.values()) > 2.0, ratio
