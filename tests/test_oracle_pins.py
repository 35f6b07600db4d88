"""Pins of the CPU oracle against things other than itself (CPU only).

Each check ties one oracle function to a published value, a closed form, a
library routine, an invariant, or the separately written float64 brute force
in tests/brute.  The last group plants plausible mistakes in the oracle and
shows the brute-force comparison catches every one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import model as omodel
from oracle import weights as oweights
from tests.brute import reference as brute
from transformer_encoder_bf16_amd.inputs import MODEL, TINY, random_batch, random_normal

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_ints(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [int(l) for l in f if l.strip() and not l.startswith("#")]


# ---------------------------------------------------------------- weights ----

def test_splitmix64_published_outputs():
    want = _golden_ints("splitmix64_seed1234567.txt")
    got = [oweights.splitmix64_at(1234567, k) for k in range(len(want))]
    assert got == want


def _py_splitmix(seed, key):
    m = (1 << 64) - 1
    z = (seed + (key + 1) * 0x9E3779B97F4A7C15) & m
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
    return z ^ (z >> 31)


@pytest.mark.parametrize("seed", [0, 1, 0xFFFFFFFFFFFFFFFF])
def test_irwin_hall_matches_python_integers(seed):
    rng = np.random.default_rng(7)
    for _ in range(50):
        tid = int(rng.integers(0, 121))
        idx = int(rng.integers(0, 51_000_000))
        s = 0
        for j in range(3):
            r = _py_splitmix(seed, (tid << 40) | (3 * idx + j))
            s += sum((r >> (16 * q)) & 0xFFFF for q in range(4))
        want = (s - 393210) / 65536.0
        assert oweights.irwin_hall(seed, tid, idx) == want


def test_weights_match_brute_numpy_generator():
    for tid, shape in [(0, (97, 128)), (5, (128, 192)), (13, (384, 128))]:
        got = oracle.bf16_bits_to_f32(oracle.tensor_bits(1, tid, shape)).astype(np.float64)
        want = brute.weights_f64(1, tid, shape)
        assert np.array_equal(got, want)


def test_weight_statistics_full_embedding():
    bits = oracle.tensor_bits(1, 0, (MODEL["vocab"], MODEL["hidden"]))
    w = oracle.bf16_bits_to_f32(bits).astype(np.float64)
    assert abs(w.mean()) < 2e-5
    assert abs(w.std() - 0.02) < 1e-4
    assert np.abs(w).max() <= 0.02 * 6.0 + 1e-3


def test_fnv1a64_known_values():
    # FNV-1a 64-bit: offset basis for the empty input, and "a".
    assert oracle.fnv1a64(np.zeros(0, np.uint8)) == 0xCBF29CE484222325
    assert oracle.fnv1a64(np.frombuffer(b"a", np.uint8)) == 0xAF63DC4C8601EC8C


# ------------------------------------------------------------------ bf16 -----

def test_bf16_round_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 100000).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-40, -1e-40,
                  1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20], np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = oracle.bf16_round(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert np.isnan(oracle.bf16_round(np.array([np.nan], np.float32))[0])


def test_f64_to_bf16_matches_brute():
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.uniform(-1, 1, 3000), [1.0, -1.0, 0.0, 1.0 + 2.0 ** -8,
                                                   1.0 + 2.0 ** -8 + 2.0 ** -40, 0.5 + 2.0 ** -10]])
    assert np.array_equal(oracle.f64_to_bf16(v).astype(np.float64), brute.bf16_direct(v))


# ------------------------------------------------------------------ RoPE -----

@pytest.mark.parametrize("theta", [10000.0, 160000.0])
def test_rope_tables(theta):
    c, s = oracle.rope_tables(theta, 512, 64)
    assert c.shape == (512, 32) and c.dtype == np.float32
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)
    p = np.arange(512)[:, None]
    ang = p * theta ** (-2.0 * np.arange(32)[None, :] / 64)
    for tab, exact in ((c, np.cos(ang)), (s, np.sin(ang))):
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 7)
        assert np.all(np.abs(tab - exact) <= ulp / 2 + 1e-300)
    # the independently rounded brute-force table agrees bit for bit (64 rows)
    bc, bs = brute.rope_table(theta, 64, 64)
    assert np.array_equal(c[:64].astype(np.float64), bc)
    assert np.array_equal(s[:64].astype(np.float64), bs)


def test_rope_position_zero_is_identity_and_v_is_not_touched():
    c, s = oracle.rope_tables(10000.0, 512, 64)
    v = oracle.bf16_round(random_normal((5, 3, 64), 1))
    out = oracle.rope_apply(v, np.zeros(5, np.int64), c, s)
    assert np.array_equal(out, v)


def test_rope_matches_complex_rotation():
    c, s = oracle.rope_tables(160000.0, 512, 64)
    v = oracle.bf16_round(random_normal((40, 4, 64), 2))
    pos = np.random.default_rng(2).integers(0, 512, 40)
    got = oracle.rope_apply(v, pos, c, s)
    z = (v[..., :32].astype(np.float64) + 1j * v[..., 32:]) * (c[pos][:, None, :] + 1j * s[pos][:, None, :])
    want = brute.bf16(np.concatenate([z.real, z.imag], axis=-1))
    assert np.array_equal(got.astype(np.float64), want)


def test_rope_relative_position_property():
    # with exact (unrounded) tables, q_m . k_n depends only on m - n
    th = 10000.0
    p = np.arange(512)[:, None]
    ang = p * th ** (-2.0 * np.arange(32)[None, :] / 64)
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    q = random_normal((1, 1, 64), 5)
    k = random_normal((1, 1, 64), 6)
    dots = []
    for m, n in [(10, 3), (100, 93), (400, 393)]:
        qm = oracle.rope_apply(q, np.array([m]), c, s, rounding=False).astype(np.float64)
        kn = oracle.rope_apply(k, np.array([n]), c, s, rounding=False).astype(np.float64)
        dots.append(float((qm * kn).sum()))
    assert max(dots) - min(dots) < 1e-4 * max(1.0, abs(dots[0]))


# ---------------------------------------------------- LayerNorm / GELU -------

def test_layer_norm_against_float64_and_moments():
    x = random_normal((64, 1024), 8, scale=3.0) + np.float32(0.5)
    g = np.ones(1024, np.float32)
    y = oracle.layer_norm(x, g, 1e-5)
    xd = x.astype(np.float64)
    want = (xd - xd.mean(1, keepdims=True)) / np.sqrt(xd.var(1, keepdims=True) + 1e-5)
    assert np.abs(y - want).max() < 1e-5
    assert np.abs(y.mean(1)).max() < 1e-5
    assert np.abs(y.astype(np.float64).var(1) - 1.0).max() < 1e-4
    g2 = (1.0 + 0.1 * random_normal(1024, 9)).astype(np.float32)
    assert np.abs(oracle.layer_norm(x, g2, 1e-5) - want * g2).max() < 2e-5


def test_gelu_closed_forms():
    rows = []
    with open(os.path.join(GOLDEN, "normal_cdf.txt")) as f:
        for l in f:
            if l.strip() and not l.startswith("#"):
                z, phi = map(float, l.split())
                rows.append((z, phi))
    for z, phi in rows:
        assert abs(float(oracle.gelu(np.array([z], np.float32))[0]) - z * phi) < 1e-7 * max(1, abs(z))
    assert oracle.gelu(np.array([0.0], np.float32))[0] == 0.0
    z = np.linspace(-8, 8, 1001).astype(np.float32)
    odd = oracle.gelu(z).astype(np.float64) - oracle.gelu(-z).astype(np.float64)
    assert np.abs(odd - z).max() < 1e-6
    big = np.array([12.0, 30.0], np.float32)
    assert np.array_equal(oracle.gelu(big), big)


# -------------------------------------------------------------- attention ----

def _qkv(T, nh, seed):
    q = oracle.bf16_round(random_normal((T, nh * 64), seed))
    k = oracle.bf16_round(random_normal((T, nh * 64), seed + 1))
    v = oracle.bf16_round(random_normal((T, nh * 64), seed + 2))
    return q, k, v


def test_attention_single_key_returns_v():
    q, k, v = _qkv(1, 2, 10)
    o = oracle.attention(q, k, v, np.array([0]), np.array([0]), 2, 64, None)
    assert np.array_equal(o, v)


def test_attention_identical_keys_average_values():
    q, k, v = _qkv(7, 1, 11)
    k[:] = k[0]
    o = oracle.attention(q, k, v, np.arange(7), np.arange(7), 1, 64, None, rounding=False)
    assert np.abs(o - v.mean(0)).max() < 1e-6


def test_attention_local_equals_global_inside_window():
    q, k, v = _qkv(65, 2, 12)
    pos = np.arange(65)
    a = oracle.attention(q, k, v, pos, pos, 2, 64, 64)
    b = oracle.attention(q, k, v, pos, pos, 2, 64, None)
    assert np.array_equal(a, b)


def test_attention_ignores_keys_outside_window():
    q, k, v = _qkv(200, 1, 13)
    pos = np.arange(200)
    a = oracle.attention(q, k, v, pos, pos, 1, 64, 64)
    k2, v2 = k.copy(), v.copy()
    k2[150:] = 7.0
    v2[150:] = -3.0
    b = oracle.attention(q, k2, v2, pos, pos, 1, 64, 64)
    assert np.array_equal(a[:86], b[:86])       # queries < 86 cannot see key 150
    assert not np.array_equal(a[86:], b[86:])


def test_attention_against_brute_force_loop():
    q, k, v = _qkv(30, 2, 14)
    pos = np.arange(30)
    for hw in (None, 4):
        got = oracle.attention(q, k, v, pos, pos, 2, 64, hw, rounding=False)
        want = np.zeros_like(got, dtype=np.float64)
        for h in range(2):
            sl = slice(64 * h, 64 * h + 64)
            for i in range(30):
                sc = np.array([q[i, sl].astype(np.float64) @ k[j, sl] for j in range(30)]) / 8.0
                if hw is not None:
                    sc[np.abs(np.arange(30) - i) > hw] = -np.inf
                p = np.exp(sc - sc.max())
                want[i, sl] = (p / p.sum()) @ v[:, sl]
        assert np.abs(got - want).max() < 1e-5


# ------------------------------------------------------------ whole model ----

@pytest.fixture(scope="module")
def tiny_batch():
    return random_batch(TINY, 3, 24, seed=5, len_lo=5)


@pytest.fixture(scope="module")
def tiny_weights():
    return oracle.Weights(TINY, 1)


@pytest.fixture(scope="module")
def brute_unrounded(tiny_batch):
    return brute.forward(TINY, 1, tiny_batch.ids, tiny_batch.lengths, rounding=False, capture=True)


# float32 (oracle) against float64 (brute force) with no BF16 rounding: the
# observed per-layer nRMS is ~4e-7; every planted mistake below exceeds 1e-5.
UNROUNDED_BOUND = 2e-6


def _max_layer_nrms(got, want):
    return max(oracle.nrms(a, b) for (_, a), (_, b) in zip(got["layers"], want["layers"]))


def test_model_matches_brute_without_rounding(tiny_batch, tiny_weights, brute_unrounded):
    got = oracle.Oracle(TINY, tiny_weights, rounding=False).forward(
        tiny_batch.ids, tiny_batch.lengths, capture=True)
    assert [n for n, _ in got["layers"]] == [n for n, _ in brute_unrounded["layers"]]
    assert _max_layer_nrms(got, brute_unrounded) < UNROUNDED_BOUND


def test_model_matches_brute_with_rounding(tiny_batch, tiny_weights):
    want = brute.forward(TINY, 1, tiny_batch.ids, tiny_batch.lengths, rounding=True, capture=True)
    got = oracle.Oracle(TINY, tiny_weights).forward(tiny_batch.ids, tiny_batch.lengths, capture=True)
    assert oracle.nrms(got["out"], want["out"]) < 5e-3
    assert np.array_equal(got["layers"][0][1], want["layers"][0][1])  # embedding, exact
    for name, a in got["layers"]:
        assert np.array_equal(oracle.bf16_round(a), a), name  # every stored tensor is BF16


def test_model_with_random_gammas_matches_brute(tiny_batch):
    w = oracle.Weights(TINY, 1)
    gam = {}
    for i, key in enumerate(list(w.gamma)):
        gam[key] = oracle.bf16_round(1.0 + 0.1 * random_normal(TINY["hidden"], 100 + i))
        w.gamma[key] = gam[key]
    want = brute.forward(TINY, 1, tiny_batch.ids, tiny_batch.lengths, rounding=False, gammas=gam)
    got = oracle.Oracle(TINY, w, rounding=False).forward(tiny_batch.ids, tiny_batch.lengths)
    assert oracle.nrms(got["out"], want["out"]) < 1e-5


@pytest.mark.parametrize("seed", range(8))
def test_marker_subset_equals_full_rows(tiny_weights, seed):
    """The marker path (last layer on the marker rows only, keys and values
    over every token) gives bitwise the full pass's rows: each row's products
    are the same sums whichever rows are in the matrix."""
    b = random_batch(TINY, 1 + seed % 4, 24, seed=6 + seed, len_lo=3,
                     markers_per_row=1 + seed % 5)
    o = oracle.Oracle(TINY, tiny_weights)
    full = o.forward(b.ids, b.lengths)
    sub = o.forward(b.ids, b.lengths, markers=b.markers)
    rows = full["row_off"][b.markers[:, 0]] + b.markers[:, 1]
    assert sub["out"].shape == (len(b.markers), TINY["hidden"])
    assert np.array_equal(sub["out"], full["out"][rows])


def test_nrms_closed_forms():
    """nRMS(g, o) = |g - o|_2 / |o|_2 in float64: a uniform relative error e
    gives |e| whatever o is; it is 0 for g = o, 1 for g = 0 and 2 for g = -o;
    it is invariant under a common scale; a hand example: g = (3, 5) against
    o = (3, 4) gives 1 / 5."""
    rng = np.random.default_rng(5)
    o = rng.standard_normal((37, 64)).astype(np.float32)
    for eps in (1e-3, -2.5e-2, 0.5):
        g = o.astype(np.float64) * (1.0 + eps)
        assert oracle.nrms(g, o) == pytest.approx(abs(eps), rel=1e-12)
    assert oracle.nrms(o, o) == 0.0
    assert oracle.nrms(np.zeros_like(o), o) == pytest.approx(1.0, rel=1e-15)
    assert oracle.nrms(-o, o) == pytest.approx(2.0, rel=1e-15)
    g = o + 0.01 * rng.standard_normal(o.shape).astype(np.float32)
    assert oracle.nrms(8.0 * g, 8.0 * o) == pytest.approx(oracle.nrms(g, o), rel=1e-12)
    assert oracle.nrms(np.array([3.0, 5.0]), np.array([3.0, 4.0])) == pytest.approx(0.2, rel=1e-15)
    assert oracle.nrms(np.zeros(3), np.zeros(3)) == 0.0
    assert oracle.nrms(np.ones(3), np.zeros(3)) == float("inf")


def test_layerwise_on_own_captures_reproduces_forward(tiny_weights):
    b = random_batch(TINY, 3, 24, seed=8, len_lo=4, markers_per_row=3)
    o = oracle.Oracle(TINY, tiny_weights)
    for mk in (None, b.markers):
        caps = dict(o.forward(b.ids, b.lengths, markers=mk, capture=True)["layers"])
        lw = o.forward_layerwise(b.ids, b.lengths, caps, markers=mk)
        assert list(lw) == o.layer_names()[1:]
        for name, y in lw.items():
            assert np.array_equal(y, caps[name]), name


def test_reversed_rows_and_padding_ids_do_not_change_outputs(tiny_weights):
    b = random_batch(TINY, 4, 20, seed=7, len_lo=3)
    o = oracle.Oracle(TINY, tiny_weights)
    a = o.forward(b.ids, b.lengths)
    ids2 = b.ids[::-1].copy()
    len2 = b.lengths[::-1].copy()
    for r in range(4):
        ids2[r, len2[r]:] = 50 + r  # different padding IDs
    c = o.forward(ids2, len2)
    for r in range(4):
        ra = slice(a["row_off"][r], a["row_off"][r + 1])
        rc = slice(c["row_off"][3 - r], c["row_off"][4 - r])
        assert oracle.nrms(a["out"][ra], c["out"][rc]) < 1e-3


# ------------------------------------------------------- planted mistakes ----

def _flip_rope(v, pos, cos, sin, rounding=True):
    return _orig_rope(v, pos, cos, -sin, rounding)


_orig_rope = omodel.rope_apply
_orig_kinds = omodel.layer_kinds
_orig_ln = omodel.layer_norm
_orig_gelu = omodel.gelu
_orig_attn = omodel.attention


def _kinds_off_by_one(cfg):
    k = _orig_kinds(cfg)
    out = []
    for i, (g, th) in enumerate(k):
        if i < cfg["n_enc_layers"]:
            g = (i + 1) % cfg["global_every"] == 0
            th = cfg["theta_global"] if g else cfg["theta_local"]
        out.append((g, th))
    return out


def _ln_unbiased(x, gamma, eps):
    n = x.shape[-1]
    return _orig_ln(x, gamma, eps) * np.float32(math.sqrt((n - 1) / n))


def _gelu_tanh(u):
    u = np.asarray(u, np.float64)
    return (0.5 * u * (1 + np.tanh(math.sqrt(2 / math.pi) * (u + 0.044715 * u ** 3)))).astype(np.float32)


def _attn_window_full(q, k, v, qp, kp, nh, hd, hw, rounding=True):
    return _orig_attn(q, k, v, qp, kp, nh, hd, None if hw is None else 2 * hw, rounding)


def _attn_no_scale(q, k, v, qp, kp, nh, hd, hw, rounding=True):
    return _orig_attn(q * np.float32(8.0), k, v, qp, kp, nh, hd, hw, rounding)


def _attn_swap_qk(q, k, v, qp, kp, nh, hd, hw, rounding=True):
    if q.shape == k.shape:
        return _orig_attn(k, q, v, qp, kp, nh, hd, hw, rounding)
    return _orig_attn(q, k, v, qp, kp, nh, hd, hw, rounding)


class _SwapGLU:
    def __init__(self, w, F):
        self.w, self.F = w, F
        self.gamma = w.gamma

    def f32(self, name):
        a = self.w.f32(name)
        if name.endswith(".wi"):
            return np.concatenate([a[self.F:], a[:self.F]])
        return a


MUTATIONS = {
    "rope_sign": ("rope_apply", _flip_rope),
    "global_layer_index": ("layer_kinds", _kinds_off_by_one),
    "ln_variance": ("layer_norm", _ln_unbiased),
    "gelu_form": ("gelu", _gelu_tanh),
    "window_width": ("attention", _attn_window_full),
    "attention_scale": ("attention", _attn_no_scale),
    "q_k_swapped": ("attention", _attn_swap_qk),
    "glu_halves": (None, None),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(mutation, tiny_batch, tiny_weights, brute_unrounded, monkeypatch):
    attr, fn = MUTATIONS[mutation]
    w = tiny_weights
    if attr is not None:
        monkeypatch.setattr(omodel, attr, fn)
    else:
        w = _SwapGLU(tiny_weights, TINY["ffn"])
    got = omodel.Oracle(TINY, w, rounding=False).forward(tiny_batch.ids, tiny_batch.lengths, capture=True)
    assert _max_layer_nrms(got, brute_unrounded) > UNROUNDED_BOUND


# ------------------------------------------------------- biased head variant --
# The decision layers as the biased head of "perf(model): exact Metal
# speed-ups of the forward pass": biased projections (bias added to the BF16
# product in the same precision), a 4x-wide plain-GELU FFN.

TINY_HEAD = dict(TINY, dec_head=1)


@pytest.fixture(scope="module")
def head_weights():
    return oracle.Weights(TINY_HEAD, 1)


@pytest.fixture(scope="module")
def head_brute_unrounded(tiny_batch):
    return brute.forward(TINY_HEAD, 1, tiny_batch.ids, tiny_batch.lengths, rounding=False,
                         capture=True)


def test_head_tensors_match_brute_generator(head_weights):
    H = TINY["hidden"]
    n_enc, NL = TINY["n_enc_layers"], TINY["n_enc_layers"] + TINY["n_dec_layers"]
    shapes = {n: sh for _, n, sh in oracle.tensor_shapes(TINY_HEAD)}
    assert shapes[f"L{n_enc}.w1"] == (4 * H, H) and shapes[f"L{n_enc}.w2"] == (H, 4 * H)
    assert shapes[f"L{NL - 1}.b1"] == (4 * H,)
    for tid, name, shape in oracle.tensor_shapes(TINY_HEAD):
        if name.split(".")[-1] in ("bqkv", "bo", "b1", "b2", "w1", "w2"):
            want = brute.weights_f64(1, tid, shape)
            assert np.array_equal(head_weights.f32(name).astype(np.float64), want), name


def test_head_variant_matches_brute_without_rounding(tiny_batch, head_weights,
                                                     head_brute_unrounded):
    got = oracle.Oracle(TINY_HEAD, head_weights, rounding=False).forward(
        tiny_batch.ids, tiny_batch.lengths, capture=True)
    assert _max_layer_nrms(got, head_brute_unrounded) < UNROUNDED_BOUND
    # and it is a different model than the GeGLU decision layers
    plain = brute.forward(TINY, 1, tiny_batch.ids, tiny_batch.lengths, rounding=False)
    assert oracle.nrms(got["out"], plain["out"]) > 1e-2


def test_head_variant_matches_brute_with_rounding(tiny_batch, head_weights):
    want = brute.forward(TINY_HEAD, 1, tiny_batch.ids, tiny_batch.lengths, rounding=True,
                         capture=True)
    got = oracle.Oracle(TINY_HEAD, head_weights).forward(tiny_batch.ids, tiny_batch.lengths,
                                                         capture=True)
    assert oracle.nrms(got["out"], want["out"]) < 5e-3
    for name, a in got["layers"]:
        assert np.array_equal(oracle.bf16_round(a), a), name


def test_head_variant_marker_subset_equals_full_rows(head_weights):
    b = random_batch(TINY_HEAD, 3, 24, seed=6, len_lo=10, markers_per_row=4)
    o = oracle.Oracle(TINY_HEAD, head_weights)
    full = o.forward(b.ids, b.lengths)
    sub = o.forward(b.ids, b.lengths, markers=b.markers)
    rows = full["row_off"][b.markers[:, 0]] + b.markers[:, 1]
    assert np.array_equal(sub["out"], full["out"][rows])


class _DropBias:
    """Planted mistake: one bias of the head left out."""

    def __init__(self, w, suffix):
        self.w, self.suffix = w, suffix
        self.gamma = w.gamma

    def f32(self, name):
        a = self.w.f32(name)
        return np.zeros_like(a) if name.endswith(self.suffix) else a


class _GatedHead:
    """Planted mistake: the head's FFN read as a GeGLU of two halves of W_1."""

    def __init__(self, w):
        self.w = w
        self.gamma = w.gamma

    def f32(self, name):
        a = self.w.f32(name)
        if name.endswith(".w1"):
            half = a.shape[0] // 2
            return np.concatenate([a[:half] * 0.5, a[half:]])
        return a


@pytest.mark.parametrize("mutation", ["b_qkv", "b_o", "b_1", "b_2", "ffn_halves"])
def test_head_planted_mistakes_are_caught(mutation, tiny_batch, head_weights,
                                          head_brute_unrounded):
    w = (_GatedHead(head_weights) if mutation == "ffn_halves"
         else _DropBias(head_weights, "." + mutation.replace("_", "")))
    got = omodel.Oracle(TINY_HEAD, w, rounding=False).forward(tiny_batch.ids, tiny_batch.lengths,
                                                              capture=True)
    assert _max_layer_nrms(got, head_brute_unrounded) > UNROUNDED_BOUND
