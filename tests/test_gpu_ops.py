"""Single-step parity of the HIP kernels against the CPU oracle (GPU only).

Each kernel is called through the C ABI (laya_op_*) on seeded inputs and
compared with the oracle element by element: bit-exact for the gather and
for RoPE, within one BF16 ulp (float32 summation order) for LayerNorm and the
GEMMs, within a small nRMS for attention (online softmax, and P carried into
the P V product as a BF16 head plus a BF16 tail).
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import bf16_close, bits_of, ensure_built, from_dev, report, to_dev, ulp_diff
from transformer_encoder_bf16_amd.inputs import random_gamma, random_normal

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    ensure_built()
    import torch
    torch.cuda.init()
    from transformer_encoder_bf16_amd import binding
    return binding


def _sync():
    import torch
    torch.cuda.synchronize()


# ------------------------------------------------------------------ gather ---

@pytest.mark.parametrize("T", [1, 37, 4096])
def test_gather_bit_exact(B, T):
    import torch
    emb_h = oracle.bf16_round(random_normal((1000, 1024), 1, 0.02))
    ids_h = np.random.default_rng(T).integers(0, 1000, T).astype(np.int32)
    ids_h[0] = 999
    emb = to_dev(emb_h)
    ids = torch.from_numpy(ids_h).cuda()
    out = torch.full((T, 1024), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.op_gather(emb, ids, out)
    _sync()
    assert np.array_equal(bits_of(from_dev(out)), bits_of(emb_h[ids_h]))


def test_gather_empty(B):
    import torch
    emb = torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.zeros((1, 128), dtype=torch.bfloat16, device="cuda")
    B.op_gather(emb, ids[:0], out[:0])
    _sync()


# --------------------------------------------------------------- layernorm ---

@pytest.mark.parametrize("T,H,resid", [(1, 1024, True), (7, 128, False), (130, 1024, True),
                                       (1000, 2048, True), (257, 384, False), (64, 1024, False),
                                       (3001, 1024, True), (2049, 512, False)])
def test_layernorm(B, T, H, resid):
    import torch
    x_h = oracle.bf16_round(random_normal((T, H), T + H, 2.0) + np.float32(0.3))
    r_h = oracle.bf16_round(random_normal((T, H), T + H + 1, 0.5)) if resid else None
    g_h = oracle.bf16_round(random_gamma(H, H))
    x = to_dev(x_h)
    r = to_dev(r_h) if resid else None
    n = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    g = torch.from_numpy(g_h).cuda()
    B.op_layernorm(x, r, n, g, 1e-5)
    _sync()
    xs = oracle.bf16_round(x_h + r_h) if resid else x_h
    assert np.array_equal(bits_of(from_dev(x)), bits_of(xs))  # residual sum: exact
    want = oracle.bf16_round(oracle.layer_norm(xs, g_h, 1e-5))
    got = from_dev(n)
    d = ulp_diff(got, want)
    assert d.max() <= 1
    assert (d > 0).mean() < 0.005
    report("layernorm", {"T": T, "H": H, "resid": resid, "max_ulp": int(d.max()),
                         "frac_diff": float((d > 0).mean())})


# -------------------------------------------------------------------- gemm ---

GEMM_SHAPES = [(1, 64, 64), (48, 1024, 1024), (130, 3072, 1024), (300, 1024, 2624),
               (257, 384, 128), (4096, 1024, 1024)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_plain(B, M, N, K):
    import torch
    a_h = oracle.bf16_round(random_normal((M, K), M + K))
    w_h = oracle.bf16_round(random_normal((N, K), N + K, 0.02))
    a, w = to_dev(a_h), to_dev(w_h)
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.op_gemm(a, w, c, M, N, K, 0)
    _sync()
    want = oracle.bf16_round(oracle.linear(a_h, w_h))
    got = from_dev(c)
    bad, frac = bf16_close(got, want)
    e = oracle.nrms(got, want)
    report("gemm", {"M": M, "N": N, "K": K, "bad": bad, "frac_diff": frac, "nrms": e})
    assert bad == 0, (M, N, K)
    assert frac < 0.01
    assert e < 1e-4


@pytest.mark.parametrize("M,F,K", [(1, 192, 128), (48, 2624, 1024), (333, 2624, 1024),
                                   (70, 64, 64)])
def test_gemm_geglu(B, M, F, K):
    import torch
    a_h = oracle.bf16_round(random_normal((M, K), M + F))
    w_h = oracle.bf16_round(random_normal((2 * F, K), F + K, 0.05))
    a, w = to_dev(a_h), to_dev(w_h)
    c = torch.full((M, F), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.op_gemm(a, w, c, M, F, K, 1)
    _sync()
    ug = oracle.linear(a_h, w_h)
    want = oracle.bf16_round(oracle.gelu(ug[:, :F]) * ug[:, F:])
    got = from_dev(c)
    bad, frac = bf16_close(got, want)
    e = oracle.nrms(got, want)
    report("gemm_geglu", {"M": M, "F": F, "K": K, "bad": bad, "frac_diff": frac, "nrms": e})
    assert bad == 0, (M, F, K)
    assert frac < 0.02
    assert e < 1e-4


def test_gelu_epilogue_across_its_range(B):
    """The GeGLU epilogue's GELU on BF16 values across [-12, 12] (u = one
    weight times 1, gate 1): within one BF16 ulp of bf16(GELU) evaluated in
    float64, and exact for nearly all, including the negative tail where
    GELU falls to ~1e-32 (the range where its value is a normal float32)."""
    import torch
    u = oracle.bf16_round(np.linspace(-12.0, 12.0, 8192).astype(np.float32))
    u = np.unique(u)
    F = (len(u) + 63) // 64 * 64
    u = np.concatenate([u, np.zeros(F - len(u), np.float32)])
    K, M = 64, 64
    a_h = np.zeros((M, K), np.float32)
    a_h[:, 0] = 1.0
    w_h = np.zeros((2 * F, K), np.float32)
    w_h[:F, 0] = u
    w_h[F:, 0] = 1.0
    c = torch.full((M, F), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.op_gemm(to_dev(a_h), to_dev(w_h), c, M, F, K, 1)
    _sync()
    got = from_dev(c)[0]
    want = oracle.bf16_round(oracle.gelu(u))
    d = ulp_diff(got, want)
    report("gelu_range", {"values": int(len(u)), "max_ulp": int(d.max()),
                          "frac_exact": float((d == 0).mean())})
    assert d.max() <= 1
    assert (d == 0).mean() > 0.99
    assert np.array_equal(from_dev(c)[1:], np.broadcast_to(got, (M - 1, F)))


def test_gemm_rejects_bad_shapes(B):
    import torch
    a = torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((64, 96), dtype=torch.bfloat16, device="cuda")
    c = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.LayaError):
        B.op_gemm(a, w, c, 4, 64, 96, 0)  # K not a multiple of 64


# -------------------------------------------------------------------- rope ---

ROPE_ROWS = [1, 2, 3, 5, 7, 8, 13, 16, 31, 32, 33, 48, 63, 64, 65, 100, 127, 128, 129, 160,
             187, 200, 255, 256, 257, 300, 333, 400, 464, 500, 511, 512, 600, 777, 1024, 1496,
             1715, 2048, 4050, 8192]
ROPE_HEADS = [1, 2, 16, 32]


@pytest.mark.parametrize("theta", [160000.0, 10000.0])
def test_rope_bit_exact_160_shapes(B, theta):
    """160 shapes (40 row counts x 4 head counts) per table, both tables: 320
    bit-exact comparisons, with the V block's bytes checked unchanged."""
    import torch
    cb, sb = B.rope_table(theta, 512, 64)
    ct = torch.from_numpy(cb.view(np.int16)).cuda()
    st = torch.from_numpy(sb.view(np.int16)).cuda()
    oc, os_ = oracle.rope_tables(theta, 512, 64)
    n_cmp = 0
    for rows in ROPE_ROWS:
        pos_h = np.random.default_rng(rows).integers(0, 512, rows).astype(np.int32)
        pos_h[0] = 0
        pos = torch.from_numpy(pos_h).cuda()
        for nrot in ROPE_HEADS:
            width = nrot * 64 + 128  # rotated heads, then an untouched "V" block
            buf_h = oracle.bf16_round(random_normal((rows, width), rows * 7 + nrot))
            want = oracle.rope_apply(buf_h[:, :nrot * 64].reshape(rows, nrot, 64), pos_h, oc, os_)
            # the optimized kernel and the original-geometry one, each on a fresh copy
            for original in (False, True):
                buf = to_dev(buf_h)
                B.op_rope(buf, nrot, pos, ct, st, original=original)
                _sync()
                got = from_dev(buf)
                assert np.array_equal(bits_of(got[:, :nrot * 64]),
                                      bits_of(want.reshape(rows, -1))), (theta, rows, nrot, original)
                assert np.array_equal(bits_of(got[:, nrot * 64:]), bits_of(buf_h[:, nrot * 64:]))
            n_cmp += 1
    assert n_cmp == 160
    report("rope", {"theta": theta, "shapes": n_cmp, "bit_exact": True})


# --------------------------------------------------------------- attention ---

KEY_LENGTHS = [1, 37, 48, 64, 65, 129, 187, 400, 464, 512]


def _attn_inputs(lengths, nh, seed):
    T = int(sum(lengths))
    row_off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q = oracle.bf16_round(random_normal((T, nh * 64), seed))
    kv = oracle.bf16_round(random_normal((T, 2 * nh * 64), seed + 1))
    return T, row_off, q, kv


def _vt_of(v, row_off, align=64, fill=float("nan")):
    """V transposed into the layout the QKV epilogue writes: row b's keys at
    columns vt_col0[b] .. (multiples of `align`); every other column holds
    `fill`, which the kernel must never let into an output."""
    import torch
    lens = np.diff(row_off)
    spans = (lens + align - 1) // align * align
    vcol0 = np.concatenate([[0], np.cumsum(spans)])[:-1].astype(np.int32)
    ld = int(vcol0[-1] + spans[-1])
    vt = torch.full((v.shape[1], ld), fill, dtype=torch.bfloat16, device="cuda")
    for b in range(len(lens)):
        vt[:, vcol0[b]:vcol0[b] + lens[b]] = v[row_off[b]:row_off[b + 1]].t()
    return vt, vcol0


def _attn_oracle(q, kv, row_off, nh, hw, q_tok=None):
    H = nh * 64
    k, v = kv[:, :H], kv[:, H:]
    B_ = len(row_off) - 1
    if q_tok is None:
        out = np.zeros_like(q)
        for b in range(B_):
            s = slice(row_off[b], row_off[b + 1])
            pos = np.arange(row_off[b + 1] - row_off[b])
            out[s] = oracle.attention(q[s], k[s], v[s], pos, pos, nh, 64, hw)
        return out
    out = np.zeros((len(q_tok), H), np.float32)
    for r, t in enumerate(q_tok):
        b = np.searchsorted(row_off, t, side="right") - 1
        s = slice(row_off[b], row_off[b + 1])
        pos = np.arange(row_off[b + 1] - row_off[b])
        out[r:r + 1] = oracle.attention(q[t:t + 1], k[s], v[s], np.array([t - row_off[b]]), pos,
                                        nh, 64, hw)
    return out


# Element-wise bound of the attention kernel against the oracle's float32
# softmax: every output within one BF16 ulp of the oracle's (or 2^-16 of the
# row block's rms, where the ulp shrinks near zero), none more than two ulps
# away, and nRMS <= 5e-4.  The kernel's only departures are the order of its
# float32 sums and a weight carried as a BF16 head plus a BF16 tail (about 16
# significant bits); a weight rounded to BF16 alone (~2e-3 nRMS), a dropped
# tail, a wrong scale or mask all break it.
ATTN_NRMS = 5e-4


def _attn_close(got, want):
    bad, frac = bf16_close(got, want, ulps=1.0, floor_rel=2.0 ** -16)
    # the ulp count where the ulp, not the near-zero floor, is the binding
    # tolerance (|want| at least 2^-8 of the block's rms)
    rms = float(np.sqrt(np.mean(np.asarray(want, np.float64) ** 2))) if want.size else 0.0
    big = np.abs(want) >= rms * 2.0 ** -8
    worst_ulp = int(ulp_diff(got[big], want[big]).max()) if big.any() else 0
    e = oracle.nrms(got, want)
    assert bad == 0 and worst_ulp <= 2 and e <= ATTN_NRMS, (bad, worst_ulp, e)
    return {"nrms": e, "max_ulp": worst_ulp, "frac_not_bitwise": frac}


@pytest.mark.parametrize("hw", [-1, 64])
@pytest.mark.parametrize("align", [64, 8])
def test_attention_against_oracle(B, hw, align):
    """Every key length, global and local; V^T rows packed at 64- or 8-aligned
    columns with NaN between them (a tile's tail then reads NaN or the next
    row's values, which must not reach the output)."""
    import torch
    nh = 4
    T, row_off, q_h, kv_h = _attn_inputs(KEY_LENGTHS, nh, 20 + hw)
    q, kv = to_dev(q_h), to_dev(kv_h)
    vt, vcol0 = _vt_of(kv[:, nh * 64:], row_off, align)
    o = torch.full((T, nh * 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.op_attention(q, kv[:, :nh * 64], vt, vcol0, o, nh, row_off, None, hw)
    _sync()
    got = from_dev(o)
    want = _attn_oracle(q_h, kv_h, row_off, nh, None if hw < 0 else hw)
    assert np.isfinite(got).all()
    stats = {}
    for b in range(len(KEY_LENGTHS)):
        s = slice(row_off[b], row_off[b + 1])
        stats[KEY_LENGTHS[b]] = _attn_close(got[s], want[s])
    report("attention", {"half_window": hw, "align": align, "per_length": stats})


@pytest.mark.parametrize("hw", [-1, 64])
@pytest.mark.parametrize("n_rows", [1, 2, 3, 96])
def test_attention_subset_rows_equal_full_rows(B, hw, n_rows):
    """Attention for a chosen list of query rows gives bitwise the same rows as
    attention for every query, with the key-padding row (and window) applied."""
    import torch
    nh = 2
    lens = [187, 37, 512, 64]
    T, row_off, q_h, kv_h = _attn_inputs(lens, nh, 40)
    q, kv = to_dev(q_h), to_dev(kv_h)
    k = kv[:, :nh * 64]
    vt, vcol0 = _vt_of(kv[:, nh * 64:], row_off)
    full = torch.empty((T, nh * 64), dtype=torch.bfloat16, device="cuda")
    B.op_attention(q, k, vt, vcol0, full, nh, row_off, None, hw)
    rng = np.random.default_rng(n_rows)
    per_row = []
    for b in range(len(lens)):
        cnt = min(lens[b], max(1, n_rows // len(lens) + (b < n_rows % len(lens))))
        per_row.append(np.sort(rng.choice(lens[b], cnt, replace=False)) + row_off[b])
    q_tok = np.concatenate(per_row)[:n_rows].astype(np.int32)
    qsub = q[torch.from_numpy(q_tok.astype(np.int64)).cuda()].contiguous()
    osub = torch.full((len(q_tok), nh * 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.op_attention(qsub, k, vt, vcol0, osub, nh, row_off, q_tok, hw)
    _sync()
    got = from_dev(osub)
    assert np.array_equal(bits_of(got), bits_of(from_dev(full)[q_tok]))
    want = _attn_oracle(q_h, kv_h, row_off, nh, None if hw < 0 else hw, q_tok)
    _attn_close(got, want)


def test_attention_single_row_honours_padding(B):
    """One query row of a short sequence in a batch of long ones only sees its
    own row's keys (the pages' fused single-query kernel ignored the mask)."""
    import torch
    nh = 2
    lens = [512, 37, 512]
    T, row_off, q_h, kv_h = _attn_inputs(lens, nh, 50)
    q, kv = to_dev(q_h), to_dev(kv_h)
    t = int(row_off[1] + 5)
    osub = torch.empty((1, nh * 64), dtype=torch.bfloat16, device="cuda")
    vt, vcol0 = _vt_of(kv[:, nh * 64:], row_off)
    B.op_attention(q[t:t + 1].contiguous(), kv[:, :nh * 64], vt, vcol0, osub, nh, row_off,
                   np.array([t], np.int32), -1)
    _sync()
    want = _attn_oracle(q_h, kv_h, row_off, nh, None, [t])
    _attn_close(from_dev(osub), want)


def test_attention_keys_outside_window_do_not_matter(B):
    import torch
    nh = 1
    lens = [400]
    T, row_off, q_h, kv_h = _attn_inputs(lens, nh, 60)
    q = to_dev(q_h)
    o1 = torch.empty((T, 64), dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty((T, 64), dtype=torch.bfloat16, device="cuda")
    kv = to_dev(kv_h)
    vt, vcol0 = _vt_of(kv[:, 64:], row_off)
    B.op_attention(q, kv[:, :64], vt, vcol0, o1, nh, row_off, None, 64)
    kv2_h = kv_h.copy()
    kv2_h[300:] = 5.0  # keys/values at positions >= 300
    kv2 = to_dev(kv2_h)
    vt2, _ = _vt_of(kv2[:, 64:], row_off)
    B.op_attention(q, kv2[:, :64], vt2, vcol0, o2, nh, row_off, None, 64)
    _sync()
    a, b = from_dev(o1), from_dev(o2)
    assert np.array_equal(bits_of(a[:236]), bits_of(b[:236]))  # queries < 236 never see key 300
    assert not np.array_equal(bits_of(a[236:]), bits_of(b[236:]))


# ------------------------------------------------- gemm tile shapes / split K --

@pytest.mark.parametrize("M,N,K,epi", [(48, 1024, 2624, 0), (200, 3072, 1024, 0),
                                       (97, 2624, 1024, 1), (300, 1024, 1024, 0)])
def test_gemm_every_tile_shape_and_split(B, M, N, K, epi):
    """All tile shapes give bitwise the same result for the same K split, and
    every split matches the oracle."""
    import torch
    a_h = oracle.bf16_round(random_normal((M, K), 7 * M + K))
    rows = 2 * N if epi else N
    w_h = oracle.bf16_round(random_normal((rows, K), 3 * N + K, 0.03))
    a, w = to_dev(a_h), to_dev(w_h)
    if epi:
        ug = oracle.linear(a_h, w_h)
        want = oracle.bf16_round(oracle.gelu(ug[:, :N]) * ug[:, N:])
    else:
        want = oracle.bf16_round(oracle.linear(a_h, w_h))
    for splits in (1, 2, 5):
        outs = []
        for cfg in range(12):
            if (epi and cfg == 0) or (splits > 1 and cfg in (4, 5, 6, 9, 10, 11)):
                continue
            c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
            B.op_gemm(a, w, c, M, N, K, epi, config=cfg, splits=splits)
            _sync()
            outs.append((cfg, bits_of(from_dev(c))))
        for cfg, o in outs[1:]:
            assert np.array_equal(o, outs[0][1]), (splits, cfg)
        got = (outs[0][1].astype(np.uint32) << 16).view(np.float32)
        bad, frac = bf16_close(got, want)
        assert bad == 0 and frac < 0.02, (splits, bad, frac)


@pytest.mark.parametrize("M,N,K,cfg,splits,bias", [
    (48, 1024, 1024, 7, 4, False), (48, 1024, 2624, 7, 8, False), (64, 1024, 2624, 0, 8, False),
    (200, 1024, 2624, 2, 4, False), (97, 1024, 4096, 8, 8, True), (33, 512, 1024, 3, 2, True),
    (1, 1024, 1024, 1, 3, False),
    # whole K: the residual add in the GEMM's store, every one-kernel tile shape
    (300, 1024, 1024, 3, 1, False), (300, 1024, 2624, 6, 1, False), (130, 512, 1024, 2, 1, True),
    (257, 1024, 1024, 5, 1, False), (100, 1024, 1024, 4, 1, True), (65, 1024, 1024, 0, 1, False),
    (48, 1024, 1024, 7, 1, False), (20, 1024, 1024, 8, 1, True), (5, 1024, 1024, 1, 1, False),
    (517, 1024, 2624, 6, 1, True), (300, 1024, 1024, 10, 1, False), (300, 1024, 1024, 11, 1, True)])
def test_gemm_layernorm_equals_gemm_then_layernorm(B, M, N, K, cfg, splits, bias):
    """The projection with the residual add and LayerNorm fused in (in the split's
    reduce launch, or in the whole-K GEMM's store followed by a LayerNorm of x
    alone) is bitwise the GEMM followed by the LayerNorm kernel, and matches the
    oracle."""
    import torch
    a_h = oracle.bf16_round(random_normal((M, K), 11 * M + K))
    w_h = oracle.bf16_round(random_normal((N, K), 5 * N + K, 0.03))
    x_h = oracle.bf16_round(random_normal((M, N), M + 3 * N, 1.5))
    g_h = oracle.bf16_round(random_gamma(N, N + 1))
    b_h = oracle.bf16_round(random_normal((N,), N + 7, 0.5)) if bias else None
    a, w, g = to_dev(a_h), to_dev(w_h), torch.from_numpy(g_h).cuda()
    bb = to_dev(b_h) if bias else None
    # reference: the GEMM into r, then the LayerNorm kernel on a copy of x
    r = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.op_gemm(a, w, r, M, N, K, 0, config=cfg, splits=splits, bias=bb)
    x_ref, n_ref = to_dev(x_h), torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    B.op_layernorm(x_ref, r, n_ref, g, 1e-5)
    x, n = to_dev(x_h), torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.op_gemm_layernorm(a, w, x, n, g, M, N, K, cfg, splits, bias=bb)
    _sync()
    assert np.array_equal(bits_of(from_dev(x)), bits_of(from_dev(x_ref)))
    assert np.array_equal(bits_of(from_dev(n)), bits_of(from_dev(n_ref)))
    # against the oracle: the product within one BF16 ulp (the biased product
    # has its own bound, pinned by the bias tests above), then the residual
    # and the LayerNorm of the GPU's own product
    if not bias:
        bad, frac = bf16_close(from_dev(r), oracle.bf16_round(oracle.linear(a_h, w_h)))
        assert bad == 0 and frac < 0.02, (bad, frac)
    xs = oracle.bf16_round(x_h + from_dev(r))
    assert np.array_equal(bits_of(from_dev(x)), bits_of(xs))
    d = ulp_diff(from_dev(n), oracle.bf16_round(oracle.layer_norm(xs, g_h, 1e-5)))
    assert d.max() <= 1 and (d > 0).mean() < 0.005
    report("gemm_layernorm", {"M": M, "N": N, "K": K, "config": cfg, "splits": splits,
                              "bias": bias, "max_ulp": int(d.max())})


def test_gemm_split_k_repeats_bitwise(B):
    """The split-K counters reset themselves: repeated launches agree bit for bit."""
    import torch
    M, N, K = 48, 3072, 1024
    a = to_dev(oracle.bf16_round(random_normal((M, K), 1)))
    w = to_dev(oracle.bf16_round(random_normal((N, K), 2, 0.02)))
    outs = []
    for _ in range(3):
        c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        B.op_gemm(a, w, c, M, N, K, 0, config=0, splits=8)
        _sync()
        outs.append(bits_of(from_dev(c)))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])


# ------------------------------------------------------- QKV epilogue (fused) --

@pytest.mark.parametrize("M,H,cfgs,splits", [(48, 128, (1, 2, 3, 7, 8), (1, 2, 5)),
                                             (300, 1024, (2, 3, 4, 5, 6, 7, 9, 10, 11), (1,)),
                                             (97, 256, (1, 2, 3, 7), (1, 4))])
def test_gemm_qkv_epilogue_equals_gemm_then_rope(B, M, H, cfgs, splits):
    """The QKV epilogue gives bitwise the plain GEMM followed by the RoPE
    kernel on the Q and K columns (which is bit-exact against the oracle), and
    V transposed to per-token columns, for every tile shape and K split."""
    import torch
    K, N = 1024, 3 * H
    a_h = oracle.bf16_round(random_normal((M, K), M + 5))
    w_h = oracle.bf16_round(random_normal((N, K), N + 7, 0.03))
    a, w = to_dev(a_h), to_dev(w_h)
    cb, sb = B.rope_table(160000.0, 512, 64)
    ct = torch.from_numpy(cb.view(np.int16)).cuda()
    st = torch.from_numpy(sb.view(np.int16)).cuda()
    rng = np.random.default_rng(M)
    pos_h = rng.integers(0, 512, M).astype(np.int32)
    pos = torch.from_numpy(pos_h).cuda()
    # V^T columns: a permutation with gaps, as packed rows with aligned starts
    vtok_h = (np.arange(M) + 3 * (np.arange(M) // 17)).astype(np.int32)
    vtok = torch.from_numpy(vtok_h).cuda()
    ldvt = int(vtok_h.max()) + 9
    for sp in splits:
        ref = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        B.op_gemm(a, w, ref, M, N, K, 0, config=cfgs[0], splits=sp)
        B.op_rope(ref, 2 * H // 64, pos, ct, st)
        _sync()
        ref_h = bits_of(from_dev(ref))
        if sp == 1:
            ref1 = ref_h
        for cfg in cfgs:
            c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
            vt = torch.full((H, ldvt), float("nan"), dtype=torch.bfloat16, device="cuda")
            B.op_gemm_qkv(a, w, c, M, N, K, pos, ct, st, 2 * H, vt, vtok, 2 * H, config=cfg,
                          splits=sp)
            _sync()
            got = bits_of(from_dev(c))
            assert np.array_equal(got[:, :2 * H], ref_h[:, :2 * H]), (cfg, sp)
            vt_h = bits_of(from_dev(vt))
            assert np.array_equal(vt_h[:, vtok_h].T, ref_h[:, 2 * H:]), (cfg, sp)
            assert np.isnan(from_dev(c)[:, 2 * H:]).all()  # V block of C not written
    # the rotated Q/K (split 1) against the oracle's RoPE of the plain GEMM's values
    plain = _plain(B, a, w, M, N, K, cfgs[0])
    want = oracle.rope_apply(plain[:, :2 * H].reshape(M, 2 * H // 64, 64), pos_h,
                             *oracle.rope_tables(160000.0, 512, 64))
    assert np.array_equal(bits_of(want.reshape(M, -1)), ref1[:, :2 * H])


def _plain(B, a, w, M, N, K, cfg):
    import torch
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    B.op_gemm(a, w, c, M, N, K, 0, config=cfg, splits=1)
    _sync()
    return from_dev(c)


# ------------------------------------- biased dense layers (decision head) --

def _f32_of(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("M,N,K", [(1, 512, 128), (48, 4096, 1024), (97, 1024, 4096),
                                   (300, 4096, 1024)])
def test_gemm_bias_and_bias_gelu_every_tile_shape(B, M, N, K):
    """For every tile shape and K split: epilogue 0 with a bias is bitwise
    bf16(plain + bias) of the same shape and split, and epilogue 3 is within
    one BF16 ulp of the oracle's GELU of that.  Against the oracle's biased
    dense layer from the inputs: the product may differ by one ulp of the
    product (summation order), which the bias addition carries over
    unchanged, so y is within ulp(product) + ulp(y) of the oracle's, and
    GELU (slope at most 1.13) keeps that."""
    import torch
    a_h = oracle.bf16_round(random_normal((M, K), 11 * M + K))
    w_h = oracle.bf16_round(random_normal((N, K), 5 * N + K, 0.03))
    b_h = oracle.bf16_round(random_normal((N,), N + 3, 0.5))
    a, w, bias = to_dev(a_h), to_dev(w_h), to_dev(b_h)
    p_or = oracle.bf16_round(oracle.linear(a_h, w_h))
    y_or = oracle.bf16_round(p_or + b_h)
    h_or = oracle.bf16_round(oracle.gelu(y_or))

    def ulp(x):
        return np.exp2(np.floor(np.log2(np.maximum(np.abs(x.astype(np.float64)), 2.0 ** -126))) - 7)

    # the product's tolerance is bf16_close's: one ulp, or 2^-16 of its rms
    y_tol = ulp(p_or) + 2.0 ** -16 * float(np.sqrt(np.mean(p_or.astype(np.float64) ** 2))) + ulp(y_or)
    h_tol = 1.13 * y_tol + ulp(h_or) + 2.0 ** -126
    worst = {"y": 0.0, "h": 0.0}
    for splits in (1, 2, 4):
        for cfg in range(12):
            if (splits > 1 and cfg in (4, 5, 6, 9, 10, 11)) or splits > K // 64:
                continue
            outs = {}
            for epi, bb in ((0, None), (0, bias), (3, bias)):
                c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
                B.op_gemm(a, w, c, M, N, K, epi, config=cfg, splits=splits, bias=bb)
                _sync()
                outs[(epi, bb is not None)] = bits_of(from_dev(c))
            plain = _f32_of(outs[(0, False)])
            y = _f32_of(outs[(0, True)])
            h = _f32_of(outs[(3, True)])
            bad, _ = bf16_close(plain, p_or)
            assert bad == 0, (cfg, splits)
            assert np.array_equal(bits_of(y), bits_of(oracle.bf16_round(plain + b_h))), (cfg, splits)
            assert ulp_diff(h, oracle.bf16_round(oracle.gelu(y))).max() <= 1, (cfg, splits)
            ey = np.abs(y.astype(np.float64) - y_or) / y_tol
            eh = np.abs(h.astype(np.float64) - h_or) / h_tol
            worst["y"] = max(worst["y"], float(ey.max()))
            worst["h"] = max(worst["h"], float(eh.max()))
            assert ey.max() <= 1.0 and eh.max() <= 1.0, (cfg, splits)
    report("gemm_bias", {"M": M, "N": N, "K": K, "worst_frac_of_bound": worst})


def test_gemm_bias_rules(B):
    import torch
    a = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((128, 64), dtype=torch.bfloat16, device="cuda")
    c = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    bias = torch.zeros(128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.LayaError):
        B.op_gemm(a, w, c, 4, 64, 64, 3)  # bias + GELU needs a bias
    with pytest.raises(B.LayaError):
        B.op_gemm(a, w, c, 4, 64, 64, 1, bias=bias)  # GeGLU takes none


@pytest.mark.parametrize("M,H,cfgs,splits", [(48, 128, (1, 2, 3, 7), (1, 2)),
                                             (300, 1024, (2, 3, 4, 5, 7, 10), (1,))])
def test_gemm_qkv_bias_equals_biased_gemm_then_rope(B, M, H, cfgs, splits):
    """With a bias the QKV epilogue equals the biased plain GEMM followed by
    the RoPE kernel, and V^T holds the biased V columns, bitwise."""
    import torch
    K, N = 1024, 3 * H
    a_h = oracle.bf16_round(random_normal((M, K), M + 15))
    w_h = oracle.bf16_round(random_normal((N, K), N + 17, 0.03))
    b_h = oracle.bf16_round(random_normal((N,), N + 19, 0.5))
    a, w, bias = to_dev(a_h), to_dev(w_h), to_dev(b_h)
    cb, sb = B.rope_table(160000.0, 512, 64)
    ct = torch.from_numpy(cb.view(np.int16)).cuda()
    st = torch.from_numpy(sb.view(np.int16)).cuda()
    pos_h = np.random.default_rng(M + 1).integers(0, 512, M).astype(np.int32)
    pos = torch.from_numpy(pos_h).cuda()
    vtok_h = (np.arange(M) + 5 * (np.arange(M) // 13)).astype(np.int32)
    vtok = torch.from_numpy(vtok_h).cuda()
    ldvt = int(vtok_h.max()) + 9
    for sp in splits:
        ref = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        B.op_gemm(a, w, ref, M, N, K, 0, config=cfgs[0], splits=sp, bias=bias)
        _sync()
        biased = bits_of(from_dev(ref))
        B.op_rope(ref, 2 * H // 64, pos, ct, st)
        _sync()
        ref_h = bits_of(from_dev(ref))
        for cfg in cfgs:
            c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
            vt = torch.full((H, ldvt), float("nan"), dtype=torch.bfloat16, device="cuda")
            B.op_gemm_qkv(a, w, c, M, N, K, pos, ct, st, 2 * H, vt, vtok, 2 * H, config=cfg,
                          splits=sp, bias=bias)
            _sync()
            got = bits_of(from_dev(c))
            assert np.array_equal(got[:, :2 * H], ref_h[:, :2 * H]), (cfg, sp)
            vt_h = bits_of(from_dev(vt))
            assert np.array_equal(vt_h[:, vtok_h].T, biased[:, 2 * H:]), (cfg, sp)
            # no rotation: the Q/K columns are the biased product itself
            c2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
            B.op_gemm_qkv(a, w, c2, M, N, K, pos, ct, st, 0, vt, vtok, 2 * H, config=cfg,
                          splits=sp, bias=bias)
            _sync()
            assert np.array_equal(bits_of(from_dev(c2))[:, :2 * H], biased[:, :2 * H])


# ------------------------------------------- 2-D XCD split of large grids --

@pytest.mark.parametrize("M,N,K,epi,cfgs", [(4049, 2624, 1024, 1, (3, 4, 5, 6, 9, 11, 10)),
                                            (4050, 3072, 1024, 0, (3, 5, 6, 9, 10, 11)),
                                            (2049, 4096, 1024, 0, (3, 6, 9)),
                                            (8192, 2624, 1024, 1, (6, 9))])
def test_gemm_two_dimensional_xcd_split_writes_every_tile(B, M, N, K, epi, cfgs):
    """Grids of >= 512 tiles take the 2-D split of the tile grid over the
    XCDs (a padded grid, tile blocks chosen on the device from the row
    count).  Every output element is written (the output starts as NaN),
    every tile shape gives the same bits, and the result is the oracle's
    within one BF16 ulp."""
    import torch
    a_h = oracle.bf16_round(random_normal((M, K), M + 3 * K))
    rows = 2 * N if epi else N
    w_h = oracle.bf16_round(random_normal((rows, K), N + 7, 0.03))
    a, w = to_dev(a_h), to_dev(w_h)
    if epi:
        ug = oracle.linear(a_h, w_h)
        want = oracle.bf16_round(oracle.gelu(ug[:, :N]) * ug[:, N:])
    else:
        want = oracle.bf16_round(oracle.linear(a_h, w_h))
    outs = []
    for cfg in cfgs:
        c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        B.op_gemm(a, w, c, M, N, K, epi, config=cfg, splits=1)
        _sync()
        got = from_dev(c)
        assert not np.isnan(got).any(), cfg
        outs.append(bits_of(got))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    bad, frac = bf16_close((outs[0].astype(np.uint32) << 16).view(np.float32), want)
    assert bad == 0, (bad, frac)
