"""The C-ABI library on the CPU: it loads, exports every symbol its header
declares, and its host-only logic (validation, rotary tables) is right.  No
device compute happens here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from transformer_encoder_bf16_amd import binding as b
from transformer_encoder_bf16_amd.inputs import MODEL, TINY, WORKLOADS, make_batch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(b.LIB_PATH):
        from transformer_encoder_bf16_amd import build_lib
        build_lib.build()
    return b.load()


def test_exports_every_declared_symbol(lib):
    hdr = open(os.path.join(ROOT, "include", "laya_encoder.h")).read()
    declared = set(re.findall(r"^\s*(?:int|void|const char \*)\s*(laya_\w+)\s*\(", hdr, re.M))
    assert declared == set(b.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.laya_abi_version() == b.LAYA_ABI_VERSION == 6


def test_default_config_is_the_model(lib):
    d = b.default_config()
    for k, v in MODEL.items():
        assert d[k] == pytest.approx(v), k


@pytest.mark.parametrize("cfg", [MODEL, TINY, dict(MODEL, dec_head=1), dict(TINY, dec_head=1)])
def test_valid_configs(lib, cfg):
    assert b.validate_config(cfg) == b.LAYA_OK


@pytest.mark.parametrize("change,code", [
    (dict(head_dim=32, n_heads=32), b.LAYA_E_UNSUPPORTED),
    (dict(hidden=1000), b.LAYA_E_INVALID),
    (dict(hidden=960, n_heads=15), b.LAYA_E_UNSUPPORTED),
    (dict(hidden=1152, n_heads=18), b.LAYA_E_UNSUPPORTED),
    (dict(hidden=2048, n_heads=32), b.LAYA_E_UNSUPPORTED),
    (dict(ffn=2600), b.LAYA_E_UNSUPPORTED),
    (dict(max_batch=17), b.LAYA_E_UNSUPPORTED),
    (dict(max_seq=513), b.LAYA_E_UNSUPPORTED),
    (dict(max_markers=4096), b.LAYA_E_UNSUPPORTED),
    (dict(n_dec_layers=0), b.LAYA_E_INVALID),
    (dict(window=127), b.LAYA_E_UNSUPPORTED),
    (dict(vocab=0), b.LAYA_E_INVALID),
    (dict(ln_eps=0.0), b.LAYA_E_INVALID),
    (dict(max_graphs=0), b.LAYA_E_INVALID),
    (dict(workspace_budget_mib=0), b.LAYA_E_INVALID),
    (dict(dec_head=2), b.LAYA_E_INVALID),
    (dict(dec_head=-1), b.LAYA_E_INVALID),
])
def test_invalid_configs(lib, change, code):
    cfg = dict(MODEL)
    cfg.update(change)
    assert b.validate_config(cfg) == code


# split-capable tile shapes and the most K ranges each takes (laya_op_gemm)
SPLIT_MAX = {0: 8, 1: 8, 2: 8, 3: 8, 7: 8, 8: 8}


def _launchable(cfg_id, splits, K, epi, N, fused):
    if not 0 <= cfg_id <= 11 or splits < 1 or splits > K // 64:
        return False
    if splits > SPLIT_MAX.get(cfg_id, 1):
        return False
    if epi in (1, 2) and cfg_id == 0:
        return False
    if fused and (N > 1024 or cfg_id not in SPLIT_MAX):
        return False
    return True


@pytest.mark.parametrize("hidden", list(range(128, 1025, 128)))
def test_every_accepted_width_plans_launchable_gemms(lib, hidden):
    """Every hidden width the handle accepts: at every token count the pass
    can see, with and without markers, each planned GEMM launch is one the
    kernels support (tile shape, K split within the shape's limit, paired
    epilogues on paired shapes, the fused reduce + LayerNorm only on
    split-capable shapes and rows of at most 1024 values)."""
    cfg = dict(MODEL, hidden=hidden, n_heads=hidden // 64, ffn=(hidden * 41 // 16) // 64 * 64)
    assert b.validate_config(cfg) == b.LAYA_OK
    H, F = cfg["hidden"], cfg["ffn"]
    shapes = [(3 * H, H, 2), (H, H, 0), (F, H, 1), (H, F, 0)]
    marker = [(2 * H, H, 2), (H, H, 2), (H, H, 0), (F, H, 1), (H, F, 0)]
    T = 1
    while T <= cfg["max_batch"] * cfg["max_seq"]:
        lo, hi, plans = b.pass_plans(cfg, T, 96)
        assert lo == T
        for (cid, sp, fused), (N, K, epi) in zip(plans, shapes + marker):
            assert _launchable(cid, sp, K, epi, N, fused), (T, N, K, cid, sp, fused)
        T = hi + 1


def test_plans_are_the_planners_choice_for_the_exact_token_count(lib):
    """A pass over T live tokens uses the planner's plans for exactly T
    (laya_plan_gemm), reported with the maximal run of counts that share them
    (one captured graph serves such a run); runs split wherever any
    projection's plan changes, which includes the K-split thresholds; the
    splits of the marker layer are those of the full pass."""
    H, F = MODEL["hidden"], MODEL["ffn"]
    shapes = [(3 * H, H, 2), (H, H, 0), (F, H, 1), (H, F, 0)]
    edges = []
    prev = None
    T = 1
    while T <= 8192:
        lo, hi, plans = b.pass_plans(MODEL, T)
        assert lo == T
        for t in sorted({lo, hi, (lo + hi) // 2, min(hi, lo + 1)}):
            assert b.pass_plans(MODEL, t) == (lo, hi, plans), t
            assert [b.plan_gemm(t, N, K, e) for N, K, e in shapes] == \
                [(p[0], p[1]) for p in plans[:4]], t
        assert plans != prev  # maximal runs
        prev = plans
        _, _, with_markers = b.pass_plans(MODEL, hi, 37)
        assert with_markers[:4] == plans
        assert [p[1] for p in with_markers[4:]] == [plans[0][1], plans[0][1], plans[1][1],
                                                   plans[2][1], plans[3][1]]
        edges.append(hi)
        T = hi + 1
    for split_edge in (64, 256, 1024, 2048):
        assert split_edge in edges
    # every count, not only the samples above
    for t in range(1, 8193, 7):
        lo, hi, plans = b.pass_plans(MODEL, t)
        assert [b.plan_gemm(t, N, K, e) for N, K, e in shapes] == [(p[0], p[1]) for p in plans[:4]]
    # the configs' token counts
    assert b.pass_plans(MODEL, 48)[:2] == (1, 64)
    assert b.pass_plans(MODEL, 4050)[:2] == (3585, 4096)
    with pytest.raises(b.LayaError):
        b.pass_plans(MODEL, 0)
    with pytest.raises(b.LayaError):
        b.pass_plans(MODEL, 8193)


def test_plan_gemm_arguments(lib):
    """laya_plan_gemm is host-only and refuses shapes the GEMMs cannot run."""
    H = MODEL["hidden"]
    assert b.plan_gemm(48, 3 * H, H, 2) == b.pass_plans(MODEL, 48)[2][0][:2]
    for bad in ((0, H, H, 0), (1, 0, H, 0), (1, H, 100, 0), (1, H, H, 4), (1, H, H, -1)):
        with pytest.raises(b.LayaError):
            b.plan_gemm(*bad)


def test_abi_mismatch(lib):
    c = b.Config.from_dict(MODEL)
    c.abi_version = b.LAYA_ABI_VERSION + 1
    assert lib.laya_validate_config(ctypes.byref(c)) == b.LAYA_E_ABI


def test_run_args_validation(lib):
    batch = make_batch(MODEL, WORKLOADS["short_3"])
    ok = b.validate_run_args(MODEL, batch.ids, batch.lengths)
    assert ok == b.LAYA_OK
    # padding positions are not validated (any id there is fine)
    ids = batch.ids.copy()
    ids[0, batch.lengths[0]:] = -5
    if batch.lengths[0] < ids.shape[1]:
        assert b.validate_run_args(MODEL, ids, batch.lengths) == b.LAYA_OK
    bad = batch.ids.copy()
    bad[1, 0] = MODEL["vocab"]
    assert b.validate_run_args(MODEL, bad, batch.lengths) == b.LAYA_E_INVALID
    bad[1, 0] = -1
    assert b.validate_run_args(MODEL, bad, batch.lengths) == b.LAYA_E_INVALID
    ln = batch.lengths.copy()
    ln[2] = 0
    assert b.validate_run_args(MODEL, batch.ids, ln) == b.LAYA_E_INVALID
    ln[2] = batch.ids.shape[1] + 1
    assert b.validate_run_args(MODEL, batch.ids, ln) == b.LAYA_E_INVALID
    # markers
    mk = np.array([[0, 0], [3, int(batch.lengths[3]) - 1]], np.int32)
    assert b.validate_run_args(MODEL, batch.ids, batch.lengths, mk) == b.LAYA_OK
    mk2 = np.array([[0, int(batch.lengths[0])]], np.int32)
    assert b.validate_run_args(MODEL, batch.ids, batch.lengths, mk2) == b.LAYA_E_INVALID
    mk3 = np.array([[4, 0]], np.int32)
    assert b.validate_run_args(MODEL, batch.ids, batch.lengths, mk3) == b.LAYA_E_INVALID
    # limits: 16 rows, 512 tokens, 2048 markers
    big = np.zeros((17, 8), np.int32)
    assert b.validate_run_args(MODEL, big, np.full(17, 8)) == b.LAYA_E_INVALID
    long = np.zeros((1, 513), np.int32)
    assert b.validate_run_args(MODEL, long, np.array([513])) == b.LAYA_E_INVALID
    many = np.zeros((2049, 2), np.int32)
    assert b.validate_run_args(MODEL, np.zeros((1, 4), np.int32), np.array([4]), many) == b.LAYA_E_INVALID
    # the empty batch is valid
    assert b.validate_run_args(MODEL, np.zeros((0, 4), np.int32), np.zeros(0, np.int32)) == b.LAYA_OK


@pytest.mark.parametrize("theta", [MODEL["theta_global"], MODEL["theta_local"]])
def test_rope_tables_match_oracle(lib, theta):
    c_bits, s_bits = b.rope_table(theta, 512, 64)
    oc, os_ = oracle.rope_tables(theta, 512, 64)
    assert np.array_equal(c_bits, oracle.f32_to_bf16_bits(oc))
    assert np.array_equal(s_bits, oracle.f32_to_bf16_bits(os_))


def test_create_without_gpu_fails_cleanly(lib):
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is visible")
    except ImportError:
        pass
    c = b.Config.from_dict(TINY)
    h = ctypes.c_void_p()
    rc = lib.laya_encoder_create(ctypes.byref(c), 1, 0, ctypes.byref(h))
    assert rc == b.LAYA_E_DEVICE
    assert not h.value
    assert lib.laya_encoder_destroy(None) == b.LAYA_OK


def test_queue_and_health_reject_null_handles(lib):
    q = ctypes.c_void_p()
    assert lib.laya_queue_create(None, 32, 30000.0, ctypes.byref(q)) == b.LAYA_E_INVALID
    assert lib.laya_queue_health(None) == b.LAYA_E_INVALID
    assert lib.laya_queue_wait(None, 1, None, None) == b.LAYA_E_INVALID
    assert lib.laya_queue_destroy(None) == b.LAYA_OK
    assert lib.laya_encoder_health(None) == b.LAYA_E_INVALID
    assert lib.laya_encoder_inject_failure(None) == b.LAYA_E_INVALID


def test_gemm_layernorm_rejects_bad_arguments(lib):
    """The fused projection + residual + LayerNorm validates on the host before
    any device call (dummy aligned addresses are never dereferenced)."""
    P = ctypes.c_void_p
    A, W, x, n, g = P(0x1000), P(0x2000), P(0x3000), P(0x4000), P(0x5000)

    def call(M=48, N=1024, K=1024, config=7, splits=4, bias=None, x_=x, n_=n, eps=1e-5):
        return lib.laya_op_gemm_layernorm(None, A, K, W, K, x_, n_, g, M, N, K, config, splits,
                                          bias, eps)
    assert call(config=9, splits=1) == b.LAYA_E_INVALID  # whole K: not the ping-pong shape
    assert call(config=12, splits=1) == b.LAYA_E_INVALID  # no such shape
    assert call(splits=17) == b.LAYA_E_INVALID         # more ranges than 64-wide K pieces
    assert call(N=2048) == b.LAYA_E_INVALID            # one wave per row: N <= 1024
    assert call(config=4) == b.LAYA_E_INVALID          # whole-K-only tile shape
    assert call(n_=x) == b.LAYA_E_INVALID              # n must not alias x
    assert call(bias=P(0x6008)) == b.LAYA_E_INVALID    # bias must be 16-byte aligned
    assert call(K=1000) == b.LAYA_E_INVALID            # K a multiple of 64
    assert call(eps=0.0) == b.LAYA_E_INVALID
    assert call(M=0) == b.LAYA_OK                      # nothing to do, no device call
