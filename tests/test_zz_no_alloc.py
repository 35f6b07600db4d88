"""The allocation-free GEMM entry point (laya_op_gemm_noalloc) against
laya_op_gemm, through the C ABI (GPU only).

Its callers are code that cannot allocate device memory (graph capture,
serving loops, harnesses that forbid allocation).  Two calls in a row, the
second with fewer rows, each bitwise equal to laya_op_gemm with the same
arguments, with and without a K split (the split's partials live in the
library's own per-device buffer, which the second call reuses); a split
needing more than that buffer is refused before any device work."""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import bits_of, ensure_built, from_dev, to_dev
from transformer_encoder_bf16_amd.inputs import random_normal

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    ensure_built()
    import torch
    torch.cuda.init()
    from transformer_encoder_bf16_amd import binding
    return binding


def _pair(B, M, N, K, epi, cfg, splits, seed):
    import torch
    a_h = oracle.bf16_round(random_normal((M, K), seed))
    rows = 2 * N if epi == 1 else N
    w_h = oracle.bf16_round(random_normal((rows, K), seed + 1, 0.03))
    bias = to_dev(oracle.bf16_round(random_normal((N,), seed + 2, 0.5))) if epi == 3 else None
    a, w = to_dev(a_h), to_dev(w_h)
    ref = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    got = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.op_gemm(a, w, ref, M, N, K, epi, config=cfg, splits=splits, bias=bias)
    B.op_gemm_noalloc(a, w, got, M, N, K, epi, config=cfg, splits=splits, bias=bias)
    torch.cuda.synchronize()
    return bits_of(from_dev(ref)), bits_of(from_dev(got))


@pytest.mark.parametrize("first,second", [
    ((300, 1024, 2624, 0, 2, 4), (48, 2624, 1024, 1, 7, 4)),
    ((257, 1024, 1024, 0, 7, 8), (64, 1024, 2624, 3, 0, 8)),
    ((200, 3072, 1024, 0, -1, 1), (37, 1024, 1024, 0, 3, 2)),
])
def test_noalloc_gemm_equals_gemm_twice(B, first, second):
    for i, (M, N, K, epi, cfg, splits) in enumerate((first, second)):
        ref, got = _pair(B, M, N, K, epi, cfg, splits, 100 * i + M)
        assert not np.isnan((ref.astype(np.uint32) << 16).view(np.float32)).any()
        assert np.array_equal(ref, got), (i, M, N, K, epi, cfg, splits)


def test_noalloc_gemm_refuses_oversized_split(B):
    import torch
    M, N, K = 2048, 3072, 1024
    a = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    c = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.LayaError) as ei:
        B.op_gemm_noalloc(a, w, c, M, N, K, 0, config=3, splits=8)
    assert ei.value.code == B.LAYA_E_INVALID
