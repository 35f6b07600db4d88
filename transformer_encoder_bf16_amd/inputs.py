"""Seeded synthetic inputs for the encoder forward pass.

This module draws random numbers and nothing else: it holds none of the
model's arithmetic, so both the HIP path and the CPU oracle can be fed the
very same arrays.  Everything here is plain data (model shapes, workload
shapes, seeds) plus numpy ``default_rng`` draws.

Model shapes: the synthetic Laya-sized encoder (hidden 1024, 16 heads of 64,
GeGLU inner width 2624, 28 encoder layers then 2 decision layers, vocab 50368, global
attention on every 3rd encoder layer with RoPE theta 160000, the others a
128-token window with theta 10000).  The pages describe the same stack, an
encoder of 28 layers followed by two decision layers, run in BF16 (page
"Run Laya encoder and decision layers on CUDA", section Purpose), and the
worker's limits of at most 16 rows, 512 tokens per row and 2048 markers
(page "Laya native CUDA worker", section Start and check).

Workload shapes follow the batch shapes the pages time (the table in the
Test Result section of "Run Laya encoder and decision layers on CUDA":
1x48, 4x64, 4x464, 16x512) plus the b=8, s=187, K=12 marker batch of
"perf(model): exact Metal speed-ups of the forward pass".
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

# Model dimensions.  Keys mirror the fields of the C ``laya_config`` struct.
MODEL = dict(
    vocab=50368,
    hidden=1024,
    n_heads=16,
    head_dim=64,
    ffn=2624,            # GeGLU inner width: Wi has 2*ffn rows, Wo2 has ffn columns
    n_enc_layers=28,
    n_dec_layers=2,
    global_every=3,      # encoder layer l is global iff l % global_every == 0
    window=128,          # local layers: |i - j| <= window // 2
    theta_global=160000.0,
    theta_local=10000.0,
    ln_eps=1e-5,
    max_batch=16,
    max_seq=512,
    max_markers=2048,
    max_graphs=4,              # captured graphs kept, LRU over shape keys
    workspace_budget_mib=512,  # the workspace must fit this
    dec_head=0,                # 1: biased head variant of the decision layers
)

# A tiny model of the same structure, for brute-force checks of the oracle and
# fast whole-model GPU checks.
TINY = dict(
    vocab=97,
    hidden=128,
    n_heads=2,
    head_dim=64,
    ffn=192,
    n_enc_layers=3,
    n_dec_layers=2,
    global_every=3,
    window=16,
    theta_global=160000.0,
    theta_local=10000.0,
    ln_eps=1e-5,
    max_batch=4,
    max_seq=64,
    max_markers=64,
    max_graphs=4,
    workspace_budget_mib=512,
    dec_head=0,
)

WEIGHT_SEED = 1


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int
    len_lo: int
    len_hi: int
    seed: int
    markers_per_row: int = 0


WORKLOADS = {
    "short_1": Workload("short_1", 1, 48, 48, 48, 11),
    "short_3": Workload("short_3", 4, 64, 16, 64, 13),
    "long_3": Workload("long_3", 4, 464, 400, 464, 23),
    "mixed_16": Workload("mixed_16", 16, 512, 64, 512, 31),
    "marker_subset": Workload("marker_subset", 8, 187, 187, 187, 41, 12),
}

# Further shapes the pages time: long_1 (one 464-token request, the H800
# comparison table of "Run Laya encoder and decision layers on CUDA") and a
# set of five single-request inputs (the recipe benchmark of the same page,
# section CUDA-event timings and reproduction, which does not list their
# lengths: here one request at each single-row length the pages use, 48, 64,
# 187, 464 and 512 tokens).
EXTRA_WORKLOADS = {
    "long_1": Workload("long_1", 1, 464, 464, 464, 17),
    "b1_48": Workload("b1_48", 1, 48, 48, 48, 51),
    "b1_64": Workload("b1_64", 1, 64, 64, 64, 52),
    "b1_187": Workload("b1_187", 1, 187, 187, 187, 53),
    "b1_464": Workload("b1_464", 1, 464, 464, 464, 54),
    "b1_512": Workload("b1_512", 1, 512, 512, 512, 55),
}
B1_SET = ("b1_48", "b1_64", "b1_187", "b1_464", "b1_512")
ALL_WORKLOADS = {**WORKLOADS, **EXTRA_WORKLOADS}


@dataclass
class Batch:
    """One right-padded batch: ``ids[B, S]`` (int32), ``lengths[B]`` (int32)
    and, optionally, ``markers[R, 2]`` (int32 pairs of (row, position))."""

    ids: np.ndarray
    lengths: np.ndarray
    markers: Optional[np.ndarray] = None

    @property
    def B(self) -> int:
        return int(self.ids.shape[0])

    @property
    def S(self) -> int:
        return int(self.ids.shape[1])

    @property
    def T(self) -> int:
        return int(self.lengths.sum())


def make_batch(model: dict, wl: Workload, pad_id: int = 0) -> Batch:
    """Draw one batch for workload ``wl`` with ``numpy.random.default_rng``.

    Lengths are uniform integers in [len_lo, len_hi] (inclusive), token IDs
    uniform in [0, vocab); padded positions hold ``pad_id``.  Markers (if any)
    are ``markers_per_row`` positions per row drawn without replacement from
    [0, len_b) and sorted ascending, listed row by row.
    """
    rng = np.random.default_rng(wl.seed)
    lengths = rng.integers(wl.len_lo, wl.len_hi + 1, size=wl.B).astype(np.int32)
    ids = rng.integers(0, model["vocab"], size=(wl.B, wl.S)).astype(np.int32)
    for b in range(wl.B):
        ids[b, lengths[b]:] = pad_id
    markers = None
    if wl.markers_per_row:
        rows = []
        for b in range(wl.B):
            p = np.sort(rng.choice(int(lengths[b]), size=wl.markers_per_row, replace=False))
            rows.extend((b, int(x)) for x in p)
        markers = np.asarray(rows, dtype=np.int32).reshape(-1, 2)
    return Batch(ids=ids, lengths=lengths, markers=markers)


def random_batch(model: dict, B: int, S: int, seed: int, len_lo: int = 1,
                 len_hi: Optional[int] = None, markers_per_row: int = 0) -> Batch:
    """An ad-hoc batch with the same recipe (used by tests at other shapes)."""
    wl = Workload("adhoc", B, S, len_lo, S if len_hi is None else len_hi, seed,
                  markers_per_row)
    return make_batch(model, wl)


def random_gamma(n: int, seed: int) -> np.ndarray:
    """LayerNorm gains ~ N(1, 0.1), rounded to BF16 by the consumer; used only by
    kernel unit tests (the model itself keeps every gain at 1)."""
    rng = np.random.default_rng(seed)
    return (1.0 + 0.1 * rng.standard_normal(n)).astype(np.float32)


def random_normal(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """Float32 N(0, scale^2) draws for kernel unit tests."""
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal(shape)).astype(np.float32)
