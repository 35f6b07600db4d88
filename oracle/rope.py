"""Rotary position embedding for the CPU oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Tables.  The pages keep four rotary tables -- global and local, cos and sin --
whose entries carry the BF16 rounding of the official model (exported once
with that rounding and then fixed: page "Laya native CUDA worker", section
Prepare the checkpoint and bundle; one table pair for the global layers and
one for the local ones: page "[Performance]: Optimize native Rust/CUDA Laya
inference #66", section Starting evidence).  Reading taken here: the angle of pair i at
position p is p * theta^(-2i/d) with d = head_dim; cos and sin are evaluated
in float64 and rounded once to BF16 (nearest even).  Positions run 0..511
(the 512-token maximum of the issue's section Recorded baseline and
environment).

Rotation.  Pairs are (i, i + d/2) ("rotate half").  For one head vector v of
length d, with x = v[i], y = v[i + d/2] and c, s the table entries of the
token's position:
    v[i]       <- bf16( fl32(x*c - y*s) )
    v[i + d/2] <- bf16( fl32(y*c + x*s) )
Both products of BF16 values are exact in float32, so the only roundings are
the float32 difference/sum and the BF16 store.  Only query and key heads are
rotated; value bytes are left as they were (V's bytes kept, section
Starting evidence of the same issue).
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_round


def rope_tables(theta: float, max_pos: int, head_dim: int):
    """(cos, sin) tables, float32 arrays [max_pos, head_dim // 2] of BF16 values."""
    half = head_dim // 2
    p = np.arange(max_pos, dtype=np.float64)[:, None]
    i = np.arange(half, dtype=np.float64)[None, :]
    inv_freq = np.power(np.float64(theta), -2.0 * i / head_dim)
    ang = p * inv_freq
    return f64_to_bf16(np.cos(ang)), f64_to_bf16(np.sin(ang))


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values straight to the nearest BF16 value (ties to even),
    with no intermediate float32 step.  Returned as float32 (exact).

    x = m * 2^e with 0.5 <= |m| < 1; m * 256 is exact in float64 and np.rint
    rounds it half-to-even to the 8-bit significand of BF16.  Valid for zero
    and for |x| in BF16's normal range, which covers every cos/sin entry.
    """
    x = np.asarray(x, dtype=np.float64)
    nz = x[x != 0]
    if nz.size and np.abs(nz).min() < 2.0 ** -126:
        raise ValueError("value below the BF16 normal range")
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8).astype(np.float32)


def rope_apply(v: np.ndarray, pos: np.ndarray, cos: np.ndarray, sin: np.ndarray,
               rounding: bool = True) -> np.ndarray:
    """Rotate head vectors ``v`` [T, n_heads, d] (float32, BF16 values) at
    positions ``pos`` [T]; returns a new array."""
    d = v.shape[-1]
    half = d // 2
    c = cos[pos][:, None, :]
    s = sin[pos][:, None, :]
    x = v[..., :half]
    y = v[..., half:]
    xn = (x * c - y * s).astype(np.float32)
    yn = (y * c + x * s).astype(np.float32)
    out = np.concatenate([xn, yn], axis=-1)
    return bf16_round(out) if rounding else out
