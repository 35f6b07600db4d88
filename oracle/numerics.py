"""Scalar building blocks of the CPU oracle: BF16 rounding, GELU, nRMS.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

BF16 is the storage format of every tensor of the forward pass (the encoder
and decision layers run in BF16, page "Run Laya encoder and decision layers
on CUDA", section Purpose); arithmetic between
two stored tensors happens in float32 and its result is rounded once, to
nearest-even, when it is stored again.
"""
from __future__ import annotations

import math

import numpy as np


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest BF16 value (ties to even).

    Returns float32 holding BF16-representable values.  NaN stays NaN (made
    quiet), overflow goes to +-inf, denormals are kept (no flush to zero).
    Adding 0x7FFF plus the lowest kept bit and truncating the low 16 bits is
    round-half-to-even on the bit pattern; it cannot wrap for non-NaN input.
    """
    f = np.array(x, dtype=np.float32, copy=True, order="C")
    u = f.view(np.uint32)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    if nan.any():
        orig = np.asarray(x, dtype=np.float32).view(np.uint32)
        u[nan] = (orig[nan] | np.uint32(0x00400000)) & np.uint32(0xFFFF0000)
    return f


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns (uint16) to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) of the RNE rounding of float32 values."""
    return (bf16_round(x).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def gelu(u: np.ndarray) -> np.ndarray:
    """GELU(z) = z * Phi(z) = 0.5 * z * (1 + erf(z / sqrt 2)), the exact (erf)
    form, written as 0.5 * z * erfc(-z / sqrt 2) so that the negative tail
    keeps its relative accuracy; evaluated in float64 (torch's CPU erfc) and
    returned as the nearest float32."""
    import torch

    z = torch.from_numpy(np.asarray(u, dtype=np.float64))
    g = 0.5 * z * torch.special.erfc(z * (-1.0 / math.sqrt(2.0)))
    return g.numpy().astype(np.float32)


def nrms(got: np.ndarray, ref: np.ndarray) -> float:
    """Normalised RMS error sqrt(sum (g - o)^2) / sqrt(sum o^2), in float64.

    The pages' parity limit is nRMS <= 0.005 ("[Performance]: Optimize native
    Rust/CUDA Laya inference #66", section Starting evidence).
    """
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    den = math.sqrt(float((o * o).sum()))
    num = math.sqrt(float(((g - o) ** 2).sum()))
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return num / den
