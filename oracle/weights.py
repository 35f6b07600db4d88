"""Synthetic model weights for the CPU oracle (counter-based, seeded).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The generator itself lives in ``oracle/csrc/oracle_weights.c`` (SplitMix64 ->
Irwin-Hall(12) -> 0.02 * z -> BF16); this module builds and loads it and
assembles the per-tensor arrays.

Tensor numbering (nn.Linear [out][in] layout everywhere):
  0              embedding            [vocab, hidden]
  1 + 4L + 0     W_qkv of layer L     [3*hidden, hidden]   rows [Q | K | V]
  1 + 4L + 1     W_o                  [hidden, hidden]
  1 + 4L + 2     W_i (GeGLU up)       [2*ffn, hidden]      rows [gelu half | gate half]
  1 + 4L + 3     W_o2 (down)          [hidden, ffn]
Layers 0 .. n_enc-1 are the encoder, n_enc .. n_enc+n_dec-1 the decision
layers.  Every LayerNorm gain is 1 and there are no biases (the stack is
"pre-LayerNorm (no bias)").

With cfg["dec_head"] = 1 the decision layers are the biased head variant
("perf(model): exact Metal speed-ups of the forward pass": biased
projections, a packed projection over every token, a 4x-wide FFN):
  1 + 4L + 2     W_1 (FFN in)         [4*hidden, hidden]
  1 + 4L + 3     W_2 (FFN out)        [hidden, 4*hidden]
and after all weight tensors, for decision layer d (layer L = n_enc + d):
  1 + 4*NL + 4d + 0   b_qkv  [3*hidden]
  1 + 4*NL + 4d + 1   b_o    [hidden]
  1 + 4*NL + 4d + 2   b_1    [4*hidden]
  1 + 4*NL + 4d + 3   b_2    [hidden]
(NL = n_enc + n_dec), drawn by the same generator as the weights.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from .numerics import bf16_bits_to_f32

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csrc", "oracle_weights.c")
_LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle's C helpers with gcc (OpenMP) into oracle/_build."""
    if force or not os.path.exists(_LIB_PATH):
        os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC",
                               "-o", tmp, _SRC])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            lib.oracle_splitmix64_at.restype = ctypes.c_uint64
            lib.oracle_splitmix64_at.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
            lib.oracle_irwin_hall.restype = ctypes.c_float
            lib.oracle_irwin_hall.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64]
            lib.oracle_weights_bf16.restype = None
            lib.oracle_weights_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint32,
                                                ctypes.c_uint64, ctypes.c_void_p]
            lib.oracle_fnv1a64.restype = ctypes.c_uint64
            lib.oracle_fnv1a64.argtypes = [ctypes.c_void_p, ctypes.c_uint64]
            _lib = lib
    return _lib


def splitmix64_at(seed: int, key: int) -> int:
    return int(_load().oracle_splitmix64_at(seed, key))


def irwin_hall(seed: int, tensor_id: int, idx: int) -> float:
    return float(_load().oracle_irwin_hall(seed, tensor_id, idx))


def tensor_shapes(cfg: dict) -> list:
    """[(tensor_id, name, shape)] in tensor-id order."""
    H, F = cfg["hidden"], cfg["ffn"]
    n_enc, n_dec = cfg["n_enc_layers"], cfg["n_dec_layers"]
    head = bool(cfg.get("dec_head", 0))
    NL = n_enc + n_dec
    out = [(0, "emb", (cfg["vocab"], H))]
    for L in range(NL):
        base = 1 + 4 * L
        if head and L >= n_enc:
            out += [(base + 0, f"L{L}.wqkv", (3 * H, H)),
                    (base + 1, f"L{L}.wo", (H, H)),
                    (base + 2, f"L{L}.w1", (4 * H, H)),
                    (base + 3, f"L{L}.w2", (H, 4 * H))]
        else:
            out += [(base + 0, f"L{L}.wqkv", (3 * H, H)),
                    (base + 1, f"L{L}.wo", (H, H)),
                    (base + 2, f"L{L}.wi", (2 * F, H)),
                    (base + 3, f"L{L}.wo2", (H, F))]
    if head:
        for d in range(n_dec):
            L, base = n_enc + d, 1 + 4 * NL + 4 * d
            out += [(base + 0, f"L{L}.bqkv", (3 * H,)),
                    (base + 1, f"L{L}.bo", (H,)),
                    (base + 2, f"L{L}.b1", (4 * H,)),
                    (base + 3, f"L{L}.b2", (H,))]
    return out


def tensor_bits(seed: int, tensor_id: int, shape) -> np.ndarray:
    """BF16 bits (uint16) of one tensor."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    _load().oracle_weights_bf16(seed, tensor_id, n, out.ctypes.data)
    return out.reshape(shape)


def fnv1a64(arr: np.ndarray) -> int:
    a = np.ascontiguousarray(arr)
    return int(_load().oracle_fnv1a64(a.ctypes.data, a.nbytes))


class Weights:
    """All tensors of one seeded model, kept as BF16 bits; ``f32(name)`` widens
    one tensor to float32 on demand (exact)."""

    def __init__(self, cfg: dict, seed: int):
        self.cfg = dict(cfg)
        self.seed = seed
        self.bits = {}
        for tid, name, shape in tensor_shapes(cfg):
            self.bits[name] = tensor_bits(seed, tid, shape)
        H = cfg["hidden"]
        n_layers = cfg["n_enc_layers"] + cfg["n_dec_layers"]
        # LayerNorm gains (float32, BF16-valued); all ones for the model.
        self.gamma = {f"L{L}.ln_attn": np.ones(H, np.float32) for L in range(n_layers)}
        self.gamma.update({f"L{L}.ln_ffn": np.ones(H, np.float32) for L in range(n_layers)})
        self.gamma["ln_enc_final"] = np.ones(H, np.float32)
        self.gamma["ln_dec_final"] = np.ones(H, np.float32)
        self._cache = {}

    def f32(self, name: str) -> np.ndarray:
        if name not in self._cache:
            self._cache[name] = bf16_bits_to_f32(self.bits[name])
        return self._cache[name]

    def drop_cache(self):
        self._cache.clear()

    def digest(self, name: str) -> int:
        return fnv1a64(self.bits[name])
