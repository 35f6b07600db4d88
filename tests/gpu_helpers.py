"""Helpers for the GPU tests: moving BF16 data between numpy and device
tensors, BF16 ulp distances, and the parity report file."""
import json
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def to_dev(a):
    """float32 numpy array of BF16 values -> contiguous torch.bfloat16 on cuda (exact)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).cuda()


def from_dev(t) -> np.ndarray:
    import torch
    return t.detach().cpu().to(torch.float32).numpy()


def bits_of(a: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in BF16 ulps between arrays of BF16 values (sign-magnitude aware)."""
    def ordered(x):
        u = bits_of(x).astype(np.int32)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a) - ordered(b))


def bf16_close(got: np.ndarray, want: np.ndarray, ulps: float = 1.0,
               floor_rel: float = 2.0 ** -16):
    """Element-wise check for float32-accumulated results stored as BF16.

    An element passes if it is within `ulps` BF16 ulps of the reference, or
    within floor_rel * rms(reference) of it: near zero the BF16 ulp shrinks
    without bound while the float32 summation error does not.  Returns
    (number of failing elements, fraction of elements not bitwise equal)."""
    g = np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    rms = float(np.sqrt(np.mean(w * w))) if w.size else 0.0
    mag = np.maximum(np.abs(w), 1e-38)
    ulp = np.exp2(np.floor(np.log2(mag)) - 7)
    allowed = np.maximum(ulps * ulp, floor_rel * rms)
    bad = int((np.abs(g - w) > allowed).sum())
    frac = float((bits_of(got) != bits_of(want)).mean()) if w.size else 0.0
    return bad, frac


def report(name: str, payload: dict):
    """Append a parity record to $LAYA_REPORT_DIR/parity_report.jsonl when
    that variable names an existing directory (no report otherwise)."""
    d = os.environ.get("LAYA_REPORT_DIR")
    if not d or not os.path.isdir(d):
        return
    with open(os.path.join(d, "parity_report.jsonl"), "a") as f:
        f.write(json.dumps({"test": name, **payload}) + "\n")


def ensure_built():
    from transformer_encoder_bf16_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from transformer_encoder_bf16_amd import build_lib
        build_lib.build()
    return binding.load()
