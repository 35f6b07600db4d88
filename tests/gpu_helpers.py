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


def report(name: str, payload: dict):
    """Append a parity record to <report dir>/parity_report.jsonl when the
    report directory exists (gpurun_out/ on a GPU run)."""
    d = os.environ.get("LAYA_REPORT_DIR", os.path.join(ROOT, "gpurun_out"))
    if not os.path.isdir(d):
        return
    with open(os.path.join(d, "parity_report.jsonl"), "a") as f:
        f.write(json.dumps({"test": name, **payload}) + "\n")


def ensure_built():
    from transformer_encoder_bf16_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from transformer_encoder_bf16_amd import build_lib
        build_lib.build()
    return binding.load()
