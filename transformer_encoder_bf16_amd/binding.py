"""ctypes binding of liblaya_encoder.so (include/laya_encoder.h).

Argument marshalling only: every step of the forward pass runs in the HIP
library.  PyTorch, when used, supplies device memory and the HIP stream
handle; nothing here computes on the CPU.  If the library is missing the
loader raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblaya_encoder.so")

LAYA_ABI_VERSION = 6
LAYA_OK = 0
LAYA_E_INVALID = -1
LAYA_E_UNSUPPORTED = -2
LAYA_E_NOMEM = -3
LAYA_E_DEVICE = -4
LAYA_E_POISONED = -5
LAYA_E_ABI = -6
LAYA_E_BUSY = -7
LAYA_E_TIMEOUT = -8
LAYA_E_CANCELLED = -9
RUN_EAGER = 1
RUN_CAPTURE_LAYERS = 2
RUN_RESIDENT = 4
RUN_ROPE_STANDALONE = 8
RUN_ROPE_ORIGINAL = 16

ERROR_NAMES = {
    LAYA_E_INVALID: "LAYA_E_INVALID", LAYA_E_UNSUPPORTED: "LAYA_E_UNSUPPORTED",
    LAYA_E_NOMEM: "LAYA_E_NOMEM", LAYA_E_DEVICE: "LAYA_E_DEVICE",
    LAYA_E_POISONED: "LAYA_E_POISONED", LAYA_E_ABI: "LAYA_E_ABI", LAYA_E_BUSY: "LAYA_E_BUSY",
    LAYA_E_TIMEOUT: "LAYA_E_TIMEOUT", LAYA_E_CANCELLED: "LAYA_E_CANCELLED",
}

# Every symbol the header declares (checked by the CPU tests).
EXPORTS = [
    "laya_abi_version", "laya_config_init", "laya_validate_config", "laya_validate_run_args",
    "laya_pass_plans",
    "laya_plan_gemm",
    "laya_encoder_create", "laya_encoder_run", "laya_encoder_destroy",
    "laya_encoder_last_error", "laya_last_error", "laya_encoder_layer_output",
    "laya_encoder_weight_digest", "laya_encoder_weight", "laya_encoder_stats",
    "laya_encoder_profile", "laya_encoder_fill_workspace", "laya_encoder_config",
    "laya_encoder_health", "laya_encoder_inject_failure", "laya_queue_create", "laya_queue_submit",
    "laya_queue_wait", "laya_queue_health", "laya_queue_destroy", "laya_rope_table", "laya_memcpy", "laya_op_gather", "laya_op_layernorm", "laya_op_gemm",
    "laya_op_gemm_noalloc", "laya_op_gemm_layernorm", "laya_op_gemm_qkv", "laya_op_rope",
    "laya_op_rope_original",
    "laya_op_attention",
]


class LayaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32), ("vocab", ctypes.c_int32),
        ("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
        ("n_enc_layers", ctypes.c_int32), ("n_dec_layers", ctypes.c_int32),
        ("global_every", ctypes.c_int32), ("window", ctypes.c_int32),
        ("theta_global", ctypes.c_float), ("theta_local", ctypes.c_float),
        ("ln_eps", ctypes.c_float), ("max_batch", ctypes.c_int32),
        ("max_seq", ctypes.c_int32), ("max_markers", ctypes.c_int32),
        ("max_graphs", ctypes.c_int32), ("workspace_budget_mib", ctypes.c_int32),
        ("dec_head", ctypes.c_int32),
    ]

    @classmethod
    def from_dict(cls, d: dict) -> "Config":
        c = cls()
        c.abi_version = LAYA_ABI_VERSION
        for name, _ in cls._fields_:
            if name == "dec_head":
                c.dec_head = int(d.get("dec_head", 0))
            elif name != "abi_version":
                setattr(c, name, d[name])
        return c


class Output(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_void_p), ("rows", ctypes.c_int32),
                ("dim", ctypes.c_int32), ("row_off", ctypes.c_void_p)]


class OpTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 24), ("calls", ctypes.c_int32),
                ("total_ms", ctypes.c_double), ("flops", ctypes.c_double),
                ("bytes", ctypes.c_double)]


class Stats(ctypes.Structure):
    _fields_ = [("create_ms", ctypes.c_double), ("last_capture_ms", ctypes.c_double),
                ("graphs_cached", ctypes.c_int32), ("graph_evictions", ctypes.c_int32),
                ("launches_last_run", ctypes.c_int32),
                ("weight_bytes", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64)]


class GemmPlanC(ctypes.Structure):
    _fields_ = [("config", ctypes.c_int32), ("splits", ctypes.c_int32), ("fused", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m transformer_encoder_bf16_amd.build_lib`")
    lib = ctypes.CDLL(path)
    sig = {
        "laya_abi_version": (ctypes.c_int, []),
        "laya_config_init": (None, [ctypes.POINTER(Config)]),
        "laya_validate_config": (ctypes.c_int, [ctypes.POINTER(Config)]),
        "laya_pass_plans": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.c_int32,
                                           ctypes.c_int32, _I32P, _I32P,
                                           ctypes.POINTER(GemmPlanC), ctypes.c_int32, _I32P]),
        "laya_plan_gemm": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.POINTER(GemmPlanC)]),
        "laya_validate_run_args": (ctypes.c_int, [ctypes.POINTER(Config), _P, _P, ctypes.c_int32,
                                                  ctypes.c_int32, _P, ctypes.c_int32]),
        "laya_encoder_create": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.c_uint64,
                                               ctypes.c_int, ctypes.POINTER(_P)]),
        "laya_encoder_run": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P,
                                            ctypes.c_int32, ctypes.c_uint32,
                                            ctypes.POINTER(Output)]),
        "laya_encoder_destroy": (ctypes.c_int, [_P]),
        "laya_encoder_last_error": (ctypes.c_char_p, [_P]),
        "laya_last_error": (ctypes.c_char_p, []),
        "laya_encoder_layer_output": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.POINTER(Output),
                                                     ctypes.c_char_p, ctypes.c_size_t]),
        "laya_encoder_weight_digest": (ctypes.c_int, [_P, ctypes.c_int32,
                                                      ctypes.POINTER(ctypes.c_uint64)]),
        "laya_encoder_weight": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.POINTER(_P), _I32P,
                                               _I32P]),
        "laya_encoder_stats": (ctypes.c_int, [_P, ctypes.POINTER(Stats)]),
        "laya_encoder_fill_workspace": (ctypes.c_int, [_P, _P, ctypes.c_uint8]),
        "laya_encoder_config": (ctypes.c_int, [_P, ctypes.POINTER(Config)]),
        "laya_encoder_health": (ctypes.c_int, [_P]),
        "laya_encoder_inject_failure": (ctypes.c_int, [_P]),
        "laya_queue_create": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_double,
                                             ctypes.POINTER(_P)]),
        "laya_queue_submit": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P,
                                             ctypes.c_int32, _P, ctypes.c_size_t,
                                             ctypes.POINTER(ctypes.c_uint64)]),
        "laya_queue_wait": (ctypes.c_int, [_P, ctypes.c_uint64, _I32P,
                                           ctypes.POINTER(ctypes.c_double)]),
        "laya_queue_health": (ctypes.c_int, [_P]),
        "laya_queue_destroy": (ctypes.c_int, [_P]),
        "laya_encoder_profile": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                                _P, ctypes.c_int32, ctypes.c_uint32,
                                                ctypes.POINTER(OpTime),
                                                ctypes.c_int32, _I32P,
                                                ctypes.POINTER(ctypes.c_double)]),
        "laya_rope_table": (ctypes.c_int, [ctypes.c_float, ctypes.c_int32, ctypes.c_int32, _P,
                                           _P]),
        "laya_memcpy": (ctypes.c_int, [_P, _P, ctypes.c_size_t, ctypes.c_int32, _P]),
        "laya_op_gather": (ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int32, _P,
                                          ctypes.c_int32, _P]),
        "laya_op_layernorm": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_float]),
        "laya_op_gemm": (ctypes.c_int, [_P, _P, ctypes.c_int32, _P, ctypes.c_int32, _P,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, _P]),
        "laya_op_gemm_noalloc": (ctypes.c_int, [_P, _P, ctypes.c_int32, _P, ctypes.c_int32, _P,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, _P]),
        "laya_op_gemm_layernorm": (ctypes.c_int, [_P, _P, ctypes.c_int32, _P, ctypes.c_int32,
                                                  _P, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                  _P, ctypes.c_float]),
        "laya_op_rope": (ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        _P, _P, _P, ctypes.c_int32]),
        "laya_op_rope_original": (ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_int32, _P, _P, _P, ctypes.c_int32]),
        "laya_op_gemm_qkv": (ctypes.c_int, [_P, _P, ctypes.c_int32, _P, ctypes.c_int32, _P,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, _P, _P, _P, ctypes.c_int32, _P,
                                            ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, _P]),
        "laya_op_attention": (ctypes.c_int, [_P, _P, ctypes.c_int32, _P, ctypes.c_int32, _P,
                                             ctypes.c_int32, _P, _P, ctypes.c_int32,
                                             ctypes.c_int32, _P, ctypes.c_int32, _P,
                                             ctypes.c_int32, ctypes.c_int32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(rc: int, where: str, handle=None):
    if rc != LAYA_OK:
        lib = load()
        msg = lib.laya_encoder_last_error(handle) if handle else lib.laya_last_error()
        raise LayaError(rc, f"{where}: {msg.decode() if msg else ''}")


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def default_config() -> dict:
    c = Config()
    load().laya_config_init(ctypes.byref(c))
    return {name: getattr(c, name) for name, _ in Config._fields_ if name != "abi_version"}


def validate_config(cfg: dict) -> int:
    c = Config.from_dict(cfg)
    return load().laya_validate_config(ctypes.byref(c))


def pass_plans(cfg: dict, T: int, R: int = 0):
    """(t_first, t_last, [(config, splits, fused)]) of laya_pass_plans."""
    c = Config.from_dict(cfg)
    lo, hi, n = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    out = (GemmPlanC * 16)()
    _check(load().laya_pass_plans(ctypes.byref(c), T, R, ctypes.byref(lo), ctypes.byref(hi), out,
                                  16, ctypes.byref(n)), "laya_pass_plans")
    return lo.value, hi.value, [(out[i].config, out[i].splits, out[i].fused)
                                for i in range(min(n.value, 16))]


def plan_gemm(M: int, N: int, K: int, epilogue: int = 0):
    """(config, splits) that laya_op_gemm uses for exactly M rows."""
    out = GemmPlanC()
    _check(load().laya_plan_gemm(M, N, K, epilogue, ctypes.byref(out)), "laya_plan_gemm")
    return out.config, out.splits


def validate_run_args(cfg: dict, ids, lengths, markers=None) -> int:
    c = Config.from_dict(cfg)
    ids = _i32(ids)
    lengths = _i32(lengths)
    B = int(lengths.shape[0])
    S = int(ids.shape[1]) if ids.ndim == 2 else 0
    mk = None if markers is None else _i32(markers).reshape(-1, 2)
    R = 0 if mk is None else int(mk.shape[0])
    return load().laya_validate_run_args(ctypes.byref(c), _ptr(ids), _ptr(lengths), B, S,
                                         _ptr(mk), R)


def rope_table(theta: float, max_pos: int, head_dim: int = 64):
    """The library's rotary tables as BF16 bit arrays [max_pos, head_dim/2]."""
    c = np.empty((max_pos, head_dim // 2), np.uint16)
    s = np.empty_like(c)
    _check(load().laya_rope_table(theta, max_pos, head_dim, c.ctypes.data, s.ctypes.data),
           "laya_rope_table")
    return c, s


def copy_to_host(dev_ptr: int, nbytes: int, stream: int = 0) -> np.ndarray:
    out = np.empty(nbytes, np.uint8)
    if nbytes:
        _check(load().laya_memcpy(out.ctypes.data, dev_ptr, nbytes, 0, stream), "laya_memcpy")
    return out


def current_stream() -> int:
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


class Encoder:
    """One laya_encoder handle."""

    def __init__(self, cfg: Optional[dict] = None, seed: int = 1, device: int = 0):
        self.lib = load()
        self.cfg = dict(cfg) if cfg is not None else default_config()
        c = Config.from_dict(self.cfg)
        h = ctypes.c_void_p()
        _check(self.lib.laya_encoder_create(ctypes.byref(c), seed, device, ctypes.byref(h)),
               "laya_encoder_create")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            self.lib.laya_encoder_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    def run(self, ids, lengths, markers=None, flags: int = 0, stream: Optional[int] = None):
        """Queue one forward pass; returns an Output (device pointers)."""
        ids = _i32(ids)
        lengths = _i32(lengths)
        B = int(lengths.shape[0])
        S = int(ids.shape[1]) if ids.ndim == 2 and B else 0
        mk = None if markers is None else _i32(markers).reshape(-1, 2)
        R = 0 if mk is None else int(mk.shape[0])
        if flags & RUN_RESIDENT:
            ids = lengths = mk = None
        out = Output()
        st = current_stream() if stream is None else stream
        rc = self.lib.laya_encoder_run(self.handle, st, _ptr(ids), _ptr(lengths), B, S,
                                       _ptr(mk), R, flags, ctypes.byref(out))
        _check(rc, "laya_encoder_run", self.handle)
        return out

    def hidden(self, out: Output, stream: Optional[int] = None) -> np.ndarray:
        """Copy an output's BF16 rows to the host as float32 [rows, dim] (waits)."""
        n = out.rows * out.dim
        st = current_stream() if stream is None else stream
        raw = copy_to_host(out.hidden, n * 2, st).view(np.uint16)
        return (raw.astype(np.uint32) << 16).view(np.float32).reshape(out.rows, out.dim)

    def hidden_bits(self, out: Output, stream: Optional[int] = None) -> np.ndarray:
        n = out.rows * out.dim
        st = current_stream() if stream is None else stream
        return copy_to_host(out.hidden, n * 2, st).view(np.uint16).reshape(out.rows, out.dim)

    def layer_outputs(self, stream: Optional[int] = None):
        """[(name, float32 array)] of the last LAYA_RUN_CAPTURE_LAYERS run."""
        res = []
        i = 0
        name = ctypes.create_string_buffer(32)
        while True:
            o = Output()
            rc = self.lib.laya_encoder_layer_output(self.handle, i, ctypes.byref(o), name, 32)
            if rc != LAYA_OK:
                break
            res.append((name.value.decode(), self.hidden(o, stream)))
            i += 1
        return res

    def weight_digest(self, tensor_id: int) -> int:
        v = ctypes.c_uint64()
        _check(self.lib.laya_encoder_weight_digest(self.handle, tensor_id, ctypes.byref(v)),
               "laya_encoder_weight_digest", self.handle)
        return int(v.value)

    def weight_bits(self, tensor_id: int) -> np.ndarray:
        p = ctypes.c_void_p()
        r = ctypes.c_int32()
        c = ctypes.c_int32()
        _check(self.lib.laya_encoder_weight(self.handle, tensor_id, ctypes.byref(p),
                                            ctypes.byref(r), ctypes.byref(c)),
               "laya_encoder_weight", self.handle)
        return copy_to_host(p.value, r.value * c.value * 2, 0).view(np.uint16).reshape(
            r.value, c.value)

    def profile(self, ids, lengths, markers=None, stream: Optional[int] = None, flags: int = 0):
        """Per-op-class event times of one eager pass: ({name: {calls, ms, flops,
        bytes}}, total_ms)."""
        ids = _i32(ids)
        lengths = _i32(lengths)
        B = int(lengths.shape[0])
        S = int(ids.shape[1]) if ids.ndim == 2 and B else 0
        mk = None if markers is None else _i32(markers).reshape(-1, 2)
        R = 0 if mk is None else int(mk.shape[0])
        arr = (OpTime * 32)()
        n = ctypes.c_int32()
        tot = ctypes.c_double()
        st = current_stream() if stream is None else stream
        _check(self.lib.laya_encoder_profile(self.handle, st, _ptr(ids), _ptr(lengths), B, S,
                                             _ptr(mk), R, flags, arr, 32, ctypes.byref(n),
                                             ctypes.byref(tot)),
               "laya_encoder_profile", self.handle)
        res = {}
        for i in range(n.value):
            a = arr[i]
            res[a.name.decode()] = {"calls": a.calls, "ms": a.total_ms, "flops": a.flops,
                                    "bytes": a.bytes}
        return res, tot.value

    def fill_workspace(self, byte: int, stream: Optional[int] = None):
        """Diagnostic: every workspace byte set to `byte` (0xFF: NaN everywhere)."""
        st = current_stream() if stream is None else stream
        _check(self.lib.laya_encoder_fill_workspace(self.handle, st, byte),
               "laya_encoder_fill_workspace", self.handle)

    def health(self) -> int:
        """LAYA_OK, or LAYA_E_POISONED once a device failure stopped the handle."""
        return self.lib.laya_encoder_health(self.handle)

    def inject_failure(self):
        """Diagnostic: mark the handle failed (no device work)."""
        _check(self.lib.laya_encoder_inject_failure(self.handle), "laya_encoder_inject_failure",
               self.handle)

    def stats(self) -> dict:
        s = Stats()
        _check(self.lib.laya_encoder_stats(self.handle, ctypes.byref(s)), "laya_encoder_stats")
        return {name: getattr(s, name) for name, _ in Stats._fields_}


# ---------------------------------------------------------------- single steps
def _dp(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def op_gather(emb, ids, out, stream: Optional[int] = None):
    st = current_stream() if stream is None else stream
    _check(load().laya_op_gather(st, _dp(emb), emb.shape[0], emb.shape[1], _dp(ids),
                                 ids.shape[0], _dp(out)), "laya_op_gather")


def op_layernorm(x, r, n, gamma, eps: float, stream: Optional[int] = None):
    st = current_stream() if stream is None else stream
    _check(load().laya_op_layernorm(st, _dp(x), _dp(r), _dp(n), _dp(gamma), x.shape[0],
                                    x.shape[1], eps), "laya_op_layernorm")


def op_gemm(A, W, C, M: int, N: int, K: int, epilogue: int = 0, config: int = -1,
            splits: int = 1, bias=None, stream: Optional[int] = None):
    """C = bf16(A W^T) (epilogue 0, optionally + bias), GeGLU (1), or
    bias then GELU (3)."""
    st = current_stream() if stream is None else stream
    _check(load().laya_op_gemm(st, _dp(A), A.stride(0), _dp(W), W.stride(0), _dp(C),
                               C.stride(0), M, N, K, epilogue, config, splits, _dp(bias)),
           "laya_op_gemm")


def op_gemm_noalloc(A, W, C, M: int, N: int, K: int, epilogue: int = 0, config: int = -1,
                    splits: int = 1, bias=None, stream: Optional[int] = None):
    """op_gemm without any allocation (split-K partials in the library's own
    per-device buffer); queues only, does not synchronise."""
    st = current_stream() if stream is None else stream
    _check(load().laya_op_gemm_noalloc(st, _dp(A), A.stride(0), _dp(W), W.stride(0), _dp(C),
                                       C.stride(0), M, N, K, epilogue, config, splits, _dp(bias)),
           "laya_op_gemm_noalloc")


def op_gemm_layernorm(A, W, x, n, gamma, M: int, N: int, K: int, config: int, splits: int,
                      bias=None, eps: float = 1e-5, stream: Optional[int] = None):
    """x <- bf16(x + bf16(A W^T) [+ bias]), n <- LN(x) * gamma, on a K split whose
    reduce launch does the residual and the LayerNorm."""
    st = current_stream() if stream is None else stream
    _check(load().laya_op_gemm_layernorm(st, _dp(A), A.stride(0), _dp(W), W.stride(0), _dp(x),
                                         _dp(n), _dp(gamma), M, N, K, config, splits, _dp(bias),
                                         eps), "laya_op_gemm_layernorm")


def op_rope(buf, n_heads_rot: int, pos, cos_tab, sin_tab, rows: Optional[int] = None,
            stream: Optional[int] = None, original: bool = False):
    """RoPE in place; original=True runs the original-geometry kernel."""
    st = current_stream() if stream is None else stream
    fn = load().laya_op_rope_original if original else load().laya_op_rope
    _check(fn(st, _dp(buf), buf.stride(0), n_heads_rot, buf.shape[0] if rows is None else rows,
              _dp(pos), _dp(cos_tab), _dp(sin_tab), cos_tab.shape[0]),
           "laya_op_rope_original" if original else "laya_op_rope")


def op_gemm_qkv(A, W, C, M: int, N: int, K: int, pos, cos_tab, sin_tab, rope_cols: int,
                vt, vt_tok, vt_col0: int, config: int = -1, splits: int = 1, bias=None,
                stream: Optional[int] = None):
    """QKV projection with RoPE on columns [0, rope_cols) and columns
    [vt_col0, N) stored transposed into vt at columns vt_tok[m]."""
    st = current_stream() if stream is None else stream
    _check(load().laya_op_gemm_qkv(st, _dp(A), A.stride(0), _dp(W), W.stride(0), _dp(C),
                                   C.stride(0), M, N, K, _dp(pos), _dp(cos_tab), _dp(sin_tab),
                                   rope_cols, _dp(vt), 0 if vt is None else vt.stride(0),
                                   _dp(vt_tok), vt_col0, config, splits, _dp(bias)),
           "laya_op_gemm_qkv")


def op_attention(q, k, vt, vt_col0, o, n_heads: int, row_off, q_tok=None,
                 half_window: int = -1, stream: Optional[int] = None):
    """q, k, o: device tensors (2-D, row-major; k may be a column view of a
    wider buffer); vt: device [n_heads*64][ldvt] transposed values with row b's
    keys at columns vt_col0[b]...  row_off, vt_col0, q_tok: host int arrays."""
    st = current_stream() if stream is None else stream
    ro = _i32(row_off)
    vc = _i32(vt_col0)
    qt = None if q_tok is None else _i32(q_tok)
    _check(load().laya_op_attention(st, _dp(q), q.stride(0), _dp(k), k.stride(0), _dp(vt),
                                    vt.stride(0), _ptr(vc), _dp(o), o.stride(0), n_heads,
                                    _ptr(ro), len(ro) - 1, _ptr(qt),
                                    0 if qt is None else len(qt), half_window),
           "laya_op_attention")


class Queue:
    """The serial request queue over an Encoder (laya_queue_*): one worker
    runs whole requests in order; submit() copies a request and returns a
    ticket, wait() returns (status, hidden BF16 bits [rows, hidden], latency_ms)."""

    def __init__(self, enc: "Encoder", capacity: int = 32, deadline_ms: float = 30000.0):
        self.lib = load()
        self.enc = enc
        self.hidden = enc.cfg["hidden"] if hasattr(enc, "cfg") else None
        h = _P()
        _check(self.lib.laya_queue_create(enc.handle, capacity, deadline_ms, ctypes.byref(h)),
               "laya_queue_create")
        self.handle = h
        self._bufs = {}

    def submit(self, ids, lengths, markers=None, hidden: Optional[int] = None) -> int:
        """Queue one request; returns its ticket.  Raises LayaError (e.g.
        LAYA_E_BUSY when the queue is full)."""
        ids = _i32(ids)
        lengths = _i32(lengths)
        mk = None if markers is None else _i32(markers).reshape(-1, 2)
        B, S = ids.shape
        R = 0 if mk is None else mk.shape[0]
        rows = R if R else int(lengths.sum())
        hid = hidden or self.hidden
        buf = np.empty((rows, hid), dtype=np.uint16)
        t = ctypes.c_uint64()
        rc = self.lib.laya_queue_submit(self.handle, _ptr(ids), _ptr(lengths), B, S, _ptr(mk), R,
                                        buf.ctypes.data, buf.nbytes, ctypes.byref(t))
        if rc != LAYA_OK:
            raise LayaError(rc, "laya_queue_submit")
        self._bufs[t.value] = (buf, ids, lengths, mk)
        return t.value

    def wait(self, ticket: int):
        rows = ctypes.c_int32()
        lat = ctypes.c_double()
        rc = self.lib.laya_queue_wait(self.handle, ticket, ctypes.byref(rows), ctypes.byref(lat))
        buf = self._bufs.pop(ticket, (None,))[0]
        return rc, (buf[:rows.value] if rc == LAYA_OK else None), lat.value

    def health(self) -> int:
        return self.lib.laya_queue_health(self.handle)

    def close(self):
        if self.handle:
            self.lib.laya_queue_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
