"""The forward pass of the encoder, written out plainly for the CPU oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed (the stack of page "Run Laya encoder and decision layers on
CUDA", section Purpose: a token embedding, the 28-layer encoder, then the two
decision layers, in BF16, the final hidden states kept for the scorer):

  x = Emb[id]                                          (exact copy)
  for every layer L (encoder 0..n_enc-1, then decision layers):
      n   = R(LN_attn(x))
      qkv = R(n W_qkv^T)                 columns [Q | K | V], head-major, 64 per head
      q,k = RoPE(q), RoPE(k)             V untouched (oracle/rope.py)
      o   = R(Attention(q, k, v))        bidirectional, key-padding mask, and on
                                         local layers |i - j| <= window/2
      x   = R(x + R(o W_o^T))
      n2  = R(LN_ffn(x))
      [u | g] = n2 W_i^T                 float32, not rounded
      h   = R(GELU(u) * g)
      x   = R(x + R(h W_o2^T))
      after the last encoder layer:  x = R(LN_enc_final(x))
  out = R(LN_dec_final(x))

With cfg["dec_head"] = 1 the decision layers are the biased head variant of
"perf(model): exact Metal speed-ups of the forward pass": every projection
adds a bias to its BF16 product in the same precision (the page's dense
layer is the matmul followed by x + b in the model dtype),
D(a, W, b) = R(R(a W^T) + b), and the FFN is 4x wide and not gated:
      qkv = D(n, W_qkv, b_qkv)     a = D(o, W_o, b_o)
      h   = R(GELU(D(n2, W_1, b_1)))      f = D(h, W_2, b_2)

R() is float32 -> BF16 round-to-nearest-even: every stored tensor is BF16,
every other intermediate is float32.  The QKV projection, the rotation and
attention as distinct steps follow "[RFC]: Native Laya inference with Rust and CUDA #14", section Design.
Encoder layer l is global iff l % global_every == 0; decision layers are
global; global layers use the theta_global table, local ones theta_local.
LayerNorm: mean and biased variance in float32 (two passes), eps 1e-5, gain
gamma, no bias.  Attention scale 1/sqrt(head_dim); softmax in float32 with
the row maximum subtracted.  Padding positions are never computed: tokens of
all rows are packed, and each query sees only the keys of its own row.

Marker rows ("perf(model): exact Metal speed-ups of the forward pass"): in
the last decision layer keys and values are needed for every token, while
queries, attention, the output projection and the FFN are needed only for
the marker rows; ``forward(..., markers=...)`` runs that layer only for the
marker rows, and ``forward`` without markers gives the full result whose
rows the subset must reproduce.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_round, gelu
from .rope import rope_apply, rope_tables


def pack(ids: np.ndarray, lengths: np.ndarray):
    """Packed token IDs, in-row positions and row offsets of a right-padded batch."""
    ids = np.asarray(ids)
    lengths = np.asarray(lengths, dtype=np.int64)
    B = ids.shape[0]
    row_off = np.zeros(B + 1, dtype=np.int64)
    row_off[1:] = np.cumsum(lengths)
    tok = np.concatenate([ids[b, :lengths[b]] for b in range(B)]) if B else np.zeros(0, np.int64)
    pos = np.concatenate([np.arange(lengths[b]) for b in range(B)]) if B else np.zeros(0, np.int64)
    return tok.astype(np.int64), pos.astype(np.int64), row_off


def layer_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) * gamma over the last axis, float32,
    with the biased variance of the centred values (two passes)."""
    x = np.asarray(x, dtype=np.float32)
    mu = np.mean(x, axis=-1, keepdims=True, dtype=np.float32)
    d = (x - mu).astype(np.float32)
    var = np.mean(d * d, axis=-1, keepdims=True, dtype=np.float32)
    return (d / np.sqrt(var + np.float32(eps)) * gamma).astype(np.float32)


def linear(a: np.ndarray, w: np.ndarray, accumulate: str = "float32") -> np.ndarray:
    """a [T, K] times w [N, K] transposed (nn.Linear without bias), returned in
    float32.  The sum is accumulated in float32 (the pass's stated precision)
    or, with accumulate="float64", in float64 and rounded once to float32: the
    same definition with a different accumulation error, used to measure how
    far two valid implementations of the BF16 pass drift apart.
    accumulate="chunk16" is a third valid order: the K range in consecutive
    pieces of 16, each piece's float32 sum added to a float32 running total
    in K order (the shape of a chain of 16-deep matrix-core steps)."""
    if accumulate == "float64":
        return np.matmul(np.asarray(a, np.float64), np.asarray(w, np.float64).T).astype(np.float32)
    a32, w32 = np.asarray(a, np.float32), np.asarray(w, np.float32)
    if accumulate == "chunk16":
        y = np.zeros((a32.shape[0], w32.shape[0]), np.float32)
        for k0 in range(0, a32.shape[1], 16):
            y += np.matmul(a32[:, k0:k0 + 16], w32[:, k0:k0 + 16].T)
        return y
    return np.matmul(a32, w32.T)


def attention(q, k, v, q_pos, k_pos, n_heads, head_dim, half_window, rounding=True):
    """Softmax attention of queries q [Tq, nh*d] over keys/values k, v [Tk, nh*d]
    of ONE sequence.  ``half_window`` None = global; otherwise key j is visible
    to query i iff |pos_i - pos_j| <= half_window.  Returns R(o) [Tq, nh*d]."""
    out = np.empty((q.shape[0], n_heads * head_dim), dtype=np.float32)
    scale = np.float32(1.0 / np.sqrt(head_dim))
    for h in range(n_heads):
        sl = slice(h * head_dim, (h + 1) * head_dim)
        s = np.matmul(q[:, sl], k[:, sl].T).astype(np.float32) * scale
        if half_window is not None:
            vis = np.abs(q_pos[:, None] - k_pos[None, :]) <= half_window
            s = np.where(vis, s, np.float32(-np.inf))
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m).astype(np.float32)
        p = e / e.sum(axis=1, keepdims=True, dtype=np.float32)
        out[:, sl] = np.matmul(p, v[:, sl])
    return bf16_round(out) if rounding else out


def layer_kinds(cfg: dict):
    """[(is_global, theta)] per layer: encoder layers first, then decision layers."""
    kinds = []
    for l in range(cfg["n_enc_layers"]):
        g = (l % cfg["global_every"]) == 0
        kinds.append((g, cfg["theta_global"] if g else cfg["theta_local"]))
    for _ in range(cfg["n_dec_layers"]):
        kinds.append((True, cfg["theta_global"]))
    return kinds


class Oracle:
    """The CPU oracle for one model configuration and one set of weights."""

    def __init__(self, cfg: dict, weights, rounding: bool = True, accumulate: str = "float32"):
        self.cfg = dict(cfg)
        self.w = weights
        self.rounding = rounding
        self.accumulate = accumulate
        hd = cfg["head_dim"]
        self.tables = {th: rope_tables(th, cfg["max_seq"], hd)
                       for th in {cfg["theta_global"], cfg["theta_local"]}}

    def R(self, x):
        return bf16_round(x) if self.rounding else np.asarray(x, dtype=np.float32)

    def lin(self, a, w):
        return linear(a, w, self.accumulate)

    # -- one layer -----------------------------------------------------------
    def layer(self, L: int, x: np.ndarray, pos: np.ndarray, row_off: np.ndarray,
              q_tok: np.ndarray | None = None) -> np.ndarray:
        """Run layer L on the packed residual stream x [T, H].  With ``q_tok``
        (token indices, grouped by row) only those rows leave the layer:
        keys and values still cover every token."""
        cfg, R = self.cfg, self.R
        H, nh, hd, F = cfg["hidden"], cfg["n_heads"], cfg["head_dim"], cfg["ffn"]
        is_global, theta = layer_kinds(cfg)[L]
        cos, sin = self.tables[theta]
        hw = None if is_global else cfg["window"] // 2
        eps = cfg["ln_eps"]
        g_attn = self.w.gamma[f"L{L}.ln_attn"]
        g_ffn = self.w.gamma[f"L{L}.ln_ffn"]
        wqkv = self.w.f32(f"L{L}.wqkv")
        head = bool(cfg.get("dec_head", 0)) and L >= cfg["n_enc_layers"]
        bias = (lambda name: self.w.f32(f"L{L}.{name}")) if head else (lambda name: None)
        bqkv = bias("bqkv")

        def dense(a, w, b):
            y = R(self.lin(a, w))
            return y if b is None else R(y + b)

        n = R(layer_norm(x, g_attn, eps))
        T = x.shape[0]
        if q_tok is None:
            qkv = dense(n, wqkv, bqkv)
            q = qkv[:, :H]
            kv = qkv[:, H:]
            q_pos = pos
            rows_q = [np.arange(row_off[b], row_off[b + 1]) for b in range(len(row_off) - 1)]
            x_q = x
        else:
            kv = dense(n, wqkv[H:], None if bqkv is None else bqkv[H:])
            q = dense(n[q_tok], wqkv[:H], None if bqkv is None else bqkv[:H])
            q_pos = pos[q_tok]
            x_q = x[q_tok]
            rows_q = []
            for b in range(len(row_off) - 1):
                rows_q.append(np.nonzero((q_tok >= row_off[b]) & (q_tok < row_off[b + 1]))[0])
        q = rope_apply(q.reshape(-1, nh, hd), q_pos, cos, sin, self.rounding).reshape(-1, H)
        k = rope_apply(kv[:, :H].reshape(T, nh, hd), pos, cos, sin, self.rounding).reshape(T, H)
        v = kv[:, H:]

        o = np.zeros((q.shape[0], H), dtype=np.float32)
        for b in range(len(row_off) - 1):
            qi = rows_q[b]
            if len(qi) == 0:
                continue
            ks = slice(row_off[b], row_off[b + 1])
            o[qi] = attention(q[qi], k[ks], v[ks], q_pos[qi], pos[ks], nh, hd, hw,
                              self.rounding)

        a = dense(o, self.w.f32(f"L{L}.wo"), bias("bo"))
        x1 = R(x_q + a)
        n2 = R(layer_norm(x1, g_ffn, eps))
        if head:
            h = R(gelu(dense(n2, self.w.f32(f"L{L}.w1"), bias("b1"))))
            f = dense(h, self.w.f32(f"L{L}.w2"), bias("b2"))
        else:
            ug = self.lin(n2, self.w.f32(f"L{L}.wi"))
            h = R(gelu(ug[:, :F]) * ug[:, F:])
            f = R(self.lin(h, self.w.f32(f"L{L}.wo2")))
        return R(x1 + f)

    def final_norm(self, x: np.ndarray, which: str) -> np.ndarray:
        """R(LN(x)) with the gain of "ln_enc_final" or "ln_dec_final"."""
        return self.R(layer_norm(x, self.w.gamma[which], self.cfg["ln_eps"]))

    # -- the whole pass ------------------------------------------------------
    def forward(self, ids, lengths, markers=None, capture: bool = False):
        """Returns {'out': [T or R, H] float32 BF16 values, 'row_off', 'pos',
        'layers': [(name, array)] when capture}."""
        cfg = self.cfg
        tok, pos, row_off = pack(ids, lengths)
        n_enc, n_dec = cfg["n_enc_layers"], cfg["n_dec_layers"]
        layers = []
        x = self.w.f32("emb")[tok]
        if capture:
            layers.append(("emb", x.copy()))
        q_tok = None
        if markers is not None:
            m = np.asarray(markers, dtype=np.int64).reshape(-1, 2)
            q_tok = row_off[m[:, 0]] + m[:, 1]
        n_layers = n_enc + n_dec
        for L in range(n_layers):
            last = L == n_layers - 1
            x = self.layer(L, x, pos, row_off, q_tok if last else None)
            if capture:
                name = f"enc{L:02d}" if L < n_enc else f"dec{L - n_enc}"
                layers.append((name, x.copy()))
            if L == n_enc - 1:
                x = self.final_norm(x, "ln_enc_final")
                if capture:
                    layers.append(("enc_final", x.copy()))
        out = self.final_norm(x, "ln_dec_final")
        if capture:
            layers.append(("out", out.copy()))
        return {"out": out, "row_off": row_off, "pos": pos, "tok": tok,
                "q_tok": q_tok, "layers": layers}

    def layer_names(self):
        n_enc, n_dec = self.cfg["n_enc_layers"], self.cfg["n_dec_layers"]
        names = ["emb"] + [f"enc{L:02d}" for L in range(n_enc)] + ["enc_final"]
        return names + [f"dec{L}" for L in range(n_dec)] + ["out"]

    def forward_layerwise(self, ids, lengths, inputs: dict, markers=None) -> dict:
        """Each step of the pass applied to a GIVEN input instead of the
        oracle's own previous output: for every captured name except "emb",
        the oracle's result of that one layer (or closing LayerNorm) when fed
        inputs[previous name].  Isolates the error each layer adds."""
        cfg = self.cfg
        tok, pos, row_off = pack(ids, lengths)
        n_enc, n_dec = cfg["n_enc_layers"], cfg["n_dec_layers"]
        q_tok = None
        if markers is not None:
            m = np.asarray(markers, dtype=np.int64).reshape(-1, 2)
            q_tok = row_off[m[:, 0]] + m[:, 1]
        names = self.layer_names()
        out = {}
        prev = "emb"
        L = 0
        for name in names[1:]:
            x = np.asarray(inputs[prev], dtype=np.float32)
            if name == "enc_final":
                out[name] = self.final_norm(x, "ln_enc_final")
            elif name == "out":
                out[name] = self.final_norm(x, "ln_dec_final")
            else:
                last = L == n_enc + n_dec - 1
                out[name] = self.layer(L, x, pos, row_off, q_tok if last else None)
                L += 1
            prev = name
        return out
