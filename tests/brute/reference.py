"""A float64 brute-force definition of the encoder pass, for tiny shapes only.

This is written separately from ``oracle/`` and shares no code with it; its
only purpose is to pin the oracle.  It formulates each step differently from
the oracle on purpose:
  * weights: SplitMix64 on numpy uint64 arrays (wrap-around arithmetic);
  * BF16 rounding: torch's float32 -> bfloat16 conversion (RNE), and for the
    rotary tables a nearest-neighbour search in float64;
  * RoPE: multiplication by the complex number c + i s;
  * attention: one big masked score matrix over all packed tokens, with the
    mask "same row and (global or |i - j| <= window/2)", and a per-query loop;
  * GELU: z * Phi(z) with scipy's normal CDF;
  * LayerNorm: numpy's var in float64.
With ``rounding=False`` every intermediate stays float64; with
``rounding=True`` values are rounded (via float32) to BF16 at the same tensor
boundaries the pass stores.
"""
from __future__ import annotations

import numpy as np
import torch
from scipy.special import ndtr

GOLD = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)


def _mix(z):
    z = (z ^ (z >> np.uint64(30))) * M1
    z = (z ^ (z >> np.uint64(27))) * M2
    return z ^ (z >> np.uint64(31))


def weights_f64(seed: int, tensor_id: int, shape) -> np.ndarray:
    n = int(np.prod(shape))
    idx = np.arange(n, dtype=np.uint64)
    total = np.zeros(n, dtype=np.int64)
    with np.errstate(over="ignore"):
        for j in range(3):
            key = (np.uint64(tensor_id) << np.uint64(40)) | (np.uint64(3) * idx + np.uint64(j))
            r = _mix(np.uint64(seed) + (key + np.uint64(1)) * GOLD)
            for q in range(4):
                total += ((r >> np.uint64(16 * q)) & np.uint64(0xFFFF)).astype(np.int64)
    z = (total.astype(np.float64) - 393210.0) / 65536.0
    w32 = (np.float32(0.02) * z.astype(np.float32)).astype(np.float32)
    return bf16(w32).reshape(shape)


def bf16(x) -> np.ndarray:
    """Float64 array of the BF16 rounding of float32(x) (torch's RNE conversion)."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32).copy())
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def bf16_direct(v: np.ndarray) -> np.ndarray:
    """Nearest BF16 value to each float64 value (ties to even mantissa): the
    BF16 value obtained by truncating float32(x) and its two neighbours are
    compared with x in float64, where those differences are exact."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    for k, x in np.ndenumerate(v):
        if x == 0.0:
            out[k] = 0.0
            continue
        base = int(np.array([x], dtype=np.float32).view(np.uint32)[0]) & 0xFFFF0000
        best = None
        for step in (-1, 0, 1):
            bits = base + step * 0x10000
            c = float(np.array([bits], dtype=np.uint32).view(np.float32)[0])
            key = (abs(c - x), (bits >> 16) & 1)
            if best is None or key < best[0]:
                best = (key, c)
        out[k] = best[1]
    return out


def rope_table(theta: float, max_pos: int, d: int):
    half = d // 2
    ang = np.array([[p * theta ** (-2.0 * i / d) for i in range(half)] for p in range(max_pos)])
    return bf16_direct(np.cos(ang)), bf16_direct(np.sin(ang))


def forward(cfg: dict, seed: int, ids, lengths, rounding: bool = True, capture: bool = False,
            gammas: dict | None = None):
    H, nh, d, F = cfg["hidden"], cfg["n_heads"], cfg["head_dim"], cfg["ffn"]
    n_enc, n_dec = cfg["n_enc_layers"], cfg["n_dec_layers"]
    R = (lambda a: bf16(a)) if rounding else (lambda a: np.asarray(a, np.float64))
    gam = gammas or {}

    def g(name):
        return np.asarray(gam.get(name, np.ones(H)), dtype=np.float64)

    # packed tokens and bookkeeping
    toks, rows, poss = [], [], []
    for b, L in enumerate(lengths):
        for p in range(int(L)):
            toks.append(int(ids[b][p]))
            rows.append(b)
            poss.append(p)
    rows = np.array(rows)
    poss = np.array(poss)
    T = len(toks)

    emb = weights_f64(seed, 0, (cfg["vocab"], H))
    x = emb[np.array(toks, dtype=np.int64)]
    caps = [("emb", x.copy())]

    def ln(v, gamma):
        mu = v.mean(axis=1, keepdims=True)
        var = v.var(axis=1, keepdims=True)
        return (v - mu) / np.sqrt(var + cfg["ln_eps"]) * gamma

    tables = {}
    for L in range(n_enc + n_dec):
        is_global = L >= n_enc or L % cfg["global_every"] == 0
        theta = cfg["theta_global"] if is_global else cfg["theta_local"]
        if theta not in tables:
            tables[theta] = rope_table(theta, cfg["max_seq"], d)
        c, s = tables[theta]
        head = bool(cfg.get("dec_head", 0)) and L >= n_enc
        NL = n_enc + n_dec
        wqkv = weights_f64(seed, 1 + 4 * L, (3 * H, H))
        wo = weights_f64(seed, 2 + 4 * L, (H, H))
        if head:
            # biased head layer: 4x-wide plain-GELU FFN, biases after all weights
            w1 = weights_f64(seed, 3 + 4 * L, (4 * H, H))
            w2 = weights_f64(seed, 4 + 4 * L, (H, 4 * H))
            bb = 1 + 4 * NL + 4 * (L - n_enc)
            b_qkv = weights_f64(seed, bb, (3 * H,))
            b_o = weights_f64(seed, bb + 1, (H,))
            b_1 = weights_f64(seed, bb + 2, (4 * H,))
            b_2 = weights_f64(seed, bb + 3, (H,))
        else:
            wi = weights_f64(seed, 3 + 4 * L, (2 * F, H))
            wo2 = weights_f64(seed, 4 + 4 * L, (H, F))

        n = R(ln(x, g(f"L{L}.ln_attn")))
        qkv = R(n @ wqkv.T)
        if head:
            qkv = R(qkv + b_qkv)
        q, k, v = qkv[:, :H], qkv[:, H:2 * H], qkv[:, 2 * H:]

        def rot(m):
            m = m.reshape(T, nh, d)
            z = m[..., : d // 2] + 1j * m[..., d // 2:]
            e = c[poss][:, None, :] + 1j * s[poss][:, None, :]
            w = z * e
            return R(np.concatenate([w.real, w.imag], axis=-1).reshape(T, H))

        q, k = rot(q), rot(k)
        vis = rows[:, None] == rows[None, :]
        if not is_global:
            vis &= np.abs(poss[:, None] - poss[None, :]) <= cfg["window"] // 2
        o = np.zeros((T, H))
        for h in range(nh):
            sl = slice(h * d, (h + 1) * d)
            for i in range(T):
                sc = np.array([q[i, sl] @ k[j, sl] for j in range(T)]) / np.sqrt(d)
                sc[~vis[i]] = -np.inf
                p = np.exp(sc - sc.max())
                p /= p.sum()
                o[i, sl] = p @ v[:, sl]
        o = R(o)
        att = R(o @ wo.T)
        if head:
            att = R(att + b_o)
        x = R(x + att)
        n2 = R(ln(x, g(f"L{L}.ln_ffn")))
        if head:
            u = R(R(n2 @ w1.T) + b_1)
            hmid = R(u * ndtr(u))
            x = R(x + R(R(hmid @ w2.T) + b_2))
        else:
            u = n2 @ wi[:F].T
            gate = n2 @ wi[F:].T
            hmid = R(u * ndtr(u) * gate)
            x = R(x + R(hmid @ wo2.T))
        caps.append((f"enc{L:02d}" if L < n_enc else f"dec{L - n_enc}", x.copy()))
        if L == n_enc - 1:
            x = R(ln(x, g("ln_enc_final")))
            caps.append(("enc_final", x.copy()))
    out = R(ln(x, g("ln_dec_final")))
    caps.append(("out", out.copy()))
    return {"out": out, "layers": caps if capture else None}
