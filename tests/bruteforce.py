"""Independent numpy brute force used to pin the oracle on tiny inputs.

Written from the textbook definitions (softmax-weighted pooling over a window,
ReLU-gated weighted head sum + lexicographic top-k, softmax attention) with
vectorised numpy, so it shares neither code nor loop structure with oracle.c.
Stored formats are decoded with torch's own casts (bf16, fp8 e4m3fn) and the e2m1
value list from the chenxutan.com page, section 6.2.
"""
import os

import numpy as np
import torch

F32, BF16, KV_PACKED, MXFP4 = 0, 1, 2, 3

_E2M1 = None


def e2m1_table():
    global _E2M1
    if _E2M1 is None:
        vals = {}
        with open(os.path.join(os.path.dirname(__file__), "golden", "e2m1_values.txt")) as f:
            for line in f:
                if line.strip() and not line.startswith("#"):
                    c, v = line.split()
                    vals[int(c)] = float(v)
        pos = np.array([vals[i] for i in range(8)])
        _E2M1 = np.concatenate([pos, -pos])
    return _E2M1


def decode(stored, fmt, d, r=0, scales=None):
    """Stored rows -> float64 [..., d] using torch casts / the e2m1 table."""
    a = np.ascontiguousarray(stored)
    if fmt == F32:
        return a.view(np.float32).reshape(-1, d).astype(np.float64)
    u8 = torch.from_numpy(a.view(np.uint8)).reshape(-1)
    if fmt == BF16:
        return u8.view(torch.bfloat16).float().numpy().astype(np.float64).reshape(-1, d)
    if fmt == KV_PACKED:
        rows = u8.reshape(-1, 2 * r + d - r)
        lo = rows[:, :2 * r].contiguous().view(torch.bfloat16).float().numpy()
        hi = rows[:, 2 * r:].contiguous().view(torch.float8_e4m3fn).float().numpy()
        return np.concatenate([lo, hi], axis=1).astype(np.float64)
    if fmt == MXFP4:
        b = u8.numpy().reshape(-1, d // 2)
        codes = np.stack([b & 15, b >> 4], axis=-1).reshape(-1, d)
        v = e2m1_table()[codes]
        sc = np.ascontiguousarray(scales).reshape(-1, d // 32).astype(np.float64)
        return v * np.repeat(2.0 ** (sc - 127.0), 32, axis=1)
    raise ValueError(fmt)


def softmax(a, axis=-1):
    a = a - np.max(a, axis=axis, keepdims=True)
    e = np.exp(a)
    return e / e.sum(axis=axis, keepdims=True)


def compress(x, z, bias, m, overlap, entries, roles=1):
    """x [n_tok, roles*d] raw rows at positions 0..n_tok-1; z [n_tok, C]; bias [win, C].
    roles = 2: window slots j < m take the first d values of a row, the others the last d."""
    win = 2 * m if overlap else m
    d = x.shape[1] // roles
    out = []
    for i in entries:
        P = np.arange((i + 1) * m - win, (i + 1) * m)
        keep = P >= 0
        logits = z[P[keep]] + bias[keep]          # [nv, C]
        wts = softmax(logits, axis=0)             # normalise over window positions
        if wts.shape[1] == 1:
            wts = np.broadcast_to(wts, (wts.shape[0], d))
        vals = x[P[keep]]
        if roles == 2:
            slot = np.arange(win)[keep]
            vals = np.where((slot < m)[:, None], vals[:, :d], vals[:, d:])
        out.append((wts * vals).sum(axis=0))
    return np.array(out)


def index_topk(q, w, K, t, m, k):
    """q [H, d], w [H], K [N, d] for one query at position t."""
    n = min((t + 1) // m, K.shape[0]) if t >= 0 else 0
    s = (w[None, :] * np.maximum(K[:n] @ q.T, 0.0)).sum(axis=1)
    order = np.lexsort((np.arange(n), -s))[:k]   # score desc, index asc
    sel = np.sort(order)
    idx = np.full(k, -1, np.int64)
    idx[:len(sel)] = sel
    sc = np.full(k, -np.inf)
    sc[:len(sel)] = s[sel]
    return idx, sc, s


def attend(q, rows, scale):
    """q [H, d], rows [n, d] (key = value): returns o [H, d], lse [H]."""
    if rows.shape[0] == 0:
        return np.zeros_like(q), np.full(q.shape[0], -np.inf)
    l = scale * (q @ rows.T)
    mx = l.max(axis=1, keepdims=True)
    p = np.exp(l - mx)
    den = p.sum(axis=1, keepdims=True)
    return (p / den) @ rows, (mx + np.log(den))[:, 0]


def attend_sink(q, rows, scale, sink):
    """attend() with one extra logit per head (sink [H]) in the softmax denominator."""
    l = scale * (q @ rows.T) if rows.shape[0] else np.zeros((q.shape[0], 0))
    full = np.concatenate([l, np.asarray(sink, np.float64)[:, None]], axis=1)
    mx = full.max(axis=1, keepdims=True)
    p = np.exp(full - mx)
    den = p.sum(axis=1, keepdims=True)
    return (p[:, :-1] / den) @ rows if rows.shape[0] else np.zeros_like(q), (mx + np.log(den))[:, 0]


def causal_mqa(q, kv, scale, extra=None):
    """Textbook causal attention over raw rows: q [T, H, d] at positions 0..T-1 and
    kv [T, d]; `extra` [T, T] is added to the logits (masked entries ignored)."""
    T = kv.shape[0]
    l = scale * np.einsum("thd,sd->ths", q, kv)
    if extra is not None:
        l = l + extra[:, None, :]
    mask = np.tril(np.ones((T, T), bool))
    l = np.where(mask[:, None, :], l, -np.inf)
    p = softmax(l, axis=-1)
    return np.einsum("ths,sd->thd", p, kv)
