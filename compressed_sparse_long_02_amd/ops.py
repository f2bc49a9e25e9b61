"""Torch-facing binding of the C ABI (include/csl.h): argument marshalling only.

Every function has the name of its C entry point, takes CUDA (HIP) tensors,
passes their device pointers, byte strides and torch's current HIP stream, and
raises CslError on a non-zero status.  PyTorch only provides device memory and
streams; every step of the computation runs in libcsl.so's kernels.

Layouts (B = batch, rows dense inside a sequence):
  stored rows   uint8 [B, N, row_bytes(fmt, d, r)], or float32 [B, N, d] for F32
  MXFP4 scales  uint8 [B, N, d/32]
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import check

F32, BF16, KV_PACKED, MXFP4 = 0, 1, 2, 3


def row_bytes(fmt: int, d: int, r: int = 0) -> int:
    return int(_lib.lib().csl_row_bytes(fmt, d, r))


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _bstride(t: torch.Tensor) -> int:
    return t.stride(0) * t.element_size() if t.dim() > 0 else 0


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def _rows_ok(t: torch.Tensor, rb: int, name: str):
    """Rows of one sequence must be dense: dim-1 stride == row bytes."""
    if t.dim() < 2:
        raise ValueError("%s must be [B, N, ...]" % name)
    if t.shape[1] > 1 and t.stride(1) * t.element_size() != rb:
        raise ValueError("%s: rows of a sequence must be dense (%d bytes each)" % (name, rb))
    if t.dim() > 2 and not t[0, 0].is_contiguous():
        raise ValueError("%s: a row must be contiguous" % name)


_ws = {}


def workspace(nbytes: int, device) -> torch.Tensor | None:
    """Per-device scratch tensor reused across calls on the same stream."""
    if nbytes <= 0:
        return None
    key = torch.device(device)
    t = _ws.get(key)
    if t is None or t.numel() < nbytes:
        t = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=key)
        _ws[key] = t
    return t


def kv_compress(x, x_fmt, z, bias, *, d, m, overlap, e_begin, n_e, r=0, x_pos0=0, out_fmt=F32, out=None,
                out_scales=None):
    """Compress raw rows x [B, n_tok, .] (F32 or BF16) into entries e_begin..e_begin+n_e-1.
    z: float32 [B, n_tok, z_ch]; bias float32 [win, z_ch].  Returns (out, out_scales)."""
    _need_cuda(x, z, bias, out, out_scales)
    B, n_tok = x.shape[0], x.shape[1]
    _rows_ok(x, row_bytes(x_fmt, d), "x")
    if z.dtype != torch.float32 or bias.dtype != torch.float32:
        raise ValueError("z and bias must be float32")
    z_ch = z.shape[-1]
    orb = row_bytes(out_fmt, d, r)
    if out is None:
        out = (torch.empty((B, n_e, d), dtype=torch.float32, device=x.device) if out_fmt == F32 else
               torch.empty((B, n_e, orb), dtype=torch.uint8, device=x.device))
    if out_fmt == MXFP4 and out_scales is None:
        out_scales = torch.empty((B, n_e, d // 32), dtype=torch.uint8, device=x.device)
    _rows_ok(out, orb, "out")
    rc = _lib.lib().kv_compress(_ptr(x), x_fmt, _bstride(x), x_pos0, n_tok, _ptr(z), z_ch, _bstride(z), _ptr(bias),
                                B, d, r, m, int(bool(overlap)), e_begin, n_e, _ptr(out), out_fmt,
                                _ptr(out_scales) if out_fmt == MXFP4 else None, _bstride(out),
                                _bstride(out_scales) if out_fmt == MXFP4 else 0, _stream())
    check("kv_compress", rc)
    return out, out_scales


def index_topk(qi, w, ki, q_pos, *, fmt, H_I, d_I, m, n_cap, k, qi_scales=None, ki_scales=None, out_idx=None,
               out_score=None, with_scores=True):
    """qi [B, Tq, H_I, .] in `fmt`; w float32 [B, Tq, H_I]; ki [B, N, .]; q_pos int32 [B, Tq].
    Returns (idx int32 [B, Tq, k], scores float32 [B, Tq, k] or None)."""
    _need_cuda(qi, w, ki, q_pos, qi_scales, ki_scales)
    B, Tq = q_pos.shape
    if q_pos.dtype != torch.int32 or not q_pos.is_contiguous():
        raise ValueError("q_pos must be contiguous int32 [B, Tq]")
    if not qi.is_contiguous() or not w.is_contiguous() or w.dtype != torch.float32:
        raise ValueError("qi and w must be contiguous (w float32)")
    _rows_ok(ki, row_bytes(fmt, d_I), "ki")
    dev = q_pos.device
    if out_idx is None:
        out_idx = torch.empty((B, Tq, k), dtype=torch.int32, device=dev)
    if with_scores and out_score is None:
        out_score = torch.empty((B, Tq, k), dtype=torch.float32, device=dev)
    nb = int(_lib.lib().csl_index_topk_workspace(B, Tq, n_cap, k))
    ws = workspace(nb, dev)
    rc = _lib.lib().index_topk(_ptr(qi), fmt, _ptr(qi_scales), _ptr(w), _ptr(ki), fmt, _ptr(ki_scales),
                               _bstride(ki), _bstride(ki_scales) if ki_scales is not None else 0, _ptr(q_pos),
                               B, Tq, H_I, d_I, m, n_cap, k, _ptr(out_idx), _ptr(out_score), _ptr(ws),
                               0 if ws is None else ws.numel(), _stream())
    check("index_topk", rc)
    return out_idx, out_score


def _q_fmt(q):
    if q.dtype == torch.float32:
        return F32
    if q.dtype == torch.bfloat16:
        return BF16
    raise ValueError("q must be float32 or bfloat16")


def _attend(name, q, kv_c, kv_w, q_pos, idx, *, kv_fmt, n_cap, m, kvw_pos0, kvw_rows, W, H, d, r, scale, out_fmt,
            out, lse, with_lse):
    _need_cuda(q, kv_c, kv_w, q_pos, idx, out, lse)
    B, Tq = q_pos.shape
    if q_pos.dtype != torch.int32 or not q_pos.is_contiguous() or not q.is_contiguous():
        raise ValueError("q and q_pos must be contiguous (q_pos int32)")
    rb = row_bytes(kv_fmt, d, r)
    _rows_ok(kv_c, rb, "kv_c")
    _rows_ok(kv_w, rb, "kv_w")
    dev = q.device
    if out is None:
        out = torch.empty((B, Tq, H, d), dtype=torch.float32 if out_fmt == F32 else torch.bfloat16, device=dev)
    if with_lse and lse is None:
        lse = torch.empty((B, Tq, H), dtype=torch.float32, device=dev)
    rows_max = (idx.shape[-1] if idx is not None else n_cap) + W
    nb = int(_lib.lib().csl_attend_workspace(B, Tq, H, d, rows_max))
    ws = workspace(nb, dev)
    L = _lib.lib()
    if name == "csa_attend":
        if idx.dtype != torch.int32 or not idx.is_contiguous():
            raise ValueError("idx must be contiguous int32 [B, Tq, k]")
        rc = L.csa_attend(_ptr(q), _q_fmt(q), _ptr(kv_c), kv_fmt, _bstride(kv_c), n_cap, _ptr(idx), idx.shape[-1],
                          _ptr(kv_w), _bstride(kv_w), kvw_pos0, kvw_rows, _ptr(q_pos), W, B, Tq, H, d, r, scale,
                          _ptr(out), out_fmt, _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel(), _stream())
    else:
        rc = L.hca_attend(_ptr(q), _q_fmt(q), _ptr(kv_c), kv_fmt, _bstride(kv_c), n_cap, m, _ptr(kv_w),
                          _bstride(kv_w), kvw_pos0, kvw_rows, _ptr(q_pos), W, B, Tq, H, d, r, scale, _ptr(out),
                          out_fmt, _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel(), _stream())
    check(name, rc)
    return out, lse


def csa_attend(q, kv_c, idx, kv_w, q_pos, *, kv_fmt, n_cap, kvw_pos0, kvw_rows, W, H, d, r=0, scale,
               out_fmt=F32, out=None, lse=None, with_lse=True):
    """q [B, Tq, H, d] (bf16 for BF16/packed KV, f32 for F32 KV); idx int32 [B, Tq, k].
    Returns (out [B, Tq, H, d], lse float32 [B, Tq, H] or None)."""
    return _attend("csa_attend", q, kv_c, kv_w, q_pos, idx, kv_fmt=kv_fmt, n_cap=n_cap, m=1, kvw_pos0=kvw_pos0,
                   kvw_rows=kvw_rows, W=W, H=H, d=d, r=r, scale=scale, out_fmt=out_fmt, out=out, lse=lse,
                   with_lse=with_lse)


def hca_attend(q, kv_c, kv_w, q_pos, *, kv_fmt, n_cap, m, kvw_pos0, kvw_rows, W, H, d, r=0, scale, out_fmt=F32,
               out=None, lse=None, with_lse=True):
    return _attend("hca_attend", q, kv_c, kv_w, q_pos, None, kv_fmt=kv_fmt, n_cap=n_cap, m=m, kvw_pos0=kvw_pos0,
                   kvw_rows=kvw_rows, W=W, H=H, d=d, r=r, scale=scale, out_fmt=out_fmt, out=out, lse=lse,
                   with_lse=with_lse)
