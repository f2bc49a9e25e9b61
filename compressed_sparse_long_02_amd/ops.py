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

import ctypes as C

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


def _check_table(bt):
    _need_cuda(bt)
    if bt.dtype != torch.int32 or not bt.is_contiguous() or bt.dim() != 2:
        raise ValueError("block table must be contiguous int32 [B, max_blocks]")


def _rows_ok(t: torch.Tensor, rb: int, name: str):
    """Rows of one sequence must be dense: dim-1 stride == row bytes."""
    if t.dim() < 2:
        raise ValueError("%s must be [B, N, ...]" % name)
    if t.shape[1] > 1 and t.stride(1) * t.element_size() != rb:
        raise ValueError("%s: rows of a sequence must be dense (%d bytes each)" % (name, rb))
    if t.dim() > 2 and t.shape[0] > 0 and t.shape[1] > 0 and not t[0, 0].is_contiguous():
        raise ValueError("%s: a row must be contiguous" % name)


_ws = {}


def workspace(nbytes: int, device) -> torch.Tensor | None:
    """Scratch tensor for the current stream of `device`, reused by later calls on that
    stream (which run after the previous call's kernels, so they may share it).  Calls on
    different streams get different buffers, so they may run concurrently.  A buffer is
    replaced only when a call needs more; it was allocated on that same stream, so the
    caching allocator hands its memory out again only in that stream's order, after the
    work already queued there."""
    if nbytes <= 0:
        return None
    dev = torch.device(device)
    key = (dev, torch.cuda.current_stream(dev).cuda_stream)
    t = _ws.get(key)
    if t is None or t.numel() < nbytes:
        t = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _ws[key] = t
    return t


def kv_compress(x, x_fmt, z, bias, *, d, m, overlap, e_begin, n_e, r=0, x_pos0=0, out_fmt=F32, out=None,
                out_scales=None, x_roles=1):
    """Compress raw rows x [B, n_tok, .] (F32 or BF16; x_roles*d values per row) into entries
    e_begin..e_begin+n_e-1.  z: float32 [B, n_tok, z_ch]; bias float32 [win, z_ch].
    Returns (out, out_scales)."""
    _need_cuda(x, z, bias, out, out_scales)
    B, n_tok = x.shape[0], x.shape[1]
    _rows_ok(x, row_bytes(x_fmt, x_roles * d), "x")
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
    rc = _lib.lib().kv_compress(_ptr(x), x_fmt, x_roles, _bstride(x), x_pos0, n_tok, _ptr(z), z_ch, _bstride(z),
                                _ptr(bias), B, d, r, m, int(bool(overlap)), e_begin, n_e, _ptr(out), out_fmt,
                                _ptr(out_scales) if out_fmt == MXFP4 else None, _bstride(out),
                                _bstride(out_scales) if out_fmt == MXFP4 else 0, _stream())
    check("kv_compress", rc)
    return out, out_scales


def _step_job(x_ring, x_fmt, z_ring, bias, *, d, m, overlap, out, out_fmt, r=0, out_scales=None, x_roles=1,
              pages=None):
    """One decode-time compression job as the C struct csl_compress_job."""
    _need_cuda(x_ring, z_ring, bias, out, out_scales)
    _rows_ok(x_ring, row_bytes(x_fmt, x_roles * d), "x_ring")
    sc = _ptr(out_scales) if out_fmt == MXFP4 else None
    if pages is None:
        _rows_ok(out, row_bytes(out_fmt, d, r), "out")
        ob, sb = _bstride(out), (_bstride(out_scales) if out_fmt == MXFP4 else 0)
        tail = dict(n_cap=out.shape[1])
    else:
        bt, epb, blk, sblk, nblk = pages
        _check_table(bt)
        ob, sb = 0, 0
        tail = dict(block_table=_ptr(bt), bt_stride=bt.shape[1], entries_per_block=epb, block_bytes=blk,
                    scale_block_bytes=sblk, n_blocks=nblk)
    return _lib.CompressJob(x_ring=_ptr(x_ring), x_fmt=x_fmt, x_roles=x_roles, x_bstride=_bstride(x_ring),
                            x_rows=x_ring.shape[1], z_ring=_ptr(z_ring), z_ch=z_ring.shape[-1],
                            z_bstride=_bstride(z_ring), bias=_ptr(bias), d=d, r=r, m=m, overlap=int(bool(overlap)),
                            out=_ptr(out), out_fmt=out_fmt, out_scales=sc, out_bstride=ob, sc_bstride=sb, **tail)


def _check_pos(pos, B):
    _need_cuda(pos)
    if pos.dtype != torch.int32 or not pos.is_contiguous() or pos.dim() != 2 or pos.shape[0] != B:
        raise ValueError("pos must be contiguous int32 [B, T]")


def kv_compress_step(x_ring, x_fmt, z_ring, bias, pos, *, d, m, overlap, out, out_fmt, r=0, out_scales=None,
                     x_roles=1, pages=None):
    """Decode-time compression from the state rings: x_ring [B, x_rows, .], z_ring float32
    [B, x_rows, z_ch] (position p in row p % x_rows); pos int32 [B, T] new token positions.
    out: the compressed cache -- linear [B, n_cap, row] (out_scales [B, n_cap, d/32]) or, with
    pages = (block_table int32 [B, max_blocks], entries_per_block, block_bytes,
    scale_block_bytes, n_blocks), a pool of blocks (out / out_scales point at the first
    block's rows)."""
    j = _step_job(x_ring, x_fmt, z_ring, bias, d=d, m=m, overlap=overlap, out=out, out_fmt=out_fmt, r=r,
                  out_scales=out_scales, x_roles=x_roles, pages=pages)
    B = x_ring.shape[0]
    _check_pos(pos, B)
    rc = _lib.lib().kv_compress_step(j.x_ring, j.x_fmt, j.x_roles, j.x_bstride, j.x_rows, j.z_ring, j.z_ch,
                                     j.z_bstride, j.bias, _ptr(pos), B, pos.shape[1], d, r, m, j.overlap, j.out,
                                     j.out_fmt, j.out_scales, j.out_bstride, j.sc_bstride, j.n_cap, j.block_table,
                                     j.bt_stride, j.entries_per_block, j.block_bytes, j.scale_block_bytes,
                                     j.n_blocks, _stream())
    check("kv_compress_step", rc)
    return out, out_scales


def kv_compress_step_pair(first, second, pos):
    """Two kv_compress_step jobs over the same new tokens in one launch (a CSA layer's KV
    entry and its indexer key).  `first` and `second` are dicts of kv_compress_step's
    keyword arguments plus x_ring, x_fmt, z_ring and bias."""
    j0, j1 = _step_job(**first), _step_job(**second)
    B = first["x_ring"].shape[0]
    _check_pos(pos, B)
    rc = _lib.lib().kv_compress_step_pair(C.byref(j0), C.byref(j1), _ptr(pos), B, pos.shape[1], _stream())
    check("kv_compress_step_pair", rc)


def index_topk(qi, w, ki, q_pos, *, fmt, H_I, d_I, m, n_cap, k, qi_scales=None, ki_scales=None, out_idx=None,
               out_score=None, with_scores=True, pages=None):
    """qi [B, Tq, H_I, .] in `fmt`; w float32 [B, Tq, H_I]; ki [B, N, .]; q_pos int32 [B, Tq].
    pages = (block_table int32 [B, max_blocks], entries_per_block, block_bytes,
    scale_block_bytes, n_blocks): ki / ki_scales point into pools of blocks (index_topk_paged).
    Returns (idx int32 [B, Tq, k], scores float32 [B, Tq, k] or None)."""
    _need_cuda(qi, w, ki, q_pos, qi_scales, ki_scales)
    B, Tq = q_pos.shape
    if q_pos.dtype != torch.int32 or not q_pos.is_contiguous():
        raise ValueError("q_pos must be contiguous int32 [B, Tq]")
    if not qi.is_contiguous() or not w.is_contiguous() or w.dtype != torch.float32:
        raise ValueError("qi and w must be contiguous (w float32)")
    if pages is None:
        _rows_ok(ki, row_bytes(fmt, d_I), "ki")
    dev = q_pos.device
    if out_idx is None:
        out_idx = torch.empty((B, Tq, k), dtype=torch.int32, device=dev)
    if with_scores and out_score is None:
        out_score = torch.empty((B, Tq, k), dtype=torch.float32, device=dev)
    nb = int(_lib.lib().csl_index_topk_workspace(B, Tq, n_cap, k))
    ws = workspace(nb, dev)
    wsn = 0 if ws is None else ws.numel()
    if pages is None:
        rc = _lib.lib().index_topk(_ptr(qi), fmt, _ptr(qi_scales), _ptr(w), _ptr(ki), fmt, _ptr(ki_scales),
                                   _bstride(ki), _bstride(ki_scales) if ki_scales is not None else 0, _ptr(q_pos),
                                   B, Tq, H_I, d_I, m, n_cap, k, _ptr(out_idx), _ptr(out_score), _ptr(ws), wsn,
                                   _stream())
        check("index_topk", rc)
    else:
        bt, epb, blk, sblk, nblk = pages
        _check_table(bt)
        rc = _lib.lib().index_topk_paged(_ptr(qi), fmt, _ptr(qi_scales), _ptr(w), _ptr(ki), fmt, _ptr(ki_scales),
                                         _ptr(bt), bt.shape[1], epb, blk, sblk, nblk, _ptr(q_pos), B, Tq, H_I, d_I,
                                         m, n_cap, k, _ptr(out_idx), _ptr(out_score), _ptr(ws), wsn, _stream())
        check("index_topk_paged", rc)
    return out_idx, out_score


def csa_index_step(kv, key, qi, w, ki, q_pos, *, fmt, H_I, d_I, m, n_cap, k, qi_scales=None, ki_scales=None,
                   out_idx=None, out_score=None, with_scores=True, pages=None):
    """A CSA layer's compression (kv and key: dicts of kv_compress_step's keyword arguments
    plus x_ring, x_fmt, z_ring and bias, as for kv_compress_step_pair) and its index_topk,
    in that order, the compression inside the indexer's scoring kernel where the shapes
    allow.  q_pos int32 [B, Tq] is also the jobs' token positions; the other arguments and
    the results are index_topk's."""
    _need_cuda(qi, w, ki, q_pos, qi_scales, ki_scales)
    j0, j1 = _step_job(**kv), _step_job(**key)
    B, Tq = q_pos.shape
    _check_pos(q_pos, B)
    if not qi.is_contiguous() or not w.is_contiguous() or w.dtype != torch.float32:
        raise ValueError("qi and w must be contiguous (w float32)")
    if pages is None:
        _rows_ok(ki, row_bytes(fmt, d_I), "ki")
    dev = q_pos.device
    if out_idx is None:
        out_idx = torch.empty((B, Tq, k), dtype=torch.int32, device=dev)
    if with_scores and out_score is None:
        out_score = torch.empty((B, Tq, k), dtype=torch.float32, device=dev)
    nb = int(_lib.lib().csl_index_topk_workspace(B, Tq, n_cap, k))
    ws = workspace(nb, dev)
    wsn = 0 if ws is None else ws.numel()
    if pages is None:
        bt, bts, epb, blk, sblk, nblk = None, 0, 0, 0, 0, 0
        kbs, sbs = _bstride(ki), (_bstride(ki_scales) if ki_scales is not None else 0)
    else:
        bt, epb, blk, sblk, nblk = pages
        _check_table(bt)
        bts, kbs, sbs = bt.shape[1], 0, 0
    rc = _lib.lib().csa_index_step(C.byref(j0), C.byref(j1), _ptr(qi), fmt, _ptr(qi_scales), _ptr(w), _ptr(ki), fmt,
                                   _ptr(ki_scales), kbs, sbs, _ptr(bt), bts, epb, blk, sblk, nblk, _ptr(q_pos), B, Tq,
                                   H_I, d_I, m, n_cap, k, _ptr(out_idx), _ptr(out_score), _ptr(ws), wsn, _stream())
    check("csa_index_step", rc)
    return out_idx, out_score


def index_topk_noalloc(qi, w, ki, q_pos, *, fmt, H_I, d_I, m, n_cap, k, qi_scales=None, ki_scales=None,
                       out_idx, out_score=None):
    """index_topk through the entry point that allocates nothing: the caller passes the
    outputs (idx int32 [B, Tq, k], scores float32 [B, Tq, k] or None); the staging lives
    in the library's static device scratch."""
    _need_cuda(qi, w, ki, q_pos, qi_scales, ki_scales, out_idx, out_score)
    B, Tq = q_pos.shape
    if q_pos.dtype != torch.int32 or not q_pos.is_contiguous():
        raise ValueError("q_pos must be contiguous int32 [B, Tq]")
    if not qi.is_contiguous() or not w.is_contiguous() or w.dtype != torch.float32:
        raise ValueError("qi and w must be contiguous (w float32)")
    _rows_ok(ki, row_bytes(fmt, d_I), "ki")
    rc = _lib.lib().index_topk_noalloc(_ptr(qi), fmt, _ptr(qi_scales), _ptr(w), _ptr(ki), fmt, _ptr(ki_scales),
                                       _bstride(ki), _bstride(ki_scales) if ki_scales is not None else 0,
                                       _ptr(q_pos), B, Tq, H_I, d_I, m, n_cap, k, _ptr(out_idx), _ptr(out_score),
                                       _stream())
    check("index_topk_noalloc", rc)
    return out_idx, out_score


def _q_fmt(q):
    if q.dtype == torch.float32:
        return F32
    if q.dtype == torch.bfloat16:
        return BF16
    raise ValueError("q must be float32 or bfloat16")


def _attend(name, q, kv_c, kv_w, q_pos, idx, *, kv_fmt, n_cap, m, kvw_pos0, kvw_rows, W, H, d, r, scale, out_fmt,
            out, lse, with_lse, sink=None, pages=None, job=None):
    _need_cuda(q, kv_c, kv_w, q_pos, idx, out, lse, sink)
    B, Tq = q_pos.shape
    if q_pos.dtype != torch.int32 or not q_pos.is_contiguous() or not q.is_contiguous():
        raise ValueError("q and q_pos must be contiguous (q_pos int32)")
    if sink is not None and (sink.dtype != torch.float32 or not sink.is_contiguous() or sink.numel() < H):
        raise ValueError("sink must be contiguous float32 [H]")
    rb = row_bytes(kv_fmt, d, r)
    if pages is None:
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
    tail = (_ptr(kv_w), _bstride(kv_w), kvw_pos0, kvw_rows, _ptr(sink), _ptr(q_pos), W, B, Tq, H, d, r, scale,
            _ptr(out), out_fmt, _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel(), _stream())
    if idx is not None and (idx.dtype != torch.int32 or not idx.is_contiguous()):
        raise ValueError("idx must be contiguous int32 [B, Tq, k]")
    if job is not None:
        if pages is None:
            geo = (_bstride(kv_c), None, 0, 0, 0, 0)
        else:
            bt, epb, blk_bytes, n_blocks = pages
            _check_table(bt)
            geo = (0, _ptr(bt), bt.shape[1], epb, blk_bytes, n_blocks)
        rc = L.hca_attend_step(C.byref(job), _ptr(q), _q_fmt(q), _ptr(kv_c), kv_fmt, *geo, n_cap, m, *tail)
    elif pages is None:
        if name == "csa_attend":
            rc = L.csa_attend(_ptr(q), _q_fmt(q), _ptr(kv_c), kv_fmt, _bstride(kv_c), n_cap, _ptr(idx),
                              idx.shape[-1], *tail)
        else:
            rc = L.hca_attend(_ptr(q), _q_fmt(q), _ptr(kv_c), kv_fmt, _bstride(kv_c), n_cap, m, *tail)
    else:
        bt, epb, blk_bytes, n_blocks = pages
        _check_table(bt)
        head = (_ptr(q), _q_fmt(q), _ptr(kv_c), kv_fmt, _ptr(bt), bt.shape[1], epb, blk_bytes, n_blocks, n_cap)
        if name == "csa_attend":
            rc = L.csa_attend_paged(*head, _ptr(idx), idx.shape[-1], *tail)
        else:
            rc = L.hca_attend_paged(*head, m, *tail)
        name += "_paged"
    check(name, rc)
    return out, lse


def hca_attend_step(job, q, kv_c, kv_w, q_pos, *, kv_fmt, n_cap, m, kvw_pos0, kvw_rows, W, H, d, r=0, scale,
                    out_fmt=F32, out=None, lse=None, with_lse=True, sink=None, pages=None):
    """An HCA layer's compression (job: a dict of kv_compress_step's keyword arguments plus
    x_ring, x_fmt, z_ring and bias, q_pos doubling as the token positions) and its
    attention, in that order, the compression inside the attention kernel where the shapes
    allow.  kv_c: the dense entries [B, N, row], or with pages = (block_table, entries per
    block, block bytes, n_blocks) the pool.  The other arguments and the results are
    hca_attend's."""
    j = _step_job(**job)
    _check_pos(q_pos, q_pos.shape[0])
    return _attend("hca_attend_step", q, kv_c, kv_w, q_pos, None, kv_fmt=kv_fmt, n_cap=n_cap, m=m,
                   kvw_pos0=kvw_pos0, kvw_rows=kvw_rows, W=W, H=H, d=d, r=r, scale=scale, out_fmt=out_fmt, out=out,
                   lse=lse, with_lse=with_lse, sink=sink, pages=pages, job=j)


def csa_attend(q, kv_c, idx, kv_w, q_pos, *, kv_fmt, n_cap, kvw_pos0, kvw_rows, W, H, d, r=0, scale,
               out_fmt=F32, out=None, lse=None, with_lse=True, sink=None):
    """q [B, Tq, H, d] (bf16 for BF16/packed KV, f32 for F32 KV); idx int32 [B, Tq, k];
    sink float32 [H] or None.  Returns (out [B, Tq, H, d], lse float32 [B, Tq, H] or None)."""
    return _attend("csa_attend", q, kv_c, kv_w, q_pos, idx, kv_fmt=kv_fmt, n_cap=n_cap, m=1, kvw_pos0=kvw_pos0,
                   kvw_rows=kvw_rows, W=W, H=H, d=d, r=r, scale=scale, out_fmt=out_fmt, out=out, lse=lse,
                   with_lse=with_lse, sink=sink)


def hca_attend(q, kv_c, kv_w, q_pos, *, kv_fmt, n_cap, m, kvw_pos0, kvw_rows, W, H, d, r=0, scale, out_fmt=F32,
               out=None, lse=None, with_lse=True, sink=None):
    return _attend("hca_attend", q, kv_c, kv_w, q_pos, None, kv_fmt=kv_fmt, n_cap=n_cap, m=m, kvw_pos0=kvw_pos0,
                   kvw_rows=kvw_rows, W=W, H=H, d=d, r=r, scale=scale, out_fmt=out_fmt, out=out, lse=lse,
                   with_lse=with_lse, sink=sink)


def csa_attend_paged(q, pool, block_table, idx, kv_w, q_pos, *, entries_per_block, block_bytes, n_blocks, kv_fmt,
                     n_cap, kvw_pos0, kvw_rows, W, H, d, r=0, scale, out_fmt=F32, out=None, lse=None, with_lse=True,
                     sink=None):
    """csa_attend over a paged pool (`pool` points at block 0's first entry row; blocks are
    block_bytes apart, n_blocks of them) with block_table int32 [B, max_blocks]: entry s of
    sequence b is row s % entries_per_block of block block_table[b, s // entries_per_block]."""
    return _attend("csa_attend", q, pool, kv_w, q_pos, idx, kv_fmt=kv_fmt, n_cap=n_cap, m=1, kvw_pos0=kvw_pos0,
                   kvw_rows=kvw_rows, W=W, H=H, d=d, r=r, scale=scale, out_fmt=out_fmt, out=out, lse=lse,
                   with_lse=with_lse, sink=sink, pages=(block_table, entries_per_block, block_bytes, n_blocks))


def hca_attend_paged(q, pool, block_table, kv_w, q_pos, *, entries_per_block, block_bytes, n_blocks, kv_fmt, n_cap,
                     m, kvw_pos0, kvw_rows, W, H, d, r=0, scale, out_fmt=F32, out=None, lse=None, with_lse=True,
                     sink=None):
    return _attend("hca_attend", q, pool, kv_w, q_pos, None, kv_fmt=kv_fmt, n_cap=n_cap, m=m, kvw_pos0=kvw_pos0,
                   kvw_rows=kvw_rows, W=W, H=H, d=d, r=r, scale=scale, out_fmt=out_fmt, out=out, lse=lse,
                   with_lse=with_lse, sink=sink, pages=(block_table, entries_per_block, block_bytes, n_blocks))


def grouped_out_proj(x, w, *, G, out_fmt=F32, out=None):
    """x bf16 [M, G*K] (e.g. the attention output [B, Tq, H, d] viewed as [B*Tq, H*d]);
    w bf16 [G, R, K].  Returns out [M, G*R] (float32 or bfloat16): group g's outputs are
    x[:, g*K:(g+1)*K] @ w[g].T."""
    _need_cuda(x, w, out)
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16 or not x.is_contiguous() or not w.is_contiguous():
        raise ValueError("x and w must be contiguous bfloat16")
    G_, R, K = w.shape
    if G_ != G or x.shape[-1] != G * K:
        raise ValueError("x must be [M, G*K] and w [G, R, K]")
    M = x.numel() // (G * K)
    if out is None:
        out = torch.empty((M, G * R), dtype=torch.float32 if out_fmt == F32 else torch.bfloat16, device=x.device)
    rc = _lib.lib().grouped_out_proj(_ptr(x), BF16, _ptr(w), BF16, M, G, K, R, _ptr(out), out_fmt, _stream())
    check("grouped_out_proj", rc)
    return out
