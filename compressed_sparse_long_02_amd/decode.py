"""Decode-step orchestration of the hybrid compressed attention layer.

For the new token(s) of every sequence a layer (x-techcon article on DeepSeek-V4,
section 2: CSA steps 1-3 and the HCA subsection; section 4, KV-cache paragraph, for the
two cache tiers):

  1. compresses the entries the new tokens complete, if any, from the state ring into
     the compressed cache (CSA: the KV entry and the indexer key in one launch);
  2. CSA only: the lightning indexer selects the top-k complete entries;
  3. attends over the selected entries (CSA) or every complete entry (HCA) plus the
     sliding window, with an optional per-head sink.

Only the order of the library calls and the cache bookkeeping live here; every step runs
in the HIP kernels behind include/csl.h (through ops.py).  A cache is dense (one array of
entries per sequence) or paged: blocks of a pool reached through a block table that all
layers share (entry s of a sequence in row s % entries_per_block of block
table[s // entries_per_block]).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import ops


@dataclass
class BlockTable:
    """The block table shared by the layers of a paged cache: int32 [B, max_blocks] ids of
    physical blocks, `n_blocks` blocks in each layer's pool."""
    table: torch.Tensor
    n_blocks: int


@dataclass
class Ring:
    """A layer's state ring: raw rows (bf16 bytes [B, R, roles * d]) and their compression
    logits (float32 [B, R, 1]), position p in row p % R, plus the per-slot bias
    (float32 [window, 1])."""
    raw: torch.Tensor
    z: torch.Tensor
    bias: torch.Tensor
    roles: int = 1


@dataclass
class CsaCache:
    """One CSA layer: rings of the KV rows and of the indexer key rows, the packed window
    ring [B, Wr, row], and the compressed tier.  Dense: `entries` [B, n_cap, row], `keys`
    [B, n_cap, d_I/2 or 2 d_I] and (MXFP4) `key_scales` [B, n_cap, d_I/32].  Paged: `pool`
    [n_blocks, block_bytes], a block holding entries_per_block packed entries, then their
    keys at byte `key_off`, then (MXFP4) their scales at `scale_off`."""
    d: int
    r: int
    m: int
    d_I: int
    key_fmt: int
    n_cap: int
    kv_ring: Ring
    key_ring: Ring
    window: torch.Tensor
    entries: Optional[torch.Tensor] = None
    keys: Optional[torch.Tensor] = None
    key_scales: Optional[torch.Tensor] = None
    pool: Optional[torch.Tensor] = None
    entries_per_block: int = 0
    block_bytes: int = 0
    key_off: int = 0
    scale_off: int = 0


@dataclass
class HcaCache:
    """One HCA layer: the ring of its KV rows, the packed window ring, and the compressed
    tier (dense `entries` [B, n_cap, row], or a `pool` of blocks of entries_per_block
    entries)."""
    d: int
    r: int
    m: int
    n_cap: int
    kv_ring: Ring
    window: torch.Tensor
    entries: Optional[torch.Tensor] = None
    pool: Optional[torch.Tensor] = None
    entries_per_block: int = 0
    block_bytes: int = 0


def _pages(c, bt: Optional[BlockTable]):
    return None if bt is None else (bt.table, c.entries_per_block, c.block_bytes, c.block_bytes, bt.n_blocks)


# ---- CSA ------------------------------------------------------------------------------
def _csa_jobs(c: CsaCache, bt: Optional[BlockTable]):
    """The compression jobs of a CSA layer: its KV entries and its indexer keys."""
    kv = dict(x_ring=c.kv_ring.raw, x_fmt=ops.BF16, z_ring=c.kv_ring.z, bias=c.kv_ring.bias, d=c.d, r=c.r, m=c.m,
              overlap=True, out_fmt=ops.KV_PACKED, x_roles=c.kv_ring.roles)
    key = dict(x_ring=c.key_ring.raw, x_fmt=ops.BF16, z_ring=c.key_ring.z, bias=c.key_ring.bias, d=c.d_I, m=c.m,
               overlap=True, out_fmt=c.key_fmt, x_roles=c.key_ring.roles)
    if bt is None:
        kv.update(out=c.entries)
        key.update(out=c.keys, out_scales=c.key_scales)
    else:
        pg = _pages(c, bt)
        kv.update(out=c.pool, pages=pg)
        key.update(out=c.pool[:, c.key_off:], pages=pg,
                   out_scales=c.pool[:, c.scale_off:] if c.key_fmt == ops.MXFP4 else None)
    return kv, key


def csa_compress(c: CsaCache, q_pos: torch.Tensor, bt: Optional[BlockTable] = None):
    """Step 1: the KV entries and indexer keys the new tokens (positions q_pos int32 [B, T])
    complete, pooled from the rings (window 2m, overlapping) into the cache."""
    kv, key = _csa_jobs(c, bt)
    ops.kv_compress_step_pair(kv, key, q_pos)


def csa_select(c: CsaCache, q_pos, qi, w, *, H_I, k, qi_scales=None, out_idx=None, with_scores=False,
               bt: Optional[BlockTable] = None):
    """Step 2: the top-k complete entries per query by the indexer score.  Returns (idx int32
    [B, T, k], scores float32 [B, T, k] or None)."""
    kw = dict(fmt=c.key_fmt, H_I=H_I, d_I=c.d_I, m=c.m, n_cap=c.n_cap, k=k, qi_scales=qi_scales, out_idx=out_idx,
              with_scores=with_scores)
    if bt is None:
        return ops.index_topk(qi, w, c.keys, q_pos, ki_scales=c.key_scales, **kw)
    return ops.index_topk(qi, w, c.pool[:, c.key_off:], q_pos, pages=_pages(c, bt),
                          ki_scales=c.pool[:, c.scale_off:] if c.key_fmt == ops.MXFP4 else None, **kw)


def csa_compress_select(c: CsaCache, q_pos, qi, w, *, H_I, k, qi_scales=None, out_idx=None, with_scores=False,
                        bt: Optional[BlockTable] = None):
    """Steps 1 and 2 through one call (csa_index_step): the compression of the completed
    entries, then the top-k; with one query per sequence the compression runs inside the
    indexer's scoring kernel."""
    kv, key = _csa_jobs(c, bt)
    kw = dict(fmt=c.key_fmt, H_I=H_I, d_I=c.d_I, m=c.m, n_cap=c.n_cap, k=k, qi_scales=qi_scales, out_idx=out_idx,
              with_scores=with_scores)
    if bt is None:
        return ops.csa_index_step(kv, key, qi, w, c.keys, q_pos, ki_scales=c.key_scales, **kw)
    return ops.csa_index_step(kv, key, qi, w, c.pool[:, c.key_off:], q_pos, pages=_pages(c, bt),
                              ki_scales=c.pool[:, c.scale_off:] if c.key_fmt == ops.MXFP4 else None, **kw)


def csa_attend(c: CsaCache, q, idx, q_pos, *, H, W, scale, out=None, out_fmt=ops.BF16, with_lse=False, sink=None,
               bt: Optional[BlockTable] = None):
    """Step 3: MQA over the selected entries plus the window (ring position p in row
    p % window rows)."""
    kw = dict(kv_fmt=ops.KV_PACKED, n_cap=c.n_cap, kvw_pos0=0, kvw_rows=c.window.shape[1], W=W, H=H, d=c.d, r=c.r,
              scale=scale, out_fmt=out_fmt, out=out, with_lse=with_lse, sink=sink)
    if bt is None:
        return ops.csa_attend(q, c.entries, idx, c.window, q_pos, **kw)
    return ops.csa_attend_paged(q, c.pool, bt.table, idx, c.window, q_pos, entries_per_block=c.entries_per_block,
                                block_bytes=c.block_bytes, n_blocks=bt.n_blocks, **kw)


def csa_decode_step(c: CsaCache, q_pos, q, qi, w, *, H, H_I, k, W, scale, idx, out, qi_scales=None, sink=None,
                    bt: Optional[BlockTable] = None):
    """One CSA layer for the new tokens: compress, select, attend (out [B, T, H, d] bf16)."""
    csa_compress_select(c, q_pos, qi, w, H_I=H_I, k=k, qi_scales=qi_scales, out_idx=idx, bt=bt)
    csa_attend(c, q, idx, q_pos, H=H, W=W, scale=scale, out=out, sink=sink, bt=bt)
    return out


# ---- HCA ------------------------------------------------------------------------------
def hca_compress(c: HcaCache, q_pos, bt: Optional[BlockTable] = None):
    """Step 1 at m' (window m', no overlap)."""
    kw = dict(d=c.d, r=c.r, m=c.m, overlap=False, out_fmt=ops.KV_PACKED, x_roles=c.kv_ring.roles)
    if bt is None:
        ops.kv_compress_step(c.kv_ring.raw, ops.BF16, c.kv_ring.z, c.kv_ring.bias, q_pos, out=c.entries, **kw)
    else:
        ops.kv_compress_step(c.kv_ring.raw, ops.BF16, c.kv_ring.z, c.kv_ring.bias, q_pos, out=c.pool,
                             pages=_pages(c, bt), **kw)


def hca_attend(c: HcaCache, q, q_pos, *, H, W, scale, out=None, out_fmt=ops.BF16, with_lse=False, sink=None,
               bt: Optional[BlockTable] = None):
    """Dense MQA over every complete entry plus the window."""
    kw = dict(kv_fmt=ops.KV_PACKED, n_cap=c.n_cap, m=c.m, kvw_pos0=0, kvw_rows=c.window.shape[1], W=W, H=H, d=c.d,
              r=c.r, scale=scale, out_fmt=out_fmt, out=out, with_lse=with_lse, sink=sink)
    if bt is None:
        return ops.hca_attend(q, c.entries, c.window, q_pos, **kw)
    return ops.hca_attend_paged(q, c.pool, bt.table, c.window, q_pos, entries_per_block=c.entries_per_block,
                                block_bytes=c.block_bytes, n_blocks=bt.n_blocks, **kw)


def hca_compress_attend(c: HcaCache, q, q_pos, *, H, W, scale, out=None, out_fmt=ops.BF16, with_lse=False,
                        sink=None, bt: Optional[BlockTable] = None):
    """Step 1 and the attention through one call (hca_attend_step); with one query per
    sequence the compression runs inside the attention kernel."""
    job = dict(x_ring=c.kv_ring.raw, x_fmt=ops.BF16, z_ring=c.kv_ring.z, bias=c.kv_ring.bias, d=c.d, r=c.r, m=c.m,
               overlap=False, out_fmt=ops.KV_PACKED, x_roles=c.kv_ring.roles)
    kw = dict(kv_fmt=ops.KV_PACKED, n_cap=c.n_cap, m=c.m, kvw_pos0=0, kvw_rows=c.window.shape[1], W=W, H=H, d=c.d,
              r=c.r, scale=scale, out_fmt=out_fmt, out=out, with_lse=with_lse, sink=sink)
    if bt is None:
        job.update(out=c.entries)
        return ops.hca_attend_step(job, q, c.entries, c.window, q_pos, **kw)
    job.update(out=c.pool, pages=_pages(c, bt))
    return ops.hca_attend_step(job, q, c.pool, c.window, q_pos,
                               pages=(bt.table, c.entries_per_block, c.block_bytes, bt.n_blocks), **kw)


def hca_decode_step(c: HcaCache, q_pos, q, *, H, W, scale, out, sink=None, bt: Optional[BlockTable] = None):
    """One HCA layer for the new tokens: compress, attend (out [B, T, H, d] bf16)."""
    hca_compress_attend(c, q, q_pos, H=H, W=W, scale=scale, out=out, sink=sink, bt=bt)
    return out
