"""Synthetic workloads of the benchmark configurations: device-resident caches and inputs,
built from the seeded generators in gen.py, and the step each configuration times.

  Stack    the interleaved 4-layer CSA, HCA, CSA, HCA decode stack at 1M context, batch 16,
           with linear or paged caches (the default benchmark line);
  Layer    one CSA decode layer (batch 8 at 131,072 tokens, bf16 indexer 16 x 128, top-512)
           or one HCA decode layer (batch 4 at 1M tokens);
  Prefill  one CSA layer appending an 8,192-token chunk to 1,048,576 cached tokens.

The decode steps go through decode.py (compress from the state ring, index, attend); the
prefill step calls the library directly.  Nothing here does any of the method's arithmetic:
inputs are seeded draws cast to the storage formats (MXFP4 keys through kv_compress with
m = 1), and every step runs in the HIP kernels.
"""
from __future__ import annotations

import math

import torch

from . import decode as D
from . import gen, ops


class Stack:
    """Device-resident caches and inputs of the 4-layer decode step.

    Per layer, the two tiers of the cache: a state ring per sequence (the last RING raw
    rows -- bf16, with their compression logits -- and the window rows, packed) and the
    compressed cache.  layout "linear": one dense array of entries per sequence; layout
    "paged": blocks of BLOCK_TOKENS = lcm(4, 128) = 128 raw tokens behind one block
    table shared by all layers (a CSA block holds 32 packed entries, their 32 MXFP4
    indexer keys and the keys' scales; an HCA block 1 entry), the physical blocks in a
    seeded random order."""

    RING = 128
    BLOCK_TOKENS = 128

    def __init__(self, B, ctx, device, layout="linear"):
        F = ops
        self.B, self.ctx, self.dev, self.layout = B, ctx, device, layout
        self.t = ctx - 1
        self.H, self.d, self.r, self.W = 64, 512, 64, 128
        self.m, self.mh = 4, 128
        self.HI, self.dI, self.k = 64, 128, 1024
        self.N = ctx // self.m
        self.Nh = ctx // self.mh
        self.ring = 256
        self.scale = 1.0 / math.sqrt(self.d)
        B, d, r = self.B, self.d, self.r
        rb = F.row_bytes(F.KV_PACKED, d, r)
        self.rb = rb
        # paged layout: one block table for every layer, physical blocks shuffled
        self.nblk = ctx // self.BLOCK_TOKENS
        self.epb_csa = self.BLOCK_TOKENS // self.m
        self.epb_hca = self.BLOCK_TOKENS // self.mh
        self.csa_key_off = self.epb_csa * rb                       # bytes of a CSA block: entries, keys, scales
        self.csa_sc_off = self.csa_key_off + self.epb_csa * self.dI // 2
        self.csa_blk = self.csa_sc_off + self.epb_csa * self.dI // 32
        self.csa_blk = (self.csa_blk + 15) // 16 * 16
        self.hca_blk = self.epb_hca * rb
        self.n_phys = B * self.nblk
        if layout == "paged":
            g = torch.Generator(device="cpu")
            g.manual_seed(77)
            self.bt = torch.randperm(self.n_phys, generator=g).to(torch.int32).reshape(B, self.nblk).to(device)
        self.layers = []
        seed = 1000
        for li, kind in enumerate(["csa", "hca", "csa", "hca"]):
            L = {"kind": kind}
            seed += 100
            n = self.N if kind == "csa" else self.Nh
            # compressed KV cache: packed rows of N(0,1) values with outlier channels
            cache = torch.empty((B, n, rb), dtype=torch.uint8, device=device)
            chunk = 16384
            for s0 in range(0, n, chunk):
                c = min(chunk, n - s0)
                x = gen.with_outliers(gen.normal((B, c, d), seed + s0, device=device), seed)
                cache[:, s0:s0 + c] = gen.pack_kv(x, r)
            L["cache"] = cache
            # the state ring: window rows (packed) and the raw rows + logits of the last RING
            # positions (row p % RING), from which the completed entries are compressed
            xw = gen.with_outliers(gen.normal((B, self.ring, d), seed + 1, device=device), seed)
            L["ring"] = gen.pack_kv(xw, r)
            mm = self.m if kind == "csa" else self.mh
            L["win"] = 2 * mm if kind == "csa" else mm
            xr = gen.with_outliers(gen.normal((B, self.RING, d), seed + 2, device=device), seed)
            L["raw"] = gen.bf16_bytes(xr)
            L["z"] = gen.random_logits((B, self.RING, 1), seed + 3, device=device)
            L["bias"] = gen.random_logits((L["win"], 1), seed + 4, device=device)
            L["q"] = gen.with_outliers(gen.normal((B, 1, self.H, d), seed + 5, device=device), seed).to(torch.bfloat16)
            L["out"] = torch.empty((B, 1, self.H, d), dtype=torch.bfloat16, device=device)
            if kind == "csa":
                # MXFP4 indexer keys, quantised through kv_compress with m = 1 (identity pooling)
                keys = torch.empty((B, n, self.dI // 2), dtype=torch.uint8, device=device)
                ksc = torch.empty((B, n, self.dI // 32), dtype=torch.uint8, device=device)
                z1 = torch.zeros((B, chunk, 1), device=device)
                b1 = torch.zeros((1, 1), device=device)
                for s0 in range(0, n, chunk):
                    c = min(chunk, n - s0)
                    x = gen.with_outliers(gen.normal((B, c, self.dI), seed + 7 + s0, device=device), seed + 1)
                    F.kv_compress(gen.bf16_bytes(x), F.BF16, z1[:, :c], b1, d=self.dI, m=1, overlap=False, e_begin=0,
                                  n_e=c, out_fmt=F.MXFP4, out=keys[:, s0:s0 + c], out_scales=ksc[:, s0:s0 + c])
                L["keys"], L["kscales"] = keys, ksc
                xi = gen.with_outliers(gen.normal((B, self.RING, self.dI), seed + 8, device=device), seed + 1)
                L["raw_i"] = gen.bf16_bytes(xi)
                L["z_i"] = gen.random_logits((B, self.RING, 1), seed + 9, device=device)
                L["bias_i"] = gen.random_logits((L["win"], 1), seed + 10, device=device)
                qi = gen.with_outliers(gen.normal((B * self.HI, 1, self.dI), seed + 11, device=device), seed + 1)
                qic, qis = F.kv_compress(gen.bf16_bytes(qi), F.BF16, torch.zeros((B * self.HI, 1, 1), device=device),
                                         b1, d=self.dI, m=1, overlap=False, e_begin=0, n_e=1, out_fmt=F.MXFP4)
                L["qi"] = qic.reshape(B, 1, self.HI, self.dI // 2).contiguous()
                L["qis"] = qis.reshape(B, 1, self.HI, self.dI // 32).contiguous()
                L["w"] = gen.normal((B, 1, self.HI), seed + 12, 1 / math.sqrt(self.HI), device=device)
                L["idx"] = torch.empty((B, 1, self.k), dtype=torch.int32, device=device)
            if layout == "paged":
                self._to_pool(L)
            self.layers.append(L)
        self.q_pos = torch.full((B, 1), self.t, dtype=torch.int32, device=device)
        self.btab = D.BlockTable(self.bt, self.n_phys) if layout == "paged" else None
        for L in self.layers:
            L["dc"] = self._decode_cache(L)
        torch.cuda.synchronize()

    def _decode_cache(self, L):
        """The layer's cache tiers as the decode step takes them (views of the tensors above)."""
        F = ops
        paged = self.layout == "paged"
        if L["kind"] == "csa":
            c = D.CsaCache(d=self.d, r=self.r, m=self.m, d_I=self.dI, key_fmt=F.MXFP4, n_cap=self.N,
                           kv_ring=D.Ring(L["raw"], L["z"], L["bias"]), key_ring=D.Ring(L["raw_i"], L["z_i"], L["bias_i"]),
                           window=L["ring"])
            if paged:
                c.pool, c.entries_per_block, c.block_bytes = L["pool"], self.epb_csa, self.csa_blk
                c.key_off, c.scale_off = self.csa_key_off, self.csa_sc_off
            else:
                c.entries, c.keys, c.key_scales = L["cache"], L["keys"], L["kscales"]
            return c
        c = D.HcaCache(d=self.d, r=self.r, m=self.mh, n_cap=self.Nh, kv_ring=D.Ring(L["raw"], L["z"], L["bias"]),
                       window=L["ring"])
        if paged:
            c.pool, c.entries_per_block, c.block_bytes = L["pool"], self.epb_hca, self.hca_blk
        else:
            c.entries = L["cache"]
        return c

    def _to_pool(self, L):
        """Move a layer's linear cache into its block pool (physical block bt[b, j] holds the
        entries of raw tokens 128 j .. 128 j + 127 of sequence b); the linear arrays are
        dropped, and `cache` / `keys` / `kscales` become views of the pool's blocks."""
        B, rb = self.B, self.rb
        bt = self.bt.long()
        if L["kind"] == "csa":
            epb, blk = self.epb_csa, self.csa_blk
            pool = torch.zeros((self.n_phys, blk), dtype=torch.uint8, device=self.dev)
            for b in range(B):
                ids = bt[b]
                pool[ids, :self.csa_key_off] = L["cache"][b].reshape(self.nblk, epb * rb)
                pool[ids, self.csa_key_off:self.csa_sc_off] = L["keys"][b].reshape(self.nblk, -1)
                pool[ids, self.csa_sc_off:self.csa_sc_off + epb * self.dI // 32] = L["kscales"][b].reshape(self.nblk, -1)
            del L["keys"], L["kscales"]
            L["pool"] = pool
        else:
            epb, blk = self.epb_hca, self.hca_blk
            pool = torch.zeros((self.n_phys, blk), dtype=torch.uint8, device=self.dev)
            for b in range(B):
                pool[bt[b]] = L["cache"][b].reshape(self.nblk, epb * rb)
            L["pool"] = pool
        del L["cache"]
        torch.cuda.synchronize()

    # -- views of the compressed cache ----------------------------------------------
    def entries(self, L):
        """Linear [B, n, row] entries of a layer (gathered through the block table when
        paged: a host-side copy for the oracle, not part of the step)."""
        if self.layout != "paged":
            return L["cache"]
        epb = self.epb_csa if L["kind"] == "csa" else self.epb_hca
        bt = self.bt.long()
        rows = L["pool"][:, :epb * self.rb]
        return torch.stack([rows[bt[b]].reshape(-1, self.rb) for b in range(self.B)])

    def index_keys(self, L):
        """Linear MXFP4 keys and scales of a CSA layer ([B, N, 64], [B, N, 4])."""
        if self.layout != "paged":
            return L["keys"], L["kscales"]
        bt = self.bt.long()
        p = L["pool"]
        k = torch.stack([p[bt[b], self.csa_key_off:self.csa_sc_off].reshape(-1, self.dI // 2) for b in range(self.B)])
        s = torch.stack([p[bt[b], self.csa_sc_off:self.csa_sc_off + self.epb_csa * self.dI // 32]
                         .reshape(-1, self.dI // 32) for b in range(self.B)])
        return k, s

    # -- one layer's steps (the call order lives in decode.py) ------------------------
    def compress(self, L):
        """The entries completed by the new token, pooled from the state ring into the cache."""
        if L["kind"] == "csa":
            D.csa_compress(L["dc"], self.q_pos, self.btab)
        else:
            D.hca_compress(L["dc"], self.q_pos, self.btab)

    def index(self, L, with_scores=False, out_idx=None):
        return D.csa_select(L["dc"], self.q_pos, L["qi"], L["w"], H_I=self.HI, k=self.k, qi_scales=L["qis"],
                            out_idx=L["idx"] if out_idx is None else out_idx, with_scores=with_scores, bt=self.btab)

    def attend(self, L, out=None, out_fmt=None, with_lse=False):
        F = ops
        kw = dict(H=self.H, W=self.W, scale=self.scale, out_fmt=F.BF16 if out_fmt is None else out_fmt,
                  out=L["out"] if out is None and out_fmt is None else out, with_lse=with_lse, bt=self.btab)
        if L["kind"] == "csa":
            return D.csa_attend(L["dc"], L["q"], L["idx"], self.q_pos, **kw)
        return D.hca_attend(L["dc"], L["q"], self.q_pos, **kw)

    def step(self):
        for L in self.layers:
            if L["kind"] == "csa":
                D.csa_decode_step(L["dc"], self.q_pos, L["q"], L["qi"], L["w"], H=self.H, H_I=self.HI, k=self.k,
                                  W=self.W, scale=self.scale, idx=L["idx"], out=L["out"], qi_scales=L["qis"],
                                  bt=self.btab)
            else:
                D.hca_decode_step(L["dc"], self.q_pos, L["q"], H=self.H, W=self.W, scale=self.scale, out=L["out"],
                                  bt=self.btab)

    # -- algorithmic bytes -----------------------------------------------------
    def index_bytes(self):
        B = self.B
        keys = B * self.N * (self.dI // 2 + self.dI // 32)
        q = B * self.HI * (self.dI // 2 + self.dI // 32 + 4)
        out = B * self.k * 4
        return keys + q + out

    def csa_bytes(self):
        B, rb = self.B, 2 * self.r + (self.d - self.r)
        return B * ((self.k + self.W) * rb + self.k * 4 + self.H * self.d * 2 * 2)

    def hca_bytes(self):
        B, rb = self.B, 2 * self.r + (self.d - self.r)
        return B * ((self.Nh + self.W) * rb + self.H * self.d * 2 * 2)

    def compress_bytes(self):
        B = self.B
        csa = B * (2 * self.m * (self.d * 2 + 4) + 576 + 2 * self.m * (self.dI * 2 + 4) + 68)
        hca = B * (self.mh * (self.d * 2 + 4) + 576)
        return 2 * csa + 2 * hca

    def step_bytes(self):
        return 2 * self.index_bytes() + 2 * self.csa_bytes() + 2 * self.hca_bytes() + self.compress_bytes()


class Prefill:
    """One CSA layer appending a chunk of 8,192 tokens to 1,048,576 cached ones: compress the
    chunk's 2,048 entries (KV and indexer keys, with the 4 look-back rows), index the 8,192
    queries against the 264,192 entries (64 heads x 128, top-1024, causal) and attend with 128
    heads of 512 over the selected entries plus a 128-token window.  The indexer's queries and
    keys are bf16, or MXFP4 (key_fmt=ops.MXFP4: cached keys drawn as random codes and block
    scales, the chunk's keys compressed to MXFP4, the queries quantised to MXFP4)."""

    def __init__(self, device, key_fmt=ops.BF16):
        self.key_fmt = key_fmt
        self.H, self.d, self.r, self.m, self.HI, self.dI, self.k, self.W, self.C = 128, 512, 64, 4, 64, 128, 1024, 128, 8192
        self.T0 = 1 << 20
        self.N0 = self.T0 // self.m
        self.N = (self.T0 + self.C) // self.m
        d, r, dI, m, C, W = self.d, self.r, self.dI, self.m, self.C, self.W
        self.cache = torch.empty((1, self.N, d + r), dtype=torch.uint8, device=device)
        fp4 = key_fmt == ops.MXFP4
        self.keys = torch.empty((1, self.N, dI // 2 if fp4 else dI * 2), dtype=torch.uint8, device=device)
        self.kscales = torch.empty((1, self.N, dI // 32), dtype=torch.uint8, device=device) if fp4 else None
        for s0 in range(0, self.N0, 32768):
            c = min(32768, self.N0 - s0)
            self.cache[:, s0:s0 + c] = gen.pack_kv(gen.normal((1, c, d), 5000 + s0, device=device), r)
            if fp4:
                kc, ks = gen.random_mxfp4(c, dI, 6000 + s0, device=device)
                self.keys[0, s0:s0 + c], self.kscales[0, s0:s0 + c] = kc, ks
            else:
                self.keys[:, s0:s0 + c] = gen.bf16_bytes(gen.normal((1, c, dI), 6000 + s0, device=device))
        self.x = gen.bf16_bytes(gen.normal((1, C + m, d), 7001, device=device))
        self.xi = gen.bf16_bytes(gen.normal((1, C + m, dI), 7002, device=device))
        self.z = gen.random_logits((1, C + m, 1), 7003, device=device)
        self.zi = gen.random_logits((1, C + m, 1), 7004, device=device)
        self.bias = gen.random_logits((2 * m, 1), 7005, device=device)
        self.bias_i = gen.random_logits((2 * m, 1), 7006, device=device)
        self.kvw = gen.pack_kv(gen.normal((1, W + C, d), 7007, device=device), r)
        self.q_pos = torch.arange(self.T0, self.T0 + C, dtype=torch.int32, device=device).view(1, C)
        if fp4:
            qc, qs = gen.random_mxfp4(C * self.HI, dI, 7008, device=device)
            self.qi, self.qis = qc.reshape(1, C, self.HI, -1), qs.reshape(1, C, self.HI, -1)
        else:
            self.qi, self.qis = gen.bf16_bytes(gen.normal((1, C, self.HI, dI), 7008, device=device)), None
        self.w = gen.normal((1, C, self.HI), 7009, 1 / math.sqrt(self.HI), device=device)
        self.q = gen.normal((1, C, self.H, d), 7010, device=device).to(torch.bfloat16)
        self.idx = torch.empty((1, C, self.k), dtype=torch.int32, device=device)
        self.out = torch.empty((1, C, self.H, d), dtype=torch.bfloat16, device=device)
        torch.cuda.synchronize()

    def compress(self):
        F = ops
        ne = self.C // self.m
        kw = dict(m=self.m, overlap=True, e_begin=self.N0, n_e=ne, x_pos0=self.T0 - self.m)
        F.kv_compress(self.x, F.BF16, self.z, self.bias, d=self.d, r=self.r, out_fmt=F.KV_PACKED,
                      out=self.cache[:, self.N0:self.N], **kw)
        F.kv_compress(self.xi, F.BF16, self.zi, self.bias_i, d=self.dI, out_fmt=self.key_fmt,
                      out=self.keys[:, self.N0:self.N],
                      out_scales=None if self.kscales is None else self.kscales[:, self.N0:self.N], **kw)

    def index(self):
        F = ops
        F.index_topk(self.qi, self.w, self.keys, self.q_pos, fmt=self.key_fmt, H_I=self.HI, d_I=self.dI, m=self.m,
                     n_cap=self.N, k=self.k, out_idx=self.idx, with_scores=False, qi_scales=self.qis,
                     ki_scales=self.kscales)

    def attend(self):
        F = ops
        F.csa_attend(self.q, self.cache, self.idx, self.kvw, self.q_pos, kv_fmt=F.KV_PACKED, n_cap=self.N,
                     kvw_pos0=self.T0 - self.W, kvw_rows=self.W + self.C, W=self.W, H=self.H, d=self.d, r=self.r,
                     scale=1 / math.sqrt(self.d), out_fmt=F.BF16, out=self.out, with_lse=False)

    def step(self):
        self.compress()
        self.index()
        self.attend()

    def index_flops(self):
        """2 * H_I * d_I per visible (query, entry) pair."""
        pairs = sum(min((self.T0 + j + 1) // self.m, self.N) for j in range(self.C))
        return 2 * self.HI * self.dI * pairs

    def attend_flops(self):
        return 4 * self.C * self.H * (self.k + self.W) * self.d


class Layer:
    """One decode layer on its own, with its inputs in `copies` independent sets so that the
    timed steps cycle through more data than the 256 MB last-level cache holds.
      csa_decode: batch 8, context 131,072 (t = 131,071), 32,768 packed entries per sequence,
                  bf16 indexer keys (16 heads x 128, top-512), 64 heads x 512, window 128.
      hca_decode: batch 4, context 1,048,576, m' = 128: 8,192 packed entries per sequence,
                  64 heads x 512, window 128.
    A step: compress the entry the new token completes (from the 128-row state ring), then
    index + csa_attend, or hca_attend."""

    RING = 128

    def __init__(self, kind, device, copies):
        F = ops
        self.kind, self.dev = kind, device
        self.H, self.d, self.r, self.W = 64, 512, 64, 128
        if kind == "csa_decode":
            self.B, self.ctx, self.m, self.HI, self.dI, self.k = 8, 1 << 17, 4, 16, 128, 512
        else:
            self.B, self.ctx, self.m = 4, 1 << 20, 128
        self.t = self.ctx - 1
        self.N = self.ctx // self.m
        self.win = 2 * self.m if kind == "csa_decode" else self.m
        self.scale = 1.0 / math.sqrt(self.d)
        B, d, r = self.B, self.d, self.r
        self.rb = F.row_bytes(F.KV_PACKED, d, r)
        self.q_pos = torch.full((B, 1), self.t, dtype=torch.int32, device=device)
        self.sets = []
        for c in range(copies):
            seed = 9000 + 100 * c
            S = {}
            S["cache"] = torch.empty((B, self.N, self.rb), dtype=torch.uint8, device=device)
            for s0 in range(0, self.N, 16384):
                n = min(16384, self.N - s0)
                S["cache"][:, s0:s0 + n] = gen.pack_kv(gen.normal((B, n, d), seed + s0, device=device), r)
            S["ring"] = gen.pack_kv(gen.normal((B, 256, d), seed + 1, device=device), r)
            S["raw"] = gen.bf16_bytes(gen.normal((B, self.RING, d), seed + 2, device=device))
            S["z"] = gen.random_logits((B, self.RING, 1), seed + 3, device=device)
            S["bias"] = gen.random_logits((self.win, 1), seed + 4, device=device)
            S["q"] = gen.normal((B, 1, self.H, d), seed + 5, device=device).to(torch.bfloat16)
            S["out"] = torch.empty((B, 1, self.H, d), dtype=torch.bfloat16, device=device)
            if kind == "csa_decode":
                S["keys"] = gen.bf16_bytes(gen.normal((B, self.N, self.dI), seed + 6, device=device))
                S["raw_i"] = gen.bf16_bytes(gen.normal((B, self.RING, self.dI), seed + 7, device=device))
                S["z_i"] = gen.random_logits((B, self.RING, 1), seed + 8, device=device)
                S["bias_i"] = gen.random_logits((self.win, 1), seed + 9, device=device)
                S["qi"] = gen.bf16_bytes(gen.normal((B, 1, self.HI, self.dI), seed + 10, device=device))
                S["w"] = gen.normal((B, 1, self.HI), seed + 11, device=device)
                S["idx"] = torch.empty((B, 1, self.k), dtype=torch.int32, device=device)
            if kind == "csa_decode":
                S["dc"] = D.CsaCache(d=d, r=r, m=self.m, d_I=self.dI, key_fmt=F.BF16, n_cap=self.N,
                                     kv_ring=D.Ring(S["raw"], S["z"], S["bias"]),
                                     key_ring=D.Ring(S["raw_i"], S["z_i"], S["bias_i"]), window=S["ring"],
                                     entries=S["cache"], keys=S["keys"])
            else:
                S["dc"] = D.HcaCache(d=d, r=r, m=self.m, n_cap=self.N, kv_ring=D.Ring(S["raw"], S["z"], S["bias"]),
                                     window=S["ring"], entries=S["cache"])
            self.sets.append(S)
        torch.cuda.synchronize()

    def compress(self, S):
        if self.kind == "csa_decode":   # the KV entry and the indexer key, one launch
            D.csa_compress(S["dc"], self.q_pos)
        else:
            D.hca_compress(S["dc"], self.q_pos)

    def index(self, S, with_scores=False):
        return D.csa_select(S["dc"], self.q_pos, S["qi"], S["w"], H_I=self.HI, k=self.k, out_idx=S["idx"],
                            with_scores=with_scores)

    def attend(self, S, out_fmt=None, with_lse=False):
        kw = dict(H=self.H, W=self.W, scale=self.scale, out_fmt=ops.BF16 if out_fmt is None else out_fmt,
                  out=S["out"] if out_fmt is None else None, with_lse=with_lse)
        if self.kind == "csa_decode":
            return D.csa_attend(S["dc"], S["q"], S["idx"], self.q_pos, **kw)
        return D.hca_attend(S["dc"], S["q"], self.q_pos, **kw)

    def step(self, S):
        if self.kind == "csa_decode":
            D.csa_decode_step(S["dc"], self.q_pos, S["q"], S["qi"], S["w"], H=self.H, H_I=self.HI, k=self.k, W=self.W,
                              scale=self.scale, idx=S["idx"], out=S["out"])
        else:
            D.hca_decode_step(S["dc"], self.q_pos, S["q"], H=self.H, W=self.W, scale=self.scale, out=S["out"])

    def index_bytes(self):
        B = self.B
        return B * self.N * self.dI * 2 + B * self.HI * (self.dI * 2 + 4) + B * self.k * 4

    def attend_bytes(self):
        rows = (self.k if self.kind == "csa_decode" else self.N) + self.W
        idx = self.k * 4 if self.kind == "csa_decode" else 0
        return self.B * (rows * self.rb + idx + self.H * self.d * 2 * 2)

    def compress_bytes(self):
        kv = self.win * (self.d * 2 + 4) + self.rb
        ik = self.win * (self.dI * 2 + 4) + self.dI * 2 if self.kind == "csa_decode" else 0
        return self.B * (kv + ik)

    def step_bytes(self):
        return (self.index_bytes() if self.kind == "csa_decode" else 0) + self.attend_bytes() + self.compress_bytes()
