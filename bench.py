"""Decode throughput of the hybrid compressed attention stack on one MI355X.

Workload (default): an interleaved 4-layer stack (CSA, HCA, CSA, HCA) decoding one
token per sequence at 1M context (t = 2^20 - 1), batch 16.  CSA: m = 4 (2m window),
262,144 compressed entries per sequence stored as packed rows (64 bf16 RoPE dims +
448 fp8 e4m3fn dims = 576 B), MXFP4 indexer keys (d_I = 128, e8m0 per 32) with 64
indexer heads, top-k 1024, 128-token window.  HCA: m' = 128, 8,192 entries, dense.
64 query heads of dim 512.  Seeded synthetic N(0,1) activations with 1% x10
outlier channels.  The token at 2^20 - 1 completes a CSA block and an HCA block, so
every layer also compresses its new entry (KV, and the indexer key for CSA) in the
step.  One step = the whole stack for the batch, replayed as one HIP graph.

Prints one JSON line (metric, value = tokens/s, roofline of the dominant kernel,
oracle CPU baseline on a bounded sample).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA/HCA decode tokens/sec at 1M ctx; achieved HBM GB/s & indexer MFMA %"
HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--batch", type=int, default=16)
    p.add_argument("--ctx", type=int, default=1 << 20)
    p.add_argument("--cpu-seqs", type=int, default=16, help="sequences in the oracle CPU sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--kernel-iters", type=int, default=20)
    p.add_argument("--workload", choices=["stack", "prefill"], default="stack",
                   help="stack: the 4-layer decode stack (default); prefill: one CSA prefill chunk")
    p.add_argument("--copy-mb", type=int, default=0,
                   help="also run a plain device copy of this many MiB (the reference kernel for HBM counters)")
    return p.parse_args()


class Stack:
    """Device-resident caches and inputs of the 4-layer decode step."""

    def __init__(self, B, ctx, device):
        import torch
        from compressed_sparse_long_02_amd import gen, ops
        F = ops
        self.B, self.ctx, self.dev = B, ctx, device
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
            # sliding-window state: ring of packed rows
            xw = gen.with_outliers(gen.normal((B, self.ring, d), seed + 1, device=device), seed)
            L["ring"] = gen.pack_kv(xw, r)
            # raw tail of the new block (bf16) + compression logits and slot biases
            mm = self.m if kind == "csa" else self.mh
            win = 2 * mm if kind == "csa" else mm
            L["win"] = win
            xr = gen.with_outliers(gen.normal((B, win, d), seed + 2, device=device), seed)
            L["raw"] = gen.bf16_bytes(xr)
            L["z"] = gen.random_logits((B, win, 1), seed + 3, device=device)
            L["bias"] = gen.random_logits((win, 1), seed + 4, device=device)
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
                xi = gen.with_outliers(gen.normal((B, win, self.dI), seed + 8, device=device), seed + 1)
                L["raw_i"] = gen.bf16_bytes(xi)
                L["z_i"] = gen.random_logits((B, win, 1), seed + 9, device=device)
                L["bias_i"] = gen.random_logits((win, 1), seed + 10, device=device)
                qi = gen.with_outliers(gen.normal((B * self.HI, 1, self.dI), seed + 11, device=device), seed + 1)
                qic, qis = F.kv_compress(gen.bf16_bytes(qi), F.BF16, torch.zeros((B * self.HI, 1, 1), device=device),
                                         b1, d=self.dI, m=1, overlap=False, e_begin=0, n_e=1, out_fmt=F.MXFP4)
                L["qi"] = qic.reshape(B, 1, self.HI, self.dI // 2).contiguous()
                L["qis"] = qis.reshape(B, 1, self.HI, self.dI // 32).contiguous()
                L["w"] = gen.normal((B, 1, self.HI), seed + 12, 1 / math.sqrt(self.HI), device=device)
                L["idx"] = torch.empty((B, 1, self.k), dtype=torch.int32, device=device)
            self.layers.append(L)
        self.q_pos = torch.full((B, 1), self.t, dtype=torch.int32, device=device)
        torch.cuda.synchronize()

    # -- the ABI calls of one layer ------------------------------------------
    def compress(self, L):
        from compressed_sparse_long_02_amd import ops as F
        t = self.t
        if L["kind"] == "csa":
            i = (t + 1) // self.m - 1          # the entry completed by token t
            F.kv_compress(L["raw"], F.BF16, L["z"], L["bias"], d=self.d, r=self.r, m=self.m, overlap=True,
                          e_begin=i, n_e=1, x_pos0=t - L["win"] + 1, out_fmt=F.KV_PACKED,
                          out=L["cache"][:, i:i + 1])
            F.kv_compress(L["raw_i"], F.BF16, L["z_i"], L["bias_i"], d=self.dI, m=self.m, overlap=True,
                          e_begin=i, n_e=1, x_pos0=t - L["win"] + 1, out_fmt=F.MXFP4,
                          out=L["keys"][:, i:i + 1], out_scales=L["kscales"][:, i:i + 1])
        else:
            i = (t + 1) // self.mh - 1
            F.kv_compress(L["raw"], F.BF16, L["z"], L["bias"], d=self.d, r=self.r, m=self.mh, overlap=False,
                          e_begin=i, n_e=1, x_pos0=t - L["win"] + 1, out_fmt=F.KV_PACKED,
                          out=L["cache"][:, i:i + 1])

    def index(self, L):
        from compressed_sparse_long_02_amd import ops as F
        F.index_topk(L["qi"], L["w"], L["keys"], self.q_pos, fmt=F.MXFP4, H_I=self.HI, d_I=self.dI, m=self.m,
                     n_cap=self.N, k=self.k, qi_scales=L["qis"], ki_scales=L["kscales"], out_idx=L["idx"],
                     with_scores=False)

    def attend(self, L):
        from compressed_sparse_long_02_amd import ops as F
        kw = dict(kv_fmt=F.KV_PACKED, kvw_pos0=0, kvw_rows=self.ring, W=self.W, H=self.H, d=self.d, r=self.r,
                  scale=self.scale, out_fmt=F.BF16, out=L["out"], with_lse=False)
        if L["kind"] == "csa":
            F.csa_attend(L["q"], L["cache"], L["idx"], L["ring"], self.q_pos, n_cap=self.N, **kw)
        else:
            F.hca_attend(L["q"], L["cache"], L["ring"], self.q_pos, n_cap=self.Nh, m=self.mh, **kw)

    def step(self):
        for L in self.layers:
            self.compress(L)
            if L["kind"] == "csa":
                self.index(L)
            self.attend(L)

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


COUNTERS = os.path.join(ROOT, "profiles", "index_topk_hbm_counters_stack_1M_b16.txt")
INDEX_SOURCES = ["compressed_sparse_long_02_amd/csrc/index_topk.hip", "compressed_sparse_long_02_amd/csrc/device.h",
                 "compressed_sparse_long_02_amd/csrc/launch.h"]


def recorded_traffic(B, ctx):
    """HBM bytes per index_topk launch from the committed FETCH_SIZE / WRITE_SIZE summary, when that
    summary was taken on this workload and the kernel sources are unchanged since; else None."""
    import hashlib
    if B != 16 or ctx != 1 << 20 or not os.path.exists(COUNTERS):
        return None
    fields = {}
    for line in open(COUNTERS):
        if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "source_sha256_16"):
            k, v = line.split(":", 1)
            fields[k] = v.split()[0]
    h = hashlib.sha256()
    for f in INDEX_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if fields.get("source_sha256_16") != h.hexdigest()[:16] or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


class Prefill:
    """One CSA layer appending a chunk of 8,192 tokens to 1,048,576 cached ones: compress the
    chunk's 2,048 entries (KV and bf16 indexer keys, with the 4 look-back rows), index the
    8,192 queries against the 264,192 entries (64 heads x 128, bf16, top-1024, causal) and
    attend with 128 heads of 512 over the selected entries plus a 128-token window."""

    def __init__(self, device):
        import torch
        from compressed_sparse_long_02_amd import gen
        self.H, self.d, self.r, self.m, self.HI, self.dI, self.k, self.W, self.C = 128, 512, 64, 4, 64, 128, 1024, 128, 8192
        self.T0 = 1 << 20
        self.N0 = self.T0 // self.m
        self.N = (self.T0 + self.C) // self.m
        d, r, dI, m, C, W = self.d, self.r, self.dI, self.m, self.C, self.W
        self.cache = torch.empty((1, self.N, d + r), dtype=torch.uint8, device=device)
        self.keys = torch.empty((1, self.N, dI * 2), dtype=torch.uint8, device=device)
        for s0 in range(0, self.N0, 32768):
            c = min(32768, self.N0 - s0)
            self.cache[:, s0:s0 + c] = gen.pack_kv(gen.normal((1, c, d), 5000 + s0, device=device), r)
            self.keys[:, s0:s0 + c] = gen.bf16_bytes(gen.normal((1, c, dI), 6000 + s0, device=device))
        self.x = gen.bf16_bytes(gen.normal((1, C + m, d), 7001, device=device))
        self.xi = gen.bf16_bytes(gen.normal((1, C + m, dI), 7002, device=device))
        self.z = gen.random_logits((1, C + m, 1), 7003, device=device)
        self.zi = gen.random_logits((1, C + m, 1), 7004, device=device)
        self.bias = gen.random_logits((2 * m, 1), 7005, device=device)
        self.bias_i = gen.random_logits((2 * m, 1), 7006, device=device)
        self.kvw = gen.pack_kv(gen.normal((1, W + C, d), 7007, device=device), r)
        self.q_pos = torch.arange(self.T0, self.T0 + C, dtype=torch.int32, device=device).view(1, C)
        self.qi = gen.bf16_bytes(gen.normal((1, C, self.HI, dI), 7008, device=device))
        self.w = gen.normal((1, C, self.HI), 7009, 1 / math.sqrt(self.HI), device=device)
        self.q = gen.normal((1, C, self.H, d), 7010, device=device).to(torch.bfloat16)
        self.idx = torch.empty((1, C, self.k), dtype=torch.int32, device=device)
        self.out = torch.empty((1, C, self.H, d), dtype=torch.bfloat16, device=device)
        torch.cuda.synchronize()

    def compress(self):
        from compressed_sparse_long_02_amd import ops as F
        ne = self.C // self.m
        kw = dict(m=self.m, overlap=True, e_begin=self.N0, n_e=ne, x_pos0=self.T0 - self.m)
        F.kv_compress(self.x, F.BF16, self.z, self.bias, d=self.d, r=self.r, out_fmt=F.KV_PACKED,
                      out=self.cache[:, self.N0:self.N], **kw)
        F.kv_compress(self.xi, F.BF16, self.zi, self.bias_i, d=self.dI, out_fmt=F.BF16,
                      out=self.keys[:, self.N0:self.N], **kw)

    def index(self):
        from compressed_sparse_long_02_amd import ops as F
        F.index_topk(self.qi, self.w, self.keys, self.q_pos, fmt=F.BF16, H_I=self.HI, d_I=self.dI, m=self.m,
                     n_cap=self.N, k=self.k, out_idx=self.idx, with_scores=False)

    def attend(self):
        from compressed_sparse_long_02_amd import ops as F
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


def prefill_cpu_baseline(pf, nq):
    """The oracle on `nq` of the chunk's queries (index + attend over the same inputs), timed on the
    host cores and scaled to the 8,192 queries of the chunk (compression excluded: < 0.1% of it)."""
    import numpy as np
    import torch
    import oracle as O
    sel = np.linspace(0, pf.C - 1, nq).astype(np.int64)
    h = lambda x: x.detach().cpu().numpy()
    qi, w, qpos = h(pf.qi[:, sel]), h(pf.w[:, sel]), h(pf.q_pos[:, sel])
    keys, cache, kvw, q = h(pf.keys), h(pf.cache), h(pf.kvw), h(pf.q[:, sel].view(torch.int16))
    t0 = time.perf_counter()
    idx, _ = O.index_topk(qi, O.BF16, w, keys, O.BF16, qpos, H_I=pf.HI, d_I=pf.dI, m=pf.m, n_cap=pf.N, k=pf.k)
    O.csa_attend(q, O.BF16, cache, O.KV_PACKED, pf.N, idx, kvw, pf.T0 - pf.W, pf.W + pf.C, qpos, W=pf.W, H=pf.H,
                 d=pf.d, r=pf.r, scale=1 / math.sqrt(pf.d))
    dt = time.perf_counter() - t0
    return {"value": round(nq / dt, 4), "unit": "tokens/s", "cores": min(nq, O.num_threads()), "kind": "oracle",
            "sample": "%d of the chunk's 8192 queries (index_topk + csa_attend), %.1f s on the host" % (nq, dt)}


def main_prefill(args):
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("[bench] building the prefill-chunk inputs", file=sys.stderr, flush=True)
    pf = Prefill(dev)
    pf.step()
    torch.cuda.synchronize()
    steps, warm = max(1, min(args.steps, 5)), max(1, min(args.warmup, 2))
    for _ in range(warm):
        pf.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        pf.step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    t_idx = time_calls(pf.index, 3)
    t_att = time_calls(pf.attend, 3)
    t_cmp = time_calls(pf.compress, 3)
    fi = pf.index_flops()
    ach = fi / (t_idx * 1e-3) / 1e12
    roof = {"bound": "mfma", "kernel": "index_topk (bf16 64x128 indexer, 8192 queries x 264,192 entries, top-1024)",
            "achieved": round(ach, 1), "peak": 2500.0, "unit": "TFLOP/s", "frac": round(ach / 2500.0, 4),
            "traffic": None, "flops_per_launch": fi, "ms_per_launch": round(t_idx, 3)}
    kernels = {"index_topk": {"ms": round(t_idx, 3), "TFLOP/s": round(ach, 1)},
               "csa_attend": {"ms": round(t_att, 3), "TFLOP/s": round(pf.attend_flops() / (t_att * 1e-3) / 1e12, 1)},
               "kv_compress_x2": {"ms": round(t_cmp, 3)}}
    cpu = None if args.no_cpu_baseline else prefill_cpu_baseline(pf, 48)
    line = {
        "metric": "CSA prefill-chunk tokens/sec at 1M ctx; indexer MFMA %", "value": round(pf.C / (ms * 1e-3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warm, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "CSA prefill chunk: 8192 tokens on 1,048,576 cached (compress + index + attend)",
                   "global_batch": 1, "seq_len": pf.T0 + pf.C, "heads": pf.H, "head_dim": pf.d,
                   "indexer": "bf16 64x128, top-k 1024", "parallelism": "single GPU"},
        "roofline": roof, "cpu_baseline": cpu, "kernels": kernels,
    }
    print(json.dumps(line), flush=True)


def time_sequence(calls, iters):
    """Average duration of each call of a repeating sequence, by HIP events recorded
    between the calls on torch's current stream.  Cycling through the layers of the
    stack keeps the working set above the 256 MB last-level cache, as in the step."""
    import torch
    s = torch.cuda.current_stream()
    for fn in calls:
        fn()
    n = len(calls)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n * iters + 1)]
    ev[0].record(s)
    for i in range(iters):
        for j, fn in enumerate(calls):
            fn()
            ev[i * n + j + 1].record(s)
    ev[-1].synchronize()
    tot = [0.0] * n
    for i in range(iters):
        for j in range(n):
            tot[j] += ev[i * n + j].elapsed_time(ev[i * n + j + 1])
    return [t / iters for t in tot]


def time_calls(fn, iters):
    """Average duration of fn() on torch's current stream, by HIP events."""
    import torch
    s = torch.cuda.current_stream()
    fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(iters):
        fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / iters


def cpu_baseline(st, nseq, min_s=10.0):
    """The oracle on a bounded sample: `nseq` sequences through one CSA layer and one
    HCA layer (compress the new entry, index, attend), timed on the host cores and
    repeated until about `min_s` seconds have passed (the median pass counts); scaled
    to tokens/s of the 4-layer stack (two CSA+HCA pairs)."""
    import numpy as np
    import torch
    import oracle as O

    h = lambda x: x[:nseq].detach().cpu().numpy()
    csa, hca = st.layers[0], st.layers[1]
    t, d, r = st.t, st.d, st.r
    arrs = dict(c_raw=h(csa["raw"]), c_z=h(csa["z"]), c_bias=csa["bias"].cpu().numpy(), c_rawi=h(csa["raw_i"]),
                c_zi=h(csa["z_i"]), c_biasi=csa["bias_i"].cpu().numpy(), qi=h(csa["qi"]), qis=h(csa["qis"]),
                w=h(csa["w"]), keys=h(csa["keys"]), ksc=h(csa["kscales"]), c_cache=h(csa["cache"]),
                c_ring=h(csa["ring"]), c_q=h(csa["q"].view(torch.int16)), h_raw=h(hca["raw"]), h_z=h(hca["z"]),
                h_bias=hca["bias"].cpu().numpy(), h_cache=h(hca["cache"]), h_ring=h(hca["ring"]),
                h_q=h(hca["q"].view(torch.int16)))
    qpos = np.full((nseq, 1), t, np.int32)
    a = arrs
    reps, total = [], 0.0
    while not reps or (total < min_s and len(reps) < 50):
        dt = _oracle_pass(st, a, qpos)
        reps.append(dt)
        total += dt
    dt = float(np.median(reps))
    value = nseq / (2.0 * dt)
    return {"value": round(value, 4), "unit": "tokens/s", "cores": min(nseq, O.num_threads()), "kind": "oracle",
            "sample": "%d of %d sequences through one CSA and one HCA layer (compress + index + attend), "
                      "median of %d passes (%.1f s each, %.1f s in all) on the host, x2 for the 4-layer stack"
                      % (nseq, st.B, len(reps), dt, total)}


def _oracle_pass(st, a, qpos):
    """One timed pass of the oracle over the sample (seconds)."""
    import oracle as O
    t, d, r = st.t, st.d, st.r
    t0 = time.perf_counter()
    i = (t + 1) // st.m - 1
    O.kv_compress(a["c_raw"], O.BF16, a["c_z"], a["c_bias"], d=d, r=r, m=st.m, overlap=True, e_begin=i, n_e=1,
                  x_pos0=t - 7, out_fmt=O.KV_PACKED)
    O.kv_compress(a["c_rawi"], O.BF16, a["c_zi"], a["c_biasi"], d=st.dI, m=st.m, overlap=True, e_begin=i, n_e=1,
                  x_pos0=t - 7, out_fmt=O.MXFP4)
    idx, _ = O.index_topk(a["qi"], O.MXFP4, a["w"], a["keys"], O.MXFP4, qpos, H_I=st.HI, d_I=st.dI, m=st.m,
                          n_cap=st.N, k=st.k, qi_scales=a["qis"], ki_scales=a["ksc"])
    O.csa_attend(a["c_q"], O.BF16, a["c_cache"], O.KV_PACKED, st.N, idx, a["c_ring"], 0, st.ring, qpos, W=st.W,
                 H=st.H, d=d, r=r, scale=st.scale)
    ih = (t + 1) // st.mh - 1
    O.kv_compress(a["h_raw"], O.BF16, a["h_z"], a["h_bias"], d=d, r=r, m=st.mh, overlap=False, e_begin=ih, n_e=1,
                  x_pos0=t - 127, out_fmt=O.KV_PACKED)
    O.hca_attend(a["h_q"], O.BF16, a["h_cache"], O.KV_PACKED, st.Nh, st.mh, a["h_ring"], 0, st.ring, qpos,
                 W=st.W, H=st.H, d=d, r=r, scale=st.scale)
    return time.perf_counter() - t0


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.workload == "prefill":
        return main_prefill(args)
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("[bench] building inputs (B=%d, ctx=%d)" % (args.batch, args.ctx), file=sys.stderr, flush=True)
    st = Stack(args.batch, args.ctx, dev)
    st.step()                       # eager warm-up: allocates workspaces before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            st.step()
    torch.cuda.synchronize()
    print("[bench] graph captured; warmup %d, timed %d" % (args.warmup, args.steps), file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    value = args.batch / (ms / 1e3)
    # spread of single steps: the same replays, one HIP event pair each (not the headline)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in ev:
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    per = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    pct = lambda f: per[min(len(per) - 1, int(f * len(per)))]
    step_ms = {"p10": round(pct(0.1), 4), "p50": round(pct(0.5), 4), "p90": round(pct(0.9), 4)}
    # per-call durations (HIP events on the launching stream), eager launches in step
    # order through all four layers
    L0, L1, L2, L3 = st.layers
    tt = time_sequence([lambda: st.index(L0), lambda: st.attend(L0), lambda: st.attend(L1),
                        lambda: st.index(L2), lambda: st.attend(L2), lambda: st.attend(L3)], args.kernel_iters)
    t_idx, t_csa, t_hca = (tt[0] + tt[3]) / 2, (tt[1] + tt[4]) / 2, (tt[2] + tt[5]) / 2
    ib = st.index_bytes()
    ach = ib / (t_idx * 1e-3) / 1e9
    roof = {"bound": "hbm", "kernel": "index_topk (MXFP4 scores + top-1024 of 262,144 per sequence)",
            "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(args.batch, args.ctx), "bytes_per_launch": ib, "ms_per_launch": round(t_idx, 4)}
    kernels = {
        "index_topk": {"ms": round(t_idx, 4), "GB/s": round(ach, 1)},
        "csa_attend": {"ms": round(t_csa, 4), "GB/s": round(st.csa_bytes() / (t_csa * 1e-3) / 1e9, 1)},
        "hca_attend": {"ms": round(t_hca, 4), "GB/s": round(st.hca_bytes() / (t_hca * 1e-3) / 1e9, 1)},
        "step_GB/s": round(st.step_bytes() / (ms * 1e-3) / 1e9, 1),
        "step_ms": step_ms,
        "step_bytes": st.step_bytes(),
    }
    if args.copy_mb > 0:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE per dispatch calibrate the counters
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] oracle CPU baseline on %d sequences" % args.cpu_seqs, file=sys.stderr, flush=True)
        cpu = cpu_baseline(st, args.cpu_seqs)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp4+bf16", "data": "synthetic",
        "config": {"workload": "4-layer CSA,HCA,CSA,HCA decode at 1M ctx (t=2^20-1), batch %d" % args.batch,
                   "global_batch": args.batch, "seq_len": args.ctx, "heads": 64, "head_dim": 512,
                   "kv": "bf16 rope64 + fp8 e4m3 (576 B)", "indexer": "MXFP4 64x128, top-k 1024", "m": 4,
                   "m_hca": 128, "window": 128, "parallelism": "single GPU"},
        "roofline": roof, "cpu_baseline": cpu, "kernels": kernels,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
