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
    p.add_argument("--workload", choices=["stack", "prefill", "csa_decode", "hca_decode"], default="stack",
                   help="stack: the 4-layer decode stack (default); prefill: one CSA prefill chunk; csa_decode: one "
                        "CSA layer, batch 8 at 128K; hca_decode: one HCA layer, batch 4 at 1M")
    p.add_argument("--indexer", choices=["bf16", "mxfp4"], default="bf16",
                   help="prefill workload: the indexer's queries and keys in bf16 (default) or MXFP4")
    p.add_argument("--layout", choices=["linear", "paged"], default="linear",
                   help="compressed cache of the stack: dense per sequence, or 128-token blocks behind a block table")
    p.add_argument("--copy-mb", type=int, default=0,
                   help="also run a plain device copy of this many MiB (the reference kernel for HBM counters)")
    return p.parse_args()


COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters_stack_1M_b16.txt")
INDEX_SOURCES = ["compressed_sparse_long_02_amd/csrc/index_topk.hip", "compressed_sparse_long_02_amd/csrc/device.h",
                 "compressed_sparse_long_02_amd/csrc/launch.h"]


def recorded_traffic(B, ctx, layout):
    """HBM bytes per index_topk launch from the committed FETCH_SIZE / WRITE_SIZE summary, when that
    summary was taken on this workload (linear caches) and the kernel sources are unchanged since;
    else None."""
    import hashlib
    if B != 16 or ctx != 1 << 20 or layout != "linear" or not os.path.exists(COUNTERS):
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
    sc = {} if pf.qis is None else dict(qi_scales=h(pf.qis[:, sel]), ki_scales=h(pf.kscales))
    t0 = time.perf_counter()
    idx, _ = O.index_topk(qi, pf.key_fmt, w, keys, pf.key_fmt, qpos, H_I=pf.HI, d_I=pf.dI, m=pf.m, n_cap=pf.N,
                          k=pf.k, **sc)
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
    from compressed_sparse_long_02_amd import ops
    from compressed_sparse_long_02_amd.workloads import Prefill
    fp4 = args.indexer == "mxfp4"
    pf = Prefill(dev, key_fmt=ops.MXFP4 if fp4 else ops.BF16)
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
    peak = 10100.0 if fp4 else 2500.0                  # dense FP4 / bf16 MFMA peaks of the part
    roof = {"bound": "mfma", "kernel": "index_topk (%s 64x128 indexer, 8192 queries x 264,192 entries, top-1024)"
                                       % args.indexer,
            "achieved": round(ach, 1), "peak": peak, "unit": "TFLOP/s", "frac": round(ach / peak, 4),
            "traffic": None, "flops_per_launch": fi, "ms_per_launch": round(t_idx, 3)}
    kernels = {"index_topk": {"ms": round(t_idx, 3), "TFLOP/s": round(ach, 1)},
               "csa_attend": {"ms": round(t_att, 3), "TFLOP/s": round(pf.attend_flops() / (t_att * 1e-3) / 1e12, 1)},
               "kv_compress_x2": {"ms": round(t_cmp, 3)}}
    cpu = None if args.no_cpu_baseline else prefill_cpu_baseline(pf, 48)
    line = {
        "metric": "CSA prefill-chunk tokens/sec at 1M ctx; indexer MFMA %", "value": round(pf.C / (ms * 1e-3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warm, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "mxfp4+bf16" if fp4 else "bf16",
        "data": "synthetic",
        "config": {"workload": "CSA prefill chunk: 8192 tokens on 1,048,576 cached (compress + index + attend)",
                   "global_batch": 1, "seq_len": pf.T0 + pf.C, "heads": pf.H, "head_dim": pf.d,
                   "indexer": "%s 64x128, top-k 1024" % args.indexer, "parallelism": "single GPU"},
        "roofline": roof, "cpu_baseline": cpu, "kernels": kernels,
    }
    print(json.dumps(line), flush=True)


def layer_cpu_baseline(ly, min_s=10.0):
    """The oracle on the whole batch of one input set (compress the new entry, index, attend),
    repeated until about min_s seconds have passed; the median pass counts."""
    import numpy as np
    import torch
    import oracle as O
    S = ly.sets[0]
    h = lambda x: x.detach().cpu().numpy()
    a = {k: h(v) for k, v in S.items() if torch.is_tensor(v) and k not in ("out", "idx", "q")}
    a["q"] = h(S["q"].view(torch.int16))
    qpos = np.full((ly.B, 1), ly.t, np.int32)
    i = (ly.t + 1) // ly.m - 1
    okw = dict(W=ly.W, H=ly.H, d=ly.d, r=ly.r, scale=ly.scale)
    reps, total = [], 0.0
    while not reps or (total < min_s and len(reps) < 50):
        t0 = time.perf_counter()
        O.kv_compress(a["raw"], O.BF16, a["z"], a["bias"], d=ly.d, r=ly.r, m=ly.m, overlap=ly.kind == "csa_decode",
                      e_begin=i, n_e=1, x_rows=ly.RING, out_fmt=O.KV_PACKED)
        if ly.kind == "csa_decode":
            O.kv_compress(a["raw_i"], O.BF16, a["z_i"], a["bias_i"], d=ly.dI, m=ly.m, overlap=True, e_begin=i, n_e=1,
                          x_rows=ly.RING, out_fmt=O.BF16)
            idx, _ = O.index_topk(a["qi"], O.BF16, a["w"], a["keys"], O.BF16, qpos, H_I=ly.HI, d_I=ly.dI, m=ly.m,
                                  n_cap=ly.N, k=ly.k)
            O.csa_attend(a["q"], O.BF16, a["cache"], O.KV_PACKED, ly.N, idx, a["ring"], 0, 256, qpos, **okw)
        else:
            O.hca_attend(a["q"], O.BF16, a["cache"], O.KV_PACKED, ly.N, ly.m, a["ring"], 0, 256, qpos, **okw)
        dt = time.perf_counter() - t0
        reps.append(dt)
        total += dt
    dt = float(np.median(reps))
    return {"value": round(ly.B / dt, 4), "unit": "tokens/s", "cores": min(ly.B, O.num_threads()), "kind": "oracle",
            "sample": "the whole batch (%d sequences) of one input set through the layer (compress + %s), median of "
                      "%d passes (%.2f s each) on the host" % (ly.B, "index + attend" if ly.kind == "csa_decode"
                                                               else "attend", len(reps), dt)}


def main_layer(args):
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    copies = 3 if args.workload == "csa_decode" else 28
    print("[bench] building %s inputs (%d copies)" % (args.workload, copies), file=sys.stderr, flush=True)
    from compressed_sparse_long_02_amd.workloads import Layer
    ly = Layer(args.workload, dev, copies)
    for S in ly.sets:
        ly.step(S)
    torch.cuda.synchronize()
    graphs = []
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    for S in ly.sets:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                ly.step(S)
        graphs.append(g)
    torch.cuda.synchronize()
    print("[bench] graphs captured; warmup %d, timed %d" % (args.warmup, args.steps), file=sys.stderr, flush=True)
    n = len(graphs)
    for i in range(args.warmup):
        graphs[i % n].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % n].replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # per-call durations, cycling through the input sets
    if args.workload == "csa_decode":
        calls = [f for S in ly.sets for f in (lambda S=S: ly.index(S), lambda S=S: ly.attend(S))]
        tt = time_sequence(calls, args.kernel_iters)
        t_idx = sum(tt[0::2]) / n
        t_att = sum(tt[1::2]) / n
    else:
        tt = time_sequence([lambda S=S: ly.attend(S) for S in ly.sets], args.kernel_iters)
        t_idx, t_att = None, sum(tt) / n
    tc = time_sequence([lambda S=S: ly.compress(S) for S in ly.sets], max(3, args.kernel_iters // 4))
    t_cmp = sum(tc) / n
    kernels = {"csa_attend" if args.workload == "csa_decode" else "hca_attend":
               {"ms": round(t_att, 4), "GB/s": round(ly.attend_bytes() / (t_att * 1e-3) / 1e9, 1)},
               "kv_compress_step": {"ms": round(t_cmp, 4)},
               "step_GB/s": round(ly.step_bytes() / (ms * 1e-3) / 1e9, 1), "step_bytes": ly.step_bytes(),
               "input_sets": n}
    if t_idx is not None:
        kernels["index_topk"] = {"ms": round(t_idx, 4), "GB/s": round(ly.index_bytes() / (t_idx * 1e-3) / 1e9, 1)}
        dom, db, dt = "index_topk (bf16 16x128 scores + top-512 of 32,768 per sequence)", ly.index_bytes(), t_idx
    else:
        dom, db, dt = "hca_attend (64 heads x 512 over 8,192 entries + 128-token window)", ly.attend_bytes(), t_att
    ach = db / (dt * 1e-3) / 1e9
    roof = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "bytes_per_launch": db, "ms_per_launch": round(dt, 4)}
    cpu = None if args.no_cpu_baseline else layer_cpu_baseline(ly)
    wl = ("CSA decode layer: batch 8 at 131,072 tokens (32,768 entries), bf16 indexer 16x128 top-512"
          if args.workload == "csa_decode" else "HCA decode layer: batch 4 at 1,048,576 tokens (8,192 entries)")
    line = {
        "metric": METRIC, "value": round(ly.B / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl, "global_batch": ly.B, "seq_len": ly.ctx, "heads": ly.H, "head_dim": ly.d,
                   "kv": "bf16 rope64 + fp8 e4m3 (576 B)", "m": ly.m, "window": ly.W, "parallelism": "single GPU"},
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
    keys, kscales = st.index_keys(csa)
    arrs = dict(c_raw=h(csa["raw"]), c_z=h(csa["z"]), c_bias=csa["bias"].cpu().numpy(), c_rawi=h(csa["raw_i"]),
                c_zi=h(csa["z_i"]), c_biasi=csa["bias_i"].cpu().numpy(), qi=h(csa["qi"]), qis=h(csa["qis"]),
                w=h(csa["w"]), keys=h(keys), ksc=h(kscales), c_cache=h(st.entries(csa)),
                c_ring=h(csa["ring"]), c_q=h(csa["q"].view(torch.int16)), h_raw=h(hca["raw"]), h_z=h(hca["z"]),
                h_bias=hca["bias"].cpu().numpy(), h_cache=h(st.entries(hca)), h_ring=h(hca["ring"]),
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
                  x_rows=st.RING, out_fmt=O.KV_PACKED)
    O.kv_compress(a["c_rawi"], O.BF16, a["c_zi"], a["c_biasi"], d=st.dI, m=st.m, overlap=True, e_begin=i, n_e=1,
                  x_rows=st.RING, out_fmt=O.MXFP4)
    idx, _ = O.index_topk(a["qi"], O.MXFP4, a["w"], a["keys"], O.MXFP4, qpos, H_I=st.HI, d_I=st.dI, m=st.m,
                          n_cap=st.N, k=st.k, qi_scales=a["qis"], ki_scales=a["ksc"])
    O.csa_attend(a["c_q"], O.BF16, a["c_cache"], O.KV_PACKED, st.N, idx, a["c_ring"], 0, st.ring, qpos, W=st.W,
                 H=st.H, d=d, r=r, scale=st.scale)
    ih = (t + 1) // st.mh - 1
    O.kv_compress(a["h_raw"], O.BF16, a["h_z"], a["h_bias"], d=d, r=r, m=st.mh, overlap=False, e_begin=ih, n_e=1,
                  x_rows=st.RING, out_fmt=O.KV_PACKED)
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
    if args.workload in ("csa_decode", "hca_decode"):
        return main_layer(args)
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("[bench] building inputs (B=%d, ctx=%d)" % (args.batch, args.ctx), file=sys.stderr, flush=True)
    from compressed_sparse_long_02_amd.workloads import Stack
    st = Stack(args.batch, args.ctx, dev, layout=args.layout)
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
            "traffic": recorded_traffic(args.batch, args.ctx, args.layout), "bytes_per_launch": ib, "ms_per_launch": round(t_idx, 4)}
    # the indexer's contraction as MFMA work: 2 * H_I * d_I flops per (query, entry), on the
    # scaled FP4 MFMA (dense fp4 peak 10.1 PFLOP/s)
    idx_tf = 2.0 * st.HI * st.dI * st.N * st.B / (t_idx * 1e-3) / 1e12
    kernels = {
        "index_topk": {"ms": round(t_idx, 4), "GB/s": round(ach, 1), "TFLOP/s": round(idx_tf, 1),
                       "mfma_frac_fp4": round(idx_tf / 10100.0, 4)},
        "csa_attend": {"ms": round(t_csa, 4), "GB/s": round(st.csa_bytes() / (t_csa * 1e-3) / 1e9, 1)},
        "hca_attend": {"ms": round(t_hca, 4), "GB/s": round(st.hca_bytes() / (t_hca * 1e-3) / 1e9, 1)},
        "step_GB/s": round(st.step_bytes() / (ms * 1e-3) / 1e9, 1),
        "step_ms": step_ms,
        "step_bytes": st.step_bytes(),
    }
    # the grouped output projection after each layer's attention (not part of the
    # configured step): 64 heads x 512 in 8 groups -> 8 x 1024, the batch's 16 tokens
    G, R = 8, 1024
    K = st.H * st.d // G
    xo = st.layers[0]["out"].reshape(st.B, st.H * st.d)
    wo = torch.randn((G, R, K), device=dev, dtype=torch.float32).mul_(K ** -0.5).to(torch.bfloat16)
    yo = torch.empty((st.B, G * R), dtype=torch.bfloat16, device=dev)
    from compressed_sparse_long_02_amd import ops as F
    t_op = time_calls(lambda: F.grouped_out_proj(xo, wo, G=G, out_fmt=F.BF16, out=yo), args.kernel_iters)
    op_bytes = G * R * K * 2 + st.B * st.H * st.d * 2 + st.B * G * R * 2
    kernels["grouped_out_proj (decode, not in the step)"] = {"ms": round(t_op, 4),
                                                             "GB/s": round(op_bytes / (t_op * 1e-3) / 1e9, 1)}
    del wo
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
                   "cache_layout": args.layout,
                   "global_batch": args.batch, "seq_len": args.ctx, "heads": 64, "head_dim": 512,
                   "kv": "bf16 rope64 + fp8 e4m3 (576 B)", "indexer": "MXFP4 64x128, top-k 1024", "m": 4,
                   "m_hca": 128, "window": 128, "parallelism": "single GPU"},
        "roofline": roof, "cpu_baseline": cpu, "kernels": kernels,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
