"""GPU parity of index_topk against the oracle (lightning indexer + top-k: x-techcon
article, section 2, CSA step 2; FP4 indexer QK: the mixed-precision paragraph and
section 4).  Index sets must match except for swaps between entries whose oracle
scores tie with the k-th score within the fp32 accumulation bound."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from compressed_sparse_long_02_amd import gen, ops
from tests import bruteforce as BF
from tests.gpu_util import check_topk, dev, host, oracle_all_scores, score_error_bound

pytestmark = pytest.mark.gpu


def _inputs(fmt, B, Tq, H_I, d_I, N, seed):
    """Stored q / keys (bytes) and their exact decoded values."""
    if fmt == O.MXFP4:
        qc, qs = gen.random_mxfp4(B * Tq * H_I, d_I, seed)
        kc, ks = gen.random_mxfp4(B * N, d_I, seed + 1)
        qc, qs = qc.reshape(B, Tq, H_I, -1), qs.reshape(B, Tq, H_I, -1)
        kc, ks = kc.reshape(B, N, -1), ks.reshape(B, N, -1)
        qd = BF.decode(host(qc), BF.MXFP4, d_I, scales=host(qs)).reshape(B, Tq, H_I, d_I)
        kd = BF.decode(host(kc), BF.MXFP4, d_I, scales=host(ks)).reshape(B, N, d_I)
        return qc, qs, kc, ks, qd, kd
    q = gen.normal((B, Tq, H_I, d_I), seed, 1 / math.sqrt(d_I))
    k = gen.normal((B, N, d_I), seed + 1, 1 / math.sqrt(d_I))
    qs_, ks_ = gen.store(q, fmt), gen.store(k, fmt)
    qd = BF.decode(host(qs_), fmt, d_I).reshape(B, Tq, H_I, d_I)
    kd = BF.decode(host(ks_), fmt, d_I).reshape(B, N, d_I)
    return qs_, None, ks_, None, qd, kd


CASES = [
    # (fmt, B, Tq, H_I, d_I, N, m, k, positions)
    ("cfg1", O.F32, 1, 64, 4, 32, 512, 4, 64, "last"),        # config 1 indexer: single slice
    ("bf16_multi", O.BF16, 2, 3, 16, 128, 4096, 4, 512, "last"),  # config-2-like, split path
    ("bf16_ragged", O.BF16, 3, 4, 16, 64, 3000, 4, 256, "ragged"),
    ("fp4_multi", O.MXFP4, 2, 2, 64, 128, 20000, 4, 1024, "last"),
    ("fp4_short", O.MXFP4, 2, 3, 64, 128, 5000, 4, 1024, "ragged"),  # n(t) < k: padding
    ("f32_128", O.F32, 1, 5, 8, 128, 700, 1, 33, "ragged"),
]


def _positions(kind, B, Tq, N, m):
    if kind == "last":
        return gen.positions(B, Tq, N * m - 1)
    rng = np.random.default_rng(5)
    p = rng.integers(-2, N * m + 40, size=(B, Tq)).astype(np.int32)
    p[0, 0] = 2          # no entry visible yet (t < m - 1 for m = 4)
    p[-1, -1] = N * m - 1
    return torch.from_numpy(p)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_index_topk_parity(gpu, case):
    _, fmt, B, Tq, H_I, d_I, N, m, k, pk = case
    qi, qs, ki, ks, qd, kd = _inputs(fmt, B, Tq, H_I, d_I, N, 300 + N)
    w = gen.normal((B, Tq, H_I), 301 + N, 1 / math.sqrt(H_I))
    qpos = _positions(pk, B, Tq, N, m).to(torch.int32)
    kw = dict(H_I=H_I, d_I=d_I, m=m, n_cap=N)
    gi, gs = ops.index_topk(dev(qi), dev(w), dev(ki), dev(qpos), fmt=fmt, k=k, qi_scales=dev(qs) if qs is not None
                            else None, ki_scales=dev(ks) if ks is not None else None, **kw)
    torch.cuda.synchronize()
    oq = dict(qi_scales=None if qs is None else host(qs), ki_scales=None if ks is None else host(ks))
    oi, osc = O.index_topk(host(qi), fmt, host(w), host(ki), fmt, host(qpos), k=k, **kw, **oq)
    allsc = oracle_all_scores(host(qi), fmt, host(w), host(ki), fmt, host(qpos), **kw, **oq)
    bound = np.stack([score_error_bound(qd[b], host(w)[b].astype(np.float64), kd[b]) for b in range(B)])
    n_sw, gap = check_topk(host(gi), oi, allsc, k, abs_bound=bound)
    # scores of the selected entries: fp32 vs fp64 within the accumulation bound
    gi_h, gs_h = host(gi), host(gs)
    for b in range(B):
        for j in range(Tq):
            v = gi_h[b, j] >= 0
            ref = allsc[b, j, gi_h[b, j, v]]
            assert np.all(np.abs(gs_h[b, j, v] - ref) <= bound[b, j] + 1e-6 * np.abs(ref)), (b, j)
            assert np.all(np.isneginf(gs_h[b, j, ~v]))
    print("case %s: queries with tie swaps %d, largest gap %.3g" % (case[0], n_sw, gap))


@pytest.mark.parametrize("N,k", [(3000, 100), (30000, 1024)])
def test_index_topk_ties_take_the_smallest_indices(gpu, N, k):
    # every key identical -> every score ties -> the first k indices win (the larger
    # case leaves more tied candidates than the split path's filter keeps in LDS, so
    # the row select refines the threshold down to the last key bit)
    B, Tq, H_I, d_I = 1, 2, 16, 128
    q = gen.normal((B, Tq, H_I, d_I), 1)
    key = gen.normal((1, 1, d_I), 2).expand(B, N, d_I).contiguous()
    w = torch.ones((B, Tq, H_I))
    qpos = gen.positions(B, Tq, 4 * N - 1)
    gi, _ = ops.index_topk(dev(gen.store(q, O.BF16)), dev(w), dev(gen.store(key, O.BF16)), dev(qpos), fmt=O.BF16,
                           H_I=H_I, d_I=d_I, m=4, n_cap=N, k=k)
    torch.cuda.synchronize()
    assert np.array_equal(host(gi)[0, 0], np.arange(k))
    assert np.array_equal(host(gi)[0, 1], np.arange(k))


def test_index_topk_clustered_scores_refine_the_threshold(gpu):
    # keys = one shared key + 1% noise: nearly every score lands in the same top-11-bit
    # bin, more candidates than the split path's filter keeps in LDS, so the row select
    # refines the threshold with the next digits
    B, Tq, H_I, d_I, N, k = 1, 2, 16, 128, 40000, 1024
    base = gen.normal((1, 1, d_I), 21)
    keys = base.expand(B, N, d_I) + 0.01 * gen.normal((B, N, d_I), 22)
    q = gen.normal((B, Tq, H_I, d_I), 23)
    w = torch.ones((B, Tq, H_I))
    qpos = gen.positions(B, Tq, 4 * N - 1)
    qs_, ks_ = gen.store(q, O.BF16), gen.store(keys, O.BF16)
    kw = dict(H_I=H_I, d_I=d_I, m=4, n_cap=N)
    gi, _ = ops.index_topk(dev(qs_), dev(w), dev(ks_), dev(qpos), fmt=O.BF16, k=k, **kw)
    torch.cuda.synchronize()
    oi, _ = O.index_topk(host(qs_), O.BF16, host(w), host(ks_), O.BF16, host(qpos), k=k, **kw)
    allsc = oracle_all_scores(host(qs_), O.BF16, host(w), host(ks_), O.BF16, host(qpos), **kw)
    qd = BF.decode(host(qs_), O.BF16, d_I).reshape(B, Tq, H_I, d_I)
    kd = BF.decode(host(ks_), O.BF16, d_I).reshape(B, N, d_I)
    bound = np.stack([score_error_bound(qd[0], host(w)[0].astype(np.float64), kd[0])])
    s = np.sort(allsc[0, 0][np.isfinite(allsc[0, 0])])[::-1]
    assert s[-1] > 0.95 * s[0]                                # one narrow band of scores
    check_topk(host(gi), oi, allsc, k, abs_bound=bound)


def test_index_topk_filter_blocks_span_several_slices(gpu):
    # 16 queries x 300,000 MXFP4 keys: slices of 16,384 keys, 19 per query, two slices per
    # filter block; rows that end inside a slice, on a slice boundary, below k and empty
    B, N, H_I, d_I, m, k = 16, 300000, 64, 128, 4, 1024
    qc, qs = gen.random_mxfp4(B * H_I, d_I, 41)
    kc, ks = gen.random_mxfp4(B * N, d_I, 42, device="cuda")
    qc, qs = qc.reshape(B, 1, H_I, -1), qs.reshape(B, 1, H_I, -1)
    kc, ks = kc.reshape(B, N, -1), ks.reshape(B, N, -1)
    w = gen.normal((B, 1, H_I), 43, 1 / math.sqrt(H_I))
    n_of = [N] * B
    n_of[1], n_of[2], n_of[3], n_of[4] = 17 * 16384 + 5, 2 * 16384, 700, 0
    qpos = torch.tensor([[n * m - 1 if n > 0 else 1] for n in n_of], dtype=torch.int32)   # n(t) = n
    gi, _ = ops.index_topk(dev(qc), dev(w), kc, dev(qpos), fmt=O.MXFP4, H_I=H_I, d_I=d_I, m=m, n_cap=N, k=k,
                           qi_scales=dev(qs), ki_scales=ks)
    torch.cuda.synchronize()
    gi_h = host(gi)
    assert np.all(gi_h[4, 0] == -1)
    assert np.array_equal(gi_h[3, 0, :700], np.arange(700)) and np.all(gi_h[3, 0, 700:] == -1)
    for b in (0, 1, 2):
        sl = slice(b, b + 1)
        kw = dict(H_I=H_I, d_I=d_I, m=m, n_cap=N)
        oq = dict(qi_scales=host(qs[sl]), ki_scales=host(ks[sl]))
        oi, _ = O.index_topk(host(qc[sl]), O.MXFP4, host(w[sl]), host(kc[sl]), O.MXFP4, host(qpos[sl]), k=k, **kw, **oq)
        allsc = oracle_all_scores(host(qc[sl]), O.MXFP4, host(w[sl]), host(kc[sl]), O.MXFP4, host(qpos[sl]), **kw, **oq)
        qd = BF.decode(host(qc[sl]), BF.MXFP4, d_I, scales=host(qs[sl])).reshape(1, H_I, d_I)
        kd = BF.decode(host(kc[sl]), BF.MXFP4, d_I, scales=host(ks[sl])).reshape(N, d_I)
        bound = score_error_bound(qd, host(w[sl])[0].astype(np.float64), kd)
        check_topk(gi_h[sl], oi, allsc, k, abs_bound=bound[None])


def test_index_topk_is_deterministic(gpu):
    B, Tq, H_I, d_I, N, k = 2, 2, 64, 128, 30000, 1024
    qc, qs = gen.random_mxfp4(B * Tq * H_I, d_I, 11)
    kc, ks = gen.random_mxfp4(B * N, d_I, 12)
    w = gen.normal((B, Tq, H_I), 13)
    qpos = gen.positions(B, Tq, 4 * N - 1)
    args = (dev(qc.reshape(B, Tq, H_I, -1)), dev(w), dev(kc.reshape(B, N, -1)), dev(qpos))
    kw = dict(fmt=O.MXFP4, H_I=H_I, d_I=d_I, m=4, n_cap=N, k=k, qi_scales=dev(qs.reshape(B, Tq, H_I, -1)),
              ki_scales=dev(ks.reshape(B, N, -1)))
    a = ops.index_topk(*args, **kw)
    b = ops.index_topk(*args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


DENSE_CASES = [
    # (name, B, Tq, H_I, N, m, k, positions): Tq >= 64 with a bf16 d_I = 128 indexer takes the
    # many-query path (every score to HBM, then one select per query)
    ("dense_h64", 1, 96, 64, 20000, 4, 512, "ragged"),
    ("dense_h16_b2", 2, 64, 16, 9000, 4, 256, "ragged"),
    ("dense_h32_small_n", 1, 70, 32, 700, 1, 1024, "ragged"),     # many queries with n(t) < k
]


@pytest.mark.parametrize("case", DENSE_CASES, ids=[c[0] for c in DENSE_CASES])
def test_index_topk_many_queries(gpu, case):
    _, B, Tq, H_I, N, m, k, pk = case
    d_I, fmt = 128, O.BF16
    qi, _, ki, _, qd, kd = _inputs(fmt, B, Tq, H_I, d_I, N, 900 + N)
    w = gen.normal((B, Tq, H_I), 901 + N, 1 / math.sqrt(H_I))
    qpos = _positions(pk, B, Tq, N, m).to(torch.int32)
    kw = dict(H_I=H_I, d_I=d_I, m=m, n_cap=N)
    gi, gs = ops.index_topk(dev(qi), dev(w), dev(ki), dev(qpos), fmt=fmt, k=k, **kw)
    torch.cuda.synchronize()
    oi, _ = O.index_topk(host(qi), fmt, host(w), host(ki), fmt, host(qpos), k=k, **kw)
    allsc = oracle_all_scores(host(qi), fmt, host(w), host(ki), fmt, host(qpos), **kw)
    bound = np.stack([score_error_bound(qd[b], host(w)[b].astype(np.float64), kd[b]) for b in range(B)])
    n_sw, gap = check_topk(host(gi), oi, allsc, k, abs_bound=bound)
    gi_h, gs_h = host(gi), host(gs)
    for b in range(B):
        for j in range(Tq):
            v = gi_h[b, j] >= 0
            ref = allsc[b, j, gi_h[b, j, v]]
            assert np.all(np.abs(gs_h[b, j, v] - ref) <= bound[b, j] + 1e-6 * np.abs(ref)), (b, j)
            assert np.all(np.isneginf(gs_h[b, j, ~v]))
    print("case %s: queries with tie swaps %d, largest gap %.3g" % (case[0], n_sw, gap))


def test_index_topk_many_queries_all_tied(gpu):
    # every score equal: the select refines all three digit levels and keeps the
    # k smallest indices among more tied keys than it can hold
    B, Tq, H_I, d_I, N, k = 1, 64, 16, 128, 12000, 1000
    q = gen.normal((B, Tq, H_I, d_I), 31)
    key = gen.normal((1, 1, d_I), 32).expand(B, N, d_I).contiguous()
    w = torch.ones((B, Tq, H_I))
    qpos = gen.positions(B, Tq, 4 * N - 1)
    gi, _ = ops.index_topk(dev(gen.store(q, O.BF16)), dev(w), dev(gen.store(key, O.BF16)), dev(qpos), fmt=O.BF16,
                           H_I=H_I, d_I=d_I, m=4, n_cap=N, k=k)
    torch.cuda.synchronize()
    assert np.array_equal(host(gi)[0], np.tile(np.arange(k), (Tq, 1)))


@pytest.mark.parametrize("order", ["rising", "falling"])
def test_index_topk_many_queries_survivors_in_one_section(gpu, order):
    # scores that rise (or fall) with the entry index: the keys at and above the first
    # threshold bin all sit in one end of each query's row, more than one wave's share of
    # the row select's survivor buffer, so the select takes its block-wide fallback scan
    B, Tq, H_I, d_I, N, m, k = 1, 64, 16, 128, 24000, 4, 1024
    v = gen.normal((d_I,), 71, 1 / math.sqrt(d_I))
    ramp = torch.linspace(0.5, 1.5, N) if order == "rising" else torch.linspace(1.5, 0.5, N)
    key = (ramp[:, None] * v[None, :]).reshape(1, N, d_I)
    q = v.reshape(1, 1, 1, d_I).expand(B, Tq, H_I, d_I).contiguous()
    w = torch.full((B, Tq, H_I), 1.0 / H_I)
    qi, ki = gen.store(q, O.BF16), gen.store(key, O.BF16)
    qpos = gen.positions(B, Tq, N * m - 1)
    kw = dict(H_I=H_I, d_I=d_I, m=m, n_cap=N)
    gi, _ = ops.index_topk(dev(qi), dev(w), dev(ki), dev(qpos), fmt=O.BF16, k=k, **kw)
    torch.cuda.synchronize()
    oi, _ = O.index_topk(host(qi), O.BF16, host(w), host(ki), O.BF16, host(qpos), k=k, **kw)
    allsc = oracle_all_scores(host(qi), O.BF16, host(w), host(ki), O.BF16, host(qpos), **kw)
    qd = BF.decode(host(qi), O.BF16, d_I).reshape(B, Tq, H_I, d_I)
    kd = BF.decode(host(ki), O.BF16, d_I).reshape(B, N, d_I)
    bound = np.stack([score_error_bound(qd[b], host(w)[b].astype(np.float64), kd[b]) for b in range(B)])
    check_topk(host(gi), oi, allsc, k, abs_bound=bound)
    sel = host(gi)[0]
    assert (sel.min(axis=1) > N // 2).all() if order == "rising" else (sel.max(axis=1) < N // 2).all()
