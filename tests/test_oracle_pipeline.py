"""Whole-layer pins on tiny inputs: compress -> index -> attend through the oracle
against the numpy brute force, and the storage arithmetic the pages quote."""
import math

import numpy as np

import oracle as O
from tests import bruteforce as BF


def test_tiny_csa_layer_end_to_end():
    # a scaled-down CSA layer: T=64 raw tokens, d=16 (rope 4), m=4 with a 2m window,
    # indexer 2 heads of dim 8, k=4, window 8, queries at the last 6 positions
    rng = np.random.default_rng(41)
    T, d, r, m, HI, dI, k, W, H = 64, 16, 4, 4, 2, 8, 4, 8, 3
    raw = (rng.standard_normal((1, T, d)) / math.sqrt(d)).astype(np.float32)
    z = rng.standard_normal((1, T, 1)).astype(np.float32)
    bias = rng.standard_normal((2 * m, 1)).astype(np.float32)
    raw_i = (rng.standard_normal((1, T, dI)) / math.sqrt(dI)).astype(np.float32)
    z_i = rng.standard_normal((1, T, 1)).astype(np.float32)
    bias_i = rng.standard_normal((2 * m, 1)).astype(np.float32)
    qpos = np.arange(T - 6, T, dtype=np.int32)[None]
    q = (rng.standard_normal((1, 6, H, d)) / math.sqrt(d)).astype(np.float32)
    qi = (rng.standard_normal((1, 6, HI, dI)) / math.sqrt(dI)).astype(np.float32)
    wi = (rng.standard_normal((1, 6, HI)) / math.sqrt(HI)).astype(np.float32)

    ent, _ = O.kv_compress(raw, O.F32, z, bias, d=d, m=m, overlap=True, e_begin=0, n_e=T // m)
    kidx, _ = O.kv_compress(raw_i, O.F32, z_i, bias_i, d=dI, m=m, overlap=True, e_begin=0, n_e=T // m)
    idx, _ = O.index_topk(qi, O.F32, wi, kidx, O.F32, qpos, H_I=HI, d_I=dI, m=m, n_cap=T // m, k=k)
    out, lse = O.csa_attend(q, O.F32, ent, O.F32, T // m, idx, raw, 0, T, qpos, W=W, H=H, d=d,
                            scale=1 / math.sqrt(d))

    e_bf = BF.compress(raw[0].astype(np.float64), z[0].astype(np.float64), bias.astype(np.float64), m, True,
                       range(T // m))
    k_bf = BF.compress(raw_i[0].astype(np.float64), z_i[0].astype(np.float64), bias_i.astype(np.float64), m,
                       True, range(T // m))
    for j in range(6):
        t = int(qpos[0, j])
        bi, _, s = BF.index_topk(qi[0, j].astype(np.float64), wi[0, j].astype(np.float64), k_bf, t, m, k)
        # the oracle's keys went through fp32 storage: compare sets up to near-ties
        got = set(int(v) for v in idx[0, j] if v >= 0)
        want = set(int(v) for v in bi if v >= 0)
        if got != want:
            kth = np.sort(s)[::-1][k - 1]
            for v in got ^ want:
                assert abs(s[v] - kth) < 1e-5
        sel = [v for v in idx[0, j] if v >= 0]
        rows = np.concatenate([e_bf[sel], raw[0, max(0, t - W + 1):t + 1].astype(np.float64)])
        o, l = BF.attend(q[0, j].astype(np.float64), rows, 1 / math.sqrt(d))
        np.testing.assert_allclose(out[0, j], o, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(lse[0, j], l, rtol=1e-5, atol=1e-6)


def test_storage_arithmetic():
    # packed row: 64 bf16 rope dims + 448 fp8 dims = 576 B, vs 1024 B in bf16 (about half)
    assert O.row_bytes(O.KV_PACKED, 512, 64) == 576
    assert O.row_bytes(O.KV_PACKED, 512, 64) / O.row_bytes(O.BF16, 512) == 0.5625
    # 1M tokens at m = 4 -> 262,144 compressed entries (quoted as about 250K)
    assert (1 << 20) // 4 == 262144
    # compressed-cache blocks cover lcm(m, m') raw tokens
    assert math.lcm(4, 128) == 128
    # KV bytes per token per layer, averaged over a CSA and an HCA layer, with MXFP4
    # indexer keys (64 B codes + 4 B scales), against a bf16 GQA-8 layer (K and V,
    # 8 heads of 128): about 2 %
    csa = (576 + 64 + 4) / 4
    hca = 576 / 128
    ratio = ((csa + hca) / 2) / (2 * 8 * 128 * 2)
    assert abs(ratio - 0.0202) < 5e-4
