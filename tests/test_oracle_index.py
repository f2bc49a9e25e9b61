"""Pins of the oracle's lightning indexer + top-k (x-techcon article, section 2, CSA
step 2).  The score formula is a reading (the pages print none): parity unpinned by
the pages; these tests pin the oracle to that reading by brute force, and to the
reading-independent properties of a top-k selection."""
import numpy as np
import pytest

import oracle as O
from tests import bruteforce as BF


def _setup(seed, B, Tq, H, d, N):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Tq, H, d)).astype(np.float32)
    w = rng.standard_normal((B, Tq, H)).astype(np.float32)
    K = rng.standard_normal((B, N, d)).astype(np.float32)
    return q, w, K


@pytest.mark.parametrize("m,k", [(4, 8), (4, 64), (1, 5), (3, 17)])
def test_matches_bruteforce(m, k):
    B, Tq, H, d, N = 2, 6, 4, 16, 40
    q, w, K = _setup(21, B, Tq, H, d, N)
    qpos = np.array([[3, 20, 50, 99, 150, 170], [0, 1, 7, 8, 159, 400]], np.int32)
    idx, sc = O.index_topk(q, O.F32, w, K, O.F32, qpos, H_I=H, d_I=d, m=m, n_cap=N, k=k)
    for b in range(B):
        for j in range(Tq):
            bi, bs, _ = BF.index_topk(q[b, j].astype(np.float64), w[b, j].astype(np.float64),
                                      K[b].astype(np.float64), int(qpos[b, j]), m, k)
            assert np.array_equal(idx[b, j], bi)
            np.testing.assert_allclose(sc[b, j], bs, rtol=1e-6, atol=1e-6)


def test_all_visible_when_k_exceeds_count():
    q, w, K = _setup(22, 1, 1, 4, 8, 30)
    idx, sc = O.index_topk(q, O.F32, w, K, O.F32, np.array([[43]], np.int32), H_I=4, d_I=8, m=4, n_cap=30, k=16)
    assert list(idx[0, 0]) == list(range(11)) + [-1] * 5
    assert np.all(np.isneginf(sc[0, 0, 11:]))


def test_positive_weight_scaling_keeps_the_set():
    q, w, K = _setup(23, 1, 3, 4, 8, 200)
    qpos = np.array([[399, 500, 799]], np.int32)
    a, _ = O.index_topk(q, O.F32, np.abs(w), K, O.F32, qpos, H_I=4, d_I=8, m=4, n_cap=200, k=20)
    b, _ = O.index_topk(q, O.F32, np.abs(w) * 7.5, K, O.F32, qpos, H_I=4, d_I=8, m=4, n_cap=200, k=20)
    assert np.array_equal(a, b)


def test_single_head_without_relu_is_plain_dot_topk():
    rng = np.random.default_rng(24)
    d, N, k = 8, 100, 10
    q = np.abs(rng.standard_normal((1, 1, 1, d))).astype(np.float32)
    K = np.abs(rng.standard_normal((1, N, d))).astype(np.float32)  # all dots positive
    idx, sc = O.index_topk(q, O.F32, np.ones((1, 1, 1), np.float32), K, O.F32, np.array([[N - 1]], np.int32),
                           H_I=1, d_I=d, m=1, n_cap=N, k=k)
    dots = K[0].astype(np.float64) @ q[0, 0, 0].astype(np.float64)
    assert set(idx[0, 0]) == set(np.argsort(-dots)[:k])
    np.testing.assert_allclose(sc[0, 0], dots[idx[0, 0]], rtol=1e-6)


def test_relu_gates_negative_head_scores():
    # head 1 has only negative dots: it must contribute nothing
    d, N = 4, 12
    K = np.zeros((1, N, d), np.float32)
    K[0, :, 0] = np.arange(N)
    q = np.zeros((1, 1, 2, d), np.float32)
    q[0, 0, 0, 0] = 1.0
    q[0, 0, 1, 0] = -1.0
    w = np.array([[[1.0, 5.0]]], np.float32)
    idx, sc = O.index_topk(q, O.F32, w, K, O.F32, np.array([[N - 1]], np.int32), H_I=2, d_I=d, m=1, n_cap=N, k=3)
    assert list(idx[0, 0]) == [9, 10, 11]
    assert list(sc[0, 0]) == [9.0, 10.0, 11.0]


def test_ties_prefer_the_smaller_index():
    d, N = 4, 20
    K = np.ones((1, N, d), np.float32)       # every entry has the same score
    q = np.ones((1, 1, 1, d), np.float32)
    idx, _ = O.index_topk(q, O.F32, np.ones((1, 1, 1), np.float32), K, O.F32, np.array([[N - 1]], np.int32),
                          H_I=1, d_I=d, m=1, n_cap=N, k=6)
    assert list(idx[0, 0]) == [0, 1, 2, 3, 4, 5]


def test_causal_count_and_capacity():
    q, w, K = _setup(25, 1, 4, 2, 8, 10)
    qpos = np.array([[-1, 2, 3, 1000]], np.int32)
    idx, _ = O.index_topk(q, O.F32, w, K, O.F32, qpos, H_I=2, d_I=8, m=4, n_cap=10, k=64)
    counts = (idx[0] >= 0).sum(axis=1)
    assert list(counts) == [0, 0, 1, 10]


def test_mxfp4_and_bf16_operands_match_bruteforce():
    import torch
    B, Tq, H, d, N, k = 1, 2, 4, 64, 50, 9
    rng = np.random.default_rng(26)
    qc = rng.integers(0, 256, (B, Tq, H, d // 2), dtype=np.uint8)
    qs = rng.integers(124, 130, (B, Tq, H, d // 32), dtype=np.uint8)
    kc = rng.integers(0, 256, (B, N, d // 2), dtype=np.uint8)
    ks = rng.integers(124, 130, (B, N, d // 32), dtype=np.uint8)
    w = rng.standard_normal((B, Tq, H)).astype(np.float32)
    qpos = np.array([[150, 199]], np.int32)
    idx, sc = O.index_topk(qc, O.MXFP4, w, kc, O.MXFP4, qpos, H_I=H, d_I=d, m=4, n_cap=N, k=k,
                           qi_scales=qs, ki_scales=ks)
    qd = BF.decode(qc, BF.MXFP4, d, scales=qs).reshape(B, Tq, H, d)
    kd = BF.decode(kc, BF.MXFP4, d, scales=ks).reshape(B, N, d)
    for j in range(Tq):
        bi, bs, _ = BF.index_topk(qd[0, j], w[0, j].astype(np.float64), kd[0], int(qpos[0, j]), 4, k)
        assert np.array_equal(idx[0, j], bi)
        np.testing.assert_allclose(sc[0, j], bs, rtol=1e-6)
    # bf16 operands
    qf = rng.standard_normal((B, Tq, H, d)).astype(np.float32)
    kf = rng.standard_normal((B, N, d)).astype(np.float32)
    qb = torch.from_numpy(qf).to(torch.bfloat16).view(torch.int16).numpy()
    kb = torch.from_numpy(kf).to(torch.bfloat16).view(torch.int16).numpy()
    idx, sc = O.index_topk(qb, O.BF16, w, kb, O.BF16, qpos, H_I=H, d_I=d, m=4, n_cap=N, k=k)
    qd = BF.decode(qb, BF.BF16, d).reshape(B, Tq, H, d)
    kd = BF.decode(kb, BF.BF16, d).reshape(B, N, d)
    for j in range(Tq):
        bi, bs, _ = BF.index_topk(qd[0, j], w[0, j].astype(np.float64), kd[0], int(qpos[0, j]), 4, k)
        assert np.array_equal(idx[0, j], bi)
