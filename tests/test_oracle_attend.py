"""Pins of the oracle's shared-KV MQA over {entries} U {window} (x-techcon article,
section 2: CSA step 3 -- the 128 most recent uncompressed tokens are attended
together with the selected entries; HCA -- dense over all entries; both use shared
KV multi-query attention)."""
import math

import numpy as np
import pytest

import oracle as O
from tests import bruteforce as BF


def _rows(rng, n, d):
    return rng.standard_normal((n, d)).astype(np.float32)


def test_csa_matches_bruteforce_with_window_and_padding():
    rng = np.random.default_rng(31)
    B, Tq, H, d, N, k, W = 2, 3, 5, 16, 30, 7, 4
    q = rng.standard_normal((B, Tq, H, d)).astype(np.float32)
    kvc = rng.standard_normal((B, N, d)).astype(np.float32)
    raw = rng.standard_normal((B, 200, d)).astype(np.float32)       # window rows at positions 0..199
    qpos = np.array([[2, 77, 120], [0, 5, 199]], np.int32)
    idx = rng.integers(-1, N + 3, (B, Tq, k)).astype(np.int32)     # includes -1 and out-of-range
    scale = 1 / math.sqrt(d)
    out, lse = O.csa_attend(q, O.F32, kvc, O.F32, N, idx, raw, 0, 200, qpos, W=W, H=H, d=d, scale=scale)
    for b in range(B):
        for j in range(Tq):
            t = qpos[b, j]
            sel = [s for s in idx[b, j] if 0 <= s < N]
            rows = np.concatenate([kvc[b, sel], raw[b, max(0, t - W + 1):t + 1]]).astype(np.float64)
            o, l = BF.attend(q[b, j].astype(np.float64), rows, scale)
            np.testing.assert_allclose(out[b, j], o, rtol=1e-5, atol=1e-6)
            np.testing.assert_allclose(lse[b, j], l, rtol=1e-6, atol=1e-6)


def test_hca_matches_bruteforce_causal_count():
    rng = np.random.default_rng(32)
    B, Tq, H, d, N, W, m = 1, 4, 3, 16, 12, 5, 8
    q = rng.standard_normal((B, Tq, H, d)).astype(np.float32)
    kvc = rng.standard_normal((B, N, d)).astype(np.float32)
    raw = rng.standard_normal((B, 128, d)).astype(np.float32)
    qpos = np.array([[6, 7, 60, 127]], np.int32)
    out, lse = O.hca_attend(q, O.F32, kvc, O.F32, N, m, raw, 0, 128, qpos, W=W, H=H, d=d, scale=0.3)
    for j in range(Tq):
        t = qpos[0, j]
        n = min((t + 1) // m, N)
        rows = np.concatenate([kvc[0, :n], raw[0, max(0, t - W + 1):t + 1]]).astype(np.float64)
        o, l = BF.attend(q[0, j].astype(np.float64), rows, 0.3)
        np.testing.assert_allclose(out[0, j], o, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(lse[0, j], l, rtol=1e-6, atol=1e-6)


def test_csa_with_every_entry_selected_equals_hca():
    rng = np.random.default_rng(33)
    B, H, d, N, W, m = 2, 4, 32, 25, 6, 4
    q = rng.standard_normal((B, 1, H, d)).astype(np.float32)
    kvc = rng.standard_normal((B, N, d)).astype(np.float32)
    raw = rng.standard_normal((B, 64, d)).astype(np.float32)
    qpos = np.array([[63], [40]], np.int32)
    idx = np.full((B, 1, 32), -1, np.int32)
    for b in range(B):
        n = min((qpos[b, 0] + 1) // m, N)
        idx[b, 0, :n] = np.arange(n)
    a, la = O.csa_attend(q, O.F32, kvc, O.F32, N, idx, raw, 0, 64, qpos, W=W, H=H, d=d, scale=0.2)
    b_, lb = O.hca_attend(q, O.F32, kvc, O.F32, N, m, raw, 0, 64, qpos, W=W, H=H, d=d, scale=0.2)
    np.testing.assert_allclose(a, b_, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(la, lb, rtol=1e-6, atol=1e-7)


def _one_hot_compression(raw, m):
    """m = 1 with overlap and bias [-big, 0]: entry i is exactly raw row i."""
    B, T, d = raw.shape
    z = np.zeros((B, T, 1), np.float32)
    bias = np.array([[-1e30], [0.0]], np.float32)
    ent, _ = O.kv_compress(raw, O.F32, z, bias, d=d, m=1, overlap=True, e_begin=0, n_e=T)
    return ent


def test_m1_one_hot_no_window_reduces_to_causal_mqa():
    rng = np.random.default_rng(34)
    T, H, d = 24, 4, 16
    raw = rng.standard_normal((1, T, d)).astype(np.float32)
    ent = _one_hot_compression(raw, 1)
    np.testing.assert_array_equal(ent, raw)
    q = rng.standard_normal((1, T, H, d)).astype(np.float32)
    qpos = np.arange(T, dtype=np.int32)[None]
    out, _ = O.hca_attend(q, O.F32, ent, O.F32, T, 1, raw, 0, T, qpos, W=0, H=H, d=d, scale=0.25)
    want = BF.causal_mqa(q[0].astype(np.float64), raw[0].astype(np.float64), 0.25)
    np.testing.assert_allclose(out[0], want, rtol=1e-5, atol=1e-6)
    # the same through CSA with a causal top-k that keeps everything
    w = np.ones((1, T, 1), np.float32)
    idx, _ = O.index_topk(q[:, :, :1], O.F32, w, ent, O.F32, qpos, H_I=1, d_I=d, m=1, n_cap=T, k=T)
    out2, _ = O.csa_attend(q, O.F32, ent, O.F32, T, idx, raw, 0, T, qpos, W=0, H=H, d=d, scale=0.25)
    np.testing.assert_allclose(out2[0], want, rtol=1e-5, atol=1e-6)


def test_window_rows_count_twice_in_the_joint_softmax():
    # entries = raw rows (m = 1); the last W positions are also window rows, so in
    # the one joint softmax they carry weight 2: logits + ln 2.
    rng = np.random.default_rng(35)
    T, H, d, W = 20, 3, 16, 5
    raw = rng.standard_normal((1, T, d)).astype(np.float32)
    ent = _one_hot_compression(raw, 1)
    q = rng.standard_normal((1, T, H, d)).astype(np.float32)
    qpos = np.arange(T, dtype=np.int32)[None]
    out, _ = O.hca_attend(q, O.F32, ent, O.F32, T, 1, raw, 0, T, qpos, W=W, H=H, d=d, scale=0.25)
    extra = np.zeros((T, T))
    for t in range(T):
        extra[t, max(0, t - W + 1):t + 1] = math.log(2.0)
    want = BF.causal_mqa(q[0].astype(np.float64), raw[0].astype(np.float64), 0.25, extra)
    np.testing.assert_allclose(out[0], want, rtol=1e-5, atol=1e-6)


def test_empty_set_gives_zero_and_minus_inf():
    rng = np.random.default_rng(36)
    q = rng.standard_normal((1, 1, 2, 8)).astype(np.float32)
    kvc = rng.standard_normal((1, 4, 8)).astype(np.float32)
    idx = np.full((1, 1, 3), -1, np.int32)
    out, lse = O.csa_attend(q, O.F32, kvc, O.F32, 4, idx, kvc, 0, 4, np.array([[3]], np.int32), W=0, H=2, d=8,
                            scale=1.0)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_selected_set_order_does_not_matter():
    rng = np.random.default_rng(37)
    q = rng.standard_normal((1, 1, 4, 16)).astype(np.float32)
    kvc = rng.standard_normal((1, 40, 16)).astype(np.float32)
    raw = rng.standard_normal((1, 16, 16)).astype(np.float32)
    idx = rng.permutation(40)[:12].astype(np.int32)[None, None]
    a, _ = O.csa_attend(q, O.F32, kvc, O.F32, 40, idx, raw, 0, 16, np.array([[15]], np.int32), W=4, H=4, d=16,
                        scale=0.3)
    b, _ = O.csa_attend(q, O.F32, kvc, O.F32, 40, idx[..., ::-1].copy(), raw, 0, 16, np.array([[15]], np.int32),
                        W=4, H=4, d=16, scale=0.3)
    np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-7)


def test_ring_and_linear_window_buffers_agree():
    rng = np.random.default_rng(38)
    d, H, W, t = 16, 2, 8, 100
    raw = rng.standard_normal((1, 128, d)).astype(np.float32)
    q = rng.standard_normal((1, 1, H, d)).astype(np.float32)
    kvc = rng.standard_normal((1, 5, d)).astype(np.float32)
    idx = np.array([[[0, 3]]], np.int32)
    qp = np.array([[t]], np.int32)
    full, _ = O.csa_attend(q, O.F32, kvc, O.F32, 5, idx, raw, 0, 128, qp, W=W, H=H, d=d, scale=0.3)
    lin, _ = O.csa_attend(q, O.F32, kvc, O.F32, 5, idx, raw[:, t - W + 1:t + 1].copy(), t - W + 1, W, qp, W=W, H=H,
                          d=d, scale=0.3)
    ring = np.zeros((1, 16, d), np.float32)
    for p in range(t - 15, t + 1):
        ring[0, p % 16] = raw[0, p]
    rg, _ = O.csa_attend(q, O.F32, kvc, O.F32, 5, idx, ring, 0, 16, qp, W=W, H=H, d=d, scale=0.3)
    np.testing.assert_array_equal(full, lin)
    np.testing.assert_array_equal(full, rg)


def test_packed_kv_and_bf16_output():
    import torch
    rng = np.random.default_rng(39)
    d, r, H, N = 128, 32, 4, 20
    vals = rng.standard_normal((1, N, d)).astype(np.float32)
    packed, _ = O.encode_rows(vals.reshape(-1, d), O.KV_PACKED, d, r)
    packed = packed.reshape(1, N, -1)
    dec = BF.decode(packed, BF.KV_PACKED, d, r).reshape(1, N, d)
    q = rng.standard_normal((1, 1, H, d)).astype(np.float32)
    qb = torch.from_numpy(q).to(torch.bfloat16).view(torch.int16).numpy()
    qd = BF.decode(qb, BF.BF16, d).reshape(1, 1, H, d)
    idx = np.arange(10, dtype=np.int32)[None, None]
    qp = np.array([[N - 1]], np.int32)
    out, lse = O.csa_attend(qb, O.BF16, packed, O.KV_PACKED, N, idx, packed, 0, N, qp, W=3, H=H, d=d, r=r,
                            scale=1 / math.sqrt(d))
    rows = np.concatenate([dec[0, :10], dec[0, N - 3:N]])
    o, l = BF.attend(qd[0, 0], rows, 1 / math.sqrt(d))
    np.testing.assert_allclose(out[0, 0], o, rtol=1e-5, atol=1e-6)
    ob, _ = O.csa_attend(qb, O.BF16, packed, O.KV_PACKED, N, idx, packed, 0, N, qp, W=3, H=H, d=d, r=r,
                         scale=1 / math.sqrt(d), out_fmt=O.BF16)
    back = torch.from_numpy(ob.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.all(np.abs(back - out) <= np.abs(out) * 2.0 ** -8 + 1e-30)
