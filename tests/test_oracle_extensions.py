"""Pins of the oracle's remaining pieces of the attention layer:

- attention sink (CSDN explainer, table of attention details, "Attention Sink"): one
  extra logit per head in the softmax's denominator, no value;
- grouped output projection (x-techcon article, HCA subsection; CSDN explainer,
  "Grouped Output Projection"): heads projected group by group;
- two-role compressor values (an alternative input suggested by the chenxutan.com
  article, section 4.2, whose projection emits 2 x head_dim per token);
- the two-tier cache's addressing (x-techcon article, section 4, KV-cache paragraph;
  CSDN explainer, KV-cache section): rings of raw rows, decode-time compression of the
  entry a new token completes, compressed entries in blocks behind a block table.

Each is pinned by a closed form, a special case that reduces to what is already
pinned, or an independent brute force."""
import math

import numpy as np
import pytest

import oracle as O
from tests import bruteforce as BF


# ---- attention sink -------------------------------------------------------------
def _attend_case(seed, B=2, Tq=3, H=4, d=16, N=20, W=5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Tq, H, d)).astype(np.float32)
    kvc = rng.standard_normal((B, N, d)).astype(np.float32)
    raw = rng.standard_normal((B, 64, d)).astype(np.float32)
    qpos = np.array([[0, 17, 63]] * B, np.int32)[:, :Tq]
    return q, kvc, raw, qpos


def test_sink_of_minus_infinity_is_no_sink():
    q, kvc, raw, qpos = _attend_case(1)
    kw = dict(W=5, H=4, d=16, scale=0.25)
    a = O.hca_attend(q, O.F32, kvc, O.F32, 20, 4, raw, 0, 64, qpos, **kw)
    b = O.hca_attend(q, O.F32, kvc, O.F32, 20, 4, raw, 0, 64, qpos, sink=np.full(4, -np.inf, np.float32), **kw)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_sink_closed_form():
    # o_sink = o * sigmoid(lse - s) and lse_sink = logaddexp(lse, s), from the no-sink call
    q, kvc, raw, qpos = _attend_case(2)
    sink = np.array([-3.0, 0.0, 1.5, 8.0], np.float32)
    kw = dict(W=5, H=4, d=16, scale=0.25)
    idx = np.tile(np.arange(0, 20, 3, dtype=np.int32), (2, 3, 1))
    o, l = O.csa_attend(q, O.F32, kvc, O.F32, 20, idx, raw, 0, 64, qpos, **kw)
    os_, ls = O.csa_attend(q, O.F32, kvc, O.F32, 20, idx, raw, 0, 64, qpos, sink=sink, **kw)
    l64, s64 = l.astype(np.float64), sink.astype(np.float64)[None, None, :]
    frac = 1.0 / (1.0 + np.exp(s64 - l64))
    np.testing.assert_allclose(os_, o * frac[..., None], rtol=2e-6, atol=1e-7)
    np.testing.assert_allclose(ls, np.logaddexp(l64, s64), rtol=1e-6, atol=1e-6)


def test_sink_matches_bruteforce_and_empty_sets():
    q, kvc, raw, qpos = _attend_case(3)
    sink = np.array([0.5, -1.0, 2.0, 0.0], np.float32)
    scale = 0.3
    out, lse = O.hca_attend(q, O.F32, kvc, O.F32, 20, 4, raw, 0, 64, qpos, W=5, H=4, d=16, scale=scale, sink=sink)
    for b in range(2):
        for j in range(3):
            t = qpos[b, j]
            n = min((t + 1) // 4, 20)
            rows = np.concatenate([kvc[b, :n], raw[b, max(0, t - 4):t + 1]]).astype(np.float64)
            o, l = BF.attend_sink(q[b, j].astype(np.float64), rows, scale, sink)
            np.testing.assert_allclose(out[b, j], o, rtol=1e-5, atol=1e-6)
            np.testing.assert_allclose(lse[b, j], l, rtol=1e-6, atol=1e-6)
    # nothing attended: o = 0 and lse = the sink logit itself
    idx = np.full((2, 3, 4), -1, np.int32)
    o, l = O.csa_attend(q, O.F32, kvc, O.F32, 20, idx, raw, 0, 64, qpos, W=0, H=4, d=16, scale=scale, sink=sink)
    assert np.all(o == 0) and np.allclose(l, np.broadcast_to(sink, l.shape))


# ---- grouped output projection ------------------------------------------------------
def test_grouped_projection_single_group_is_a_matmul():
    rng = np.random.default_rng(11)
    M, K, R = 5, 24, 7
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = rng.standard_normal((1, R, K)).astype(np.float32)
    y = O.grouped_out_proj(x, O.F32, w, O.F32, G=1, K=K, R=R)
    np.testing.assert_allclose(y, x.astype(np.float64) @ w[0].T.astype(np.float64), rtol=1e-6, atol=1e-6)


def test_grouped_projection_is_a_block_diagonal_matmul():
    rng = np.random.default_rng(12)
    M, G, K, R = 6, 4, 16, 5
    x = rng.standard_normal((M, G * K)).astype(np.float32)
    w = rng.standard_normal((G, R, K)).astype(np.float32)
    big = np.zeros((G * K, G * R))
    for g in range(G):
        big[g * K:(g + 1) * K, g * R:(g + 1) * R] = w[g].T
    y = O.grouped_out_proj(x, O.F32, w, O.F32, G=G, K=K, R=R)
    np.testing.assert_allclose(y, x.astype(np.float64) @ big, rtol=1e-6, atol=1e-6)
    # bf16 inputs are decoded exactly
    import torch
    xb = torch.from_numpy(x).to(torch.bfloat16)
    wb = torch.from_numpy(w).to(torch.bfloat16)
    yb = O.grouped_out_proj(xb.view(torch.int16).numpy(), O.BF16, wb.view(torch.int16).numpy(), O.BF16, G=G, K=K, R=R)
    ref = xb.double().numpy() @ np.block([[wb[g].double().numpy().T if gg == g else np.zeros((K, R)) for gg in range(G)]
                                          for g in range(G)])
    np.testing.assert_allclose(yb, ref, rtol=1e-6, atol=1e-6)


# ---- two-role values ---------------------------------------------------------------
def test_two_role_rows_with_equal_halves_are_one_role():
    rng = np.random.default_rng(21)
    B, T, d, m = 2, 40, 32, 4
    x = rng.standard_normal((B, T, d)).astype(np.float32)
    z = rng.standard_normal((B, T, 1)).astype(np.float32)
    bias = rng.standard_normal((2 * m, 1)).astype(np.float32)
    a, _ = O.kv_compress(x, O.F32, z, bias, d=d, m=m, overlap=True, e_begin=0, n_e=T // m)
    b, _ = O.kv_compress(np.concatenate([x, x], axis=2), O.F32, z, bias, d=d, m=m, overlap=True, e_begin=0,
                         n_e=T // m, x_roles=2)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("z_ch", [1, 32])
def test_two_role_matches_bruteforce(z_ch):
    rng = np.random.default_rng(22 + z_ch)
    B, T, d, m = 2, 36, 32, 4
    x = rng.standard_normal((B, T, 2 * d)).astype(np.float32)
    z = rng.standard_normal((B, T, z_ch)).astype(np.float32)
    bias = rng.standard_normal((2 * m, z_ch)).astype(np.float32)
    out, _ = O.kv_compress(x, O.F32, z, bias, d=d, m=m, overlap=True, e_begin=0, n_e=T // m, x_roles=2)
    for b in range(B):
        want = BF.compress(x[b].astype(np.float64), z[b].astype(np.float64), bias.astype(np.float64), m, True,
                           range(T // m), roles=2)
        np.testing.assert_allclose(out[b], want, rtol=1e-6, atol=1e-6)


def test_two_role_constant_rows_closed_form():
    # flat logits, look-back values c1 and current values c2 everywhere: every entry
    # averages m rows of each role, (c1 + c2) / 2; entry 0 has no look-back rows: c2
    B, T, d, m = 1, 32, 32, 4
    x = np.concatenate([np.full((B, T, d), 3.0), np.full((B, T, d), -1.0)], axis=2).astype(np.float32)
    z = np.zeros((B, T, 1), np.float32)
    bias = np.zeros((2 * m, 1), np.float32)
    out, _ = O.kv_compress(x, O.F32, z, bias, d=d, m=m, overlap=True, e_begin=0, n_e=T // m, x_roles=2)
    assert np.allclose(out[0, 0], -1.0) and np.allclose(out[0, 1:], 1.0)


def test_two_roles_need_overlapping_windows():
    x = np.zeros((1, 8, 64), np.float32)
    with pytest.raises(ValueError):
        O.kv_compress(x, O.F32, np.zeros((1, 8, 1), np.float32), np.zeros((4, 1), np.float32), d=32, m=4,
                      overlap=False, e_begin=0, n_e=2, x_roles=2)


# ---- ring-addressed raw rows and decode-time compression -----------------------------
def test_ring_rows_give_the_linear_result():
    rng = np.random.default_rng(31)
    B, d, m, R = 2, 32, 4, 16
    T = 200
    x = rng.standard_normal((B, T, d)).astype(np.float32)
    z = rng.standard_normal((B, T, 1)).astype(np.float32)
    bias = rng.standard_normal((2 * m, 1)).astype(np.float32)
    i = 47                                          # entry over positions 184 .. 191
    lin, _ = O.kv_compress(x, O.F32, z, bias, d=d, m=m, overlap=True, e_begin=i, n_e=2)
    # the ring holds positions 184 .. 199 in rows p mod 16
    ring_x = np.zeros((B, R, d), np.float32)
    ring_z = np.zeros((B, R, 1), np.float32)
    for p in range(T - R, T):
        ring_x[:, p % R], ring_z[:, p % R] = x[:, p], z[:, p]
    rng_out, _ = O.kv_compress(ring_x, O.F32, ring_z, bias, d=d, m=m, overlap=True, e_begin=i, n_e=2, x_rows=R)
    assert np.array_equal(lin, rng_out)


@pytest.mark.parametrize("roles,fmt", [(1, O.KV_PACKED), (2, O.F32)])
def test_compress_step_is_the_completed_entry(roles, fmt):
    rng = np.random.default_rng(41 + roles)
    B, d, r, m, R = 3, 64, 16, 4, 16
    T = 120
    x = rng.standard_normal((B, T, roles * d)).astype(np.float32)
    z = rng.standard_normal((B, T, 1)).astype(np.float32)
    bias = rng.standard_normal((2 * m, 1)).astype(np.float32)
    # ragged batch, two new tokens per sequence: (5,6) -> none; (6,7) -> entry 1 at 7;
    # (118,119) -> entry 29 at 119
    pos = np.array([[5, 6], [6, 7], [118, 119]], np.int32)
    ring_x = np.zeros((B, R, roles * d), np.float32)
    ring_z = np.zeros((B, R, 1), np.float32)
    for b in range(B):
        top = pos[b, -1]
        for p in range(max(0, top - R + 1), top + 1):
            ring_x[b, p % R], ring_z[b, p % R] = x[b, p], z[b, p]
    out, _, ent = O.kv_compress_step(ring_x, O.F32, ring_z, bias, pos, d=d, r=r, m=m, overlap=True, out_fmt=fmt,
                                     x_roles=roles)
    assert ent.tolist() == [[-1, -1], [-1, 1], [-1, 29]]
    for b, j in [(1, 1), (2, 1)]:
        want, _ = O.kv_compress(x[b:b + 1], O.F32, z[b:b + 1], bias, d=d, r=r, m=m, overlap=True,
                                e_begin=int(ent[b, j]), n_e=1, out_fmt=fmt, x_roles=roles)
        assert np.array_equal(out[b, j], want[0, 0])


# ---- paged gather -------------------------------------------------------------------------
def test_paged_gather_identity_and_permuted_tables():
    rng = np.random.default_rng(51)
    B, n, rb, epb = 2, 70, 24, 8
    nblk = (n + epb - 1) // epb
    lin = rng.integers(0, 256, (B, nblk * epb, rb), dtype=np.uint8)
    # identity: the pool is the linear buffers back to back
    bt = np.arange(B * nblk, dtype=np.int32).reshape(B, nblk)
    got = O.paged_gather(lin.reshape(-1), rb, bt, epb, epb * rb, n)
    assert np.array_equal(got, lin[:, :n])
    # permuted physical blocks with a larger block stride (room for other data per block)
    perm = rng.permutation(B * nblk + 3)[:B * nblk].astype(np.int32).reshape(B, nblk)
    bb = epb * rb + 40
    pool = rng.integers(0, 256, ((B * nblk + 3) * bb,), dtype=np.uint8)
    for b in range(B):
        for s in range(nblk * epb):
            off = perm[b, s // epb] * bb + (s % epb) * rb
            pool[off:off + rb] = lin[b, s]
    assert np.array_equal(O.paged_gather(pool, rb, perm, epb, bb, n), lin[:, :n])
    # a missing block reads as zeros
    perm[1, 3] = -1
    got = O.paged_gather(pool, rb, perm, epb, bb, n)
    assert np.all(got[1, 3 * epb:4 * epb] == 0) and np.array_equal(got[0], lin[0, :n])
