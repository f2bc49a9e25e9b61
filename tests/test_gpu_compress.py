"""GPU parity of kv_compress against the oracle (token compression: x-techcon
article, section 2, CSA step 1 and the HCA subsection)."""
import numpy as np
import pytest
import torch

import oracle as O
from compressed_sparse_long_02_amd import gen, ops
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu

CASES = [
    # (x_fmt, d, r, m, overlap, per_channel, e_begin, n_e, x_pos0)
    (O.F32, 128, 32, 4, True, False, 0, 37, 0),       # config-1 geometry, ragged entry count
    (O.BF16, 512, 64, 4, True, False, 3, 29, 8),      # CSA, buffer starting mid-sequence
    (O.BF16, 512, 64, 128, False, False, 0, 5, 0),    # HCA, m' = 128
    (O.F32, 32, 0, 4, True, False, 0, 130, 0),        # indexer keys of config 1 (d_I = 32)
    (O.BF16, 128, 0, 4, True, True, 1, 23, 0),        # per-channel logits
    (O.F32, 128, 0, 1, False, False, 0, 40, 0),       # m = 1: identity
    (O.BF16, 96, 32, 3, True, False, 0, 19, 0),       # d with idle threads per block
]


def _case(x_fmt, d, m, overlap, per_channel, e_begin, n_e, x_pos0, seed):
    B = 3
    win = 2 * m if overlap else m
    hi = (e_begin + n_e) * m
    n_tok = hi - x_pos0
    z_ch = d if per_channel else 1
    x = gen.normal((B, n_tok, d), seed)
    xs = gen.store(x, x_fmt)
    z = gen.random_logits((B, n_tok, z_ch), seed + 1)
    bias = gen.random_logits((win, z_ch), seed + 2)
    return B, xs, z, bias


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_compress_parity_all_formats(gpu, case):
    x_fmt, d, r, m, overlap, per_channel, e_begin, n_e, x_pos0 = case
    B, xs, z, bias = _case(x_fmt, d, m, overlap, per_channel, e_begin, n_e, x_pos0, 100 + d + m)
    kw = dict(d=d, r=r, m=m, overlap=overlap, e_begin=e_begin, n_e=n_e, x_pos0=x_pos0)
    ref, _ = O.kv_compress(host(xs), x_fmt, host(z), host(bias), **kw, out_fmt=O.F32)
    got, _ = ops.kv_compress(dev(xs), x_fmt, dev(z), dev(bias), **kw, out_fmt=O.F32)
    torch.cuda.synchronize()
    g = host(got).astype(np.float64)
    err = np.abs(g - ref)
    assert np.all(err <= 2e-6 * (1.0 + np.abs(ref))), float(err.max())
    fmts = [O.BF16, O.MXFP4] + ([O.KV_PACKED] if r > 0 else [])
    for fmt in fmts:
        q, sc = ops.kv_compress(dev(xs), x_fmt, dev(z), dev(bias), **kw, out_fmt=fmt)
        torch.cuda.synchronize()
        # the quantisation decision, taken on the GPU's own fp32 entries, equals the
        # oracle's encoder on the same fp32 values, byte for byte
        enc, enc_sc = O.encode_rows(g.reshape(-1, d), fmt, d, r)
        assert np.array_equal(host(q).reshape(enc.shape), enc), "format %d bytes differ" % fmt
        if fmt == O.MXFP4:
            assert np.array_equal(host(sc).reshape(enc_sc.shape), enc_sc)
        # against the oracle's own quantised entries: equal except where the fp64 value
        # sits within the fp32 error of a rounding boundary (then one step apart)
        oq, osc = O.kv_compress(host(xs), x_fmt, host(z), host(bias), **kw, out_fmt=fmt)
        dq = O.decode_rows(host(q), fmt, d, r, None if sc is None else host(sc))
        do = O.decode_rows(oq, fmt, d, r, osc)
        mism = np.mean(dq != do)
        assert mism < 1e-3, mism


def test_compress_decode_step_matches_prefill(gpu):
    """Compressing entry i alone from a short raw tail (decode) equals the same entry
    compressed in one pass over the whole sequence."""
    d, m = 512, 4
    B, xs, z, bias = _case(O.BF16, d, m, True, False, 0, 64, 0, 7)
    full, _ = ops.kv_compress(dev(xs), O.BF16, dev(z), dev(bias), d=d, r=64, m=m, overlap=True, e_begin=0, n_e=64,
                              out_fmt=O.KV_PACKED)
    i = 50
    lo = (i - 1) * m
    tail_x = dev(xs[:, lo:(i + 1) * m])
    tail_z = dev(z[:, lo:(i + 1) * m])
    one, _ = ops.kv_compress(tail_x, O.BF16, tail_z, dev(bias), d=d, r=64, m=m, overlap=True, e_begin=i, n_e=1,
                             x_pos0=lo, out_fmt=O.KV_PACKED)
    torch.cuda.synchronize()
    assert torch.equal(one[:, 0], full[:, i])


def test_compress_writes_into_a_cache_slice(gpu):
    d, m = 128, 4
    B, xs, z, bias = _case(O.F32, d, m, True, False, 0, 16, 0, 9)
    cache = torch.full((B, 40, d + 32), 7, dtype=torch.uint8, device="cuda")  # packed rows, r = 32
    view = cache[:, 10:26]
    ops.kv_compress(dev(xs), O.F32, dev(z), dev(bias), d=d, r=32, m=m, overlap=True, e_begin=0, n_e=16,
                    out_fmt=O.KV_PACKED, out=view)
    ref, _ = O.kv_compress(host(xs), O.F32, host(z), host(bias), d=d, r=32, m=m, overlap=True, e_begin=0, n_e=16,
                           out_fmt=O.KV_PACKED)
    c = host(cache)
    assert np.all(c[:, :10] == 7) and np.all(c[:, 26:] == 7)
    assert np.mean(c[:, 10:26] != ref) < 1e-3


@pytest.mark.parametrize("x_fmt,d,r,m,per_channel", [(O.F32, 128, 32, 4, False), (O.BF16, 512, 64, 4, False),
                                                     (O.BF16, 128, 0, 4, True)])
def test_compress_two_role_rows(gpu, x_fmt, d, r, m, per_channel):
    """Two-role raw rows (look-back value, then current value; chenxutan.com article,
    section 4.2 projects 2 x head_dim per token) against the oracle: fp32 entries within
    fp32 rounding, quantised entries byte-equal to the oracle's encoder on them."""
    B, n_e = 2, 33
    n_tok = n_e * m
    z_ch = d if per_channel else 1
    xs = gen.store(gen.normal((B, n_tok, 2 * d), 900 + d), x_fmt)
    z = gen.random_logits((B, n_tok, z_ch), 901)
    bias = gen.random_logits((2 * m, z_ch), 902)
    kw = dict(d=d, r=r, m=m, overlap=True, e_begin=0, n_e=n_e, x_roles=2)
    ref, _ = O.kv_compress(host(xs), x_fmt, host(z), host(bias), **kw, out_fmt=O.F32)
    got, _ = ops.kv_compress(dev(xs), x_fmt, dev(z), dev(bias), **kw, out_fmt=O.F32)
    torch.cuda.synchronize()
    g = host(got).astype(np.float64)
    assert np.all(np.abs(g - ref) <= 2e-6 * (1.0 + np.abs(ref)))
    for fmt in [O.MXFP4] + ([O.KV_PACKED] if r > 0 else [O.BF16]):
        q, sc = ops.kv_compress(dev(xs), x_fmt, dev(z), dev(bias), **kw, out_fmt=fmt)
        torch.cuda.synchronize()
        enc, enc_sc = O.encode_rows(g.reshape(-1, d), fmt, d, r)
        assert np.array_equal(host(q).reshape(enc.shape), enc)
        if fmt == O.MXFP4:
            assert np.array_equal(host(sc).reshape(enc_sc.shape), enc_sc)


@pytest.mark.parametrize("roles,out_fmt,m,overlap", [(1, O.KV_PACKED, 4, True), (2, O.KV_PACKED, 4, True),
                                                     (1, O.MXFP4, 4, True), (1, O.KV_PACKED, 128, False)])
@pytest.mark.parametrize("paged", [False, True])
def test_compress_step_from_the_ring(gpu, roles, out_fmt, m, overlap, paged):
    """Decode-time compression driven from the state ring: a ragged batch appends T = 2
    tokens per sequence; the tokens that complete a block compress their entry from the
    ring (row p mod R) into the cache -- dense, or through a block table of shuffled
    blocks of 128 raw tokens -- and nothing else in the cache changes.  Checked against
    the oracle's step and, byte for byte, against kv_compress on the same rows."""
    B, T, d, r, R = 4, 2, 512 if out_fmt == O.KV_PACKED else 128, 64 if out_fmt == O.KV_PACKED else 0, 256
    n_cap = 4096 // m
    pos = torch.tensor([[5, 6], [2 * m - 2, 2 * m - 1], [4095 - m, 4096 - m], [4094, 4095]], dtype=torch.int32)
    xr = gen.store(gen.normal((B, R, roles * d), 910 + m), O.BF16)
    zr = gen.random_logits((B, R, 1), 911)
    bias = gen.random_logits((2 * m if overlap else m, 1), 912)
    rb = O.row_bytes(out_fmt, d, r)
    fill = 0xA5
    kw = dict(d=d, r=r, m=m, overlap=overlap, x_roles=roles)
    if not paged:
        cache = torch.full((B, n_cap, rb), fill, dtype=torch.uint8)
        scales = torch.full((B, n_cap, d // 32), fill, dtype=torch.uint8) if out_fmt == O.MXFP4 else None
        out, sc = ops.kv_compress_step(dev(xr), O.BF16, dev(zr), dev(bias), dev(pos), out=dev(cache),
                                       out_scales=dev(scales) if scales is not None else None, out_fmt=out_fmt, **kw)
        torch.cuda.synchronize()
        got, got_sc = host(out), (host(sc) if sc is not None else None)
    else:
        epb = 128 // m
        nblk = n_cap // epb
        blk_bytes = (epb * rb + 15) // 16 * 16 + 16 * epb      # rows, then the scales (and slack)
        g = torch.Generator().manual_seed(5)
        bt = torch.randperm(B * nblk, generator=g).to(torch.int32).reshape(B, nblk)
        pool = torch.full((B * nblk, blk_bytes), fill, dtype=torch.uint8)
        sc_off = (epb * rb + 15) // 16 * 16
        pool_d = dev(pool)
        pg = (dev(bt), epb, blk_bytes, blk_bytes, B * nblk)
        ops.kv_compress_step(dev(xr), O.BF16, dev(zr), dev(bias), dev(pos), out=pool_d, out_fmt=out_fmt,
                             out_scales=pool_d[:, sc_off:] if out_fmt == O.MXFP4 else None, pages=pg, **kw)
        torch.cuda.synchronize()
        ph = host(pool_d)
        got = O.paged_gather(ph, rb, host(bt), epb, blk_bytes, n_cap)
        got_sc = (O.paged_gather(ph.reshape(-1)[sc_off:], d // 32, host(bt), epb, blk_bytes, n_cap)
                  if out_fmt == O.MXFP4 else None)
    want, want_sc, ent = O.kv_compress_step(host(xr), O.BF16, host(zr), host(bias), host(pos), out_fmt=out_fmt, **kw)
    assert (ent >= 0).sum() >= 3
    touched = set()
    for b in range(B):
        for j in range(T):
            e = int(ent[b, j])
            if e < 0:
                continue
            touched.add((b, e))
            assert np.array_equal(got[b, e], want[b, j]), (b, j, e)
            if out_fmt == O.MXFP4:
                assert np.array_equal(got_sc[b, e], want_sc[b, j])
            # byte-equal to kv_compress over the same ring rows, as a linear buffer (the
            # general kernel: another summation order, the same bytes on these inputs)
            p_hi = int(pos[b, j])
            lin = np.stack([host(xr)[b, p % R] for p in range(p_hi - (2 * m if overlap else m) + 1, p_hi + 1)])
            zl = np.stack([host(zr)[b, p % R] for p in range(p_hi - (2 * m if overlap else m) + 1, p_hi + 1)])
            one, one_sc = ops.kv_compress(dev(lin[None]), O.BF16, dev(zl[None]), dev(bias), e_begin=e, n_e=1,
                                          x_pos0=p_hi - (2 * m if overlap else m) + 1, out_fmt=out_fmt, **kw)
            torch.cuda.synchronize()
            assert np.array_equal(host(one)[0, 0], got[b, e])
    # every other cache row is untouched
    for b in range(B):
        for e in range(n_cap):
            if (b, e) not in touched:
                assert np.all(got[b, e] == fill), (b, e)


def _pair_jobs(B, R, roles, key_fmt, m0, seed, paged, n_cap0):
    """A CSA-layer pair: the packed KV entry (d = 512, r = 64, window m0 / overlap when
    m0 = 4) and the indexer key (d = 128, m = 4, overlap) in `key_fmt`, their rings, and
    their caches filled with 0xA5 -- linear, or one pool of shuffled blocks of 128 raw
    tokens holding both (KV rows, then key rows, then key scales)."""
    fill = 0xA5
    ov0 = m0 == 4
    xr0 = gen.store(gen.normal((B, R, roles * 512), seed), O.BF16)
    zr0 = gen.random_logits((B, R, 1), seed + 1)
    b0 = gen.random_logits((2 * m0 if ov0 else m0, 1), seed + 2)
    xr1 = gen.store(gen.normal((B, R, 128), seed + 3), O.BF16)
    zr1 = gen.random_logits((B, R, 1), seed + 4)
    b1 = gen.random_logits((8, 1), seed + 5)
    rb0, rb1 = O.row_bytes(O.KV_PACKED, 512, 64), O.row_bytes(key_fmt, 128, 0)
    j0 = dict(x_ring=dev(xr0), x_fmt=O.BF16, z_ring=dev(zr0), bias=dev(b0), d=512, r=64, m=m0, overlap=ov0,
              out_fmt=O.KV_PACKED, x_roles=roles)
    j1 = dict(x_ring=dev(xr1), x_fmt=O.BF16, z_ring=dev(zr1), bias=dev(b1), d=128, m=4, overlap=True,
              out_fmt=key_fmt)
    if not paged:
        n_cap1 = n_cap0 * m0 // 4                 # both cover the same raw tokens
        j0["out"] = dev(torch.full((B, n_cap0, rb0), fill, dtype=torch.uint8))
        j1["out"] = dev(torch.full((B, n_cap1, rb1), fill, dtype=torch.uint8))
        if key_fmt == O.MXFP4:
            j1["out_scales"] = dev(torch.full((B, n_cap1, 4), fill, dtype=torch.uint8))
        return j0, j1, None
    epb0, epb1 = 128 // m0, 32
    nblk = max(n_cap0 // epb0, 1)
    o1 = epb0 * rb0
    o2 = o1 + epb1 * rb1
    blk = o2 + epb1 * 4
    g = torch.Generator().manual_seed(seed)
    bt = dev(torch.randperm(B * nblk + 3, generator=g)[:B * nblk].to(torch.int32).reshape(B, nblk))
    pool = dev(torch.full((B * nblk + 3, blk), fill, dtype=torch.uint8))
    j0.update(out=pool, pages=(bt, epb0, blk, blk, B * nblk + 3))
    j1.update(out=pool[:, o1:], pages=(bt, epb1, blk, blk, B * nblk + 3))
    if key_fmt == O.MXFP4:
        j1["out_scales"] = pool[:, o2:]
    return j0, j1, (pool, o1)


def _pair_state(j0, j1, pool):
    if pool is not None:                       # the block's KV rows, then its keys and scales
        p, o1 = pool
        h = host(p)
        return [h[:, :o1], h[:, o1:]]
    return [host(j0["out"]), host(j1["out"])] + ([host(j1["out_scales"])] if "out_scales" in j1 else [])


@pytest.mark.parametrize("roles,key_fmt,m0", [(1, O.MXFP4, 4), (2, O.MXFP4, 4), (1, O.BF16, 4),
                                              (1, O.MXFP4, 128)])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("B,T", [(8, 1), (3, 2)])
def test_compress_step_pair_equals_two_steps(gpu, roles, key_fmt, m0, paged, B, T):
    """kv_compress_step_pair (one launch for a CSA layer's KV entry and indexer key; the
    m = 128 first job takes the two-launch route) leaves the caches byte-identical to two
    kv_compress_step calls, and writes the entries the new tokens complete."""
    R, n_cap0 = 256, (8192 // m0)
    rng = np.random.default_rng(B * 10 + T)
    base = rng.integers(0, 8192 - T, size=B)
    base[0] = 8 * m0 - T                            # completes an entry of both jobs
    pos = dev(torch.tensor(base[:, None] + np.arange(T)[None, :], dtype=torch.int32))
    s0 = 40 + 7 * roles + m0
    j0, j1, pool = _pair_jobs(B, R, roles, key_fmt, m0, s0, paged, n_cap0)
    before = [a.copy() for a in _pair_state(j0, j1, pool)]
    ops.kv_compress_step(pos=pos, **j0)
    ops.kv_compress_step(pos=pos, **j1)
    torch.cuda.synchronize()
    want = _pair_state(j0, j1, pool)
    k0, k1, pool2 = _pair_jobs(B, R, roles, key_fmt, m0, s0, paged, n_cap0)
    ops.kv_compress_step_pair(k0, k1, pos)
    torch.cuda.synchronize()
    got = _pair_state(k0, k1, pool2)
    # both jobs wrote something (a KV entry and a key)
    assert (want[0] != before[0]).any() and (want[1] != before[1]).any()
    for w, g_ in zip(want, got):
        assert np.array_equal(w, g_)


@pytest.mark.parametrize("x_fmt,z_ch,d,r,out_fmt", [(O.F32, 1, 128, 0, O.F32), (O.BF16, 256, 256, 0, O.F32),
                                                    (O.BF16, 512, 512, 64, O.KV_PACKED), (O.BF16, 1, 96, 0, O.BF16),
                                                    (O.BF16, 1, 512, 64, O.KV_PACKED)])
def test_compress_step_general_and_wave_kernels(gpu, x_fmt, z_ch, d, r, out_fmt):
    """Decode-time steps outside and inside the one-wave kernel's shape (fp32 rows or
    outputs, per-channel logits, a channel part that is no power of two; and bf16 rows
    with one logit per token) against the oracle's step: the first entry of a sequence
    (half its window before position 0), later entries, tokens that complete none and a
    negative position.  fp32 entries within fp32 rounding; quantised ones equal to the
    oracle's except where its fp64 value sits on a rounding boundary."""
    B, R, m = 3, 64, 4
    pos = torch.tensor([[m - 1, m], [-1, 2 * m - 1], [29, 31]], dtype=torch.int32)
    xr = gen.store(gen.normal((B, R, d), 930 + d), x_fmt)
    zr = gen.random_logits((B, R, z_ch), 931)
    bias = gen.random_logits((2 * m, z_ch), 932)
    n_cap = 16
    rb = O.row_bytes(out_fmt, d, r)
    cache = torch.full((B, n_cap, rb), 0xA5, dtype=torch.uint8)
    kw = dict(d=d, r=r, m=m, overlap=True)
    out, _ = ops.kv_compress_step(dev(xr), x_fmt, dev(zr), dev(bias), dev(pos), out=dev(cache), out_fmt=out_fmt, **kw)
    torch.cuda.synchronize()
    got = host(out)
    want, _, ent = O.kv_compress_step(host(xr), x_fmt, host(zr), host(bias), host(pos), out_fmt=out_fmt, **kw)
    assert sorted(int(e) for e in ent.reshape(-1) if e >= 0) == [0, 1, 7]
    touched = set()
    for b in range(B):
        for j in range(pos.shape[1]):
            e = int(ent[b, j])
            if e < 0:
                continue
            touched.add((b, e))
            if out_fmt == O.F32:
                g_ = got[b, e].view(np.float32).astype(np.float64)
                w_ = want[b, j].astype(np.float64)
                assert np.all(np.abs(g_ - w_) <= 2e-6 * (1.0 + np.abs(w_))), (b, e)
            else:
                dg = O.decode_rows(got[b, e][None], out_fmt, d, r, None)
                dw = O.decode_rows(want[b, j][None], out_fmt, d, r, None)
                assert np.mean(dg != dw) <= 2.0 / d, (b, e)
    for b in range(B):
        for e in range(n_cap):
            if (b, e) not in touched:
                assert np.all(got[b, e] == 0xA5), (b, e)


@pytest.mark.parametrize("B,T,d,r,out_fmt", [(32, 2, 512, 64, O.KV_PACKED), (128, 2, 512, 64, O.KV_PACKED),
                                             (96, 1, 128, 0, O.MXFP4), (40, 2, 256, 64, O.KV_PACKED),
                                             (64, 2, 512, 64, O.KV_PACKED)])
def test_compress_step_wide_batches(gpu, B, T, d, r, out_fmt):
    """Decode steps over many sequences: fewer channel parts per launch, so the one-wave kernel
    runs with 8, 16, 32 and 64 lanes per row (its other lane-move paths) -- against the oracle's
    step, quantised entries equal except where the fp64 value sits on a rounding boundary."""
    R, m = 32, 4
    rng = np.random.default_rng(B * 7 + T)
    base = rng.integers(0, 4000, size=B)
    pos = torch.tensor(base[:, None] + np.arange(T)[None, :], dtype=torch.int32)
    pos[0, 0] = m - 1                                     # a first entry (half its window before 0)
    xr = gen.store(gen.normal((B, R, d), 950 + B), O.BF16)
    zr = gen.random_logits((B, R, 1), 951)
    bias = gen.random_logits((2 * m, 1), 952)
    n_cap = 4096 // m + 1
    rb = O.row_bytes(out_fmt, d, r)
    cache = torch.full((B, n_cap, rb), 0xA5, dtype=torch.uint8)
    scales = torch.full((B, n_cap, d // 32), 0xA5, dtype=torch.uint8) if out_fmt == O.MXFP4 else None
    kw = dict(d=d, r=r, m=m, overlap=True)
    out, sc = ops.kv_compress_step(dev(xr), O.BF16, dev(zr), dev(bias), dev(pos), out=dev(cache),
                                   out_scales=dev(scales) if scales is not None else None, out_fmt=out_fmt, **kw)
    torch.cuda.synchronize()
    got, got_sc = host(out), (host(sc) if sc is not None else None)
    want, want_sc, ent = O.kv_compress_step(host(xr), O.BF16, host(zr), host(bias), host(pos), out_fmt=out_fmt, **kw)
    n = 0
    for b in range(B):
        for j in range(T):
            e = int(ent[b, j])
            if e < 0:
                continue
            n += 1
            dg = O.decode_rows(got[b, e][None], out_fmt, d, r, None if got_sc is None else got_sc[b, e][None])
            dw = O.decode_rows(want[b, j][None], out_fmt, d, r, None if want_sc is None else want_sc[b, j][None])
            assert np.mean(dg != dw) <= 2.0 / d, (b, e)
    assert n >= B // 8
