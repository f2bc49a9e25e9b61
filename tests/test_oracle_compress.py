"""Pins of the oracle's token compression (x-techcon article, section 2, CSA step 1:
learned per-token weights + position bias, softmax, weighted sum, overlapping
blocks; the HCA subsection: the same at m' = 128)."""
import numpy as np
import pytest

import oracle as O
from tests import bruteforce as BF


def _inputs(seed, B, n_tok, d, z_ch, win):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, n_tok, d)).astype(np.float32)
    z = rng.standard_normal((B, n_tok, z_ch)).astype(np.float32)
    bias = rng.standard_normal((win, z_ch)).astype(np.float32)
    return x, z, bias


@pytest.mark.parametrize("m,overlap,z_ch", [(4, True, 1), (4, False, 1), (4, True, 16), (8, False, 16), (1, False, 1)])
def test_matches_bruteforce(m, overlap, z_ch):
    d, n_tok, B = 16, 64, 2
    win = 2 * m if overlap else m
    x, z, bias = _inputs(11, B, n_tok, d, z_ch, win)
    n_e = n_tok // m
    got, _ = O.kv_compress(x, O.F32, z, bias, d=d, m=m, overlap=overlap, e_begin=0, n_e=n_e)
    for b in range(B):
        want = BF.compress(x[b].astype(np.float64), z[b].astype(np.float64), bias.astype(np.float64), m, overlap,
                           range(n_e))
        np.testing.assert_allclose(got[b], want, rtol=1e-6, atol=1e-6)


def test_constant_rows_reproduce_the_constant():
    # weights sum to one, including entry 0 whose look-back window is partly before 0
    d, n_tok, m = 8, 32, 4
    x, z, bias = _inputs(12, 1, n_tok, d, 1, 2 * m)
    x[:] = np.linspace(-3, 3, d, dtype=np.float32)
    got, _ = O.kv_compress(x, O.F32, z, bias, d=d, m=m, overlap=True, e_begin=0, n_e=n_tok // m)
    np.testing.assert_allclose(got[0], np.broadcast_to(x[0, 0], got[0].shape), rtol=1e-6, atol=1e-6)


def test_flat_logits_give_the_window_mean():
    d, n_tok, m = 8, 40, 4
    x, z, bias = _inputs(13, 1, n_tok, d, 1, 2 * m)
    z[:] = 0.7
    bias[:] = 0.0
    got, _ = O.kv_compress(x, O.F32, z, bias, d=d, m=m, overlap=True, e_begin=0, n_e=n_tok // m)
    for i in range(n_tok // m):
        lo = max(0, (i + 1) * m - 2 * m)
        want = x[0, lo:(i + 1) * m].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(got[0, i], want, rtol=1e-6, atol=1e-6)
    # without overlap: mean of the m rows of the block
    bias2 = np.zeros((m, 1), np.float32)
    got2, _ = O.kv_compress(x, O.F32, z, bias2, d=d, m=m, overlap=False, e_begin=0, n_e=n_tok // m)
    np.testing.assert_allclose(got2[0], x[0].reshape(-1, m, d).astype(np.float64).mean(axis=1), rtol=1e-6,
                               atol=1e-6)


def test_shift_invariance_of_logits_and_bias():
    d, n_tok, m = 8, 32, 4
    x, z, bias = _inputs(14, 1, n_tok, d, 1, 2 * m)
    a, _ = O.kv_compress(x, O.F32, z, bias, d=d, m=m, overlap=True, e_begin=0, n_e=8)
    b, _ = O.kv_compress(x, O.F32, z + 3.0, bias - 1.5, d=d, m=m, overlap=True, e_begin=0, n_e=8)
    np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-6)


def test_position_bias_is_per_window_slot():
    # a huge bias on one window slot selects exactly that raw row
    d, n_tok, m = 8, 32, 4
    x, z, bias = _inputs(15, 1, n_tok, d, 1, 2 * m)
    for slot in range(2 * m):
        bb = np.full((2 * m, 1), -1e4, np.float32)
        bb[slot] = 1e4
        got, _ = O.kv_compress(x, O.F32, z, bb, d=d, m=m, overlap=True, e_begin=1, n_e=6)
        for q in range(6):
            i = 1 + q
            np.testing.assert_array_equal(got[0, q], x[0, (i + 1) * m - 2 * m + slot])


def test_m1_is_the_identity():
    d, n_tok = 32, 10
    x, z, bias = _inputs(16, 2, n_tok, d, 1, 1)
    got, _ = O.kv_compress(x, O.F32, z, bias, d=d, m=1, overlap=False, e_begin=0, n_e=n_tok)
    np.testing.assert_array_equal(got, x)


def test_partial_range_and_pos0_offset():
    # entries 4..7 computed from a raw buffer that starts at position 12 (look-back m)
    d, m = 8, 4
    x, z, bias = _inputs(17, 1, 40, d, 1, 2 * m)
    full, _ = O.kv_compress(x, O.F32, z, bias, d=d, m=m, overlap=True, e_begin=0, n_e=10)
    part, _ = O.kv_compress(x[:, 12:36], O.F32, z[:, 12:36], bias, d=d, m=m, overlap=True, e_begin=4, n_e=4,
                            x_pos0=12)
    np.testing.assert_array_equal(part[0], full[0, 4:8])
    with pytest.raises(ValueError):
        O.kv_compress(x[:, 13:36], O.F32, z[:, 13:36], bias, d=d, m=m, overlap=True, e_begin=4, n_e=4, x_pos0=13)


def test_quantized_outputs_are_the_encoded_values():
    d, r, m = 128, 32, 4
    x, z, bias = _inputs(18, 2, 64, d, 1, 2 * m)
    f, _ = O.kv_compress(x, O.F32, z, bias, d=d, r=r, m=m, overlap=True, e_begin=0, n_e=16)
    for fmt in (O.BF16, O.KV_PACKED, O.MXFP4):
        q, sc = O.kv_compress(x, O.F32, z, bias, d=d, r=r, m=m, overlap=True, e_begin=0, n_e=16, out_fmt=fmt)
        back = BF.decode(q, fmt, d, r, sc).reshape(2, 16, d)
        # the decoded value is the nearest grid point: error at most half a step of the format
        if fmt == O.BF16:
            tol = np.abs(f) * 2.0 ** -8 + 1e-30
        elif fmt == O.KV_PACKED:
            tol = np.concatenate([np.abs(f[..., :r]) * 2.0 ** -8, np.maximum(np.abs(f[..., r:]) * 2.0 ** -4,
                                                                             2.0 ** -10)], axis=-1)
        else:
            tol = np.repeat(2.0 ** (sc.astype(np.float64) - 127), 32, axis=-1).reshape(f.shape)
        assert np.all(np.abs(back - f) <= tol * 1.0000001)
