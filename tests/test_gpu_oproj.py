"""GPU parity of grouped_out_proj (x-techcon article, section 2, HCA subsection; CSDN
explainer, "Grouped Output Projection") against the oracle: fp32 outputs within the
fp32 accumulation bound of each element (K * 2^-23 * sum_k |x_k w_k|), bf16 outputs
additionally within one bf16 rounding."""
import numpy as np
import pytest
import torch

import oracle as O
from compressed_sparse_long_02_amd import gen, ops
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


def _bits(t):
    return host(t.view(torch.int16))


CASES = [
    # (M, G, K, R): decode (few tokens: one block per 32 outputs, K split over its waves)
    # and prefill sizes (LDS-tiled), ragged M
    (16, 8, 4096, 1024),       # the benchmark's decode shape: 64 heads x 512 in 8 groups -> 8 x 1024
    (5, 2, 256, 128),
    (40, 1, 512, 256),         # the common projection (G = 1), 3 row tiles
    (300, 4, 1024, 256),       # tiled, ragged last row tile
    (2048, 8, 4096, 1024),     # a prefill chunk's worth of tokens (64 rows checked)
]


@pytest.mark.parametrize("case", CASES, ids=["x".join(map(str, c)) for c in CASES])
@pytest.mark.parametrize("out_fmt", [O.F32, O.BF16])
def test_grouped_out_proj_parity(gpu, case, out_fmt):
    M, G, K, R = case
    x = gen.with_outliers(gen.normal((M, G * K), 800 + M, device="cuda"), 801).to(torch.bfloat16)
    w = gen.normal((G, R, K), 802 + K, K ** -0.5, device="cuda").to(torch.bfloat16)
    y = ops.grouped_out_proj(x, w, G=G, out_fmt=out_fmt)
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 300 else np.linspace(0, M - 1, 64).astype(int)
    xs = _bits(x)[rows]
    want = O.grouped_out_proj(xs, O.BF16, _bits(w), O.BF16, G=G, K=K, R=R).astype(np.float64)
    xa = np.abs(x.float().cpu().numpy()[rows]).astype(np.float64).reshape(len(rows), G, K)
    wa = np.abs(w.float().cpu().numpy()).astype(np.float64)
    mag = np.einsum("mgk,grk->mgr", xa, wa).reshape(len(rows), G * R)
    bound = K * 2.0 ** -23 * mag + 1e-30
    got = y.float().cpu().numpy()[rows].astype(np.float64)
    if out_fmt == O.BF16:
        bound = bound + 2.0 ** -8 * np.abs(want)
    err = np.abs(got - want)
    assert np.all(err <= bound), "max err %.3g, at bound ratio %.3g" % (err.max(), (err / bound).max())
    print("%s: max-abs %.3g (largest fraction of the bound %.3g)" % (case, err.max(), (err / bound).max()))


def test_grouped_out_proj_is_deterministic(gpu):
    x = gen.normal((16, 8 * 4096), 811, device="cuda").to(torch.bfloat16)
    w = gen.normal((8, 1024, 4096), 812, 1 / 64, device="cuda").to(torch.bfloat16)
    a = ops.grouped_out_proj(x, w, G=8)
    b = ops.grouped_out_proj(x, w, G=8)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
