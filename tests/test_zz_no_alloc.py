"""index_topk_noalloc (the entry point for callers that cannot allocate) against
index_topk with a caller workspace: identical indices and scores, on two calls in a row
-- the second smaller, so it reuses the static scratch the first one filled -- and a
host-side refusal of a call whose staging exceeds the scratch."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from compressed_sparse_long_02_amd import _lib, gen, ops
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


def _case(fmt, B, Tq, H_I, d_I, N, seed):
    if fmt == O.MXFP4:
        qc, qs = gen.random_mxfp4(B * Tq * H_I, d_I, seed)
        kc, ks = gen.random_mxfp4(B * N, d_I, seed + 1)
        return (dev(qc.reshape(B, Tq, H_I, -1)), dev(qs.reshape(B, Tq, H_I, -1)), dev(kc.reshape(B, N, -1)),
                dev(ks.reshape(B, N, -1)))
    q = gen.store(gen.normal((B, Tq, H_I, d_I), seed, 1 / math.sqrt(d_I)), fmt)
    k = gen.store(gen.normal((B, N, d_I), seed + 1, 1 / math.sqrt(d_I)), fmt)
    return dev(q), None, dev(k), None


@pytest.mark.parametrize("calls", [
    # (fmt, B, Tq, H_I, d_I, N, m, k): the first call larger than the second
    ((O.MXFP4, 8, 1, 64, 128, 262144, 4, 1024), (O.BF16, 2, 3, 16, 128, 40000, 4, 512)),
    ((O.BF16, 4, 2, 16, 128, 100000, 4, 512), (O.MXFP4, 1, 1, 64, 128, 30000, 4, 1024)),
])
def test_noalloc_matches_index_topk(gpu, calls):
    assert _lib.lib().csl_noalloc_scratch_bytes() == 96 << 20
    for n, (fmt, B, Tq, H_I, d_I, N, m, k) in enumerate(calls):
        qi, qs, ki, ks = _case(fmt, B, Tq, H_I, d_I, N, 700 + 10 * n)
        w = dev(gen.normal((B, Tq, H_I), 705 + 10 * n, 1 / math.sqrt(H_I)))
        rng = np.random.default_rng(n)
        qpos = dev(torch.from_numpy(rng.integers(N * m // 2, N * m, size=(B, Tq)).astype(np.int32)))
        kw = dict(fmt=fmt, H_I=H_I, d_I=d_I, m=m, n_cap=N, k=k, qi_scales=qs, ki_scales=ks)
        need = _lib.lib().csl_index_topk_workspace(B, Tq, N, k)
        assert 0 < need <= _lib.lib().csl_noalloc_scratch_bytes()     # the staged (several-slice) path
        ref_i, ref_s = ops.index_topk(qi, w, ki, qpos, **kw)
        out_i = torch.full((B, Tq, k), -7, dtype=torch.int32, device=qi.device)
        out_s = torch.full((B, Tq, k), 7.0, dtype=torch.float32, device=qi.device)
        ops.index_topk_noalloc(qi, w, ki, qpos, out_idx=out_i, out_score=out_s, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out_i, ref_i), "call %d: indices differ" % n
        assert torch.equal(out_s, ref_s), "call %d: scores differ" % n


def test_noalloc_refuses_more_than_its_scratch(gpu):
    B, Tq, H_I, d_I, N, m, k = 1, 12, 16, 128, 1 << 20, 4, 1024
    qi, _, ki, _ = _case(O.BF16, B, Tq, H_I, d_I, N, 777)
    w = dev(gen.normal((B, Tq, H_I), 778))
    qpos = dev(gen.positions(B, Tq, N * m - 1))
    assert _lib.lib().csl_index_topk_workspace(B, Tq, N, k) > _lib.lib().csl_noalloc_scratch_bytes()
    out_i = torch.full((B, Tq, k), -7, dtype=torch.int32, device=qi.device)
    with pytest.raises(_lib.CslError) as e:
        ops.index_topk_noalloc(qi, w, ki, qpos, fmt=O.BF16, H_I=H_I, d_I=d_I, m=m, n_cap=N, k=k, out_idx=out_i)
    assert e.value.code == _lib.CSL_EWORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out_i == -7)                                    # nothing was launched
