"""Helpers of the GPU parity tests: host<->device moves and comparison rules."""
import numpy as np
import torch

import oracle as O


def dev(t, device="cuda:0"):
    if isinstance(t, np.ndarray):
        t = torch.from_numpy(np.ascontiguousarray(t))
    return t.contiguous().to(device)


def host(t):
    return t.detach().cpu().numpy()


def max_abs(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def oracle_all_scores(qi, qi_fmt, w, ki, ki_fmt, q_pos, *, H_I, d_I, m, n_cap, qi_scales=None, ki_scales=None):
    """Oracle scores of every visible entry, [B, Tq, n_cap] (-inf where not visible)."""
    idx, sc = O.index_topk(qi, qi_fmt, w, ki, ki_fmt, q_pos, H_I=H_I, d_I=d_I, m=m, n_cap=n_cap, k=max(n_cap, 1),
                           qi_scales=qi_scales, ki_scales=ki_scales)
    B, Tq, _ = idx.shape
    full = np.full((B, Tq, max(n_cap, 1)), -np.inf)
    for b in range(B):
        for j in range(Tq):
            v = idx[b, j] >= 0
            full[b, j, idx[b, j, v]] = sc[b, j, v]
    return full


def check_topk(gpu_idx, ora_idx, all_scores, k, rel_tie=1e-6, abs_bound=None):
    """Index sets must be equal except for swaps between entries whose oracle scores
    tie with the k-th score within max(rel_tie * max(1, |s_k|), abs_bound).  Both
    lists ascending with -1 padding.  Returns (n_swapped_queries, max_gap)."""
    B, Tq, _ = gpu_idx.shape
    n_sw, worst = 0, 0.0
    for b in range(B):
        for j in range(Tq):
            g = gpu_idx[b, j]
            o = ora_idx[b, j]
            gv, ov = g[g >= 0], o[o >= 0]
            assert len(gv) == len(ov), (b, j, len(gv), len(ov))
            assert np.all(np.diff(gv) > 0), "GPU indices must be strictly ascending"
            assert np.all(g[len(gv):] == -1)
            if np.array_equal(gv, ov):
                continue
            s = all_scores[b, j]
            kth = np.sort(s[ov])[0]
            ab = 0.0 if abs_bound is None else float(abs_bound[b, j] if np.ndim(abs_bound) else abs_bound)
            tol = max(rel_tie * max(1.0, abs(kth)), ab)
            diff = np.setxor1d(gv, ov)
            gap = float(np.max(np.abs(s[diff] - kth)))
            assert gap <= tol, "top-k set differs beyond ties at (%d,%d): gap %.3g > tol %.3g" % (b, j, gap, tol)
            n_sw += 1
            worst = max(worst, gap)
    return n_sw, worst


def score_error_bound(qd, wd, Kd):
    """Bound on the fp32 accumulation error of indexer scores, per query:
    2 * n * 2^-24 * max_s sum_h |w_h| sum_i |q_hi k_si|, n = d_I + H_I terms on the
    longest accumulation path.  qd [Tq, H, d], wd [Tq, H], Kd [N, d] (decoded)."""
    Tq, H, d = qd.shape
    wq = (np.abs(wd)[:, :, None] * np.abs(qd)).sum(axis=1)          # [Tq, d]
    mag = wq @ np.abs(Kd).T                                          # [Tq, N]
    return 2.0 * (d + H) * 2.0 ** -24 * mag.max(axis=1)
