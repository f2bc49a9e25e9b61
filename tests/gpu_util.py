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


class TopkStats:
    """What check_topk saw: queries checked, queries whose set differs from the oracle's
    (tie swaps), entries swapped, the largest oracle-score gap of a swapped entry to the
    k-th score, and the largest |GPU score - oracle score| of a selected entry."""

    def __init__(self):
        self.queries = self.swapped = self.entries = 0
        self.max_gap = self.max_err = 0.0

    def __str__(self):
        return ("%d queries, %d with tie swaps (%d entries), largest swap gap %.3g, largest score error %.3g"
                % (self.queries, self.swapped, self.entries, self.max_gap, self.max_err))


def cap(n_queries):
    """Queries allowed to carry a tie swap in one test: one in 64, plus one."""
    return 1 + n_queries // 64


def check_topk(gpu_idx, gpu_score, ora_idx, all_scores, k, *, bound=None, rel_tie=1e-6, max_swapped=0):
    """Top-k parity of the GPU against the oracle, per query (both lists ascending, -1 pads):

    - the same number of entries, GPU indices strictly ascending, pads -1 with -inf scores;
    - score accuracy: err = max |GPU score - oracle score| over the GPU's selected entries,
      and err <= bound (the worst-case fp32 accumulation bound of that query) when given;
    - the sets are equal, or differ only by tie swaps: every entry in the symmetric
      difference has an oracle score within tol = max(rel_tie * max(1, |s_k|), 2 * err) of
      the oracle's k-th score s_k (entries the GPU kept score at most s_k, entries it left
      out at least s_k), i.e. within the tie rule of 1e-6 or twice the error the kernel
      itself shows on this query's scores; and every entry the GPU kept scores, by its own
      numbers, at least its own k-th score;
    - at most `max_swapped` queries differ at all.
    Returns a TopkStats."""
    st = TopkStats()
    B, Tq, _ = gpu_idx.shape
    for b in range(B):
        for j in range(Tq):
            st.queries += 1
            g, o = gpu_idx[b, j], ora_idx[b, j]
            gs = gpu_score[b, j]
            gv, ov = g[g >= 0], o[o >= 0]
            assert len(gv) == len(ov), (b, j, len(gv), len(ov))
            assert np.all(np.diff(gv) > 0), "GPU indices must be strictly ascending"
            assert np.all(g[len(gv):] == -1) and np.all(np.isneginf(gs[len(gv):]))
            s = all_scores[b, j]
            gsv = gs[:len(gv)].astype(np.float64)
            err = float(np.max(np.abs(gsv - s[gv]))) if len(gv) else 0.0
            st.max_err = max(st.max_err, err)
            if bound is not None and len(gv):
                bq = float(bound[b, j] if np.ndim(bound) else bound)
                assert err <= bq + 1e-6 * float(np.max(np.abs(s[gv]))), \
                    "score error %.3g above the fp32 bound %.3g at (%d,%d)" % (err, bq, b, j)
            if np.array_equal(gv, ov):
                continue
            kth = float(np.min(s[ov]))
            tol = max(rel_tie * max(1.0, abs(kth)), 2.0 * err)
            extra, missing = np.setdiff1d(gv, ov), np.setdiff1d(ov, gv)
            assert np.all(s[extra] <= kth) and np.all(s[missing] >= kth), (b, j)
            gap = float(np.max(np.abs(s[np.concatenate([extra, missing])] - kth)))
            assert gap <= tol, "top-k set differs beyond ties at (%d,%d): gap %.3g > tol %.3g (err %.3g)" % (
                b, j, gap, tol, err)
            assert np.all(gsv >= gsv.min()), (b, j)
            st.swapped += 1
            st.entries += len(extra)
            st.max_gap = max(st.max_gap, gap)
    assert st.swapped <= max_swapped, "%d queries with tie swaps, more than the %d allowed (%s)" % (
        st.swapped, max_swapped, st)
    return st


def score_error_bound(qd, wd, Kd):
    """Bound on the fp32 accumulation error of indexer scores, per query:
    2 * n * 2^-24 * max_s sum_h |w_h| sum_i |q_hi k_si|, n = d_I + H_I terms on the
    longest accumulation path.  qd [Tq, H, d], wd [Tq, H], Kd [N, d] (decoded)."""
    Tq, H, d = qd.shape
    wq = (np.abs(wd)[:, :, None] * np.abs(qd)).sum(axis=1)          # [Tq, d]
    mag = wq @ np.abs(Kd).T                                          # [Tq, N]
    return 2.0 * (d + H) * 2.0 ** -24 * mag.max(axis=1)


def quantum(vals, fmt, d, r=0, scales=None):
    """Spacing of the stored format's grid at each decoded value (the size of one
    rounding step there): bf16 ulp, e4m3fn step (2^-9 below the normal range), e2m1 step
    times the block scale; [n, d] for [n, d] values."""
    v = np.abs(np.asarray(vals, np.float64)).reshape(-1, d)
    e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    if fmt == O.F32:
        return np.ldexp(1.0, (np.maximum(e, -126) - 23).astype(np.int64))
    bf = np.ldexp(1.0, (np.maximum(e, -126) - 7).astype(np.int64))
    if fmt == O.BF16:
        return bf
    if fmt == O.KV_PACKED:
        e8 = np.ldexp(1.0, (np.maximum(e, -6) - 3).astype(np.int64))
        out = e8.copy()
        out[:, :r] = bf[:, :r]
        return out
    sc = np.ldexp(1.0, np.asarray(scales, np.int64).reshape(-1, d // 32) - 127)
    sc = np.repeat(sc, 32, axis=1)
    rel = v / sc                                     # on the e2m1 grid 0 .. 6
    step = np.where(rel < 2.0, 0.5, np.where(rel < 4.0, 1.0, 2.0))
    return step * sc


def close_quantised(got, ref, fmt, d, r=0, got_sc=None, ref_sc=None, max_mismatch=2):
    """Quantised rows from fp32 (GPU) and fp64 (oracle) arithmetic: equal except for at most
    `max_mismatch` elements, each at most one rounding step of the format apart plus the
    fp32 rounding of the value before it was stored (2^-18 of the row's largest value:
    a pooled value that cancels to near zero keeps that absolute error while the bf16
    grid there is much finer).  MXFP4 rows must also carry the same block scales."""
    a = O.decode_rows(got, fmt, d, r, got_sc)
    b = O.decode_rows(ref, fmt, d, r, ref_sc)
    if fmt == O.MXFP4:
        assert np.array_equal(np.asarray(got_sc).reshape(-1), np.asarray(ref_sc).reshape(-1)), "block scales differ"
    bad = a != b
    nbad = int(np.sum(bad))
    assert nbad <= max_mismatch, "%d quantised elements differ (at most %d allowed)" % (nbad, max_mismatch)
    if nbad:
        q = quantum(np.maximum(np.abs(a), np.abs(b)), fmt, d, r, ref_sc)
        slack = 2.0 ** -18 * np.max(np.abs(b), axis=1, keepdims=True)
        ok = np.abs(a - b) <= (q + slack) * (1 + 1e-12)
        if not np.all(ok[bad]):
            i = np.argwhere(bad & ~ok)[0]
            raise AssertionError("element %s is more than one step off: GPU %r, oracle %r, step %r, slack %r"
                                 % (tuple(i), a[tuple(i)], b[tuple(i)], q[tuple(i)], slack[i[0], 0]))
    return nbad
