"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds none of the method's arithmetic: it only draws seeded random
numbers and converts them to storage dtypes with torch's own casts (bf16, OCP fp8
e4m3fn) or draws storage codes directly (MXFP4 nibbles and e8m0 scales).  Both the
HIP path and the oracle consume exactly the bytes produced here.

Packed KV rows follow the storage layout of the mixed-precision KV cache: the first
`r` (RoPE) dims as bf16, then the remaining d-r dims as fp8 e4m3fn, one row after
another (576 bytes for d=512, r=64).
"""
from __future__ import annotations

import numpy as np
import torch

F32, BF16, KV_PACKED, MXFP4 = 0, 1, 2, 3


def row_bytes(fmt: int, d: int, r: int = 0) -> int:
    if fmt == F32:
        return 4 * d
    if fmt == BF16:
        return 2 * d
    if fmt == KV_PACKED:
        return 2 * r + (d - r)
    if fmt == MXFP4:
        return d // 2
    raise ValueError("unknown format %r" % fmt)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def normal(shape, seed: int, std: float = 1.0, device="cpu") -> torch.Tensor:
    """fp32 N(0, std^2) with a torch generator seeded by `seed` on `device`."""
    x = torch.randn(tuple(shape), generator=_gen(seed, device), device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def outlier_channels(dim: int, seed: int, frac: float = 0.01) -> torch.Tensor:
    """ceil(frac*dim) distinct channel indices, seeded (heavy-tailed channels)."""
    n = max(1, int(np.ceil(frac * dim)))
    rng = np.random.Generator(np.random.PCG64(seed))
    return torch.from_numpy(np.sort(rng.choice(dim, size=n, replace=False)).astype(np.int64))


def with_outliers(x: torch.Tensor, seed: int, frac: float = 0.01, factor: float = 10.0) -> torch.Tensor:
    """Multiply a seeded set of last-dim channels by `factor` (in place)."""
    ch = outlier_channels(x.shape[-1], seed, frac).to(x.device)
    x[..., ch] *= factor
    return x


def bf16_bytes(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> bf16 (torch cast, round-to-nearest-even) as a uint8 view [..., 2d]."""
    return x.to(torch.bfloat16).contiguous().view(torch.uint8)


def pack_kv(x: torch.Tensor, r: int) -> torch.Tensor:
    """fp32 rows [..., d] -> packed rows uint8 [..., 2r + d - r] via torch casts."""
    lo = x[..., :r].to(torch.bfloat16).contiguous().view(torch.uint8)
    hi = x[..., r:].to(torch.float8_e4m3fn).contiguous().view(torch.uint8)
    return torch.cat([lo, hi], dim=-1).contiguous()


def store(x: torch.Tensor, fmt: int, r: int = 0) -> torch.Tensor:
    """fp32 rows -> stored bytes of `fmt` (F32 returns the fp32 tensor itself)."""
    if fmt == F32:
        return x.contiguous()
    if fmt == BF16:
        return bf16_bytes(x)
    if fmt == KV_PACKED:
        return pack_kv(x, r)
    raise ValueError("store() covers F32/BF16/KV_PACKED; draw MXFP4 with random_mxfp4()")


def random_mxfp4(n_rows: int, d: int, seed: int, scale_lo: int = 124, scale_hi: int = 129,
                 device="cpu"):
    """Random MXFP4 rows drawn directly as codes: nibbles uniform over the 16 e2m1 codes
    and e8m0 block scales uniform in [scale_lo, scale_hi].  Returns (codes uint8
    [n_rows, d/2], scales uint8 [n_rows, d/32])."""
    g = _gen(seed, device)
    codes = torch.randint(0, 256, (n_rows, d // 2), generator=g, device=device, dtype=torch.int32).to(torch.uint8)
    scales = torch.randint(scale_lo, scale_hi + 1, (n_rows, d // 32), generator=g, device=device,
                           dtype=torch.int32).to(torch.uint8)
    return codes, scales


def random_e8m0(n_rows: int, ranges, seed: int, device="cpu") -> torch.Tensor:
    """e8m0 block-scale codes [n_rows, len(ranges)]: block j uniform in ranges[j] = (lo, hi)."""
    g = _gen(seed, device)
    cols = [torch.randint(lo, hi + 1, (n_rows, 1), generator=g, device=device, dtype=torch.int32)
            for lo, hi in ranges]
    return torch.cat(cols, dim=1).to(torch.uint8)


def random_logits(shape, seed: int, device="cpu") -> torch.Tensor:
    """Compression logits / biases: plain N(0,1) fp32."""
    return normal(shape, seed, 1.0, device)


def positions(B: int, Tq: int, last: int | list, device="cpu") -> torch.Tensor:
    """Query positions [B, Tq] int32: the Tq positions ending at `last` (per sequence)."""
    last = [last] * B if np.isscalar(last) else list(last)
    rows = [np.arange(l - Tq + 1, l + 1, dtype=np.int32) for l in last]
    return torch.from_numpy(np.stack(rows)).to(device)
