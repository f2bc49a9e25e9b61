"""CPU oracle of the hybrid compressed attention layer (CSA + HCA): TEST INFRASTRUCTURE.

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls anything here, and this package
imports nothing from it.

``oracle.c`` holds the arithmetic (plain C, fp64, OpenMP over independent queries);
this module only compiles it with gcc on first use and marshals numpy arrays.
Every function mirrors one C-ABI call of the library, with host arrays.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, KV_PACKED, MXFP4 = 0, 1, 2, 3


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(build())
        L = _lib
        vp, i64, i32, f64 = C.c_void_p, C.c_int64, C.c_int, C.c_double
        L.orc_bf16_decode.restype = f64
        L.orc_bf16_decode.argtypes = [C.c_uint16]
        L.orc_e4m3_decode.restype = f64
        L.orc_e4m3_decode.argtypes = [C.c_uint8]
        L.orc_e2m1_decode.restype = f64
        L.orc_e2m1_decode.argtypes = [C.c_uint8]
        L.orc_e8m0_decode.restype = f64
        L.orc_e8m0_decode.argtypes = [C.c_uint8]
        L.orc_bf16_encode.restype = C.c_uint16
        L.orc_bf16_encode.argtypes = [f64]
        L.orc_e4m3_encode.restype = C.c_uint8
        L.orc_e4m3_encode.argtypes = [f64]
        L.orc_e2m1_encode.restype = C.c_uint8
        L.orc_e2m1_encode.argtypes = [f64]
        L.orc_mx_block_exponent.restype = i32
        L.orc_mx_block_exponent.argtypes = [f64]
        L.orc_row_bytes.restype = i64
        L.orc_row_bytes.argtypes = [i32, i32, i32]
        L.orc_decode_rows.restype = None
        L.orc_decode_rows.argtypes = [vp, vp, i32, i32, i32, i64, vp]
        L.orc_encode_rows.restype = None
        L.orc_encode_rows.argtypes = [vp, i32, i32, i32, i64, vp, vp]
        L.orc_kv_compress.restype = i32
        L.orc_kv_compress.argtypes = [vp, i32, i64, i64, i64, i64, i32, vp, i32, i64, vp,
                                      i32, i32, i32, i32, i32, i64, i64, vp, i32, vp, i64, i64]
        L.orc_kv_compress_step.restype = i32
        L.orc_kv_compress_step.argtypes = [vp, i32, i64, i64, i32, vp, i32, i64, vp, vp, i32, i32, i32, i32, i32,
                                           i32, vp, i32, vp, vp]
        L.orc_paged_gather.restype = None
        L.orc_paged_gather.argtypes = [vp, i64, vp, i64, i32, i64, i32, i64, vp, i64]
        L.orc_grouped_out_proj.restype = i32
        L.orc_grouped_out_proj.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, vp]
        L.orc_index_topk.restype = i32
        L.orc_index_topk.argtypes = [vp, i32, vp, vp, vp, i32, vp, i64, i64,
                                     vp, i32, i32, i32, i32, i32, i64, i32, vp, vp]
        L.orc_csa_attend.restype = i32
        L.orc_csa_attend.argtypes = [vp, i32, vp, i32, i64, i64, vp, i32, vp, i64, i64, i64, vp,
                                     vp, i32, i32, i32, i32, i32, i32, f64, vp, i32, vp]
        L.orc_hca_attend.restype = i32
        L.orc_hca_attend.argtypes = [vp, i32, vp, i32, i64, i64, i32, vp, i64, i64, i64, vp,
                                     vp, i32, i32, i32, i32, i32, i32, f64, vp, i32, vp]
        L.orc_num_threads.restype = i32
        L.orc_num_threads.argtypes = []
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def row_bytes(fmt: int, d: int, r: int = 0) -> int:
    return int(lib().orc_row_bytes(fmt, d, r))


def num_threads() -> int:
    return int(lib().orc_num_threads())


# ---- codecs -----------------------------------------------------------------

def decode_rows(data: np.ndarray, fmt: int, d: int, r: int = 0, scales: np.ndarray | None = None) -> np.ndarray:
    """Decode stored rows (uint8 [..., rowbytes] or f32) into float64 [..., d]."""
    rb = row_bytes(fmt, d, r)
    raw = np.ascontiguousarray(data).view(np.uint8).reshape(-1)
    n = raw.size // rb
    out = np.empty((n, d), np.float64)
    sc = _c(scales, np.uint8)
    lib().orc_decode_rows(_p(raw), _p(sc), fmt, d, r, n, _p(out))
    return out


def encode_rows(values: np.ndarray, fmt: int, d: int, r: int = 0):
    """Encode float rows [n, d] -> (uint8 [n, rowbytes], scales uint8 [n, d/32] or None)."""
    v = np.ascontiguousarray(values, np.float64).reshape(-1, d)
    n = v.shape[0]
    out = np.zeros((n, row_bytes(fmt, d, r)), np.uint8)
    sc = np.zeros((n, d // 32), np.uint8) if fmt == MXFP4 else None
    lib().orc_encode_rows(_p(v), fmt, d, r, n, _p(out), _p(sc))
    return out, sc


def bf16_decode(code: int) -> float:
    return lib().orc_bf16_decode(code)


def e4m3_decode(code: int) -> float:
    return lib().orc_e4m3_decode(code)


def e2m1_decode(code: int) -> float:
    return lib().orc_e2m1_decode(code)


def e8m0_decode(code: int) -> float:
    return lib().orc_e8m0_decode(code)


def bf16_encode(x: float) -> int:
    return lib().orc_bf16_encode(float(x))


def e4m3_encode(x: float) -> int:
    return lib().orc_e4m3_encode(float(x))


def e2m1_encode(x: float) -> int:
    return lib().orc_e2m1_encode(float(x))


def mx_block_exponent(amax: float) -> int:
    return lib().orc_mx_block_exponent(float(amax))


# ---- the four operations ------------------------------------------------------

def kv_compress(x, x_fmt, z, bias, *, d, r=0, m, overlap, e_begin, n_e, x_pos0=0, out_fmt=F32, x_rows=0, x_roles=1):
    """x: per-sequence raw rows [B, n_tok, rowbytes] (uint8 view) or f32 [B, n_tok, x_roles*d];
    z: f32 [B, n_tok, z_ch]; bias: f32 [win, z_ch].  x_rows > 0: x and z are rings of
    x_rows rows (position p in row (p - x_pos0) mod x_rows).  x_roles = 2: two-role rows
    (look-back value, then current value).  Returns (out [B, n_e, rowbytes] uint8 (f32
    [B, n_e, d] for F32), scales [B, n_e, d/32] or None)."""
    B, n_tok = x.shape[0], x.shape[1]
    xb = np.ascontiguousarray(x).view(np.uint8).reshape(B, -1)
    zz = _c(z, np.float32).reshape(B, n_tok, -1)
    z_ch = zz.shape[2]
    bb = _c(bias, np.float32)
    orb = row_bytes(out_fmt, d, r)
    out = np.zeros((B, max(n_e, 0), orb), np.uint8)
    sc = np.zeros((B, max(n_e, 0), d // 32), np.uint8) if out_fmt == MXFP4 else None
    rc = lib().orc_kv_compress(_p(xb), x_fmt, xb.shape[1], x_pos0, n_tok, x_rows, x_roles, _p(zz), z_ch,
                               zz[0].nbytes if B else 0, _p(bb), B, d, r, m, int(bool(overlap)), e_begin, n_e, _p(out),
                               out_fmt, _p(sc), out.shape[1] * orb, 0 if sc is None else sc.shape[1] * (d // 32))
    if rc != 0:
        raise ValueError("orc_kv_compress rejected its arguments (%d)" % rc)
    if out_fmt == F32:
        return out.view(np.float32).reshape(B, max(n_e, 0), d), None
    return out, sc


def kv_compress_step(x, x_fmt, z, bias, pos, *, d, r=0, m, overlap, out_fmt=F32, x_roles=1):
    """Decode-time compression from rings: x [B, x_rows, rowbytes] / f32, z [B, x_rows, z_ch]
    (position p in row p mod x_rows); pos int32 [B, T] new token positions.  Returns (out
    [B, T, rowbytes] (f32 [B, T, d]), scales [B, T, d/32] or None, entry int32 [B, T]):
    the entry a token completes (or -1) and its compressed row."""
    B, x_rows = x.shape[0], x.shape[1]
    xb = np.ascontiguousarray(x).view(np.uint8).reshape(B, -1)
    zz = _c(z, np.float32).reshape(B, x_rows, -1)
    pp = _c(pos, np.int32)
    T = pp.shape[1]
    orb = row_bytes(out_fmt, d, r)
    out = np.zeros((B, T, orb), np.uint8)
    sc = np.zeros((B, T, d // 32), np.uint8) if out_fmt == MXFP4 else None
    ent = np.zeros((B, T), np.int32)
    rc = lib().orc_kv_compress_step(_p(xb), x_fmt, xb.shape[1], x_rows, x_roles, _p(zz), zz.shape[2],
                                    zz[0].nbytes if B else 0, _p(_c(bias, np.float32)), _p(pp), B, T, d, r, m,
                                    int(bool(overlap)), _p(out), out_fmt, _p(sc), _p(ent))
    if rc != 0:
        raise ValueError("orc_kv_compress_step rejected its arguments (%d)" % rc)
    if out_fmt == F32:
        return out.view(np.float32).reshape(B, T, d), None, ent
    return out, sc, ent


def paged_gather(pool, row_bytes_, block_table, entries_per_block, block_bytes, n):
    """Rows 0..n-1 of every sequence of a paged pool (uint8 bytes), through the block table
    int32 [B, max_blocks]: uint8 [B, n, row_bytes_] (zero rows for negative block ids)."""
    pb = np.ascontiguousarray(pool).view(np.uint8).reshape(-1)
    bt = _c(block_table, np.int32)
    B = bt.shape[0]
    out = np.zeros((B, n, row_bytes_), np.uint8)
    lib().orc_paged_gather(_p(pb), row_bytes_, _p(bt), bt.shape[1], entries_per_block, block_bytes, B, n, _p(out),
                           n * row_bytes_)
    return out


def grouped_out_proj(x, x_fmt, w, w_fmt, *, G, K, R):
    """x: M rows of G*K values (f32, or bf16 bits as uint16/int16); w: [G, R, K] (f32 or bf16
    bits).  Returns f32 [M, G*R]: group g's outputs = x[:, gK:(g+1)K] @ w[g].T."""
    xb = np.ascontiguousarray(x).view(np.uint8).reshape(-1)
    wb = np.ascontiguousarray(w).view(np.uint8).reshape(-1)
    M = xb.size // row_bytes(x_fmt, G * K)
    out = np.zeros((M, G * R), np.float32)
    rc = lib().orc_grouped_out_proj(_p(xb), x_fmt, _p(wb), w_fmt, M, G, K, R, _p(out))
    if rc != 0:
        raise ValueError("orc_grouped_out_proj rejected its arguments (%d)" % rc)
    return out


def index_topk(qi, qi_fmt, w, ki, ki_fmt, q_pos, *, H_I, d_I, m, n_cap, k, qi_scales=None, ki_scales=None):
    """qi: [B, Tq, H_I, qrowbytes] bytes (or f32 [B,Tq,H_I,d_I]); w: f32 [B,Tq,H_I];
    ki: [B, N, krowbytes] bytes (or f32 [B,N,d_I]); q_pos: int32 [B,Tq].
    Returns (idx int32 [B,Tq,k], score f32 [B,Tq,k])."""
    qp = _c(q_pos, np.int32)
    B, Tq = qp.shape
    qb = np.ascontiguousarray(qi).view(np.uint8).reshape(-1)
    kb = np.ascontiguousarray(ki).view(np.uint8).reshape(B, -1)
    ww = _c(w, np.float32)
    qs = _c(qi_scales, np.uint8)
    ks = None if ki_scales is None else np.ascontiguousarray(ki_scales, np.uint8).reshape(B, -1)
    idx = np.empty((B, Tq, k), np.int32)
    sc = np.empty((B, Tq, k), np.float32)
    rc = lib().orc_index_topk(_p(qb), qi_fmt, _p(qs), _p(ww), _p(kb), ki_fmt, _p(ks), kb.shape[1],
                              0 if ks is None else ks.shape[1], _p(qp), B, Tq, H_I, d_I, m, n_cap, k,
                              _p(idx), _p(sc))
    if rc != 0:
        raise ValueError("orc_index_topk rejected its arguments (%d)" % rc)
    return idx, sc


def _attend(kind, q, q_fmt, kv_c, kv_fmt, n_cap, kv_w, kvw_pos0, kvw_rows, q_pos, *, W, H, d, r, scale,
            idx=None, m=1, out_fmt=F32, sink=None):
    qp = _c(q_pos, np.int32)
    B, Tq = qp.shape
    qb = np.ascontiguousarray(q).view(np.uint8).reshape(-1)
    cb = np.ascontiguousarray(kv_c).view(np.uint8).reshape(B, -1)
    wb = np.ascontiguousarray(kv_w).view(np.uint8).reshape(B, -1)
    out = np.zeros((B, Tq, H, d), np.float32 if out_fmt == F32 else np.uint16)
    lse = np.zeros((B, Tq, H), np.float32)
    sk = _c(sink, np.float32)
    if kind == "csa":
        ix = _c(idx, np.int32)
        k = ix.shape[-1]
        rc = lib().orc_csa_attend(_p(qb), q_fmt, _p(cb), kv_fmt, cb.shape[1], n_cap, _p(ix), k, _p(wb), wb.shape[1],
                                  kvw_pos0, kvw_rows, _p(sk), _p(qp), W, B, Tq, H, d, r, scale, _p(out), out_fmt,
                                  _p(lse))
    else:
        rc = lib().orc_hca_attend(_p(qb), q_fmt, _p(cb), kv_fmt, cb.shape[1], n_cap, m, _p(wb), wb.shape[1],
                                  kvw_pos0, kvw_rows, _p(sk), _p(qp), W, B, Tq, H, d, r, scale, _p(out), out_fmt,
                                  _p(lse))
    if rc != 0:
        raise ValueError("oracle attend rejected its arguments (%d)" % rc)
    return out, lse


def csa_attend(q, q_fmt, kv_c, kv_fmt, n_cap, idx, kv_w, kvw_pos0, kvw_rows, q_pos, *, W, H, d, r=0, scale,
               out_fmt=F32, sink=None):
    """q: [B,Tq,H,d] (f32 or bf16 bits); kv_c: [B, N, rowbytes]; idx int32 [B,Tq,k];
    kv_w: [B, kvw_rows, rowbytes]; sink: f32 [H] or None; returns (out [B,Tq,H,d], lse [B,Tq,H])."""
    return _attend("csa", q, q_fmt, kv_c, kv_fmt, n_cap, kv_w, kvw_pos0, kvw_rows, q_pos, W=W, H=H, d=d, r=r,
                   scale=scale, idx=idx, out_fmt=out_fmt, sink=sink)


def hca_attend(q, q_fmt, kv_c, kv_fmt, n_cap, m, kv_w, kvw_pos0, kvw_rows, q_pos, *, W, H, d, r=0, scale,
               out_fmt=F32, sink=None):
    return _attend("hca", q, q_fmt, kv_c, kv_fmt, n_cap, kv_w, kvw_pos0, kvw_rows, q_pos, W=W, H=H, d=d, r=r,
                   scale=scale, m=m, out_fmt=out_fmt, sink=sink)
