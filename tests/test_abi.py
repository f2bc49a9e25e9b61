"""CPU checks of the C ABI: libcsl.so loads, exports every symbol include/csl.h
declares, and rejects bad arguments on the host before touching a device."""
import ctypes as C
import os
import re

import pytest

from compressed_sparse_long_02_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "csl.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def test_header_symbols_are_exported():
    L = C.CDLL(_lib.LIB_PATH)
    names = _declared()
    assert {"kv_compress", "index_topk", "csa_attend", "hca_attend"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert sorted(names) == sorted(_lib.EXPORTS)


def test_helpers():
    L = _lib.lib()
    assert L.csl_row_bytes(2, 512, 64) == 576
    assert L.csl_row_bytes(3, 128, 0) == 64
    assert L.csl_row_bytes(9, 128, 0) == -1
    assert L.csl_status_string(-3) == b"workspace missing or too small"
    assert L.csl_version() >= 100
    # workspace planning: multi-slice candidate lists for a 1M-context CSA decode
    assert L.csl_index_topk_workspace(16, 1, 262144, 1024) > 0
    assert L.csl_index_topk_workspace(1, 1, 200, 64) == 0           # single slice
    assert L.csl_attend_workspace(4096, 2, 128, 512, 1152) == 0     # enough queries: no splits


def _compress(**over):
    a = dict(x=16, x_fmt=1, x_roles=1, x_bstride=0, x_pos0=0, n_tok=8, z=16, z_ch=1, z_bstride=0, bias=16, B=1, d=512, r=64,
             m=4, overlap=1, e_begin=0, n_e=1, out=16, out_fmt=2, out_scales=None, out_bstride=0, sc_bstride=0,
             stream=None)
    a.update(over)
    return _lib.lib().kv_compress(*a.values())


def test_compress_rejects_bad_arguments_on_the_host():
    assert _compress(d=100) == _lib.CSL_EUNSUPPORTED
    assert _compress(m=0) == _lib.CSL_EINVAL
    assert _compress(z_ch=3) == _lib.CSL_EINVAL
    assert _compress(x=None) == _lib.CSL_EINVAL
    assert _compress(x=8) == _lib.CSL_EINVAL                        # misaligned
    assert _compress(n_tok=3) == _lib.CSL_EINVAL                    # window not resident
    assert _compress(out_fmt=3) == _lib.CSL_EINVAL                  # MXFP4 without scales
    assert _compress(r=4) == _lib.CSL_EINVAL                        # packed needs r % 8 == 0
    assert _compress(x_roles=3) == _lib.CSL_EINVAL
    assert _compress(x_roles=2, overlap=0) == _lib.CSL_EINVAL       # two roles need overlapping windows
    assert _compress(n_e=0) == _lib.CSL_OK                          # nothing to do, no device needed
    assert "window" in _lib.last_error() or _lib.last_error() == ""


def _attend(fn="hca", **over):
    a = dict(q=16, q_fmt=1, kv_c=16, kv_fmt=2, kvc_bstride=0, n_cap=10, m=4, kv_w=16, kvw_bstride=0, kvw_pos0=0,
             kvw_rows=10, sink=None, q_pos=16, W=4, B=1, Tq=1, H=64, d=512, r=64, scale=0.1, out=16, out_fmt=0, out_lse=None,
             ws=None, ws_bytes=0, stream=None)
    a.update(over)
    return _lib.lib().hca_attend(*a.values())


def test_attend_rejects_bad_arguments_on_the_host():
    assert _attend(d=100) == _lib.CSL_EUNSUPPORTED
    assert _attend(q_fmt=0) == _lib.CSL_EUNSUPPORTED                # f32 q with packed KV
    assert _attend(r=4) == _lib.CSL_EINVAL
    assert _attend(W=4, kv_w=None) == _lib.CSL_EINVAL
    assert _attend(W=16, kvw_rows=10) == _lib.CSL_EINVAL              # ring shorter than the window
    assert "below the window" in _lib.last_error()
    assert _attend(m=0) == _lib.CSL_EINVAL
    assert _attend(out=None) == _lib.CSL_EINVAL
    assert _attend(kvc_bstride=8) == _lib.CSL_EINVAL
    assert _attend(ws=None, n_cap=10000) == _lib.CSL_EWORKSPACE     # one query: split partials needed
    assert "workspace" in _lib.last_error()
    assert _attend(B=0) == _lib.CSL_OK
    assert _attend(sink=18) == _lib.CSL_EINVAL                      # misaligned sink


def test_paged_attend_rejects_bad_tables_on_the_host():
    L = _lib.lib()

    def call(**over):
        a = dict(q=16, q_fmt=1, pool=16, kv_fmt=2, bt=16, bt_stride=8, epb=32, block_bytes=32 * 576, n_blocks=100,
                 n_cap=256, m=128, kv_w=16, kvw_bstride=0, kvw_pos0=0, kvw_rows=128, sink=None, q_pos=16, W=128,
                 B=1, Tq=1, H=64, d=512, r=64, scale=0.1, out=16, out_fmt=0, out_lse=None, ws=16, ws_bytes=1 << 30,
                 stream=None)
        a.update(over)
        return L.hca_attend_paged(*a.values())

    assert call(bt=None) == _lib.CSL_EINVAL
    assert call(epb=0) == _lib.CSL_EINVAL
    assert call(bt_stride=7) == _lib.CSL_EINVAL                     # 8 blocks of 32 needed for 256 entries
    assert "block-table" in _lib.last_error()
    assert call(block_bytes=32 * 576 - 16) == _lib.CSL_EINVAL       # a block cannot hold its rows
    assert call(n_blocks=0) == _lib.CSL_EINVAL
    assert call(B=0) == _lib.CSL_OK


def test_index_rejects_bad_arguments_on_the_host():
    L = _lib.lib()

    def call(**over):
        a = dict(qi=16, qi_fmt=3, qi_scales=16, w=16, ki=16, ki_fmt=3, ki_scales=16, ki_bstride=0, ks_bstride=0,
                 q_pos=16, B=1, Tq=1, H_I=64, d_I=128, m=4, n_cap=1000, k=1024, out_idx=16, out_score=None,
                 ws=None, ws_bytes=0, stream=None)
        a.update(over)
        return L.index_topk(*a.values())

    assert call(k=0) == _lib.CSL_EUNSUPPORTED
    assert call(k=4096) == _lib.CSL_EUNSUPPORTED
    assert call(d_I=64) == _lib.CSL_EUNSUPPORTED                    # MXFP4 needs d_I = 128
    assert call(qi_fmt=1) == _lib.CSL_EUNSUPPORTED                  # formats must match
    assert call(H_I=200) == _lib.CSL_EUNSUPPORTED
    assert call(qi_scales=None) == _lib.CSL_EINVAL
    assert call(n_cap=(1 << 24) + 1) == _lib.CSL_EUNSUPPORTED       # beyond 1024 slices of 16384
    assert call(Tq=0) == _lib.CSL_OK


def test_valid_call_without_gpu_reports_no_device():
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is visible")
    except Exception:
        pass
    rc = _compress(x=16, n_tok=8)
    assert rc in (_lib.CSL_EDEVICE, _lib.CSL_EUNSUPPORTED)


def test_noalloc_refuses_oversized_calls_on_the_host():
    L = _lib.lib()
    assert L.csl_noalloc_scratch_bytes() == 96 << 20
    # 16 queries x 4M entries would stage ~800 MB: refused before any device work
    rc = L.index_topk_noalloc(16, 3, 16, 16, 16, 3, 16, 0, 0, 16, 16, 1, 64, 128, 4, 1 << 22, 1024, 16, None, None)
    assert rc == _lib.CSL_EWORKSPACE
    assert "scratch" in _lib.last_error()


def test_compress_step_rejects_bad_arguments_on_the_host():
    L = _lib.lib()

    def call(**over):
        a = dict(x=16, x_fmt=1, x_roles=1, x_bstride=0, x_rows=16, z=16, z_ch=1, z_bstride=0, bias=16, pos=16, B=2,
                 T=1, d=512, r=64, m=4, overlap=1, out=16, out_fmt=2, out_scales=None, out_bstride=0, sc_bstride=0,
                 n_cap=100, bt=None, bt_stride=0, epb=0, block_bytes=0, sblk=0, n_blocks=0, stream=None)
        a.update(over)
        return L.kv_compress_step(*a.values())

    assert call(x_rows=7) == _lib.CSL_EINVAL                        # ring shorter than the 8-row window
    assert "ring" in _lib.last_error()
    assert call(x_rows=8, T=2) == _lib.CSL_EINVAL                   # two new tokens need 9 rows
    assert call(pos=None) == _lib.CSL_EINVAL
    assert call(bt=16, bt_stride=4, epb=32, block_bytes=100, n_blocks=10) == _lib.CSL_EINVAL   # block too small
    assert call(T=0) == _lib.CSL_OK


def test_compress_step_pair_rejects_bad_jobs_on_the_host():
    L = _lib.lib()

    def job(**over):
        a = dict(x_ring=16, x_fmt=1, x_roles=1, x_bstride=0, x_rows=16, z_ring=16, z_ch=1, z_bstride=0, bias=16,
                 d=512, r=64, m=4, overlap=1, out=16, out_fmt=2, out_scales=None, n_cap=100)
        a.update(over)
        return _lib.CompressJob(**a)

    def call(j0, j1, pos=16, B=2, T=1):
        return L.kv_compress_step_pair(C.byref(j0), C.byref(j1), pos, B, T, None)

    key = dict(d=128, r=0, out_fmt=3, out_scales=16)
    assert call(job(), job(**key), T=0) == _lib.CSL_OK
    assert call(job(), job(x_rows=7, **key)) == _lib.CSL_EINVAL           # the second job's ring is too short
    assert "kv_compress_step_pair" in _lib.last_error() and "ring" in _lib.last_error()
    assert call(job(out=None), job(**key)) == _lib.CSL_EINVAL             # the first job has no output
    assert call(job(), job(**key), pos=None) == _lib.CSL_EINVAL
    assert call(job(), job(**dict(key, out_scales=None))) == _lib.CSL_EINVAL   # MXFP4 needs its scales
    assert call(job(), job(block_table=16, bt_stride=4, entries_per_block=32, block_bytes=100, n_blocks=10,
                           **key)) == _lib.CSL_EINVAL                      # block too small for 32 keys
    assert L.kv_compress_step_pair(None, C.byref(job()), 16, 2, 1, None) == _lib.CSL_EINVAL


def test_grouped_out_proj_rejects_bad_arguments_on_the_host():
    L = _lib.lib()

    def call(**over):
        a = dict(x=16, x_fmt=1, w=16, w_fmt=1, M=16, G=8, K=4096, R=1024, out=16, out_fmt=0, stream=None)
        a.update(over)
        return L.grouped_out_proj(*a.values())

    assert call(K=4000) == _lib.CSL_EUNSUPPORTED                     # K a multiple of 128
    assert call(R=100) == _lib.CSL_EUNSUPPORTED
    assert call(x_fmt=0) == _lib.CSL_EUNSUPPORTED
    assert call(x=None) == _lib.CSL_EINVAL
    assert call(out_fmt=2) == _lib.CSL_EINVAL
    assert call(M=0) == _lib.CSL_OK


def test_csa_index_step_checks_both_jobs_and_the_index_on_the_host():
    L = _lib.lib()
    job = dict(x_ring=16, x_fmt=1, x_roles=1, x_bstride=0, x_rows=16, z_ring=16, z_ch=1, z_bstride=0, bias=16, d=512,
               r=64, m=4, overlap=1, out=16, out_fmt=2, out_scales=None, out_bstride=0, sc_bstride=0, n_cap=100,
               block_table=None, bt_stride=0, entries_per_block=0, block_bytes=0, scale_block_bytes=0, n_blocks=0)
    key = dict(job, d=128, r=0, out_fmt=3, out_scales=16)

    def call(kv=job, ky=key, **over):
        a = dict(qi=16, qi_fmt=3, qi_scales=16, w=16, ki=16, ki_fmt=3, ki_scales=16, ki_bstride=0, ks_bstride=0,
                 block_table=None, bt_stride=0, entries_per_block=0, block_bytes=0, scale_block_bytes=0, n_blocks=0,
                 q_pos=16, B=1, Tq=1, H_I=64, d_I=128, m=4, n_cap=100, k=64, out_idx=16, out_score=None, ws=None,
                 ws_bytes=0, stream=None)
        a.update(over)
        j0 = _lib.CompressJob(**kv) if kv is not None else None
        j1 = _lib.CompressJob(**ky) if ky is not None else None
        return L.csa_index_step(C.byref(j0) if j0 else None, C.byref(j1) if j1 else None, *a.values())

    assert call(kv=None) == _lib.CSL_EINVAL                          # a job is missing
    assert call(kv=dict(job, x_rows=4)) == _lib.CSL_EINVAL           # the KV window is not in the ring
    assert call(ky=dict(key, out_scales=None)) == _lib.CSL_EINVAL    # MXFP4 key without scales
    assert call(k=0) == _lib.CSL_EUNSUPPORTED                        # the index arguments too
    assert call(qi_fmt=1) == _lib.CSL_EUNSUPPORTED                   # qi and keys in different formats
