"""ctypes loader of libcsl.so, the gfx950 HIP library (declared in include/csl.h).

There is no fallback: if the library is missing or does not load, every call
raises.  Build it with ``python -m compressed_sparse_long_02_amd.build`` (or
``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcsl.so")

CSL_OK, CSL_EINVAL, CSL_EUNSUPPORTED, CSL_EWORKSPACE, CSL_ELAUNCH, CSL_EDEVICE = 0, -1, -2, -3, -4, -5

# every symbol include/csl.h declares
EXPORTS = ["csl_row_bytes", "kv_compress", "kv_compress_step", "kv_compress_step_pair", "index_topk", "index_topk_paged",
           "csa_index_step", "hca_attend_step",
           "csl_index_topk_workspace", "index_topk_noalloc", "csl_noalloc_scratch_bytes", "csa_attend", "hca_attend",
           "csa_attend_paged", "hca_attend_paged", "csl_attend_workspace", "grouped_out_proj", "csl_status_string",
           "csl_last_error", "csl_version"]


class CompressJob(C.Structure):
    """csl_compress_job: one decode-time compression job (kv_compress_step's arguments)."""
    _fields_ = [("x_ring", C.c_void_p), ("x_fmt", C.c_int), ("x_roles", C.c_int), ("x_bstride", C.c_int64),
                ("x_rows", C.c_int64), ("z_ring", C.c_void_p), ("z_ch", C.c_int), ("z_bstride", C.c_int64),
                ("bias", C.c_void_p), ("d", C.c_int), ("r", C.c_int), ("m", C.c_int), ("overlap", C.c_int),
                ("out", C.c_void_p), ("out_fmt", C.c_int), ("out_scales", C.c_void_p), ("out_bstride", C.c_int64),
                ("sc_bstride", C.c_int64), ("n_cap", C.c_int64), ("block_table", C.c_void_p),
                ("bt_stride", C.c_int64), ("entries_per_block", C.c_int), ("block_bytes", C.c_int64),
                ("scale_block_bytes", C.c_int64), ("n_blocks", C.c_int64)]


class CslError(RuntimeError):
    def __init__(self, fn: str, code: int, text: str):
        super().__init__("%s failed (%d): %s" % (fn, code, text))
        self.code = code


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libcsl.so is not built (%s); run compressed_sparse_long_02_amd/build.py" % LIB_PATH)
    L = C.CDLL(LIB_PATH)
    vp, i64, i32, f32, sz = C.c_void_p, C.c_int64, C.c_int, C.c_float, C.c_size_t
    L.csl_row_bytes.restype = i64
    L.csl_row_bytes.argtypes = [i32, i32, i32]
    L.kv_compress.restype = i32
    L.kv_compress.argtypes = [vp, i32, i32, i64, i64, i64, vp, i32, i64, vp, i32, i32, i32, i32, i32, i64, i64,
                              vp, i32, vp, i64, i64, vp]
    L.kv_compress_step.restype = i32
    L.kv_compress_step.argtypes = [vp, i32, i32, i64, i64, vp, i32, i64, vp, vp, i32, i32, i32, i32, i32, i32,
                                   vp, i32, vp, i64, i64, i64, vp, i64, i32, i64, i64, i64, vp]
    L.kv_compress_step_pair.restype = i32
    L.kv_compress_step_pair.argtypes = [C.POINTER(CompressJob), C.POINTER(CompressJob), vp, i32, i32, vp]
    L.index_topk_paged.restype = i32
    L.index_topk_paged.argtypes = [vp, i32, vp, vp, vp, i32, vp, vp, i64, i32, i64, i64, i64, vp, i32, i32, i32,
                                   i32, i32, i64, i32, vp, vp, vp, sz, vp]
    L.csa_index_step.restype = i32
    L.csa_index_step.argtypes = [C.POINTER(CompressJob), C.POINTER(CompressJob), vp, i32, vp, vp, vp, i32, vp, i64,
                                 i64, vp, i64, i32, i64, i64, i64, vp, i32, i32, i32, i32, i32, i64, i32, vp, vp,
                                 vp, sz, vp]
    L.index_topk.restype = i32
    L.index_topk.argtypes = [vp, i32, vp, vp, vp, i32, vp, i64, i64, vp, i32, i32, i32, i32, i32, i64, i32,
                             vp, vp, vp, sz, vp]
    L.index_topk_noalloc.restype = i32
    L.index_topk_noalloc.argtypes = [vp, i32, vp, vp, vp, i32, vp, i64, i64, vp, i32, i32, i32, i32, i32, i64, i32,
                                     vp, vp, vp]
    L.csl_noalloc_scratch_bytes.restype = sz
    L.csl_noalloc_scratch_bytes.argtypes = []
    L.csl_index_topk_workspace.restype = sz
    L.csl_index_topk_workspace.argtypes = [i32, i32, i64, i32]
    L.csa_attend.restype = i32
    L.csa_attend.argtypes = [vp, i32, vp, i32, i64, i64, vp, i32, vp, i64, i64, i64, vp, vp, i32, i32, i32, i32,
                             i32, i32, f32, vp, i32, vp, vp, sz, vp]
    L.hca_attend.restype = i32
    L.hca_attend.argtypes = [vp, i32, vp, i32, i64, i64, i32, vp, i64, i64, i64, vp, vp, i32, i32, i32, i32, i32,
                             i32, f32, vp, i32, vp, vp, sz, vp]
    L.csa_attend_paged.restype = i32
    L.csa_attend_paged.argtypes = [vp, i32, vp, i32, vp, i64, i32, i64, i64, i64, vp, i32, vp, i64, i64, i64, vp,
                                   vp, i32, i32, i32, i32, i32, i32, f32, vp, i32, vp, vp, sz, vp]
    L.hca_attend_paged.restype = i32
    L.hca_attend_paged.argtypes = [vp, i32, vp, i32, vp, i64, i32, i64, i64, i64, i32, vp, i64, i64, i64, vp,
                                   vp, i32, i32, i32, i32, i32, i32, f32, vp, i32, vp, vp, sz, vp]
    L.hca_attend_step.restype = i32
    L.hca_attend_step.argtypes = [C.POINTER(CompressJob), vp, i32, vp, i32, i64, vp, i64, i32, i64, i64, i64, i32,
                                  vp, i64, i64, i64, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp, i32, vp, vp, sz,
                                  vp]
    L.csl_attend_workspace.restype = sz
    L.csl_attend_workspace.argtypes = [i32, i32, i32, i32, i64]
    L.grouped_out_proj.restype = i32
    L.grouped_out_proj.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, vp, i32, vp]
    L.csl_status_string.restype = C.c_char_p
    L.csl_status_string.argtypes = [i32]
    L.csl_last_error.restype = i32
    L.csl_last_error.argtypes = [C.c_char_p, sz]
    L.csl_version.restype = i32
    L.csl_version.argtypes = []
    _lib = L
    return L


def last_error() -> str:
    buf = C.create_string_buffer(1024)
    lib().csl_last_error(buf, 1024)
    return buf.value.decode()


def check(fn: str, rc: int) -> None:
    if rc != CSL_OK:
        raise CslError(fn, rc, last_error() or lib().csl_status_string(rc).decode())
