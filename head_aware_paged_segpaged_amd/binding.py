"""ctypes binding of libsegpaged.so: the calls of include/segpaged.h under the same names.

Argument marshalling only: host arrays become contiguous int32 buffers, device buffers are
torch tensors whose data pointers are passed through, and the stream defaults to torch's
current stream. Every computation runs in the library's HIP kernels; if the library is missing
the calls raise instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch  # imported before the library so both share one HIP runtime

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsegpaged.so")

SP_OK = 0
SP_ERR_INVALID_ARG = -1
SP_ERR_UNSUPPORTED = -2
SP_ERR_POOL_TOO_SMALL = -3
SP_ERR_WORKSPACE_TOO_SMALL = -4
SP_ERR_HIP = -5
SP_ERR_PLAN_MISMATCH = -6
SP_ERR_SEGMENT_FULL = -7

SP_BF16 = 0
SP_F32 = 1
SP_GLOBAL = 0
SP_LOCAL = 1
SP_LOCAL_ADAPTIVE = 2
SP_RETRIEVAL = 3

EXPORTED = [
    "segpaged_status_string",
    "segpaged_plan_pages",
    "segpaged_plan_pages_layers",
    "segpaged_layout_tables",
    "segpaged_layout_tables_layers",
    "segpaged_build",
    "segpaged_build_layers",
    "segpaged_retrieval_rows",
    "segpaged_build_scored",
    "segpaged_plan_pages_growable",
    "segpaged_layout_tables_growable",
    "segpaged_build_growable",
    "segpaged_append",
    "segpaged_decode_workspace_size",
    "segpaged_decode_plan",
    "segpaged_decode",
    "segpaged_attention_workspace_size",
    "segpaged_attention_plan",
    "segpaged_attention",
    "segpaged_attention_profiled",
    "segpaged_attention_static",
    "segpaged_attention_check",
    "segpaged_attention_plan_host",
    "segpaged_dense_mask_workspace_size",
    "segpaged_dense_mask_plan",
    "segpaged_dense_mask_attention",
]


class SegPagedError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s" % (where, status_string(status)))


_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_f = ctypes.c_float

_SIGS = {
    "segpaged_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "segpaged_plan_pages": (_i32, [_i32, _vp, _vp, _i32, _vp, _i32, ctypes.POINTER(_i64)]),
    "segpaged_layout_tables": (_i32, [_i32, _vp, _vp, _i32, _vp, _i32, _vp, _vp]),
    "segpaged_plan_pages_layers": (_i32, [_i32, _i32, _vp, _vp, _i32, _vp, _i32,
                                          ctypes.POINTER(_i64)]),
    "segpaged_layout_tables_layers": (_i32, [_i32, _i32, _vp, _vp, _i32, _vp, _i32, _vp, _vp]),
    "segpaged_build_layers": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "segpaged_build": (_i32, [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                              _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "segpaged_retrieval_rows": (_i32, [_i32, _vp, _vp, _i32, _vp, ctypes.POINTER(_i64)]),
    "segpaged_build_scored": (_i32, [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "segpaged_plan_pages_growable": (_i32, [_i32, _vp, _vp, _vp, _i32, _vp, _i32,
                                            ctypes.POINTER(_i64)]),
    "segpaged_layout_tables_growable": (_i32, [_i32, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _vp]),
    "segpaged_build_growable": (_i32, [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "segpaged_append": (_i32, [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                               _vp, _vp, _vp, _i64, _vp, _vp]),
    "segpaged_decode_workspace_size": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                              ctypes.POINTER(_sz)]),
    "segpaged_decode_plan": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _sz,
                                    _vp]),
    "segpaged_decode": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i64,
                               _vp, _vp, _vp, _f, _vp, _vp, _sz, _vp]),
    "segpaged_attention_workspace_size": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                                 _vp, ctypes.POINTER(_sz)]),
    "segpaged_attention_plan": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                       _sz, _vp]),
    "segpaged_attention": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _i64, _vp, _vp, _vp, _f, _vp, _vp, _sz, _vp]),
    "segpaged_attention_profiled": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                           _vp, _vp, _vp, _i64, _vp, _vp, _vp, _f, _vp, _vp,
                                           _sz, _vp, _vp, _vp]),
    "segpaged_attention_static": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                         _vp, _vp, _vp, _i64, _vp, _vp, _vp, _f, _vp, _vp,
                                         _vp]),
    "segpaged_attention_check": (_i32, [_vp, _sz, _vp]),
    "segpaged_attention_plan_host": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                            _vp, _i32, _i32, _vp, _sz, ctypes.POINTER(_sz),
                                            ctypes.POINTER(_sz)]),
    "segpaged_dense_mask_workspace_size": (_i32, [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                                  ctypes.POINTER(_sz)]),
    "segpaged_dense_mask_plan": (_i32, [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz,
                                        _vp]),
    "segpaged_dense_mask_attention": (_i32, [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                             _vp, _vp, _f, _vp, _vp, _sz, _vp]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libsegpaged.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libsegpaged.so is not built (%s); run __graft_entry__.build()"
                               % LIB_PATH)
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().segpaged_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != SP_OK:
        raise SegPagedError(status, where)


def _dtype_code(dtype) -> int:
    if dtype in (SP_BF16, "bf16", torch.bfloat16):
        return SP_BF16
    if dtype in (SP_F32, "f32", torch.float32):
        return SP_F32
    raise ValueError("unsupported dtype %r" % (dtype,))


def _host_i32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_vp) if a.size else None


def _dev(t, name: str):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous device tensor" % name)
    return _vp(t.data_ptr())


def _stream(stream):
    if stream is None:
        return _vp(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return _vp(stream.cuda_stream)
    return _vp(int(stream))


def segpaged_plan_pages(ctx_len, q_len, policy, page_size: int) -> int:
    c, q, p = _host_i32(ctx_len), _host_i32(q_len), _host_i32(policy).reshape(-1, 3)
    out = _i64(0)
    _check(lib().segpaged_plan_pages(len(c), _ptr(c), _ptr(q), p.shape[0], _ptr(p), page_size,
                                     ctypes.byref(out)), "segpaged_plan_pages")
    return int(out.value)


def segpaged_layout_tables(ctx_len, q_len, policy, page_size: int):
    c, q, p = _host_i32(ctx_len), _host_i32(q_len), _host_i32(policy).reshape(-1, 3)
    B, Hkv = len(c), p.shape[0]
    seg = np.zeros((B, Hkv, 2, 4), dtype=np.int32)
    kvl = np.zeros((B, Hkv), dtype=np.int32)
    _check(lib().segpaged_layout_tables(B, _ptr(c), _ptr(q), Hkv, _ptr(p), page_size,
                                        seg.ctypes.data_as(_vp), kvl.ctypes.data_as(_vp)),
           "segpaged_layout_tables")
    return seg, kvl


def segpaged_build(dtype, D: int, page_size: int, ctx_len, q_len, policy, k_dense, v_dense,
                   free_pages, n_phys: int, k_pool, v_pool, seg_table, kv_len, v2p,
                   stream=None) -> None:
    c, q, p = _host_i32(ctx_len), _host_i32(q_len), _host_i32(policy).reshape(-1, 3)
    fl = _host_i32(free_pages)
    _check(lib().segpaged_build(_dtype_code(dtype), len(c), p.shape[0], D, page_size, _ptr(c),
                                _ptr(q), _ptr(p), _dev(k_dense, "k_dense"),
                                _dev(v_dense, "v_dense"), _ptr(fl), fl.size, n_phys,
                                _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                _dev(seg_table, "seg_table"), _dev(kv_len, "kv_len"),
                                _dev(v2p, "v2p"), _stream(stream)), "segpaged_build")


def _layers_policy(policy):
    """[n_layers][Hkv][3] int32 host policies."""
    p = _host_i32(policy)
    if p.ndim != 3 or p.shape[2] != 3:
        raise ValueError("policy must be [n_layers][Hkv][3]")
    return p


def segpaged_plan_pages_layers(ctx_len, q_len, policy, page_size: int) -> int:
    c, q, p = _host_i32(ctx_len), _host_i32(q_len), _layers_policy(policy)
    out = _i64(0)
    _check(lib().segpaged_plan_pages_layers(p.shape[0], len(c), _ptr(c), _ptr(q), p.shape[1],
                                            _ptr(p), page_size, ctypes.byref(out)),
           "segpaged_plan_pages_layers")
    return int(out.value)


def segpaged_layout_tables_layers(ctx_len, q_len, policy, page_size: int):
    c, q, p = _host_i32(ctx_len), _host_i32(q_len), _layers_policy(policy)
    n_layers, B, Hkv = p.shape[0], len(c), p.shape[1]
    seg = np.zeros((n_layers, B, Hkv, 2, 4), dtype=np.int32)
    kvl = np.zeros((n_layers, B, Hkv), dtype=np.int32)
    _check(lib().segpaged_layout_tables_layers(n_layers, B, _ptr(c), _ptr(q), Hkv, _ptr(p),
                                               page_size, seg.ctypes.data_as(_vp),
                                               kvl.ctypes.data_as(_vp)),
           "segpaged_layout_tables_layers")
    return seg, kvl


def segpaged_build_layers(dtype, D: int, page_size: int, ctx_len, q_len, policy, k_dense,
                          v_dense, free_pages, n_phys: int, k_pool, v_pool, seg_table, kv_len,
                          v2p, stream=None) -> None:
    c, q, p = _host_i32(ctx_len), _host_i32(q_len), _layers_policy(policy)
    fl = _host_i32(free_pages)
    _check(lib().segpaged_build_layers(_dtype_code(dtype), p.shape[0], len(c), p.shape[1], D,
                                       page_size, _ptr(c), _ptr(q), _ptr(p),
                                       _dev(k_dense, "k_dense"), _dev(v_dense, "v_dense"),
                                       _ptr(fl), fl.size, n_phys, _dev(k_pool, "k_pool"),
                                       _dev(v_pool, "v_pool"), _dev(seg_table, "seg_table"),
                                       _dev(kv_len, "kv_len"), _dev(v2p, "v2p"),
                                       _stream(stream)), "segpaged_build_layers")


def segpaged_retrieval_rows(ctx_len, q_len, policy) -> int:
    c, q, p = _host_i32(ctx_len), _host_i32(q_len), _host_i32(policy).reshape(-1, 3)
    out = _i64(0)
    _check(lib().segpaged_retrieval_rows(len(c), _ptr(c), _ptr(q), p.shape[0], _ptr(p),
                                         ctypes.byref(out)), "segpaged_retrieval_rows")
    return int(out.value)


def segpaged_build_scored(dtype, D: int, page_size: int, ctx_len, q_len, policy, importance,
                          k_dense, v_dense, free_pages, n_phys: int, k_pool, v_pool, seg_table,
                          kv_len, v2p, row_pos, stream=None, reserve=None) -> None:
    """importance: device float32 [Hkv][sum(ctx_len)] (head-major); row_pos: device int32 (or None);
    reserve: host [B] (growable layout) or None."""
    c, q, p = _host_i32(ctx_len), _host_i32(q_len), _host_i32(policy).reshape(-1, 3)
    fl = _host_i32(free_pages)
    r = _host_i32(reserve) if reserve is not None else None
    if importance is not None and importance.dtype != torch.float32:
        raise ValueError("importance must be float32")
    _check(lib().segpaged_build_scored(_dtype_code(dtype), len(c), p.shape[0], D, page_size,
                                       _ptr(c), _ptr(q), _ptr(r) if r is not None else None,
                                       _ptr(p), _dev(importance, "importance"),
                                       _dev(k_dense, "k_dense"), _dev(v_dense, "v_dense"),
                                       _ptr(fl), fl.size, n_phys, _dev(k_pool, "k_pool"),
                                       _dev(v_pool, "v_pool"), _dev(seg_table, "seg_table"),
                                       _dev(kv_len, "kv_len"), _dev(v2p, "v2p"),
                                       _dev(row_pos, "row_pos"), _stream(stream)),
           "segpaged_build_scored")


def segpaged_plan_pages_growable(ctx_len, q_len, reserve, policy, page_size: int) -> int:
    c, q, r = _host_i32(ctx_len), _host_i32(q_len), _host_i32(reserve)
    p = _host_i32(policy).reshape(-1, 3)
    out = _i64(0)
    _check(lib().segpaged_plan_pages_growable(len(c), _ptr(c), _ptr(q), _ptr(r), p.shape[0],
                                              _ptr(p), page_size, ctypes.byref(out)),
           "segpaged_plan_pages_growable")
    return int(out.value)


def segpaged_layout_tables_growable(ctx_len, q_len, reserve, policy, page_size: int):
    c, q, r = _host_i32(ctx_len), _host_i32(q_len), _host_i32(reserve)
    p = _host_i32(policy).reshape(-1, 3)
    B, Hkv = len(c), p.shape[0]
    seg = np.zeros((B, Hkv, 2, 4), dtype=np.int32)
    kvl = np.zeros((B, Hkv), dtype=np.int32)
    _check(lib().segpaged_layout_tables_growable(B, _ptr(c), _ptr(q), _ptr(r), Hkv, _ptr(p),
                                                 page_size, seg.ctypes.data_as(_vp),
                                                 kvl.ctypes.data_as(_vp)),
           "segpaged_layout_tables_growable")
    return seg, kvl


def segpaged_build_growable(dtype, D: int, page_size: int, ctx_len, q_len, reserve, policy,
                            k_dense, v_dense, free_pages, n_phys: int, k_pool, v_pool, seg_table,
                            kv_len, v2p, stream=None) -> None:
    c, q, r = _host_i32(ctx_len), _host_i32(q_len), _host_i32(reserve)
    p, fl = _host_i32(policy).reshape(-1, 3), _host_i32(free_pages)
    _check(lib().segpaged_build_growable(_dtype_code(dtype), len(c), p.shape[0], D, page_size,
                                         _ptr(c), _ptr(q), _ptr(r), _ptr(p),
                                         _dev(k_dense, "k_dense"), _dev(v_dense, "v_dense"),
                                         _ptr(fl), fl.size, n_phys, _dev(k_pool, "k_pool"),
                                         _dev(v_pool, "v_pool"), _dev(seg_table, "seg_table"),
                                         _dev(kv_len, "kv_len"), _dev(v2p, "v2p"),
                                         _stream(stream)), "segpaged_build_growable")


def segpaged_append(dtype, D: int, page_size: int, policy, n_new, k_new, v_new, k_pool, v_pool,
                    n_phys: int, seg_table, kv_len, v2p, error, stream=None) -> None:
    """k_new, v_new: device [B][Hkv][D]; n_new: device int32 [B] or None; error: device int32."""
    p = _host_i32(policy).reshape(-1, 3)
    B = int(k_new.shape[0])
    _check(lib().segpaged_append(_dtype_code(dtype), B, p.shape[0], D, page_size, _ptr(p),
                                 _dev(n_new, "n_new"), _dev(k_new, "k_new"),
                                 _dev(v_new, "v_new"), _dev(k_pool, "k_pool"),
                                 _dev(v_pool, "v_pool"), int(n_phys),
                                 _dev(seg_table, "seg_table"), _dev(kv_len, "kv_len"),
                                 _dev(v2p, "v2p"), int(v2p.numel()), _dev(error, "error"),
                                 _stream(stream)), "segpaged_append")


def segpaged_decode_workspace_size(dtype, Hq: int, Hkv: int, D: int, page_size: int, ctx_hint,
                                   policy) -> int:
    c, p = _host_i32(ctx_hint), _host_i32(policy).reshape(-1, 3)
    out = _sz(0)
    _check(lib().segpaged_decode_workspace_size(_dtype_code(dtype), len(c), Hq, Hkv, D,
                                                page_size, _ptr(c), _ptr(p), ctypes.byref(out)),
           "segpaged_decode_workspace_size")
    return int(out.value)


def segpaged_decode_plan(dtype, Hq: int, Hkv: int, D: int, page_size: int, ctx_hint, policy,
                         workspace, stream=None) -> None:
    c, p = _host_i32(ctx_hint), _host_i32(policy).reshape(-1, 3)
    _check(lib().segpaged_decode_plan(_dtype_code(dtype), len(c), Hq, Hkv, D, page_size, _ptr(c),
                                      _ptr(p), _dev(workspace, "workspace"),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(stream)), "segpaged_decode_plan")


def segpaged_decode(dtype, Hq: int, Hkv: int, D: int, page_size: int, policy, q, k_pool, v_pool,
                    n_phys: int, seg_table, kv_len, v2p, scale: float, o, workspace,
                    stream=None) -> None:
    """q, o: device [B][Hq][D] (one decode query per request)."""
    p = _host_i32(policy).reshape(-1, 3)
    _check(lib().segpaged_decode(_dtype_code(dtype), int(q.shape[0]), Hq, Hkv, D, page_size,
                                 _ptr(p), _dev(q, "q"), _dev(k_pool, "k_pool"),
                                 _dev(v_pool, "v_pool"), int(n_phys),
                                 _dev(seg_table, "seg_table"), _dev(kv_len, "kv_len"),
                                 _dev(v2p, "v2p"), float(scale), _dev(o, "o"),
                                 _dev(workspace, "workspace"),
                                 workspace.numel() * workspace.element_size(), _stream(stream)),
           "segpaged_decode")


def segpaged_attention_workspace_size(dtype, Hq: int, Hkv: int, D: int, page_size: int, ctx_len,
                                      q_len, policy) -> int:
    c, q, p = _host_i32(ctx_len), _host_i32(q_len), _host_i32(policy).reshape(-1, 3)
    out = _sz(0)
    _check(lib().segpaged_attention_workspace_size(_dtype_code(dtype), len(c), Hq, Hkv, D,
                                                   page_size, _ptr(c), _ptr(q), _ptr(p),
                                                   ctypes.byref(out)),
           "segpaged_attention_workspace_size")
    return int(out.value)


def segpaged_attention_plan(dtype, Hq: int, Hkv: int, D: int, page_size: int, ctx_len, q_len,
                            policy, workspace, stream=None) -> None:
    c, q, p = _host_i32(ctx_len), _host_i32(q_len), _host_i32(policy).reshape(-1, 3)
    _check(lib().segpaged_attention_plan(_dtype_code(dtype), len(c), Hq, Hkv, D, page_size,
                                         _ptr(c), _ptr(q), _ptr(p), _dev(workspace, "workspace"),
                                         workspace.numel() * workspace.element_size(),
                                         _stream(stream)), "segpaged_attention_plan")


def _attention_args(dtype, Hq, Hkv, D, page_size, ctx_len, q_len, policy, q, k_pool, v_pool,
                    n_phys, seg_table, kv_len, v2p, scale, o, workspace, stream):
    c, ql, p = _host_i32(ctx_len), _host_i32(q_len), _host_i32(policy).reshape(-1, 3)
    keep = (c, ql, p)
    args = [_dtype_code(dtype), len(c), Hq, Hkv, D, page_size, _ptr(c), _ptr(ql), _ptr(p),
            _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), int(n_phys),
            _dev(seg_table, "seg_table"), _dev(kv_len, "kv_len"), _dev(v2p, "v2p"),
            float(scale), _dev(o, "o"), _dev(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream)]
    return keep, args


def segpaged_attention(dtype, Hq: int, Hkv: int, D: int, page_size: int, ctx_len, q_len, policy,
                       q, k_pool, v_pool, n_phys: int, seg_table, kv_len, v2p, scale: float, o,
                       workspace, stream=None) -> None:
    keep, args = _attention_args(dtype, Hq, Hkv, D, page_size, ctx_len, q_len, policy, q, k_pool,
                                 v_pool, n_phys, seg_table, kv_len, v2p, scale, o, workspace,
                                 stream)
    _check(lib().segpaged_attention(*args), "segpaged_attention")
    del keep


def segpaged_attention_profiled(dtype, Hq: int, Hkv: int, D: int, page_size: int, ctx_len, q_len,
                                policy, q, k_pool, v_pool, n_phys: int, seg_table, kv_len, v2p,
                                scale: float, o, workspace, main_begin, main_end,
                                stream=None) -> None:
    keep, args = _attention_args(dtype, Hq, Hkv, D, page_size, ctx_len, q_len, policy, q, k_pool,
                                 v_pool, n_phys, seg_table, kv_len, v2p, scale, o, workspace,
                                 stream)
    args += [_vp(main_begin.handle if main_begin else 0), _vp(main_end.handle if main_end else 0)]
    _check(lib().segpaged_attention_profiled(*args), "segpaged_attention_profiled")
    del keep


def segpaged_attention_static(dtype, Hq: int, Hkv: int, D: int, page_size: int, ctx_len, q_len,
                              policy, q, k_pool, v_pool, n_phys: int, seg_table, kv_len, v2p,
                              scale: float, o, error=None, stream=None) -> None:
    """segpaged_attention on the library's own device workspace (no workspace argument);
    `error` is an optional device int32 tensor that receives the device-side status."""
    c, ql, p = _host_i32(ctx_len), _host_i32(q_len), _host_i32(policy).reshape(-1, 3)
    _check(lib().segpaged_attention_static(
        _dtype_code(dtype), len(c), Hq, Hkv, D, page_size, _ptr(c), _ptr(ql), _ptr(p),
        _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), int(n_phys),
        _dev(seg_table, "seg_table"), _dev(kv_len, "kv_len"), _dev(v2p, "v2p"), float(scale),
        _dev(o, "o"), _dev(error, "error") if error is not None else None, _stream(stream)),
        "segpaged_attention_static")


def segpaged_attention_check(workspace, stream=None) -> int:
    """Returns (and clears) the device-side error word of a workspace."""
    return int(lib().segpaged_attention_check(_dev(workspace, "workspace"),
                                              workspace.numel() * workspace.element_size(),
                                              _stream(stream)))


def segpaged_attention_plan_host(dtype, Hq: int, Hkv: int, D: int, page_size: int, ctx_len,
                                 q_len, policy, slots_prefill: int, slots_decode: int,
                                 dense_mask: bool = False):
    """Host copy of the plan bytes (header + work lists) and the workspace size."""
    c, q, p = _host_i32(ctx_len), _host_i32(q_len), _host_i32(policy).reshape(-1, 3)
    nb, wb = _sz(0), _sz(0)
    args = [_dtype_code(dtype), len(c), Hq, Hkv, D, page_size, int(bool(dense_mask)), _ptr(c),
            _ptr(q), _ptr(p), slots_prefill, slots_decode]
    _check(lib().segpaged_attention_plan_host(*args, None, 0, ctypes.byref(nb),
                                              ctypes.byref(wb)), "segpaged_attention_plan_host")
    buf = np.zeros(nb.value, dtype=np.uint8)
    _check(lib().segpaged_attention_plan_host(*args, buf.ctypes.data_as(_vp), buf.size,
                                              ctypes.byref(nb), ctypes.byref(wb)),
           "segpaged_attention_plan_host")
    return buf, int(wb.value)


def segpaged_dense_mask_workspace_size(dtype, Hq: int, Hkv: int, D: int, ctx_len, q_len,
                                       policy) -> int:
    c, q, p = _host_i32(ctx_len), _host_i32(q_len), _host_i32(policy).reshape(-1, 3)
    out = _sz(0)
    _check(lib().segpaged_dense_mask_workspace_size(_dtype_code(dtype), len(c), Hq, Hkv, D,
                                                    _ptr(c), _ptr(q), _ptr(p), ctypes.byref(out)),
           "segpaged_dense_mask_workspace_size")
    return int(out.value)


def segpaged_dense_mask_plan(dtype, Hq: int, Hkv: int, D: int, ctx_len, q_len, policy,
                             workspace, stream=None) -> None:
    c, q, p = _host_i32(ctx_len), _host_i32(q_len), _host_i32(policy).reshape(-1, 3)
    _check(lib().segpaged_dense_mask_plan(_dtype_code(dtype), len(c), Hq, Hkv, D, _ptr(c),
                                          _ptr(q), _ptr(p), _dev(workspace, "workspace"),
                                          workspace.numel() * workspace.element_size(),
                                          _stream(stream)), "segpaged_dense_mask_plan")


def segpaged_dense_mask_attention(dtype, Hq: int, Hkv: int, D: int, ctx_len, q_len, policy, q,
                                  k_dense, v_dense, scale: float, o, workspace,
                                  stream=None) -> None:
    c, ql, p = _host_i32(ctx_len), _host_i32(q_len), _host_i32(policy).reshape(-1, 3)
    _check(lib().segpaged_dense_mask_attention(_dtype_code(dtype), len(c), Hq, Hkv, D, _ptr(c),
                                               _ptr(ql), _ptr(p), _dev(q, "q"),
                                               _dev(k_dense, "k_dense"), _dev(v_dense, "v_dense"),
                                               float(scale), _dev(o, "o"),
                                               _dev(workspace, "workspace"),
                                               workspace.numel() * workspace.element_size(),
                                               _stream(stream)),
           "segpaged_dense_mask_attention")


class HipEvent:
    """A raw hipEvent_t from the HIP runtime torch already loaded (for timing)."""

    _hip = None

    def __init__(self):
        if HipEvent._hip is None:
            h = ctypes.CDLL("libamdhip64.so.7")
            h.hipEventCreate.argtypes = [ctypes.POINTER(_vp)]
            h.hipEventDestroy.argtypes = [_vp]
            h.hipEventRecord.argtypes = [_vp, _vp]
            h.hipEventSynchronize.argtypes = [_vp]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(_f), _vp, _vp]
            HipEvent._hip = h
        ev = _vp(0)
        if HipEvent._hip.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.handle = ev.value

    def record(self, stream=None) -> None:
        if HipEvent._hip.hipEventRecord(_vp(self.handle), _stream(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def synchronize(self) -> None:
        if HipEvent._hip.hipEventSynchronize(_vp(self.handle)) != 0:
            raise RuntimeError("hipEventSynchronize failed")

    def elapsed_ms(self, end: "HipEvent") -> float:
        out = _f(0)
        if HipEvent._hip.hipEventElapsedTime(ctypes.byref(out), _vp(self.handle),
                                             _vp(end.handle)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def __del__(self):
        try:
            if self.handle and HipEvent._hip is not None:
                HipEvent._hip.hipEventDestroy(_vp(self.handle))
        except Exception:
            pass
