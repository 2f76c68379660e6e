"""ctypes binding of libpa.so (include/pa.h), argument marshalling only.

Functions carry the C names.  Device buffers may be given as torch tensors
(their ``data_ptr()`` is passed) or as integer addresses; streams as a
``torch.cuda.Stream``, an integer ``hipStream_t`` or None (torch's current
stream).  Every non-OK status raises :class:`PAError`.  There is no fallback:
if the library is not built, loading raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libpa.so")

PA_BLOCK_SIZE = 16
PA_DECODE_COUNTER_BYTES = 262144
PA_DTYPE = {"f32": 0, "bf16": 1, "fp8_e4m3": 2, "int8_kivi": 3, "int4_kivi": 4}

PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE = 0, 1, 2, 3
PA_ERR_UNSUPPORTED, PA_ERR_STATE, PA_ERR_WORKSPACE, PA_ERR_HIP = 4, 5, 6, 7
PA_ERR_NO_BLOCKS, PA_ERR_SEQUENCE = 8, 9

# (name, restype, argtypes) for every exported symbol of include/pa.h
_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_i64, _pi32 = ctypes.c_int64, ctypes.POINTER(ctypes.c_int32)
SIGNATURES = [
    ("pa_kv_pool_create", _i32, [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                 ctypes.POINTER(_vp)]),
    ("pa_kv_pool_destroy", None, [_vp]),
    ("pa_kv_pool_placement", _i32, [_i32, _i32, _i32, _i32, ctypes.POINTER(_sz),
                                    ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
    ("pa_block_table_set", _i32, [_vp, _vp, _vp, _i32, _i32, _i32]),
    ("pa_block_table_validate", _i32, [_vp, _vp]),
    ("pa_cache_append", _i32, [_vp, _vp, _vp, _i32, _vp]),
    ("pa_chunk_run", _i32, [_vp, _vp, _i32, _i32, _vp, _i32, _i32, _f32, _vp, _vp]),
    ("pa_chunk_tiles", _i32, [_vp, _i32, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    ("pa_copy_blocks", _i32, [_vp, _vp, _i32, _vp]),
    ("pa_kv_pool_create_kivi", _i32, [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                      ctypes.POINTER(_vp)]),
    ("pa_kivi_residual_set", _i32, [_vp, _vp, _vp]),
    ("pa_decode_kivi_run", _i32, [_vp, _vp, _i32, _i32, _f32, _vp, _vp]),
    ("pa_bm_create", _i32, [_i32, _i32, ctypes.POINTER(_vp)]),
    ("pa_bm_destroy", None, [_vp]),
    ("pa_bm_add", _i32, [_vp, _i64, _vp, _i32, _pi32]),
    ("pa_bm_append", _i32, [_vp, _i64, _i32, _pi32, _pi32, _pi32]),
    ("pa_bm_fork", _i32, [_vp, _i64, _i64]),
    ("pa_bm_free", _i32, [_vp, _i64]),
    ("pa_bm_table", _i32, [_vp, _vp, _i32, _i32, _vp, _vp]),
    ("pa_bm_stats", _i32, [_vp, _pi32, _pi32, _pi32]),
    ("pa_decode_workspace_bytes", _i32, [_vp, _i32, ctypes.POINTER(_sz)]),
    ("pa_decode_workspace_clear", _i32, [_vp, _sz, _vp]),
    ("pa_decode_run", _i32, [_vp, _vp, _i32, _i32, _f32, _vp, _vp, _sz, _vp]),
    ("pa_decode_fp8_run", _i32, [_vp, _vp, _i32, _i32, _f32, _vp, _vp, _sz, _vp]),
    ("pa_decode_run_noalloc", _i32, [_vp, _vp, _i32, _i32, _f32, _vp, _vp]),
    ("pa_decode_set_workgroups", _i32, [_vp, _i32]),
    ("pa_decode_workgroups", _i32, [_vp, ctypes.POINTER(_i32)]),
    ("pa_decode_set_heads_per_workgroup", _i32, [_vp, _i32]),
    ("pa_decode_heads_per_workgroup", _i32, [_vp, ctypes.POINTER(_i32)]),
    ("pa_profile_enable", _i32, [_vp, _i32]),
    ("pa_profile_read", _i32, [_vp, ctypes.POINTER(_f32), _i32, ctypes.POINTER(_i32)]),
    ("pa_status_str", ctypes.c_char_p, [_i32]),
    ("pa_last_error", ctypes.c_char_p, []),
]


class PAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_name(status)}: {message}")
        self.status = status
        self.message = message


def _name(status: int) -> str:
    return {0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_DTYPE",
            4: "PA_ERR_UNSUPPORTED", 5: "PA_ERR_STATE", 6: "PA_ERR_WORKSPACE",
            7: "PA_ERR_HIP", 8: "PA_ERR_NO_BLOCKS",
            9: "PA_ERR_SEQUENCE"}.get(status, f"status {status}")


_LIB = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libpa.so once; raise if it has not been built."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with "
                           "`python -m paged_kv_cache_398_amd.build`")
    # torch's wheel carries its own HIP runtime (same soname as ROCm's).
    # Loaded first, it is the one libpa.so binds to, so the process has one
    # runtime; loading libpa.so first would bind torch to the system copy,
    # and kernel launches then fail with "no ROCm-capable device".
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(p)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _LIB = lib
    return lib


def _check(status: int) -> None:
    if status != PA_OK:
        raise PAError(status, load_library().pa_last_error().decode())


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _dtype(d) -> int:
    return PA_DTYPE[d] if isinstance(d, str) else int(d)


def pa_kv_pool_create(num_blocks, block_size, num_kv_heads, head_dim, kv_dtype, k_cache,
                      v_cache, k_scale=None, v_scale=None) -> int:
    out = _vp()
    _check(load_library().pa_kv_pool_create(num_blocks, block_size, num_kv_heads, head_dim,
                                            _dtype(kv_dtype), _ptr(k_cache), _ptr(v_cache),
                                            _ptr(k_scale), _ptr(v_scale), ctypes.byref(out)))
    return out.value


def pa_kv_pool_placement(num_blocks, num_kv_heads, head_dim, kv_dtype) -> tuple:
    """(pool_bytes, v_offset, total_bytes) of the recommended one-buffer
    layout of a K and a V pool (include/pa.h)."""
    pb, vo, tb = _sz(), _sz(), _sz()
    _check(load_library().pa_kv_pool_placement(num_blocks, num_kv_heads, head_dim,
                                               _dtype(kv_dtype), ctypes.byref(pb),
                                               ctypes.byref(vo), ctypes.byref(tb)))
    return pb.value, vo.value, tb.value


def pa_kv_pool_destroy(pool: int) -> None:
    load_library().pa_kv_pool_destroy(pool)


def pa_block_table_set(pool, block_table, context_lens, batch, max_blocks_per_seq,
                       max_context_len) -> None:
    _check(load_library().pa_block_table_set(pool, _ptr(block_table), _ptr(context_lens),
                                             batch, max_blocks_per_seq, max_context_len))


def pa_block_table_validate(pool, stream=None) -> None:
    _check(load_library().pa_block_table_validate(pool, _stream(stream)))


def pa_cache_append(pool, k_new, v_new, src_dtype, stream=None) -> None:
    _check(load_library().pa_cache_append(pool, _ptr(k_new), _ptr(v_new), _dtype(src_dtype),
                                          _stream(stream)))


def pa_chunk_run(pool, q, q_dtype, num_q_heads, q_start, total_q, max_q_len, scale, out,
                 stream=None) -> None:
    _check(load_library().pa_chunk_run(pool, _ptr(q), _dtype(q_dtype), num_q_heads,
                                       _ptr(q_start), total_q, max_q_len, float(scale),
                                       _ptr(out), _stream(stream)))


def pa_chunk_tiles(pool, num_q_heads, max_q_len) -> tuple:
    rows, per_head = _i32(), _i32()
    _check(load_library().pa_chunk_tiles(pool, num_q_heads, max_q_len, ctypes.byref(rows),
                                         ctypes.byref(per_head)))
    return rows.value, per_head.value


def pa_kv_pool_create_kivi(num_blocks, num_kv_heads, head_dim, kv_dtype, k_codes, v_codes,
                           k_params, v_params) -> int:
    out = _vp()
    _check(load_library().pa_kv_pool_create_kivi(num_blocks, num_kv_heads, head_dim,
                                                 _dtype(kv_dtype), _ptr(k_codes), _ptr(v_codes),
                                                 _ptr(k_params), _ptr(v_params),
                                                 ctypes.byref(out)))
    return out.value


def pa_kivi_residual_set(pool, res_k, res_v) -> None:
    _check(load_library().pa_kivi_residual_set(pool, _ptr(res_k), _ptr(res_v)))


def pa_decode_kivi_run(pool, q, q_dtype, num_q_heads, scale, out, stream=None) -> None:
    _check(load_library().pa_decode_kivi_run(pool, _ptr(q), _dtype(q_dtype), num_q_heads,
                                             float(scale), _ptr(out), _stream(stream)))


def pa_copy_blocks(pool, pairs, n, stream=None) -> None:
    _check(load_library().pa_copy_blocks(pool, _ptr(pairs), n, _stream(stream)))


def _host_i32(a):
    import numpy as np
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data


def pa_bm_create(num_blocks, prefix_caching) -> int:
    out = _vp()
    _check(load_library().pa_bm_create(num_blocks, int(bool(prefix_caching)), ctypes.byref(out)))
    return out.value


def pa_bm_destroy(bm) -> None:
    load_library().pa_bm_destroy(bm)


def pa_bm_add(bm, seq, tokens) -> int:
    arr, p = _host_i32(tokens)
    cached = _i32()
    _check(load_library().pa_bm_add(bm, seq, p if arr.size else None, arr.size,
                                    ctypes.byref(cached)))
    return cached.value


def pa_bm_append(bm, seq, token) -> list:
    src, dst, n = _i32(), _i32(), _i32()
    _check(load_library().pa_bm_append(bm, seq, token, ctypes.byref(src), ctypes.byref(dst),
                                       ctypes.byref(n)))
    return [(src.value, dst.value)] if n.value else []


def pa_bm_fork(bm, parent, child) -> None:
    _check(load_library().pa_bm_fork(bm, parent, child))


def pa_bm_free(bm, seq) -> None:
    _check(load_library().pa_bm_free(bm, seq))


def pa_bm_table(bm, seqs, max_blocks):
    """-> (int32 [n][max_blocks] numpy table, int32 [n] lengths)."""
    import numpy as np
    ids = np.ascontiguousarray(seqs, dtype=np.int64)
    n = ids.size
    table = np.empty((n, max_blocks), np.int32)
    lens = np.empty(n, np.int32)
    _check(load_library().pa_bm_table(bm, ids.ctypes.data if n else None, n, max_blocks,
                                      table.ctypes.data if n else None,
                                      lens.ctypes.data if n else None))
    return table, lens


def pa_bm_stats(bm) -> tuple:
    f, c, s = _i32(), _i32(), _i32()
    _check(load_library().pa_bm_stats(bm, ctypes.byref(f), ctypes.byref(c), ctypes.byref(s)))
    return f.value, c.value, s.value


def pa_decode_workspace_bytes(pool, num_q_heads) -> int:
    n = _sz()
    _check(load_library().pa_decode_workspace_bytes(pool, num_q_heads, ctypes.byref(n)))
    return n.value


def pa_decode_workspace_clear(workspace, workspace_bytes, stream=None) -> None:
    _check(load_library().pa_decode_workspace_clear(_ptr(workspace), workspace_bytes,
                                                    _stream(stream)))


def pa_decode_run(pool, q, q_dtype, num_q_heads, scale, out, workspace, workspace_bytes,
                  stream=None) -> None:
    _check(load_library().pa_decode_run(pool, _ptr(q), _dtype(q_dtype), num_q_heads,
                                        float(scale), _ptr(out), _ptr(workspace),
                                        workspace_bytes, _stream(stream)))


def pa_decode_fp8_run(pool, q, q_dtype, num_q_heads, scale, out, workspace, workspace_bytes,
                      stream=None) -> None:
    _check(load_library().pa_decode_fp8_run(pool, _ptr(q), _dtype(q_dtype), num_q_heads,
                                            float(scale), _ptr(out), _ptr(workspace),
                                            workspace_bytes, _stream(stream)))


def pa_decode_run_noalloc(pool, q, q_dtype, num_q_heads, scale, out, stream=None) -> None:
    _check(load_library().pa_decode_run_noalloc(pool, _ptr(q), _dtype(q_dtype), num_q_heads,
                                                float(scale), _ptr(out), _stream(stream)))


def pa_decode_set_workgroups(pool, count) -> None:
    _check(load_library().pa_decode_set_workgroups(pool, count))


def pa_decode_workgroups(pool) -> int:
    t = _i32()
    _check(load_library().pa_decode_workgroups(pool, ctypes.byref(t)))
    return t.value


def pa_decode_set_heads_per_workgroup(pool, heads) -> None:
    _check(load_library().pa_decode_set_heads_per_workgroup(pool, heads))


def pa_decode_heads_per_workgroup(pool) -> int:
    t = _i32()
    _check(load_library().pa_decode_heads_per_workgroup(pool, ctypes.byref(t)))
    return t.value


def pa_profile_enable(pool, capacity) -> None:
    _check(load_library().pa_profile_enable(pool, capacity))


def pa_profile_read(pool, capacity) -> list:
    """Kernel durations (ms) of the runs recorded since enabling."""
    kern = (_f32 * max(capacity, 1))()
    n = _i32()
    _check(load_library().pa_profile_read(pool, kern, capacity, ctypes.byref(n)))
    return list(kern[:min(n.value, capacity)])


def pa_status_str(status) -> str:
    return load_library().pa_status_str(status).decode()


def pa_last_error() -> str:
    return load_library().pa_last_error().decode()
