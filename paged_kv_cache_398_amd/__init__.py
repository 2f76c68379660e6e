"""Single-token decode attention over a paged KV cache on MI355X (gfx950).

The computation lives in ``lib/libpa.so`` (C ABI in ``include/pa.h``; HIP
kernels in ``csrc/``).  :mod:`.binding` exposes the C functions under their
own names; :class:`PagedKVPool` is a small owner of one pool handle that
keeps the tensors it was given alive.  PyTorch is used only for device
memory and streams.
"""

from .binding import (  # noqa: F401
    PA_BLOCK_SIZE,
    PA_DECODE_COUNTER_BYTES,
    PA_DTYPE,
    PAError,
    load_library,
    pa_block_table_set,
    pa_block_table_validate,
    pa_bm_add,
    pa_bm_append,
    pa_bm_create,
    pa_bm_destroy,
    pa_bm_fork,
    pa_bm_free,
    pa_bm_stats,
    pa_bm_table,
    pa_cache_append,
    pa_copy_blocks,
    pa_chunk_run,
    pa_chunk_tiles,
    pa_decode_fp8_run,
    pa_decode_heads_per_workgroup,
    pa_decode_kivi_run,
    pa_decode_run,
    pa_decode_run_noalloc,
    pa_decode_set_heads_per_workgroup,
    pa_decode_set_workgroups,
    pa_decode_workgroups,
    pa_decode_workspace_bytes,
    pa_decode_workspace_clear,
    pa_kivi_residual_set,
    pa_kv_pool_create,
    pa_kv_pool_create_kivi,
    pa_kv_pool_destroy,
    pa_kv_pool_placement,
    pa_last_error,
    pa_profile_enable,
    pa_profile_read,
    pa_status_str,
)


def _torch_dtypes(*names):
    import torch  # dtype objects only
    table = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
             "i32": torch.int32, "u8": torch.uint8}
    return tuple(table[n] for n in names)


def check_tensors(*specs):
    """Raise ValueError unless every ``(name, tensor, shape, dtypes)`` names a
    contiguous CUDA tensor of ``shape`` (None entries match any size) with
    one of the torch dtypes ``dtypes``.  Shapes, dtypes and layouts of all
    of them are checked before any device, so the first message names the
    mismatch.  Called before every library call that takes buffers, so that
    a buffer of the wrong size or type never reaches a kernel."""
    for name, t, shape, dtypes in specs:
        if t is None:
            raise ValueError(f"{name} is None")
        if len(t.shape) != len(shape) or any(w is not None and g != w
                                             for g, w in zip(t.shape, shape)):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype not in dtypes:
            raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for name, t, _, _ in specs:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU (cuda) tensor")


def _kv_tensor_dtypes(kv_dtype):
    import torch
    return {"f32": (torch.float32,), "bf16": (torch.bfloat16, torch.int16, torch.uint16),
            "fp8_e4m3": (torch.uint8, torch.float8_e4m3fn, torch.int8)}[kv_dtype]


def allocate_kv_pools(num_blocks, num_kv_heads, head_dim, kv_dtype, device="cuda"):
    """K and V pools ``[num_blocks][16][num_kv_heads][head_dim]`` placed in
    one device buffer as :func:`pa_kv_pool_placement` recommends (V shifted
    by 256 B against K's 2 KiB address classes).  Returns ``(k, v)`` views
    (float32, bfloat16, or uint8 for FP8 codes) that keep the buffer alive;
    the contents are uninitialised."""
    import torch  # device memory only

    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.uint8}[kv_dtype]
    pool_bytes, v_off, total = pa_kv_pool_placement(num_blocks, num_kv_heads, head_dim, kv_dtype)
    buf = torch.empty(total, dtype=torch.uint8, device=device)
    shape = (num_blocks, PA_BLOCK_SIZE, num_kv_heads, head_dim)
    k = buf[:pool_bytes].view(tdt).view(shape)
    v = buf[v_off:v_off + pool_bytes].view(tdt).view(shape)
    return k, v


class PagedKVPool:
    """One physical block pool and the block tables of the current step.

    ``k_cache``/``v_cache``: device tensors ``[num_blocks][16][Hkv][d]`` of
    ``kv_dtype`` ("f32", "bf16" or "fp8_e4m3" -- any torch dtype of that
    width; only the bytes matter); ``k_scale``/``v_scale``: device float32
    ``[num_blocks][Hkv][16]`` for FP8.
    """

    def __init__(self, k_cache, v_cache, kv_dtype, k_scale=None, v_scale=None):
        if kv_dtype not in ("f32", "bf16", "fp8_e4m3"):
            raise ValueError(f"kv_dtype {kv_dtype!r}: f32, bf16 or fp8_e4m3")
        if len(k_cache.shape) != 4:
            raise ValueError(f"k_cache has shape {tuple(k_cache.shape)}, expected "
                             "[num_blocks][16][num_kv_heads][head_dim]")
        n, bs, hkv, d = k_cache.shape
        specs = [("k_cache", k_cache, (n, bs, hkv, d), _kv_tensor_dtypes(kv_dtype)),
                 ("v_cache", v_cache, (n, bs, hkv, d), _kv_tensor_dtypes(kv_dtype))]
        if kv_dtype == "fp8_e4m3":
            specs += [("k_scale", k_scale, (n, hkv, bs), _torch_dtypes("f32")),
                      ("v_scale", v_scale, (n, hkv, bs), _torch_dtypes("f32"))]
        check_tensors(*specs)
        self.kv_dtype = kv_dtype
        self.num_blocks, self.num_kv_heads, self.head_dim = n, hkv, d
        self.batch = None
        self._keep = [k_cache, v_cache, k_scale, v_scale]
        self.handle = pa_kv_pool_create(n, bs, hkv, d, kv_dtype, k_cache, v_cache,
                                        k_scale, v_scale)

    def set_block_table(self, block_table, context_lens, max_context_len):
        """``block_table``: device int32 [B][max_blocks]; ``context_lens``:
        device int32 [B]; ``max_context_len``: host bound of the lengths."""
        self._set_tables(block_table, context_lens, max_context_len)

    def _set_tables(self, block_table, context_lens, max_context_len):
        if len(block_table.shape) != 2:
            raise ValueError(f"block_table has shape {tuple(block_table.shape)}, expected [B][max_blocks]")
        b, mb = block_table.shape
        check_tensors(("block_table", block_table, (b, mb), _torch_dtypes("i32")),
                      ("context_lens", context_lens, (b,), _torch_dtypes("i32")))
        self._tables = [block_table, context_lens]
        pa_block_table_set(self.handle, block_table, context_lens, b, mb, max_context_len)
        self.batch = b

    def set_workgroups(self, count):
        pa_decode_set_workgroups(self.handle, count)

    def workgroups(self):
        return pa_decode_workgroups(self.handle)

    def set_heads_per_workgroup(self, heads):
        pa_decode_set_heads_per_workgroup(self.handle, heads)

    def heads_per_workgroup(self):
        return pa_decode_heads_per_workgroup(self.handle)

    def append(self, k_new, v_new, stream=None):
        """Write each sequence's new token (``k_new``/``v_new`` device
        [B][Hkv][d]) at position context_lens[b] - 1 of the tables set last.
        f32/bf16 pools take rows of their own dtype; an FP8 pool quantises
        float32 or bfloat16 rows."""
        import torch  # only for the dtype of the rows
        self._need_table()
        shape = (self.batch, self.num_kv_heads, self.head_dim)
        allowed = {"f32": (torch.float32,), "bf16": (torch.bfloat16,),
                   "fp8_e4m3": (torch.float32, torch.bfloat16)}[self.kv_dtype]
        if v_new.dtype != k_new.dtype:
            raise ValueError(f"k_new ({k_new.dtype}) and v_new ({v_new.dtype}) dtypes differ")
        check_tensors(("k_new", k_new, shape, allowed), ("v_new", v_new, shape, allowed))
        src = {torch.float32: "f32", torch.bfloat16: "bf16"}[k_new.dtype]
        pa_cache_append(self.handle, k_new, v_new, src, stream)

    def chunk(self, q, q_start, max_q_len, out, scale=None, stream=None):
        """Attention of several new tokens per sequence (bf16 or FP8 pool):
        ``q`` [T][Hq][d] bf16 (rows of sequence b are q_start[b] ..
        q_start[b+1]-1, the last of its cached positions), ``q_start`` device
        int32 [B+1], ``max_q_len`` host bound of the rows per sequence ->
        ``out`` float32 [T'][Hq][d], T' >= T."""
        self._need_table()
        if len(q.shape) != 3:
            raise ValueError(f"q has shape {tuple(q.shape)}, expected [T][Hq][{self.head_dim}]")
        t, hq = q.shape[0], q.shape[1]
        if len(out.shape) == 3 and out.shape[0] < t:  # more rows than q's are never written
            raise ValueError(f"out has {out.shape[0]} rows, q has {t}")
        check_tensors(("q", q, (t, hq, self.head_dim), _torch_dtypes("bf16")),
                      ("q_start", q_start, (self.batch + 1,), _torch_dtypes("i32")),
                      ("out", out, (None, hq, self.head_dim), _torch_dtypes("f32")))
        if scale is None:
            scale = 1.0 / self.head_dim ** 0.5
        pa_chunk_run(self.handle, q, "bf16", hq, q_start, t, max_q_len, scale, out, stream)

    def _need_table(self):
        if self.batch is None:
            raise ValueError("no block table set (set_block_table)")

    def workspace_bytes(self, num_q_heads):
        return pa_decode_workspace_bytes(self.handle, num_q_heads)

    def new_workspace(self, num_q_heads, device="cuda"):
        """A zeroed device workspace for decode runs with the tables set last
        (None when none is needed).  Zero-filled at allocation, it is ready
        for its first run; runs leave its counter region zero."""
        import torch  # device memory only
        n = self.workspace_bytes(num_q_heads)
        return torch.zeros(n, dtype=torch.uint8, device=device) if n else None

    def decode(self, q, out, workspace, scale=None, stream=None):
        """One decode step: ``q`` [B][Hq][d] (f32 for an f32 pool, else bf16)
        -> ``out`` float32 [B][Hq][d].  ``workspace``: device tensor of at
        least :meth:`workspace_bytes` bytes (256-byte aligned, its counter
        region zero: see :meth:`new_workspace`) or None when that size is 0.
        ``scale`` defaults to 1/sqrt(head_dim)."""
        self._need_table()
        if len(q.shape) != 3:
            raise ValueError(f"q has shape {tuple(q.shape)}, expected [B][Hq][{self.head_dim}]")
        hq = q.shape[1]
        qd = "f32" if self.kv_dtype == "f32" else "bf16"
        specs = [("q", q, (self.batch, hq, self.head_dim), _torch_dtypes(qd)),
                 ("out", out, (self.batch, hq, self.head_dim), _torch_dtypes("f32"))]
        if workspace is not None:
            specs.append(("workspace", workspace, (None,), _torch_dtypes("u8")))
        check_tensors(*specs)
        if scale is None:
            scale = 1.0 / self.head_dim ** 0.5
        ws_bytes = 0 if workspace is None else workspace.numel()
        fn = pa_decode_fp8_run if self.kv_dtype == "fp8_e4m3" else pa_decode_run
        fn(self.handle, q, qd, hq, scale, out, workspace, ws_bytes, stream)

    def close(self):
        if getattr(self, "handle", None):
            pa_kv_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class KiviKVPool:
    """An INT8 / INT4 pool quantised the KIVI way (see include/pa.h).

    ``k_codes``/``v_codes``: device uint8 [N][Hkv][16][d * bits / 8];
    ``k_params``: device fp16 [N][Hkv][2][d]; ``v_params``: device fp16
    [N][Hkv][16][2]; ``bits``: 8 or 4."""

    def __init__(self, k_codes, v_codes, k_params, v_params, bits):
        if bits not in (8, 4):
            raise ValueError(f"bits {bits}: 8 or 4")
        if len(k_params.shape) != 4 or len(k_codes.shape) != 4:
            raise ValueError("k_codes [N][Hkv][16][d*bits/8] and k_params [N][Hkv][2][d] expected")
        n, hkv, _, d = k_params.shape
        u8, f16 = _torch_dtypes("u8", "f16")
        check_tensors(("k_codes", k_codes, (n, hkv, 16, d * bits // 8), (u8,)),
                      ("v_codes", v_codes, (n, hkv, 16, d * bits // 8), (u8,)),
                      ("k_params", k_params, (n, hkv, 2, d), (f16,)),
                      ("v_params", v_params, (n, hkv, 16, 2), (f16,)))
        self.num_kv_heads, self.head_dim, self.bits = hkv, d, bits
        self.batch = None
        self._keep = [k_codes, v_codes, k_params, v_params]
        self.handle = pa_kv_pool_create_kivi(n, hkv, d, "int8_kivi" if bits == 8 else "int4_kivi",
                                             k_codes, v_codes, k_params, v_params)

    def set_block_table(self, block_table, context_lens, max_context_len):
        PagedKVPool._set_tables(self, block_table, context_lens, max_context_len)

    def set_residual(self, res_k, res_v):
        """bf16 [B][16][Hkv][d]: each sequence's partly filled last block
        (row b for sequence b of the tables; B at least their batch)."""
        if len(res_k.shape) != 4:
            raise ValueError(f"res_k has shape {tuple(res_k.shape)}, expected [B][16][Hkv][d]")
        shape = (res_k.shape[0], 16, self.num_kv_heads, self.head_dim)
        check_tensors(("res_k", res_k, shape, _torch_dtypes("bf16")),
                      ("res_v", res_v, shape, _torch_dtypes("bf16")))
        self._res = [res_k, res_v]
        pa_kivi_residual_set(self.handle, res_k, res_v)

    def _need_table(self):
        if self.batch is None:
            raise ValueError("no block table set (set_block_table)")
        res = getattr(self, "_res", None)
        if res is None:
            raise ValueError("no residual set (set_residual)")
        if res[0].shape[0] < self.batch:
            raise ValueError(f"the residual has {res[0].shape[0]} rows, the tables {self.batch}")

    def append(self, k_new, v_new, stream=None):
        self._need_table()
        shape = (self.batch, self.num_kv_heads, self.head_dim)
        check_tensors(("k_new", k_new, shape, _torch_dtypes("bf16")),
                      ("v_new", v_new, shape, _torch_dtypes("bf16")))
        pa_cache_append(self.handle, k_new, v_new, "bf16", stream)

    def decode(self, q, out, scale=None, stream=None):
        self._need_table()
        if len(q.shape) != 3:
            raise ValueError(f"q has shape {tuple(q.shape)}, expected [B][Hq][{self.head_dim}]")
        hq = q.shape[1]
        check_tensors(("q", q, (self.batch, hq, self.head_dim), _torch_dtypes("bf16")),
                      ("out", out, (self.batch, hq, self.head_dim), _torch_dtypes("f32")))
        if scale is None:
            scale = 1.0 / self.head_dim ** 0.5
        pa_decode_kivi_run(self.handle, q, "bf16", hq, scale, out, stream)

    def close(self):
        if getattr(self, "handle", None):
            pa_kv_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class BlockManager:
    """Owner of one native block manager (host memory; see include/pa.h)."""

    def __init__(self, num_blocks, prefix_caching=True):
        self.handle = pa_bm_create(num_blocks, prefix_caching)

    def add(self, seq, tokens):
        return pa_bm_add(self.handle, seq, tokens)

    def append(self, seq, token):
        return pa_bm_append(self.handle, seq, token)

    def fork(self, parent, child):
        pa_bm_fork(self.handle, parent, child)

    def free(self, seq):
        pa_bm_free(self.handle, seq)

    def table(self, seqs, max_blocks):
        return pa_bm_table(self.handle, seqs, max_blocks)

    def stats(self):
        return pa_bm_stats(self.handle)

    def close(self):
        if getattr(self, "handle", None):
            pa_bm_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
