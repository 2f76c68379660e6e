"""Single-token decode attention over a paged KV cache on MI355X (gfx950).

The computation lives in ``lib/libpa.so`` (C ABI in ``include/pa.h``; HIP
kernels in ``csrc/``).  :mod:`.binding` exposes the C functions under their
own names; :class:`PagedKVPool` is a small owner of one pool handle that
keeps the tensors it was given alive.  PyTorch is used only for device
memory and streams.
"""

from .binding import (  # noqa: F401
    PA_BLOCK_SIZE,
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
    pa_decode_set_heads_per_workgroup,
    pa_decode_set_workgroups,
    pa_decode_workgroups,
    pa_decode_workspace_bytes,
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
        n, bs, hkv, d = k_cache.shape
        self.kv_dtype = kv_dtype
        self.num_kv_heads, self.head_dim = hkv, d
        self._keep = [k_cache, v_cache, k_scale, v_scale]
        self.handle = pa_kv_pool_create(n, bs, hkv, d, kv_dtype, k_cache, v_cache,
                                        k_scale, v_scale)

    def set_block_table(self, block_table, context_lens, max_context_len):
        """``block_table``: device int32 [B][max_blocks]; ``context_lens``:
        device int32 [B]; ``max_context_len``: host bound of the lengths."""
        b, mb = block_table.shape
        self._tables = [block_table, context_lens]
        self.batch = b
        pa_block_table_set(self.handle, block_table, context_lens, b, mb, max_context_len)

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
        src = {torch.float32: "f32", torch.bfloat16: "bf16"}.get(k_new.dtype, self.kv_dtype)
        pa_cache_append(self.handle, k_new, v_new, src, stream)

    def chunk(self, q, q_start, max_q_len, out, scale=None, stream=None):
        """Attention of several new tokens per sequence: ``q`` [T][Hq][d]
        bf16 (rows of sequence b are q_start[b] .. q_start[b+1]-1, the last
        of its cached positions), ``q_start`` device int32 [B+1],
        ``max_q_len`` host bound of the rows per sequence -> ``out`` float32
        [T][Hq][d]."""
        t, hq = q.shape[0], q.shape[1]
        if scale is None:
            scale = 1.0 / self.head_dim ** 0.5
        pa_chunk_run(self.handle, q, "bf16", hq, q_start, t, max_q_len, scale, out, stream)

    def workspace_bytes(self, num_q_heads):
        return pa_decode_workspace_bytes(self.handle, num_q_heads)

    def decode(self, q, out, workspace, scale=None, stream=None):
        """One decode step: ``q`` [B][Hq][d] (f32 for an f32 pool, else bf16)
        -> ``out`` float32 [B][Hq][d].  ``workspace``: device tensor of at
        least :meth:`workspace_bytes` bytes (256-byte aligned) or None when
        that size is 0.  ``scale`` defaults to 1/sqrt(head_dim)."""
        hq = q.shape[1]
        qd = "f32" if self.kv_dtype == "f32" else "bf16"
        if scale is None:
            scale = 1.0 / self.head_dim ** 0.5
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
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
        n, hkv, _, _ = k_codes.shape
        d = k_params.shape[-1]
        self.head_dim, self.bits = d, bits
        self._keep = [k_codes, v_codes, k_params, v_params]
        self.handle = pa_kv_pool_create_kivi(n, hkv, d, "int8_kivi" if bits == 8 else "int4_kivi",
                                             k_codes, v_codes, k_params, v_params)

    def set_block_table(self, block_table, context_lens, max_context_len):
        b, mb = block_table.shape
        self._tables = [block_table, context_lens]
        pa_block_table_set(self.handle, block_table, context_lens, b, mb, max_context_len)

    def set_residual(self, res_k, res_v):
        """bf16 [B][16][Hkv][d]: each sequence's partly filled last block."""
        self._res = [res_k, res_v]
        pa_kivi_residual_set(self.handle, res_k, res_v)

    def append(self, k_new, v_new, stream=None):
        pa_cache_append(self.handle, k_new, v_new, "bf16", stream)

    def decode(self, q, out, scale=None, stream=None):
        if scale is None:
            scale = 1.0 / self.head_dim ** 0.5
        pa_decode_kivi_run(self.handle, q, "bf16", q.shape[1], scale, out, stream)

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
