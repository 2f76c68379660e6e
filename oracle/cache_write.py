"""Writing a decode step's new token into the paged cache, in plain numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where it is stated:

* The decode step appends the new token's key and value to its sequence's
  cache before attending ([d7kj] section 一 and the minimal implementation
  of section 六).  Reading of the pages: ``context_lens[b]`` already counts
  the new token, so it is written at position ``t = context_lens[b] - 1``.
* Its slot is the one the block table gives ([d7kj] section 三;
  [qingdujian] section 二 appends at the next offset of the last block):
  physical block ``table[b][t // 16]``, slot ``t % 16``, one ``[d]`` row per
  KV head, K and V in separate pools.
* FP8 KV ([d7kj] section 四): E4M3 values with a scale per token and head.
  Reading: the scale is ``absmax / 448`` of the (token, head) row (448 is the
  largest finite E4M3FN value), 1 for an all-zero row; each value is
  ``x / scale`` clamped to [-448, 448] and rounded to the nearest E4M3FN
  value, ties to the even code.  The decisions are taken in float32 (the
  arithmetic the GPU uses): absmax, the division by 448 and by the scale
  are single float32 operations, each correctly rounded.

Sequences with ``context_lens[b] == 0`` have no new token and are left
alone; positions whose block id lies outside the pool are not written.
"""

import numpy as np

from .decode_attention import BLOCK_SIZE
from .formats import E4M3FN_TABLE

E4M3FN_MAX = 448.0

# finite non-negative E4M3FN values in code order (codes 0x00..0x7E); they
# increase with the code, so a search over them finds the neighbours
_POS_VALUES = E4M3FN_TABLE[:0x7F]


def e4m3fn_encode(y) -> np.ndarray:
    """Nearest E4M3FN code to each value (ties to the even code).

    ``y`` must lie in [-448, 448] (or be NaN, which gives the NaN code
    0x7F); the sign bit is the value's sign bit (so -0.0 gives 0x80).
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)
    return np.where(np.isnan(y), np.uint8(0x7F), code).astype(np.uint8)


def quantize_row(x) -> tuple:
    """One (token, head) row -> (E4M3FN codes uint8 [d], float32 scale)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x)) if x.size else np.float32(0)
    scale = np.float32(amax) / np.float32(E4M3FN_MAX) if amax > 0 else np.float32(1.0)
    y = np.clip(x / scale, np.float32(-E4M3FN_MAX), np.float32(E4M3FN_MAX))
    return e4m3fn_encode(y), np.float32(scale)


def append_new_tokens(k_pool, v_pool, block_table, context_lens, k_new, v_new,
                      kv_dtype, k_scale=None, v_scale=None):
    """Pools after writing each sequence's new token; the inputs are not changed.

    ``k_pool``/``v_pool``: ``[N][16][Hkv][d]`` in the storage format (float32,
    bf16 bit patterns as uint16, or E4M3FN codes as uint8 with float32 scales
    ``[N][Hkv][16]``).  ``k_new``/``v_new``: ``[B][Hkv][d]``; for float32 and
    bf16 pools in the pool's own format (stored as they are), for an FP8 pool
    as float32 values (bf16 inputs widened exactly beforehand).
    Returns ``(k, v, k_scale, v_scale)`` (scales None unless FP8).
    """
    k, v = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    fp8 = kv_dtype == "fp8_e4m3"
    ks = np.array(k_scale, copy=True) if fp8 else None
    vs = np.array(v_scale, copy=True) if fp8 else None
    n_blocks, _, hkv, _ = k.shape
    for b, n in enumerate(np.asarray(context_lens)):
        if n <= 0:
            continue
        t = int(n) - 1
        phys = int(block_table[b][t // BLOCK_SIZE])
        slot = t % BLOCK_SIZE
        if not 0 <= phys < n_blocks:
            continue
        for g in range(hkv):
            if fp8:
                k[phys, slot, g], ks[phys, g, slot] = quantize_row(k_new[b][g])
                v[phys, slot, g], vs[phys, g, slot] = quantize_row(v_new[b][g])
            else:
                k[phys, slot, g] = k_new[b][g]
                v[phys, slot, g] = v_new[b][g]
    return k, v, ks, vs
