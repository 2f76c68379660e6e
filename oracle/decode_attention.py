"""Single-token decode attention over a paged KV cache, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where it is stated:

* Decode step with a KV cache -- [d7kj] section 一 (KV Cache 是什么) and
  section 六 (最小实现): the new token's query attends over every cached K/V
  of its sequence, the new token's own K/V included (the minimal
  implementation appends the token's k/v before attending).  So
  ``context_lens[b]`` counts every cached token the query attends to.
* Attention -- [d7kj] section 一: softmax(q K^T / sqrt(d)) V; section 六
  subtracts the maximum score before exponentiating and divides by the sum.
* Paging -- [d7kj] section 三 (PagedAttention): the cache is cut into
  16-token blocks; a per-sequence block table maps logical block j to a
  physical block; logical order is contiguous, physical placement is not.
  Token t therefore sits in physical block ``table[t // 16]`` at slot
  ``t % 16`` (blocks fill in order; [qingdujian] section 二 appends each
  token at the next offset of the last block and opens a new block when it
  is full).  In-block layout ``[slot][kv_head][dim]`` with separate K and V
  pools follows the block tensors of [qingdujian] section 二.
* GQA -- [freetools] section "从架构层面重新设计：GQA与MQA": the H query
  heads are split into groups that each share one K/V head (one group per
  head is MHA, a single group is MQA).  The pages do not say which heads form
  a group; this oracle takes contiguous groups: query head h reads KV head
  ``h // (Hq / Hkv)``.
* FP8 KV -- [d7kj] section 四 (KV Cache 量化): E4M3 values with per-token,
  per-head scales; the stored value is ``decode(code) * scale`` with the
  scale of that (block, kv head, slot).

Readings where the pages are silent: an empty sequence (length 0) yields a
zero output; positions past a sequence's length, unused blocks and table
padding are never read.

This is the plain two-pass definition: no tiling, no online softmax, no
split over the context.  The GPU path's online/split evaluation is an exact
reformulation of it ([k1-blog] section "FlashAttention"; [freetools] section
"FlashAttention：重新思考IO"), so the two must agree to rounding.
"""

from typing import Iterable, Optional, Tuple

import numpy as np

from .formats import bf16_bits_to_f64, e4m3fn_to_f64

BLOCK_SIZE = 16


def token_position(t):
    """(logical block, slot) of token t: blocks fill in order, 16 slots each."""
    return t // BLOCK_SIZE, t % BLOCK_SIZE


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head h: contiguous groups of Hq/Hkv heads."""
    return h // (num_q_heads // num_kv_heads)


def scores(K: np.ndarray, q: np.ndarray, scale: float) -> np.ndarray:
    """Scaled dot products of one query with every cached key ([d7kj] section 一)."""
    return scale * (K @ q)


def softmax(s: np.ndarray) -> np.ndarray:
    """Max-subtracted softmax ([d7kj] section 六)."""
    s = s - s.max()
    w = np.exp(s)
    return w / w.sum()


def _decode(raw: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f64":
        return np.asarray(raw, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if dtype == "fp8_e4m3":
        return e4m3fn_to_f64(raw)
    raise ValueError(f"unknown dtype {dtype!r}")


def gather_sequence_head(k_pool, v_pool, table_row, n: int, kv_head: int, kv_dtype: str,
                         k_scale=None, v_scale=None) -> Tuple[np.ndarray, np.ndarray]:
    """K and V rows of one KV head of one sequence, in logical order, float64.

    Returns two ``[n, d]`` arrays: row t is the cached key/value of token t,
    read from physical block ``table_row[t // 16]``, slot ``t % 16``.
    """
    logical, slot = token_position(np.arange(n))
    phys = np.asarray(table_row, dtype=np.int64)[logical]
    K = _decode(k_pool[phys, slot, kv_head, :], kv_dtype)
    V = _decode(v_pool[phys, slot, kv_head, :], kv_dtype)
    if kv_dtype == "fp8_e4m3":
        K = K * np.asarray(k_scale, dtype=np.float64)[phys, kv_head, slot][:, None]
        V = V * np.asarray(v_scale, dtype=np.float64)[phys, kv_head, slot][:, None]
    return K, V


def paged_decode_attention(q, k_pool, v_pool, block_table, context_lens, scale, *,
                           kv_dtype: str, q_dtype: str, k_scale=None, v_scale=None,
                           seqs: Optional[Iterable[int]] = None) -> np.ndarray:
    """out[b, h] = softmax(scale * q[b, h] . K_b^T) V_b, in float64.

    ``q``: [B][Hq][d] (float32, or uint16 bf16 bits); ``k_pool``/``v_pool``:
    [N][16][Hkv][d] in ``kv_dtype`` ("f32", "bf16", "fp8_e4m3", or "f64" for
    float64 values used as-is); ``k_scale``/``v_scale``: [N][Hkv][16]
    float32 for FP8; ``block_table``: [B][max_blocks] int; ``context_lens``:
    [B]; ``scale``: the softmax scale (1/sqrt(d), as the fp32 value the GPU
    receives).  ``seqs`` restricts the work to some sequences; the rows of the
    other sequences are left as NaN.
    """
    qf = _decode(q, q_dtype)
    B, Hq, d = qf.shape
    Hkv = k_pool.shape[2]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    scale = float(scale)
    out = np.full((B, Hq, d), np.nan, dtype=np.float64)
    for b in (range(B) if seqs is None else seqs):
        n = int(context_lens[b])
        if n <= 0:
            out[b] = 0.0
            continue
        cur = None
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            if g != cur:  # one KV head's rows at a time keeps memory bounded
                K, V = gather_sequence_head(k_pool, v_pool, block_table[b], n, g,
                                            kv_dtype, k_scale, v_scale)
                cur = g
            w = softmax(scores(K, qf[b, h], scale))  # weights over the n cached tokens
            out[b, h] = w @ V
    return out
