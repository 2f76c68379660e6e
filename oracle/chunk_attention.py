"""Attention of several new tokens per sequence over a paged KV cache, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where it is stated:

* Several new tokens of one sequence are attended at once in chunked prefill
  ([d7kj] section 五: a long prompt's prefill is cut into chunks that are
  interleaved with decode steps; section 七 quotes a default chunk of 2048
  tokens) and in speculative decoding ([freetools] section "技术演进的未来方向":
  the large model checks a draft model's candidate tokens in one forward
  pass).
* As for a single decode token ([d7kj] section 六 appends the token's k/v
  before it attends), the new tokens' K/V are already in the cache when they
  attend.  A sequence with ``ctx`` cached tokens whose last ``n`` are the new
  ones therefore has query rows at positions ``ctx - n, ..., ctx - 1``.
* Row ``i`` at position ``p`` attends causally: to the cached tokens
  ``0 .. p`` (itself included) and to nothing after it.  This is exactly what
  the minimal implementation of [d7kj] section 六 produces when it feeds the
  prompt one position at a time (each step attends over the cache built so
  far), so a chunk must give the outputs of those steps.
* Everything else (paging, GQA grouping, the softmax, FP8 scales) is the
  single-token definition of ``decode_attention``.

Readings where the pages are silent: query rows are stored token-major,
``q[row][head][dim]``, rows ``q_start[b] .. q_start[b+1]-1`` belonging to
sequence ``b`` in position order; a row whose position would be negative
(more new rows than cached tokens) attends to nothing and yields zeros, like
an empty sequence.
"""

from typing import Iterable, Optional

import numpy as np

from . import decode_attention as da


def chunk_positions(ctx: int, n: int) -> np.ndarray:
    """Sequence positions of the n new rows of a sequence of ctx tokens."""
    return ctx - n + np.arange(n)


def visible_tokens(p: int) -> int:
    """How many cached tokens the query at position p attends to (0 .. p)."""
    return p + 1


def paged_chunk_attention(q, k_pool, v_pool, block_table, context_lens, q_start, scale, *,
                          kv_dtype: str, q_dtype: str, k_scale=None, v_scale=None,
                          seqs: Optional[Iterable[int]] = None) -> np.ndarray:
    """out[r, h] for every query row r of every sequence, float64.

    ``q``: [T][Hq][d] (float32, or uint16 bf16 bits, or "f64" values);
    ``q_start``: [B+1] nondecreasing row offsets (``q_start[0] = 0``,
    ``q_start[B] = T``); pools, scales, table, lengths and ``scale`` as in
    :func:`decode_attention.paged_decode_attention`.  ``seqs`` restricts the
    work to some sequences; rows of the others are left as NaN.
    """
    qf = da._decode(q, q_dtype)
    T, Hq, d = qf.shape
    Hkv = k_pool.shape[2]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    q_start = np.asarray(q_start, dtype=np.int64)
    scale = float(scale)
    out = np.full((T, Hq, d), np.nan, dtype=np.float64)
    for b in (range(len(q_start) - 1) if seqs is None else seqs):
        r0, r1 = int(q_start[b]), int(q_start[b + 1])
        n = r1 - r0
        if n <= 0:
            continue
        ctx = int(context_lens[b])
        pos = chunk_positions(ctx, n)
        cur = None
        for h in range(Hq):
            g = da.kv_head_of(h, Hq, Hkv)
            if g != cur:
                K, V = da.gather_sequence_head(k_pool, v_pool, block_table[b], max(ctx, 0), g,
                                               kv_dtype, k_scale, v_scale)
                cur = g
            for i in range(n):
                m = visible_tokens(int(pos[i]))
                if m <= 0:
                    out[r0 + i, h] = 0.0
                    continue
                w = da.softmax(da.scores(K[:m], qf[r0 + i, h], scale))
                out[r0 + i, h] = w @ V[:m]
    return out
