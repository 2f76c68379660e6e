"""Seeded query rows for multi-token (chunk) attention workloads.

A chunk workload is a decode workload's cache (``make_inputs``) plus, per
sequence, the number of new query rows: the last ``n_b`` of its
``context_lens[b]`` cached positions.  The rows are drawn here, standard
normal float32 from ``numpy.random.Generator(PCG64(seed))`` in row order,
stored like the decode queries (float32, or bf16 bit patterns), token-major
``[total_rows][Hq][d]``, with row offsets ``q_start[b]`` (``q_start[B]`` =
total rows).  Nothing here computes attention.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

from .synthetic import NAMED_SPECS, Inputs, _to_bf16_bits, make_inputs


@dataclass
class ChunkInputs:
    base: Inputs           # the cache: pools, scales, table, lengths, scale
    q: np.ndarray          # float32 or uint16 (bf16 bits): [T][Hq][d]
    q_start: np.ndarray    # int32 [B+1]
    q_lens: np.ndarray     # int32 [B]

    @property
    def total_rows(self) -> int:
        return int(self.q_start[-1])

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.q_lens.size else 0


def chunk_queries(base: Inputs, q_lens, seed: int) -> ChunkInputs:
    """Draw the query rows of a chunk workload on top of the cache ``base``."""
    s = base.spec
    q_lens = np.asarray(q_lens, dtype=np.int64)
    if q_lens.shape != (s.batch,):
        raise ValueError("one query length per sequence")
    q_start = np.zeros(s.batch + 1, np.int64)
    np.cumsum(q_lens, out=q_start[1:])
    rng = np.random.Generator(np.random.PCG64(seed))
    qf = rng.standard_normal((int(q_start[-1]), s.num_q_heads, s.head_dim), dtype=np.float32)
    q = qf if s.q_dtype == "f32" else _to_bf16_bits(qf)
    return ChunkInputs(base=base, q=q, q_start=q_start.astype(np.int32),
                       q_lens=q_lens.astype(np.int32))


# Named chunk workloads: (decode workload of the cache, overrides, new rows per
# sequence, seed of the rows).
CHUNK_SPECS = {
    # speculative verification on the Llama-3-8B-shaped step: 4 rows per
    # sequence (3 draft tokens and the last accepted one), bf16 KV
    "spec_verify_b32_ctx4k": ("llama3_8b_b32_ctx4k", {}, 4, 398101),
    # one 2048-token prefill chunk (the default chunk size the pages quote)
    # at the end of a 4096-token prompt, 2 sequences, Llama-3-8B heads
    "prefill_chunk2k_b2_ctx4k": ("llama3_8b_b32_ctx4k",
                                 {"name": "prefill_chunk2k_b2_ctx4k", "batch": 2,
                                  "context_lens": (4096, 4096), "pool_blocks": 512,
                                  "seed": 398102}, 2048, 398103),
}


def make_chunk_inputs(name: str, poison: bool = False) -> ChunkInputs:
    base_name, over, n, seed = CHUNK_SPECS[name]
    base = make_inputs(replace(NAMED_SPECS[base_name], **over), poison=poison)
    return chunk_queries(base, [n] * base.spec.batch, seed)
