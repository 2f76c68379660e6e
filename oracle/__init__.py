"""CPU oracle for paged single-token decode attention.

TEST INFRASTRUCTURE ONLY.  This package is the slow, float64, obviously
correct statement of what the GPU path computes.  It may be imported only by
``tests/``, by ``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of
``bench.py``; the library and its Python binding never import, call or link
anything here, and this package imports nothing from them.

Sources (cited by title and section throughout):

* [d7kj] "KV Cache 深度解析:显存黑洞、PagedAttention 与三路省内存方案"
  (d7kj.com, 2026-08-18).
* [qingdujian] LLM inference-optimization notes (qingdujian.com,
  notes/llm-inference-optimization).
* [freetools] "大模型推理为何这么慢？从内存带宽瓶颈到KV Cache优化的技术突围"
  (answer.freetools.me, 2026-03-06).
* [k1-blog] AI daily note of 2026-07-13 (k1-blog.pages.dev).

Every function here is pinned by ``tests/test_oracle_pins.py`` to something
other than itself (closed forms, a library attention routine, exact
invariances, printed worked values, the FP8 format definition).
"""

from .formats import bf16_bits_to_f64, e4m3fn_to_f64, E4M3FN_TABLE  # noqa: F401
from .decode_attention import (  # noqa: F401
    BLOCK_SIZE,
    gather_sequence_head,
    paged_decode_attention,
)
from .chunk_attention import (  # noqa: F401
    chunk_positions,
    paged_chunk_attention,
    visible_tokens,
)
from .block_manager import BlockManager, OutOfBlocks, block_hash  # noqa: F401
from .kivi import kivi_append, kivi_decode_attention, quantize_block  # noqa: F401
from .kv_size import kv_cache_bytes  # noqa: F401
from .cache_write import (  # noqa: F401
    E4M3FN_MAX,
    append_new_tokens,
    e4m3fn_encode,
    quantize_row,
)
