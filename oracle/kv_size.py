"""KV-cache size closed form.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[d7kj] section 二 (显存账本) gives the KV bytes of a model as the product of
2 (K and V), layers, KV heads, head dimension, sequence length, batch and
bytes per element; [freetools] section "Prefill与Decode" states the same
product per token.  ([k1-blog] section "KV Cache 為什麼是長上下文的真正天花板"
writes "attention heads" for the head factor; with GQA the heads that are
stored are the KV heads, which is what the other two pages and their worked
numbers use.)
"""


def kv_cache_bytes(layers: int, kv_heads: int, head_dim: int, seq_len: int,
                   batch: int, bytes_per_elem: float) -> float:
    """Bytes held (and read once per decode step) by a KV cache."""
    return 2 * layers * kv_heads * head_dim * seq_len * batch * bytes_per_elem
