"""Seeded synthetic workloads for single-token paged decode attention.

What is drawn, in this order, from ``numpy.random.Generator(PCG64(seed))``:

1. context lengths (only for specs with a length range),
2. a permutation of the physical block pool (which physical block holds
   which logical block of which sequence),
3. outlier channels (only for specs with outliers),
4. q, then the whole K pool, then the whole V pool, each standard normal
   float32 (drawn in chunks of blocks; the chunked stream equals one draw).

Storage formats (the bytes the GPU reads and the oracle decodes):

* ``f32``  -- IEEE binary32.
* ``bf16`` -- top 16 bits of binary32 after round-to-nearest-even
  (``torch.Tensor.to(torch.bfloat16)``), kept as ``uint16`` bit patterns.
* ``fp8_e4m3`` -- OCP E4M3FN codes (``uint8``) plus one fp32 scale per
  (block, kv head, slot).  Scale = absmax over the head dimension / 448
  (1.0 for an all-zero row); codes = round-to-nearest-even of
  ``clamp(x / scale, -448, 448)`` via ``torch.float8_e4m3fn``.

Layouts: K and V pools are ``[num_blocks][16][num_kv_heads][head_dim]``;
FP8 scales are ``[num_blocks][num_kv_heads][16]``; the block table is
``int32[batch][max_blocks]`` padded with -1; context lengths ``int32[batch]``.

The page "KV Cache 深度解析:显存黑洞、PagedAttention 与三路省内存方案"
(d7kj.com), section 三 (PagedAttention), fixes the 16-token block and the
logical-to-physical table; the note "LLM 推理优化" (qingdujian.com),
section 二 (PagedAttention：分页式 KV Cache 管理), gives the in-block
layout ``[block_size, heads, head_dim]`` with K and V stored apart.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np
import torch

BLOCK_SIZE = 16
FP8_MAX = 448.0

_DTYPE_BYTES = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}


@dataclass(frozen=True)
class Spec:
    """Shape and distribution of one decode-attention workload."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: str  # "f32" | "bf16" | "fp8_e4m3"
    q_dtype: str  # "f32" | "bf16"
    seed: int
    context_lens: Optional[Tuple[int, ...]] = None  # fixed lengths, or
    ctx_range: Optional[Tuple[int, int]] = None  # uniform integers, inclusive
    shared_prefix_seqs: int = 0  # first S sequences share a prefix ...
    shared_prefix_tokens: int = 0  # ... of this many tokens (whole blocks)
    outlier_frac: float = 0.0  # fraction of (kv_head, dim) channels ...
    outlier_gain: float = 8.0  # ... multiplied by this gain in K and V
    pool_blocks: Optional[int] = None  # None: exactly the blocks needed
    description: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


@dataclass
class Inputs:
    """One seeded workload in the cache's storage formats (host numpy)."""

    spec: Spec
    q: np.ndarray  # float32 or uint16 (bf16 bits): [B][Hq][d]
    k_pool: np.ndarray  # float32 / uint16 / uint8: [N][16][Hkv][d]
    v_pool: np.ndarray
    k_scale: Optional[np.ndarray]  # float32 [N][Hkv][16] (FP8 only)
    v_scale: Optional[np.ndarray]
    block_table: np.ndarray  # int32 [B][max_blocks], -1 padded
    context_lens: np.ndarray  # int32 [B]
    scale: np.float32  # softmax scale 1/sqrt(d), rounded to fp32
    used_blocks: np.ndarray = field(repr=False, default=None)  # bool [N]

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def logical_tokens(self) -> int:
        """Cached tokens attended, summed over the batch."""
        return int(self.context_lens.astype(np.int64).sum())

    @property
    def unique_tokens(self) -> int:
        """Distinct physical (block, slot) positions attended.

        Shared prefix blocks are counted once.
        """
        s = self.spec
        shared = 0
        if s.shared_prefix_seqs > 1:
            shared = (s.shared_prefix_seqs - 1) * s.shared_prefix_tokens
        return self.logical_tokens - shared


def _blocks_for(n: int) -> int:
    return (n + BLOCK_SIZE - 1) // BLOCK_SIZE


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _to_fp8(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-(token, head) absmax/448 scales and E4M3FN codes.

    ``x``: float32 [n, 16, Hkv, d].  Returns codes uint8 [n, 16, Hkv, d]
    and scales float32 [n, Hkv, 16].
    """
    xt = torch.from_numpy(x)
    amax = xt.abs().amax(dim=-1)  # [n, 16, Hkv]
    sc = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    y = (xt / sc[..., None]).clamp_(-FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, np.ascontiguousarray(sc.numpy().transpose(0, 2, 1))


def _draw_pool(rng, n_blocks, hkv, d, kv_dtype, out_ch, gain, chunk_blocks):
    """Draw one pool (K or V) chunk by chunk and store it in kv_dtype."""
    shape = (n_blocks, BLOCK_SIZE, hkv, d)
    if kv_dtype == "f32":
        data = np.empty(shape, np.float32)
    elif kv_dtype == "bf16":
        data = np.empty(shape, np.uint16)
    else:
        data = np.empty(shape, np.uint8)
    scales = np.empty((n_blocks, hkv, BLOCK_SIZE), np.float32) if kv_dtype == "fp8_e4m3" else None
    for b0 in range(0, n_blocks, chunk_blocks):
        nb = min(chunk_blocks, n_blocks - b0)
        x = rng.standard_normal((nb, BLOCK_SIZE, hkv, d), dtype=np.float32)
        if out_ch is not None and len(out_ch):
            flat = x.reshape(nb, BLOCK_SIZE, hkv * d)
            flat[:, :, out_ch] *= np.float32(gain)
        if kv_dtype == "f32":
            data[b0:b0 + nb] = x
        elif kv_dtype == "bf16":
            data[b0:b0 + nb] = _to_bf16_bits(x)
        else:
            c, s = _to_fp8(x)
            data[b0:b0 + nb] = c
            scales[b0:b0 + nb] = s
    return data, scales


def make_inputs(spec: Spec, poison: bool = False, seed: Optional[int] = None) -> Inputs:
    """Draw the workload ``spec`` (seeded) in the cache's storage formats.

    With ``poison=True`` every position the method must never read gets a
    NaN: the dead slots of each sequence's last block and every physical
    block no table references (FP8: code 0x7F and a NaN scale).
    """
    s = spec
    rng = np.random.Generator(np.random.PCG64(s.seed if seed is None else seed))
    ctx, table, used, n_pool, out_ch, q = _layout_and_queries(s, rng)
    B, hkv, d = s.batch, s.num_kv_heads, s.head_dim

    # 4. values, continued: K pool, V pool
    per_block = BLOCK_SIZE * hkv * d
    chunk = max(1, (1 << 26) // per_block)
    k_pool, k_scale = _draw_pool(rng, n_pool, hkv, d, s.kv_dtype, out_ch, s.outlier_gain, chunk)
    v_pool, v_scale = _draw_pool(rng, n_pool, hkv, d, s.kv_dtype, out_ch, s.outlier_gain, chunk)

    inp = Inputs(
        spec=s, q=q, k_pool=k_pool, v_pool=v_pool, k_scale=k_scale, v_scale=v_scale,
        block_table=table, context_lens=ctx.astype(np.int32),
        scale=np.float32(1.0 / math.sqrt(d)), used_blocks=used,
    )
    if poison:
        _poison(inp)
    return inp


def _layout_and_queries(s: Spec, rng):
    """Steps 1-4 up to the pools: lengths, block table, outlier channels and
    q.  Returns (ctx int64 [B], table int32 [B][max_blocks], used bool [N],
    N, outlier channels or None, q)."""
    if s.num_q_heads % s.num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    B, hkv, d = s.batch, s.num_kv_heads, s.head_dim

    # 1. context lengths
    if s.context_lens is not None:
        ctx = np.asarray(s.context_lens, dtype=np.int64)
        if ctx.shape != (B,):
            raise ValueError("context_lens must have one entry per sequence")
    else:
        lo, hi = s.ctx_range
        S = s.shared_prefix_seqs
        ctx = np.empty(B, np.int64)
        if S:
            ctx[:S] = rng.integers(max(lo, s.shared_prefix_tokens), hi + 1, size=S)
        ctx[S:] = rng.integers(lo, hi + 1, size=B - S)

    # 2. block placement
    if s.shared_prefix_tokens % BLOCK_SIZE:
        raise ValueError("a shared prefix must be whole blocks")
    pre_blocks = s.shared_prefix_tokens // BLOCK_SIZE if s.shared_prefix_seqs else 0
    nb_seq = [_blocks_for(int(n)) for n in ctx]
    private = []
    for b in range(B):
        if b < s.shared_prefix_seqs:
            if ctx[b] < s.shared_prefix_tokens:
                raise ValueError("a prefix-sharing sequence must hold the whole prefix")
            private.append(nb_seq[b] - pre_blocks)
        else:
            private.append(nb_seq[b])
    needed = pre_blocks + sum(private)
    n_pool = needed if s.pool_blocks is None else s.pool_blocks
    if n_pool < needed:
        raise ValueError(f"pool of {n_pool} blocks cannot hold the {needed} needed")
    n_pool = max(n_pool, 1)
    perm = rng.permutation(n_pool).astype(np.int64)
    max_blocks = max(max(nb_seq) if nb_seq else 0, 1)
    table = np.full((B, max_blocks), -1, np.int32)
    cur = pre_blocks
    prefix_ids = perm[:pre_blocks]
    for b in range(B):
        row = []
        if b < s.shared_prefix_seqs:
            row.extend(prefix_ids.tolist())
        row.extend(perm[cur:cur + private[b]].tolist())
        cur += private[b]
        table[b, :len(row)] = row
    used = np.zeros(n_pool, bool)
    used[perm[:needed]] = True

    # 3. outlier channels
    out_ch = None
    if s.outlier_frac > 0:
        n_out = int(round(s.outlier_frac * hkv * d))
        out_ch = np.sort(rng.choice(hkv * d, size=n_out, replace=False))

    # 4. values: q (the pools follow)
    qf = rng.standard_normal((B, s.num_q_heads, d), dtype=np.float32)
    q = qf if s.q_dtype == "f32" else _to_bf16_bits(qf)
    return ctx, table, used, n_pool, out_ch, q


@dataclass
class DeviceWorkload:
    """A workload drawn for timing: lengths, table and q as ``make_inputs``
    draws them (same seed, same order), the pools' values drawn directly in
    GPU memory by torch's generator (standard normal float32, the same
    outlier channels, the same storage casts).  Same shapes, sizes and
    distributions as ``make_inputs``; different pool values."""

    spec: Spec
    q: "torch.Tensor"
    k_pool: "torch.Tensor"
    v_pool: "torch.Tensor"
    k_scale: Optional["torch.Tensor"]
    v_scale: Optional["torch.Tensor"]
    block_table: "torch.Tensor"
    context_lens: "torch.Tensor"
    scale: np.float32
    ctx_host: np.ndarray
    num_blocks: int

    @property
    def max_context_len(self) -> int:
        return int(self.ctx_host.max()) if self.ctx_host.size else 0

    @property
    def logical_tokens(self) -> int:
        return int(self.ctx_host.astype(np.int64).sum())

    @property
    def unique_tokens(self) -> int:
        s = self.spec
        shared = (s.shared_prefix_seqs - 1) * s.shared_prefix_tokens if s.shared_prefix_seqs > 1 else 0
        return self.logical_tokens - shared


def _device_pool(gen, n_blocks, hkv, d, kv_dtype, out_ch, gain, device):
    shape = (n_blocks, BLOCK_SIZE, hkv, d)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.uint8}[kv_dtype]
    data = torch.empty(shape, dtype=tdt, device=device)
    scales = (torch.empty((n_blocks, hkv, BLOCK_SIZE), dtype=torch.float32, device=device)
              if kv_dtype == "fp8_e4m3" else None)
    ch = None if out_ch is None or not len(out_ch) else torch.from_numpy(out_ch).to(device)
    step = max(1, (1 << 26) // (BLOCK_SIZE * hkv * d))
    for b0 in range(0, n_blocks, step):
        nb = min(step, n_blocks - b0)
        x = torch.randn((nb, BLOCK_SIZE, hkv, d), generator=gen, dtype=torch.float32,
                        device=device)
        if ch is not None:
            flat = x.view(nb, BLOCK_SIZE, hkv * d)
            flat[:, :, ch] *= gain
        if kv_dtype == "fp8_e4m3":
            amax = x.abs().amax(dim=-1)
            sc = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
            y = (x / sc[..., None]).clamp_(-FP8_MAX, FP8_MAX)
            data[b0:b0 + nb] = y.to(torch.float8_e4m3fn).view(torch.uint8)
            scales[b0:b0 + nb] = sc.transpose(1, 2)
        else:
            data[b0:b0 + nb] = x.to(tdt)
    return data, scales


def make_device_workload(spec: Spec, device="cuda") -> DeviceWorkload:
    """``spec`` drawn for timing, pools generated on the GPU (seconds instead
    of the minutes numpy takes for multi-GB pools)."""
    s = spec
    rng = np.random.Generator(np.random.PCG64(s.seed))
    ctx, table, used, n_pool, out_ch, q = _layout_and_queries(s, rng)
    gen = torch.Generator(device=device)
    gen.manual_seed(s.seed)
    k, ks = _device_pool(gen, n_pool, s.num_kv_heads, s.head_dim, s.kv_dtype, out_ch,
                         s.outlier_gain, device)
    v, vs = _device_pool(gen, n_pool, s.num_kv_heads, s.head_dim, s.kv_dtype, out_ch,
                         s.outlier_gain, device)
    qt = torch.from_numpy(np.ascontiguousarray(q))
    if q.dtype == np.uint16:
        qt = qt.view(torch.int16).view(torch.bfloat16)
    return DeviceWorkload(
        spec=s, q=qt.to(device), k_pool=k, v_pool=v, k_scale=ks, v_scale=vs,
        block_table=torch.from_numpy(table).to(device),
        context_lens=torch.from_numpy(ctx.astype(np.int32)).to(device),
        scale=np.float32(1.0 / math.sqrt(s.head_dim)), ctx_host=ctx.astype(np.int32),
        num_blocks=n_pool)


def _poison(inp: Inputs) -> None:
    kv = inp.spec.kv_dtype
    nan_val = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "fp8_e4m3": np.uint8(0x7F)}[kv]
    unused = np.flatnonzero(~inp.used_blocks)
    for pool in (inp.k_pool, inp.v_pool):
        pool[unused] = nan_val
    for sc in (inp.k_scale, inp.v_scale):
        if sc is not None:
            sc[unused] = np.nan
    for b, n in enumerate(inp.context_lens.tolist()):
        if n <= 0 or n % BLOCK_SIZE == 0:
            continue
        phys = int(inp.block_table[b, (n - 1) // BLOCK_SIZE])
        dead = slice(n % BLOCK_SIZE, BLOCK_SIZE)
        inp.k_pool[phys, dead] = nan_val
        inp.v_pool[phys, dead] = nan_val
        for sc in (inp.k_scale, inp.v_scale):
            if sc is not None:
                sc[phys, :, dead] = np.nan


# ---------------------------------------------------------------------------
# The five named workloads.  Seeds are 398000 + workload number.

NAMED_SPECS = {
    "tiny_f32": Spec(
        name="tiny_f32", batch=2, num_q_heads=8, num_kv_heads=2, head_dim=64,
        kv_dtype="f32", q_dtype="f32", seed=398001, context_lens=(37, 100),
        pool_blocks=32,
        description="batch 2, 8q/2kv heads (GQA 4:1), d64, ctx {37,100}, "
                    "32-block pool, fp32",
    ),
    "llama3_8b_b32_ctx4k": Spec(
        name="llama3_8b_b32_ctx4k", batch=32, num_q_heads=32, num_kv_heads=8,
        head_dim=128, kv_dtype="bf16", q_dtype="bf16", seed=398002,
        context_lens=(4096,) * 32, pool_blocks=8192,
        description="Llama-3-8B-shaped layer: batch 32, 32q/8kv, d128, ctx 4096, "
                    "8192-block pool, bf16 KV, fp32 accumulate",
    ),
    "continuous_batch_b64": Spec(
        name="continuous_batch_b64", batch=64, num_q_heads=32, num_kv_heads=8,
        head_dim=128, kv_dtype="bf16", q_dtype="bf16", seed=398003,
        ctx_range=(128, 16384), shared_prefix_seqs=16, shared_prefix_tokens=1024,
        outlier_frac=0.01, outlier_gain=8.0,
        description="batch 64, 32q/8kv, d128, ctx U[128,16384], first 16 share a "
                    "1024-token prefix, 1% outlier channels x8, bf16",
    ),
    "long_ctx_b4_128k": Spec(
        name="long_ctx_b4_128k", batch=4, num_q_heads=32, num_kv_heads=8,
        head_dim=128, kv_dtype="bf16", q_dtype="bf16", seed=398004,
        context_lens=(131072,) * 4, pool_blocks=32768,
        description="batch 4, 32q/8kv, d128, ctx 131072, 32768-block pool, bf16",
    ),
    "fp8_mha_b32_ctx8k": Spec(
        name="fp8_mha_b32_ctx8k", batch=32, num_q_heads=32, num_kv_heads=32,
        head_dim=128, kv_dtype="fp8_e4m3", q_dtype="bf16", seed=398005,
        context_lens=(8192,) * 32, pool_blocks=16384,
        description="MHA 7B-shaped: batch 32, 32q/32kv, d128, ctx 8192, FP8 E4M3 "
                    "KV with per-token per-head fp32 scales, bf16 q",
    ),
}


def named_spec(name: str, **overrides) -> Spec:
    return replace(NAMED_SPECS[name], **overrides)


def kv_dtype_bytes(kv_dtype: str) -> int:
    return _DTYPE_BYTES[kv_dtype]
