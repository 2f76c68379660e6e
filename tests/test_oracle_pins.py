"""Pins of the float64 CPU oracle to facts other than itself.

Each ``pin_*`` function checks the oracle against something it does not
share code with: a library attention routine (torch's scaled-dot-product
attention in float64) fed from an independently built paged pool, closed
forms (one token, two tokens, zero query, saturated scores), exact
invariances (physical block relabelling, prefix sharing, GQA vs repeated
MHA, shift of all keys, linearity in V), the FP8 E4M3FN and bf16 format
definitions against torch's own casts, and the KV sizes printed on the pages.
``test_planted_mistakes_are_caught`` plants plausible mistakes in the oracle
(on the CPU) and checks that every one of them breaks at least one pin.
"""

import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import decode_attention as da
from workloads import BLOCK_SIZE, Spec, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_cache_sizes.txt")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


class AppendOnlyPool:
    """A paged pool filled the way an engine appends decode tokens.

    Each sequence owns a list of physical blocks.  A token is written at the
    next free slot of the sequence's last block; when that block is full a
    new one is taken from a shuffled free list ("LLM 推理优化" notes,
    section 二).  Unwritten positions hold NaN so that any stray read shows.
    """

    def __init__(self, num_blocks, hkv, d, rng):
        self.k = np.full((num_blocks, BLOCK_SIZE, hkv, d), np.nan)
        self.v = np.full((num_blocks, BLOCK_SIZE, hkv, d), np.nan)
        self.free = [int(x) for x in rng.permutation(num_blocks)]
        self.blocks = {}
        self.fill = {}

    def append(self, seq, k, v):
        blocks = self.blocks.setdefault(seq, [])
        if not blocks or self.fill[seq] == BLOCK_SIZE:
            blocks.append(self.free.pop())
            self.fill[seq] = 0
        blk, off = blocks[-1], self.fill[seq]
        self.k[blk, off] = k
        self.v[blk, off] = v
        self.fill[seq] += 1

    def table(self, nseq):
        width = max([len(self.blocks.get(s, [])) for s in range(nseq)] + [1])
        t = np.full((nseq, width), -1, np.int32)
        for s in range(nseq):
            row = self.blocks.get(s, [])
            t[s, :len(row)] = row
        return t


def _sdpa(qb, K, V, scale):
    """torch scaled-dot-product attention, float64, one sequence.

    qb: [Hq, d]; K, V: [n, Hkv, d] contiguous in token order.
    """
    Hq, Hkv = qb.shape[0], K.shape[1]
    qt = torch.from_numpy(qb)[None, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=Hq != Hkv)
    return o[0, :, 0, :].numpy()


def _oracle(q, k, v, table, ctx, scale, kv="f64", qd="f64", **kw):
    return oracle.paged_decode_attention(q, k, v, table, np.asarray(ctx), scale,
                                         kv_dtype=kv, q_dtype=qd, **kw)


# ---------------------------------------------------------------------------
# pins


def _pin_library_attention(Hq, Hkv, d, lens, seed):
    rng = _rng(seed)
    B = len(lens)
    Ks = [rng.standard_normal((n, Hkv, d)) for n in lens]
    Vs = [rng.standard_normal((n, Hkv, d)) for n in lens]
    q = rng.standard_normal((B, Hq, d))
    nblk = sum((n + 15) // 16 for n in lens) + 3
    pool = AppendOnlyPool(nblk, Hkv, d, rng)
    for t in range(max(lens)):  # interleave the sequences' appends
        for b, n in enumerate(lens):
            if t < n:
                pool.append(b, Ks[b][t], Vs[b][t])
    scale = 1.0 / math.sqrt(d)
    got = _oracle(q, pool.k, pool.v, pool.table(B), lens, scale)
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(got[b] == 0.0)
        else:
            np.testing.assert_allclose(got[b], _sdpa(q[b], Ks[b], Vs[b], scale),
                                       rtol=0, atol=1e-12)


def pin_library_attention_mha():
    _pin_library_attention(4, 4, 16, [1, 15, 16, 17, 50, 0], seed=11)


def pin_library_attention_gqa():
    _pin_library_attention(8, 2, 32, [33, 5, 64, 100], seed=12)


def pin_library_attention_mqa():
    _pin_library_attention(6, 1, 8, [7, 48, 49], seed=13)


def pin_minimal_step_by_step():
    """The growing single-head cache of "KV Cache 深度解析" section 六.

    At every step the token's k/v is appended, then its q attends over the
    whole cache.  Re-stated here with a contiguous cache; the oracle, given
    the same tokens in a paged pool, must give the same output each step.
    """
    rng = _rng(21)
    d, steps = 8, 40
    qs, ks, vs = (rng.standard_normal((steps, d)) for _ in range(3))
    pool = AppendOnlyPool(8, 1, d, rng)
    kc = np.zeros((0, d))
    vc = np.zeros((0, d))
    for i in range(steps):
        kc = np.concatenate([kc, ks[i][None]])
        vc = np.concatenate([vc, vs[i][None]])
        e = np.exp(qs[i] @ kc.T / math.sqrt(d) - (qs[i] @ kc.T / math.sqrt(d)).max())
        want = (e / e.sum()) @ vc
        pool.append(0, ks[i][None], vs[i][None])
        got = _oracle(qs[i][None, None], pool.k, pool.v, pool.table(1), [i + 1],
                      1.0 / math.sqrt(d))
        np.testing.assert_allclose(got[0, 0], want, rtol=0, atol=1e-13)


def _single_seq_pool(K, V, rng, extra=2):
    """Place tokens K, V ([n, Hkv, d]) of one sequence at random blocks."""
    n, hkv, d = K.shape
    pool = AppendOnlyPool((n + 15) // 16 + extra, hkv, d, rng)
    for t in range(n):
        pool.append(0, K[t], V[t])
    return pool


def pin_single_token_is_its_value():
    rng = _rng(31)
    K, V = rng.standard_normal((1, 2, 16)), rng.standard_normal((1, 2, 16))
    q = 50.0 * rng.standard_normal((1, 4, 16))
    pool = _single_seq_pool(K, V, rng)
    got = _oracle(q, pool.k, pool.v, pool.table(1), [1], 0.25)
    assert np.array_equal(got[0, :2], np.broadcast_to(V[0, 0], (2, 16)))
    assert np.array_equal(got[0, 2:], np.broadcast_to(V[0, 1], (2, 16)))


def pin_two_tokens_logistic():
    rng = _rng(32)
    d = 16
    K, V = rng.standard_normal((2, 1, d)), rng.standard_normal((2, 1, d))
    q = rng.standard_normal((1, 1, d))
    scale = 0.3
    pool = _single_seq_pool(K, V, rng)
    got = _oracle(q, pool.k, pool.v, pool.table(1), [2], scale)[0, 0]
    s0, s1 = scale * (q[0, 0] @ K[0, 0]), scale * (q[0, 0] @ K[1, 0])
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    np.testing.assert_allclose(got, w0 * V[0, 0] + (1 - w0) * V[1, 0], rtol=0, atol=1e-14)


def pin_zero_query_is_mean():
    rng = _rng(33)
    n, d = 37, 8
    K, V = rng.standard_normal((n, 1, d)), rng.standard_normal((n, 1, d))
    pool = _single_seq_pool(K, V, rng)
    got = _oracle(np.zeros((1, 2, d)), pool.k, pool.v, pool.table(1), [n], 0.5)[0]
    for h in range(2):
        np.testing.assert_allclose(got[h], V[:, 0].mean(axis=0), rtol=0, atol=1e-14)


def pin_saturated_scores_pick_the_max():
    """Huge scores: the softmax becomes a one-hot on the largest score."""
    rng = _rng(34)
    n, d = 40, 8
    K, V = rng.standard_normal((n, 1, d)), rng.standard_normal((n, 1, d))
    q = rng.standard_normal((1, 1, d))
    sc = K[:, 0] @ q[0, 0]
    assert np.sort(sc)[-1] - np.sort(sc)[-2] > 1e-3
    pool = _single_seq_pool(K, V, rng)
    got = _oracle(q * 1e6, pool.k, pool.v, pool.table(1), [n], 1.0)[0, 0]
    assert np.array_equal(got, V[int(np.argmax(sc)), 0])


def pin_shift_of_all_keys_is_invisible():
    rng = _rng(35)
    n, hkv, d = 50, 2, 16
    K, V = rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hkv, d))
    q = rng.standard_normal((1, 4, d))
    u = rng.standard_normal((1, hkv, d))
    a = _single_seq_pool(K, V, _rng(1))
    b = _single_seq_pool(K + u, V, _rng(1))
    ga = _oracle(q, a.k, a.v, a.table(1), [n], 0.25)
    gb = _oracle(q, b.k, b.v, b.table(1), [n], 0.25)
    np.testing.assert_allclose(gb, ga, rtol=0, atol=1e-12)


def pin_linear_in_values():
    rng = _rng(36)
    n, hkv, d = 45, 2, 16
    K, V1, V2 = (rng.standard_normal((n, hkv, d)) for _ in range(3))
    q = rng.standard_normal((1, 4, d))
    outs = []
    for V in (V1, V2, V1 + 2.0 * V2):
        p = _single_seq_pool(K, V, _rng(2))
        outs.append(_oracle(q, p.k, p.v, p.table(1), [n], 0.25))
    np.testing.assert_allclose(outs[2], outs[0] + 2.0 * outs[1], rtol=0, atol=1e-12)


_SMALL = Spec(name="pin_small", batch=4, num_q_heads=8, num_kv_heads=2, head_dim=32,
              kv_dtype="f32", q_dtype="f32", seed=41, context_lens=(1, 16, 33, 90),
              pool_blocks=20)


def _online_state(qh, K, V, scale, tile):
    """One head's (running max m, running sum l, unnormalised output acc)
    over tokens K, V ([n, d]) taken `tile` at a time: the FlashAttention
    recurrence of the "LLM 推理优化" notes, section 三, with the standard
    log-sum-exp (section 三's printed one is garbled).  Base-e throughout."""
    m, l, acc = -math.inf, 0.0, np.zeros(K.shape[1])
    for t0 in range(0, K.shape[0], tile):
        s = scale * (K[t0:t0 + tile] @ qh)
        m_new = max(m, float(s.max()))
        c = 0.0 if m == -math.inf else math.exp(m - m_new)
        p = np.exp(s - m_new)
        l = c * l + float(p.sum())
        acc = c * acc + p @ V[t0:t0 + tile]
        m = m_new
    return m, l, acc


def _recurrence_case(seed):
    """Four sequences of GQA tokens (Hq 4, Hkv 2, d 16) placed in a paged pool."""
    rng = _rng(seed)
    lens = [1, 7, 37, 100]
    Hq, Hkv, d = 4, 2, 16
    seqs = [(rng.standard_normal((n, Hkv, d)), rng.standard_normal((n, Hkv, d))) for n in lens]
    q = rng.standard_normal((len(lens), Hq, d))
    pool = AppendOnlyPool(sum((n + 15) // 16 for n in lens) + 3, Hkv, d, rng)
    for t in range(max(lens)):
        for b, (K, V) in enumerate(seqs):
            if t < lens[b]:
                pool.append(b, K[t], V[t])
    scale = 1.0 / math.sqrt(d)
    got = _oracle(q, pool.k, pool.v, pool.table(len(lens)), lens, scale)
    return q, seqs, scale, got, Hq // Hkv


def pin_online_recurrence_at_several_tile_sizes():
    """The one-pass recurrence (rescale the partial sums whenever the max
    rises) reaches the two-pass definition: at tiles of 1, 3, 16, 17 and
    whole sequences it matches the oracle to 1e-12."""
    q, seqs, scale, got, G = _recurrence_case(51)
    for b, (K, V) in enumerate(seqs):
        for h in range(q.shape[1]):
            g = h // G
            for tile in (1, 3, 16, 17, K.shape[0]):
                m, l, acc = _online_state(q[b, h], K[:, g], V[:, g], scale, tile)
                np.testing.assert_allclose(acc / l, got[b, h], rtol=0, atol=1e-12)


def pin_split_parts_merge_to_the_whole():
    """A sequence cut into parts (some empty), each reduced to (m, l, acc) on
    its own, then merged with weights exp(m_p - M), M = max m_p (an empty
    part weighs 0): out = sum w_p acc_p / sum w_p l_p -- the combination of
    split sequences -- matches the oracle to 1e-12."""
    q, seqs, scale, got, G = _recurrence_case(52)
    rng = _rng(53)
    for b, (K, V) in enumerate(seqs):
        n = K.shape[0]
        for _ in range(3):
            cuts = sorted(int(x) for x in rng.integers(0, n + 1, size=3))
            bounds = [0] + cuts + [n]
            for h in range(q.shape[1]):
                g = h // G
                parts = [_online_state(q[b, h], K[lo:hi, g], V[lo:hi, g], scale, 5)
                         for lo, hi in zip(bounds[:-1], bounds[1:])]
                M = max(m for m, _, _ in parts)
                w = [0.0 if m == -math.inf else math.exp(m - M) for m, _, _ in parts]
                num = sum(wi * acc for wi, (_, _, acc) in zip(w, parts))
                den = sum(wi * l for wi, (_, l, _) in zip(w, parts))
                np.testing.assert_allclose(num / den, got[b, h], rtol=0, atol=1e-12)


def pin_block_relabelling_is_bit_exact():
    inp = make_inputs(_SMALL)
    base = _oracle(inp.q, inp.k_pool, inp.v_pool, inp.block_table, inp.context_lens,
                   inp.scale, kv="f32", qd="f32")
    pi = _rng(42).permutation(inp.num_blocks)
    k2 = np.empty_like(inp.k_pool)
    v2 = np.empty_like(inp.v_pool)
    k2[pi] = inp.k_pool
    v2[pi] = inp.v_pool
    t2 = np.where(inp.block_table >= 0, pi[np.maximum(inp.block_table, 0)], -1)
    got = _oracle(inp.q, k2, v2, t2, inp.context_lens, inp.scale, kv="f32", qd="f32")
    assert np.array_equal(got, base)


def pin_prefix_sharing_is_bit_exact():
    spec = Spec(name="pin_prefix", batch=5, num_q_heads=4, num_kv_heads=2, head_dim=16,
                kv_dtype="bf16", q_dtype="bf16", seed=43, ctx_range=(40, 120),
                shared_prefix_seqs=3, shared_prefix_tokens=32)
    inp = make_inputs(spec)
    shared = inp.block_table[:3, :2]
    assert (shared == shared[0]).all()
    base = _oracle(inp.q, inp.k_pool, inp.v_pool, inp.block_table, inp.context_lens,
                   inp.scale, kv="bf16", qd="bf16")
    # give sequences 1 and 2 private copies of the prefix blocks
    k, v, t = inp.k_pool, inp.v_pool, inp.block_table.copy()
    for b in (1, 2):
        new = np.arange(k.shape[0], k.shape[0] + 2)
        k = np.concatenate([k, k[t[b, :2]]])
        v = np.concatenate([v, v[t[b, :2]]])
        t[b, :2] = new
    got = _oracle(inp.q, k, v, t, inp.context_lens, inp.scale, kv="bf16", qd="bf16")
    assert np.array_equal(got, base)


def pin_gqa_is_repeated_mha():
    inp = make_inputs(_SMALL)
    G = _SMALL.num_q_heads // _SMALL.num_kv_heads
    gqa = _oracle(inp.q, inp.k_pool, inp.v_pool, inp.block_table, inp.context_lens,
                  inp.scale, kv="f32", qd="f32")
    k = np.repeat(inp.k_pool, G, axis=2)
    v = np.repeat(inp.v_pool, G, axis=2)
    mha = _oracle(inp.q, k, v, inp.block_table, inp.context_lens, inp.scale,
                  kv="f32", qd="f32")
    np.testing.assert_allclose(mha, gqa, rtol=0, atol=1e-15)


_FP8 = Spec(name="pin_fp8", batch=3, num_q_heads=4, num_kv_heads=2, head_dim=32,
            kv_dtype="fp8_e4m3", q_dtype="bf16", seed=44, context_lens=(5, 31, 70),
            pool_blocks=12)


def _dequant_with_torch(codes, sc):
    """codes [N][16][Hkv][d], scales [N][Hkv][16] -> float64 [N][16][Hkv][d]."""
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return vals * sc.astype(np.float64).transpose(0, 2, 1)[..., None]


def pin_fp8_equals_dequantised_values():
    inp = make_inputs(_FP8)
    got = _oracle(inp.q, inp.k_pool, inp.v_pool, inp.block_table, inp.context_lens,
                  inp.scale, kv="fp8_e4m3", qd="bf16", k_scale=inp.k_scale,
                  v_scale=inp.v_scale)
    kd = _dequant_with_torch(inp.k_pool, inp.k_scale)
    vd = _dequant_with_torch(inp.v_pool, inp.v_scale)
    want = _oracle(inp.q, kd, vd, inp.block_table, inp.context_lens, inp.scale,
                   kv="f64", qd="bf16")
    assert np.array_equal(got, want)


def pin_fp8_close_to_unquantised():
    """E4M3 keeps 3 mantissa bits: values move by at most 1/16 relative."""
    spec = _FP8
    q8 = make_inputs(spec)
    f = make_inputs(Spec(**{**spec.__dict__, "kv_dtype": "f32"}))
    a = _oracle(q8.q, q8.k_pool, q8.v_pool, q8.block_table, q8.context_lens, q8.scale,
                kv="fp8_e4m3", qd="bf16", k_scale=q8.k_scale, v_scale=q8.v_scale)
    b = _oracle(f.q, f.k_pool, f.v_pool, f.block_table, f.context_lens, f.scale,
                kv="f32", qd="bf16")
    assert np.abs(a - b).max() < 0.1


def pin_e4m3fn_format():
    vals = oracle.E4M3FN_TABLE
    lib = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    lib = lib.to(torch.float64).numpy()
    nan = np.isnan(vals)
    assert np.array_equal(nan, np.isnan(lib))
    assert np.array_equal(vals[~nan], lib[~nan])
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert vals[0x7E] == 448.0 and np.nanmax(vals) == 448.0
    assert vals[0x01] == 2.0 ** -9 and vals[0x08] == 2.0 ** -6
    assert np.all(np.diff(vals[:0x7F]) > 0)
    assert np.array_equal(vals[0x80:0xFF], -vals[:0x7F])


def pin_bf16_format():
    bits = np.arange(0, 1 << 16, 7, dtype=np.uint32).astype(np.uint16)
    mine = oracle.bf16_bits_to_f64(bits)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], lib[~nan])


def _golden_rows():
    rows = []
    with open(GOLDEN, encoding="utf-8") as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, args, val, unit, tol, src = [c.strip() for c in line.split("|")]
            rows.append((name, [float(x) for x in args.split()], float(val), unit,
                         float(tol), src))
    return rows


_UNIT = {"KB": 2 ** 10, "MB": 2 ** 20, "GB": 2 ** 30}


def pin_kv_sizes_printed_on_the_pages():
    rows = _golden_rows()
    assert len(rows) >= 9
    for name, args, val, unit, tol, _src in rows:
        got = oracle.kv_cache_bytes(*args)
        want = val * _UNIT[unit]
        assert abs(got - want) <= tol * want, (name, got, want)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


def test_gqa_and_mha_sizes():
    """GQA with 32 query / 8 KV heads stores a quarter of MHA's KV.

    "KV Cache 深度解析" section 四 states the factor 4; its per-token MHA
    figure of 8 KB disagrees with that factor and with the page's own
    closed form (16 KiB for 32 KV heads x 128 x 2 B x 2), which is what
    section 七's 16 GB -> 64 GB also implies.  The closed form governs.
    """
    mha = oracle.kv_cache_bytes(1, 32, 128, 1, 1, 2)
    gqa = oracle.kv_cache_bytes(1, 8, 128, 1, 1, 2)
    assert mha == 16384 and mha / gqa == 4


def test_cpu_offload_time():
    """"KV Cache 深度解析" section 七: 512 MB per token over ~32 GB/s is ~16 ms."""
    per_step = oracle.kv_cache_bytes(32, 8, 128, 4096, 1, 2)
    for link in (32 * 2 ** 30, 32e9):
        assert abs(per_step / link - 0.016) / 0.016 < 0.06


# ---------------------------------------------------------------------------
# planted mistakes: each must break at least one pin


def _gather_v_from_k(k_pool, v_pool, table_row, n, kv_head, kv_dtype, k_scale=None,
                     v_scale=None):
    K, _ = _REAL_GATHER(k_pool, v_pool, table_row, n, kv_head, kv_dtype, k_scale, v_scale)
    return K, K


def _gather_drops_newest(k_pool, v_pool, table_row, n, kv_head, kv_dtype, k_scale=None,
                         v_scale=None):
    K, V = _REAL_GATHER(k_pool, v_pool, table_row, max(n - 1, 1), kv_head, kv_dtype,
                        k_scale, v_scale)
    return K, V


def _gather_v_unscaled(k_pool, v_pool, table_row, n, kv_head, kv_dtype, k_scale=None,
                       v_scale=None):
    K, V = _REAL_GATHER(k_pool, v_pool, table_row, n, kv_head, kv_dtype, k_scale, None
                        if kv_dtype != "fp8_e4m3" else np.ones_like(v_scale))
    return K, V


_REAL_GATHER = da.gather_sequence_head

MUTANTS = {
    "slot_and_block_swapped": ("token_position", lambda t: (t % 16, t // 16)),
    "blocks_of_8": ("token_position", lambda t: (t // 8, t % 8)),
    "interleaved_groups": ("kv_head_of", lambda h, hq, hkv: h % hkv),
    "unscaled_scores": ("scores", lambda K, q, scale: K @ q),
    "sqrt_scale": ("scores", lambda K, q, scale: math.sqrt(scale) * (K @ q)),
    "no_normalisation": ("softmax", lambda s: np.exp(s - s.max())),
    "no_max_subtraction": ("softmax", lambda s: np.exp(s) / np.exp(s).sum()),
    "values_read_from_keys": ("gather_sequence_head", _gather_v_from_k),
    "newest_token_dropped": ("gather_sequence_head", _gather_drops_newest),
    "fp8_value_scale_ignored": ("gather_sequence_head", _gather_v_unscaled),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistakes_are_caught(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(da, attr, fn)
    broken = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin()
            except Exception:  # an assertion or a crash: the pin noticed
                broken.append(pin.__name__)
    assert broken, f"no pin catches the planted mistake {mutant!r}"


# ---------------------------------------------------------------------------
# pins of the cache write (the new token's K/V into its slot; FP8 on write)


def test_e4m3fn_encode_matches_torch_cast():
    """Nearest-even encoding against torch's own float8_e4m3fn cast."""
    rng = _rng(11)
    y = np.concatenate([
        rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 3,
        rng.standard_normal(5000) * 2.0 ** -8,  # subnormal range
        oracle.E4M3FN_TABLE[:0x7F], -oracle.E4M3FN_TABLE[1:0x7F],
    ]).astype(np.float32)
    want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3fn_encode(y)
    assert np.array_equal(got, want)


def test_e4m3fn_encode_ties_to_even():
    """Midpoints between neighbouring codes go to the even code."""
    v = oracle.E4M3FN_TABLE
    for c in range(0, 0x7E):
        mid = (v[c] + v[c + 1]) / 2  # exact in float64
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3fn_encode(np.array([mid]))[0] == even, c
        assert oracle.e4m3fn_encode(np.array([-mid]))[0] == (even | 0x80), c
        # just off the midpoint goes to the nearer code
        assert oracle.e4m3fn_encode(np.array([np.nextafter(mid, 0)]))[0] == c
        assert oracle.e4m3fn_encode(np.array([np.nextafter(mid, 1000)]))[0] == c + 1


def test_quantize_row_scale_and_bound():
    """Scale = absmax/448 in float32; the absmax element is +-448 exactly;
    zero rows get scale 1; every value is within half an E4M3 step of
    x/scale (relative 2^-4 for normals, 2^-10 absolute in the subnormals)."""
    rng = _rng(12)
    for trial in range(200):
        x = (rng.standard_normal(128) * 10.0 ** rng.uniform(-6, 4)).astype(np.float32)
        codes, sc = oracle.quantize_row(x)
        assert sc == np.float32(np.max(np.abs(x))) / np.float32(448)
        i = int(np.argmax(np.abs(x)))
        assert oracle.E4M3FN_TABLE[codes[i]] == 448.0 * np.sign(x[i])
        y = np.clip(x.astype(np.float64) / np.float64(sc), -448, 448)
        dq = oracle.E4M3FN_TABLE[codes]
        bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10)
        assert np.all(np.abs(dq - y) <= bound + 1e-12 * np.abs(y)), trial
    codes, sc = oracle.quantize_row(np.zeros(64, np.float32))
    assert sc == 1.0 and np.all(codes == 0)


def test_quantize_row_matches_the_input_fixture():
    """The write quantiser and the (torch) quantiser that produced the FP8
    workloads agree code for code and scale for scale."""
    from workloads.synthetic import _to_fp8
    x = _rng(13).standard_normal((3, 16, 2, 128)).astype(np.float32)
    codes, scales = _to_fp8(x)
    for n in range(3):
        for s in range(16):
            for g in range(2):
                c, sc = oracle.quantize_row(x[n, s, g])
                assert np.array_equal(c, codes[n, s, g]) and sc == scales[n, g, s]


def test_append_writes_exactly_the_new_slots():
    """Only row (table[b][(n-1)//16], (n-1)%16, g) changes, for every b with
    n > 0 and every KV head g; empty sequences and other slots keep their
    bytes."""
    for kv in ("f32", "bf16", "fp8_e4m3"):
        spec = Spec(name="app", batch=5, num_q_heads=4, num_kv_heads=2, head_dim=64,
                    kv_dtype=kv, q_dtype="f32" if kv == "f32" else "bf16", seed=21,
                    context_lens=(1, 16, 17, 0, 40))
        inp = make_inputs(spec, poison=True)
        rng = _rng(22)
        x_k = rng.standard_normal((5, 2, 64)).astype(np.float32)
        x_v = rng.standard_normal((5, 2, 64)).astype(np.float32)
        if kv == "bf16":
            kn = torch.from_numpy(x_k).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            vn = torch.from_numpy(x_v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        else:
            kn, vn = x_k, x_v
        k2, v2, ks2, vs2 = oracle.append_new_tokens(
            inp.k_pool, inp.v_pool, inp.block_table, inp.context_lens, kn, vn, kv,
            inp.k_scale, inp.v_scale)
        changed = np.zeros(inp.k_pool.shape[:3], bool)
        for b, n in enumerate(inp.context_lens):
            if n == 0:
                continue
            t = n - 1
            p, o = inp.block_table[b, t // 16], t % 16
            changed[p, o, :] = True
            if kv == "fp8_e4m3":
                for g in range(2):
                    c, sc = oracle.quantize_row(x_k[b, g])
                    assert np.array_equal(k2[p, o, g], c) and ks2[p, g, o] == sc
            else:
                assert np.array_equal(k2[p, o], kn[b]) and np.array_equal(v2[p, o], vn[b])
        same = lambda a, b: np.array_equal(a.view(np.uint8), b.view(np.uint8))  # NaN-safe
        assert same(k2[~changed], inp.k_pool[~changed]) and same(v2[~changed], inp.v_pool[~changed])


def test_append_then_attend_is_contiguous_attention():
    """Append each new token, then attend: the result equals torch's float64
    attention over the contiguous cache that includes the new token (the
    decode step of [d7kj] section 六)."""
    rng = _rng(23)
    Hq, Hkv, d = 8, 2, 64
    lens = [5, 16, 33]
    pool = AppendOnlyPool(16, Hkv, d, rng)
    cache_k = [rng.standard_normal((n, Hkv, d)) for n in lens]
    cache_v = [rng.standard_normal((n, Hkv, d)) for n in lens]
    for s, n in enumerate(lens):
        for t in range(n - 1):  # all but the newest token are already cached
            pool.append(s, cache_k[s][t], cache_v[s][t])
        pool.append(s, np.full((Hkv, d), np.nan), np.full((Hkv, d), np.nan))  # its slot
    table = pool.table(len(lens))
    k_new = np.stack([cache_k[s][-1] for s in range(len(lens))])
    v_new = np.stack([cache_v[s][-1] for s in range(len(lens))])
    k2, v2, _, _ = oracle.append_new_tokens(pool.k, pool.v, table, lens, k_new, v_new, "f64")
    q = rng.standard_normal((len(lens), Hq, d))
    got = _oracle(q, k2, v2, table, lens, 0.125)
    for s in range(len(lens)):
        want = _sdpa(q[s], cache_k[s], cache_v[s], 0.125)
        assert np.allclose(got[s], want, rtol=0, atol=1e-12)
