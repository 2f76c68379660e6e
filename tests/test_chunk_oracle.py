"""Pins of the multi-token (chunk) attention oracle to facts other than itself.

* The minimal implementation of "KV Cache 深度解析" section 六, re-stated with
  a contiguous cache: feeding a prompt one position at a time, each step's
  output is what the chunk oracle must give for that position's row.
* torch's scaled-dot-product attention in float64 with a causal mask (the
  full-prefill case, where every cached token is new) and with an explicit
  boolean mask (a chunk after a cached prefix).
* A chunk of one row per sequence is a decode step (the decode oracle is
  pinned on its own).
* Exact invariances: tokens after a row's position cannot change it.
``test_planted_chunk_mistakes_are_caught`` plants plausible mistakes (on the
CPU) and checks that each one breaks at least one pin.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import chunk_attention as ca
from workloads import BLOCK_SIZE

from test_oracle_pins import AppendOnlyPool


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _chunk(q, pool, table, ctx, q_start, scale, **kw):
    return oracle.paged_chunk_attention(q, pool.k, pool.v, table, np.asarray(ctx),
                                        np.asarray(q_start), scale, kv_dtype="f64",
                                        q_dtype="f64", **kw)


def _build(lens, Hkv, d, rng):
    """Per-sequence tokens K, V ([n, Hkv, d]) appended into one paged pool."""
    Ks = [rng.standard_normal((n, Hkv, d)) for n in lens]
    Vs = [rng.standard_normal((n, Hkv, d)) for n in lens]
    pool = AppendOnlyPool(sum((n + 15) // 16 for n in lens) + 2, Hkv, d, rng)
    for t in range(max(lens)):
        for b, n in enumerate(lens):
            if t < n:
                pool.append(b, Ks[b][t], Vs[b][t])
    return Ks, Vs, pool


def _q_start(nq):
    s = np.zeros(len(nq) + 1, np.int64)
    np.cumsum(nq, out=s[1:])
    return s


# ---------------------------------------------------------------------------
# pins


def pin_step_by_step_prompt():
    """Feed each sequence's prompt one position at a time into a growing
    contiguous cache (append k/v, then attend); the chunk rows of the last
    n positions must equal those steps' outputs."""
    rng = _rng(31)
    Hq, Hkv, d = 4, 2, 8
    lens, nq = [21, 40, 16, 5], [7, 40, 1, 5]
    Ks, Vs, pool = _build(lens, Hkv, d, rng)
    qs = [rng.standard_normal((n, Hq, d)) for n in lens]  # a query per position
    scale = 1.0 / math.sqrt(d)
    q = np.concatenate([qs[b][lens[b] - nq[b]:] for b in range(len(lens))])
    got = _chunk(q, pool, pool.table(len(lens)), lens, _q_start(nq), scale)
    row = 0
    for b, n in enumerate(lens):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            kc, vc = np.zeros((0, d)), np.zeros((0, d))
            outs = []
            for t in range(n):
                kc = np.concatenate([kc, Ks[b][t, g][None]])
                vc = np.concatenate([vc, Vs[b][t, g][None]])
                s = qs[b][t, h] @ kc.T * scale
                e = np.exp(s - s.max())
                outs.append((e / e.sum()) @ vc)
            for i in range(nq[b]):
                np.testing.assert_allclose(got[row + i, h], outs[n - nq[b] + i],
                                           rtol=0, atol=1e-13)
        row += nq[b]


def pin_full_prefill_is_causal_library_attention():
    """Every cached token new: torch SDPA with is_causal=True (GQA)."""
    rng = _rng(32)
    Hq, Hkv, d = 8, 2, 16
    lens = [33, 16, 1]
    Ks, Vs, pool = _build(lens, Hkv, d, rng)
    q = rng.standard_normal((sum(lens), Hq, d))
    scale = 1.0 / math.sqrt(d)
    got = _chunk(q, pool, pool.table(len(lens)), lens, _q_start(lens), scale)
    row = 0
    for b, n in enumerate(lens):
        qt = torch.from_numpy(np.ascontiguousarray(q[row:row + n].transpose(1, 0, 2)))[None]
        kt = torch.from_numpy(np.ascontiguousarray(Ks[b].transpose(1, 0, 2)))[None]
        vt = torch.from_numpy(np.ascontiguousarray(Vs[b].transpose(1, 0, 2)))[None]
        want = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale,
                                              enable_gqa=True)[0].numpy().transpose(1, 0, 2)
        np.testing.assert_allclose(got[row:row + n], want, rtol=0, atol=1e-12)
        row += n


def pin_chunk_after_prefix_is_masked_library_attention():
    """A chunk after a cached prefix: SDPA with the mask t <= ctx - n + i."""
    rng = _rng(33)
    Hq, Hkv, d = 6, 3, 8
    lens, nq = [50, 17, 64], [9, 17, 3]
    Ks, Vs, pool = _build(lens, Hkv, d, rng)
    q = rng.standard_normal((sum(nq), Hq, d))
    scale = 0.3
    got = _chunk(q, pool, pool.table(len(lens)), lens, _q_start(nq), scale)
    row = 0
    for b, n in enumerate(lens):
        m = nq[b]
        mask = np.arange(n)[None, :] <= (n - m + np.arange(m))[:, None]
        qt = torch.from_numpy(np.ascontiguousarray(q[row:row + m].transpose(1, 0, 2)))[None]
        kt = torch.from_numpy(np.ascontiguousarray(Ks[b].transpose(1, 0, 2)))[None]
        vt = torch.from_numpy(np.ascontiguousarray(Vs[b].transpose(1, 0, 2)))[None]
        want = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask),
                                              scale=scale, enable_gqa=True)
        np.testing.assert_allclose(got[row:row + m], want[0].numpy().transpose(1, 0, 2),
                                   rtol=0, atol=1e-12)
        row += m


def pin_single_row_chunks_are_decode_steps():
    rng = _rng(34)
    Hq, Hkv, d = 4, 1, 8
    lens = [3, 31, 47]
    _, _, pool = _build(lens, Hkv, d, rng)
    q = rng.standard_normal((len(lens), Hq, d))
    table = pool.table(len(lens))
    got = _chunk(q, pool, table, lens, _q_start([1] * len(lens)), 0.25)
    want = oracle.paged_decode_attention(q, pool.k, pool.v, table, np.asarray(lens), 0.25,
                                         kv_dtype="f64", q_dtype="f64")
    np.testing.assert_array_equal(got, want)


def pin_later_tokens_are_invisible():
    """Changing the K/V of positions > p leaves row p bit-identical (and
    changes the rows that see them)."""
    rng = _rng(35)
    Hq, Hkv, d = 2, 2, 8
    n, m = 40, 12
    Ks, Vs, pool = _build([n], Hkv, d, rng)
    table = pool.table(1)
    q = rng.standard_normal((m, Hq, d))
    before = _chunk(q, pool, table, [n], [0, m], 0.5)
    cut = n - m + 5  # positions > cut are altered
    for t in range(cut + 1, n):
        blk, off = table[0, t // BLOCK_SIZE], t % BLOCK_SIZE
        pool.k[blk, off] += 3.0
        pool.v[blk, off] -= 2.0
    after = _chunk(q, pool, table, [n], [0, m], 0.5)
    np.testing.assert_array_equal(after[:6], before[:6])
    assert np.all(np.abs(after[6:] - before[6:]).max(axis=(1, 2)) > 1e-6)


def pin_rows_before_position_zero_are_zero():
    """More new rows than cached tokens: the excess rows (negative
    positions) are zero, the others are the full-prefill rows."""
    rng = _rng(36)
    Hq, Hkv, d = 2, 1, 8
    Ks, Vs, pool = _build([5], Hkv, d, rng)
    q = rng.standard_normal((8, Hq, d))
    table = pool.table(1)
    got = _chunk(q, pool, table, [5], [0, 8], 0.5)
    assert np.all(got[:3] == 0.0)
    np.testing.assert_array_equal(got[3:], _chunk(q[3:], pool, table, [5], [0, 5], 0.5))


PINS = [
    pin_step_by_step_prompt,
    pin_full_prefill_is_causal_library_attention,
    pin_chunk_after_prefix_is_masked_library_attention,
    pin_single_row_chunks_are_decode_steps,
    pin_later_tokens_are_invisible,
    pin_rows_before_position_zero_are_zero,
]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_chunk_pin(pin):
    pin()


MUTANTS = {
    "positions_one_late": ("chunk_positions", lambda ctx, n: ctx - n + 1 + np.arange(n)),
    "positions_ignore_prefix": ("chunk_positions", lambda ctx, n: np.arange(n)),
    "row_does_not_see_itself": ("visible_tokens", lambda p: p),
    "no_causal_mask": ("visible_tokens", lambda p: 1 << 30),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_chunk_mistakes_are_caught(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(ca, attr, fn)
    broken = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin()
            except Exception:
                broken.append(pin.__name__)
    assert broken, f"no pin catches the planted mistake {mutant!r}"
