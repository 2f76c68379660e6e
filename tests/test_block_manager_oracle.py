"""Pins of the block-manager model (oracle/block_manager.py).

The model is checked against what the pages fix, not against itself:

* content: a driver writes every token's identity into the slot the manager
  reserves for it (and performs the copies it orders); reading any live
  sequence back through its block table must give exactly its own tokens,
  whatever blocks it shares ("KV Cache 深度解析" section 三: logical order
  through the table, shared physical blocks);
* accounting: reference counts equal the table entries that point at a
  block; free, cached and used blocks partition the pool; a sequence holds
  ceil(len / 16) blocks, so at most one partly filled block (section 三);
* prefix reuse: the tokens reported as cached equal, by brute force, the
  longest run of leading full blocks whose exact token prefix was registered
  and is still cached, and one different early token defeats all reuse
  (section 七);
* attention: the decode oracle run over the manager's tables and a pool
  filled through them equals torch's attention over each sequence's own
  contiguous K/V.

``test_planted_block_manager_mistakes_are_caught`` plants plausible mistakes
and checks that each one breaks a pin.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import block_manager as bm

BLOCK = 16


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


class Driver:
    """Runs random operations on a manager and mirrors the pool's contents.

    What a slot holds stands for the K/V a model computes there, which
    depend on the token and on every token before it: the slot of position p
    stores the identity of the prefix tokens[0..p] (an index into a table of
    the distinct prefixes seen)."""

    def __init__(self, mgr, num_blocks, rng, vocab=5):
        self.m, self.rng, self.vocab = mgr, rng, vocab
        self.content = np.full((num_blocks, BLOCK), -1, np.int64)
        self.live = []
        self.next_id = 0
        self.prompts = []  # prompts issued so far, to draw shared prefixes from
        self.prefix_ids = {}

    def prefix_id(self, toks, pos):
        key = tuple(toks[:pos + 1])
        return self.prefix_ids.setdefault(key, len(self.prefix_ids))

    def _write(self, seq, pos, tok):
        blk = self.m.tables[seq][pos // BLOCK]
        toks = self.m.tokens[seq]
        assert toks[pos] == tok
        self.content[blk, pos % BLOCK] = self.prefix_id(toks, pos)

    def _prompt(self):
        r = self.rng
        if self.prompts and r.random() < 0.6:  # reuse a prefix of an earlier prompt
            base = self.prompts[r.integers(len(self.prompts))]
            cut = int(r.integers(0, len(base) + 1))
            tail = r.integers(0, self.vocab, size=int(r.integers(0, 40))).tolist()
            p = base[:cut] + tail
        else:
            p = r.integers(0, self.vocab, size=int(r.integers(1, 70))).tolist()
        return p or [int(r.integers(self.vocab))]

    def step(self):
        r = self.rng
        op = r.random()
        try:
            if op < 0.3 or not self.live:
                p = self._prompt()
                s = self.next_id
                self.next_id += 1
                cached = self.m.add(s, p)
                # the engine computes (writes) the tokens past the cached ones
                for pos in range(cached, len(p)):
                    self._write(s, pos, p[pos])
                self.live.append(s)
                self.prompts.append(p)
                return ("add", s, cached)
            s = self.live[int(r.integers(len(self.live)))]
            if op < 0.75:
                tok = int(r.integers(self.vocab))
                pos = len(self.m.tokens[s])
                copies = self.m.append(s, tok)
                for src, dst in copies:
                    self.content[dst] = self.content[src]
                self._write(s, pos, tok)
                return ("append", s)
            if op < 0.85:
                c = self.next_id
                self.next_id += 1
                self.m.fork(s, c)
                self.live.append(c)
                return ("fork", s, c)
            self.m.free_seq(s)
            self.live.remove(s)
            return ("free", s)
        except bm.OutOfBlocks:
            return ("full",)

    def check(self):
        m = self.m
        for s in self.live:
            toks = m.tokens[s]
            t = m.tables[s]
            assert len(t) == -(-len(toks) // BLOCK)  # at most one block partly filled
            got = [int(self.content[t[p // BLOCK], p % BLOCK]) for p in range(len(toks))]
            want = [self.prefix_ids.get(tuple(toks[:p + 1]), -2) for p in range(len(toks))]
            assert got == want, f"sequence {s} reads back K/V of another prefix"
        refs = np.zeros(m.n, np.int64)
        for s in self.live:
            for b in m.tables[s]:
                refs[b] += 1
        assert refs.tolist() == m.ref
        used = {b for b in range(m.n) if refs[b] > 0}
        free, cached = set(m.free), set(m.cached_lru)
        assert len(free) == len(m.free) and len(cached) == len(m.cached_lru)
        assert not (free & cached) and not (free & used) and not (cached & used)
        assert len(free) + len(cached) + len(used) == m.n


def _run(seed, n_ops, num_blocks, caching, check_every=1):
    d = Driver(bm.BlockManager(num_blocks, caching), num_blocks, _rng(seed))
    for i in range(n_ops):
        d.step()
        if i % check_every == 0:
            d.check()
    d.check()
    return d


# ---------------------------------------------------------------------------
# pins


def pin_contents_and_accounting_without_caching():
    for seed in range(3):
        _run(100 + seed, 400, 64, caching=False)


def pin_contents_and_accounting_with_caching():
    for seed in range(3):
        _run(200 + seed, 400, 64, caching=True)


def pin_out_of_blocks_leaves_state_unchanged():
    m = bm.BlockManager(4, True)
    m.add(0, list(range(40)))  # 3 blocks
    before = (list(m.free), list(m.cached_lru), list(m.ref), {k: list(v) for k, v in m.tables.items()})
    with pytest.raises(bm.OutOfBlocks):
        m.add(1, list(range(100, 140)))
    assert before == (list(m.free), list(m.cached_lru), list(m.ref),
                      {k: list(v) for k, v in m.tables.items()})


def pin_cached_prefix_by_brute_force():
    """Prompts are cut from earlier ones or assembled from a few recurring
    16-token blocks (so equal blocks often follow different histories)."""
    rng = _rng(7)
    m = bm.BlockManager(512, True)
    pieces = [rng.integers(0, 3, size=BLOCK).tolist() for _ in range(3)]
    registered = []  # every prompt added so far
    live = []
    for i in range(120):
        u = rng.random()
        if registered and u < 0.4:
            base = registered[int(rng.integers(len(registered)))]
            p = base[: int(rng.integers(0, len(base) + 1))] + rng.integers(0, 3, size=int(rng.integers(0, 30))).tolist()
        elif u < 0.8:
            p = sum((pieces[int(k)] for k in rng.integers(0, 3, size=int(rng.integers(1, 5)))), [])
            p = p + rng.integers(0, 3, size=int(rng.integers(0, 20))).tolist()
        else:
            p = rng.integers(0, 3, size=int(rng.integers(1, 60))).tolist()
        if not p:
            p = [0]
        # brute force: leading full blocks within p[:-1] whose exact token
        # prefix is the prefix of an earlier prompt (all still cached: the
        # pool is large enough that nothing is evicted)
        want = 0
        for j in range((len(p) - 1) // BLOCK):
            pre = p[: BLOCK * (j + 1)]
            if any(len(q) >= len(pre) and q[: len(pre)] == pre for q in registered):
                want = BLOCK * (j + 1)
            else:
                break
        assert m.add(i, p) == want
        registered.append(p)
        live.append(i)
        if rng.random() < 0.4:
            s = live.pop(int(rng.integers(len(live))))
            m.free_seq(s)  # released blocks stay cached: still counted


def pin_one_early_token_defeats_reuse():
    m = bm.BlockManager(64, True)
    p = list(range(200))
    m.add(0, p)
    q = list(p)
    q[3] = 999  # one different token in the first block
    assert m.add(1, q) == 0
    r = list(p)
    r[20] = 999  # in the second block: the first block is still reused
    assert m.add(2, r) == BLOCK


def pin_same_block_after_a_different_history_is_not_reused():
    m = bm.BlockManager(64, True)
    A, B, X, Y = ([k] * BLOCK for k in (1, 2, 3, 4))
    m.add(0, A + X + [0])
    m.add(1, Y + B + [0])
    assert m.add(2, A + B + [0]) == BLOCK  # block A is reused, block B is not
    assert m.tables[2][0] == m.tables[0][0]
    assert m.tables[2][1] != m.tables[1][1]


def pin_eviction_takes_least_recently_released():
    m = bm.BlockManager(6, True)
    m.add(0, list(range(32)) + [7])    # blocks 0, 1 full (registered), 2 partial
    m.add(1, list(range(100, 132)) + [7])  # blocks 3, 4, 5
    m.free_seq(0)  # releases 2 (unregistered: free), then 1, 0 (cached)
    assert m.free == [2] and m.cached_lru == [1, 0]
    m.add(2, list(range(500, 540)))  # needs 3 blocks: 2, then evicts 1, then 0
    assert m.tables[2] == [2, 1, 0]
    assert m.stats() == (0, 0)


def pin_paged_attention_through_the_manager():
    """Fill a pool through the manager's tables, then the decode oracle
    equals attention over each sequence's own contiguous K/V.  The K/V of a
    slot are those of the prefix it was computed for (the driver's mirror),
    so a block shared between sequences with different histories would give
    a wrong result."""
    rng = _rng(9)
    d, hkv, hq = 8, 2, 4
    N = 48
    dr = Driver(bm.BlockManager(N, True), N, rng)
    for _ in range(150):
        dr.step()
    dr.check()
    kv_of = rng.standard_normal((2, len(dr.prefix_ids) + 1, hkv, d))  # [K/V][prefix id]
    k_pool = np.full((N, BLOCK, hkv, d), np.nan)
    v_pool = np.full((N, BLOCK, hkv, d), np.nan)
    seqs = list(dr.live)
    for s in seqs:
        for pos in range(len(dr.m.tokens[s])):
            blk = dr.m.tables[s][pos // BLOCK]
            pid = dr.content[blk, pos % BLOCK]  # what the pool holds there
            k_pool[blk, pos % BLOCK] = kv_of[0, pid]
            v_pool[blk, pos % BLOCK] = kv_of[1, pid]
    width = max(len(dr.m.tables[s]) for s in seqs)
    rows, lens = dr.m.table(seqs, width)
    q = rng.standard_normal((len(seqs), hq, d))
    got = oracle.paged_decode_attention(q, k_pool, v_pool, np.asarray(rows), np.asarray(lens),
                                        0.3, kv_dtype="f64", q_dtype="f64")
    for i, s in enumerate(seqs):
        toks = dr.m.tokens[s]
        K = np.stack([kv_of[0, dr.prefix_id(toks, p)] for p in range(len(toks))])
        V = np.stack([kv_of[1, dr.prefix_id(toks, p)] for p in range(len(toks))])
        qt = torch.from_numpy(q[i])[None, :, None, :]
        kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]
        vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
        want = F.scaled_dot_product_attention(qt, kt, vt, scale=0.3, enable_gqa=True)[0, :, 0]
        np.testing.assert_allclose(got[i], want.numpy(), rtol=0, atol=1e-12)


PINS = [
    pin_contents_and_accounting_without_caching,
    pin_contents_and_accounting_with_caching,
    pin_out_of_blocks_leaves_state_unchanged,
    pin_cached_prefix_by_brute_force,
    pin_one_early_token_defeats_reuse,
    pin_same_block_after_a_different_history_is_not_reused,
    pin_eviction_takes_least_recently_released,
    pin_paged_attention_through_the_manager,
]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_block_manager_pin(pin):
    pin()


def _no_copy_on_write(self, seq, token):
    table, toks = self.tables[seq], self.tokens[seq]
    t = len(toks)
    if t % BLOCK == 0:
        table.append(self._take())
    toks.append(int(token))
    if (t + 1) % BLOCK == 0:
        self._register_full(seq, t // BLOCK)
    return []


def _hash_without_parent(parent, tokens):
    return _REAL_HASH(0, tokens)


def _release_leaks(self, b):
    self.ref[b] -= 1


class _LeaveRevivedInList(list):
    def remove(self, x):  # a revived cached block stays evictable
        pass


def _add_leaving_revived(self, seq, prompt):
    self.cached_lru = _LeaveRevivedInList(self.cached_lru)
    try:
        return _REAL_ADD(self, seq, prompt)
    finally:
        self.cached_lru = list(self.cached_lru)


def _chain_one_block_more(self, toks, nblocks):
    n = nblocks + 1 if nblocks * BLOCK + BLOCK <= len(toks) else nblocks
    return _REAL_CHAIN(self, toks, n)


def _match_without_token_compare(self, h, toks):
    for t, b in self.by_hash.get(h, []):
        return b
    return None


_REAL_HASH = bm.block_hash
_REAL_ADD = bm.BlockManager.add
_REAL_CHAIN = bm.BlockManager._chain

MUTANTS = {
    "no_copy_on_write": (bm.BlockManager, "append", _no_copy_on_write),
    "hash_ignores_earlier_blocks": (bm, "block_hash", _hash_without_parent),
    "release_never_frees": (bm.BlockManager, "_release", _release_leaks),
    "revived_block_stays_evictable": (bm.BlockManager, "add", _add_leaving_revived),
    "last_prompt_block_reused": (bm.BlockManager, "_chain", _chain_one_block_more),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_block_manager_mistakes_are_caught(mutant, monkeypatch):
    obj, attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(obj, attr, fn)
    broken = []
    for pin in PINS:
        try:
            pin()
        except Exception:
            broken.append(pin.__name__)
    assert broken, f"no pin catches the planted mistake {mutant!r}"
