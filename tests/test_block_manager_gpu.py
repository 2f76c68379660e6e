"""GPU side of the block manager: block copies, and a whole engine loop.

* pa_copy_blocks copies K, V (and FP8 scales) of whole blocks bit for bit and
  skips pairs with an id outside the pool or src == dst.
* Engine loop: the native manager hands out blocks for prompts that share
  prefixes (prefix cache), forks branches (copy-on-write of the shared
  partial block), frees and re-adds sequences; the GPU performs the copies
  (pa_copy_blocks), writes each new token (pa_cache_append) and attends
  (pa_decode_run).  Every step's output must equal the oracle's attention
  over each sequence's own contiguous K/V, where the K/V of a position are
  those of the prefix ending there (so a block shared by sequences with
  different histories would be caught).
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_398_amd as pa

pytestmark = pytest.mark.gpu
BLOCK = 16


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8_e4m3"])
def test_copy_blocks_bit_exact(kv):
    N, hkv, d = 12, 2, 64
    eb = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[kv]
    rng = np.random.Generator(np.random.PCG64(5))
    k = torch.from_numpy(rng.integers(0, 256, size=(N, BLOCK, hkv, d * eb), dtype=np.uint8)).cuda()
    v = torch.from_numpy(rng.integers(0, 256, size=(N, BLOCK, hkv, d * eb), dtype=np.uint8)).cuda()
    ks = vs = None
    if kv == "fp8_e4m3":
        ks = torch.from_numpy(rng.standard_normal((N, hkv, BLOCK), dtype=np.float32)).cuda()
        vs = torch.from_numpy(rng.standard_normal((N, hkv, BLOCK), dtype=np.float32)).cuda()
    k0, v0 = k.cpu().numpy(), v.cpu().numpy()
    ks0 = None if ks is None else ks.cpu().numpy()
    vs0 = None if vs is None else vs.cpu().numpy()
    pairs = np.array([[1, 5], [2, 2], [3, 99], [-1, 4], [7, 0], [9, 11]], np.int32)
    h = pa.pa_kv_pool_create(N, BLOCK, hkv, d, kv, k, v, ks, vs)  # raw bytes, explicit shape
    try:
        say(f"[bm] copy blocks kv={kv}")
        pa.pa_copy_blocks(h, torch.from_numpy(pairs).cuda(), len(pairs))
        torch.cuda.synchronize()
    finally:
        pa.pa_kv_pool_destroy(h)
    wk, wv = k0.copy(), v0.copy()
    for s, t in ((1, 5), (7, 0), (9, 11)):
        wk[t], wv[t] = k0[s], v0[s]
    assert np.array_equal(k.cpu().numpy(), wk) and np.array_equal(v.cpu().numpy(), wv)
    if ks is not None:
        wks, wvs = ks0.copy(), vs0.copy()
        for s, t in ((1, 5), (7, 0), (9, 11)):
            wks[t], wvs[t] = ks0[s], vs0[s]
        assert np.array_equal(ks.cpu().numpy(), wks) and np.array_equal(vs.cpu().numpy(), wvs)


class Engine:
    """A miniature serving loop over one bf16 pool, driven by the native
    block manager."""

    def __init__(self, N, hkv, hq, d, seed):
        self.N, self.hkv, self.hq, self.d = N, hkv, hq, d
        self.rng = np.random.Generator(np.random.PCG64(seed))
        self.k = torch.full((N, BLOCK, hkv, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        self.v = torch.full((N, BLOCK, hkv, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        self.pool = pa.PagedKVPool(self.k, self.v, "bf16")
        self.bm = pa.BlockManager(N, True)
        self.tokens = {}      # seq -> tokens
        self.prefix_kv = {}   # prefix tuple -> (k, v) rows [hkv][d] as bf16-exact float32
        self.copies = 0

    def kv_of(self, toks, pos):
        key = tuple(toks[:pos + 1])
        if key not in self.prefix_kv:
            kv = self.rng.standard_normal((2, self.hkv, self.d), dtype=np.float32)
            kv = torch.from_numpy(kv).to(torch.bfloat16).float().numpy()
            self.prefix_kv[key] = kv
        return self.prefix_kv[key]

    def add(self, seq, prompt):
        cached = self.bm.add(seq, prompt)
        self.tokens[seq] = list(prompt)
        table, _ = self.bm.table([seq], max(1, -(-len(prompt) // BLOCK)))
        for pos in range(cached, len(prompt)):  # the prompt's own K/V (prefill)
            kv = self.kv_of(prompt, pos)
            b, o = int(table[0, pos // BLOCK]), pos % BLOCK
            self.k[b, o] = torch.from_numpy(kv[0]).to(torch.bfloat16).cuda()
            self.v[b, o] = torch.from_numpy(kv[1]).to(torch.bfloat16).cuda()
        return cached

    def fork(self, parent, child):
        self.bm.fork(parent, child)
        self.tokens[child] = list(self.tokens[parent])

    def free(self, seq):
        self.bm.free(seq)
        del self.tokens[seq]

    def step(self):
        """One decode step of every live sequence: reserve, copy, write,
        attend; returns (GPU output, oracle output)."""
        seqs = sorted(self.tokens)
        pairs = []
        for s in seqs:
            tok = int(self.rng.integers(0, 3))
            pairs += self.bm.append(s, tok)
            self.tokens[s].append(tok)
        if pairs:
            p = torch.tensor(pairs, dtype=torch.int32, device="cuda")
            pa.pa_copy_blocks(self.pool.handle, p, len(pairs))
            self.copies += len(pairs)
        width = max(-(-len(self.tokens[s]) // BLOCK) for s in seqs)
        table, lens = self.bm.table(seqs, width)
        tb = torch.from_numpy(table).cuda()
        ln = torch.from_numpy(lens).cuda()
        self.pool.set_block_table(tb, ln, int(lens.max()))
        new = np.stack([self.kv_of(self.tokens[s], len(self.tokens[s]) - 1) for s in seqs])
        k_new = torch.from_numpy(new[:, 0]).to(torch.bfloat16).cuda()
        v_new = torch.from_numpy(new[:, 1]).to(torch.bfloat16).cuda()
        self.pool.append(k_new, v_new)
        q = torch.from_numpy(self.rng.standard_normal((len(seqs), self.hq, self.d),
                                                      dtype=np.float32)).to(torch.bfloat16)
        out = torch.empty((len(seqs), self.hq, self.d), dtype=torch.float32, device="cuda")
        wsb = self.pool.workspace_bytes(self.hq)
        ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
        self.pool.decode(q.cuda(), out, ws if wsb else None)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        # oracle: each sequence's own contiguous K/V (table 0, 1, 2, ...)
        qb = q.view(torch.int16).numpy().view(np.uint16)
        want = np.empty_like(got, dtype=np.float64)
        scale = np.float32(1.0 / np.sqrt(self.d))
        for i, s in enumerate(seqs):
            toks = self.tokens[s]
            n = len(toks)
            rows = np.stack([self.kv_of(toks, p) for p in range(n)])  # [n][2][hkv][d]
            nb = -(-n // BLOCK)
            kp = np.zeros((nb, BLOCK, self.hkv, self.d))
            vp = np.zeros((nb, BLOCK, self.hkv, self.d))
            kp.reshape(-1, self.hkv, self.d)[:n] = rows[:, 0]
            vp.reshape(-1, self.hkv, self.d)[:n] = rows[:, 1]
            want[i] = oracle.paged_decode_attention(
                qb[i:i + 1], kp, vp, np.arange(nb, dtype=np.int32)[None], np.array([n]), scale,
                kv_dtype="f64", q_dtype="bf16")[0]
        return got, want

    def close(self):
        self.pool.close()
        self.bm.close()


def test_engine_loop_with_prefix_cache_and_copy_on_write():
    eng = Engine(N=64, hkv=2, hq=8, d=64, seed=17)
    try:
        base = [int(x) for x in eng.rng.integers(0, 3, size=40)]
        assert eng.add(0, base) == 0
        assert eng.add(1, base[:32] + [2, 2, 1, 0, 1]) == 32  # two cached blocks shared
        eng.fork(0, 2)  # shares the partial third block: copy-on-write next step
        worst = 0.0
        for step in range(40):
            if step == 10:
                eng.free(1)
            if step == 12:
                assert eng.add(3, base[:35]) == 32  # blocks kept cached after the free
            if step == 20:
                eng.fork(3, 4)
            got, want = eng.step()
            err = float(np.abs(got - want).max())
            worst = max(worst, err)
            assert err <= 2e-3, (step, err)
        say(f"[bm] engine loop: {eng.copies} block copies, max err {worst:.2e}, "
            f"stats {eng.bm.stats()}")
        assert eng.copies >= 2
    finally:
        eng.close()
