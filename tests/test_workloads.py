"""The seeded input generator: determinism, table structure, poison, formats."""

import numpy as np
import pytest
import torch

from workloads import (BLOCK_SIZE, CHUNK_SPECS, NAMED_SPECS, Spec, make_chunk_inputs, make_inputs,
                       named_spec)


def test_deterministic():
    a = make_inputs(NAMED_SPECS["tiny_f32"])
    b = make_inputs(NAMED_SPECS["tiny_f32"])
    for x, y in ((a.q, b.q), (a.k_pool, b.k_pool), (a.v_pool, b.v_pool),
                 (a.block_table, b.block_table), (a.context_lens, b.context_lens)):
        assert np.array_equal(x, y)
    c = make_inputs(NAMED_SPECS["tiny_f32"], seed=1)
    assert not np.array_equal(a.k_pool, c.k_pool)


def test_tiny_structure():
    inp = make_inputs(NAMED_SPECS["tiny_f32"])
    assert inp.k_pool.shape == (32, 16, 2, 64) and inp.k_pool.dtype == np.float32
    assert inp.q.shape == (2, 8, 64)
    assert list(inp.context_lens) == [37, 100]
    assert inp.block_table.shape == (2, 7)
    assert (inp.block_table[0, 3:] == -1).all() and (inp.block_table[0, :3] >= 0).all()
    used = inp.block_table[inp.block_table >= 0]
    assert len(set(used.tolist())) == 10 and used.max() < 32
    assert inp.scale == np.float32(0.125)


def _check_tables(inp):
    N = inp.num_blocks
    for b, n in enumerate(inp.context_lens.tolist()):
        nb = (n + BLOCK_SIZE - 1) // BLOCK_SIZE
        row = inp.block_table[b]
        assert (row[:nb] >= 0).all() and (row[:nb] < N).all()
        assert (row[nb:] == -1).all()


def test_continuous_batch_structure():
    # full-size lengths and placement, tiny heads to keep it quick
    spec = named_spec("continuous_batch_b64", num_q_heads=4, num_kv_heads=1, head_dim=8)
    inp = make_inputs(spec)
    ctx = inp.context_lens
    assert ctx.shape == (64,)
    assert (ctx[:16] >= 1024).all() and (ctx >= 128).all() and (ctx <= 16384).all()
    _check_tables(inp)
    pre = inp.block_table[:16, :64]
    assert (pre == pre[0]).all()
    # all other referenced blocks are private
    others = np.concatenate([inp.block_table[0, 64:]] +
                            [inp.block_table[b, 64 if b < 16 else 0:] for b in range(1, 64)])
    others = others[others >= 0]
    assert len(set(others.tolist())) == len(others)
    assert not set(others.tolist()) & set(pre[0].tolist())
    assert inp.num_blocks == 64 + len(others)
    assert inp.unique_tokens == int(ctx.sum()) - 15 * 1024


def test_outlier_channels():
    spec = Spec(name="outliers", batch=2, num_q_heads=8, num_kv_heads=8, head_dim=128,
                kv_dtype="f32", q_dtype="f32", seed=5, context_lens=(400, 300),
                outlier_frac=0.01, outlier_gain=8.0)
    inp = make_inputs(spec)
    std = inp.k_pool.reshape(-1, 8 * 128).std(axis=0)
    big = np.flatnonzero(std > 4)
    assert len(big) == 10
    assert np.allclose(std[big], 8, rtol=0.15) and np.allclose(np.delete(std, big), 1, rtol=0.15)
    vstd = inp.v_pool.reshape(-1, 8 * 128).std(axis=0)
    assert np.array_equal(np.flatnonzero(vstd > 4), big)


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8_e4m3"])
def test_poison_marks_only_dead_positions(kv):
    spec = Spec(name="p", batch=3, num_q_heads=4, num_kv_heads=2, head_dim=16, kv_dtype=kv,
                q_dtype="bf16", seed=6, context_lens=(5, 16, 40), pool_blocks=9)
    clean = make_inputs(spec)
    dirty = make_inputs(spec, poison=True)
    if kv == "f32":
        bad = np.isnan(dirty.k_pool)
    elif kv == "bf16":
        bad = dirty.k_pool == 0x7FC0
    else:
        bad = dirty.k_pool == 0x7F
    expect = np.zeros_like(bad)
    expect[~clean.used_blocks] = True
    for b, n in enumerate(clean.context_lens.tolist()):
        if n % 16:
            expect[clean.block_table[b, (n - 1) // 16], n % 16:] = True
    assert np.array_equal(bad, expect)
    live = ~expect
    assert np.array_equal(dirty.k_pool[live], clean.k_pool[live])


def test_fp8_scales_are_absmax_over_448():
    spec = Spec(name="f8", batch=2, num_q_heads=2, num_kv_heads=2, head_dim=64,
                kv_dtype="fp8_e4m3", q_dtype="bf16", seed=7, context_lens=(30, 20))
    inp = make_inputs(spec)
    f = make_inputs(Spec(**{**spec.__dict__, "kv_dtype": "f32"}))
    vals = torch.from_numpy(inp.k_pool).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.all(np.abs(vals).max(axis=-1) == 448.0)
    sc = inp.k_scale.transpose(0, 2, 1)  # -> [N][16][Hkv]
    np.testing.assert_allclose(sc, np.abs(f.k_pool).max(axis=-1) / 448.0, rtol=1e-6)
    deq = vals * sc[..., None]
    err = np.abs(deq - f.k_pool)
    assert np.all(err <= np.abs(f.k_pool) / 16 + sc[..., None] * 2.0 ** -10)


@pytest.mark.parametrize("name", sorted(CHUNK_SPECS))
def test_named_chunk_workloads(name):
    """Each chunk workload builds; its rows are the last positions of every
    sequence, in sequence order, and the rows are seeded."""
    ci = make_chunk_inputs(name)
    s = ci.base.spec
    assert ci.q.shape == (ci.total_rows, s.num_q_heads, s.head_dim)
    assert ci.q_start[0] == 0 and np.all(np.diff(ci.q_start) == ci.q_lens)
    assert np.all(ci.q_lens <= ci.base.context_lens)
    again = make_chunk_inputs(name)
    assert np.array_equal(ci.q, again.q)
