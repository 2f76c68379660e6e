"""GPU parity of the multi-token chunk attention (pa_chunk_run) with the oracle.

Tolerance, from the kernel's arithmetic: q and K are bf16 (FP8 codes are
widened to bf16 exactly, and their per-token scales multiply the fp32
scores), so the products in the scores are exact and summed in fp32.  Each
softmax weight (times the V scale, for FP8) enters the PV product as hi + lo,
two bf16 values within a relative 2^-16 of it, and the normaliser sums the
same hi + lo of the weights, so each output element is a convex combination
of V values whose weights are off by at most a relative 2^-15:
  |out - ref| <= 2^-15 * sum_t w_t |V_t| + 1e-4
(the last term covers fp32 accumulation and the hardware exp2).  The wide
kernel (more than 256 rows per (sequence, KV head)) over a bf16 pool instead
rounds each weight to the nearest fp16 (a relative 2^-11) and takes V as
fp16 (exact for bf16 magnitudes in [2^-14, 65504], an absolute error under
2^-24 below), with the normaliser summing the same fp16 weights:
  |out - ref| <= 2^-10 * sum_t w_t |V_t| + 1e-4.
The bound is evaluated with the oracle itself, by running it on |V|.  Every
case must also meet the decode bar, 2e-3.
"""

import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_398_amd as pa
from workloads import Spec, chunk_queries, make_chunk_inputs, make_inputs
from workloads.device import to_device

from gpu_util import host_threads as gpu_host_threads

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _q_dev(ci):
    return torch.from_numpy(ci.q.view(np.int16)).view(torch.bfloat16).cuda()


def gpu_chunk(ci, dev=None, extra_rows=0, q_start=None, max_q=None):
    base = ci.base
    dev = dev or to_device(base)
    s = base.spec
    T = ci.total_rows
    out = torch.full((T + extra_rows, s.num_q_heads, s.head_dim), float("nan"),
                     dtype=torch.float32, device="cuda")
    qs = torch.from_numpy(ci.q_start if q_start is None else q_start).cuda()
    pool = pa.PagedKVPool(dev.k_pool, dev.v_pool, s.kv_dtype, dev.k_scale, dev.v_scale)
    try:
        pool.set_block_table(dev.block_table, dev.context_lens, base.max_context_len)
        pool.chunk(_q_dev(ci), qs, ci.max_q_len if max_q is None else max_q, out,
                   scale=float(base.scale))
        torch.cuda.synchronize()
    finally:
        pool.close()
    return out.cpu().numpy()


def oracle_chunk(ci, seqs=None, abs_v=False):
    """The oracle's rows; with abs_v, over |V| (sign bits cleared: bf16 and
    E4M3FN are sign-magnitude, and FP8 scales are positive)."""
    b = ci.base
    kv = b.spec.kv_dtype
    v = b.v_pool
    if abs_v:
        v = v & (np.uint16(0x7FFF) if kv == "bf16" else np.uint8(0x7F))
    return oracle.paged_chunk_attention(ci.q, b.k_pool, v, b.block_table, b.context_lens,
                                        ci.q_start, b.scale, kv_dtype=kv, q_dtype="bf16",
                                        k_scale=b.k_scale, v_scale=b.v_scale, seqs=seqs)


REL_HL = 2.0 ** -15   # hi + lo bf16 weights
REL_F16 = 2.0 ** -10  # fp16 weights and V (the wide kernel over a bf16 pool)


def rel_of(ci):
    """The bound's factor for the kernel pa_chunk_run picks: more than 256
    rows per (sequence, KV head) go to the wide kernel, which takes fp16
    weights over a bf16 pool; every other case takes hi + lo bf16."""
    s = ci.base.spec
    rows = ci.max_q_len * (s.num_q_heads // s.num_kv_heads)
    return REL_F16 if (s.kv_dtype == "bf16" and rows > 256) else REL_HL


def bound_of(ci, seqs=None):
    return rel_of(ci) * oracle_chunk(ci, seqs, abs_v=True) + 1e-4


def rows_of(ci, seqs):
    return np.concatenate([np.arange(ci.q_start[b], ci.q_start[b + 1]) for b in seqs]
                          + [np.zeros(0, np.int64)]).astype(np.int64)


def assert_parity(ci, got, seqs=None):
    seqs = list(range(ci.base.spec.batch)) if seqs is None else list(seqs)
    want, bound = oracle_chunk(ci, seqs), bound_of(ci, seqs)
    r = rows_of(ci, seqs)
    err = np.abs(got[r] - want[r])
    assert np.all(np.isfinite(got[r]))
    bad = err > bound[r]
    assert not bad.any(), (f"{bad.sum()} elements over the bound; max err {err.max():.3e}, "
                           f"worst excess {(err - bound[r]).max():.3e}")
    # and the decode bar, which the derived bound does not imply for large |V|
    assert not err.size or err.max() <= 2e-3, f"max err {err.max():.3e} > 2e-3"
    return float(err.max()) if err.size else 0.0


def _spec(name, d, hq, hkv, ctx, seed, kv="bf16"):
    return Spec(name=name, batch=len(ctx), num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                kv_dtype=kv, q_dtype="bf16", seed=seed, context_lens=tuple(ctx))


GROUPS = [(8, 8), (8, 4), (8, 2), (16, 2)]  # G = 1, 2, 4, 8


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", GROUPS)
def test_chunk_small_shapes(d, hq, hkv):
    """Full prefills (n = ctx), chunks after a prefix, single rows, ragged
    block tails; unused slots and blocks hold NaN."""
    ctx = (1, 17, 40, 100, 33, 16, 70)
    nq = (1, 5, 40, 7, 33, 16, 1)
    base = make_inputs(_spec("chunk-small", d, hq, hkv, ctx, 700 + d + hq + hkv), poison=True)
    ci = chunk_queries(base, nq, 800 + d + hq)
    say(f"[chunk] small d={d} hq={hq} hkv={hkv} rows={ci.total_rows}")
    err = assert_parity(ci, gpu_chunk(ci))
    say(f"  max err {err:.2e}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nq", [2, 4, 9, 64, 200])
def test_chunk_tile_shapes(d, nq):
    """Each rows-per-workgroup choice (16, 32, and 256 rows staged through
    LDS), with a partial last tile."""
    ctx = (300, 257, nq)
    base = make_inputs(_spec("chunk-tiles", d, 8, 2, ctx, 900 + d + nq), poison=True)
    ci = chunk_queries(base, [nq, nq, nq], 950 + nq)
    say(f"[chunk] tiles d={d} nq={nq}")
    assert_parity(ci, gpu_chunk(ci))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", GROUPS)
def test_chunk_wide_shapes(d, hq, hkv):
    """More than 256 rows per sequence (256-row workgroups, K/V staged in
    LDS): partial last workgroups, a short sequence in the same launch, rows
    before position zero, ragged block tails; unused slots and blocks hold
    NaN."""
    ctx = (700, 300, 129, 1000, 40)
    nq = (300, 300, 129, 17, 60)
    base = make_inputs(_spec("chunk-wide", d, hq, hkv, ctx, 1100 + d + hq + hkv), poison=True)
    ci = chunk_queries(base, nq, 1150 + d + hq)
    say(f"[chunk] wide d={d} hq={hq} hkv={hkv} rows={ci.total_rows}")
    got = gpu_chunk(ci)
    r4 = int(ci.q_start[4])
    assert np.all(got[r4:r4 + 20] == 0.0)
    err = assert_parity(ci, got)
    say(f"  max err {err:.2e}")


@pytest.mark.parametrize("scale", [1.0, -0.3, 0.0])
def test_chunk_scale_extremes(scale):
    """Softmax scales other than 1/sqrt(d) through each kernel (16, 32 and
    256 rows per workgroup): 1.0 keeps raising the running maximum after the
    first pair, so the accumulated rows are rescaled (in the wide kernel with
    per-row factors gathered through LDS); a negative scale; 0 (uniform
    weights, masked slots still contribute nothing)."""
    ctx = (1000, 700, 300, 64)
    base = dataclasses.replace(make_inputs(_spec("chunk-scale", 128, 8, 2, ctx, 1300), poison=True),
                               scale=np.float32(scale))
    dev = to_device(base)
    for nq in ((4, 4, 4, 4), (40, 17, 40, 5), (300, 260, 129, 64)):
        ci = chunk_queries(base, nq, 1310 + nq[0])
        say(f"[chunk] scale={scale} rows/seq={nq}")
        err = assert_parity(ci, gpu_chunk(ci, dev=dev))
        say(f"  max err {err:.2e}")


def test_chunk_rows_before_position_zero():
    """More new rows than cached tokens: the excess rows are zero."""
    ctx = (5, 0, 20)
    nq = (9, 3, 20)
    base = make_inputs(_spec("chunk-neg", 128, 8, 2, ctx, 1001))
    ci = chunk_queries(base, nq, 1002)
    got = gpu_chunk(ci)
    assert np.all(got[0:4] == 0.0) and np.all(got[9:12] == 0.0)
    assert_parity(ci, got)


def test_chunk_skipped_rows_and_canary():
    """Sequences with no rows, or with row offsets outside [0, total_q), are
    skipped; rows past total_q are never written."""
    ctx = (40, 30, 50, 20)
    nq = (6, 0, 5, 4)
    base = make_inputs(_spec("chunk-skip", 64, 4, 2, ctx, 1011))
    ci = chunk_queries(base, nq, 1012)
    got = gpu_chunk(ci, extra_rows=3)
    assert np.all(np.isnan(got[ci.total_rows:]))
    assert_parity(ci, got)
    # sequence 3's rows running past total_q: skipped, its rows keep their NaN
    bad = ci.q_start.copy()
    bad[4] = ci.total_rows + 2
    got = gpu_chunk(ci, q_start=bad)
    assert np.all(np.isnan(got[ci.q_start[3]:]))
    assert_parity(ci, got, seqs=[0, 2])
    # more rows than max_q_len: skipped as well
    got = gpu_chunk(ci, max_q=5)
    assert np.all(np.isnan(got[ci.q_start[0]:ci.q_start[1]]))
    assert_parity(ci, got, seqs=[2, 3])


def test_chunk_is_deterministic():
    base = make_inputs(_spec("chunk-det", 128, 32, 8, (1000, 513), 1021))
    ci = chunk_queries(base, [300, 64], 1022)
    dev = to_device(base)
    a, b = gpu_chunk(ci, dev=dev), gpu_chunk(ci, dev=dev)
    assert np.array_equal(a, b, equal_nan=True)


def test_chunk_single_rows_match_decode_path():
    """One row per sequence is a decode step: the chunk kernel agrees with
    the decode kernel on the same cache and queries (within the chunk
    bound), and both with the oracle."""
    base = make_inputs(_spec("chunk-vs-decode", 128, 32, 8, (4096, 100, 1, 777), 1031))
    ci = chunk_queries(base, [1, 1, 1, 1], 1032)
    got = gpu_chunk(ci)
    assert_parity(ci, got)
    dev = to_device(base)
    q = _q_dev(ci)
    out = torch.empty((4, 32, 128), dtype=torch.float32, device="cuda")
    pool = pa.PagedKVPool(dev.k_pool, dev.v_pool, "bf16")
    try:
        pool.set_block_table(dev.block_table, dev.context_lens, base.max_context_len)
        ws_b = pool.workspace_bytes(32)
        ws = torch.zeros(max(ws_b, 1), dtype=torch.uint8, device="cuda")
        pool.decode(q, out, ws if ws_b else None, scale=float(base.scale))
        torch.cuda.synchronize()
    finally:
        pool.close()
    bound = bound_of(ci)
    assert np.all(np.abs(out.cpu().numpy() - got) <= bound + 2e-3)


def test_chunk_spec_verify_full_size():
    """The speculative-verification workload as the benchmark runs it: every
    row checked."""
    ci = make_chunk_inputs("spec_verify_b32_ctx4k")
    say(f"[chunk] spec verify full size, rows={ci.total_rows}")
    err = assert_parity(ci, gpu_chunk(ci))
    say(f"  max err {err:.2e}")


def test_chunk_prefill_full_size():
    """The 2048-row prefill chunk as the benchmark runs it: every row of both
    sequences against the oracle (one oracle call per sequence, for the
    values and for the bound, run concurrently)."""
    from concurrent.futures import ThreadPoolExecutor
    ci = make_chunk_inputs("prefill_chunk2k_b2_ctx4k")
    base = ci.base
    say(f"[chunk] prefill full size, rows={ci.total_rows}")
    got = gpu_chunk(ci)
    assert np.all(np.isfinite(got))
    B = base.spec.batch
    jobs = [(b, absv) for b in range(B) for absv in (False, True)]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        res = dict(zip(jobs, ex.map(lambda j: oracle_chunk(ci, [j[0]], abs_v=j[1]), jobs)))
    for b in range(B):
        r = rows_of(ci, [b])
        want, bound = res[(b, False)][r], rel_of(ci) * res[(b, True)][r] + 1e-4
        err = np.abs(got[r] - want)
        say(f"  sequence {b}: max err {err.max():.2e}")
        assert np.all(err <= bound), (b, float(err.max()))
        assert err.max() <= 2e-3


def test_chunk_wide_v_at_fp16_range_edge():
    """The wide kernel over a bf16 pool takes V as fp16.  65280, the largest
    finite bf16 magnitude not above fp16's 65504, converts exactly: with V
    entries of +-65280 planted all over the cache, every row stays within the
    derived bound 2^-10 * sum w|V| + 1e-4.  (The absolute 2e-3 bar means
    nothing at these magnitudes: fp32 sums alone err by about 65280 * 2^-24.)"""
    ctx = (300, 700)
    nq = (300, 129)  # up to 1200 rows per (sequence, KV head) at G = 4: the wide kernel
    base = make_inputs(_spec("chunk-v-edge", 128, 8, 2, ctx, 1900))
    v = base.v_pool.copy()
    rng = np.random.default_rng(1901)
    idx = rng.integers(0, v.size, size=v.size // 50)
    v.flat[idx] = np.where(rng.random(idx.size) < 0.5, np.uint16(0x477F), np.uint16(0xC77F))
    base = dataclasses.replace(base, v_pool=v)
    ci = chunk_queries(base, nq, 1902)
    assert rel_of(ci) == REL_F16
    say(f"[chunk] V at the fp16 range edge, rows={ci.total_rows}")
    got = gpu_chunk(ci)
    r = rows_of(ci, range(base.spec.batch))
    want, bound = oracle_chunk(ci)[r], bound_of(ci)[r]
    assert np.all(np.isfinite(got[r]))
    err = np.abs(got[r] - want)
    assert np.all(err <= bound), f"max excess {(err - bound).max():.3e}"
    say(f"  max err {err.max():.2e}, max |out| {np.abs(want).max():.3e}")


# ---------------------------------------------------------------------------
# FP8 E4M3 caches (per-token, per-head scales): codes widened to bf16 in the
# kernels' LDS tiles, the K scale on the score, the V scale on the weight


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 2), (16, 2)])
def test_chunk_fp8_shapes(d, hq, hkv):
    """Short chunks (16- and 32-row workgroups) and long ones (256 rows,
    staged per 64 tokens): full prefills, chunks after a prefix, rows before
    position zero, ragged tails; unused slots hold NaN codes and NaN scales."""
    ctx = (1, 17, 40, 100, 700, 300, 5)
    nq = (1, 5, 40, 7, 300, 129, 9)
    base = make_inputs(_spec("chunk-fp8", d, hq, hkv, ctx, 1500 + d + hq + hkv, kv="fp8_e4m3"),
                       poison=True)
    for rows in (nq, tuple(min(n, 4) for n in nq)):
        ci = chunk_queries(base, rows, 1600 + d + hq + rows[0])
        say(f"[chunk] fp8 d={d} hq={hq} hkv={hkv} rows={ci.total_rows}")
        err = assert_parity(ci, gpu_chunk(ci))
        say(f"  max err {err:.2e}")


@pytest.mark.parametrize("scale", [1.0, -0.3, 0.0])
def test_chunk_fp8_scale_extremes(scale):
    ctx = (1000, 300, 64)
    base = dataclasses.replace(
        make_inputs(_spec("chunk-fp8-scale", 128, 8, 2, ctx, 1700, kv="fp8_e4m3"), poison=True),
        scale=np.float32(scale))
    dev = to_device(base)
    for nq in ((4, 4, 4), (40, 17, 5), (300, 260, 64)):
        ci = chunk_queries(base, nq, 1710 + nq[0])
        say(f"[chunk] fp8 scale={scale} rows/seq={nq}")
        err = assert_parity(ci, gpu_chunk(ci, dev=dev))
        say(f"  max err {err:.2e}")


def test_chunk_fp8_spec_verify_full_size():
    """Speculative verification (4 rows per sequence: 3 drafts and the last
    accepted token) over the full FP8 MHA cache (32 sequences of 8192 tokens,
    32 KV heads): every row against the oracle, sequences checked
    concurrently."""
    from concurrent.futures import ThreadPoolExecutor
    from workloads import NAMED_SPECS
    base = make_inputs(NAMED_SPECS["fp8_mha_b32_ctx8k"])
    ci = chunk_queries(base, [4] * base.spec.batch, 1800)
    say(f"[chunk] fp8 spec verify full size, rows={ci.total_rows}")
    got = gpu_chunk(ci)
    assert np.all(np.isfinite(got))
    B = base.spec.batch
    jobs = [(b, absv) for b in range(B) for absv in (False, True)]
    with ThreadPoolExecutor(max_workers=gpu_host_threads()) as ex:
        res = dict(zip(jobs, ex.map(lambda j: oracle_chunk(ci, [j[0]], abs_v=j[1]), jobs)))
    worst = 0.0
    for b in range(B):
        r = rows_of(ci, [b])
        want, bound = res[(b, False)][r], rel_of(ci) * res[(b, True)][r] + 1e-4
        err = np.abs(got[r] - want)
        worst = max(worst, float(err.max()))
        assert np.all(err <= bound), (b, float(err.max()))
    say(f"  max err {worst:.2e}")
    assert worst <= 2e-3
