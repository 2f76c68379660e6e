#!/usr/bin/env python3
"""Decode-attention bandwidth benchmark on one MI355X.

One step = one decode-attention call (one kernel launch) for one layer of
the Llama-3-8B-shaped workload: batch 32, 32 query / 8 KV heads, head_dim
128, every context 4096 tokens, bf16 KV in 16-token blocks placed by a
seeded random permutation of an 8192-block pool.  Inputs are synthetic and
resident in HBM before timing starts.  The timed loop cycles over
``--layers`` independent copies of the KV pool (different layers' caches),
so no step finds its 512 MiB of KV in the 256 MB Infinity Cache that the
previous steps filled.

Printed: one JSON line on stdout.  ``value`` is KV bytes read per step
(unique cached tokens x KV heads x head_dim x 2 (K and V) x element bytes)
over the wall-clock time per step of the K timed steps.  ``roofline`` prices
the attention kernel alone (HIP events around the launches of every
``--layers``-th step of the timed loop) against MI355X's 8 TB/s HBM peak.
``cpu_baseline`` times the float64 CPU oracle on a bounded sample of the
same workload.
"""

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention KV-read TB/s, % of 8 TB/s HBM peak; µs per decode step"
HBM_PEAK_GBS = 8000.0
KERNEL_SRCS = [os.path.join(ROOT, "paged_kv_cache_398_amd", "csrc", f)
               for f in ("pa_kernels.hip", "pa_internal.h", "pa_mfma.h")]


def traffic_file(workload):
    """Committed HBM-counter figures of the attention kernel on ``workload``."""
    return os.path.join(ROOT, "profiles", f"traffic_attention_kernel_{workload}.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha():
    """Hash of the attention kernel's sources (kernel file and the headers it includes)."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kv_bytes(inp):
    s = inp.spec
    eb = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[s.kv_dtype]
    per_token = s.num_kv_heads * s.head_dim * 2 * eb
    if s.kv_dtype == "fp8_e4m3":
        per_token += s.num_kv_heads * 2 * 4
    return inp.unique_tokens * per_token


def stored_traffic(workload):
    """HBM bytes per launch of the attention kernel on ``workload`` from the
    committed counter runs, if taken on that workload with the current
    kernel sources."""
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_sha() or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch")


def roofline_hbm(nbytes, kernel_s, kernel="attention_kernel", traffic=None):
    a = nbytes / kernel_s / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(a / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
            "kernel_us": round(kernel_s * 1e6, 2)}


def decode_leg(name, steps, warmup, layers=1, separate=False, main_inp=None):
    """Time pa_decode_run / pa_decode_fp8_run on a named workload.

    ``layers`` KV pools are cycled (so that no step finds its KV in the
    256 MB Infinity Cache left by the previous one), each warmed by one run
    first; then ``warmup`` untimed and ``steps`` timed back-to-back steps.
    Returned: wall clock per step over the timed steps, and the attention
    kernel's average duration from the library's HIP events around the
    kernel on the steps that use pool 0.  Pools come from ``main_inp`` (host
    arrays) when given, else are drawn on the GPU (make_device_workload).
    ``separate``: K and V as two allocations instead of the recommended
    one-buffer placement (pa_kv_pool_placement)."""
    import numpy as np
    import torch

    import paged_kv_cache_398_amd as pa
    from workloads import make_device_workload, named_spec
    from workloads.device import to_device

    s = named_spec(name)
    w = to_device(main_inp) if main_inp is not None else make_device_workload(s)
    n_blocks = int(w.k_pool.shape[0])
    ctx_host = main_inp.context_lens if main_inp is not None else w.ctx_host
    max_ctx = int(ctx_host.max())
    pools = []
    for r in range(layers):
        if separate:
            k, v = torch.empty_like(w.k_pool), torch.empty_like(w.v_pool)
        else:
            k, v = pa.allocate_kv_pools(n_blocks, s.num_kv_heads, s.head_dim, s.kv_dtype)
        k.copy_(w.k_pool.view(k.dtype))
        v.copy_(w.v_pool.view(v.dtype))
        ks = None if w.k_scale is None else (w.k_scale if r == 0 else w.k_scale.clone())
        vs = None if w.v_scale is None else (w.v_scale if r == 0 else w.v_scale.clone())
        p = pa.PagedKVPool(k, v, s.kv_dtype, ks, vs)
        p.set_block_table(w.block_table, w.context_lens, max_ctx)
        pools.append(p)
    q = w.q
    scale = float(main_inp.scale if main_inp is not None else w.scale)
    ws = pools[0].new_workspace(s.num_q_heads)
    out = torch.empty((s.batch, s.num_q_heads, s.head_dim), dtype=torch.float32, device="cuda")
    R = len(pools)

    # The timed steps call the C ABI through the binding with the arguments
    # marshalled once, as a serving engine would; PagedKVPool.decode, which
    # checks every tensor on every call (tens of us of Python per step), runs
    # the untimed steps, so the arguments are validated before timing.
    run = pa.pa_decode_fp8_run if s.kv_dtype == "fp8_e4m3" else pa.pa_decode_run
    qd = "f32" if s.kv_dtype == "f32" else "bf16"
    stream = int(torch.cuda.current_stream().cuda_stream)
    ws_ptr, ws_bytes = (None, 0) if ws is None else (ws.data_ptr(), ws.numel())
    call_args = [(p.handle, q.data_ptr(), qd, s.num_q_heads, scale, out.data_ptr(), ws_ptr,
                  ws_bytes, stream) for p in pools]

    def checked_step(i):
        pools[i % R].decode(q, out, ws, scale=scale)

    def step(i):
        run(*call_args[i % R])

    for i in range(R + warmup):  # every pool once, then the warm-up steps
        checked_step(i)
    torch.cuda.synchronize()
    n_prof = (steps + R - 1) // R
    pa.pa_profile_enable(pools[0].handle, n_prof)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern_ms = pa.pa_profile_read(pools[0].handle, n_prof)
    pa.pa_profile_enable(pools[0].handle, 0)
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError(f"non-finite output ({name})")
    eb = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[s.kv_dtype]
    shared = (s.shared_prefix_seqs - 1) * s.shared_prefix_tokens if s.shared_prefix_seqs > 1 else 0
    unique = int(ctx_host.astype(np.int64).sum()) - shared
    per_token = s.num_kv_heads * s.head_dim * 2 * eb + (s.num_kv_heads * 2 * 4 if eb == 1 else 0)
    nbytes = unique * per_token
    sec = (t1 - t0) / steps
    kern = statistics.fmean(kern_ms) * 1e-3
    res = {
        "workload": name, "kv_dtype": s.kv_dtype, "batch": s.batch,
        "max_context_tokens": max_ctx, "kv_bytes_per_step": nbytes,
        "steps": steps, "layers_cycled": R, "us_per_step": round(sec * 1e6, 2),
        "tb_s": round(nbytes / sec / 1e12, 4),
        "pct_of_hbm_peak": round(100 * nbytes / sec / 1e9 / HBM_PEAK_GBS, 2),
        "workgroups": pools[0].workgroups(),
        "kv_heads_per_workgroup_equal_lengths": pools[0].heads_per_workgroup(),
        "kv_placement": "two separate allocations" if separate else
                        "one buffer, V at a 2 KiB boundary + 256 B (pa_kv_pool_placement)",
        "roofline": roofline_hbm(nbytes, kern, traffic=stored_traffic(name) if not separate
                                 else None),
        "kernel_event_pairs": len(kern_ms),
    }
    log(f"{name}{' (separate K/V)' if separate else ''}: {sec * 1e6:.1f} us/step, "
        f"{res['tb_s']:.3f} TB/s; kernel {kern * 1e6:.1f} us "
        f"({100 * res['roofline']['frac']:.1f}% of HBM peak)")
    for p in pools:
        p.close()
    return res


def cpu_baseline(inp, seconds):
    """The float64 oracle on whole sequences of the workload, ~``seconds``."""
    import numpy as np
    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = 1
    s = inp.spec
    eb = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[s.kv_dtype]
    done_tokens, n_seq = 0, 0
    t0 = time.perf_counter()
    b = 0
    while True:
        oracle.paged_decode_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                      inp.context_lens, inp.scale, kv_dtype=s.kv_dtype,
                                      q_dtype=s.q_dtype, k_scale=inp.k_scale,
                                      v_scale=inp.v_scale, seqs=[b])
        done_tokens += int(inp.context_lens[b])
        n_seq += 1
        b = (b + 1) % s.batch
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    nbytes = done_tokens * s.num_kv_heads * s.head_dim * 2 * eb
    return {
        "value": nbytes / dt / 1e12, "unit": "TB/s", "cores": int(threads), "kind": "oracle",
        "host_cpus": os.cpu_count(),
        "sample": f"{n_seq} whole sequences ({done_tokens} tokens x {s.num_kv_heads} KV heads) "
                  f"of the same workload in {dt:.1f} s; float64 numpy, BLAS threads={threads}",
        "seconds_per_step_equivalent": dt * inp.logical_tokens / max(done_tokens, 1),
    }


MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix peak


def chunk_flops(ci):
    """Algorithmic flops of a chunk: 4 d per (row, query head, visible token)
    (QK^T and PV, a multiply and an add each)."""
    import numpy as np
    s = ci.base.spec
    tot = 0
    for b in range(s.batch):
        n, ctx = int(ci.q_lens[b]), int(ci.base.context_lens[b])
        tot += int(np.clip(np.arange(ctx - n, ctx) + 1, 0, None).sum())
    return 4 * s.head_dim * s.num_q_heads * tot


def chunk_leg(name, iters, main_inp, main_pools):
    """Time pa_chunk_run on a named chunk workload: HIP events around every
    launch (on torch's current stream, the one the launches use)."""
    import numpy as np
    import torch

    import paged_kv_cache_398_amd as pa
    from workloads import CHUNK_SPECS, chunk_queries, make_chunk_inputs
    from workloads.device import to_device

    base_name, over, n, seed = CHUNK_SPECS[name]
    own = []
    if not over and main_inp is not None and main_inp.spec.name == base_name:
        ci = chunk_queries(main_inp, [n] * main_inp.spec.batch, seed)
        pools = main_pools  # the decode leg's cycled KV pools, same cache
    else:
        ci = make_chunk_inputs(name)
        dev = to_device(ci.base)
        bs = ci.base.spec
        k, v = pa.allocate_kv_pools(ci.base.num_blocks, bs.num_kv_heads, bs.head_dim, "bf16")
        k.copy_(dev.k_pool)
        v.copy_(dev.v_pool)
        p = pa.PagedKVPool(k, v, "bf16")
        p.set_block_table(dev.block_table, dev.context_lens, ci.base.max_context_len)
        own = pools = [p]
    s = ci.base.spec
    q = torch.from_numpy(ci.q.view(np.int16)).view(torch.bfloat16).cuda()
    qs = torch.from_numpy(ci.q_start).cuda()
    out = torch.empty((ci.total_rows, s.num_q_heads, s.head_dim), dtype=torch.float32,
                      device="cuda")
    scale = float(ci.base.scale)
    for i in range(5):
        pools[i % len(pools)].chunk(q, qs, ci.max_q_len, out, scale=scale)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for i, (e0, e1) in enumerate(evs):
        e0.record()
        pools[i % len(pools)].chunk(q, qs, ci.max_q_len, out, scale=scale)
        e1.record()
    torch.cuda.synchronize()
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError(f"non-finite chunk output ({name})")
    us = statistics.fmean(e0.elapsed_time(e1) for e0, e1 in evs) * 1e3
    rows, per_head = pa.pa_chunk_tiles(pools[0].handle, s.num_q_heads, ci.max_q_len)
    for p in own:
        p.close()
    eb = 2
    nbytes = sum(int(ci.base.context_lens[b]) for b in range(s.batch)) * s.num_kv_heads * \
        s.head_dim * 2 * eb
    flops = chunk_flops(ci)
    ridge = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)  # flop per byte
    hbm_bound = flops / nbytes < ridge
    res = {
        "workload": name, "rows_per_sequence": n, "batch": s.batch,
        "context_tokens": int(ci.base.max_context_len), "kernel_us": round(us, 2),
        "kv_bytes": nbytes, "flops": flops, "iters": iters,
        "rows_per_workgroup": rows, "workgroups": s.batch * s.num_kv_heads * per_head,
        "pools_cycled": len(pools),
    }
    # 256-row workgroups are the wide kernel's (long chunks)
    kname = "chunk_wide_kernel" if rows >= 256 else "chunk_kernel"
    if hbm_bound:
        a = nbytes / (us * 1e-6) / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(a / HBM_PEAK_GBS, 4),
                           "kernel": kname}
    else:
        a = flops / (us * 1e-6) / 1e12
        res["roofline"] = {"bound": "mfma", "achieved": round(a, 1),
                           "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                           "frac": round(a / MFMA_BF16_PEAK_TFS, 4), "kernel": kname}
    log(f"chunk {name}: {us:.1f} us, {res['roofline']['achieved']} "
        f"{res['roofline']['unit']} ({100 * res['roofline']['frac']:.1f}% of peak)")
    return res


def kivi_leg(bits, steps, main_inp, layers):
    """Decode over the INT8 / INT4 (KIVI-style) pool of the decode workload's
    shape: same table, lengths and queries, codes and fp16 parameters drawn
    directly; ``layers`` pools cycled; the library's HIP events around
    each launch on the first pool."""
    import numpy as np
    import torch

    import paged_kv_cache_398_amd as pa
    from workloads import kivi_state

    s = main_inp.spec
    rng = np.random.Generator(np.random.PCG64(398400 + bits))
    pools, keep = [], []
    for r in range(layers):
        kc, vc, kp, vp, rk, rv = kivi_state(rng, main_inp.num_blocks, s.batch, s.num_kv_heads,
                                            s.head_dim, bits)
        t = [torch.from_numpy(x).cuda() for x in (kc, vc, kp, vp)]
        res = [torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() for x in (rk, rv)]
        p = pa.KiviKVPool(*t, bits)
        p.set_residual(*res)
        keep.append((t, res))
        pools.append(p)
    tb = torch.from_numpy(main_inp.block_table).cuda()
    ln = torch.from_numpy(main_inp.context_lens).cuda()
    for p in pools:
        p.set_block_table(tb, ln, main_inp.max_context_len)
    q = torch.from_numpy(main_inp.q.view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.empty((s.batch, s.num_q_heads, s.head_dim), dtype=torch.float32, device="cuda")
    scale = float(main_inp.scale)
    for i in range(10):
        pools[i % layers].decode(q, out, scale=scale)
    torch.cuda.synchronize()
    n_prof = (steps + layers - 1) // layers
    pa.pa_profile_enable(pools[0].handle, n_prof)
    t0 = time.perf_counter()
    for i in range(steps):
        pools[i % layers].decode(q, out, scale=scale)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern = pa.pa_profile_read(pools[0].handle, n_prof)
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("non-finite INT8/INT4 output")
    for p in pools:
        p.close()
    # bytes a step must read: codes and parameters of the full blocks, bf16
    # residual rows of the partial ones
    hkv, d = s.num_kv_heads, s.head_dim
    per_block = 2 * 16 * hkv * d * bits // 8 + hkv * 2 * d * 2 + hkv * 16 * 4
    nbytes = 0
    for n in main_inp.context_lens.tolist():
        nbytes += (n // 16) * per_block + (n % 16) * hkv * d * 2 * 2
    bf16_bytes = int(main_inp.context_lens.astype(np.int64).sum()) * hkv * d * 2 * 2
    us_step = (t1 - t0) / steps * 1e6
    kus = statistics.fmean(kern) * 1e3
    a = nbytes / (kus * 1e-6) / 1e9
    res = {"bits": bits, "us_per_step": round(us_step, 2), "kernel_us": round(kus, 2),
           "bytes_per_step": nbytes, "bf16_bytes_of_same_cache": bf16_bytes,
           "bf16_equivalent_tb_s": round(bf16_bytes / (us_step * 1e-6) / 1e12, 3),
           "roofline": {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(a / HBM_PEAK_GBS, 4),
                        "kernel": "kivi_attention_kernel"}}
    log(f"INT{bits} KIVI decode: {us_step:.1f} us/step, kernel {kus:.1f} us "
        f"({a:.0f} GB/s of its {nbytes / 1e6:.0f} MB; bf16-equivalent "
        f"{res['bf16_equivalent_tb_s']} TB/s)")
    return res


def block_manager_leg(iters):
    """Host cost of the block manager per operation (through the binding),
    and the block-copy kernel's bandwidth on a batch of copies."""
    import numpy as np
    import torch

    import paged_kv_cache_398_amd as pa

    rng = np.random.Generator(np.random.PCG64(398200))
    n_blocks = 65536
    m = pa.BlockManager(n_blocks, True)
    prompts = [rng.integers(0, 1000, size=int(n)).tolist() for n in rng.integers(100, 2000, 64)]
    t0 = time.perf_counter()
    for i, p in enumerate(prompts):
        m.add(i, p)
    t1 = time.perf_counter()
    n_app = 0
    for _ in range(iters):
        for i in range(len(prompts)):
            m.append(i, 7)
            n_app += 1
    t2 = time.perf_counter()
    for i in range(len(prompts)):
        m.free(i)
    t3 = time.perf_counter()
    m.close()
    # block copies: 4096 distinct (src, dst) pairs of a bf16 Llama-3-8B-shaped pool
    hkv, d, n_copy = 8, 128, 4096
    k = torch.empty((2 * n_copy, 16, hkv, d), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    pool = pa.PagedKVPool(k, v, "bf16")
    perm = torch.randperm(2 * n_copy, generator=torch.Generator().manual_seed(7)).to(torch.int32)
    pairs = perm.view(n_copy, 2).contiguous().cuda()
    for _ in range(3):
        pa.pa_copy_blocks(pool.handle, pairs, n_copy)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(20)]
    for e0, e1 in evs:
        e0.record()
        pa.pa_copy_blocks(pool.handle, pairs, n_copy)
        e1.record()
    torch.cuda.synchronize()
    us = statistics.fmean(e0.elapsed_time(e1) for e0, e1 in evs) * 1e3
    pool.close()
    nbytes = n_copy * 16 * hkv * d * 2 * 2 * 2  # K and V, read and written
    a = nbytes / (us * 1e-6) / 1e9
    res = {
        "add_us_per_token": round((t1 - t0) * 1e6 / sum(len(p) for p in prompts), 4),
        "append_us": round((t2 - t1) * 1e6 / n_app, 3),
        "free_us_per_sequence": round((t3 - t2) * 1e6 / len(prompts), 2),
        "note": "host time per operation through the Python binding (ctypes call included)",
        "copy_blocks": {"pairs": n_copy, "kernel_us": round(us, 2), "bytes": nbytes,
                        "roofline": {"bound": "hbm", "achieved": round(a, 1),
                                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": round(a / HBM_PEAK_GBS, 4),
                                     "kernel": "copy_blocks_kernel"}},
    }
    log(f"block manager: append {res['append_us']} us; copy_blocks {us:.1f} us "
        f"({a:.0f} GB/s)")
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3_8b_b32_ctx4k")
    ap.add_argument("--layers", type=int, default=8,
                    help="independent KV pools cycled by the timed loop")
    ap.add_argument("--workgroups", type=int, default=0, help="0: automatic")
    ap.add_argument("--heads-per-workgroup", type=int, default=0, help="0: automatic")
    ap.add_argument("--cold-iters", type=int, default=30,
                    help="extra steps timed after a 1 GiB cache flush each")
    ap.add_argument("--append-iters", type=int, default=100,
                    help="timed launches of the cache write (0: skip)")
    ap.add_argument("--chunk-iters", type=int, default=50,
                    help="timed launches of each multi-token chunk workload (0: skip)")
    ap.add_argument("--kivi-steps", type=int, default=200,
                    help="timed steps of each INT8/INT4 decode leg (0: skip)")
    ap.add_argument("--bm-iters", type=int, default=20,
                    help="append rounds of the block-manager leg (0: skip)")
    ap.add_argument("--decode-steps", type=int, default=20,
                    help="timed steps of each other named decode workload, and of the "
                         "main workload with K and V in separate allocations (0: skip)")
    ap.add_argument("--warm-ms", type=float, default=300.0,
                    help="untimed steps for at least this long before the timed ones")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="after the steps, run one plain device copy of this many MiB "
                         "(reference for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_398_amd as pa
    from workloads import make_inputs, named_spec
    from workloads.device import to_device

    pa.load_library()  # raises if libpa.so is not built
    log(f"generating {args.workload}")
    inp = make_inputs(named_spec(args.workload))
    s = inp.spec
    dev = to_device(inp)
    log("inputs resident on the GPU")
    R = max(1, args.layers)
    pools = []
    for r in range(R):
        # each layer's K and V pools in one buffer, placed as the library
        # recommends (pa_kv_pool_placement: V shifted 256 B against K)
        k, v = pa.allocate_kv_pools(inp.num_blocks, s.num_kv_heads, s.head_dim, s.kv_dtype)
        k.copy_(dev.k_pool.view(k.dtype))
        v.copy_(dev.v_pool.view(v.dtype))
        ks = None if dev.k_scale is None else (dev.k_scale if r == 0 else dev.k_scale.clone())
        vs = None if dev.v_scale is None else (dev.v_scale if r == 0 else dev.v_scale.clone())
        p = pa.PagedKVPool(k, v, s.kv_dtype, ks, vs)
        p.set_block_table(dev.block_table, dev.context_lens, inp.max_context_len)
        if args.workgroups:
            p.set_workgroups(args.workgroups)
        if args.heads_per_workgroup:
            p.set_heads_per_workgroup(args.heads_per_workgroup)
        pools.append(p)
    nwg = pools[0].workgroups()
    hc = pools[0].heads_per_workgroup()
    ws_bytes = pools[0].workspace_bytes(s.num_q_heads)
    ws = pools[0].new_workspace(s.num_q_heads)
    out = torch.empty((s.batch, s.num_q_heads, s.head_dim), dtype=torch.float32, device="cuda")
    scale = float(inp.scale)

    # The timed steps call the C ABI through the binding with the arguments
    # marshalled once, as a serving engine would; PagedKVPool.decode, which
    # checks every tensor on every call (tens of us of Python per step), runs
    # the first untimed steps, so the arguments are validated before timing.
    run = pa.pa_decode_fp8_run if s.kv_dtype == "fp8_e4m3" else pa.pa_decode_run
    qd = "f32" if s.kv_dtype == "f32" else "bf16"
    stream = int(torch.cuda.current_stream().cuda_stream)
    ws_ptr = None if ws is None else ws.data_ptr()
    call_args = [(p.handle, dev.q.data_ptr(), qd, s.num_q_heads, scale, out.data_ptr(), ws_ptr,
                  ws_bytes, stream) for p in pools]

    def checked_step(i):
        pools[i % R].decode(dev.q, out, ws, scale=scale)

    def step(i):
        run(*call_args[i % R])

    # every pool runs once before the warm-up steps, so that no first use of
    # a pool falls inside the timed region whatever --warmup is; then more
    # untimed steps until --warm-ms of them have run, so that the timed
    # region does not start while the GPU's clocks still ramp up from the
    # idle of the input generation
    for i in range(R + args.warmup):
        checked_step(i)
    torch.cuda.synchronize()
    warm_runs = R + args.warmup
    t_w = time.perf_counter()
    while (time.perf_counter() - t_w) * 1e3 < args.warm_ms:
        for i in range(R):
            step(i)
        torch.cuda.synchronize()
        warm_runs += R
    # HIP events around the kernels of the steps that use pool 0 (every R-th
    # step of the timed region): recording them on every step would itself
    # add several microseconds between back-to-back launches.
    n_prof = (args.steps + R - 1) // R
    pa.pa_profile_enable(pools[0].handle, n_prof)
    log(f"timing {args.steps} steps ({nwg} workgroups, {hc} KV heads per workgroup, "
        f"{R} layers cycled, events on every {R}-th step)")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern_ms = pa.pa_profile_read(pools[0].handle, n_prof)
    pa.pa_profile_enable(pools[0].handle, 0)
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("non-finite output")

    nbytes = kv_bytes(inp)
    sec_per_step = (t1 - t0) / args.steps
    tbs = nbytes / sec_per_step / 1e12
    kern_avg = statistics.fmean(kern_ms) * 1e-3
    achieved = nbytes / kern_avg / 1e9
    log(f"{sec_per_step * 1e6:.1f} us/step, {tbs:.3f} TB/s; attention kernel "
        f"{kern_avg * 1e6:.1f} us ({achieved:.0f} GB/s) over {len(kern_ms)} event pairs")

    # cold steps: every step after reading 1 GiB elsewhere, which evicts the
    # KV from the caches without leaving dirty lines behind (flush outside
    # the events)
    cold = []
    if args.cold_iters > 0:
        flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(args.cold_iters):
            flush.sum()
            ev0.record()
            step(i)
            ev1.record()
            ev1.synchronize()
            cold.append(ev0.elapsed_time(ev1) * 1e-3)
        del flush
    # the write half of a decode step: each sequence's new token into the
    # cache (one launch), timed on its own with HIP events
    append = None
    if args.append_iters > 0:
        g = torch.Generator(device="cpu").manual_seed(398)
        src_dtype = torch.float32 if s.kv_dtype == "f32" else torch.bfloat16
        k_new = torch.randn((s.batch, s.num_kv_heads, s.head_dim), generator=g).to(src_dtype).cuda()
        v_new = torch.randn((s.batch, s.num_kv_heads, s.head_dim), generator=g).to(src_dtype).cuda()
        for _ in range(5):
            pools[0].append(k_new, v_new)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(args.append_iters):
            pools[0].append(k_new, v_new)
        ev1.record()
        ev1.synchronize()
        us = ev0.elapsed_time(ev1) * 1e3 / args.append_iters
        eb = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[s.kv_dtype]
        written = s.batch * s.num_kv_heads * (s.head_dim * eb + (4 if eb == 1 else 0)) * 2
        append = {"us": round(us, 2), "bytes_written": written, "iters": args.append_iters,
                  "note": "pa_cache_append of one new token per sequence, back-to-back launches"}
        log(f"cache write: {us:.2f} us per launch")
    # the other named decode workloads, and the main one with K and V in two
    # separate allocations (the usual engine layout)
    others = []
    if args.decode_steps > 0:
        others.append(decode_leg(s.name, args.decode_steps, args.warmup, layers=R,
                                 separate=True, main_inp=inp))
        for name in ("continuous_batch_b64", "long_ctx_b4_128k", "fp8_mha_b32_ctx8k"):
            if name != s.name:
                torch.cuda.empty_cache()
                others.append(decode_leg(name, args.decode_steps, args.warmup))
        torch.cuda.empty_cache()
    chunk = None
    if args.chunk_iters > 0:
        chunk = [chunk_leg(name, args.chunk_iters, inp, pools)
                 for name in ("spec_verify_b32_ctx4k", "prefill_chunk2k_b2_ctx4k")]
    block_mgr = block_manager_leg(args.bm_iters) if args.bm_iters > 0 else None
    kivi_res = None
    if args.kivi_steps > 0 and s.kv_dtype == "bf16":
        kivi_res = [kivi_leg(bits, args.kivi_steps, inp, min(R, 3)) for bits in (8, 4)]
    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib << 18  # float32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calibration_copy_mib} MiB read + written")
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for ~{args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(inp, args.cpu_seconds)

    traffic = stored_traffic(s.name)
    res = {
        "metric": METRIC,
        "value": round(tbs, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec_per_step * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": s.name, "batch": s.batch, "q_heads": s.num_q_heads,
            "kv_heads": s.num_kv_heads, "head_dim": s.head_dim,
            "context_tokens": int(inp.max_context_len), "block_size": 16,
            "kv_dtype": s.kv_dtype, "q_dtype": s.q_dtype, "out_dtype": "f32",
            "kv_bytes_per_step": nbytes, "workgroups": nwg,
            "layers_cycled": R, "kv_heads_per_workgroup": hc,
            "kv_placement": "K and V pools of a layer in one buffer, V at a 2 KiB "
                            "boundary + 256 B (pa_kv_pool_placement)",
            "untimed_runs_before_timing": warm_runs,
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "attention_kernel", "kernel_us": round(kern_avg * 1e6, 2),
        },
        "us_per_step": round(sec_per_step * 1e6, 2),
        "pct_of_hbm_peak": round(100 * tbs * 1e3 / HBM_PEAK_GBS, 2),
        "cold": None if not cold else {
            "median_step_us": round(statistics.median(cold) * 1e6, 2),
            "p10_step_us": round(float(np.percentile(cold, 10)) * 1e6, 2),
            "p90_step_us": round(float(np.percentile(cold, 90)) * 1e6, 2),
            "tb_s": round(nbytes / statistics.median(cold) / 1e12, 4),
            "iters": len(cold),
            "note": "one step after reading 1 GiB elsewhere; event-timed step",
        },
        "cpu_baseline": cpu,
        "decode_workloads": others,
        "cache_append": append,
        "chunk": chunk,
        "block_manager": block_mgr,
        "int_kv": kivi_res,
    }
    print(json.dumps(res), flush=True)
    for p in pools:
        p.close()


if __name__ == "__main__":
    main()
