"""Seeded inputs for the INT8 / INT4 (KIVI-style) KV cache.

The pool is drawn directly in its stored form -- uniform codes, positive
fp16 scales and fp16 minimums of the size that puts values in a few units
around zero, bf16 residual rows -- so no quantisation arithmetic happens
here (the quantiser is the cache write's, tested on its own).  Shapes and
block placement come from a decode workload (``make_inputs``): same table,
lengths and query.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .synthetic import Inputs, _to_bf16_bits, make_inputs

BLOCK = 16


@dataclass
class KiviInputs:
    base: Inputs          # table, lengths, q (bf16), scale, spec
    bits: int
    k_codes: np.ndarray   # uint8 [N][Hkv][16][d * bits / 8] (head-major)
    v_codes: np.ndarray
    k_params: np.ndarray  # float16 [N][Hkv][2][d]
    v_params: np.ndarray  # float16 [N][Hkv][16][2]
    res_k: np.ndarray     # uint16 (bf16 bits) [B][16][Hkv][d]
    res_v: np.ndarray


def _pack4(c):
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def kivi_state(rng, n_blocks, batch, hkv, d, bits):
    L = (1 << bits) - 1
    kc = rng.integers(0, L + 1, size=(n_blocks, hkv, BLOCK, d), dtype=np.uint8)
    vc = rng.integers(0, L + 1, size=(n_blocks, hkv, BLOCK, d), dtype=np.uint8)
    kp = np.empty((n_blocks, hkv, 2, d), np.float16)
    kp[:, :, 0] = (np.abs(rng.standard_normal((n_blocks, hkv, d), dtype=np.float32)) * 6 / L
                   + 1e-3).astype(np.float16)
    kp[:, :, 1] = (rng.standard_normal((n_blocks, hkv, d), dtype=np.float32) - 3).astype(np.float16)
    vp = np.empty((n_blocks, hkv, BLOCK, 2), np.float16)
    vp[..., 0] = (np.abs(rng.standard_normal((n_blocks, hkv, BLOCK), dtype=np.float32)) * 6 / L
                  + 1e-3).astype(np.float16)
    vp[..., 1] = (rng.standard_normal((n_blocks, hkv, BLOCK), dtype=np.float32) - 3).astype(np.float16)
    if bits == 4:
        kc, vc = _pack4(kc), _pack4(vc)
    rk = _to_bf16_bits(rng.standard_normal((batch, BLOCK, hkv, d), dtype=np.float32))
    rv = _to_bf16_bits(rng.standard_normal((batch, BLOCK, hkv, d), dtype=np.float32))
    return kc, vc, kp, vp, rk, rv


def make_kivi_inputs(spec, bits: int, seed: int) -> KiviInputs:
    """A bf16-shaped decode workload ``spec`` with its pool drawn as KIVI
    codes and parameters (the spec's own pool values are not used)."""
    base = make_inputs(spec)
    s = base.spec
    rng = np.random.Generator(np.random.PCG64(seed))
    kc, vc, kp, vp, rk, rv = kivi_state(rng, base.num_blocks, s.batch, s.num_kv_heads,
                                        s.head_dim, bits)
    return KiviInputs(base=base, bits=bits, k_codes=kc, v_codes=vc, k_params=kp, v_params=vp,
                      res_k=rk, res_v=rv)
