"""Pins of the INT8 / INT4 (KIVI-style) KV oracle, oracle/kivi.py.

* Quantiser: codes in range and within the error bound; values already on a
  grid are reproduced exactly (codes, scale and min); a constant group.
* KIVI's grouping ("大模型推理为何这么慢" section on KV cache quantisation):
  an outlier channel of K changes only that channel's parameters and codes;
  an outlier token of V changes only that token's.
* INT4 packing: a worked example (codes 1, 2, 15, 0 -> bytes 0x21, 0x0F) and
  round trips.
* Attention: equals the decode oracle on a pool dequantised independently
  (vectorised over all blocks, residual rows placed in extra blocks); and,
  after appending tokens one by one from an empty cache, equals torch's
  float64 SDPA over contiguous K/V made of the quantised-then-dequantised
  full blocks and the exact residual tokens.
``test_planted_kivi_mistakes_are_caught`` plants mistakes in the oracle.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import kivi
from oracle.formats import bf16_bits_to_f64

BLOCK = 16


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def random_state(rng, N, B, hkv, d, bits):
    L = (1 << bits) - 1
    kc = rng.integers(0, L + 1, size=(N, hkv, BLOCK, d), dtype=np.uint8)
    vc = rng.integers(0, L + 1, size=(N, hkv, BLOCK, d), dtype=np.uint8)
    kp = np.empty((N, hkv, 2, d), np.float16)
    kp[:, :, 0] = (np.abs(rng.standard_normal((N, hkv, d))) * 6 / L + 1e-3).astype(np.float16)
    kp[:, :, 1] = (rng.standard_normal((N, hkv, d)) - 3).astype(np.float16)
    vp = np.empty((N, hkv, BLOCK, 2), np.float16)
    vp[..., 0] = (np.abs(rng.standard_normal((N, hkv, BLOCK))) * 6 / L + 1e-3).astype(np.float16)
    vp[..., 1] = (rng.standard_normal((N, hkv, BLOCK)) - 3).astype(np.float16)
    if bits == 4:
        kc, vc = kivi.pack_int4(kc), kivi.pack_int4(vc)
    rk = _bf16_bits(rng.standard_normal((B, BLOCK, hkv, d)))
    rv = _bf16_bits(rng.standard_normal((B, BLOCK, hkv, d)))
    return kc, vc, kp, vp, rk, rv


# ---------------------------------------------------------------------------
# pins


def pin_quantiser_bound():
    rng = _rng(1)
    for bits in (8, 4):
        L = (1 << bits) - 1
        for _ in range(200):
            x = (rng.standard_normal(int(rng.integers(2, 130))) * rng.uniform(0.01, 50)
                 + rng.uniform(-20, 20)).astype(np.float32)
            c, s, m = kivi.quantize_group(x, bits)
            assert c.dtype == np.uint8 and c.max() <= L
            err = np.abs(x.astype(np.float64) - kivi.dequantize(c, s, m))
            lo = np.float64(x.min())
            bound = float(s) * (0.5 + L * 2.0 ** -10) + abs(lo - float(m)) + 1e-6 * np.abs(x).max()
            assert err.max() <= bound


def pin_values_on_the_grid_are_exact():
    rng = _rng(2)
    for bits in (8, 4):
        L = (1 << bits) - 1
        for _ in range(100):
            s = np.float16(rng.uniform(0.01, 2.0))
            m = np.float16(rng.uniform(-10, 10))
            k = rng.integers(0, L + 1, size=40)
            k[0], k[1] = 0, L  # min and max attained
            x = (k * np.float32(s) + np.float32(m)).astype(np.float32)
            if not np.all(x.astype(np.float64) == k * np.float64(s) + np.float64(m)):
                continue  # not exact in float32: skip this draw
            c, s2, m2 = kivi.quantize_group(x, bits)
            assert s2 == s and m2 == m and np.array_equal(c, k)


def pin_constant_group():
    c, s, m = kivi.quantize_group(np.full(16, 2.7, np.float32), 8)
    assert s == np.float16(1.0) and m == np.float16(2.7) and not c.any()


def pin_k_per_channel_and_v_per_token():
    rng = _rng(3)
    k = rng.standard_normal((BLOCK, 32)).astype(np.float32)
    v = rng.standard_normal((BLOCK, 32)).astype(np.float32)
    kc, kp, vc, vp = kivi.quantize_block(k, v, 8)
    k2, v2 = k.copy(), v.copy()
    k2[:, 5] *= 8  # an outlier channel of K
    v2[3] *= 8     # an outlier token of V
    kc2, kp2, vc2, vp2 = kivi.quantize_block(k2, v2, 8)
    other_c = [c for c in range(32) if c != 5]
    other_t = [t for t in range(BLOCK) if t != 3]
    assert np.array_equal(kc2[:, other_c], kc[:, other_c])
    assert np.array_equal(kp2[:, other_c], kp[:, other_c])
    assert not np.array_equal(kp2[:, 5], kp[:, 5])
    assert np.array_equal(vc2[other_t], vc[other_t]) and np.array_equal(vp2[other_t], vp[other_t])
    assert not np.array_equal(vp2[3], vp[3])


def pin_int4_packing():
    assert kivi.pack_int4(np.array([1, 2, 15, 0], np.uint8)).tolist() == [0x21, 0x0F]
    assert kivi.unpack_int4(np.array([0x21, 0x0F], np.uint8)).tolist() == [1, 2, 15, 0]
    c = _rng(4).integers(0, 16, size=(3, 5, 64), dtype=np.uint8)
    assert np.array_equal(kivi.unpack_int4(kivi.pack_int4(c)), c)


def pin_attention_over_independently_dequantised_pool():
    rng = _rng(5)
    for bits in (8, 4):
        N, B, hkv, hq, d = 20, 4, 2, 8, 32
        kc, vc, kp, vp, rk, rv = random_state(rng, N, B, hkv, d, bits)
        lens = np.array([37, 16, 5, 64])
        table = np.full((B, 5), -1, np.int32)
        perm = rng.permutation(N)
        used = 0
        for b, n in enumerate(lens):
            for j in range(n // BLOCK):
                table[b, j] = perm[used]
                used += 1
        q = _bf16_bits(rng.standard_normal((B, hq, d)))
        got = kivi.kivi_decode_attention(q, kc, vc, kp, vp, rk, rv, table, lens, 0.2, bits)
        # independent: dequantise the whole pool at once, residual rows as
        # extra blocks N..N+B-1 appended to each table
        codes_k = kivi.unpack_int4(kc) if bits == 4 else kc
        codes_v = kivi.unpack_int4(vc) if bits == 4 else vc
        # codes [N][Hkv][16][d] -> values, then to the pool layout [N][16][Hkv][d]
        Kd = (codes_k * kp[:, :, 0:1, :].astype(np.float64) + kp[:, :, 1:2, :]).transpose(0, 2, 1, 3)
        Vd = (codes_v * vp[..., 0:1].astype(np.float64) + vp[..., 1:2]).transpose(0, 2, 1, 3)
        Kx = np.concatenate([Kd, bf16_bits_to_f64(rk)])
        Vx = np.concatenate([Vd, bf16_bits_to_f64(rv)])
        t2 = np.concatenate([table, np.full((B, 1), -1, np.int32)], axis=1)
        for b, n in enumerate(lens):
            t2[b, n // BLOCK] = N + b  # the partial block's tokens, slots 0..n%16-1
        want = oracle.paged_decode_attention(q, Kx, Vx, t2, lens, 0.2, kv_dtype="f64",
                                             q_dtype="bf16")
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def pin_append_then_attend_from_empty():
    """Tokens appended one by one: completed blocks are quantised, the tail
    stays exact; attention after each step equals SDPA over those values."""
    rng = _rng(6)
    for bits in (8, 4):
        N, hkv, hq, d, steps = 4, 2, 4, 16, 40
        kc = np.zeros((N, hkv, BLOCK, d // 2 if bits == 4 else d), np.uint8)
        vc = np.zeros_like(kc)
        kp = np.zeros((N, hkv, 2, d), np.float16)
        vp = np.zeros((N, hkv, BLOCK, 2), np.float16)
        rk = np.zeros((1, BLOCK, hkv, d), np.uint16)
        rv = np.zeros_like(rk)
        state = (kc, vc, kp, vp, rk, rv)
        table = np.array([[2, 0, 3]], np.int32)
        raw_k = _bf16_bits(rng.standard_normal((steps, hkv, d)))
        raw_v = _bf16_bits(rng.standard_normal((steps, hkv, d)))
        for n in range(1, steps + 1):
            state = kivi.kivi_append(state, table, np.array([n]), raw_k[n - 1][None],
                                     raw_v[n - 1][None], bits)
            q = _bf16_bits(rng.standard_normal((1, hq, d)))
            got = kivi.kivi_decode_attention(q, *state, table, np.array([n]), 0.25, bits)
            K = bf16_bits_to_f64(raw_k[:n]).copy()
            V = bf16_bits_to_f64(raw_v[:n]).copy()
            for j in range(n // BLOCK):
                for g in range(hkv):
                    kq, kpar, vq, vpar = kivi.quantize_block(
                        K[BLOCK * j: BLOCK * (j + 1), g].astype(np.float32),
                        V[BLOCK * j: BLOCK * (j + 1), g].astype(np.float32), bits)
                    K[BLOCK * j: BLOCK * (j + 1), g] = kq * kpar[0].astype(np.float64) + kpar[1]
                    V[BLOCK * j: BLOCK * (j + 1), g] = vq * vpar[:, :1].astype(np.float64) + vpar[:, 1:]
            qt = torch.from_numpy(bf16_bits_to_f64(q[0]))[None, :, None, :]
            kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]
            vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
            want = F.scaled_dot_product_attention(qt, kt, vt, scale=0.25, enable_gqa=True)
            np.testing.assert_allclose(got[0], want[0, :, 0].numpy(), rtol=0, atol=1e-12)


def pin_int8_is_close_to_the_unquantised_cache():
    rng = _rng(7)
    n, hkv, hq, d = 64, 1, 2, 64
    raw_k = _bf16_bits(rng.standard_normal((n, hkv, d)))
    raw_v = _bf16_bits(rng.standard_normal((n, hkv, d)))
    state = (np.zeros((4, hkv, BLOCK, d), np.uint8), np.zeros((4, hkv, BLOCK, d), np.uint8),
             np.zeros((4, hkv, 2, d), np.float16), np.zeros((4, hkv, BLOCK, 2), np.float16),
             np.zeros((1, BLOCK, hkv, d), np.uint16), np.zeros((1, BLOCK, hkv, d), np.uint16))
    table = np.array([[0, 1, 2, 3]], np.int32)
    for t in range(n):
        state = kivi.kivi_append(state, table, np.array([t + 1]), raw_k[t][None], raw_v[t][None], 8)
    q = _bf16_bits(rng.standard_normal((1, hq, d)))
    got = kivi.kivi_decode_attention(q, *state, table, np.array([n]), 1 / 8, 8)
    exact = oracle.paged_decode_attention(q, raw_k.reshape(4, BLOCK, hkv, d),
                                          raw_v.reshape(4, BLOCK, hkv, d), table,
                                          np.array([n]), 1 / 8, kv_dtype="bf16", q_dtype="bf16")
    assert np.abs(got - exact).max() < 0.02


PINS = [
    pin_quantiser_bound,
    pin_values_on_the_grid_are_exact,
    pin_constant_group,
    pin_k_per_channel_and_v_per_token,
    pin_int4_packing,
    pin_attention_over_independently_dequantised_pool,
    pin_append_then_attend_from_empty,
    pin_int8_is_close_to_the_unquantised_cache,
]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_kivi_pin(pin):
    pin()


_REAL_QB = kivi.quantize_block
_REAL_GATHER = kivi.gather_kivi


def _k_per_token(k_rows, v_rows, bits):
    kc, kp, vc, vp = _REAL_QB(k_rows, v_rows, bits)
    # quantise K like V (per token) instead of per channel
    k_rows = np.asarray(k_rows, np.float32)
    for t in range(BLOCK):
        kc[t], s, m = kivi.quantize_group(k_rows[t], bits)
        kp[0, :], kp[1, :] = s, m
    return kc, kp, vc, vp


def _residual_dropped(k_codes, v_codes, k_par, v_par, res_k, res_v, table_row, b, n, g, bits):
    K, V = _REAL_GATHER(k_codes, v_codes, k_par, v_par, res_k, res_v, table_row, b, n, g, bits)
    r = n % BLOCK
    if r:
        K[n - r:], V[n - r:] = 0.0, 0.0
    return K, V


def _nibbles_swapped(codes):
    c = np.asarray(codes, np.uint8)
    return (c[..., 1::2] | (c[..., 0::2] << 4)).astype(np.uint8)


def _v_min_ignored(codes, scale, mn):
    return np.asarray(codes, np.float64) * np.float64(scale)


MUTANTS = {
    "k_quantised_per_token": ("quantize_block", _k_per_token),
    "residual_dropped": ("gather_kivi", _residual_dropped),
    "nibbles_swapped": ("pack_int4", _nibbles_swapped),
    "min_ignored_in_dequantise": ("dequantize", _v_min_ignored),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_kivi_mistakes_are_caught(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(kivi, attr, fn)
    broken = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin()
            except Exception:
                broken.append(pin.__name__)
    assert broken, f"no pin catches the planted mistake {mutant!r}"
