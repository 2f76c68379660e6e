"""INT8 / INT4 KV cache with KIVI-style quantisation, float64 oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where it is stated ([freetools] section
"KV Cache量化：用精度换空间"; [k1-blog] section on KV cache quantisation):

* K and V are stored as 8- or 4-bit integers instead of 16-bit floats
  (INT8 halves, INT4 quarters the bytes).
* KIVI's asymmetric scheme: Key quantised per channel (K's outliers sit in a
  few channels), Value per token; the quantisation parameters come from the
  data (dynamic scaling); the most recent tokens are kept at full precision
  (a residual) so errors do not build up on them.

Readings where the pages are silent (the GPU path follows the same):

* Asymmetric uniform codes 0 .. 2^b - 1 with a scale and a minimum per
  group: value = code * scale + min.
* Groups: K per (16-token block, KV head, channel) over the block's 16
  tokens; V per (token, KV head) over head_dim.  A block is quantised when
  its 16th token arrives; the tokens of a sequence's partly filled last
  block are its full-precision residual (bf16), kept per sequence apart from
  the pool.
* Parameters are stored as IEEE float16 (round to nearest even):
  scale = fp16((max - min) / (2^b - 1)) computed in float32, 1 if that is
  zero; min = fp16(min).  Codes use the stored parameters:
  code = clamp(rint((x - min) / scale), 0, 2^b - 1) in float32 (IEEE
  division, ties to even).
* Storage: codes [N][Hkv][16][d], head-major so that one head's rows are
  contiguous (INT8: one byte per code; INT4: two codes per byte, channel 2i
  in the low nibble and 2i+1 in the high one); K
  parameters [N][Hkv][2][d] (scales, then minimums); V parameters
  [N][Hkv][16][2] (scale, min per slot); residual rows [B][16][Hkv][d] bf16
  (slot t % 16 of sequence b's partial block).
"""

import numpy as np

from . import decode_attention as da

BLOCK = 16


def levels(bits: int) -> int:
    return (1 << bits) - 1


def quantize_group(x, bits: int):
    """Codes (uint8), fp16 scale and fp16 min of one group of values."""
    x = np.asarray(x, dtype=np.float32)
    lo, hi = np.float32(x.min()), np.float32(x.max())
    s = np.float16((hi - lo) / np.float32(levels(bits)))
    if s == 0:
        s = np.float16(1.0)
    m = np.float16(lo)
    y = (x - np.float32(m)) / np.float32(s)
    codes = np.clip(np.rint(y), 0, levels(bits)).astype(np.uint8)
    return codes, s, m


def dequantize(codes, scale, mn):
    return np.asarray(codes, np.float64) * np.float64(scale) + np.float64(mn)


def quantize_block(k_rows, v_rows, bits: int):
    """One block of one KV head: k_rows, v_rows [16][d] float32 ->
    K codes [16][d], K params [2][d] (scales, mins), V codes [16][d],
    V params [16][2]."""
    k_rows = np.asarray(k_rows, np.float32)
    v_rows = np.asarray(v_rows, np.float32)
    d = k_rows.shape[1]
    kc = np.empty((BLOCK, d), np.uint8)
    kp = np.empty((2, d), np.float16)
    for c in range(d):  # per channel, over the block's tokens
        kc[:, c], kp[0, c], kp[1, c] = quantize_group(k_rows[:, c], bits)
    vc = np.empty((BLOCK, d), np.uint8)
    vp = np.empty((BLOCK, 2), np.float16)
    for t in range(BLOCK):  # per token, over the channels
        vc[t], vp[t, 0], vp[t, 1] = quantize_group(v_rows[t], bits)
    return kc, kp, vc, vp


def pack_int4(codes):
    c = np.asarray(codes, np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed):
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def codes_of(stored, bits: int):
    return unpack_int4(stored) if bits == 4 else np.asarray(stored, np.uint8)


def gather_kivi(k_codes, v_codes, k_par, v_par, res_k, res_v, table_row, b, n, g, bits):
    """K, V [n][d] float64 of KV head g of sequence b: full blocks
    dequantised through the table, the partial last block from the residual."""
    kc_all = codes_of(k_codes, bits)
    vc_all = codes_of(v_codes, bits)
    nf = n // BLOCK
    d = kc_all.shape[-1]
    K = np.empty((n, d))
    V = np.empty((n, d))
    for j in range(nf):
        p = int(table_row[j])
        kp = k_par[p, g].astype(np.float64)      # [2][d]
        vp = v_par[p, g].astype(np.float64)      # [16][2]
        K[BLOCK * j: BLOCK * (j + 1)] = kc_all[p, g] * kp[0] + kp[1]
        V[BLOCK * j: BLOCK * (j + 1)] = vc_all[p, g] * vp[:, :1] + vp[:, 1:]
    r = n - BLOCK * nf
    if r:
        from .formats import bf16_bits_to_f64
        K[BLOCK * nf:] = bf16_bits_to_f64(res_k[b, :r, g, :])
        V[BLOCK * nf:] = bf16_bits_to_f64(res_v[b, :r, g, :])
    return K, V


def kivi_decode_attention(q, k_codes, v_codes, k_par, v_par, res_k, res_v, block_table,
                          context_lens, scale, bits: int, q_dtype: str = "bf16"):
    """out[b, h] = softmax(scale * q[b, h] . K_b^T) V_b over the sequence's
    n tokens: quantised full blocks and the bf16 residual."""
    qf = da._decode(q, q_dtype)
    B, Hq, d = qf.shape
    Hkv = k_par.shape[1]
    out = np.zeros((B, Hq, d))
    for b in range(B):
        n = int(context_lens[b])
        if n <= 0:
            continue
        cur = None
        for h in range(Hq):
            g = da.kv_head_of(h, Hq, Hkv)
            if g != cur:
                K, V = gather_kivi(k_codes, v_codes, k_par, v_par, res_k, res_v,
                                   block_table[b], b, n, g, bits)
                cur = g
            w = da.softmax(da.scores(K, qf[b, h], float(scale)))
            out[b, h] = w @ V
    return out


def kivi_append(state, block_table, context_lens, k_new, v_new, bits: int):
    """Write each sequence's new token (position n - 1) into its residual
    row; a token that fills its block has the whole block quantised into the
    pool.  ``state`` = (k_codes, v_codes, k_par, v_par, res_k, res_v) with
    residual rows as bf16 bits; k_new, v_new [B][Hkv][d] bf16 bits.
    Returns the new state (inputs unchanged)."""
    from .formats import bf16_bits_to_f64
    kc, vc, kp, vp, rk, rv = (np.array(a, copy=True) for a in state)
    n_blocks = kp.shape[0]
    hkv = kp.shape[1]
    for b, n in enumerate(np.asarray(context_lens)):
        if n <= 0:
            continue
        t = int(n) - 1
        slot = t % BLOCK
        rk[b, slot] = k_new[b]
        rv[b, slot] = v_new[b]
        if slot != BLOCK - 1:
            continue
        p = int(block_table[b][t // BLOCK])
        if not 0 <= p < n_blocks:
            continue
        for g in range(hkv):
            krows = bf16_bits_to_f64(rk[b, :, g, :]).astype(np.float32)
            vrows = bf16_bits_to_f64(rv[b, :, g, :]).astype(np.float32)
            kq, kpar, vq, vpar = quantize_block(krows, vrows, bits)
            if bits == 4:
                kc[p, g] = pack_int4(kq)
                vc[p, g] = pack_int4(vq)
            else:
                kc[p, g] = kq
                vc[p, g] = vq
            kp[p, g] = kpar
            vp[p, g] = vpar
    return kc, vc, kp, vp, rk, rv
