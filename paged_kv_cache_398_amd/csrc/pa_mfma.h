// pa_mfma.h -- device helpers shared by the kernels that run their products
// on the matrix cores (v_mfma_f32_16x16x32_bf16 and _f16): operand types,
// the 4-lane maximum of a 16x16 result column, the two-term bf16 split of
// the softmax weights and their fp16 rounding, and the staged loads of K/V
// block pairs into a per-wave LDS tile.  Internal; included by the .hip
// sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8_t, x); }

// fp16 operands (v_mfma_f32_16x16x32_f16): the wide chunk kernel's PV
// products over bf16 pools take fp16 weights and fp16 V.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// 1.0 in all eight fp16 lanes
__device__ __forceinline__ f16x8_t f16x8_ones() {
  return __builtin_bit_cast(f16x8_t, make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u));
}

// Eight fp32 values rounded to the nearest fp16 (a relative 2^-11 for the
// softmax weights, which lie in (0, 2^8]; below 2^-24 they become 0).
__device__ __forceinline__ f16x8_t to_f16x8(const float (&p)[8]) {
  f16x8_t h;
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (_Float16)p[e];
  return h;
}

// Eight bf16 values (16 bytes) as fp16: exact for magnitudes in
// [2^-14, 65504]; rounded toward zero below that (an absolute error under
// 2^-24) and above it saturated at 65504 (round-toward-zero never
// overflows to infinity).
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 x) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w[i] << 16),
                                                                   __uint_as_float(w[i] & 0xFFFF0000u)));
  return make_uint4(r[0], r[1], r[2], r[3]);
}

// 1.0 in all eight bf16 lanes (the "ones" operand whose product gives row sums)
__device__ __forceinline__ bf16x8_t bf16x8_ones() {
  return as_bf16x8(make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
}

// Maximum over lanes c, c+16, c+32, c+48 (the four lanes of one column of a
// 16x16 product).  A compare and select: the values are scores or -inf,
// never NaN, so no quieting of NaN inputs (which fmaxf would add after the
// lane swaps) is needed.
__device__ __forceinline__ float max4q(float x) {
  {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float u = __uint_as_float(r[0]), v = __uint_as_float(r[1]);
    x = u > v ? u : v;
  }
  {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float u = __uint_as_float(r[0]), v = __uint_as_float(r[1]);
    x = u > v ? u : v;
  }
  return x;
}

__device__ __forceinline__ float max8(const float (&x)[2][4]) {
  return fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
               fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
}

// p = hi + lo in bf16: hi is p truncated to bf16 (the upper half of its
// bits, one byte permute per pair), the remainder p - hi is exact in fp32
// and below 2^-7 p, and lo is that remainder rounded to the nearest bf16;
// so hi + lo is within a relative 2^-16 of p.
__device__ __forceinline__ void split_bf16(const float (&p)[8], bf16x8_t &hi, bf16x8_t &lo) {
  uint32_t h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = __float_as_uint(p[2 * i]), b = __float_as_uint(p[2 * i + 1]);
    h[i] = __builtin_amdgcn_perm(b, a, 0x07060302u);  // upper halves of a (low), b (high)
    lo[2 * i] = (__bf16)(p[2 * i] - __uint_as_float(a & 0xFFFF0000u));
    lo[2 * i + 1] = (__bf16)(p[2 * i + 1] - __uint_as_float(b & 0xFFFF0000u));
  }
  hi = as_bf16x8(make_uint4(h[0], h[1], h[2], h[3]));
}


// ---------------------------------------------------------------------------
// Staged loads of a pair of K/V blocks (32 tokens of one KV head).
//
// Each load instruction covers whole 128-byte pieces of 8 token rows (16
// bytes per lane), the layout that streams fastest: loading straight into
// the MFMA operand layout (16 rows x 64 bytes per instruction) measured 23%
// slower as pure loads over the Llama-3-8B-shaped pools.  A landed pair is
// written to a per-wave LDS tile as bf16 rows (FP8 codes widened on the
// way, which is exact: every E4M3FN value is a bf16 value), rows past the
// limit and blocks outside the pool as zeros, and read back from there as
// operands: K rows by 16-byte reads, V by transposing reads.

template <int KV, int D>
struct MCfg {
  static constexpr int EB = KV == KV_FP8 ? 1 : 2;    // stored bytes per element
  static constexpr int ROW = D * EB;                 // bytes of one head row in the pool
  static constexpr int SEG = ROW < 128 ? ROW : 128;  // bytes of a row per load instruction
  static constexpr int LPR = SEG / 16;               // lanes per row segment (16 B each)
  static constexpr int RPI = 64 / LPR;               // rows per load instruction
  static constexpr int NSEG = ROW / SEG;             // segments per row
  static constexpr int NI = (16 / RPI) * NSEG;       // load instructions per block (K, and V)
  static constexpr int KM = D / 32;                  // S^T products per block
  static constexpr int EV = D / 16;                  // 16-dim slabs of O
  static constexpr int RSK = D * 2 + 16;             // LDS row strides of the bf16 rows (bytes):
  static constexpr int RSV = D * 2 + 32;             // K and V operand reads cover the banks once
  static constexpr int TILE = 32 * (RSK + RSV);      // one pair: 32 K rows, then 32 V rows
  static_assert(16 % RPI == 0 && ROW % SEG == 0, "whole rows per load instruction");
};

// A pair's loads in flight (registers), and what the compute needs of it.
template <int KV, int D>
struct PairLoads {
  uint4 k[2][MCfg<KV, D>::NI], v[2][MCfg<KV, D>::NI];
  float4 ks[2], vs[2];  // FP8: scales of tokens 4q .. 4q+3 of each block
  int tok[2];           // sequence position of each block's slot 0
  bool ok[2];           // block id inside the pool (no block: false)
};
struct PairMeta {
  float4 ks[2], vs[2];
  int tok[2];
  bool ok[2];
};

// This lane's row and offsets for load instruction ii: in a pool block of
// KV head g (bytes), and in the bf16 tile row.
template <int KV, int D>
struct StageLanes {
  int row[MCfg<KV, D>::NI];
  uint32_t loff[MCfg<KV, D>::NI], toff[MCfg<KV, D>::NI];
};
template <int KV, int D>
__device__ __forceinline__ StageLanes<KV, D> stage_lanes(int hkv, int g) {
  using M = MCfg<KV, D>;
  const int lane = threadIdx.x & 63;
  StageLanes<KV, D> L;
#pragma unroll
  for (int ii = 0; ii < M::NI; ++ii) {
    L.row[ii] = (ii / M::NSEG) * M::RPI + lane / M::LPR;
    const int byte = (ii % M::NSEG) * M::SEG + (lane % M::LPR) * 16;
    L.loff[ii] = (uint32_t)((L.row[ii] * hkv + g) * M::ROW + byte);
    L.toff[ii] = (uint32_t)(byte * (2 / M::EB));
  }
  return L;
}

// Issue the loads of two blocks (ids id0, id1; an id outside [0, num_blocks)
// reads block 0 and is marked not ok) whose slot 0 sits at positions tok0,
// tok1.  Unconditional loads, so that no branch around a load breaks the
// compiler's wait counting.  FP8 codes and scales use plain loads (faster
// than the non-temporal hint on 128-byte rows); bf16 rows stream.
template <int KV, int D>
__device__ __forceinline__ void issue_pair(PairLoads<KV, D> &P, const StageLanes<KV, D> &L,
                                           const void *k_cache, const void *v_cache,
                                           const float *k_scale, const float *v_scale,
                                           size_t block_bytes, int hkv, int g, int num_blocks,
                                           int id0, int id1, int tok0, int tok1) {
  using M = MCfg<KV, D>;
  const int q = (threadIdx.x & 63) >> 4;
  const char *kbase = static_cast<const char *>(k_cache);
  const char *vbase = static_cast<const char *>(v_cache);
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int id = hb ? id1 : id0;
    P.tok[hb] = hb ? tok1 : tok0;
    P.ok[hb] = (unsigned)id < (unsigned)num_blocks;
    const size_t boff = P.ok[hb] ? (size_t)id * block_bytes : 0;
#pragma unroll
    for (int ii = 0; ii < M::NI; ++ii) {
      if constexpr (KV == KV_FP8) {
        P.k[hb][ii] = *reinterpret_cast<const uint4 *>(kbase + boff + L.loff[ii]);
        P.v[hb][ii] = *reinterpret_cast<const uint4 *>(vbase + boff + L.loff[ii]);
      } else {
        P.k[hb][ii] = load_stream16(kbase + boff + L.loff[ii]);
        P.v[hb][ii] = load_stream16(vbase + boff + L.loff[ii]);
      }
    }
    if constexpr (KV == KV_FP8) {
      const size_t si = ((P.ok[hb] ? (size_t)id : 0) * hkv + g) * 16 + 4 * q;
      P.ks[hb] = *reinterpret_cast<const float4 *>(k_scale + si);
      P.vs[hb] = *reinterpret_cast<const float4 *>(v_scale + si);
    } else {
      P.ks[hb] = P.vs[hb] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// 16 FP8 codes -> 16 bf16 (exact)
__device__ __forceinline__ void widen_fp8x16(uint4 x, uint4 &lo, uint4 &hi) {
  const uint32_t d[4] = {x.x, x.y, x.z, x.w};
  uint32_t r[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[2 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[j], 1.0f, false));
    r[2 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[j], 1.0f, true));
  }
  lo = make_uint4(r[0], r[1], r[2], r[3]);
  hi = make_uint4(r[4], r[5], r[6], r[7]);
}

// Write a landed pair into the tile: K rows 0..31 at RSK, then V rows at
// RSV (block hb's slot s in row 16 hb + s).  A slot at or past `limit`, or
// in a block outside the pool, is stored as zeros (the scores of such slots
// are masked; zero V rows keep NaN garbage out of the products).
template <int KV, int D>
__device__ __forceinline__ PairMeta stage_pair(const PairLoads<KV, D> &P,
                                               const StageLanes<KV, D> &L, char *tile,
                                               int limit) {
  using M = MCfg<KV, D>;
  PairMeta mt;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const bool all = P.ok[hb] && P.tok[hb] + 16 <= limit;  // wave-uniform
#pragma unroll
    for (int ii = 0; ii < M::NI; ++ii) {
      const bool live = all || (P.ok[hb] && P.tok[hb] + L.row[ii] < limit);
      const uint32_t mk = live ? 0xFFFFFFFFu : 0u;
      uint4 kx = P.k[hb][ii], vx = P.v[hb][ii];
      if (!all) {
        kx = make_uint4(kx.x & mk, kx.y & mk, kx.z & mk, kx.w & mk);
        vx = make_uint4(vx.x & mk, vx.y & mk, vx.z & mk, vx.w & mk);
      }
      char *kd = tile + (16 * hb + L.row[ii]) * M::RSK + L.toff[ii];
      char *vd = tile + 32 * M::RSK + (16 * hb + L.row[ii]) * M::RSV + L.toff[ii];
      if constexpr (KV == KV_FP8) {
        uint4 a0, a1;
        widen_fp8x16(kx, a0, a1);
        *reinterpret_cast<uint4 *>(kd) = a0;
        *reinterpret_cast<uint4 *>(kd + 16) = a1;
        widen_fp8x16(vx, a0, a1);
        *reinterpret_cast<uint4 *>(vd) = a0;
        *reinterpret_cast<uint4 *>(vd + 16) = a1;
      } else {
        *reinterpret_cast<uint4 *>(kd) = kx;
        *reinterpret_cast<uint4 *>(vd) = vx;
      }
    }
    mt.tok[hb] = P.tok[hb];
    mt.ok[hb] = P.ok[hb];
    mt.ks[hb] = P.ks[hb];
    mt.vs[hb] = P.vs[hb];
  }
  return mt;
}

// B operands of O = P V for 16-dim slab m: lane (n, q) receives dim 16m + n
// of tokens 4q .. 4q+3 of both blocks of the tile.  ds_read_b64_tr_b16 gives
// lane i of a 16-lane group element i % 4 of the 8 bytes addressed by lanes
// 4r + i / 4, r = 0..3 (checked on the GPU with a one-wave probe); so lane
// 4r + s addresses token 4q + r, dims 16m + 4s .. 16m + 4s + 3.
template <int D>
__device__ __forceinline__ bf16x8_t v_operand_tr(const char *lv, int rsv, int m) {
  const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
  v4s_t h[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
    h[hb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4s_t *)(lv + (16 * hb + 4 * q + (c >> 2)) * rsv + (16 * m + 4 * (c & 3)) * 2));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace pa
