// pa_kernels.hip -- gfx950 (CDNA4) kernels for single-token decode attention
// over a paged KV cache.
//
// What is computed: for each sequence b and query head h,
//   out[b][h] = softmax_t(scale * q[b][h] . K[t][g]) V[t][g],  g = h / G,
// over the tokens t < context_lens[b], token t read from physical block
// table[b][t / 16], slot t % 16 ("KV Cache 深度解析:显存黑洞、PagedAttention
// 与三路省内存方案", sections 一, 三 and 六; grouping of query heads as in the
// GQA section of "大模型推理为何这么慢？从内存带宽瓶颈到KV Cache优化的技术突围").
//
// How (one kernel, attention_kernel; details above it):
//
//  - The work is counted in units (one 16-token block of one (sequence,
//    chunk of hc adjacent KV heads) pair) and split into equal contiguous
//    ranges, one per workgroup of kWaves waves, whatever the mix of context
//    lengths.  A range is cut into pieces at pair boundaries.  hc is the
//    host's choice for a batch whose sequences all have the block count of
//    max_context_len, and the widest chunk otherwise (ranges then cut
//    across pairs anyway, and fewer, longer pieces stream faster).
//  - In a piece, wave w works on head w % hc of the chunk and takes every
//    (kWaves/hc)-th block.  A wave holds a whole block of its head in
//    registers: each token row is split over LPT lanes, 64/LPT tokens per
//    pass, with 8- or 16-byte loads per lane.  Every K/V element is loaded
//    from HBM once and used by all G query heads of its group, which sit in
//    the same lane's registers.  The loop is a two-stage software pipeline:
//    the next block's loads are in flight while the current block is
//    computed, and the block table of up to 64 blocks is read by one vector
//    load before it starts.
//  - Scores are reduced over the LPT lanes of a token with DPP.  The
//    softmax is accumulated online (running max and sum, as in the
//    FlashAttention sections of the pages): the running max is kept
//    wave-uniform and is only raised when a block's maximum exceeds it by
//    more than kTau (log2 units), so the rescale of the accumulators is
//    rare; any running max gives the same normalised result, it only bounds
//    the exponentials (by 2^kTau).
//  - At the end of a piece the lanes' states and the phases of each head
//    are combined exactly in LDS.  A piece that is a whole pair writes the
//    normalised output; a pair split between ranges leaves a (max, sum,
//    unnormalised output) record per piece, and the last piece to finish
//    merges them (log-sum-exp: M = max_p m_p, w_p = 2^(m_p - M),
//    out = sum w_p acc_p / sum w_p l_p).
//
// Positions past a sequence's length contribute exactly nothing (selects,
// not multiplications, so NaN garbage in unused slots cannot leak), table
// entries past the last used block are never read, and block ids outside
// [0, num_blocks) are never dereferenced: block 0 is read in their place and
// masked out.

#include "pa_internal.h"
#include "pa_mfma.h"

#include <hip/hip_ext.h>

#include <mutex>
#include <vector>

namespace pa {
namespace {

constexpr int kBlock = 16;         // tokens per physical block
constexpr int kThreads = kWaves * 64;
constexpr float kTau = 8.0f;       // lag allowed to the running max (log2 units)
// Start of the running max: the lowest finite float rather than -inf, so
// that exp2(s - m) is 0 for a masked score (-inf) even before any valid
// token was seen (a wave whose first blocks are all masked, e.g. block ids
// outside the pool), never exp2(-inf - -inf) = NaN.  Any valid score raises
// the max above it on its first block.
constexpr float kNoMax = -3.402823466e38f;

__host__ __device__ constexpr int elem_bytes(int kv) {
  return kv == KV_F32 ? 4 : (kv == KV_BF16 ? 2 : 1);
}

// Most fp32 output accumulators one lane keeps (G * D / LPT).
constexpr int kAccRegs = 64;
// Lanes per token row: as few as possible while keeping the per-lane output
// accumulators (G * D / LPT floats) at kAccRegs registers or fewer, and
// each lane's slice of a row at 8 bytes or more.
__host__ __device__ constexpr int lanes_per_token(int d, int g, int eb) {
  int l = (g * d / 4 <= kAccRegs) ? 4 : ((g * d / 8 <= kAccRegs) ? 8 : 16);
  while (l > 4 && d * eb / l < 8) l /= 2;
  return l;
}

template <int KV, int D, int G>
struct Cfg {
  static constexpr int EB = elem_bytes(KV);
  static constexpr int LPT = lanes_per_token(D, G, EB);
  static constexpr int ROW = D * EB;               // bytes of one token row (one head)
  static constexpr int LB = ROW / LPT;             // bytes per lane per token
  static constexpr int CH = LB < 16 ? LB : 16;     // bytes per load instruction
  static constexpr int NCH = LB / CH;              // loads per lane per token row
  static constexpr int EPC = CH / EB;              // elements per load
  static constexpr int EPL = D / LPT;              // elements per lane per token
  static constexpr int DW = LB / 4;                // dwords per lane per token row
  static constexpr int TPP = 64 / LPT;             // tokens per pass
  static constexpr int NPASS = kBlock / TPP;       // passes per block
  static_assert(LB >= 8 && LB % 8 == 0, "per-lane slice must be >= 8 bytes");
  static_assert(NPASS >= 1, "a block needs at least one pass");
};

// ---------------------------------------------------------------------------
// cross-lane helpers

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the LPT consecutive lanes of one token row; every lane of the
// group ends with the same value (each step adds a pair in both orders).
template <int LPT>
__device__ __forceinline__ float row_group_sum(float x) {
  x += dpp<0xB1>(x);                       // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp<0x4E>(x);                       // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (LPT >= 8) x += dpp<0x141>(x);   // row_half_mirror: quads of 8
  if constexpr (LPT >= 16) x += dpp<0x140>(x);  // row_mirror: halves of 16
  return x;
}

// Combine the 64/LPT token slots of a wave (lanes with equal lane % LPT).
template <int LPT, bool MAX>
__device__ __forceinline__ float slot_reduce(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  if constexpr (LPT <= 4) x = op(x, dpp<0x124>(x));  // row_ror:4
  if constexpr (LPT <= 8) x = op(x, dpp<0x128>(x));  // row_ror:8
  {  // rows 0<->1 and 2<->3
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  {  // lanes 0-31 <-> 32-63
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return x;
}

__device__ __forceinline__ float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// NT: with the non-temporal hint.  FP8 pools are read without it: their
// 128-byte rows (and 64-byte scale runs) sustained about 7% less bandwidth
// with the hint than without, the opposite of the 2-byte pools.
template <int CH, bool NT>
__device__ __forceinline__ void load_chunk(const char *p, uint32_t *dst) {
  if constexpr (CH == 16) {
    const uint4 x = NT ? load_stream16(p) : *reinterpret_cast<const uint4 *>(p);
    dst[0] = x.x; dst[1] = x.y; dst[2] = x.z; dst[3] = x.w;
  } else {
    static_assert(CH == 8, "8- or 16-byte loads only");
    const uint2 x = NT ? load_stream8(p) : *reinterpret_cast<const uint2 *>(p);
    dst[0] = x.x; dst[1] = x.y;
  }
}

// Widen one lane's slice of a token row (DW dwords) to EPL floats.
template <int KV, int DW, int EPL>
__device__ __forceinline__ void to_float(const uint32_t *r, float *f) {
  if constexpr (KV == KV_F32) {
#pragma unroll
    for (int i = 0; i < DW; ++i) f[i] = __uint_as_float(r[i]);
  } else if constexpr (KV == KV_BF16) {
#pragma unroll
    for (int i = 0; i < DW; ++i) {
      f[2 * i] = __uint_as_float(r[i] << 16);
      f[2 * i + 1] = __uint_as_float(r[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < DW; ++i) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(r[i], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(r[i], true);
      f[4 * i] = lo[0]; f[4 * i + 1] = lo[1];
      f[4 * i + 2] = hi[0]; f[4 * i + 3] = hi[1];
    }
  }
}

// ---------------------------------------------------------------------------
// attention kernel

template <int KV, int D, int G>
struct Block {  // one block's K/V slice held by one lane
  using C = Cfg<KV, D, G>;
  uint32_t k[C::NPASS][C::DW];
  uint32_t v[C::NPASS][C::DW];
  float ks[C::NPASS], vs[C::NPASS];  // FP8 per-token scales
  int tok;                            // sequence position of the block's slot 0
  bool ok;                            // block id in range
};

// The query rows of the G heads of KV head g, sliced as the lanes of a wave
// hold K/V: lane-local fp32 copies, and bf16 pairs for the bf16 dot product.
template <int KV, int D, int G>
struct Query {
  using C = Cfg<KV, D, G>;
  float f[G][C::EPL];
  uint32_t bf2[G][C::DW];
  bf16x8_t qm[D / 32];  // MFMA form: lane (row c, quarter q) holds q[h0 + c][32m + 8q .. +7]
};

// bf16 pools run their products on the matrix cores; f32 and FP8 pools on
// the vector ALUs.  (The matrix-core form handles FP8 too, widening the
// codes to bf16 in its LDS tile, but on the FP8 MHA step, one query row per
// KV head, it measured 402 us against 367 us for the vector form.)
template <int KV>
constexpr bool uses_mfma() { return KV == KV_BF16; }

template <int KV, int D, int G>
__device__ __forceinline__ void load_query(const LaunchArgs &a, int b, int g, Query<KV, D, G> &qry) {
  if constexpr (uses_mfma<KV>()) {
    // B operand of S^T = K Q^T: column = query row c (rows G.. are zero),
    // k = 8 dims at 32m + 8q
    const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) +
                         ((size_t)b * a.hq + g * G + (c < G ? c : 0)) * D + 8 * q;
#pragma unroll
    for (int m = 0; m < D / 32; ++m)
      qry.qm[m] = as_bf16x8(c < G ? *reinterpret_cast<const uint4 *>(qp + 32 * m)
                                  : make_uint4(0u, 0u, 0u, 0u));
    return;
  }
  using C = Cfg<KV, D, G>;
  constexpr int LPT = C::LPT;
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPT;
  const int h0 = g * G;
  float(&qf)[G][C::EPL] = qry.f;
  uint32_t(&q2)[G][C::DW] = qry.bf2;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) {
      const int e0 = (c * LPT + sub) * C::EPC;
      const size_t qi = ((size_t)b * a.hq + h0 + hh) * D + e0;
      if constexpr (KV == KV_F32) {
        const float *qp = static_cast<const float *>(a.q) + qi;
#pragma unroll
        for (int j = 0; j < C::EPC; ++j) qf[hh][c * C::EPC + j] = qp[j];
      } else {
        const uint16_t *qp = static_cast<const uint16_t *>(a.q) + qi;
#pragma unroll
        for (int j = 0; j < C::EPC; ++j)
          qf[hh][c * C::EPC + j] = __uint_as_float((uint32_t)qp[j] << 16);
        if constexpr (KV == KV_BF16) {
#pragma unroll
          for (int j = 0; j < C::EPC / 2; ++j)
            q2[hh][c * C::EPC / 2 + j] = (uint32_t)qp[2 * j] | ((uint32_t)qp[2 * j + 1] << 16);
        }
      }
    }
  }

}

// Table entries of up to 64 of a wave's blocks, one per lane: lane j holds
// the entry of the wave's block c0 + j (block blk0 + ph + (c0 + j) * nph of
// the sequence), -1 past the wave's nb_w blocks.
__device__ __forceinline__ int load_table(const LaunchArgs &a, int b, int blk0, int ph, int nph,
                                          int c0, int nb_w) {
  const int lane = threadIdx.x & 63;
  const int *trow = a.table + (size_t)b * a.max_blocks + blk0 + ph;
  return c0 + lane < nb_w ? trow[(size_t)(c0 + lane) * nph] : -1;
}

// Blocks of a piece that fall to the wave of phase ph.
__device__ __forceinline__ int wave_blocks(int tok0, int tok_end, int ph, int nph) {
  const int nblk = (tok_end - tok0 + kBlock - 1) / kBlock;
  return nblk > ph ? (nblk - ph + nph - 1) / nph : 0;
}

// One wave's share of a piece: tokens [tok0, tok_end) of sequence b (tok0 a
// multiple of 16), KV head g; the wave takes blocks ph, ph + nph, ... of the
// piece.  qry holds the query rows (load_query) and tv0 the table entries of
// the wave's first 64 blocks (load_table), both loaded by the caller so that
// they can be in flight early.  Leaves the wave's exact state (running max,
// sum, unnormalised output of each of the G query heads) in s_m[w], s_l[w],
// s_acc[w].
template <int KV, int D, int G>
__device__ __forceinline__ void attend_piece(const LaunchArgs &a, int b, int g, int tok0,
                                             int tok_end, int ph, int nph, int w,
                                             const Query<KV, D, G> &qry, int tv0,
                                             float (*s_acc)[G][D], float (*s_m)[G],
                                             float (*s_l)[G]) {
  using C = Cfg<KV, D, G>;
  constexpr int LPT = C::LPT, NPASS = C::NPASS, DW = C::DW, EPL = C::EPL;
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPT;   // which slice of the row
  const int slot = lane / LPT;  // which token of the pass
  const int blk0 = tok0 / kBlock;
  const int nb_w = wave_blocks(tok0, tok_end, ph, nph);

  const float(&qf)[G][EPL] = qry.f;
  const uint32_t(&q2)[G][DW] = qry.bf2;

  // ---- lane offsets inside a block, and the block table of this wave
  const size_t block_bytes = (size_t)kBlock * a.hkv * C::ROW;
  uint32_t lane_off[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p)
    lane_off[p] = (uint32_t)(((p * C::TPP + slot) * a.hkv + g) * C::ROW + sub * C::CH);
  const char *kbase = static_cast<const char *>(a.k_cache);
  const char *vbase = static_cast<const char *>(a.v_cache);

  // Loads of a block are issued unconditionally (an id outside the pool is
  // replaced by block 0 and the block masked in compute), so the loop below
  // has no branch around a load and the next block's loads stay in flight
  // while the current block is computed.
  auto issue = [&](Block<KV, D, G> &bk, int i, int phys) {
    bk.tok = (blk0 + ph + i * nph) * kBlock;
    bk.ok = (unsigned)phys < (unsigned)a.num_blocks;
    const size_t boff = bk.ok ? (size_t)phys * block_bytes : 0;
    const char *kb = kbase + boff;  // wave-uniform base, 32-bit lane offsets
    const char *vb = vbase + boff;
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
#pragma unroll
      for (int c = 0; c < C::NCH; ++c) {
        load_chunk<C::CH, KV != KV_FP8>(kb + (lane_off[p] + c * LPT * C::CH), &bk.k[p][c * (C::CH / 4)]);
        load_chunk<C::CH, KV != KV_FP8>(vb + (lane_off[p] + c * LPT * C::CH), &bk.v[p][c * (C::CH / 4)]);
      }
      if constexpr (KV == KV_FP8) {
        const size_t si = ((bk.ok ? (size_t)phys : 0) * a.hkv + g) * kBlock + p * C::TPP + slot;
        bk.ks[p] = a.k_scale[si];
        bk.vs[p] = a.v_scale[si];
      }
    }
  };

  // ---- online softmax state (per lane; m is wave-uniform)
  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = kNoMax;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.f;
  }
  const float sl2 = a.scale_log2e;

  auto compute = [&](const Block<KV, D, G> &bk) {
    // a partial last block, or a block id outside the pool: mask slots
    const bool tail = !bk.ok || bk.tok + kBlock > tok_end;  // wave-uniform
    float s[NPASS][G];
    bool live[NPASS];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      live[p] = !tail || (bk.ok && bk.tok + p * C::TPP + slot < tok_end);
      float kf[EPL];
      if constexpr (KV != KV_BF16) to_float<KV, DW, EPL>(bk.k[p], kf);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float d0 = 0.f, d1 = 0.f;
        if constexpr (KV == KV_BF16) {
#pragma unroll
          for (int i = 0; i < DW; i += 2) {
            d0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q2[hh][i]),
                                                 __builtin_bit_cast(bf16x2_t, bk.k[p][i]), d0, false);
            d1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q2[hh][i + 1]),
                                                 __builtin_bit_cast(bf16x2_t, bk.k[p][i + 1]), d1, false);
          }
        } else {
#pragma unroll
          for (int e = 0; e < EPL; e += 2) {
            d0 = fmaf(qf[hh][e], kf[e], d0);
            d1 = fmaf(qf[hh][e + 1], kf[e + 1], d1);
          }
        }
        float x = row_group_sum<LPT>(d0 + d1) * sl2;
        if constexpr (KV == KV_FP8) x *= bk.ks[p];
        s[p][hh] = live[p] ? x : -__builtin_huge_valf();
      }
    }
    // block maximum per head, wave-uniform
    bool raise = false;
    float bm[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float x = s[0][hh];
#pragma unroll
      for (int p = 1; p < NPASS; ++p) x = fmaxf(x, s[p][hh]);
      bm[hh] = uniform(slot_reduce<LPT, true>(x));
      raise |= bm[hh] > m[hh] + kTau;
    }
    if (raise) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float mn = fmaxf(m[hh], bm[hh]);
        const float c = fast_exp2(m[hh] - mn);
        m[hh] = mn;
        l[hh] *= c;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hh][e] *= c;
      }
    }
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      float vf[EPL];
      to_float<KV, DW, EPL>(bk.v[p], vf);
      if (tail) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[e] = live[p] ? vf[e] : 0.f;
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float pr = fast_exp2(s[p][hh] - m[hh]);
        l[hh] += pr;
        float pw = pr;
        if constexpr (KV == KV_FP8) pw = live[p] ? pr * bk.vs[p] : 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hh][e] = fmaf(pw, vf[e], acc[hh][e]);
      }
    }
  };

  constexpr bool kOneBlock = KV == KV_F32 && G * D >= 1024;
  // ---- main loop: a two-stage pipeline over the wave's blocks, block i+1 in
  // flight while block i is computed.  The table entries of up to 64 blocks
  // are fetched by one vector load (lane j holds block c0 + j) before the
  // pipeline starts, so the loop itself reads nothing but K and V.
  for (int c0 = 0; c0 < nb_w; c0 += 64) {
    const int cn = min(64, nb_w - c0);
    const int tv = c0 == 0 ? tv0 : load_table(a, b, blk0, ph, nph, c0, nb_w);
    auto entry = [&](int i) { return __builtin_amdgcn_readlane(tv, min(i, cn - 1)); };
    Block<KV, D, G> A, B;
    issue(A, c0, entry(0));
    if constexpr (kOneBlock) {
      // fp32 rows with eight query heads: the accumulators and queries
      // (2 G D / LPT registers) leave no room for a second block in flight
      for (int i = 0; i < cn; ++i) {
        if (i > 0) issue(A, c0 + i, entry(i));
        compute(A);
      }
      continue;
    }
    // The scheduling barriers keep the next block's loads ahead of the
    // first use of the current block; without them the compiler sinks the
    // loads below that use and the two blocks are fetched one after another.
    int i = 0;
    for (; i + 2 < cn; i += 2) {
      issue(B, c0 + i + 1, entry(i + 1));
      __builtin_amdgcn_sched_barrier(0);
      compute(A);
      issue(A, c0 + i + 2, entry(i + 2));
      __builtin_amdgcn_sched_barrier(0);
      compute(B);
    }
    if (i + 1 < cn) {
      issue(B, c0 + i + 1, entry(i + 1));
      __builtin_amdgcn_sched_barrier(0);
      compute(A);
      compute(B);
    } else {
      compute(A);
    }
  }

  // ---- combine the wave's token slots, then the phases of each head, exactly
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    l[hh] = slot_reduce<LPT, false>(l[hh]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hh][e] = slot_reduce<LPT, false>(acc[hh][e]);
  }
  if (lane < LPT) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int c = 0; c < C::NCH; ++c)
#pragma unroll
        for (int j = 0; j < C::EPC; ++j)
          s_acc[w][hh][(c * LPT + sub) * C::EPC + j] = acc[hh][c * C::EPC + j];
  }
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      s_m[w][hh] = m[hh];
      s_l[w][hh] = l[hh];
    }
  }
}

// ---------------------------------------------------------------------------
// The matrix-core form of a wave's share of a piece (bf16 pools; f32 and
// FP8 pools take the vector-ALU form above, which measured faster for FP8's
// half-width rows).
//
// A wave takes its blocks two at a time (a pair: 32 tokens).  Each load
// instruction covers whole 128-byte pieces of 8 token rows (16 bytes per
// lane), the layout that streams fastest: loading straight into the MFMA
// operand layout (16 rows x 64 bytes per instruction) measured 23% slower
// as pure loads over the same pools.  The pair is written to a per-wave
// LDS tile (FP8 codes widened to bf16 on the way, which is exact; slots
// past the piece's end and blocks outside the pool as zeros) and read back
// as operands of v_mfma_f32_16x16x32_bf16:
//  - S^T = K Q^T: A = K (token c of a block, 8 dims at 32m + 8q), B = Q^T
//    (query row c of the group; rows G..15 zero): lane (c, q) gets row c's
//    scores of tokens 4q .. 4q+3 of the block.
//  - O = P V: A = P (the lane's own eight weights: row c, tokens 4q .. 4q+3
//    of both blocks), B = V from transposing LDS reads (ds_read_b64_tr_b16:
//    lane (n, q) receives dim 16m + n of those tokens); lane (n, q) then
//    holds O[rows 4q .. 4q+3][16m + n].  The weights enter as hi + lo bf16
//    (two products, within a relative 2^-16 of the fp32 weights); the row
//    sums come from the same two products against a ones operand.
// The running max is per query row (lanes (c, *)), lagged by kTau; its rare
// rescale hands the row factors to the output layout through 16 floats of
// per-wave LDS.

// The loads of the wave's blocks i and i + 1 (ids id0, id1) of a piece whose
// first block is blk0: blocks blk0 + ph + i * nph and blk0 + ph + (i + 1) * nph
// of the sequence, KV head g.
template <int KV, int D>
__device__ __forceinline__ void issue_piece_pair(const LaunchArgs &a, const StageLanes<KV, D> &sl,
                                                 int g, int blk0, int ph, int nph,
                                                 PairLoads<KV, D> &P, int i, int id0, int id1) {
  const size_t block_bytes = (size_t)kBlock * a.hkv * MCfg<KV, D>::ROW;
  issue_pair<KV, D>(P, sl, a.k_cache, a.v_cache, a.k_scale, a.v_scale, block_bytes, a.hkv, g,
                    a.num_blocks, id0, id1, (blk0 + ph + i * nph) * kBlock,
                    (blk0 + ph + (i + 1) * nph) * kBlock);
}

// The first loads of a wave's share of a piece (its first two pairs), as
// attend_piece_mfma issues them; the kernel issues them early for the piece
// it guesses, before the scan of the lengths, and hands A and B over with
// pre = true.  tv0: the table entries of the wave's first 64 blocks.
template <int KV, int D>
__device__ __forceinline__ void issue_first_pairs(const LaunchArgs &a, int g, int tok0,
                                                  int tok_end, int ph, int nph, int tv0,
                                                  PairLoads<KV, D> &A, PairLoads<KV, D> &B) {
  const int nb_w = wave_blocks(tok0, tok_end, ph, nph);
  if (nb_w == 0) return;
  const int blk0 = tok0 / kBlock;
  const StageLanes<KV, D> sl = stage_lanes<KV, D>(a.hkv, g);
  issue_piece_pair<KV, D>(a, sl, g, blk0, ph, nph, A, 0, __builtin_amdgcn_readlane(tv0, 0),
                          __builtin_amdgcn_readlane(tv0, 1));
  if (nb_w > 2)
    issue_piece_pair<KV, D>(a, sl, g, blk0, ph, nph, B, 2, __builtin_amdgcn_readlane(tv0, 2),
                            __builtin_amdgcn_readlane(tv0, 3));
}

// A and B hold the pairs in flight; with pre, the first two pairs' loads were
// issued into them already (issue_first_pairs, same arguments).
template <int KV, int D, int G>
__device__ __forceinline__ void attend_piece_mfma(const LaunchArgs &a, int b, int g, int tok0,
                                                  int tok_end, int ph, int nph, int w,
                                                  const Query<KV, D, G> &qry, int tv0,
                                                  float (*s_acc)[G][D], float (*s_m)[G],
                                                  float (*s_l)[G], char *tile, float *s_f,
                                                  PairLoads<KV, D> &A, PairLoads<KV, D> &B,
                                                  bool pre) {
  static_assert(KV == KV_BF16, "the matrix-core form reads bf16 pools");
  using M = MCfg<KV, D>;
  constexpr int KM = M::KM, EV = M::EV, RSK = M::RSK, RSV = M::RSV;
  const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
  const int blk0 = tok0 / kBlock;
  const int nb_w = wave_blocks(tok0, tok_end, ph, nph);
  const StageLanes<KV, D> sl = stage_lanes<KV, D>(a.hkv, g);
  auto issue = [&](PairLoads<KV, D> &P, int i, int id0, int id1) {
    issue_piece_pair<KV, D>(a, sl, g, blk0, ph, nph, P, i, id0, id1);
  };
  auto stage = [&](const PairLoads<KV, D> &P) { return stage_pair<KV, D>(P, sl, tile, tok_end); };

  float mrun = kNoMax;  // running max of query row c
  f32x4_t o[EV], l4 = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < EV; ++m) o[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bf16x8_t ones = bf16x8_ones();
  const float sl2 = a.scale_log2e;

  auto compute = [&](const PairMeta &mt) {
    __builtin_amdgcn_wave_barrier();  // the tile's rows were written by other lanes
    f32x4_t sc[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      sc[hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        const uint4 kop = *reinterpret_cast<const uint4 *>(tile + (16 * hb + c) * RSK + (32 * m + 8 * q) * 2);
        sc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kop), qry.qm[m], sc[hb], 0, 0, 0);
      }
    }
    const bool full = mt.ok[0] && mt.ok[1] && mt.tok[0] + kBlock <= tok_end &&
                      mt.tok[1] + kBlock <= tok_end;  // wave-uniform
    float x[2][4];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int j = 0; j < 4; ++j) x[hb][j] = sc[hb][j] * sl2;
    if (!full) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          x[hb][j] = (mt.ok[hb] && mt.tok[hb] + 4 * q + j < tok_end) ? x[hb][j] : -__builtin_huge_valf();
    }
    const float mx = max4q(max8(x));
    const bool raise = mx > mrun + kTau;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float mn = raise ? mx : mrun;
      const float f = raise ? fast_exp2(mrun - mn) : 1.f;
      mrun = mn;
      // lane (c, q) has row c's factor; its O and l entries are rows 4q .. 4q+3
      if (q == 0) s_f[c] = f;
      __builtin_amdgcn_wave_barrier();
      const float4 f4 = *reinterpret_cast<const float4 *>(&s_f[4 * q]);
      __builtin_amdgcn_wave_barrier();
      const float fr[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        l4[r] *= fr[r];
#pragma unroll
        for (int m = 0; m < EV; ++m) o[m][r] *= fr[r];
      }
    }
    float pf[8];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int j = 0; j < 4; ++j) pf[4 * hb + j] = fast_exp2(x[hb][j] - mrun);  // masked: 0
    bf16x8_t ph, pl;
    split_bf16(pf, ph, pl);
    l4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, ones, l4, 0, 0, 0);
    l4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, ones, l4, 0, 0, 0);
    const char *lv = tile + 32 * RSK;
#pragma unroll
    for (int m = 0; m < EV; ++m) {
      const bf16x8_t vb = v_operand_tr<D>(lv, RSV, m);
      o[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vb, o[m], 0, 0, 0);
      o[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, o[m], 0, 0, 0);
    }
  };

  // ---- main loop: pairs p, two stages: pair p is staged and computed while
  // pairs p + 1 and p + 2 are in flight.  The table entries of up to 64
  // blocks come from one vector load (lane j holds block c0 + j; -1 past
  // the wave's blocks), read with readlane.
  for (int c0 = 0; c0 < nb_w; c0 += 64) {
    const int cn = min(64, nb_w - c0);
    const int tv = c0 == 0 ? tv0 : load_table(a, b, blk0, ph, nph, c0, nb_w);
    auto entry = [&](int i) { return __builtin_amdgcn_readlane(tv, i); };  // i < 64
    const int np = (cn + 1) / 2;
    if (c0 > 0 || !pre) {
      issue(A, c0, entry(0), entry(1));
      if (np > 1) issue(B, c0 + 2, entry(2), entry(3));
    }
    int p = 0;
    for (; p + 3 < np; p += 2) {
      const PairMeta ma = stage(A);
      issue(A, c0 + 2 * p + 4, entry(2 * p + 4), entry(2 * p + 5));
      __builtin_amdgcn_sched_barrier(0);
      compute(ma);
      const PairMeta mb = stage(B);
      issue(B, c0 + 2 * p + 6, entry(2 * p + 6), entry(2 * p + 7));
      __builtin_amdgcn_sched_barrier(0);
      compute(mb);
    }
    // at most three pairs left: p (in A), p + 1 (in B), p + 2 (not issued)
    if (p < np) {
      const PairMeta ma = stage(A);
      if (p + 2 < np) issue(A, c0 + 2 * p + 4, entry(2 * p + 4), entry(2 * p + 5));
      __builtin_amdgcn_sched_barrier(0);
      compute(ma);
    }
    if (p + 1 < np) compute(stage(B));
    if (p + 2 < np) compute(stage(A));
  }

  // ---- the wave's state by query row hh < G: the max in lanes (hh, *);
  // sums and output rows 4q .. 4q+3 in lanes (n, q)
  if (q == 0 && c < G) s_m[w][c] = mrun;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int hh = 4 * q + r;
    if (hh < G) {
      if (c == 0) s_l[w][hh] = l4[r];
#pragma unroll
      for (int m = 0; m < EV; ++m) s_acc[w][hh][16 * m + c] = o[m][r];
    }
  }
}

// Exact combination of weighted partial states: the running maxima of the
// parts are aligned to their common maximum M.  A part that saw no valid
// token has m = kNoMax and l = acc = 0: its weight is 0 next to any part
// with a valid token (exp2(kNoMax - M) underflows) and, when no part has
// one, every weight is 1 and the sum stays 0.
__device__ __forceinline__ float part_weight(float m, float M) { return fast_exp2(m - M); }

// A workgroup barrier that orders LDS accesses only.  __syncthreads() also
// waits for every global load the wave has in flight (its release fence
// waits for all vector memory operations), which would stall the early KV
// loads of the prologue; the barriers there only publish LDS data.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sum over the workgroup, every thread gets the result.
__device__ __forceinline__ int block_sum(int x, int *part) {
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) x += __shfl_xor(x, off);
  lds_barrier();
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  lds_barrier();
  int r = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) r += part[i];
  return r;
}

// Inclusive prefix sum over the workgroup; *total gets the sum.
__device__ __forceinline__ int block_scan(int x, int *part, int *total) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off *= 2) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  lds_barrier();
  if (lane == 63) part[threadIdx.x >> 6] = x;
  lds_barrier();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int v = part[i];
    if (i < (int)(threadIdx.x >> 6)) before += v;
    all += v;
  }
  *total = all;
  return x + before;
}

// Quotient of non-negative ints (unsigned division: the shorter sequence).
__device__ __forceinline__ int udiv(int x, int y) { return (int)((unsigned)x / (unsigned)y); }

// ---------------------------------------------------------------------------
// attention kernel
//
// Work is counted in units: one unit is one 16-token block of one
// (sequence, head chunk) pair.  Units are numbered sequence-major, then
// chunk, then block, and the gridDim.x workgroups take equal contiguous
// ranges of them (the first U % gridDim.x one unit more), so every
// workgroup streams the same number of blocks whatever the mix of context
// lengths.  A range is cut at (sequence, chunk) boundaries into pieces.  A
// piece that is a whole (sequence, chunk) is finished on the spot: its
// normalised output is written.  A pair split over several ranges leaves a
// partial state per piece in the workspace (record slot 0 for the piece a
// range starts with, slot 1 for the piece it ends with); the last of those
// pieces to finish, found with an arrival counter, merges them.  The
// counters (one per workgroup) are zero before the launch and the merging
// workgroup sets its counter back to zero.

template <int KV, int D, int G>
__global__ __launch_bounds__(kThreads) void attention_kernel(LaunchArgs a) {
  __shared__ float s_acc[kWaves][G][D];
  __shared__ float s_m[kWaves][G], s_l[kWaves][G];
  __shared__ int s_scan[kWaves];
  __shared__ int s_first[3];  // first sequence, its first unit, its length
  __shared__ int s_len[kThreads];     // clamped lengths, when batch <= kThreads
  __shared__ int s_last;
  // per-wave staging tiles and rescale factors of the matrix-core form
  __shared__ __align__(16) char s_tile[uses_mfma<KV>() ? kWaves * MCfg<KV, D>::TILE : 16];
  __shared__ __align__(16) float s_fw[kWaves][16];

  const int tid = threadIdx.x;
  // wave index, known wave-uniform: everything derived from it stays scalar
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwg = gridDim.x, wgi = blockIdx.x;
  // head chunk of an equal-length batch (a.hc): the speculation below uses it.
  // Head chunks are powers of two dividing kWaves.
  const int hc0 = a.hc, lhc0 = __builtin_ctz(hc0);
  const int nph0 = kWaves >> lhc0, hl0 = w & (hc0 - 1), ph0 = w >> lhc0;

  auto seq_len = [&](int b) { return min(max(a.ctx[b], 0), a.max_ctx); };
  auto seq_blocks = [&](int b) { return (seq_len(b) + kBlock - 1) / kBlock; };
  const bool small_batch = a.batch <= kThreads;  // lengths kept in LDS
  // a length after the scan: from LDS for a small batch, else from memory
  auto len_of = [&](int b) { return small_batch ? s_len[b] : seq_len(b); };

  // ---- speculation: the first piece this workgroup gets if every context
  // is max_ctx long (an equal-length batch).  Its query rows and table
  // entries are loaded now, in flight together with the lengths the split
  // below needs, and used if the lengths confirm the guess.
  // Unit counts and indices are 32-bit: the host rejects a launch whose
  // batch * num_kv_heads * ceil(max_ctx / 16) reaches 2^31.  (64-bit
  // divisions expand to long instruction sequences, which held back every
  // workgroup's first loads by microseconds.)
  const int nbm = (a.max_ctx + kBlock - 1) / kBlock;
  const int Ug = a.batch * a.chunks * nbm;
  Query<KV, D, G> qry_g;
  int tv_g = -1;
  bool guess = false;  // early loads for the guessed piece: KV head g_g, tokens [tok0_g, tok_end_g)
  int g_g = 0, tok0_g = 0, tok_end_g = 0;
  {
    const int per_g = udiv(Ug, nwg), rem_g = Ug - per_g * nwg;
    const int u0g = wgi * per_g + min(wgi, rem_g);
    const int u1g = u0g + per_g + (wgi < rem_g ? 1 : 0);
    if (u0g < u1g) {
      const int seq_units = a.chunks * nbm;
      const int bg = udiv(u0g, seq_units);
      const int off = u0g - bg * seq_units;
      const int cg = udiv(off, nbm), lo = off - cg * nbm;
      const int hi = min(nbm, u1g - bg * seq_units - cg * nbm);
      // worth loading early only if the guessed sequence has the full
      // length (its length lands in the same round trip as the table)
      guess = seq_len(bg) == a.max_ctx;
      g_g = cg * hc0 + hl0;
      tok0_g = lo * kBlock;
      tok_end_g = min(a.max_ctx, hi * kBlock);
      load_query<KV, D, G>(a, bg, g_g, qry_g);
      tv_g = load_table(a, bg, lo, ph0, nph0, 0, wave_blocks(tok0_g, tok_end_g, ph0, nph0));
    }
  }

  // ---- total blocks TB, from which the head chunk, the total units
  // U = TB * chunks, this workgroup's range [u0, u1) and the sequence holding
  // u0.  Up to kThreads sequences: one block-wide scan of the per-sequence
  // blocks gives all of them.  More: a sum, then a chunked scan below.
  if (tid == 0) s_first[0] = -1;
  int TB, incl_b = 0;
  int my_len = 0;
  if (small_batch) my_len = tid < a.batch ? seq_len(tid) : 0;
  // Matrix-core form: the guessed piece's first KV loads go out as soon as
  // its table entries land, in flight during the scan below (unused when
  // the guess fails; every address is inside the pools).
  PairLoads<KV, D> pA, pB;
  if constexpr (uses_mfma<KV>()) {
    if (guess) issue_first_pairs<KV, D>(a, g_g, tok0_g, tok_end_g, ph0, nph0, tv_g, pA, pB);
  }
  if (small_batch) {
    s_len[tid] = my_len;
    incl_b = block_scan((my_len + kBlock - 1) / kBlock, s_scan, &TB);
  } else {
    int t = 0;
    for (int b = tid; b < a.batch; b += kThreads) t += seq_blocks(b);
    TB = block_sum(t, s_scan);
  }
  // The head chunk: a.hc when every sequence has max_ctx's block count (the
  // equal-length batch the host sized it for), else a.hc_var.  No sequence
  // has more blocks than max_ctx, so that is exactly TB == batch * nbm.
  const bool full = __builtin_amdgcn_readfirstlane((int)(TB == a.batch * nbm)) != 0;
  const int hc = full ? a.hc : a.hc_var, lhc = __builtin_ctz(hc);
  const int chunks = a.hkv >> lhc;
  const int nph = kWaves >> lhc;  // phases: waves sharing a head
  const int hl = w & (hc - 1), ph = w >> lhc;
  const int hcg = hc * G;       // query heads of a chunk
  const int U = TB * chunks;
  const int per = udiv(U, nwg), rem = U - per * nwg;
  auto range_start = [&](int wg) { return wg * per + min(wg, rem); };
  auto range_of = [&](int u) {  // workgroup whose range holds unit u
    const int big = rem * (per + 1);
    return u < big ? udiv(u, per + 1) : rem + udiv(u - big, per);
  };
  const int u0 = range_start(wgi), u1 = range_start(wgi + 1);
  if (small_batch) {
    const int ub = ((my_len + kBlock - 1) / kBlock) * chunks;
    const int incl = incl_b * chunks;
    if (ub > 0 && incl - ub <= u0 && u0 < incl) {
      s_first[0] = tid;
      s_first[1] = incl - ub;
      s_first[2] = my_len;
    }
  }

  // empty sequences: zero output rows, spread over the workgroups (done
  // after this workgroup's pieces, off the path to its first loads)
  auto zero_empty_rows = [&]() {
    for (int b = wgi; b < a.batch; b += nwg) {
      if (len_of(b) == 0)
        for (int i = tid; i < a.hq * D; i += kThreads) a.out[(size_t)b * a.hq * D + i] = 0.f;
    }
  };
  if (u0 >= u1) {
    __syncthreads();  // s_len complete
    zero_empty_rows();
    return;
  }

  if (a.batch > kThreads) {
    int base = 0;
    for (int c0 = 0; c0 < a.batch; c0 += kThreads) {
      const int b = c0 + tid;
      const int ub = b < a.batch ? seq_blocks(b) * chunks : 0;
      int total;
      const int incl = block_scan(ub, s_scan, &total);
      const int start = base + incl - ub;
      if (ub > 0 && start <= u0 && u0 < start + ub) {
        s_first[0] = b;
        s_first[1] = start;
        s_first[2] = seq_len(b);
      }
      lds_barrier();
      base += total;
      if (s_first[0] >= 0) break;
    }
  }
  lds_barrier();
  int b = s_first[0];
  int pb = s_first[1];  // first unit of sequence b
  int n = s_first[2];   // its length (the scan has read it already)

  // ---- the pieces of the range
  int pos = u0;
  bool first_piece = true;
  while (pos < u1) {
    const int nb = (n + kBlock - 1) / kBlock;
    const int ub = nb * chunks;
    if (ub == 0) {  // an empty sequence inside the range holds no units
      ++b;
      n = len_of(b);
      continue;
    }
    // the next sequence's length, read now and used after this piece
    const int n_next = b + 1 < a.batch ? len_of(b + 1) : 0;
    const int off = pos - pb;
    const int chunk = udiv(off, nb);
    const int blk_lo = off - chunk * nb;
    const int seg_start = pb + chunk * nb, seg_end = seg_start + nb;
    const int pend = min(u1, seg_end);
    const int blk_hi = pend - seg_start;

    const int g = chunk * hc + hl;
    const int tok0 = blk_lo * kBlock, tok_end = min(n, blk_hi * kBlock);
    // the guess holds when every sequence has max_ctx tokens' worth of
    // blocks and this one exactly max_ctx tokens: then the first piece is
    // the guessed one, same blocks and same tail
    auto piece = [&](const Query<KV, D, G> &qr, int tvr, bool pre) {
      if constexpr (uses_mfma<KV>())
        attend_piece_mfma<KV, D, G>(a, b, g, tok0, tok_end, ph, nph, w, qr, tvr, s_acc, s_m, s_l,
                                    s_tile + (uses_mfma<KV>() ? w * MCfg<KV, D>::TILE : 0), s_fw[w],
                                    pA, pB, pre);
      else
        attend_piece<KV, D, G>(a, b, g, tok0, tok_end, ph, nph, w, qr, tvr, s_acc, s_m, s_l);
    };
    if (first_piece && full && U == Ug && n == a.max_ctx) {
      piece(qry_g, tv_g, guess);  // guess: its first pairs are in flight
    } else {
      Query<KV, D, G> qry;
      load_query<KV, D, G>(a, b, g, qry);
      piece(qry, load_table(a, b, blk_lo, ph, nph, 0, wave_blocks(tok0, tok_end, ph, nph)), false);
    }
    __syncthreads();

    // combine the phases of each head; then output or partial record
    const size_t bh0 = (size_t)b * a.hq + (size_t)chunk * hcg;
    const bool whole = blk_lo == 0 && blk_hi == nb;
    const size_t rec0 = ((size_t)wgi * 2 + (first_piece ? 0 : 1)) * hcg;
    for (int idx = tid; idx < hcg * D; idx += kThreads) {
      const int r = idx / D, e = idx % D;  // r = hl * G + hh
      const int hh = r % G, hw = r / G;
      // the waves of head hw are hw, hw + hc, ... (nph of them); every
      // part's values are read at once (a part past nph re-reads part 0 and
      // gets weight 0, which leaves the sums exactly those of the nph parts)
      float mv[kWaves], lv[kWaves], av[kWaves];
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const int wv = (v < nph ? v : 0) * hc + hw;
        mv[v] = s_m[wv][hh];
        lv[v] = s_l[wv][hh];
        av[v] = s_acc[wv][hh][e];
      }
      float M = kNoMax;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) M = fmaxf(M, mv[v]);
      float A = 0.f, L = 0.f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const float sc = v < nph ? part_weight(mv[v], M) : 0.f;
        A = fmaf(sc, av[v], A);
        L = fmaf(sc, lv[v], L);
      }
      if (whole) {
        a.out[(bh0 + r) * D + e] = L > 0.f ? A / L : 0.f;
      } else {
        // device-coherent stores: see the arrival below
        __hip_atomic_store(&a.ws_acc[(rec0 + r) * D + e], A, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (e == 0) {
          float *ml = reinterpret_cast<float *>(&a.ws_ml[rec0 + r]);
          __hip_atomic_store(ml, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(ml + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }

    if (!whole) {
      // Arrival.  The record was stored with device-coherent (write-through)
      // stores, and each wave waits until its own stores are complete (the
      // barrier by itself does not wait for outstanding stores), so the
      // record is in device-coherent memory before thread 0 counts the
      // arrival; a release on the counter would add a write-back of the
      // whole L2, which measured 2% of the continuous-batch step.  The
      // arrival that completes the count takes a device-scope acquire
      // (its L2 is invalidated, so its loads of the records fetch them
      // afresh) and the barrier hands that on.
      // The pair's counter is indexed by the first workgroup it touches: a
      // range holds the first unit of at most one pair that runs past its
      // end, so no two split pairs share a counter.
      const int w_lo = range_of(seg_start), w_hi = range_of(seg_end - 1);
      uint32_t *cnt = a.counters + w_lo;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        const bool last = old == (uint32_t)(w_hi - w_lo);
        if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s_last = last;
      }
      __syncthreads();
      if (s_last) {
        // the record of piece k = w_lo + j: slot 0 unless the pair starts
        // inside w_lo's range after its first unit (then it ends that range)
        const int np = (int)(w_hi - w_lo + 1);
        const int slot_lo = range_start(w_lo) == seg_start ? 0 : 1;
        auto rec_of = [&](int j) {
          return ((size_t)(w_lo + j) * 2 + (j == 0 ? slot_lo : 0)) * hcg;
        };
        const float4 *acc4 = reinterpret_cast<const float4 *>(a.ws_acc);
        for (int idx = tid; idx < hcg * (D / 4); idx += kThreads) {
          const int r = idx / (D / 4), c4 = idx % (D / 4);
          float M = kNoMax;
          for (int j = 0; j < np; ++j) M = fmaxf(M, a.ws_ml[rec_of(j) + r].x);
          float L = 0.f;
          float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
          auto add = [&](float2 ml, float4 v) {
            const float sc = part_weight(ml.x, M);
            L = fmaf(sc, ml.y, L);
            A.x = fmaf(sc, v.x, A.x); A.y = fmaf(sc, v.y, A.y);
            A.z = fmaf(sc, v.z, A.z); A.w = fmaf(sc, v.w, A.w);
          };
          int j = 0;
          for (; j + 4 <= np; j += 4) {  // four pieces' loads in flight
            float2 ml[4];
            float4 v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const size_t rr = rec_of(j + k) + r;
              ml[k] = a.ws_ml[rr];
              v[k] = acc4[rr * (D / 4) + c4];
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) add(ml[k], v[k]);
          }
          for (; j < np; ++j) {
            const size_t rr = rec_of(j) + r;
            add(a.ws_ml[rr], acc4[rr * (D / 4) + c4]);
          }
          float *o = a.out + (bh0 + r) * D + 4 * c4;  // out needs only 4-byte alignment
          o[0] = L > 0.f ? A.x / L : 0.f;
          o[1] = L > 0.f ? A.y / L : 0.f;
          o[2] = L > 0.f ? A.z / L : 0.f;
          o[3] = L > 0.f ? A.w / L : 0.f;
        }
        if (tid == 0)  // ready for the next run (ordered by the kernel boundary)
          __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();  // LDS is reused by the next piece

    first_piece = false;
    pos = pend;
    if (pos == pb + ub) {
      pb += ub;
      ++b;
      n = n_next;
    }
  }
  zero_empty_rows();
}

__global__ __launch_bounds__(256) void zero_kernel(uint32_t *p, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

template <int KV, int D, int G>
hipError_t launch_attention_t(const LaunchArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (e0)  // events attached to the dispatch: the kernel's own start and end
    hipExtLaunchKernelGGL((attention_kernel<KV, D, G>), dim3((unsigned)a.nwg), dim3(kThreads), 0, s,
                          e0, e1, 0, a);
  else
    hipLaunchKernelGGL((attention_kernel<KV, D, G>), dim3((unsigned)a.nwg), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int KV, int D>
hipError_t by_group(const LaunchArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (a.hq / a.hkv) {
    case 1: return launch_attention_t<KV, D, 1>(a, s, e0, e1);
    case 2: return launch_attention_t<KV, D, 2>(a, s, e0, e1);
    case 4: return launch_attention_t<KV, D, 4>(a, s, e0, e1);
    case 8: return launch_attention_t<KV, D, 8>(a, s, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

template <int KV>
hipError_t by_dim(const LaunchArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (a.d) {
    case 64: return by_group<KV, 64>(a, s, e0, e1);
    case 128: return by_group<KV, 128>(a, s, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool kernel_supported(int kv, int d, int group) {
  return (kv == KV_F32 || kv == KV_BF16 || kv == KV_FP8) && (d == 64 || d == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_attention(const LaunchArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (a.batch == 0 || a.nwg == 0) return hipSuccess;
  switch (a.kv) {
    case KV_F32: return by_dim<KV_F32>(a, s, e0, e1);
    case KV_BF16: return by_dim<KV_BF16>(a, s, e0, e1);
    case KV_FP8: return by_dim<KV_FP8>(a, s, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// Scratch of pa_decode_run_noalloc, for callers that cannot allocate: a
// file-scope device array (each GPU the library runs on holds its own copy,
// at its own address, until the process ends).  Host code never uses the
// array's name as an address (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, taken once per
// device with that device current and kept.

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void **ptr) {
  static std::mutex mu;
  static std::vector<void *> per_device;  // device address of scratch, by device id
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if ((size_t)dev >= per_device.size()) per_device.resize((size_t)dev + 1, nullptr);
  if (!per_device[dev]) {
    void *p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

hipError_t launch_zero(uint32_t *p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace pa
