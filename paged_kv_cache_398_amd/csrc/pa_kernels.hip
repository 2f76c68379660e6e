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
// How:
//
// 1. partition_kernel: one workgroup of kWaves waves per (sequence, chunk of
//    hc adjacent KV heads, context partition).  Wave w works on head
//    w % hc of the chunk and takes every (kWaves/hc)-th 16-token block of the
//    partition, so the workgroup as a whole reads the hc heads' rows of
//    every block it touches: hc * head_dim * elem bytes contiguous per token.
//    A wave holds a whole block of its head in registers: each token row is
//    split over LPT lanes, 64/LPT tokens per pass, with 8- or 16-byte loads
//    per lane.  Every K/V element is loaded from HBM once and used by all G
//    query heads of its group, which sit in the same lane's registers.  The
//    loop is a two-stage software pipeline: the next block's loads are in
//    flight while the current block is computed, and the block table of up
//    to 64 blocks is read by one vector load before it starts.
//    Scores are reduced over the LPT lanes of a token with DPP.  The
//    softmax is accumulated online (running max and sum, as in the
//    FlashAttention sections of the pages): the running max is kept
//    wave-uniform and is only raised when a block's maximum exceeds it by
//    more than kTau (log2 units), so the rescale of the accumulators is
//    rare; any running max gives the same normalised result, it only bounds
//    the exponentials (by 2^kTau).  At the end the lanes' states and the
//    phases of each head are combined exactly in LDS.  With one partition
//    the normalised output is written directly; otherwise (max, sum,
//    unnormalised output) per query head and partition.
//
// 2. merge_kernel (only with several partitions): one workgroup per
//    (sequence, query head) combines the partitions: M = max_p m_p,
//    w_p = 2^(m_p - M), out = sum w_p acc_p / sum w_p l_p.
//
// Positions past a sequence's length contribute exactly nothing (selects,
// not multiplications, so NaN garbage in unused slots cannot leak), table
// entries past the last used block are never read, and block ids outside
// [0, num_blocks) are never dereferenced: block 0 is read in their place and
// masked out.

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kBlock = 16;         // tokens per physical block
constexpr int kThreads = kWaves * 64;
constexpr float kTau = 8.0f;       // lag allowed to the running max (log2 units)

__host__ __device__ constexpr int elem_bytes(int kv) {
  return kv == KV_F32 ? 4 : (kv == KV_BF16 ? 2 : 1);
}

#ifndef PA_ACC_REGS
#define PA_ACC_REGS 64
#endif
// Lanes per token row: as few as possible while keeping the per-lane output
// accumulators (G * D / LPT floats) at PA_ACC_REGS registers or fewer, and
// each lane's slice of a row at 8 bytes or more.
__host__ __device__ constexpr int lanes_per_token(int d, int g, int eb) {
  int l = (g * d / 4 <= PA_ACC_REGS) ? 4 : ((g * d / 8 <= PA_ACC_REGS) ? 8 : 16);
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

template <int CH>
__device__ __forceinline__ void load_chunk(const char *p, uint32_t *dst) {
  if constexpr (CH == 16) {
    const uint4 x = *reinterpret_cast<const uint4 *>(p);
    dst[0] = x.x; dst[1] = x.y; dst[2] = x.z; dst[3] = x.w;
  } else {
    static_assert(CH == 8, "8- or 16-byte loads only");
    const uint2 x = *reinterpret_cast<const uint2 *>(p);
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

template <int KV, int D, int G>
__global__ __launch_bounds__(kThreads) void partition_kernel(LaunchArgs a) {
  using C = Cfg<KV, D, G>;
  constexpr int LPT = C::LPT, NPASS = C::NPASS, DW = C::DW, EPL = C::EPL;
  const int lane = threadIdx.x & 63;
  // wave index, known wave-uniform: everything derived from it stays scalar
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane % LPT;   // which slice of the row
  const int slot = lane / LPT;  // which token of the pass

  // workgroup -> (sequence, head chunk, partition); partitions fastest
  int u = blockIdx.x;
  const int part = u % a.parts;
  u /= a.parts;
  const int chunk = u % a.chunks;
  const int b = u / a.chunks;
  // wave -> (KV head of the chunk, phase); the phases of a head split its blocks
  const int hc = a.hc;
  const int nph = kWaves / hc;
  const int hl = w % hc;
  const int ph = w / hc;
  const int g = chunk * hc + hl;
  const int h0 = g * G;  // first query head of this wave's group

  const int n = min(max(a.ctx[b], 0), a.max_ctx);
  const int tok0 = part * a.part_tokens;
  if (tok0 >= n) {  // whole workgroup: nothing of this sequence here
    if (part == 0) {  // empty sequence: its output rows are zero
      for (int idx = threadIdx.x; idx < hc * G * D; idx += kThreads)
        a.out[((size_t)b * a.hq + chunk * hc * G) * D + idx] = 0.f;
    }
    return;
  }
  const int tok_end = min(n, tok0 + a.part_tokens);
  const int blk0 = tok0 / kBlock;
  const int nblk = (tok_end - tok0 + kBlock - 1) / kBlock;
  const int nb_w = nblk > ph ? (nblk - ph + nph - 1) / nph : 0;

  // ---- query slice of the G heads of this group (lane-local elements)
  float qf[G][EPL];
  uint32_t q2[G][DW];  // bf16 pairs (bf16 pools only)
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

  // ---- lane offsets inside a block, and the block table of this wave
  const size_t block_bytes = (size_t)kBlock * a.hkv * C::ROW;
  uint32_t lane_off[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p)
    lane_off[p] = (uint32_t)(((p * C::TPP + slot) * a.hkv + g) * C::ROW + sub * C::CH);
  // i-th block of this wave: table entry trow[i * nph]
  const int *trow = a.table + (size_t)b * a.max_blocks + blk0 + ph;
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
        load_chunk<C::CH>(kb + (lane_off[p] + c * LPT * C::CH), &bk.k[p][c * (C::CH / 4)]);
        load_chunk<C::CH>(vb + (lane_off[p] + c * LPT * C::CH), &bk.v[p][c * (C::CH / 4)]);
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
    m[hh] = -__builtin_huge_valf();
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

  // ---- main loop: a two-stage pipeline over the wave's blocks, block i+1 in
  // flight while block i is computed.  The table entries of up to 64 blocks
  // are fetched by one vector load (lane j holds block c0 + j) before the
  // pipeline starts, so the loop itself reads nothing but K and V.
  for (int c0 = 0; c0 < nb_w; c0 += 64) {
    const int cn = min(64, nb_w - c0);
    const int tv = c0 + lane < nb_w ? trow[(size_t)(c0 + lane) * nph] : -1;
    auto entry = [&](int i) { return __builtin_amdgcn_readlane(tv, min(i, cn - 1)); };
    Block<KV, D, G> A, B;
    issue(A, c0, entry(0));
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
  __shared__ float s_acc[kWaves][G][D];
  __shared__ float s_m[kWaves][G], s_l[kWaves][G];
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
  __syncthreads();
  // outputs of this workgroup: hc heads x G query rows x D, query heads
  // chunk*hc*G .. (chunk+1)*hc*G - 1 of sequence b
  const size_t bh0 = (size_t)b * a.hq + (size_t)chunk * hc * G;
  for (int idx = threadIdx.x; idx < hc * G * D; idx += kThreads) {
    const int r = idx / D, e = idx % D;  // r = hl * G + hh
    const int hh = r % G, hw = r / G;
    float M = -__builtin_huge_valf();
    for (int v = 0; v < nph; ++v) M = fmaxf(M, s_m[v * hc + hw][hh]);
    float A = 0.f, L = 0.f;
    for (int v = 0; v < nph; ++v) {
      const int wv = v * hc + hw;
      const float mv = s_m[wv][hh];
      const float sc = mv == -__builtin_huge_valf() ? 0.f : fast_exp2(mv - M);
      A = fmaf(sc, s_acc[wv][hh][e], A);
      L = fmaf(sc, s_l[wv][hh], L);
    }
    if (a.parts == 1) {
      a.out[(bh0 + r) * D + e] = L > 0.f ? A / L : 0.f;
    } else {
      const size_t rec = (bh0 + r) * a.parts + part;
      a.ws_acc[rec * D + e] = A;
      if (e == 0) a.ws_ml[rec] = make_float2(M, L);
    }
  }
}

// ---------------------------------------------------------------------------
// merge kernel: one workgroup of kMergeThreads per (sequence, query head)
//
// M = max_p m_p; w_p = 2^(m_p - M) (0 for a partition that saw no valid
// token); out = sum_p w_p acc_p / sum_p w_p l_p.  The partitions are spread
// over the workgroup: thread t takes columns 4*(t % (D/4)) .. +3 of every
// (kMergeThreads / (D/4))-th partition, with four partitions' loads in flight.

constexpr int kMergeThreads = 256;

__device__ __forceinline__ float block_reduce(float x, float *scratch, bool is_max) {
  // wave reduction (every lane ends with the result), then across waves
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) {
    const float y = __shfl_xor(x, off);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) scratch[w] = x;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int i = 1; i < kMergeThreads / 64; ++i) r = is_max ? fmaxf(r, scratch[i]) : r + scratch[i];
  __syncthreads();
  return r;
}

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(LaunchArgs a) {
  constexpr int C4 = D / 4;                    // float4 columns of a row
  constexpr int NG = kMergeThreads / C4;       // partition groups
  const size_t bh = blockIdx.x;
  const int b = (int)(bh / a.hq);
  const int n = min(max(a.ctx[b], 0), a.max_ctx);
  const int np = (n + a.part_tokens - 1) / a.part_tokens;
  float *o = a.out + bh * D;
  if (np == 0) {
    for (int e = threadIdx.x; e < D; e += kMergeThreads) o[e] = 0.f;
    return;
  }
  const float2 *ml = a.ws_ml + bh * a.parts;
  const float4 *acc4 = reinterpret_cast<const float4 *>(a.ws_acc + bh * a.parts * D);
  __shared__ float s_red[kMergeThreads / 64];
  __shared__ float4 s_part[NG][C4];

  float mx = -__builtin_huge_valf();
  for (int p = threadIdx.x; p < np; p += kMergeThreads) mx = fmaxf(mx, ml[p].x);
  const float M = block_reduce(mx, s_red, true);
  const auto weight = [&](float m) { return m == -__builtin_huge_valf() ? 0.f : fast_exp2(m - M); };
  float lw = 0.f;
  for (int p = threadIdx.x; p < np; p += kMergeThreads) {
    const float2 v = ml[p];
    lw = fmaf(weight(v.x), v.y, lw);
  }
  const float L = block_reduce(lw, s_red, false);

  const int c = threadIdx.x % C4, grp = threadIdx.x / C4;
  float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](float w, float4 v) {
    A.x = fmaf(w, v.x, A.x); A.y = fmaf(w, v.y, A.y);
    A.z = fmaf(w, v.z, A.z); A.w = fmaf(w, v.w, A.w);
  };
  int p = grp;
  for (; p + 3 * NG < np; p += 4 * NG) {
    float4 v[4];
    float w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = acc4[(size_t)(p + k * NG) * C4 + c];
      w[k] = ml[p + k * NG].x;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) add(weight(w[k]), v[k]);
  }
  for (; p < np; p += NG) add(weight(ml[p].x), acc4[(size_t)p * C4 + c]);
  s_part[grp][c] = A;
  __syncthreads();
  if (threadIdx.x < C4) {
    float4 t = s_part[0][threadIdx.x];
#pragma unroll
    for (int g = 1; g < NG; ++g) {
      const float4 u = s_part[g][threadIdx.x];
      t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
    }
    float *oo = o + 4 * threadIdx.x;  // out needs only 4-byte alignment
    oo[0] = L > 0.f ? t.x / L : 0.f;
    oo[1] = L > 0.f ? t.y / L : 0.f;
    oo[2] = L > 0.f ? t.z / L : 0.f;
    oo[3] = L > 0.f ? t.w / L : 0.f;
  }
}

template <int KV, int D, int G>
hipError_t launch_partition_t(const LaunchArgs &a, hipStream_t s) {
  const size_t wgs = (size_t)a.batch * a.chunks * a.parts;
  hipLaunchKernelGGL((partition_kernel<KV, D, G>), dim3((unsigned)wgs), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int KV, int D>
hipError_t by_group(const LaunchArgs &a, hipStream_t s) {
  switch (a.hq / a.hkv) {
    case 1: return launch_partition_t<KV, D, 1>(a, s);
    case 2: return launch_partition_t<KV, D, 2>(a, s);
    case 4: return launch_partition_t<KV, D, 4>(a, s);
    case 8: return launch_partition_t<KV, D, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int KV>
hipError_t by_dim(const LaunchArgs &a, hipStream_t s) {
  switch (a.d) {
    case 64: return by_group<KV, 64>(a, s);
    case 128: return by_group<KV, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool kernel_supported(int kv, int d, int group) {
  return (kv == KV_F32 || kv == KV_BF16 || kv == KV_FP8) && (d == 64 || d == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_partition(const LaunchArgs &a, hipStream_t s) {
  if (a.batch == 0 || a.parts == 0) return hipSuccess;
  switch (a.kv) {
    case KV_F32: return by_dim<KV_F32>(a, s);
    case KV_BF16: return by_dim<KV_BF16>(a, s);
    case KV_FP8: return by_dim<KV_FP8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_merge(const LaunchArgs &a, hipStream_t s) {
  if (a.batch == 0 || a.parts <= 1) return hipSuccess;
  const unsigned wgs = (unsigned)((size_t)a.batch * a.hq);
  if (a.d == 64)
    hipLaunchKernelGGL((merge_kernel<64>), dim3(wgs), dim3(kMergeThreads), 0, s, a);
  else if (a.d == 128)
    hipLaunchKernelGGL((merge_kernel<128>), dim3(wgs), dim3(kMergeThreads), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
