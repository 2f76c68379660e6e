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
// How (two kernels, always both):
//
// 1. partition_kernel: one workgroup of kWaves waves per (sequence, KV head,
//    context partition).  The partition's 16-token blocks are dealt
//    round-robin to the waves.  A wave reads a whole block per step: each
//    token row (head_dim elements of one KV head) is split over LPT lanes,
//    64/LPT tokens per pass, 16/LPT*4 passes per block, with 8- or 16-byte
//    loads per lane so every load instruction reads whole 64-256 B row
//    segments.  Every K/V element is loaded from HBM once and used by all G
//    query heads of its group, which sit in the same lane's registers.
//    Scores are reduced over the LPT lanes of a token with DPP.  The
//    softmax is accumulated online (running max and sum, as in the
//    FlashAttention sections of the pages): the running max is kept
//    wave-uniform and is only raised when a block's maximum exceeds it by
//    more than kTau (log2 units), so the rescale of the accumulators is
//    rare; any running max gives the same normalised result, it only bounds
//    the exponentials (by 2^kTau).  At the end the lanes' and waves' states
//    are combined exactly and written as (max, sum, unnormalised output).
//
// 2. merge_kernel: one wave per (sequence, query head) combines the
//    partitions: M = max_p m_p, w_p = 2^(m_p - M), out = sum w_p acc_p /
//    sum w_p l_p.
//
// Positions past a sequence's length contribute exactly nothing (selects,
// not multiplications, so NaN garbage in unused slots cannot leak), table
// entries past the last used block are never read, and block ids outside
// [0, num_blocks) are skipped rather than dereferenced.

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kBlock = 16;         // tokens per physical block
constexpr int kThreads = kWaves * 64;
constexpr float kTau = 8.0f;       // lag allowed to the running max (log2 units)

__host__ __device__ constexpr int elem_bytes(int kv) {
  return kv == KV_F32 ? 4 : (kv == KV_BF16 ? 2 : 1);
}

// Lanes per token row: as few as possible while keeping the per-lane output
// accumulators (G * D / LPT floats) at 64 registers or fewer.
__host__ __device__ constexpr int lanes_per_token(int d, int g) {
  return (g * d / 4 <= 64) ? 4 : ((g * d / 8 <= 64) ? 8 : 16);
}

template <int KV, int D, int G>
struct Cfg {
  static constexpr int EB = elem_bytes(KV);
  static constexpr int LPT = lanes_per_token(D, G);
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
// partition kernel

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
  const int w = threadIdx.x >> 6;
  const int sub = lane % LPT;   // which slice of the row
  const int slot = lane / LPT;  // which token of the pass

  int u = blockIdx.x;
  const int g = u % a.hkv;
  u /= a.hkv;
  const int b = u % a.batch;
  const int part = u / a.batch;

  const int n = min(max(a.ctx[b], 0), a.max_ctx);
  const int tok0 = part * a.part_tokens;
  if (tok0 >= n) return;  // whole workgroup: nothing of this sequence here
  const int tok_end = min(n, tok0 + a.part_tokens);
  const int blk0 = tok0 / kBlock;
  const int nblk = (tok_end - tok0 + kBlock - 1) / kBlock;
  const int nb_w = nblk > w ? (nblk - w + kWaves - 1) / kWaves : 0;

  // ---- query slice of the G heads of this group (lane-local elements)
  const int h0 = g * G;
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
  int lane_off[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p)
    lane_off[p] = ((p * C::TPP + slot) * a.hkv + g) * C::ROW + sub * C::CH;
  const int *trow = a.table + (size_t)b * a.max_blocks + blk0 + w;  // i-th block: trow[i*kWaves]
  const char *kbase = static_cast<const char *>(a.k_cache);
  const char *vbase = static_cast<const char *>(a.v_cache);
  int tv = -1;  // lane j holds the id of this wave's block (i & ~63) + j

  auto issue = [&](Block<KV, D, G> &bk, int i) {
    if ((i & 63) == 0) {
      const int idx = i + lane;
      tv = idx < nb_w ? trow[(size_t)idx * kWaves] : -1;
    }
    const int phys = __builtin_amdgcn_readlane(tv, i & 63);
    bk.tok = (blk0 + w + i * kWaves) * kBlock;
    bk.ok = (unsigned)phys < (unsigned)a.num_blocks;
    if (!bk.ok) return;
    const char *kb = kbase + (size_t)phys * block_bytes;
    const char *vb = vbase + (size_t)phys * block_bytes;
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
#pragma unroll
      for (int c = 0; c < C::NCH; ++c) {
        load_chunk<C::CH>(kb + lane_off[p] + c * LPT * C::CH, &bk.k[p][c * (C::CH / 4)]);
        load_chunk<C::CH>(vb + lane_off[p] + c * LPT * C::CH, &bk.v[p][c * (C::CH / 4)]);
      }
      if constexpr (KV == KV_FP8) {
        const size_t si = ((size_t)phys * a.hkv + g) * kBlock + p * C::TPP + slot;
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
    if (!bk.ok) return;
    const bool tail = bk.tok + kBlock > tok_end;  // wave-uniform
    float s[NPASS][G];
    bool live[NPASS];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      live[p] = !tail || (bk.tok + p * C::TPP + slot < tok_end);
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

  // ---- main loop, one block in flight while the previous is computed
  {
    Block<KV, D, G> A, B;
    if (nb_w > 0) issue(A, 0);
    for (int i = 0; i < nb_w; i += 2) {
      if (i + 1 < nb_w) issue(B, i + 1);
      compute(A);
      if (i + 1 < nb_w) {
        if (i + 2 < nb_w) issue(A, i + 2);
        compute(B);
      }
    }
  }

  // ---- combine the wave's token slots, then the waves, exactly
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
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int hh = idx / D, e = idx % D;
    float M = s_m[0][hh];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) M = fmaxf(M, s_m[v][hh]);
    float A = 0.f, L = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float mv = s_m[v][hh];
      const float sc = mv == -__builtin_huge_valf() ? 0.f : fast_exp2(mv - M);
      A = fmaf(sc, s_acc[v][hh][e], A);
      L = fmaf(sc, s_l[v][hh], L);
    }
    const size_t rec = ((size_t)b * a.hq + h0 + hh) * a.parts + part;
    a.ws_acc[rec * D + e] = A;
    if (e == 0) a.ws_ml[rec] = make_float2(M, L);
  }
}

// ---------------------------------------------------------------------------
// merge kernel: one wave per (sequence, query head)

template <int D>
__global__ __launch_bounds__(64) void merge_kernel(LaunchArgs a) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x;
  const size_t bh = blockIdx.x;
  const int b = (int)(bh / a.hq);
  const int n = min(max(a.ctx[b], 0), a.max_ctx);
  const int np = (n + a.part_tokens - 1) / a.part_tokens;
  float *o = a.out + bh * D;
  if (np == 0) {
#pragma unroll
    for (int k = 0; k < PER; ++k) o[lane + 64 * k] = 0.f;
    return;
  }
  const float2 *ml = a.ws_ml + bh * a.parts;
  const float *acc = a.ws_acc + bh * a.parts * D;
  float M = -__builtin_huge_valf();
  for (int p = 0; p < np; ++p) M = fmaxf(M, ml[p].x);
  float L = 0.f, A[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) A[k] = 0.f;
  for (int p = 0; p < np; ++p) {
    const float2 v = ml[p];
    const float sc = v.x == -__builtin_huge_valf() ? 0.f : fast_exp2(v.x - M);
    L = fmaf(sc, v.y, L);
#pragma unroll
    for (int k = 0; k < PER; ++k) A[k] = fmaf(sc, acc[(size_t)p * D + lane + 64 * k], A[k]);
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) o[lane + 64 * k] = L > 0.f ? A[k] / L : 0.f;
}

template <int KV, int D, int G>
hipError_t launch_partition_t(const LaunchArgs &a, hipStream_t s) {
  const size_t wgs = (size_t)a.batch * a.hkv * a.parts;
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
  if (a.batch == 0) return hipSuccess;
  const unsigned wgs = (unsigned)((size_t)a.batch * a.hq);
  if (a.d == 64)
    hipLaunchKernelGGL((merge_kernel<64>), dim3(wgs), dim3(64), 0, s, a);
  else if (a.d == 128)
    hipLaunchKernelGGL((merge_kernel<128>), dim3(wgs), dim3(64), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
