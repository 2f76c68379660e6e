// pa_kivi.hip -- gfx950 kernels for an INT8 / INT4 KV cache quantised the
// KIVI way: decode attention over it, and the write of each new token.
//
// What ("大模型推理为何这么慢？从内存带宽瓶颈到KV Cache优化的技术突围", section
// "KV Cache量化：用精度换空间"): K and V stored as 8- or 4-bit integers; Key
// quantised per channel, Value per token (asymmetric, parameters from the
// data); the most recent tokens kept at full precision.  Concretely:
//   - a full block of 16 tokens holds codes [Hkv][16][d] (head-major, so one
//     head's 16 rows are contiguous whole cache lines at either width; INT4:
//     two per byte, even channel in the low nibble); K parameters per (block, head,
//     channel) over the block's tokens, V parameters per (block, head, slot)
//     over head_dim, both as fp16 (scale, min): value = code * scale + min;
//   - the tokens of a sequence's partly filled last block stay bf16 in a
//     per-sequence residual [B][16][Hkv][d]; the token that fills a block
//     has the whole block quantised from the residual;
//   - quantiser: scale = fp16((max - min) / (2^b - 1)) in float32 (1 if
//     zero), min = fp16(min), code = clamp(rint((x - min) / scale), 0,
//     2^b - 1) with IEEE float32 division and the stored fp16 parameters.
//
// Attention (kivi_attention_kernel) runs both products on the matrix cores
// (v_mfma_f32_16x16x32_bf16) with the codes themselves as operands: every
// code (0 .. 255) is a bf16 value, so widening it is exact, and the
// parameters move to the other operand:
//   S[h][t] = sum_c (q[h][c] s_c) n[t][c] + sum_c q[h][c] m_c
//   O[h][c] = sum_t (p[h][t] s_t) n'[t][c] + sum_t p[h][t] m_t
// (s, m: the block's K channel parameters, or V token parameters; n, n' the
// K and V codes).  q s and p s_t are each split into two bf16 terms (hi +
// lo, within 2^-16 relative), the two per-row sums are float32 on the
// vector ALUs.  One workgroup per (sequence, KV head); its W waves (8, or 4
// for the widest group) take every W-th full block, in pairs of blocks (32
// tokens, the K depth of one product), and the wave whose turn it is takes
// the bf16 residual as one more pair.  Per pair and wave:
//   - K codes are loaded straight into the A-operand layout (lane (t, q):
//     token t, channels [q d/4, (q+1) d/4) -- a permutation of the block's
//     contiguous bytes) and widened in registers;
//   - V codes are loaded in rows, widened and written to a per-wave LDS
//     tile, and read back transposed (ds_read_b64_tr_b16) as B operands;
//   - the B operands of S, q s in bf16 hi and lo for each of the G query
//     rows, are made once per block by as many lanes as the group has
//     8-channel pieces and passed through LDS; lanes of rows >= G read row
//     c % G (finite duplicates that no output uses).
// INT4 codes are widened by a bit trick: OR-ing a nibble into the bf16
// pattern of 128 gives 128 + code, two channels per instruction, in the
// order (0,4), (1,5), (2,6), (3,7) of each 8 (the q s pieces follow that
// order, the output dims are permuted back at the end).  The 128 so added
// is removed from the same bf16 terms: for K, 128 times the sum of each
// row's pieces is subtracted from the row's per-block constant (v_dot2
// against -128, two terms per instruction, when the pieces are made); for
// V, the sum of the weights (a product with a ones operand) times 128.
// The waves' exact states (running max, sum, unnormalised output) are
// combined in LDS.

#include "pa_internal.h"
#include "pa_mfma.h"

#include <hip/hip_ext.h>

namespace pa {
namespace {

constexpr int kTokK = 16;
constexpr float kLagK = 8.0f;  // lag allowed to the running max (log2 units)
// Start of the running max: the lowest finite float, so that a masked score
// (-inf) gives exp2(-inf - m) = 0 even before a valid token was seen.
constexpr float kNoMaxK = -3.402823466e38f;
// Waves per workgroup: eight (two per SIMD, so that one wave's arithmetic
// runs while the other's products or loads are outstanding), except for
// head_dim 128 with eight query heads per KV head, whose registers (two q s
// pieces per lane and their parameters in flight) fit only the larger
// register budget of one wave per SIMD.
template <int D, int G>
constexpr int kivi_waves() { return D == 128 && G == 8 ? 4 : 8; }

template <int CTRL>
__device__ __forceinline__ float dppk(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float swap_sum16(float x) {  // x + x of lane l ^ 16
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_sum32(float x) {  // x + x of lane l ^ 32
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the lanes 4 SP j + (0 .. 3) + 4 k, j < N (a quad and N - 1 more
// quads spaced SP lanes apart, SP N <= 64); every lane gets its set's sum.
template <int SP, int N>
__device__ __forceinline__ float quads_sum(float x) {
  static_assert(SP * N <= 64 && (SP == 4 || SP == 8 || SP == 16 || SP == 32), "lane sets");
  x += dppk<0xB1>(x);  // quad_perm [1,0,3,2]
  x += dppk<0x4E>(x);  // quad_perm [2,3,0,1]
#pragma unroll
  for (int st = SP; st < SP * N; st *= 2) {
    if (st == 4) x += dppk<0x141>(x);  // row_half_mirror: the quad 4 lanes over (sums per quad)
    else if (st == 8) x += dppk<0x128>(x);  // row_ror:8
    else if (st == 16) x = swap_sum16(x);
    else x = swap_sum32(x);
  }
  return x;
}

// Sum over lanes c, c+16, c+32, c+48.
__device__ __forceinline__ float sum4q(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFF));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// bf16 pair of two floats whose low 16 bits are zero (small integers): the
// upper halves, lo in the low half.
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// 4 INT8 codes -> 4 bf16 (two dwords), channel order kept.
__device__ __forceinline__ uint2 widen_u8x4(uint32_t w) {
  return make_uint2(bf16_pair((float)(w & 0xFF), (float)((w >> 8) & 0xFF)),
                    bf16_pair((float)((w >> 16) & 0xFF), (float)(w >> 24)));
}

// (x & m) | c in one instruction (both constants in registers: a VOP3
// instruction takes no literal here).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "v"(c));
  return r;
}

// 8 INT4 codes -> bf16 of 128 + code, as pairs of channels (0,4), (1,5),
// (2,6), (3,7): 0x4300 is 128 in bf16 and its 7 mantissa bits count units.
__device__ __forceinline__ uint4 widen_u4x8_biased(uint32_t w) {
  const uint32_t M = 0x000F000Fu, B = 0x43004300u;
  return make_uint4(and_or(w, M, B), and_or(w >> 4, M, B), and_or(w >> 8, M, B),
                    and_or(w >> 12, M, B));
}

// 8 bf16 channels (natural order) -> the order of widen_u4x8_biased.
__device__ __forceinline__ uint4 interleave_bf16x8(uint4 x) {
  return make_uint4(__builtin_amdgcn_perm(x.z, x.x, 0x05040100u),
                    __builtin_amdgcn_perm(x.z, x.x, 0x07060302u),
                    __builtin_amdgcn_perm(x.w, x.y, 0x05040100u),
                    __builtin_amdgcn_perm(x.w, x.y, 0x07060302u));
}

// Channel of V-tile column j (INT4 tiles hold each 8 channels in the
// widen_u4x8_biased order).
template <int BITS>
__device__ __forceinline__ int v_channel(int j) {
  if constexpr (BITS == 8) return j;
  else return (j & ~7) | ((j & 7) >> 1) | ((j & 1) << 2);
}

template <int BITS, int D, int G>
struct QGeo {
  static constexpr int ROWB = D * BITS / 8;      // code bytes of one row
  static constexpr int LB = ROWB / 4;            // code bytes per lane of one block (K or V)
  static constexpr int LBI = LB < 16 ? LB : 16;  // bytes per lane of one load instruction
  static constexpr int NI = LB / LBI;            // load instructions per block (K, and V)
  static constexpr int LPR = ROWB / LBI;         // lanes per row when loading V rows
  static constexpr int RPI = 64 / LPR;           // V rows per load instruction
  static constexpr int DW = LB / 4;              // code dwords per lane of one block
  static constexpr int KM = D / 32;              // products per block for S
  static constexpr int EV = D / 16;              // 16-dim slabs of O
  static constexpr int RSV = D * 2 + 32;         // LDS row stride of the widened V rows (bytes)
  static constexpr int VT = 32 * RSV;            // V tile of a pair
  static constexpr int NFR = G * D / 8;          // 8-channel pieces of q s per block
  static constexpr int FPL = (NFR + 63) / 64;    // pieces per lane
  static constexpr int FRB = 2 * KM * G * 64;    // LDS bytes of one block's pieces (hi, lo)
  static_assert(LB % LBI == 0 && 16 % RPI == 0, "whole rows per load");
  static_assert(G * D * 4 <= VT, "the wave's output fits its tile");
};

// Loads of one pair of blocks in flight.
template <int BITS, int D, int G>
struct QLoads {
  using Q = QGeo<BITS, D, G>;
  uint32_t k[2][Q::DW];        // K codes, A-operand layout
  uint32_t v[2][Q::DW];        // V codes, rows
  uint4 ks[2][Q::FPL];         // K scales of the lane's q s pieces (8 fp16)
  uint4 km[2][Q::FPL];         // K mins of the same channels
  uint4 vp[2];                 // (scale, min) of tokens 4q .. 4q+3
  bool ok[2];
};

// What the products of a pair need once its V tile and q s pieces are in LDS.
template <int BITS, int D, int G>
struct QPair {
  using Q = QGeo<BITS, D, G>;
  bf16x8_t ka[2][Q::KM];  // A operands of S (token c, channels of piece (q, m))
  uint4 vp[2];            // V parameters of tokens 4q .. 4q+3 (fp16 scale, min)
  int lim[2];             // valid tokens of each block: 16 or 0 (a residual: 0 .. 15)
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int BITS, int D, int G>
__global__ __launch_bounds__((kivi_waves<D, G>() * 64)) void kivi_attention_kernel(KiviArgs a) {
  constexpr bool kBiased = BITS == 4;  // K codes widened to 128 + code
  constexpr int kKW = kivi_waves<D, G>();
  using Q = QGeo<BITS, D, G>;
  constexpr int KM = Q::KM, EV = Q::EV, RSV = Q::RSV, FPL = Q::FPL, NFR = Q::NFR;
  __shared__ __attribute__((aligned(16))) char s_tile[kKW][Q::VT];
  __shared__ __attribute__((aligned(16))) char s_frag[kKW][2][Q::FRB];
  __shared__ float s_cst[kKW][2][G];
  __shared__ float s_f[kKW][16];
  __shared__ float s_m[kKW][G], s_l[kKW][G];

  const int tid = threadIdx.x, lane = tid & 63, c = lane & 15, q = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv;
  const int n = min(max(a.ctx[b], 0), a.max_ctx);
  const int nf = n / kTokK;         // full (quantised) blocks
  const int nres = n - nf * kTokK;  // residual tokens
  char *tile = s_tile[w];
  const float sl2 = a.scale_log2e;

  // this lane's q s pieces: slot f = lane + 64 i of a block's LDS region,
  // f = (m G + row) 4 + qq, holds the B operand of lanes (row, qq) for
  // product m: query row pr[i], channels 8 pj[i] .. 8 pj[i] + 7 with pj =
  // qq KM + m (so that a wave writes contiguous slots).  Lanes past the NFR
  // pieces repeat the last one and write nothing.  q is held times the
  // softmax scale (in log2 units), so the products give the exponents.
  float qf[FPL][8];
  int pr[FPL], pj[FPL];
#pragma unroll
  for (int i = 0; i < FPL; ++i) {
    const int f = min(lane + 64 * i, NFR - 1);
    pr[i] = (f / 4) % G;
    pj[i] = (f % 4) * KM + f / (4 * G);
    const uint4 x = *reinterpret_cast<const uint4 *>(
        static_cast<const uint16_t *>(a.q) + ((size_t)b * a.hq + g * G + pr[i]) * D + 8 * pj[i]);
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[i][2 * e] = __uint_as_float(xs[e] << 16) * sl2;
      qf[i][2 * e + 1] = __uint_as_float(xs[e] & 0xFFFF0000u) * sl2;
    }
  }

  const size_t code_block = (size_t)kTokK * a.hkv * Q::ROWB;  // bytes of one block's codes
  const char *kc = static_cast<const char *>(a.k_codes) + (size_t)g * kTokK * Q::ROWB;
  const char *vc = static_cast<const char *>(a.v_codes) + (size_t)g * kTokK * Q::ROWB;
  const uint16_t *kpar = static_cast<const uint16_t *>(a.k_par);  // [N][Hkv][2][D]
  const uint32_t *vpar = static_cast<const uint32_t *>(a.v_par);  // [N][Hkv][16] (scale, min)
  const uint32_t k_lane = (uint32_t)(c * Q::ROWB + q * Q::LB);    // A-operand bytes of the lane
  const uint32_t v_lane = (uint32_t)(lane * Q::LBI);             // row-layout bytes of the lane

  auto issue = [&](QLoads<BITS, D, G> &L, int id0, int id1) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int id = hb ? id1 : id0;
      L.ok[hb] = (unsigned)id < (unsigned)a.num_blocks;
      const size_t pb = L.ok[hb] ? (size_t)id : 0;  // block 0 stands in, masked out
#pragma unroll
      for (int ii = 0; ii < Q::NI; ++ii) {
        const char *kp = kc + pb * code_block + k_lane + ii * Q::LBI;
        const char *vp = vc + pb * code_block + v_lane + ii * 64 * Q::LBI;
        if constexpr (Q::LBI == 16) {
          const uint4 x = load_stream16(kp), y = load_stream16(vp);
          L.k[hb][4 * ii] = x.x; L.k[hb][4 * ii + 1] = x.y; L.k[hb][4 * ii + 2] = x.z; L.k[hb][4 * ii + 3] = x.w;
          L.v[hb][4 * ii] = y.x; L.v[hb][4 * ii + 1] = y.y; L.v[hb][4 * ii + 2] = y.z; L.v[hb][4 * ii + 3] = y.w;
        } else {
          const uint2 x = load_stream8(kp), y = load_stream8(vp);
          L.k[hb][2 * ii] = x.x; L.k[hb][2 * ii + 1] = x.y;
          L.v[hb][2 * ii] = y.x; L.v[hb][2 * ii + 1] = y.y;
        }
      }
      const uint16_t *kpb = kpar + (pb * a.hkv + g) * 2 * D;
#pragma unroll
      for (int i = 0; i < FPL; ++i) {
        L.ks[hb][i] = *reinterpret_cast<const uint4 *>(kpb + 8 * pj[i]);
        L.km[hb][i] = *reinterpret_cast<const uint4 *>(kpb + D + 8 * pj[i]);
      }
      L.vp[hb] = *reinterpret_cast<const uint4 *>(vpar + (pb * a.hkv + g) * kTokK + 4 * q);
    }
  };

  // The q s pieces of block hb of the pair (fp16 scales s, mins m) into LDS,
  // and the block's per-row constant sum_c q m_c.  INT4 pieces are in the
  // channel order of the widened INT4 codes.
  auto pieces = [&](int hb, const uint4 (&s)[FPL], const uint4 (&m)[FPL], bool bias) {
    char *fr = s_frag[w][hb];
    float cst_all = 0.f;
#pragma unroll
    for (int i = 0; i < FPL; ++i) {
      const uint32_t sw[4] = {s[i].x, s[i].y, s[i].z, s[i].w};
      const uint32_t mw[4] = {m[i].x, m[i].y, m[i].z, m[i].w};
      float qs[8], cst = 0.f;
#pragma unroll
      // (products written as fma with 0: one v_fma_mix_f32 each, taking
      // the fp16 operand as it is, instead of a conversion and a multiply)
      for (int e = 0; e < 4; ++e) {
        qs[2 * e] = fmaf(qf[i][2 * e], half_lo(sw[e]), 0.f);
        qs[2 * e + 1] = fmaf(qf[i][2 * e + 1], half_hi(sw[e]), 0.f);
        cst = fmaf(qf[i][2 * e], half_lo(mw[e]), cst);
        cst = fmaf(qf[i][2 * e + 1], half_hi(mw[e]), cst);
      }
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = BITS == 8 ? qs[e] : qs[(e >> 1) + 4 * (e & 1)];
      bf16x8_t hi, lo;
      split_bf16(p, hi, lo);
      if (bias) {
        // the widened INT4 K codes carry 128 + code: their products with
        // these pieces hold 128 sum(hi + lo), removed here from the row's
        // constant with the same bf16 terms (two per dot product)
        const bf16x2_t n128 = __builtin_bit_cast(bf16x2_t, 0xC300C300u);
        const uint4 h4 = __builtin_bit_cast(uint4, hi), l4 = __builtin_bit_cast(uint4, lo);
        const uint32_t hw[4] = {h4.x, h4.y, h4.z, h4.w}, lw[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          cst = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, hw[e]), n128, cst, false);
          cst = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lw[e]), n128, cst, false);
        }
      }
      if (lane + 64 * i < NFR) {
        *reinterpret_cast<bf16x8_t *>(fr + (lane + 64 * i) * 16) = hi;
        *reinterpret_cast<bf16x8_t *>(fr + KM * G * 64 + (lane + 64 * i) * 16) = lo;
      }
      // the row's sum over its KM * 4 pieces: quads spaced 4 G lanes apart
      // (and, with two pieces per lane, the other register's)
      cst_all += quads_sum<4 * G, (4 * G * KM <= 64 ? KM : 64 / (4 * G))>(cst);
    }
    if (lane < 4 * G && lane % 4 == 0) s_cst[w][hb][lane / 4] = cst_all;
  };

  // V codes of a landed pair -> bf16 rows of the tile
  auto stage_v = [&](const QLoads<BITS, D, G> &L) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int ii = 0; ii < Q::NI; ++ii) {
        const int row = 16 * hb + ii * Q::RPI + lane / Q::LPR;
        const int ch0 = (lane % Q::LPR) * Q::LBI * 8 / BITS;
        char *dst = tile + row * RSV + ch0 * 2;
        const uint32_t *src = &L.v[hb][ii * Q::LBI / 4];
#pragma unroll
        for (int dw = 0; dw < Q::LBI / 4; ++dw) {
          if constexpr (BITS == 8) {
            const uint2 x = widen_u8x4(src[dw]);
            *reinterpret_cast<uint2 *>(dst + 8 * dw) = x;
          } else {
            *reinterpret_cast<uint4 *>(dst + 16 * dw) = widen_u4x8_biased(src[dw]);
          }
        }
      }
  };

  auto stage = [&](const QLoads<BITS, D, G> &L) {
    stage_v(L);
    pieces(0, L.ks[0], L.km[0], kBiased);
    pieces(1, L.ks[1], L.km[1], kBiased);
    QPair<BITS, D, G> P;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        if constexpr (BITS == 8) {
          const uint2 x0 = widen_u8x4(L.k[hb][2 * m]), x1 = widen_u8x4(L.k[hb][2 * m + 1]);
          P.ka[hb][m] = as_bf16x8(make_uint4(x0.x, x0.y, x1.x, x1.y));
        } else {
          P.ka[hb][m] = as_bf16x8(widen_u4x8_biased(L.k[hb][m]));
        }
      }
      P.vp[hb] = L.vp[hb];
      P.lim[hb] = L.ok[hb] ? kTokK : 0;
    }
    return P;
  };

  float mrun = kNoMaxK, lsum = 0.f, psum = 0.f;  // row c: running max, sum of p, sum of p m_t
  f32x4_t o[EV], sw4 = f32x4_t{0.f, 0.f, 0.f, 0.f};  // rows 4q .. 4q+3
#pragma unroll
  for (int m = 0; m < EV; ++m) o[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bf16x8_t ones = bf16x8_ones();

  auto compute = [&](const QPair<BITS, D, G> &P, bool biased) {
    __builtin_amdgcn_wave_barrier();  // tile and pieces were written by other lanes
    const int cs = c % G;
    f32x4_t sc[2];
    float cst[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const char *fr = s_frag[w][hb] + (cs * 4 + q) * 16;
      sc[hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        const bf16x8_t bh = *reinterpret_cast<const bf16x8_t *>(fr + m * G * 64);
        const bf16x8_t bl = *reinterpret_cast<const bf16x8_t *>(fr + (KM + m) * G * 64);
        sc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(P.ka[hb][m], bh, sc[hb], 0, 0, 0);
        sc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(P.ka[hb][m], bl, sc[hb], 0, 0, 0);
      }
      cst[hb] = s_cst[w][hb][cs];
    }
    const bool full = P.lim[0] == kTokK && P.lim[1] == kTokK;  // wave-uniform
    float x[2][4];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int j = 0; j < 4; ++j) x[hb][j] = sc[hb][j] + cst[hb];
    if (!full) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          x[hb][j] = 4 * q + j < P.lim[hb] ? x[hb][j] : -__builtin_huge_valf();
    }
    const float mx = max4q(max8(x));
    const bool raise = mx > mrun + kLagK;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float mn = raise ? mx : mrun;
      const float f = raise ? __builtin_amdgcn_exp2f(mrun - mn) : 1.f;
      mrun = mn;
      lsum *= f;
      psum *= f;
      // lane (c, q) has row c's factor; its O entries are rows 4q .. 4q+3
      if (q == 0) s_f[w][c] = f;
      __builtin_amdgcn_wave_barrier();
      const float4 f4 = *reinterpret_cast<const float4 *>(&s_f[w][4 * q]);
      __builtin_amdgcn_wave_barrier();
      const float fr[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sw4[r] *= fr[r];
#pragma unroll
        for (int m = 0; m < EV; ++m) o[m][r] *= fr[r];
      }
    }
    float pf[8], wv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pf[e] = __builtin_amdgcn_exp2f(x[e >> 2][e & 3] - mrun);  // masked: 0
      lsum += pf[e];
    }
    const uint32_t vpa[8] = {P.vp[0].x, P.vp[0].y, P.vp[0].z, P.vp[0].w,
                             P.vp[1].x, P.vp[1].y, P.vp[1].z, P.vp[1].w};
    if (full) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t vp = vpa[e];
        wv[e] = fmaf(pf[e], half_lo(vp), 0.f);
        psum = fmaf(pf[e], half_hi(vp), psum);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t vp = vpa[e];
        // a dead slot's parameters may be anything (NaN included): weight 0
        const bool live = 4 * q + (e & 3) < P.lim[e >> 2];
        wv[e] = live ? fmaf(pf[e], half_lo(vp), 0.f) : 0.f;
        psum = live ? fmaf(pf[e], half_hi(vp), psum) : psum;
      }
    }
    bf16x8_t wh, wl;
    split_bf16(wv, wh, wl);
    if (biased) {
      sw4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wh, ones, sw4, 0, 0, 0);
      sw4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wl, ones, sw4, 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < EV; ++m) {
      const bf16x8_t vb = v_operand_tr<D>(tile, RSV, m);
      o[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wh, vb, o[m], 0, 0, 0);
      o[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wl, vb, o[m], 0, 0, 0);
    }
  };

  // ---- the wave's full blocks w, w + 8, ...: pairs p, two stages (pair p
  // staged and computed while pairs p + 1 and p + 2 load).  The table
  // entries of up to 64 blocks come from one vector load (lane j holds the
  // wave's block c0 + j; -1 past the wave's blocks), read with readlane.
  const int nbw = nf > w ? (nf - w + kKW - 1) / kKW : 0;
  const int *trow = a.table + (size_t)b * a.max_blocks;
  for (int c0 = 0; c0 < nbw; c0 += 64) {
    const int cn = min(64, nbw - c0);
    const int tv = c0 + lane < nbw ? trow[(size_t)w + (size_t)kKW * (c0 + lane)] : -1;
    auto entry = [&](int i) { return __builtin_amdgcn_readlane(tv, i); };  // i < 64
    const int np = (cn + 1) / 2;
    QLoads<BITS, D, G> A, B;
    issue(A, entry(0), entry(1));
    if (np > 1) issue(B, entry(2), entry(3));
    int p = 0;
    for (; p + 3 < np; p += 2) {
      const QPair<BITS, D, G> pa_ = stage(A);
      issue(A, entry(2 * p + 4), entry(2 * p + 5));
      __builtin_amdgcn_sched_barrier(0);
      compute(pa_, kBiased);
      const QPair<BITS, D, G> pb_ = stage(B);
      issue(B, entry(2 * p + 6), entry(2 * p + 7));
      __builtin_amdgcn_sched_barrier(0);
      compute(pb_, kBiased);
    }
    // at most three pairs left: p (in A), p + 1 (in B), p + 2 (not issued)
    if (p < np) {
      const QPair<BITS, D, G> pa_ = stage(A);
      if (p + 2 < np) issue(A, entry(2 * p + 4), entry(2 * p + 5));
      __builtin_amdgcn_sched_barrier(0);
      compute(pa_, kBiased);
    }
    if (p + 1 < np) compute(stage(B), kBiased);
    if (p + 2 < np) compute(stage(A), kBiased);
  }

  // ---- the residual (bf16) tokens of the partly filled block, as one more
  // pair (its second block empty): the wave whose turn block nf is.  The
  // q s pieces are q itself (scale 1, min 0), the V weights the p's.
  if (nres > 0 && w == nf % kKW) {
    const uint16_t *rk = static_cast<const uint16_t *>(a.res_k);
    const uint16_t *rv = static_cast<const uint16_t *>(a.res_v);
    auto res_row = [&](int t) { return (((size_t)b * kTokK + t) * a.hkv + g) * D; };
    QPair<BITS, D, G> P;
    // K: lane (c, q) takes token c, channels [q D/4, (q+1) D/4) (masked in the scores)
    const uint16_t *kr = rk + res_row(c) + q * (D / 4);
#pragma unroll
    for (int m = 0; m < KM; ++m) {
      const uint4 x = *reinterpret_cast<const uint4 *>(kr + 8 * m);
      P.ka[0][m] = as_bf16x8(BITS == 4 ? interleave_bf16x8(x) : x);
      P.ka[1][m] = as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
    }
    // V: lane l takes row l / 4, channels [(l % 4) D/4, ...); rows past the
    // tokens, and the empty block's rows, as zeros
    {
      const int t = lane / 4, ch0 = (lane % 4) * (D / 4);
      const uint16_t *vr = rv + res_row(t) + ch0;
      const bool live = t < nres;
#pragma unroll
      for (int k8 = 0; k8 < D / 32; ++k8) {
        uint4 x = *reinterpret_cast<const uint4 *>(vr + 8 * k8);
        if (!live) x = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (BITS == 4) x = interleave_bf16x8(x);
        *reinterpret_cast<uint4 *>(tile + t * RSV + (ch0 + 8 * k8) * 2) = x;
        *reinterpret_cast<uint4 *>(tile + (16 + t) * RSV + (ch0 + 8 * k8) * 2) = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    uint4 s1[FPL], m0[FPL];
#pragma unroll
    for (int i = 0; i < FPL; ++i) {
      s1[i] = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);  // fp16 1.0
      m0[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    pieces(0, s1, m0, false);
    P.vp[0] = P.vp[1] = make_uint4(0x3C00u, 0x3C00u, 0x3C00u, 0x3C00u);  // (scale 1, min 0)
    P.lim[0] = nres;
    P.lim[1] = 0;
    compute(P, false);
  }

  // ---- the wave's state by query row: the max and sums of row c in lanes
  // (c, *); output rows 4q .. 4q+3 in lanes (n, q)
  lsum = sum4q(lsum);
  psum = sum4q(psum);
  if (q == 0) {
    s_f[w][c] = psum;
    if (c < G) {
      s_m[w][c] = mrun;
      s_l[w][c] = lsum;
    }
  }
  __builtin_amdgcn_wave_barrier();
  const float4 pm4 = *reinterpret_cast<const float4 *>(&s_f[w][4 * q]);
  const float pm[4] = {pm4.x, pm4.y, pm4.z, pm4.w};
  float *acc = reinterpret_cast<float *>(tile);  // [G][D]; the wave's tile is done
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int hh = 4 * q + r;
    if (hh < G) {
      const float base = pm[r] - (kBiased ? 128.f * sw4[r] : 0.f);
#pragma unroll
      for (int m = 0; m < EV; ++m) acc[hh * D + v_channel<BITS>(16 * m + c)] = o[m][r] + base;
    }
  }
  __syncthreads();

  // ---- combine the waves (exact: maxima aligned to their common maximum)
  for (int idx = tid; idx < G * D; idx += kKW * 64) {
    const int hh = idx / D, e = idx % D;
    float M = kNoMaxK;
#pragma unroll
    for (int v = 0; v < kKW; ++v) M = fmaxf(M, s_m[v][hh]);
    float A = 0.f, L = 0.f;
#pragma unroll
    for (int v = 0; v < kKW; ++v) {
      const float f = __builtin_amdgcn_exp2f(s_m[v][hh] - M);
      A = fmaf(f, reinterpret_cast<const float *>(s_tile[v])[hh * D + e], A);
      L = fmaf(f, s_l[v][hh], L);
    }
    a.out[((size_t)b * a.hq + g * G + hh) * D + e] = L > 0.f ? A / L : 0.f;
  }
}

// ---------------------------------------------------------------------------
// cache write: the new token into the residual row; a full block quantised

__device__ __forceinline__ float wave_min(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) x = fminf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// fp16 (scale, min) of a group with extremes lo, hi, and the codes' divisor.
template <int BITS>
__device__ __forceinline__ void group_params(float lo, float hi, _Float16 &s16, _Float16 &m16) {
  s16 = (_Float16)((hi - lo) / (float)((1 << BITS) - 1));
  if ((float)s16 == 0.f) s16 = (_Float16)1.0f;
  m16 = (_Float16)lo;
}

template <int BITS>
__device__ __forceinline__ uint32_t quant(float x, _Float16 s16, _Float16 m16) {
  const float y = (x - (float)m16) / (float)s16;
  return (uint32_t)fminf(fmaxf(__builtin_rintf(y), 0.f), (float)((1 << BITS) - 1));
}

// One wave per (sequence, KV head); lane i holds channels 2i, 2i+1 (lanes
// past D/2 are idle in the stores and neutral in the reductions).
template <int BITS, int D>
__global__ __launch_bounds__(64) void kivi_append_kernel(KiviArgs a, const void *k_new,
                                                         const void *v_new) {
  const int lane = threadIdx.x;
  const int b = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv;
  const int n = min(max(a.ctx[b], 0), a.max_ctx);
  if (n == 0) return;
  const int t = n - 1, slot = t % kTokK;
  const bool act = lane < D / 2;
  const int c0 = 2 * (act ? lane : 0);
  uint16_t *rk = static_cast<uint16_t *>(a.res_k);
  uint16_t *rv = static_cast<uint16_t *>(a.res_v);
  const size_t src = ((size_t)b * a.hkv + g) * D + c0;
  const uint32_t nk = *reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(k_new) + src);
  const uint32_t nv = *reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(v_new) + src);
  auto res_at = [&](int s) { return (((size_t)b * kTokK + s) * a.hkv + g) * D + c0; };
  if (act) {
    *reinterpret_cast<uint32_t *>(rk + res_at(slot)) = nk;
    *reinterpret_cast<uint32_t *>(rv + res_at(slot)) = nv;
  }
  if (slot != kTokK - 1) return;
  const int phys = a.table[(size_t)b * a.max_blocks + t / kTokK];
  if ((unsigned)phys >= (unsigned)a.num_blocks) return;

  // the block's 16 rows of this lane's two channels (the new one from
  // registers: the rows written above are not read back)
  float kx[kTokK][2], vx[kTokK][2];
#pragma unroll
  for (int s = 0; s < kTokK; ++s) {
    const uint32_t kw = s == kTokK - 1 ? nk : *reinterpret_cast<const uint32_t *>(rk + res_at(s));
    const uint32_t vw = s == kTokK - 1 ? nv : *reinterpret_cast<const uint32_t *>(rv + res_at(s));
    kx[s][0] = __uint_as_float(kw << 16); kx[s][1] = __uint_as_float(kw & 0xFFFF0000u);
    vx[s][0] = __uint_as_float(vw << 16); vx[s][1] = __uint_as_float(vw & 0xFFFF0000u);
  }
  constexpr int ROWB = D * BITS / 8;
  uint8_t *kc = static_cast<uint8_t *>(a.k_codes) + (size_t)phys * kTokK * a.hkv * ROWB;
  uint8_t *vc = static_cast<uint8_t *>(a.v_codes) + (size_t)phys * kTokK * a.hkv * ROWB;
  auto store_pair = [&](uint8_t *base, int s, uint32_t q0, uint32_t q1) {
    uint8_t *row = base + ((size_t)g * kTokK + s) * ROWB;
    if constexpr (BITS == 8) {
      *reinterpret_cast<uint16_t *>(row + c0) = (uint16_t)(q0 | (q1 << 8));
    } else {
      row[c0 / 2] = (uint8_t)(q0 | (q1 << 4));
    }
  };
  // K: per channel over the block's tokens
  if (act) {
    _Float16 s16[2], m16[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float lo = kx[0][j], hi = kx[0][j];
#pragma unroll
      for (int s = 1; s < kTokK; ++s) {
        lo = fminf(lo, kx[s][j]);
        hi = fmaxf(hi, kx[s][j]);
      }
      group_params<BITS>(lo, hi, s16[j], m16[j]);
    }
#pragma unroll
    for (int s = 0; s < kTokK; ++s)
      store_pair(kc, s, quant<BITS>(kx[s][0], s16[0], m16[0]), quant<BITS>(kx[s][1], s16[1], m16[1]));
    uint16_t *kp = static_cast<uint16_t *>(a.k_par) + ((size_t)phys * a.hkv + g) * 2 * D;
    *reinterpret_cast<uint32_t *>(kp + c0) =
        (uint32_t)__builtin_bit_cast(uint16_t, s16[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, s16[1]) << 16);
    *reinterpret_cast<uint32_t *>(kp + D + c0) =
        (uint32_t)__builtin_bit_cast(uint16_t, m16[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, m16[1]) << 16);
  }
  // V: per token over the head dimension
  uint32_t *vp = static_cast<uint32_t *>(a.v_par) + ((size_t)phys * a.hkv + g) * kTokK;
#pragma unroll
  for (int s = 0; s < kTokK; ++s) {
    const float lo = wave_min(act ? fminf(vx[s][0], vx[s][1]) : __builtin_huge_valf());
    const float hi = wave_max(act ? fmaxf(vx[s][0], vx[s][1]) : -__builtin_huge_valf());
    _Float16 s16, m16;
    group_params<BITS>(lo, hi, s16, m16);
    if (act) store_pair(vc, s, quant<BITS>(vx[s][0], s16, m16), quant<BITS>(vx[s][1], s16, m16));
    if (lane == 0)
      vp[s] = (uint32_t)__builtin_bit_cast(uint16_t, s16) | ((uint32_t)__builtin_bit_cast(uint16_t, m16) << 16);
  }
}

template <int BITS, int D, int G>
void launch_attn(const KiviArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  constexpr int threads = kivi_waves<D, G>() * 64;
  const dim3 grid((unsigned)((size_t)a.batch * a.hkv));
  if (e0)  // events attached to the dispatch: the kernel's own start and end
    hipExtLaunchKernelGGL((kivi_attention_kernel<BITS, D, G>), grid, dim3(threads), 0, s, e0, e1, 0, a);
  else
    hipLaunchKernelGGL((kivi_attention_kernel<BITS, D, G>), grid, dim3(threads), 0, s, a);
}

template <int BITS, int D>
hipError_t attn_by_group(const KiviArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (a.hq / a.hkv) {
    case 1: launch_attn<BITS, D, 1>(a, s, e0, e1); break;
    case 2: launch_attn<BITS, D, 2>(a, s, e0, e1); break;
    case 4: launch_attn<BITS, D, 4>(a, s, e0, e1); break;
    case 8: launch_attn<BITS, D, 8>(a, s, e0, e1); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kivi_attention(const KiviArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (a.batch == 0) return hipSuccess;
  if (a.bits == 8)
    return a.d == 64 ? attn_by_group<8, 64>(a, s, e0, e1) : attn_by_group<8, 128>(a, s, e0, e1);
  return a.d == 64 ? attn_by_group<4, 64>(a, s, e0, e1) : attn_by_group<4, 128>(a, s, e0, e1);
}

hipError_t launch_kivi_append(const KiviArgs &a, const void *k_new, const void *v_new,
                              hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  const dim3 grid((unsigned)((size_t)a.batch * a.hkv));
  if (a.bits == 8) {
    if (a.d == 64) hipLaunchKernelGGL((kivi_append_kernel<8, 64>), grid, dim3(64), 0, s, a, k_new, v_new);
    else hipLaunchKernelGGL((kivi_append_kernel<8, 128>), grid, dim3(64), 0, s, a, k_new, v_new);
  } else {
    if (a.d == 64) hipLaunchKernelGGL((kivi_append_kernel<4, 64>), grid, dim3(64), 0, s, a, k_new, v_new);
    else hipLaunchKernelGGL((kivi_append_kernel<4, 128>), grid, dim3(64), 0, s, a, k_new, v_new);
  }
  return hipGetLastError();
}

}  // namespace pa
