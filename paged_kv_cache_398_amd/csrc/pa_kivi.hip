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
// Attention (kivi_attention_kernel): one workgroup per (sequence, KV head),
// its W waves (4 or 8) taking every W-th full block, the residual block
// taken by the wave whose turn it is; the waves' exact states are combined in LDS.  A
// lane holds a contiguous run of EPL channels of a token row (LPT lanes per
// row), so quantised blocks and the residual share one accumulator layout.
// K is dequantised per element (k = code * s_c + m_c, one multiply-add with
// the fp16 parameters as operands) once for the G heads that use it; V's
// dequantisation is folded: with V = code * s_t + m_t per token,
//   sum_t p_t v_tc = sum_t (p_t s_t) code_tc + sum_t p_t m_t,
// the second term being one scalar per head, added at the end.

#include "pa_internal.h"

namespace pa {
namespace {

#ifndef KIVI_STAGES
#define KIVI_STAGES 2  // blocks of a wave in flight at once
#endif
static_assert(KIVI_STAGES >= 2, "the pipeline needs two stages or more");

// Waves per workgroup: eight (two per SIMD, so one wave's arithmetic runs
// while another waits for its loads) where the compiled kernel fits in the
// 256 registers a wave then has without scratch -- head_dim 64, and head_dim
// 128 with one or four query heads per KV head; four elsewhere (head_dim 128
// with two or eight spill at eight waves).  Llama-3-8B-shaped step, eight
// against four waves: INT8 87.3 against 90-91 us, INT4 84-85 against 90-92.
template <int D, int G>
constexpr int kivi_waves() { return (D == 64 || G == 1 || G == 4) ? 8 : 4; }
#ifndef KIVI_ACC
#define KIVI_ACC 64   // most accumulator registers per lane
#endif

constexpr int kTokK = 16;
constexpr float kLagK = 8.0f;

template <int CTRL>
__device__ __forceinline__ float dppk(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int LPT>
__device__ __forceinline__ float row_sum(float x) {  // over the LPT lanes of a row
  x += dppk<0xB1>(x);
  x += dppk<0x4E>(x);
  if constexpr (LPT >= 8) x += dppk<0x141>(x);
  if constexpr (LPT >= 16) x += dppk<0x140>(x);
  return x;
}

template <int LPT, bool MAX>
__device__ __forceinline__ float slots(float x) {  // over the token slots of a wave
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  if constexpr (LPT <= 4) x = op(x, dppk<0x124>(x));
  if constexpr (LPT <= 8) x = op(x, dppk<0x128>(x));
  {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return x;
}

__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFF));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Lanes per token row: keep the accumulators (G * D / LPT floats) at
// KIVI_ACC or fewer, and each lane's code slice at one dword or more.
constexpr int kivi_lpt(int d, int g, int bits) {
  int l = g * d / 4 <= KIVI_ACC ? 4 : (g * d / 8 <= KIVI_ACC ? 8 : 16);
  while (l > 4 && (d / l) * bits / 8 < 4) l /= 2;
  return l;
}

template <int BITS, int D, int G>
struct KCfg {
  static constexpr int LPT = kivi_lpt(D, G, BITS);
  static constexpr int EPL = D / LPT;              // channels per lane
  static constexpr int CB = EPL * BITS / 8;        // code bytes per lane per row
  static constexpr int CDW = CB / 4;               // code dwords per lane per row
  static constexpr int TPP = 64 / LPT;
  static constexpr int NPASS = kTokK / TPP;
  static constexpr int ROWB = D * BITS / 8;        // code bytes of one row
  static_assert(CB % 4 == 0, "code slice must be whole dwords");
};

template <int N>
__device__ __forceinline__ void load_dw(const char *p, uint32_t *dst) {
  static_assert(N == 1 || N % 2 == 0, "dword count");
  if constexpr (N == 1) {
    dst[0] = load_stream4(p);
  } else if constexpr (N == 2) {
    const uint2 x = load_stream8(p);
    dst[0] = x.x; dst[1] = x.y;
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const uint4 x = load_stream16(p + 4 * i);
      dst[i] = x.x; dst[i + 1] = x.y; dst[i + 2] = x.z; dst[i + 3] = x.w;
    }
  }
}

// A lane's code slice (N dwords) as floats.  INT4: the even and odd nibbles
// of a dword are first spread to bytes (two masks), so every element is one
// byte-to-float conversion, as for INT8.
template <int BITS, int N>
__device__ __forceinline__ void codes_to_float(const uint32_t *w, float *f) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if constexpr (BITS == 8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) f[4 * i + j] = (float)((w[i] >> (8 * j)) & 0xFF);
    } else {
      const uint32_t even = w[i] & 0x0F0F0F0Fu, odd = (w[i] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[8 * i + 2 * j] = (float)((even >> (8 * j)) & 0xFF);
        f[8 * i + 2 * j + 1] = (float)((odd >> (8 * j)) & 0xFF);
      }
    }
  }
}

template <int BITS, int D, int G>
struct KBlock {
  using C = KCfg<BITS, D, G>;
  uint32_t k[C::NPASS][C::CDW];
  uint32_t v[C::NPASS][C::CDW];
  uint32_t ks[C::EPL / 2], km[C::EPL / 2];  // fp16 pairs: K scales, mins of the lane's channels
  uint32_t vp[C::NPASS];                    // fp16 (scale, min) of the lane's token
  bool ok;
};

template <int BITS, int D, int G>
__global__ __launch_bounds__((kivi_waves<D, G>() * 64)) void kivi_attention_kernel(KiviArgs a) {
  constexpr int kKW = kivi_waves<D, G>();
  constexpr int kKThreads = kKW * 64;
  using C = KCfg<BITS, D, G>;
  constexpr int LPT = C::LPT, EPL = C::EPL, NPASS = C::NPASS, TPP = C::TPP, CDW = C::CDW;
  __shared__ float s_acc[kKW][G][D];
  __shared__ float s_m[kKW][G], s_l[kKW][G];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv;
  const int sub = lane % LPT, slot = lane / LPT;
  const int n = min(max(a.ctx[b], 0), a.max_ctx);
  const int nf = n / kTokK;       // full (quantised) blocks
  const int nres = n - nf * kTokK;  // residual tokens

  // query rows of the group, this lane's channels, fp32
  float qf[G][EPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) + ((size_t)b * a.hq + g * G + hh) * D + sub * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[hh][e] = __uint_as_float((uint32_t)qp[e] << 16);
  }
  float m[G], l[G], pm[G], acc[G][EPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -__builtin_huge_valf();
    l[hh] = 0.f;
    pm[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.f;
  }
  const float sl2 = a.scale_log2e;

  // lane offsets (bytes) inside a block, of codes and parameters
  const size_t block_codes = (size_t)kTokK * a.hkv * C::ROWB;
  uint32_t c_off[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p)
    c_off[p] = (uint32_t)((g * kTokK + p * TPP + slot) * C::ROWB + sub * C::CB);
  const char *kc = static_cast<const char *>(a.k_codes);
  const char *vc = static_cast<const char *>(a.v_codes);
  const uint16_t *kpar = static_cast<const uint16_t *>(a.k_par);  // [N][Hkv][2][D]
  const uint32_t *vpar = static_cast<const uint32_t *>(a.v_par);  // [N][Hkv][16] (scale, min)

  auto issue = [&](KBlock<BITS, D, G> &bk, int phys) {
    bk.ok = (unsigned)phys < (unsigned)a.num_blocks;
    const size_t pb = bk.ok ? (size_t)phys : 0;
    const char *kb = kc + pb * block_codes, *vb = vc + pb * block_codes;
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      load_dw<CDW>(kb + c_off[p], bk.k[p]);
      load_dw<CDW>(vb + c_off[p], bk.v[p]);
      const uint32_t vw = vpar[(pb * a.hkv + g) * kTokK + p * TPP + slot];
      bk.vp[p] = bk.ok ? vw : 0u;  // a stand-in block adds exactly nothing
    }
    const char *kp = reinterpret_cast<const char *>(kpar + (pb * a.hkv + g) * 2 * D + sub * EPL);
    load_dw<EPL / 2>(kp, bk.ks);
    load_dw<EPL / 2>(kp + 2 * D, bk.km);
  };

  // online-softmax update for a block's scores s[p][hh] (masked ones -inf),
  // then the PV step through pv(p, hh, weight)
  auto softmax_update = [&](float (&s)[NPASS][G], auto &&pv) {
    bool raise = false;
    float bm[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float x = s[0][hh];
#pragma unroll
      for (int p = 1; p < NPASS; ++p) x = fmaxf(x, s[p][hh]);
      bm[hh] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(slots<LPT, true>(x))));
      raise |= bm[hh] > m[hh] + kLagK;
    }
    if (raise) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float mn = fmaxf(m[hh], bm[hh]);
        const float c = __builtin_amdgcn_exp2f(m[hh] - mn);
        m[hh] = mn;
        l[hh] *= c;
        pm[hh] *= c;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hh][e] *= c;
      }
    }
#pragma unroll
    for (int p = 0; p < NPASS; ++p)
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float x = s[p][hh];
        const float pr = x == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(x - m[hh]);
        l[hh] += pr;
        pv(p, hh, pr);
      }
  };

  auto compute = [&](const KBlock<BITS, D, G> &bk) {
    float s[NPASS][G];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      // K of the lane's token, dequantised once for the G heads (one
      // multiply-add per element with the fp16 scale and min as operands)
      float kf[EPL];
      codes_to_float<BITS, CDW>(bk.k[p], kf);
#pragma unroll
      for (int i = 0; i < EPL / 2; ++i) {
        kf[2 * i] = fmaf(kf[2 * i], half_lo(bk.ks[i]), half_lo(bk.km[i]));
        kf[2 * i + 1] = fmaf(kf[2 * i + 1], half_hi(bk.ks[i]), half_hi(bk.km[i]));
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; e += 2) {
          d0 = fmaf(qf[hh][e], kf[e], d0);
          d1 = fmaf(qf[hh][e + 1], kf[e + 1], d1);
        }
        const float x = row_sum<LPT>(d0 + d1) * sl2;
        s[p][hh] = bk.ok ? x : -__builtin_huge_valf();
      }
    }
    float vf[NPASS][EPL];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) codes_to_float<BITS, CDW>(bk.v[p], vf[p]);
    softmax_update(s, [&](int p, int hh, float pr) {
      const float vs = half_lo(bk.vp[p]), vmn = half_hi(bk.vp[p]);
      const float pw = pr * vs;
      pm[hh] = fmaf(pr, vmn, pm[hh]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[hh][e] = fmaf(pw, vf[p][e], acc[hh][e]);
    });
  };

  // ---- the wave's full blocks w, w+4, ...: two-stage pipeline, table
  // entries of up to 64 blocks read by one vector load
  const int nbw = nf > w ? (nf - w + kKW - 1) / kKW : 0;
  const int *trow = a.table + (size_t)b * a.max_blocks;
  for (int c0 = 0; c0 < nbw; c0 += 64) {
    const int cn = min(64, nbw - c0);
    const int tv = c0 + lane < nbw ? trow[(size_t)w + (size_t)kKW * (c0 + lane)] : -1;
    auto id_of = [&](int i) { return __builtin_amdgcn_readlane(tv, min(i, cn - 1)); };
    // KIVI_STAGES blocks in flight: block i is computed while blocks
    // i+1 .. i+KIVI_STAGES-1 load.  Past the wave's last block the loads
    // repeat that block (id_of clamps; it is in the caches by then) and are
    // not computed, so no load sits behind a branch.
    KBlock<BITS, D, G> bk[KIVI_STAGES];
#pragma unroll
    for (int st = 0; st < KIVI_STAGES - 1; ++st) issue(bk[st], id_of(st));
    for (int i = 0; i < cn; i += KIVI_STAGES) {
#pragma unroll
      for (int st = 0; st < KIVI_STAGES; ++st) {
        issue(bk[(st + KIVI_STAGES - 1) % KIVI_STAGES], id_of(i + st + KIVI_STAGES - 1));
        __builtin_amdgcn_sched_barrier(0);
        if (i + st < cn) compute(bk[st]);
      }
    }
  }

  // ---- the residual (bf16) tokens of the partial block: the wave whose
  // turn block nf is
  if (nres > 0 && w == nf % kKW) {
    float s[NPASS][G];
    float vf[NPASS][EPL];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int t = p * TPP + slot;
      const bool live = t < nres;
      const uint16_t *kr = static_cast<const uint16_t *>(a.res_k) +
                           (((size_t)b * kTokK + t) * a.hkv + g) * D + sub * EPL;
      const uint16_t *vr = static_cast<const uint16_t *>(a.res_v) +
                           (((size_t)b * kTokK + t) * a.hkv + g) * D + sub * EPL;
      float kf[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        kf[e] = __uint_as_float((uint32_t)kr[e] << 16);
        const float v = __uint_as_float((uint32_t)vr[e] << 16);
        vf[p][e] = live ? v : 0.f;  // select: slots past the tokens may hold anything
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; e += 2) {
          d0 = fmaf(qf[hh][e], kf[e], d0);
          d1 = fmaf(qf[hh][e + 1], kf[e + 1], d1);
        }
        const float x = row_sum<LPT>(d0 + d1) * sl2;
        s[p][hh] = live ? x : -__builtin_huge_valf();
      }
    }
    softmax_update(s, [&](int p, int hh, float pr) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[hh][e] = fmaf(pr, vf[p][e], acc[hh][e]);
    });
  }

  // ---- combine: token slots of the wave, then the waves, in LDS
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    l[hh] = slots<LPT, false>(l[hh]);
    pm[hh] = slots<LPT, false>(pm[hh]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hh][e] = slots<LPT, false>(acc[hh][e]) + pm[hh];
  }
  if (lane < LPT) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[w][hh][sub * EPL + e] = acc[hh][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      s_m[w][hh] = m[hh];
      s_l[w][hh] = l[hh];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kKThreads) {
    const int hh = idx / D, e = idx % D;
    float M = -__builtin_huge_valf();
#pragma unroll
    for (int v = 0; v < kKW; ++v) M = fmaxf(M, s_m[v][hh]);
    float A = 0.f, L = 0.f;
#pragma unroll
    for (int v = 0; v < kKW; ++v) {
      const float f = s_m[v][hh] == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(s_m[v][hh] - M);
      A = fmaf(f, s_acc[v][hh][e], A);
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

template <int BITS, int D>
hipError_t attn_by_group(const KiviArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)((size_t)a.batch * a.hkv));
  switch (a.hq / a.hkv) {
    case 1: hipLaunchKernelGGL((kivi_attention_kernel<BITS, D, 1>), grid, dim3(kivi_waves<D, 1>() * 64), 0, s, a); break;
    case 2: hipLaunchKernelGGL((kivi_attention_kernel<BITS, D, 2>), grid, dim3(kivi_waves<D, 2>() * 64), 0, s, a); break;
    case 4: hipLaunchKernelGGL((kivi_attention_kernel<BITS, D, 4>), grid, dim3(kivi_waves<D, 4>() * 64), 0, s, a); break;
    case 8: hipLaunchKernelGGL((kivi_attention_kernel<BITS, D, 8>), grid, dim3(kivi_waves<D, 8>() * 64), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kivi_attention(const KiviArgs &a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  if (a.bits == 8) return a.d == 64 ? attn_by_group<8, 64>(a, s) : attn_by_group<8, 128>(a, s);
  return a.d == 64 ? attn_by_group<4, 64>(a, s) : attn_by_group<4, 128>(a, s);
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
