// pa_chunk.hip -- gfx950 (CDNA4) kernel for the attention of several new
// tokens per sequence over the paged KV cache: a chunk of a long prompt's
// prefill, or the candidate tokens of speculative verification.
//
// What is computed: a sequence of ctx cached tokens whose last n are new has
// query rows at positions p = ctx - n, ..., ctx - 1 (their K/V are in the
// cache already, as for a decode step, "KV Cache 深度解析:显存黑洞、
// PagedAttention 与三路省内存方案" sections 五 and 六); the row at position p
// attends to the cached tokens 0..p and to nothing later:
//   out[row][h] = softmax_{t <= p}(scale * q[row][h] . K[t][g]) V[t][g],
// g = h / G, token t read from physical block table[b][t / 16], slot t % 16.
// A row whose position would be negative attends to nothing and gets zeros.
//
// How.  One workgroup per item: (sequence, KV head g, group of query rows,
// a row being one (query token, head of the group) pair).  Two kernels:
//
//  - chunk_kernel, up to 32 rows per item (short chunks, speculative
//    verification): the four waves split the item's visible blocks in pairs
//    (wave w takes pairs w, w + 4, ...), each staging its pairs through a
//    per-wave LDS tile as the decode kernel's matrix-core form does (loads
//    covering whole 128-byte pieces of 8 token rows, FP8 codes widened to
//    bf16 on the way, exactly), and are combined exactly in LDS at the end;
//  - chunk_wide_kernel, 256 rows per item (long prefill chunks): eight
//    waves each own 32 rows for the whole visible context, and every 64
//    tokens are staged once per workgroup in LDS, from where all of them
//    read their operands; each wave overlaps a pair's softmax with the
//    products of the pairs before and after it.
//
// In both, the products run on the matrix cores (v_mfma_f32_16x16x32_bf16,
// and _f16 for the wide kernel's PV products over bf16 pools), laid out so
// that every lane holds one query row's scores:
//
//  - S^T = K Q^T per block: A = K (row = token, lane % 16; k = 8 dims,
//    lane / 16), B = Q^T (column = query row, lane % 16), D/32 products
//    over the head dimension.  The result gives lane (row c = lane % 16,
//    q = lane / 16) the scores of tokens 4q .. 4q+3 of the block for row c.
//  - The online softmax (running max m and sum l per row, as in the
//    FlashAttention sections of the pages) is lane-local apart from a
//    4-lane max; the running max is raised only when a pair's maximum
//    exceeds it by more than kLag (log2 units), so rescaling is rare.
//  - O = P V over a pair of blocks (32 tokens): A = P, lane (row c, k = 8
//    tokens: 4q..4q+3 of each block), exactly the lane's own weights; B = V
//    read from the bf16 rows in LDS by transposing reads (ds_read_b64_tr_b16:
//    lane (n, q) receives dim 16m + n of those tokens).  A lane then holds
//    one dimension of rows 4q .. 4q+3 of its tile.
//  - The row sums l come out of the matrix cores too: the same weights
//    against an all-ones operand give every lane its rows' sums.
//  - FP8 pools: the K scale multiplies the score, the V scale the weight.
//
// Probabilities enter the PV product as a sum of two bf16 values, hi (the
// probability truncated to bf16) and lo (the remainder rounded to bf16):
// two products per slab, hi + lo within a relative 2^-16 of the fp32
// probability.  The normaliser l sums the same hi + lo, so the output is a
// convex combination of V rows whose weights are off by at most a relative
// 2^-15.  (One bf16 product, a relative 2^-9 per weight, gave errors up to
// 2.8e-3 on contexts of a few tokens.)  The wide kernel over bf16 pools
// instead stages V as fp16 (exact for bf16 magnitudes in [2^-14, 65504];
// below that an absolute error under 2^-24, above it saturated) and rounds
// each probability to the nearest fp16 (a relative 2^-11): one
// v_mfma_f32_16x16x32_f16 per slab, weights off by at most a relative
// 2^-10.  Its staging threads convert V once per stage for all 256 rows.
// FP8 pools keep the two bf16 terms: the V scale multiplies the weight,
// which could leave fp16's range.  Positions past a row's own, and
// blocks or table entries outside the pool, contribute exactly nothing:
// their scores are replaced by -inf and the V rows of slots past the cached
// tokens by zeros (selects, not products, so NaN garbage there cannot leak).

#include "pa_internal.h"
#include "pa_mfma.h"

#include <type_traits>

namespace pa {
namespace {

constexpr int kTok = 16;          // tokens per physical block
constexpr int kCW = 4;            // waves per workgroup
constexpr int kCThreads = kCW * 64;
constexpr float kLag = 8.0f;      // lag allowed to the running max (log2 units)
// running max before any score: finite, so that exp2(x - m) needs no guard;
// the first visible score always raises it (anything exceeds it by kLag)
constexpr float kNoMax = -3.402823466e38f;

// Quotient of non-negative ints (unsigned division: the shorter sequence).
__device__ __forceinline__ int udiv(int x, int y) { return (int)((unsigned)x / (unsigned)y); }

// A pointer the caller knows to be the same in every lane of the wave, made
// a scalar value.
__device__ __forceinline__ const char *wave_ptr(const char *p) {
  const uint64_t x = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return reinterpret_cast<const char *>(((uint64_t)hi << 32) | lo);
}

// Maxima that return NaN when an operand is NaN (v_maximum3_f32): no
// quieting of the operands first, unlike fmaxf.  Scores here are finite or
// -inf.
__device__ __forceinline__ float max3e(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
// the maximum over the four lanes q = 0..3 of a 16-lane column c
__device__ __forceinline__ float max4q_e(float x) {
  {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return x;
}

// Workgroup barrier that publishes LDS writes only.  __syncthreads() also
// waits for every global load the wave has in flight (its release fence
// waits for all vector memory operations), which would stall the loads of a
// later stage issued just before it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int D>
struct ChunkCfg {
  static constexpr int KM = D / 32;  // S^T products per block (32 dims each)
  static constexpr int EV = D / 16;  // 16-dim slabs of O (one PV product each)
};

template <int KV, int D, int G, int NQT>
__global__ __launch_bounds__(kCThreads) void chunk_kernel(ChunkArgs a) {
  using M = MCfg<KV, D>;
  constexpr int KM = M::KM, EV = M::EV, RSK = M::RSK;
  constexpr int ROWS = 16 * NQT;
  constexpr int OS = D + 4;  // LDS row stride (floats) of the combine, spreads the banks
  __shared__ __align__(16) char s_tile[kCW * M::TILE];
  __shared__ float s_o[kCW][16][OS];
  __shared__ float s_m[kCW][ROWS], s_l[kCW][ROWS];
  __shared__ __align__(16) float s_f[kCW][16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, q = lane >> 4;
  char *tile = s_tile + w * M::TILE;

  // ---- the item: consecutive workgroup indices alternate between the 8
  // XCDs, so each XCD is given a contiguous run of items (the tiles of one
  // (sequence, head) share its L2), heaviest tiles (latest rows) first.
  // (32-bit: the host refuses more than 2^31 - 1 items)
  const int items = a.batch * a.hkv * a.tiles;
  const int per = items >> 3, rem = items & 7;
  const int xcd = (int)(blockIdx.x & 7);
  const int item = xcd * per + min(xcd, rem) + (int)(blockIdx.x >> 3);
  const int bg = udiv(item, a.tiles);
  const int tile_i = a.tiles - 1 - (item - bg * a.tiles);
  const int b = udiv(bg, a.hkv), g = bg - b * a.hkv;
  const int *trow = a.table + (size_t)b * a.max_blocks;
  // the table entries of the wave's first 32 pairs, loaded with the lengths
  // (bounded by the table row; the visible length masks them below)
  int tv_first;
  {
    const int blk = 2 * (w + kCW * (lane >> 1)) + (lane & 1);
    tv_first = blk < a.max_blocks ? trow[blk] : -1;
  }

  const int n_ctx = min(max(a.ctx[b], 0), a.max_ctx);
  const int r0 = a.q_start[b], nq = a.q_start[b + 1] - r0;
  // no rows, or offsets that would leave q/out: nothing to do
  if (nq <= 0 || nq > a.max_q || r0 < 0 || r0 > a.total_q - nq) return;
  const int nrows = nq * G;
  const int row0 = tile_i * ROWS;
  if (row0 >= nrows) return;
  const int last_row = min(row0 + ROWS, nrows) - 1;
  const int pmax = n_ctx - nq + last_row / G;  // position of the item's last row
  const int nblk = pmax >= 0 ? pmax / kTok + 1 : 0;
  const int npairs = (nblk + 1) / 2;

  // ---- query rows of each 16-row tile (B operands of S^T: column = row c),
  // their positions, and the online-softmax state: max per row in lanes
  // (c, *); sums and output rows 4q .. 4q+3 in lanes (n, q)
  bf16x8_t qf[NQT][KM];
  int prow[NQT];
  f32x4_t o[NQT][EV];
  f32x4_t l4[NQT];
  float mrun[NQT];
  const float sl2 = a.scale_log2e;
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    const int r = row0 + 16 * t + c;
    const bool v = r < nrows;
    prow[t] = v ? n_ctx - nq + r / G : -1;
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) +
                         ((size_t)(r0 + (v ? r / G : 0)) * a.hq + g * G + (v ? r % G : 0)) * D + 8 * q;
#pragma unroll
    for (int m = 0; m < KM; ++m) {
      const uint4 x = v ? *reinterpret_cast<const uint4 *>(qp + 32 * m) : make_uint4(0, 0, 0, 0);
      qf[t][m] = as_bf16x8(x);
    }
    mrun[t] = kNoMax;
    l4[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < EV; ++m) o[t][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // first position of the item: a pair ending at or before it is visible to
  // every row, and needs no mask
  const int pfirst = n_ctx - nq + row0 / G;
  const bf16x8_t ones = bf16x8_ones();

  const StageLanes<KV, D> sl = stage_lanes<KV, D>(a.hkv, g);
  const size_t block_bytes = (size_t)kTok * a.hkv * M::ROW;
  auto issue = [&](PairLoads<KV, D> &P, int pair, int id0, int id1) {
    issue_pair<KV, D>(P, sl, a.k_cache, a.v_cache, a.k_scale, a.v_scale, block_bytes, a.hkv, g,
                      a.num_blocks, id0, id1, 2 * pair * kTok, (2 * pair + 1) * kTok);
  };

  auto compute = [&](const PairMeta &mt) {
    __builtin_amdgcn_wave_barrier();  // the tile's rows were written by other lanes
    // K operands (A of S^T: token c of block hb, dims 32m + 8q) and V
    // operands (B of O = P V), shared by the NQT row tiles
    uint4 kop[2][KM];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int m = 0; m < KM; ++m)
        kop[hb][m] = *reinterpret_cast<const uint4 *>(tile + (16 * hb + c) * RSK + (32 * m + 8 * q) * 2);
    bf16x8_t vb[EV];
#pragma unroll
    for (int m = 0; m < EV; ++m) vb[m] = v_operand_tr<D>(tile + 32 * RSK, M::RSV, m);
    // the whole pair visible to every row, both blocks in the pool: no mask
    const bool full = mt.ok[0] && mt.ok[1] && mt.tok[1] + kTok - 1 <= pfirst;
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      f32x4_t sc[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        sc[hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < KM; ++m)
          sc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kop[hb][m]), qf[t][m], sc[hb], 0, 0, 0);
      }
      // scaled scores (log2 units) of row c, tokens 4q .. 4q+3 of each block
      float x[2][4];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const float ksc[4] = {mt.ks[hb].x, mt.ks[hb].y, mt.ks[hb].z, mt.ks[hb].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[hb][j] = sc[hb][j] * sl2;
          if constexpr (KV == KV_FP8) x[hb][j] *= ksc[j];
        }
      }
      if (!full) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            x[hb][j] = (mt.ok[hb] && mt.tok[hb] + 4 * q + j <= prow[t]) ? x[hb][j] : -__builtin_huge_valf();
      }
      const float mx = max4q(max8(x));
      const bool raise = mx > mrun[t] + kLag;
      if (__builtin_amdgcn_ballot_w64(raise)) {
        const float mn = raise ? mx : mrun[t];
        const float f = raise ? __builtin_amdgcn_exp2f(mrun[t] - mn) : 1.f;
        mrun[t] = mn;
        // lane (c, q) has row c's factor; its O and l entries are rows 4q .. 4q+3
        if (q == 0) s_f[w][c] = f;
        __builtin_amdgcn_wave_barrier();
        const float4 f4 = *reinterpret_cast<const float4 *>(&s_f[w][4 * q]);
        __builtin_amdgcn_wave_barrier();
        const float fr[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          l4[t][r] *= fr[r];
#pragma unroll
          for (int m = 0; m < EV; ++m) o[t][m][r] *= fr[r];
        }
      }
      const float nm = -mrun[t];
      float pf[8];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int j = 0; j < 4; ++j) pf[4 * hb + j] = __builtin_amdgcn_exp2f(x[hb][j] + nm);  // masked: 0
      bf16x8_t ph, pl;
      split_bf16(pf, ph, pl);
      // the normaliser sums the same weights (hi + lo), on the matrix cores
      l4[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, ones, l4[t], 0, 0, 0);
      l4[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, ones, l4[t], 0, 0, 0);
      bf16x8_t wh = ph, wl = pl;
      if constexpr (KV == KV_FP8) {  // the V scale multiplies the PV weight
        float pv[8];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const float vsc[4] = {mt.vs[hb].x, mt.vs[hb].y, mt.vs[hb].z, mt.vs[hb].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float v = pf[4 * hb + j] * vsc[j];
            // a masked slot's scale may be anything (NaN included): weight 0
            pv[4 * hb + j] = (full || (mt.ok[hb] && mt.tok[hb] + 4 * q + j <= prow[t])) ? v : 0.f;
          }
        }
        split_bf16(pv, wh, wl);
      }
#pragma unroll
      for (int m = 0; m < EV; ++m) {
        o[t][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wh, vb[m], o[t][m], 0, 0, 0);
        o[t][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wl, vb[m], o[t][m], 0, 0, 0);
      }
    }
  };

  // ---- main loop: the wave's pairs w, w+4, ..., in chunks of 32 pairs whose
  // 64 table entries are read by one vector load (-1 past the visible
  // blocks); pair i is staged and computed while pairs i+1 and i+2 are in
  // flight.
  const int npw = npairs > w ? (npairs - w + kCW - 1) / kCW : 0;
  for (int i0 = 0; i0 < npw; i0 += 32) {
    const int cn = min(32, npw - i0);
    int tv;
    {
      const int blk = 2 * (w + kCW * (i0 + (lane >> 1))) + (lane & 1);
      tv = blk < nblk ? (i0 == 0 ? tv_first : trow[blk]) : -1;
    }
    auto id_of = [&](int i, int hb) { return __builtin_amdgcn_readlane(tv, 2 * i + hb); };  // i < 32
    auto pair_of = [&](int i) { return w + kCW * (i0 + i); };
    PairLoads<KV, D> A, B;
    issue(A, pair_of(0), id_of(0, 0), id_of(0, 1));
    if (cn > 1) issue(B, pair_of(1), id_of(1, 0), id_of(1, 1));
    int i = 0;
    for (; i + 3 < cn; i += 2) {
      const PairMeta ma = stage_pair<KV, D>(A, sl, tile, n_ctx);
      issue(A, pair_of(i + 2), id_of(i + 2, 0), id_of(i + 2, 1));
      __builtin_amdgcn_sched_barrier(0);
      compute(ma);
      const PairMeta mb = stage_pair<KV, D>(B, sl, tile, n_ctx);
      issue(B, pair_of(i + 3), id_of(i + 3, 0), id_of(i + 3, 1));
      __builtin_amdgcn_sched_barrier(0);
      compute(mb);
    }
    // at most three pairs left: i (in A), i + 1 (in B), i + 2 (not issued)
    if (i < cn) {
      const PairMeta ma = stage_pair<KV, D>(A, sl, tile, n_ctx);
      if (i + 2 < cn) issue(A, pair_of(i + 2), id_of(i + 2, 0), id_of(i + 2, 1));
      __builtin_amdgcn_sched_barrier(0);
      compute(ma);
    }
    if (i + 1 < cn) compute(stage_pair<KV, D>(B, sl, tile, n_ctx));
    if (i + 2 < cn) compute(stage_pair<KV, D>(A, sl, tile, n_ctx));
  }

  // ---- combine the four waves exactly, one 16-row tile at a time
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    if (q == 0) s_m[w][16 * t + c] = mrun[t];
    if (c == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s_l[w][16 * t + 4 * q + r] = l4[t][r];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {  // rows 4q + r of the tile: weight exp2(m_w - M)
      const int rr = 16 * t + 4 * q + r;
      float M = kNoMax;
#pragma unroll
      for (int v = 0; v < kCW; ++v) M = fmaxf(M, s_m[v][rr]);
      const float mw = s_m[w][rr];
      const float f = mw == kNoMax ? 0.f : __builtin_amdgcn_exp2f(mw - M);
#pragma unroll
      for (int m = 0; m < EV; ++m) s_o[w][4 * q + r][16 * m + c] = o[t][m][r] * f;
    }
    __syncthreads();
    for (int idx = tid; idx < 16 * (D / 4); idx += kCThreads) {
      const int cc = idx / (D / 4), d4 = (idx % (D / 4)) * 4;
      const int r = row0 + 16 * t + cc;
      if (r < nrows) {
        float Mr = kNoMax;
#pragma unroll
        for (int v = 0; v < kCW; ++v) Mr = fmaxf(Mr, s_m[v][16 * t + cc]);
        float L = 0.f;
        float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int v = 0; v < kCW; ++v) {
          const float mv = s_m[v][16 * t + cc];
          L += mv == kNoMax ? 0.f : __builtin_amdgcn_exp2f(mv - Mr) * s_l[v][16 * t + cc];
          const float4 x = *reinterpret_cast<const float4 *>(&s_o[v][cc][d4]);
          A.x += x.x; A.y += x.y; A.z += x.z; A.w += x.w;
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        float *op = a.out + ((size_t)(r0 + r / G) * a.hq + g * G + r % G) * D + d4;
        op[0] = A.x * inv; op[1] = A.y * inv; op[2] = A.z * inv; op[3] = A.w * inv;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Long chunks.  One workgroup per kWideRows query rows of a (sequence, KV
// head); each of its eight waves owns 32 of them (two 16-row tiles) over the
// whole visible context, so no combine across waves is needed.  Every
// 64 tokens (four blocks) are staged once per workgroup in LDS, in a ring
// of four stage buffers with one barrier per stage (a stage's global loads
// are in flight for two pairs' work before they are stored), and the waves
// read their MFMA operands from there: a K/V byte brought to the CU serves
// 256 rows, a byte read from LDS serves the wave's 32.  Each wave runs its
// 32-token pairs as a software pipeline, one step per pair: the PV products
// of the pair before and the score products of the pair after are issued
// around the current pair's softmax, and the K operands are read from LDS
// a step before their products.  Two waves per SIMD; with four waves of 64
// rows, one per SIMD, the two mostly took turns.  The products, masks and
// online softmax per 16-row tile are those of chunk_kernel.

constexpr int kWW = 8;                    // waves per workgroup (two per SIMD)
constexpr int kWT = 16 / kWW;             // 16-row tiles per wave
constexpr int kWThreads = kWW * 64;
constexpr int kWideRows = kWW * kWT * 16; // rows per workgroup
constexpr int kSB = 4;                    // blocks per LDS stage (two pairs)
constexpr int kSR = kSB * 16;             // token rows per stage
static_assert(kSR == 64, "FP8 scales: one wave per stage's K or V scales");
constexpr int kRing = 4;                  // LDS stage buffers in the wide kernel

template <int KV, int D>
struct WideCfg {
  // LDS row strides (bytes), chosen by the bank-conflict counter: a K
  // operand read takes 16 B of one row per lane (lanes on consecutive rows),
  // a transposing V read 8 B from each of 4 rows x 4 lanes (32 contiguous
  // bytes per row).  With rows 32 B apart modulo 128, neither conflicts:
  // what the counter still reports comes from the staging writes.  (K rows
  // 16 B apart, 48, 64 or 80: the K reads conflicted, a third of the LDS
  // active cycles; one stride of 64 B padding for both: 44%.)
  static constexpr int RSK = D * 2 + 32;
  static constexpr int RSV = D * 2 + 32;
  static constexpr int EB = KV == KV_FP8 ? 1 : 2;      // stored bytes per element
  static constexpr int ROWB = D * EB;                  // bytes of a token row (one head) in the pool
  static constexpr int ROWCH = ROWB / 16;              // 16-byte chunks per token row
  static constexpr int NCH = (kSR * ROWCH + kWThreads - 1) / kWThreads;  // chunks per thread per stage (K, and V)
  static constexpr bool ALL = kSR * ROWCH % kWThreads == 0;             // every thread has NCH chunks
  static constexpr int STAGE = kSR * (RSK + RSV);      // one stage: kSR K rows, then kSR V rows
};

template <int KV, int D, int G>
__global__ __launch_bounds__(kWThreads) __attribute__((amdgpu_waves_per_eu(kWW / 4))) void chunk_wide_kernel(ChunkArgs a) {
  using C = ChunkCfg<D>;
  using WC = WideCfg<KV, D>;
  constexpr int KM = C::KM, EV = C::EV;
  constexpr int RSK = WC::RSK, RSV = WC::RSV, NCH = WC::NCH, ROWCH = WC::ROWCH;
  constexpr bool ALL = WC::ALL;
  // how far ahead the K operands are read: two pairs, except over FP8
  // pools, whose two-term weights leave no room for them in registers
  constexpr int kKAhead = KV == KV_FP8 ? 1 : 2;
  __shared__ __align__(16) char s_kv[kRing * WC::STAGE];  // a ring of stages
  __shared__ __align__(16) float s_f[kWW][16];  // per-row rescaling factors
  // FP8: the K and V scales of each stage's tokens (0 for slots not real)
  __shared__ __align__(16) float s_sc[KV == KV_FP8 ? kRing : 1][2][kSR];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, q = lane >> 4;

  // ---- the item (same numbering as chunk_kernel: a contiguous run per XCD,
  // latest rows first)
  // (32-bit: the host refuses more than 2^31 - 1 items)
  const int items = a.batch * a.hkv * a.tiles;
  const int per = items >> 3, rem = items & 7;
  const int xcd = (int)(blockIdx.x & 7);
  const int item = xcd * per + min(xcd, rem) + (int)(blockIdx.x >> 3);
  const int bg = udiv(item, a.tiles);
  const int tile = a.tiles - 1 - (item - bg * a.tiles);
  const int b = udiv(bg, a.hkv), g = bg - b * a.hkv;

  const int n_ctx = min(max(a.ctx[b], 0), a.max_ctx);
  const int r0 = a.q_start[b], nq = a.q_start[b + 1] - r0;
  if (nq <= 0 || nq > a.max_q || r0 < 0 || r0 > a.total_q - nq) return;
  const int nrows = nq * G;
  const int row0 = tile * kWideRows;
  if (row0 >= nrows) return;  // uniform over the workgroup, before any barrier
  const int last_row = min(row0 + kWideRows, nrows) - 1;
  const int pmax = n_ctx - nq + last_row / G;
  const int nblk = pmax >= 0 ? pmax / kTok + 1 : 0;
  const int nstages = (nblk + kSB - 1) / kSB;

  // ---- the wave's rows
  const int wrow0 = row0 + 16 * kWT * w;
  const bool has_rows = wrow0 < nrows;
  const int pfirst = n_ctx - nq + wrow0 / G;                       // first row's position
  const int plast = n_ctx - nq + (min(wrow0 + 16 * kWT, nrows) - 1) / G;  // last row's position
  const int np = has_rows && plast >= 0 ? plast / 32 + 1 : 0;  // pairs visible to the wave

  // a negative scale is carried by the queries' signs (exact in bf16), so
  // that the multiplier sl2 of the scores is non-negative
  const bool neg = a.scale_log2e < 0.f;
  const float sl2 = neg ? -a.scale_log2e : a.scale_log2e;
  const uint32_t qflip = neg ? 0x80008000u : 0u;
  bf16x8_t qf[kWT][KM];
  int prow[kWT];
  f32x4_t o[kWT][EV];
  f32x4_t l4[kWT];
  float mrun[kWT];
#pragma unroll
  for (int t = 0; t < kWT; ++t) {
    const int r = wrow0 + 16 * t + c;
    const bool v = r < nrows;
    prow[t] = v ? n_ctx - nq + r / G : -1;
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) +
                         ((size_t)(r0 + (v ? r / G : 0)) * a.hq + g * G + (v ? r % G : 0)) * D + 8 * q;
#pragma unroll
    for (int m = 0; m < KM; ++m) {
      uint4 x = v ? *reinterpret_cast<const uint4 *>(qp + 32 * m) : make_uint4(0, 0, 0, 0);
      x.x ^= qflip; x.y ^= qflip; x.z ^= qflip; x.w ^= qflip;
      qf[t][m] = as_bf16x8(x);
    }
    mrun[t] = kNoMax;
    l4[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < EV; ++m) o[t][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8_t ones = bf16x8_ones();
  const f16x8_t ones16 = f16x8_ones();
  // the type of the staged V rows and PV operands: fp16 over bf16 pools
  using VOp = std::conditional_t<KV == KV_BF16, f16x8_t, bf16x8_t>;

  const int *trow = a.table + (size_t)b * a.max_blocks;
  const size_t block_bytes = (size_t)kTok * a.hkv * WC::ROWB;
  const char *kbase = static_cast<const char *>(a.k_cache);
  const char *vbase = static_cast<const char *>(a.v_cache);
  auto block_id = [&](int blk) { return blk < nblk ? trow[blk] : -1; };

  // ---- staging: thread tid moves chunks tid, tid + 512, ... of the stage's
  // kSR K rows and kSR V rows (16 chunks of 16 B per row for head_dim 128).
  // Slots past the cached tokens and blocks outside the pool are stored as
  // zeros: their scores are masked anyway, and V garbage (NaN) cannot leak
  // into the products.
  // What a thread's chunks are is the same in every stage, so it is worked
  // out once: chunk i is row ci / ROWCH, 16-byte column ci % ROWCH of the
  // stage (ci = tid + 512 i); its block of the stage, ci / (16 ROWCH), is
  // the same for the whole wave (a wave's 64 chunks never straddle two
  // blocks), so the block id is a scalar.
  constexpr int CB = 16 * (2 / WC::EB);  // bf16 bytes a chunk fills in the stage
  uint32_t c_src[NCH];  // bytes into a pool block: (slot, head g, column)
  uint32_t c_dst[NCH];  // bytes into a stage: the K row's column (V: + c_vdst[i])
  uint32_t c_vdst[NCH];
  int c_slot[NCH], c_hb[NCH];
  bool c_live[NCH];  // the chunk exists (not every thread has NCH of them)
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int ci = tid + kWThreads * i;
    c_live[i] = ALL || ci < kSR * ROWCH;
    const int cc = c_live[i] ? ci : 0;
    const int row = cc / ROWCH, col = cc % ROWCH;
    c_slot[i] = row & 15;
    c_hb[i] = __builtin_amdgcn_readfirstlane((w * 64 + kWThreads * i) / (16 * ROWCH));
    c_src[i] = (uint32_t)((c_slot[i] * a.hkv + g) * WC::ROWB + col * 16);
    c_dst[i] = (uint32_t)(row * RSK + col * CB);
    c_vdst[i] = (uint32_t)(kSR * RSK + row * RSV + col * CB);
  }
  uint4 sk[NCH], sv[NCH];
  bool sreal[NCH];
  bool sall = true;  // every slot of the stage real (wave-uniform)
  float ssc = 0.f;   // FP8: the scale thread tid < 2 kSR moves (wave 0: K, wave 1: V)
  auto stage_load = [&](int sg) {
    const int blk0 = kSB * sg;
    int id[kSB];
    sall = (blk0 + kSB) * kTok <= n_ctx;
#pragma unroll
    for (int h = 0; h < kSB; ++h) {
      id[h] = block_id(blk0 + h);
      sall = sall && (unsigned)id[h] < (unsigned)a.num_blocks;
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      if (!c_live[i]) break;
      int bid = id[0];
#pragma unroll
      for (int h = 1; h < kSB; ++h) bid = c_hb[i] == h ? id[h] : bid;
      const bool ok = (unsigned)bid < (unsigned)a.num_blocks;
      sreal[i] = ok && (blk0 + c_hb[i]) * kTok + c_slot[i] < n_ctx;
      const size_t boff = ok ? (size_t)bid * block_bytes : 0;
      // the block's base is the same for the whole wave: held in scalar
      // registers, the load adds the lane's 32-bit offset (no 64-bit
      // address per lane kept live across the loop)
      sk[i] = *reinterpret_cast<const uint4 *>(wave_ptr(kbase + boff) + c_src[i]);
      sv[i] = *reinterpret_cast<const uint4 *>(wave_ptr(vbase + boff) + c_src[i]);
    }
    if constexpr (KV == KV_FP8) {
      if (w < 2) {  // kSR = 64: one wave per scale
        const int r = tid % kSR, hb = r >> 4, slot = r & 15;
        int bid = id[0];
#pragma unroll
        for (int h = 1; h < kSB; ++h) bid = hb == h ? id[h] : bid;
        const bool ok = (unsigned)bid < (unsigned)a.num_blocks;
        // the table's base for head g in scalar registers, the block and
        // slot per lane
        const char *sc = wave_ptr(reinterpret_cast<const char *>(w == 0 ? a.k_scale : a.v_scale) +
                                  (size_t)g * kTok * sizeof(float));
        const size_t off = ((ok ? (size_t)bid : 0) * a.hkv * kTok + slot) * sizeof(float);
        const float x = *reinterpret_cast<const float *>(sc + off);
        ssc = ok && (blk0 + hb) * kTok + slot < n_ctx ? x : 0.f;
      }
    }
  };
  // one 16-byte chunk of a K or V row into the stage: bf16 as it is, FP8
  // codes widened to 32 bytes of bf16
  auto put = [&](char *dst, uint4 x) {
    if constexpr (KV == KV_FP8) {
      uint4 lo, hi;
      widen_fp8x16(x, lo, hi);
      reinterpret_cast<uint4 *>(dst)[0] = lo;
      reinterpret_cast<uint4 *>(dst)[1] = hi;
    } else {
      *reinterpret_cast<uint4 *>(dst) = x;
    }
  };
  // V rows: fp16 over bf16 pools (the PV products take fp16 operands there),
  // as put() over FP8 pools
  auto put_v = [&](char *dst, uint4 x) {
    if constexpr (KV == KV_BF16)
      *reinterpret_cast<uint4 *>(dst) = bf16x8_to_f16x8(x);
    else
      put(dst, x);
  };
  auto stage_store = [&](int sg) {
    const int st = sg & (kRing - 1);  // its buffer in the ring
    char *base = s_kv + st * WC::STAGE;
    if constexpr (KV == KV_FP8) {
      if (w < 2) s_sc[st][w][lane] = ssc;
    }
    if (sall) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        if (!c_live[i]) break;
        put(base + c_dst[i], sk[i]);
        put_v(base + c_vdst[i], sv[i]);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      if (!c_live[i]) break;
      const uint32_t mk = sreal[i] ? 0xFFFFFFFFu : 0u;  // per word: a select of the
                                                        // whole vector would go through memory
      put(base + c_dst[i], make_uint4(sk[i].x & mk, sk[i].y & mk, sk[i].z & mk, sk[i].w & mk));
      put_v(base + c_vdst[i], make_uint4(sv[i].x & mk, sv[i].y & mk, sv[i].z & mk, sv[i].w & mk));
    }
  };

  // ---- the software pipeline.  Pair j of the wave (blocks 2j, 2j + 1, in
  // LDS stage j / 2, token rows 32 (j % 2) .. +31) goes through three steps:
  // its score products are issued at the end of step j - 1, its softmax
  // runs in step j and its PV products are issued in step j + 1.  So step j
  // holds
  //   the rescaling of O and l for a rise of the running max in step j - 1;
  //   the PV products of pair j - 1, next to the maxima of pair j;
  //   pair j's exponentials (while those products run);
  //   the score products of pair j + 1 (while the next step starts), and
  //   over bf16 pools the K operands of pair j + 2.
  // Step j reads the stages of pairs j - 1 to j + 2: the stages live in a
  // ring of kRing = 4 LDS buffers.  Stage t + 1 is stored before step 2t and
  // published by the barrier right after; it overwrites stage t - 3, whose
  // last read (the V operands of pair 2t - 5, in step 2t - 4) every wave
  // has made before the barrier of the previous stage, which the storing
  // wave has passed.
  auto stage_of = [&](int p) { return (p >> 1) & (kRing - 1); };  // LDS buffer of pair p's stage
  // FP8: scales of tokens 4q .. 4q+3 of block hb of pair p (read where used,
  // which keeps the kernel within its 256 registers)
  auto scales = [&](int which, int p, int hb) {
    return *reinterpret_cast<const float4 *>(
        &s_sc[KV == KV_FP8 ? stage_of(p) : 0][which][32 * (p & 1) + 16 * hb + 4 * q]);
  };
  // per-lane byte offsets in a stage: the K operand (token c, dims 8q ..
  // 8q + 7) and the transposing V read (token 4q + c / 4, dims 4 (c % 4) ..)
  const uint32_t lane_k = c * RSK + 16 * q;
  const uint32_t lane_v = kSR * RSK + (4 * q + (c >> 2)) * RSV + 8 * (c & 3);
  // the A operands of pair p's score products: token c of block hb, dims
  // 32m + 8q .. +7
  auto kload = [&](int p, uint4 (&kop)[2][KM]) {
    const char *lk = s_kv + stage_of(p) * WC::STAGE + 32 * (p & 1) * RSK + lane_k;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int m = 0; m < KM; ++m)
        kop[hb][m] = *reinterpret_cast<const uint4 *>(lk + 16 * hb * RSK + 64 * m);
  };
  // the score products of a pair from its A operands
  auto score = [&](const uint4 (&kop)[2][KM], f32x4_t (&s)[kWT][2]) {
#pragma unroll
    for (int u = 0; u < kWT; ++u)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        s[u][hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < KM; ++m)
          s[u][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kop[hb][m]), qf[u][m], s[u][hb], 0, 0, 0);
      }
  };
  // the weights a pair's softmax leaves for its PV products one step later:
  // fp16 over bf16 pools; over FP8 pools hi + lo bf16, for the row sums and
  // (with the V scale) for the products
  f16x8_t pw16[kWT];
  bf16x8_t pwb[KV == KV_FP8 ? kWT : 1][4];
  f32x4_t sc[kWT][2];  // the scores of the pair whose softmax runs next
  // K operands read ahead: those of pair j + 1 during step j when kKAhead
  // is 2 (read at the end of step j - 1), else read where used
  uint4 kpre[2][KM];
  // a rise of the running max in the last step, with the maxima before it
  bool pend = false;
  float mold[kWT];
  (void)pw16;
  (void)pwb;

  // step j.  hp: the PV products of pair j - 1 are due; hc: pair j has
  // scores, in sc; hn: pair j + 1's score products are issued (into sc,
  // after pair j's exponentials have read it)
  auto step = [&](int j, auto HP, auto HC, auto HN) {
    constexpr bool hp = decltype(HP)::value, hc = decltype(HC)::value, hn = decltype(HN)::value;
    // the rescaling due from the previous step's rise of the running max
    // (rows not raised: exp2(0) = 1)
    if (pend) {
#pragma unroll
      for (int u = 0; u < kWT; ++u) {
        const float f = __builtin_amdgcn_exp2f(mold[u] - mrun[u]);
        // lane (c, q) holds the factor of row c; its O and l entries are
        // rows 4q .. 4q+3: fetch those rows' factors from lanes 4q + r
        // through LDS: row c's lanes write it, then every lane reads its
        // four rows' factors at once
        if (q == 0) s_f[w][c] = f;
        __builtin_amdgcn_wave_barrier();
        const float4 f4 = *reinterpret_cast<const float4 *>(&s_f[w][4 * q]);
        __builtin_amdgcn_wave_barrier();
        const float fr[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          l4[u][r] *= fr[r];
#pragma unroll
          for (int m = 0; m < EV; ++m) o[u][m][r] *= fr[r];
        }
      }
      pend = false;
    }
    // pair j's maxima: over the raw scores when the pair needs no mask
    // (the multiplier is non-negative, so it scales the maximum too);
    // otherwise over the scaled, masked scores, which replace the raw ones
    float mloc[kWT];
    float kx = 1.f;  // multiplier of sc in the exponent (wave-uniform)
    if constexpr (hc) {
      const int blk0 = 2 * j;
      const bool ok0 = (unsigned)block_id(blk0) < (unsigned)a.num_blocks;
      const bool ok1 = (unsigned)block_id(blk0 + 1) < (unsigned)a.num_blocks;
      const bool full = ok0 && ok1 && (blk0 + 2) * kTok - 1 <= pfirst;
      if (KV == KV_BF16 && full) {
        kx = sl2;
      } else {
#pragma unroll
        for (int u = 0; u < kWT; ++u)
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            float ksc[4] = {1.f, 1.f, 1.f, 1.f};
            if constexpr (KV == KV_FP8) {
              const float4 k4 = scales(0, j, hb);
              ksc[0] = k4.x; ksc[1] = k4.y; ksc[2] = k4.z; ksc[3] = k4.w;
            }
            const bool okh = hb ? ok1 : ok0;
            const int tok0 = (blk0 + hb) * kTok + 4 * q;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float x = sc[u][hb][e] * sl2;
              if constexpr (KV == KV_FP8) x *= ksc[e];
              sc[u][hb][e] = full || (okh && tok0 + e <= prow[u]) ? x : -__builtin_huge_valf();
            }
          }
      }
#pragma unroll
      for (int u = 0; u < kWT; ++u)
        mloc[u] = max3e(max3e(sc[u][0][0], sc[u][0][1], sc[u][0][2]), max3e(sc[u][0][3], sc[u][1][0], sc[u][1][1]),
                        max3e(sc[u][1][2], sc[u][1][3], sc[u][1][3]));
    }

    // A. PV products of pair j - 1.  B operands, one per 16 dims (slab m):
    // lane (n = c, q) needs V[token 4q + e of block hb][dim 16m + n] for
    // e = 0..3, hb = 0, 1.  ds_read_b64_tr_b16 gives lane i of a 16-lane
    // group element i % 4 of the 8 bytes addressed by lanes 4r + i / 4,
    // r = 0..3 (checked on the GPU with a one-wave probe); so lane 4r + s
    // addresses token 4q + r, dims 16m + 4s .. 16m + 4s + 3, of the
    // row-major V rows in LDS.  Lane (c, q)'s eight weights are row c's
    // tokens 4q .. 4q+3 of both blocks, the same k order.
    if constexpr (hp) {
      const int p = j - 1;
      const char *lv = s_kv + stage_of(p) * WC::STAGE + 32 * (p & 1) * RSV + lane_v;
      VOp vb[EV];
#pragma unroll
      for (int m = 0; m < EV; ++m) {
        v4s_t h[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          h[hb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4s_t *)(lv + 16 * hb * RSV + 32 * m));
        vb[m] = __builtin_bit_cast(VOp, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int u = 0; u < kWT; ++u) {
        if constexpr (KV == KV_BF16) {
          // fp16 weights (within a relative 2^-11) and fp16 V, one product
          // per slab; the row sums from the same fp16 weights
          l4[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pw16[u], ones16, l4[u], 0, 0, 0);
#pragma unroll
          for (int m = 0; m < EV; ++m)
            o[u][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pw16[u], vb[m], o[u][m], 0, 0, 0);
        } else {
          // FP8: the weights as hi + lo bf16, two products per slab
          l4[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pwb[u][0], ones, l4[u], 0, 0, 0);
          l4[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pwb[u][1], ones, l4[u], 0, 0, 0);
#pragma unroll
          for (int m = 0; m < EV; ++m) {
            o[u][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pwb[u][2], vb[m], o[u][m], 0, 0, 0);
            o[u][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pwb[u][3], vb[m], o[u][m], 0, 0, 0);
          }
        }
      }
    }

    // the lagged running max: raised only when a pair's max exceeds it by
    // more than kLag.  O and l are rescaled at the start of the next step:
    // after pair j - 1's products (issued above), before pair j's.
    if constexpr (hc) {
      bool any = false;
#pragma unroll
      for (int u = 0; u < kWT; ++u) {
        const float mx = max4q_e(mloc[u]) * kx;
        const bool raise = mx > mrun[u] + kLag;
        any = any || raise;
        mold[u] = mrun[u];
        mrun[u] = raise ? mx : mrun[u];
      }
      pend = __builtin_amdgcn_ballot_w64(any) != 0;
    }

    // B. score products of pair j + 1; pair j's weights
    if constexpr (hc) {
#pragma unroll
      for (int u = 0; u < kWT; ++u) {
        const float nm = -mrun[u];
        float pf[8];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int e = 0; e < 4; ++e) pf[4 * hb + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[u][hb][e], kx, nm));
        if constexpr (KV == KV_BF16) {
          pw16[u] = to_f16x8(pf);
        } else {
          // the V scale multiplies the PV weight (masked: 0 x 0)
          split_bf16(pf, pwb[u][0], pwb[u][1]);
          float pv[8];
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            const float4 v4 = scales(1, j, hb);
            const float vsc[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) pv[4 * hb + e] = pf[4 * hb + e] * vsc[e];
          }
          split_bf16(pv, pwb[u][2], pwb[u][3]);
        }
      }
    }
    // the score products of pair j + 1, into the registers pair j's
    // exponentials have just read; then the K operands of pair j + 2
    if constexpr (hn) {
      if constexpr (kKAhead == 2) {
        score(kpre, sc);
        kload(j + 2, kpre);
      } else {
        kload(j + 1, kpre);
        score(kpre, sc);
      }
    }
  };
  // the parts of a step are fixed at compile time (branches on them would
  // make the accumulators go through copies).  Every step of the loop is
  // the steady form: step np, one past the wave's last visible pair, takes
  // the pair after it as fully masked (its positions are past every row's,
  // so its weights are exactly 0 and the running max stays), and issues
  // score products for the pair after that, never used; later steps are
  // skipped.  Their K reads stay inside the ring of LDS buffers.
  using T_ = std::true_type;
  using F_ = std::false_type;
  // before step j = 2t (even), stage t + 1 is stored and published (step
  // j reads the K operands of its first pair) and stage t + 2 loaded
  auto handoff = [&](int j) {
    const int t = j >> 1;
    if (t + 1 < nstages) {
      stage_store(t + 1);
      if (t + 2 < nstages) stage_load(t + 2);
    }
    lds_barrier();
  };

  // ---- main loop, one step per pair; every wave takes part in the staging
  // and the barriers to the end, also after its last visible pair
  if (nstages > 0) {
    stage_load(0);
    stage_store(0);
    if (nstages > 1) stage_load(1);
    lds_barrier();
    handoff(0);  // stage 1
    if (np > 0) {
      kload(0, kpre);
      score(kpre, sc);
      if constexpr (kKAhead == 2) kload(1, kpre);
      step(0, F_{}, T_{}, T_{});
    }
    // the wave's steps (none behind a branch, so that the accumulators stay
    // in place), then the staging of the rest
    const int jl = min(np, 2 * nstages - 1);
    int j = 1;
    for (; j <= jl; ++j) {
      if (!(j & 1)) handoff(j);
      step(j, T_{}, T_{}, T_{});
    }
    for (; j < 2 * nstages; ++j)
      if (!(j & 1)) handoff(j);
    // the last pair's PV products, when the wave sees every pair
    if (np == 2 * nstages) step(np, T_{}, F_{}, F_{});
  }

  // ---- normalise and write the wave's rows: lane (n = c, q) holds dim
  // 16m + n of rows 4q .. 4q+3 of each tile (and those rows' sums)
  if (!has_rows) return;
#pragma unroll
  for (int t = 0; t < kWT; ++t)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = wrow0 + 16 * t + 4 * q + rr;
      if (r < nrows) {
        const float L = l4[t][rr];
        const float inv = L > 0.f ? 1.f / L : 0.f;
        float *op = a.out + ((size_t)(r0 + r / G) * a.hq + g * G + r % G) * D + c;
#pragma unroll
        for (int m = 0; m < EV; ++m) op[16 * m] = o[t][m][rr] * inv;
      }
    }
}


template <int KV, int D, int G>
hipError_t chunk_by_tiles(const ChunkArgs &a, unsigned grid, hipStream_t s) {
  if (a.nqt == 1) {
    hipLaunchKernelGGL((chunk_kernel<KV, D, G, 1>), dim3(grid), dim3(kCThreads), 0, s, a);
  } else if (a.nqt == 2) {
    hipLaunchKernelGGL((chunk_kernel<KV, D, G, 2>), dim3(grid), dim3(kCThreads), 0, s, a);
  } else if (a.nqt == kWideRows / 16) {
    hipLaunchKernelGGL((chunk_wide_kernel<KV, D, G>), dim3(grid), dim3(kWThreads), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KV, int D>
hipError_t chunk_by_group(const ChunkArgs &a, unsigned grid, hipStream_t s) {
  switch (a.hq / a.hkv) {
    case 1: return chunk_by_tiles<KV, D, 1>(a, grid, s);
    case 2: return chunk_by_tiles<KV, D, 2>(a, grid, s);
    case 4: return chunk_by_tiles<KV, D, 4>(a, grid, s);
    case 8: return chunk_by_tiles<KV, D, 8>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int KV>
hipError_t chunk_by_dim(const ChunkArgs &a, unsigned grid, hipStream_t s) {
  switch (a.d) {
    case 64: return chunk_by_group<KV, 64>(a, grid, s);
    case 128: return chunk_by_group<KV, 128>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int chunk_tiles_per_item(int max_q, int group, int d) {
  const long long rows = (long long)max_q * group;
  (void)d;
  return rows <= 16 ? 1 : (rows <= 256 ? 2 : kWideRows / 16);
}

int chunk_items_per_head(int max_q, int group, int nqt) {
  const long long rows = (long long)max_q * group;
  return (int)((rows + 16LL * nqt - 1) / (16LL * nqt));
}

bool chunk_supported(int kv, int d, int group) {
  return (kv == KV_BF16 || kv == KV_FP8) && (d == 64 || d == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_chunk(const ChunkArgs &a, hipStream_t s) {
  const long long items = (long long)a.batch * a.hkv * a.tiles;
  if (items == 0) return hipSuccess;
  if (items > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)items;
  switch (a.kv) {
    case KV_BF16: return chunk_by_dim<KV_BF16>(a, grid, s);
    case KV_FP8: return chunk_by_dim<KV_FP8>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
