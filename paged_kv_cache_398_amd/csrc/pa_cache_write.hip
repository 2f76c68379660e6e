// pa_cache_write.hip -- gfx950 kernel that writes each sequence's new token
// into the paged cache (the write half of a decode step).
//
// What is written: the decode step appends the token's key and value to the
// sequence's cache before attending ("KV Cache 深度解析:显存黑洞、
// PagedAttention 与三路省内存方案", sections 一 and 六); context_lens[b]
// already counts the new token, so it goes to position t = context_lens[b]-1,
// i.e. physical block table[b][t / 16], slot t % 16 (same page, section 三),
// one head_dim row per KV head, K and V in their separate pools.  For an FP8
// pool each (token, head) row is quantised on the way in (same page, section
// 四): scale = absmax / 448 (1 for an all-zero row), codes = E4M3FN nearest
// even of clamp(x / scale, -448, 448), all in float32 with IEEE division.
//
// One wave per (sequence, KV head); lanes take head_dim / 64 elements each.

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kBlockTokens = 16;
constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ __forceinline__ float src_value(const void *p, size_t i, int src) {
  if (src == KV_F32) return static_cast<const float *>(p)[i];
  return __uint_as_float((uint32_t) static_cast<const uint16_t *>(p)[i] << 16);
}

// Nearest-even E4M3FN code of a value already clamped to [-448, 448].
__device__ __forceinline__ uint8_t to_e4m3fn(float y) {
  return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, 0, false) & 0xFF);
}

template <int KV, int D>
__global__ __launch_bounds__(64) void append_kernel(AppendArgs a) {
  constexpr int PER = D / 64;  // elements per lane
  const int lane = threadIdx.x;
  const int b = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv;
  const int n = min(max(a.ctx[b], 0), a.max_ctx);
  if (n == 0) return;  // no new token
  const int t = n - 1;
  const int phys = a.table[(size_t)b * a.max_blocks + t / kBlockTokens];
  if ((unsigned)phys >= (unsigned)a.num_blocks) return;  // never written out of the pool
  const int slot = t % kBlockTokens;
  const size_t row = (((size_t)phys * kBlockTokens + slot) * a.hkv + g) * D;
  const size_t src_row = ((size_t)b * a.hkv + g) * D;

#pragma unroll
  for (int which = 0; which < 2; ++which) {  // K, then V
    const void *src = which == 0 ? a.k_new : a.v_new;
    if constexpr (KV == KV_F32) {
      float *dst = static_cast<float *>(which == 0 ? a.k_cache : a.v_cache);
#pragma unroll
      for (int k = 0; k < PER; ++k)
        dst[row + lane + 64 * k] = static_cast<const float *>(src)[src_row + lane + 64 * k];
    } else if constexpr (KV == KV_BF16) {
      uint16_t *dst = static_cast<uint16_t *>(which == 0 ? a.k_cache : a.v_cache);
#pragma unroll
      for (int k = 0; k < PER; ++k)
        dst[row + lane + 64 * k] = static_cast<const uint16_t *>(src)[src_row + lane + 64 * k];
    } else {
      float x[PER], amax = 0.f;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        x[k] = src_value(src, src_row + lane + 64 * k, a.src);
        amax = fmaxf(amax, fabsf(x[k]));
      }
      amax = wave_max(amax);
      const float scale = amax > 0.f ? amax / kE4M3Max : 1.0f;
      uint8_t *dst = static_cast<uint8_t *>(which == 0 ? a.k_cache : a.v_cache);
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const float y = fminf(fmaxf(x[k] / scale, -kE4M3Max), kE4M3Max);
        dst[row + lane + 64 * k] = to_e4m3fn(y);
      }
      float *sc = which == 0 ? a.k_scale : a.v_scale;
      if (lane == 0) sc[((size_t)phys * a.hkv + g) * kBlockTokens + slot] = scale;
    }
  }
}

template <int KV>
hipError_t append_by_dim(const AppendArgs &a, hipStream_t s) {
  const unsigned grid = (unsigned)((size_t)a.batch * a.hkv);
  if (a.d == 64)
    hipLaunchKernelGGL((append_kernel<KV, 64>), dim3(grid), dim3(64), 0, s, a);
  else if (a.d == 128)
    hipLaunchKernelGGL((append_kernel<KV, 128>), dim3(grid), dim3(64), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// One workgroup per (src, dst) pair: the K and V bytes of the block in
// 16-byte pieces, then its parameters (FP8 scales, or KIVI scales and mins).  Pairs with an id outside the pool,
// or src == dst, are skipped.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a) {
  const int i = blockIdx.x;
  const int src = a.pairs[2 * i], dst = a.pairs[2 * i + 1];
  if ((unsigned)src >= (unsigned)a.num_blocks || (unsigned)dst >= (unsigned)a.num_blocks ||
      src == dst)
    return;
  const int64_t n16 = a.block_bytes / 16;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    char *base = static_cast<char *>(which == 0 ? a.k_cache : a.v_cache);
    const uint4 *from = reinterpret_cast<const uint4 *>(base + (size_t)src * a.block_bytes);
    uint4 *to = reinterpret_cast<uint4 *>(base + (size_t)dst * a.block_bytes);
    for (int64_t k = threadIdx.x; k < n16; k += 256) {
      const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(from + k));
      __builtin_nontemporal_store(x, reinterpret_cast<u32x4_t *>(to + k));
    }
    const int words = which == 0 ? a.k_par_words : a.v_par_words;
    if (words > 0) {
      uint32_t *par = static_cast<uint32_t *>(which == 0 ? a.k_par : a.v_par);
      for (int k = threadIdx.x; k < words; k += 256)
        par[(size_t)dst * words + k] = par[(size_t)src * words + k];
    }
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyArgs &a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)a.n), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs &a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  switch (a.kv) {
    case KV_F32: return append_by_dim<KV_F32>(a, s);
    case KV_BF16: return append_by_dim<KV_BF16>(a, s);
    case KV_FP8: return append_by_dim<KV_FP8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
