// Internal interface between the C-ABI layer (pa_api.cpp) and the kernels
// (pa_kernels.hip).  Not installed; the public interface is include/pa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

enum KvKind : int { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

// Waves per workgroup of the attention kernel.  A workgroup owns one context
// partition of one sequence for a chunk of `hc` KV heads; wave w works on
// head w % hc of the chunk and takes every (kWaves / hc)-th block of the
// partition, so the workgroup as a whole streams whole physical blocks.
constexpr int kWaves = 4;

// Loads of cache bytes that one launch reads exactly once.  They carry the
// non-temporal hint, so the caches do not keep lines that will not be read
// again; on the decode step this raised the sustained KV read rate by about
// 10% over plain loads.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_stream16(const void *p) {
  const u32x4_t x = __builtin_nontemporal_load(static_cast<const u32x4_t *>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ uint2 load_stream8(const void *p) {
  const u32x2_t x = __builtin_nontemporal_load(static_cast<const u32x2_t *>(p));
  return make_uint2(x[0], x[1]);
}
__device__ __forceinline__ uint32_t load_stream4(const void *p) {
  return __builtin_nontemporal_load(static_cast<const uint32_t *>(p));
}

// Everything one decode launch needs; plain pointers into device memory.
struct LaunchArgs {
  const void *k_cache;      // [num_blocks][16][hkv][d]
  const void *v_cache;
  const float *k_scale;     // [num_blocks][hkv][16] (FP8 only)
  const float *v_scale;
  const void *q;            // [batch][hq][d]
  const int32_t *table;     // [batch][max_blocks]
  const int32_t *ctx;       // [batch]
  float *out;               // [batch][hq][d]
  float2 *ws_ml;            // [nwg][2][hc*G] partial (running max, running sum)
  float *ws_acc;            // [nwg][2][hc*G][d] partial unnormalised output
  uint32_t *counters;       // [nwg] arrival counters (indexed by the first workgroup of
                            // a split pair), zero before and after every run
  int32_t num_blocks, hkv, hq, d, batch, max_blocks, max_ctx;
  int32_t nwg;              // workgroups (equal ranges of the work)
  int32_t hc;               // KV heads per workgroup when every sequence has the
                            // block count of max_ctx (divides hkv and kWaves)
  int32_t chunks;           // hkv / hc
  int32_t hc_var;           // KV heads per workgroup otherwise (>= hc)
  float scale_log2e;        // softmax scale * log2(e)
  int kv;                   // KvKind
};

// What the cache-write kernel needs: the pools (written), this step's
// tables, and the new tokens' K/V rows.
struct AppendArgs {
  void *k_cache, *v_cache;  // [num_blocks][16][hkv][d]
  float *k_scale, *v_scale; // [num_blocks][hkv][16] (FP8 only)
  const void *k_new, *v_new;  // [batch][hkv][d] of src
  const int32_t *table;     // [batch][max_blocks]
  const int32_t *ctx;       // [batch]
  int32_t num_blocks, hkv, d, batch, max_blocks, max_ctx;
  int kv;                   // KvKind of the pool
  int src;                  // KvKind of k_new / v_new (KV_F32 or KV_BF16)
};

// Enqueue the cache-write kernel (grid batch * hkv waves).
hipError_t launch_append(const AppendArgs &a, hipStream_t stream);

// What the multi-token (chunk) kernel needs.  Query rows are token-major,
// rows q_start[b] .. q_start[b+1]-1 belonging to sequence b; the work is
// counted in items (sequence, KV head, tile of 16 * nqt query rows, a row
// being one (query token, head of the group) pair).
struct ChunkArgs {
  const void *k_cache;      // [num_blocks][16][hkv][d] bf16, or FP8 codes
  const void *v_cache;
  const float *k_scale;     // [num_blocks][hkv][16] (FP8 only)
  const float *v_scale;
  const void *q;            // [total_q][hq][d] bf16
  const int32_t *table;     // [batch][max_blocks]
  const int32_t *ctx;       // [batch]
  const int32_t *q_start;   // [batch + 1]
  float *out;               // [total_q][hq][d]
  int32_t num_blocks, hkv, hq, d, batch, max_blocks, max_ctx;
  int32_t max_q;            // host bound on rows per sequence
  int32_t total_q;          // rows of q and out
  int32_t nqt;              // 16-row tiles per item (1, 2, or 4 for d = 64)
  int32_t tiles;            // items per (sequence, KV head)
  float scale_log2e;        // softmax scale * log2(e)
  int kv;                   // KvKind of the pool (KV_BF16 or KV_FP8)
};

// Tiles of 16 rows per item for a launch whose sequences have up to max_q
// new tokens each, and the items per (sequence, KV head).
int chunk_tiles_per_item(int max_q, int group, int d);
int chunk_items_per_head(int max_q, int group, int nqt);

// True when the chunk kernel is built for (pool kind, head_dim, group size).
bool chunk_supported(int kv, int d, int group);

// Enqueue the chunk kernel (one workgroup per item).
hipError_t launch_chunk(const ChunkArgs &a, hipStream_t stream);

// True when a kernel is built for (kv, head_dim, group size).
bool kernel_supported(int kv, int d, int group);

// Enqueue the attention kernel (grid nwg workgroups of kWaves waves).  With
// ev_start (and ev_stop), the two events record the start and the end of
// the kernel's own execution (attached to its dispatch).
hipError_t launch_attention(const LaunchArgs &a, hipStream_t stream,
                            hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// An INT8 / INT4 pool quantised the KIVI way (codes, fp16 parameters) with
// the bf16 residual of each sequence's partly filled last block.
struct KiviArgs {
  void *k_codes, *v_codes;  // [num_blocks][hkv][16][d * bits / 8] (head-major)
  void *k_par;              // fp16 [num_blocks][hkv][2][d]: scales, then mins
  void *v_par;              // fp16 [num_blocks][hkv][16][2]: (scale, min) per slot
  void *res_k, *res_v;      // bf16 [batch][16][hkv][d]
  const void *q;            // bf16 [batch][hq][d]
  const int32_t *table;     // [batch][max_blocks]
  const int32_t *ctx;       // [batch]
  float *out;               // [batch][hq][d]
  int32_t num_blocks, hkv, hq, d, batch, max_blocks, max_ctx, bits;
  float scale_log2e;
};
hipError_t launch_kivi_attention(const KiviArgs &a, hipStream_t stream,
                                 hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
hipError_t launch_kivi_append(const KiviArgs &a, const void *k_new, const void *v_new,
                              hipStream_t stream);

// The text pa_last_error() returns: set with a status, or cleared.
pa_status record_error(pa_status s, const char *msg);
void clear_error();

// Enqueue a kernel that copies whole blocks (K, V and, with FP8, their
// scales): pairs[i] = (src, dst), device int32 [n][2]; pairs naming a block
// outside [0, num_blocks) or src == dst are skipped.
struct CopyArgs {
  void *k_cache, *v_cache;
  void *k_par, *v_par;       // per-block parameters (FP8 scales, KIVI), or NULL
  const int32_t *pairs;
  int32_t n, num_blocks;
  int64_t block_bytes;       // K (or V) bytes of one block, a multiple of 16
  int32_t k_par_words;       // 32-bit words of K parameters per block, 0 if none
  int32_t v_par_words;       // same for V
};
hipError_t launch_copy_blocks(const CopyArgs &a, hipStream_t stream);

// Bytes of the file-scope device scratch used by pa_decode_run_noalloc.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;

// Device address of that scratch on the current device (looked up once per
// device with hipGetSymbolAddress, then cached).  Allocates nothing.
hipError_t static_scratch(void **ptr);

// Enqueue a kernel that sets n 32-bit words to zero (a kernel rather than a
// memset, so that a captured graph replays it faithfully).  Only device
// addresses (a caller's buffer, or a device symbol's address obtained with
// hipGetSymbolAddress) may be passed.
hipError_t launch_zero(uint32_t *p, size_t n, hipStream_t stream);

}  // namespace pa
