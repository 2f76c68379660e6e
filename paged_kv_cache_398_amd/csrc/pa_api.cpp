// pa_api.cpp -- the C ABI of include/pa.h: argument validation, launch
// choice, workspace layout and kernel launches on the caller's stream.
//
// Every entry point validates on the host before touching the HIP runtime,
// so argument errors are reported without a GPU.  Callers pass every data
// buffer and every scratch buffer; no entry point allocates or frees device
// memory or waits for the device (pa_block_table_validate and
// pa_profile_read, two debugging aids, wait).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

struct pa_kv_pool {
  int32_t num_blocks = 0, num_kv_heads = 0, head_dim = 0;
  pa_dtype kv_dtype = PA_DTYPE_F32;
  void *k_cache = nullptr, *v_cache = nullptr;
  float *k_scale = nullptr, *v_scale = nullptr;
  // INT8 / INT4 (KIVI) pools: bits, fp16 parameters, and this step's residual
  int32_t kivi_bits = 0;
  void *k_par = nullptr, *v_par = nullptr;
  void *res_k = nullptr, *res_v = nullptr;
  // block tables of the current step
  bool table_set = false;
  const int32_t *block_table = nullptr, *context_lens = nullptr;
  int32_t batch = 0, max_blocks_per_seq = 0, max_context_len = 0;
  int32_t workgroups_override = 0;  // 0: automatic
  int32_t heads_override = 0;       // 0: automatic
  // profiling
  int32_t prof_capacity = 0, prof_count = 0;
  std::vector<hipEvent_t> prof_events;  // 2 per run: before and after the kernel
};

namespace {

thread_local std::string g_last_error;

pa_status fail(pa_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

pa_status ok() {
  g_last_error.clear();
  return PA_OK;
}

}  // namespace

namespace pa {
pa_status record_error(pa_status s, const char *msg) {
  g_last_error = msg;
  return s;
}
void clear_error() { g_last_error.clear(); }
}  // namespace pa

namespace {

bool aligned(const void *p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int kind_of(pa_dtype t) {
  switch (t) {
    case PA_DTYPE_F32: return pa::KV_F32;
    case PA_DTYPE_BF16: return pa::KV_BF16;
    default: return pa::KV_FP8;
  }
}

// MI355X: 256 compute units in 8 XCDs.  The launch shape (and so the
// workspace size) depends only on the arguments, never on a runtime query.
constexpr int64_t kComputeUnits = 256;
// Most workgroups a caller may ask for.
constexpr int32_t kMaxWorkgroups = 1 << 16;

// Largest head chunk a workgroup may take: a power of two dividing both
// num_kv_heads and kWaves (each wave works on one head of the chunk).
int32_t max_heads_per_workgroup(int32_t hkv) {
  int32_t hc = 1;
  while (hc * 2 <= pa::kWaves && hkv % (hc * 2) == 0) hc *= 2;
  return hc;
}

// Upper bound of the work units (16-token blocks of one (sequence, head
// chunk)) for head chunk hc, from the host-side bound of the lengths.
int64_t max_units(const pa_kv_pool *p, int32_t hc) {
  const int64_t blocks = (p->max_context_len + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE;
  return (int64_t)p->batch * (p->num_kv_heads / hc) * blocks;
}

// KV heads per workgroup.  Automatic choice: the largest chunk for which the
// (sequence, chunk) pairs still number at least one per compute unit, so
// that when the contexts are of equal length every workgroup's range is one
// whole pair (no partial results); wider chunks read longer contiguous runs
// of each block.  When even single heads are too few, pairs are split
// anyway, and then the widest chunk is best.
int32_t heads_per_workgroup(const pa_kv_pool *p) {
  if (p->heads_override > 0) return p->heads_override;
  const int32_t hmax = max_heads_per_workgroup(p->num_kv_heads);
  for (int32_t hc = hmax; hc >= 1; hc /= 2)
    if ((int64_t)p->batch * (p->num_kv_heads / hc) >= kComputeUnits) return hc;
  return hmax;
}

// Workgroups: one per compute unit (fewer if there are fewer units of work).
int32_t workgroups(const pa_kv_pool *p) {
  if (p->workgroups_override > 0) return p->workgroups_override;
  const int64_t u = max_units(p, heads_per_workgroup(p));
  return (int32_t)std::max<int64_t>(1, std::min<int64_t>(kComputeUnits, u));
}

// KV heads per workgroup when the sequences' block counts differ (the kernel
// sees the lengths, the host does not): the widest chunk, unless the caller
// fixed the chunk.  With lengths that differ, ranges cut across (sequence,
// chunk) pairs whatever the chunk, and fewer, longer pieces win: batch 32,
// 8 KV heads, lengths uniform in [128, 8192]: 134 us at 1 head per
// workgroup, 108 us at 4; the 64-sequence mix of up to 16K tokens: 331 us
// at 2, 321 us at 4.
int32_t heads_per_workgroup_varied(const pa_kv_pool *p) {
  if (p->heads_override > 0) return p->heads_override;
  return max_heads_per_workgroup(p->num_kv_heads);
}

struct Layout {
  int32_t nwg, hc, chunks, hc_var;
  size_t ml_offset, acc_offset, total;
};

// Workspace, when a run may split pairs (more than one workgroup):
//   [0, PA_DECODE_COUNTER_BYTES)  arrival counters, uint32 per workgroup
//                                 (at most kMaxWorkgroups of them), zero
//                                 before and after every run;
//   then float2 ml[nwg][2][hcg]   (max, sum) of the two partial records of
//                                 each workgroup (the pieces its range
//                                 starts and ends with), and at a 256-byte
//                                 boundary float acc[nwg][2][hcg][d], for
//                                 hcg = query heads of the wider head chunk.
// The counter region has a fixed size and place whatever the launch shape,
// so one workspace, cleared once, serves runs of any shape.
Layout workspace_layout(const pa_kv_pool *p, int32_t hq) {
  static_assert(PA_DECODE_COUNTER_BYTES == 4 * kMaxWorkgroups, "one counter per workgroup");
  Layout L{};
  L.hc = heads_per_workgroup(p);
  L.chunks = p->num_kv_heads / L.hc;
  L.hc_var = heads_per_workgroup_varied(p);
  L.nwg = workgroups(p);
  const int32_t hcg = std::max(L.hc, L.hc_var) * (hq / p->num_kv_heads);
  // one workgroup never splits a (sequence, chunk): no partials to keep
  const size_t recs = L.nwg > 1 ? (size_t)L.nwg * 2 * hcg : 0;
  L.ml_offset = PA_DECODE_COUNTER_BYTES;
  L.acc_offset = (L.ml_offset + recs * sizeof(float2) + 255) & ~(size_t)255;
  L.total = recs ? L.acc_offset + recs * p->head_dim * sizeof(float) : 0;
  return L;
}

// Where a run's workspace comes from: the caller's buffer, or the library's
// static device scratch (pa_decode_run_noalloc).
enum class Scratch { kCaller, kStatic };

pa_status run(pa_kv_pool *pool, const void *q, pa_dtype q_dtype, int32_t hq, float scale,
              float *out, void *workspace, size_t ws_bytes, void *stream, bool fp8_entry,
              Scratch from = Scratch::kCaller) {
  if (!pool) return fail(PA_ERR_NULL, "pool is NULL");
  if (pool->kivi_bits) return fail(PA_ERR_DTYPE, "an INT8/INT4 pool must be run with pa_decode_kivi_run");
  const bool fp8_pool = pool->kv_dtype == PA_DTYPE_FP8_E4M3;
  if (fp8_entry && !fp8_pool)
    return fail(PA_ERR_DTYPE, "pa_decode_fp8_run needs an FP8 E4M3 pool");
  if (!fp8_entry && fp8_pool)
    return fail(PA_ERR_DTYPE, "an FP8 pool must be run with pa_decode_fp8_run");
  if (!pool->table_set) return fail(PA_ERR_STATE, "no block table set (pa_block_table_set)");
  const pa_dtype want_q = pool->kv_dtype == PA_DTYPE_F32 ? PA_DTYPE_F32 : PA_DTYPE_BF16;
  if (q_dtype != want_q)
    return fail(PA_ERR_DTYPE, "q dtype %d does not match the pool (needs %d)", (int)q_dtype,
                (int)want_q);
  if (hq < 1 || hq % pool->num_kv_heads)
    return fail(PA_ERR_SHAPE, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                hq, pool->num_kv_heads);
  const int group = hq / pool->num_kv_heads;
  if (!pa::kernel_supported(kind_of(pool->kv_dtype), pool->head_dim, group))
    return fail(PA_ERR_UNSUPPORTED, "group size %d not built (1, 2, 4 or 8)", group);
  if (!(std::isfinite(scale)))
    return fail(PA_ERR_SHAPE, "scale must be finite");
  if (pool->batch > 0 && (!q || !out)) return fail(PA_ERR_NULL, "q or out is NULL");
  const Layout L = workspace_layout(pool, hq);
  if (from == Scratch::kStatic) {
    if (L.total > pa::kStaticScratchBytes)
      return fail(PA_ERR_WORKSPACE,
                  "this launch needs %zu bytes of workspace, the static scratch holds %zu "
                  "(fewer workgroups, or pa_decode_run with a workspace)",
                  L.total, pa::kStaticScratchBytes);
  } else if (L.total > 0) {
    if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", L.total);
    if (ws_bytes < L.total)
      return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, L.total);
    if (!aligned(workspace, 256)) return fail(PA_ERR_WORKSPACE, "workspace not 256-byte aligned");
  }
  if ((size_t)pool->batch * hq >= (size_t(1) << 31))
    return fail(PA_ERR_SHAPE, "batch * num_q_heads too large");
  // the kernel counts its work (16-token blocks of one (sequence, head
  // chunk)) in 32-bit integers, with headroom for its range arithmetic
  if (max_units(pool, 1) >= (int64_t(1) << 30))
    return fail(PA_ERR_SHAPE, "batch * num_kv_heads * ceil(max_context_len / 16) must be below 2^30");
  if (pool->batch == 0) return ok();

  // ---- from here on HIP is used (launches only: no allocation, no wait)
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  char *ws = static_cast<char *>(workspace);
  if (from == Scratch::kStatic && L.total > 0) {
    void *p = nullptr;
    if ((e = pa::static_scratch(&p)) != hipSuccess)
      return fail(PA_ERR_HIP, "static scratch: %s", hipGetErrorString(e));
    // the counters this launch uses must start at zero: runs leave them
    // zero, but the scratch is shared by every call on this GPU, so clear
    // them anyway (a kernel, not a memset, so a captured graph replays it)
    if ((e = pa::launch_zero(static_cast<uint32_t *>(p), (size_t)L.nwg, s)) != hipSuccess)
      return fail(PA_ERR_HIP, "clearing the static scratch: %s", hipGetErrorString(e));
    ws = static_cast<char *>(p);
  }
  pa::LaunchArgs a{};
  a.k_cache = pool->k_cache;
  a.v_cache = pool->v_cache;
  a.k_scale = pool->k_scale;
  a.v_scale = pool->v_scale;
  a.q = q;
  a.table = pool->block_table;
  a.ctx = pool->context_lens;
  a.out = out;
  a.counters = L.total ? reinterpret_cast<uint32_t *>(ws) : nullptr;
  a.ws_ml = L.total ? reinterpret_cast<float2 *>(ws + L.ml_offset) : nullptr;
  a.ws_acc = L.total ? reinterpret_cast<float *>(ws + L.acc_offset) : nullptr;
  a.num_blocks = pool->num_blocks;
  a.hkv = pool->num_kv_heads;
  a.hq = hq;
  a.d = pool->head_dim;
  a.batch = pool->batch;
  a.max_blocks = pool->max_blocks_per_seq;
  a.max_ctx = pool->max_context_len;
  a.nwg = L.nwg;
  a.hc = L.hc;
  a.chunks = L.chunks;
  a.hc_var = L.hc_var;
  a.scale_log2e = (float)((double)scale * 1.4426950408889634);
  a.kv = kind_of(pool->kv_dtype);

  const bool prof = pool->prof_capacity > 0 && pool->prof_count < pool->prof_capacity;
  hipEvent_t *ev = prof ? &pool->prof_events[2 * (size_t)pool->prof_count] : nullptr;
  // profiling: the events are attached to the kernel's dispatch, so they
  // time its own execution (not the queue's markers around it)
  if ((e = pa::launch_attention(a, s, prof ? ev[0] : nullptr, prof ? ev[1] : nullptr)) != hipSuccess)
    return fail(PA_ERR_HIP, "attention kernel launch: %s", hipGetErrorString(e));
  if (prof) ++pool->prof_count;
  return ok();
}

pa::KiviArgs kivi_args(const pa_kv_pool *p, const void *q, int32_t hq, float scale, float *out) {
  pa::KiviArgs a{};
  a.k_codes = p->k_cache;
  a.v_codes = p->v_cache;
  a.k_par = p->k_par;
  a.v_par = p->v_par;
  a.res_k = p->res_k;
  a.res_v = p->res_v;
  a.q = q;
  a.table = p->block_table;
  a.ctx = p->context_lens;
  a.out = out;
  a.num_blocks = p->num_blocks;
  a.hkv = p->num_kv_heads;
  a.hq = hq;
  a.d = p->head_dim;
  a.batch = p->batch;
  a.max_blocks = p->max_blocks_per_seq;
  a.max_ctx = p->max_context_len;
  a.bits = p->kivi_bits;
  a.scale_log2e = (float)((double)scale * 1.4426950408889634);
  return a;
}

void release_events(pa_kv_pool *p) {
  for (hipEvent_t e : p->prof_events) (void)hipEventDestroy(e);
  p->prof_events.clear();
  p->prof_capacity = 0;
  p->prof_count = 0;
}

}  // namespace

extern "C" {

pa_status pa_kv_pool_create(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                            int32_t head_dim, pa_dtype kv_dtype, void *k_cache, void *v_cache,
                            float *k_scale, float *v_scale, pa_kv_pool **out_pool) {
  if (!out_pool) return fail(PA_ERR_NULL, "out_pool is NULL");
  *out_pool = nullptr;
  if (!k_cache || !v_cache) return fail(PA_ERR_NULL, "k_cache or v_cache is NULL");
  if (kv_dtype == PA_DTYPE_INT8_KIVI || kv_dtype == PA_DTYPE_INT4_KIVI)
    return fail(PA_ERR_DTYPE, "INT8/INT4 pools are created with pa_kv_pool_create_kivi");
  if (kv_dtype != PA_DTYPE_F32 && kv_dtype != PA_DTYPE_BF16 && kv_dtype != PA_DTYPE_FP8_E4M3)
    return fail(PA_ERR_DTYPE, "unknown kv dtype %d", (int)kv_dtype);
  const bool fp8 = kv_dtype == PA_DTYPE_FP8_E4M3;
  if (fp8 && (!k_scale || !v_scale))
    return fail(PA_ERR_NULL, "an FP8 pool needs k_scale and v_scale");
  if (!fp8 && (k_scale || v_scale))
    return fail(PA_ERR_DTYPE, "scales are only meaningful for an FP8 pool");
  if (block_size != PA_BLOCK_SIZE)
    return fail(PA_ERR_SHAPE, "block_size %d: only %d is supported", block_size, PA_BLOCK_SIZE);
  if (num_blocks < 1 || num_kv_heads < 1 || head_dim < 1)
    return fail(PA_ERR_SHAPE, "num_blocks, num_kv_heads and head_dim must be positive");
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", head_dim);
  if ((int64_t)num_kv_heads * head_dim * 4 * PA_BLOCK_SIZE > (int64_t)1 << 30)
    return fail(PA_ERR_SHAPE, "num_kv_heads too large");
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(PA_ERR_SHAPE, "k_cache and v_cache must be 16-byte aligned");
  if (fp8 && (!aligned(k_scale, 4) || !aligned(v_scale, 4)))
    return fail(PA_ERR_SHAPE, "scales must be 4-byte aligned");
  pa_kv_pool *p = new (std::nothrow) pa_kv_pool();
  if (!p) return fail(PA_ERR_SHAPE, "out of host memory");
  p->num_blocks = num_blocks;
  p->num_kv_heads = num_kv_heads;
  p->head_dim = head_dim;
  p->kv_dtype = kv_dtype;
  p->k_cache = k_cache;
  p->v_cache = v_cache;
  p->k_scale = k_scale;
  p->v_scale = v_scale;
  *out_pool = p;
  return ok();
}

pa_status pa_kv_pool_placement(int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                               pa_dtype kv_dtype, size_t *pool_bytes, size_t *v_offset,
                               size_t *total_bytes) {
  if (!pool_bytes || !v_offset || !total_bytes)
    return fail(PA_ERR_NULL, "pool_bytes, v_offset or total_bytes is NULL");
  int64_t eb = 0;
  switch (kv_dtype) {
    case PA_DTYPE_F32: eb = 4; break;
    case PA_DTYPE_BF16: eb = 2; break;
    case PA_DTYPE_FP8_E4M3: eb = 1; break;
    default: return fail(PA_ERR_DTYPE, "placement is for f32, bf16 and FP8 pools");
  }
  if (num_blocks < 1 || num_kv_heads < 1 || head_dim < 1)
    return fail(PA_ERR_SHAPE, "num_blocks, num_kv_heads and head_dim must be positive");
  const int64_t row = (int64_t)num_kv_heads * head_dim * eb * PA_BLOCK_SIZE;
  if (row > ((int64_t)1 << 30) || (int64_t)num_blocks > (((int64_t)1 << 46) / row))
    return fail(PA_ERR_SHAPE, "pool too large");
  // 2 KiB period of the address classes, shifted by 256 B (see pa.h)
  constexpr int64_t kPeriod = 2048, kShift = 256;
  const int64_t bytes = row * num_blocks;
  const int64_t voff = (bytes + kPeriod - 1) / kPeriod * kPeriod + kShift;
  *pool_bytes = (size_t)bytes;
  *v_offset = (size_t)voff;
  *total_bytes = (size_t)(voff + bytes);
  return ok();
}

void pa_kv_pool_destroy(pa_kv_pool *pool) {
  if (!pool) return;
  release_events(pool);
  delete pool;
}

pa_status pa_block_table_set(pa_kv_pool *pool, const int32_t *block_table,
                             const int32_t *context_lens, int32_t batch,
                             int32_t max_blocks_per_seq, int32_t max_context_len) {
  if (!pool) return fail(PA_ERR_NULL, "pool is NULL");
  if (batch < 0) return fail(PA_ERR_SHAPE, "batch %d < 0", batch);
  if (batch > 0 && (!block_table || !context_lens))
    return fail(PA_ERR_NULL, "block_table or context_lens is NULL");
  if (max_blocks_per_seq < 1) return fail(PA_ERR_SHAPE, "max_blocks_per_seq must be >= 1");
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * PA_BLOCK_SIZE)
    return fail(PA_ERR_SHAPE, "max_context_len %d outside [0, 16 * max_blocks_per_seq = %lld]",
                max_context_len, (long long)max_blocks_per_seq * PA_BLOCK_SIZE);
  if ((int64_t)batch * max_blocks_per_seq >= ((int64_t)1 << 31))
    return fail(PA_ERR_SHAPE, "block table too large");
  pool->block_table = block_table;
  pool->context_lens = context_lens;
  pool->batch = batch;
  pool->max_blocks_per_seq = max_blocks_per_seq;
  pool->max_context_len = max_context_len;
  pool->table_set = true;
  return ok();
}

pa_status pa_block_table_validate(pa_kv_pool *pool, void *stream) {
  if (!pool) return fail(PA_ERR_NULL, "pool is NULL");
  if (!pool->table_set) return fail(PA_ERR_STATE, "no block table set");
  if (pool->batch == 0) return ok();
  const size_t nt = (size_t)pool->batch * pool->max_blocks_per_seq;
  std::vector<int32_t> table(nt), ctx(pool->batch);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if ((e = hipMemcpyAsync(table.data(), pool->block_table, nt * 4, hipMemcpyDeviceToHost, s)) != hipSuccess ||
      (e = hipMemcpyAsync(ctx.data(), pool->context_lens, ctx.size() * 4, hipMemcpyDeviceToHost, s)) != hipSuccess ||
      (e = hipStreamSynchronize(s)) != hipSuccess)
    return fail(PA_ERR_HIP, "reading the tables: %s", hipGetErrorString(e));
  for (int32_t b = 0; b < pool->batch; ++b) {
    const int32_t n = ctx[b];
    if (n < 0 || n > pool->max_context_len)
      return fail(PA_ERR_SHAPE, "context_lens[%d] = %d outside [0, %d]", b, n, pool->max_context_len);
    const int32_t nb = (n + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE;
    for (int32_t j = 0; j < nb; ++j) {
      const int32_t id = table[(size_t)b * pool->max_blocks_per_seq + j];
      if (id < 0 || id >= pool->num_blocks)
        return fail(PA_ERR_SHAPE, "block_table[%d][%d] = %d outside [0, %d)", b, j, id,
                    pool->num_blocks);
    }
  }
  return ok();
}

pa_status pa_decode_workspace_bytes(const pa_kv_pool *pool, int32_t num_q_heads, size_t *bytes) {
  if (!pool || !bytes) return fail(PA_ERR_NULL, "pool or bytes is NULL");
  if (!pool->table_set) return fail(PA_ERR_STATE, "no block table set");
  if (num_q_heads < 1 || num_q_heads % pool->num_kv_heads)
    return fail(PA_ERR_SHAPE, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, pool->num_kv_heads);
  *bytes = workspace_layout(pool, num_q_heads).total;
  return ok();
}

pa_status pa_decode_workspace_clear(void *workspace, size_t workspace_bytes, void *stream) {
  if (workspace_bytes == 0) return ok();
  if (!workspace) return fail(PA_ERR_NULL, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(PA_ERR_WORKSPACE, "workspace not 256-byte aligned");
  const size_t words = std::min<size_t>(workspace_bytes, PA_DECODE_COUNTER_BYTES) / 4;
  const hipError_t e =
      pa::launch_zero(static_cast<uint32_t *>(workspace), words, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "clearing the workspace: %s", hipGetErrorString(e));
  return ok();
}

pa_status pa_decode_run(pa_kv_pool *pool, const void *q, pa_dtype q_dtype, int32_t num_q_heads,
                        float scale, float *out, void *workspace, size_t workspace_bytes,
                        void *stream) {
  return run(pool, q, q_dtype, num_q_heads, scale, out, workspace, workspace_bytes, stream, false);
}

pa_status pa_decode_fp8_run(pa_kv_pool *pool, const void *q, pa_dtype q_dtype,
                            int32_t num_q_heads, float scale, float *out, void *workspace,
                            size_t workspace_bytes, void *stream) {
  return run(pool, q, q_dtype, num_q_heads, scale, out, workspace, workspace_bytes, stream, true);
}

pa_status pa_decode_run_noalloc(pa_kv_pool *pool, const void *q, pa_dtype q_dtype,
                                int32_t num_q_heads, float scale, float *out, void *stream) {
  if (!pool) return fail(PA_ERR_NULL, "pool is NULL");
  return run(pool, q, q_dtype, num_q_heads, scale, out, nullptr, 0, stream,
             pool->kv_dtype == PA_DTYPE_FP8_E4M3, Scratch::kStatic);
}

pa_status pa_cache_append(pa_kv_pool *pool, const void *k_new, const void *v_new,
                          pa_dtype src_dtype, void *stream) {
  if (!pool) return fail(PA_ERR_NULL, "pool is NULL");
  if (!pool->table_set) return fail(PA_ERR_STATE, "no block table set (pa_block_table_set)");
  if (pool->kivi_bits) {
    if (src_dtype != PA_DTYPE_BF16)
      return fail(PA_ERR_DTYPE, "an INT8/INT4 pool takes bf16 new rows");
    if (pool->batch == 0) return ok();
    if (!k_new || !v_new) return fail(PA_ERR_NULL, "k_new or v_new is NULL");
    if (!pool->res_k || !pool->res_v)
      return fail(PA_ERR_STATE, "no residual set (pa_kivi_residual_set)");
    if (!aligned(k_new, 4) || !aligned(v_new, 4))
      return fail(PA_ERR_SHAPE, "k_new and v_new must be 4-byte aligned");
    const pa::KiviArgs a = kivi_args(pool, nullptr, 0, 0.f, nullptr);
    const hipError_t e = pa::launch_kivi_append(a, k_new, v_new, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "cache-write kernel launch: %s", hipGetErrorString(e));
    return ok();
  }
  const bool fp8 = pool->kv_dtype == PA_DTYPE_FP8_E4M3;
  if (fp8 ? (src_dtype != PA_DTYPE_F32 && src_dtype != PA_DTYPE_BF16)
          : src_dtype != pool->kv_dtype)
    return fail(PA_ERR_DTYPE, "new K/V dtype %d cannot be written to a pool of dtype %d",
                (int)src_dtype, (int)pool->kv_dtype);
  if (pool->batch == 0) return ok();
  if (!k_new || !v_new) return fail(PA_ERR_NULL, "k_new or v_new is NULL");
  if ((size_t)pool->batch * pool->num_kv_heads >= (size_t(1) << 31))
    return fail(PA_ERR_SHAPE, "batch * num_kv_heads too large");
  pa::AppendArgs a{};
  a.k_cache = pool->k_cache;
  a.v_cache = pool->v_cache;
  a.k_scale = pool->k_scale;
  a.v_scale = pool->v_scale;
  a.k_new = k_new;
  a.v_new = v_new;
  a.table = pool->block_table;
  a.ctx = pool->context_lens;
  a.num_blocks = pool->num_blocks;
  a.hkv = pool->num_kv_heads;
  a.d = pool->head_dim;
  a.batch = pool->batch;
  a.max_blocks = pool->max_blocks_per_seq;
  a.max_ctx = pool->max_context_len;
  a.kv = kind_of(pool->kv_dtype);
  a.src = kind_of(src_dtype);
  const hipError_t e = pa::launch_append(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "cache-write kernel launch: %s", hipGetErrorString(e));
  return ok();
}

pa_status pa_kv_pool_create_kivi(int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                                 pa_dtype kv_dtype, void *k_codes, void *v_codes, void *k_params,
                                 void *v_params, pa_kv_pool **out_pool) {
  if (!out_pool) return fail(PA_ERR_NULL, "out_pool is NULL");
  *out_pool = nullptr;
  if (kv_dtype != PA_DTYPE_INT8_KIVI && kv_dtype != PA_DTYPE_INT4_KIVI)
    return fail(PA_ERR_DTYPE, "kv dtype %d is not INT8 or INT4", (int)kv_dtype);
  if (!k_codes || !v_codes || !k_params || !v_params)
    return fail(PA_ERR_NULL, "codes or parameters are NULL");
  if (num_blocks < 1 || num_kv_heads < 1)
    return fail(PA_ERR_SHAPE, "num_blocks and num_kv_heads must be positive");
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", head_dim);
  if ((int64_t)num_kv_heads * head_dim * 4 * PA_BLOCK_SIZE > (int64_t)1 << 30)
    return fail(PA_ERR_SHAPE, "num_kv_heads too large");
  if (!aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(k_params, 16) ||
      !aligned(v_params, 16))
    return fail(PA_ERR_SHAPE, "codes and parameters must be 16-byte aligned");
  pa_kv_pool *p = new (std::nothrow) pa_kv_pool();
  if (!p) return fail(PA_ERR_SHAPE, "out of host memory");
  p->num_blocks = num_blocks;
  p->num_kv_heads = num_kv_heads;
  p->head_dim = head_dim;
  p->kv_dtype = kv_dtype;
  p->kivi_bits = kv_dtype == PA_DTYPE_INT8_KIVI ? 8 : 4;
  p->k_cache = k_codes;
  p->v_cache = v_codes;
  p->k_par = k_params;
  p->v_par = v_params;
  *out_pool = p;
  return ok();
}

pa_status pa_kivi_residual_set(pa_kv_pool *pool, void *res_k, void *res_v) {
  if (!pool) return fail(PA_ERR_NULL, "pool is NULL");
  if (!pool->kivi_bits) return fail(PA_ERR_DTYPE, "only INT8/INT4 pools have a residual");
  if ((res_k == nullptr) != (res_v == nullptr))
    return fail(PA_ERR_NULL, "res_k and res_v must both be set or both be NULL");
  if (res_k && (!aligned(res_k, 16) || !aligned(res_v, 16)))
    return fail(PA_ERR_SHAPE, "the residual must be 16-byte aligned");
  pool->res_k = res_k;
  pool->res_v = res_v;
  return ok();
}

pa_status pa_decode_kivi_run(pa_kv_pool *pool, const void *q, pa_dtype q_dtype,
                             int32_t num_q_heads, float scale, float *out, void *stream) {
  if (!pool) return fail(PA_ERR_NULL, "pool is NULL");
  if (!pool->kivi_bits) return fail(PA_ERR_DTYPE, "pa_decode_kivi_run needs an INT8/INT4 pool");
  if (!pool->table_set) return fail(PA_ERR_STATE, "no block table set (pa_block_table_set)");
  if (q_dtype != PA_DTYPE_BF16) return fail(PA_ERR_DTYPE, "INT8/INT4 decode needs bf16 q");
  if (num_q_heads < 1 || num_q_heads % pool->num_kv_heads)
    return fail(PA_ERR_SHAPE, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, pool->num_kv_heads);
  const int group = num_q_heads / pool->num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(PA_ERR_UNSUPPORTED, "group size %d not built (1, 2, 4 or 8)", group);
  if (!std::isfinite(scale)) return fail(PA_ERR_SHAPE, "scale must be finite");
  if (pool->batch == 0) return ok();
  if (!q || !out) return fail(PA_ERR_NULL, "q or out is NULL");
  if (!pool->res_k) return fail(PA_ERR_STATE, "no residual set (pa_kivi_residual_set)");
  if (!aligned(q, 16)) return fail(PA_ERR_SHAPE, "q must be 16-byte aligned");
  if (!aligned(out, 4)) return fail(PA_ERR_SHAPE, "out must be 4-byte aligned");
  if ((size_t)pool->batch * pool->num_kv_heads >= (size_t(1) << 31))
    return fail(PA_ERR_SHAPE, "batch * num_kv_heads too large");
  const pa::KiviArgs a = kivi_args(pool, q, num_q_heads, scale, out);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  const bool prof = pool->prof_capacity > 0 && pool->prof_count < pool->prof_capacity;
  hipEvent_t *ev = prof ? &pool->prof_events[2 * (size_t)pool->prof_count] : nullptr;
  if ((e = pa::launch_kivi_attention(a, s, prof ? ev[0] : nullptr, prof ? ev[1] : nullptr)) !=
      hipSuccess)
    return fail(PA_ERR_HIP, "INT8/INT4 attention kernel launch: %s", hipGetErrorString(e));
  if (prof) ++pool->prof_count;
  return ok();
}

pa_status pa_copy_blocks(pa_kv_pool *pool, const int32_t *pairs, int32_t n, void *stream) {
  if (!pool) return fail(PA_ERR_NULL, "pool is NULL");
  if (n < 0) return fail(PA_ERR_SHAPE, "n %d < 0", n);
  if (n == 0) return ok();
  if (!pairs) return fail(PA_ERR_NULL, "pairs is NULL");
  const int eb = pool->kv_dtype == PA_DTYPE_F32 ? 4 : (pool->kv_dtype == PA_DTYPE_BF16 ? 2 : 1);
  pa::CopyArgs a{};
  a.k_cache = pool->k_cache;
  a.v_cache = pool->v_cache;
  a.pairs = pairs;
  a.n = n;
  a.num_blocks = pool->num_blocks;
  a.block_bytes = (int64_t)PA_BLOCK_SIZE * pool->num_kv_heads * pool->head_dim * eb;
  if (pool->kv_dtype == PA_DTYPE_FP8_E4M3) {
    a.k_par = pool->k_scale;
    a.v_par = pool->v_scale;
    a.k_par_words = a.v_par_words = pool->num_kv_heads * PA_BLOCK_SIZE;
  } else if (pool->kivi_bits) {
    a.block_bytes = (int64_t)PA_BLOCK_SIZE * pool->num_kv_heads * pool->head_dim * pool->kivi_bits / 8;
    a.k_par = pool->k_par;
    a.v_par = pool->v_par;
    a.k_par_words = pool->num_kv_heads * pool->head_dim;  // 2 * d fp16 per head
    a.v_par_words = pool->num_kv_heads * PA_BLOCK_SIZE;   // (scale, min) per slot
  }
  const hipError_t e = pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "block copy launch: %s", hipGetErrorString(e));
  return ok();
}

pa_status pa_chunk_tiles(const pa_kv_pool *pool, int32_t num_q_heads, int32_t max_q_len,
                         int32_t *rows_per_workgroup, int32_t *workgroups_per_head) {
  if (!pool || !rows_per_workgroup || !workgroups_per_head)
    return fail(PA_ERR_NULL, "pool or an output is NULL");
  if (num_q_heads < 1 || num_q_heads % pool->num_kv_heads)
    return fail(PA_ERR_SHAPE, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, pool->num_kv_heads);
  if (max_q_len < 0) return fail(PA_ERR_SHAPE, "max_q_len %d < 0", max_q_len);
  const int group = num_q_heads / pool->num_kv_heads;
  const int nqt = pa::chunk_tiles_per_item(max_q_len, group, pool->head_dim);
  *rows_per_workgroup = 16 * nqt;
  *workgroups_per_head = pa::chunk_items_per_head(max_q_len, group, nqt);
  return ok();
}

pa_status pa_chunk_run(pa_kv_pool *pool, const void *q, pa_dtype q_dtype, int32_t num_q_heads,
                       const int32_t *q_start, int32_t total_q, int32_t max_q_len, float scale,
                       float *out, void *stream) {
  if (!pool) return fail(PA_ERR_NULL, "pool is NULL");
  if (!pool->table_set) return fail(PA_ERR_STATE, "no block table set (pa_block_table_set)");
  if (pool->kivi_bits || (pool->kv_dtype != PA_DTYPE_BF16 && pool->kv_dtype != PA_DTYPE_FP8_E4M3))
    return fail(PA_ERR_UNSUPPORTED, "chunk attention is built for bf16 and FP8 pools");
  if (q_dtype != PA_DTYPE_BF16) return fail(PA_ERR_DTYPE, "chunk attention needs bf16 q");
  if (num_q_heads < 1 || num_q_heads % pool->num_kv_heads)
    return fail(PA_ERR_SHAPE, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, pool->num_kv_heads);
  const int group = num_q_heads / pool->num_kv_heads;
  if (!pa::chunk_supported(kind_of(pool->kv_dtype), pool->head_dim, group))
    return fail(PA_ERR_UNSUPPORTED, "group size %d not built (1, 2, 4 or 8)", group);
  if (!std::isfinite(scale)) return fail(PA_ERR_SHAPE, "scale must be finite");
  if (total_q < 0 || max_q_len < 0)
    return fail(PA_ERR_SHAPE, "total_q %d and max_q_len %d must be >= 0", total_q, max_q_len);
  if (pool->batch == 0 || total_q == 0 || max_q_len == 0) return ok();
  if (!q || !out || !q_start) return fail(PA_ERR_NULL, "q, out or q_start is NULL");
  if (!aligned(q, 16)) return fail(PA_ERR_SHAPE, "q must be 16-byte aligned");
  if (!aligned(out, 4)) return fail(PA_ERR_SHAPE, "out must be 4-byte aligned");
  const int nqt = pa::chunk_tiles_per_item(max_q_len, group, pool->head_dim);
  const int tiles = pa::chunk_items_per_head(max_q_len, group, nqt);
  if ((int64_t)pool->batch * pool->num_kv_heads * tiles > (int64_t)0x7FFFFFFF)
    return fail(PA_ERR_SHAPE, "too many workgroups (batch * num_kv_heads * tiles)");
  pa::ChunkArgs a{};
  a.k_cache = pool->k_cache;
  a.v_cache = pool->v_cache;
  a.k_scale = pool->k_scale;
  a.v_scale = pool->v_scale;
  a.kv = kind_of(pool->kv_dtype);
  a.q = q;
  a.table = pool->block_table;
  a.ctx = pool->context_lens;
  a.q_start = q_start;
  a.out = out;
  a.num_blocks = pool->num_blocks;
  a.hkv = pool->num_kv_heads;
  a.hq = num_q_heads;
  a.d = pool->head_dim;
  a.batch = pool->batch;
  a.max_blocks = pool->max_blocks_per_seq;
  a.max_ctx = pool->max_context_len;
  a.max_q = max_q_len;
  a.total_q = total_q;
  a.nqt = nqt;
  a.tiles = tiles;
  a.scale_log2e = (float)((double)scale * 1.4426950408889634);
  const hipError_t e = pa::launch_chunk(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "chunk kernel launch: %s", hipGetErrorString(e));
  return ok();
}

pa_status pa_decode_set_workgroups(pa_kv_pool *pool, int32_t count) {
  if (!pool) return fail(PA_ERR_NULL, "pool is NULL");
  if (count < 0 || count > kMaxWorkgroups)
    return fail(PA_ERR_SHAPE, "workgroups %d: 0 or in [1, %d]", count, kMaxWorkgroups);
  pool->workgroups_override = count;
  return ok();
}

pa_status pa_decode_workgroups(const pa_kv_pool *pool, int32_t *count) {
  if (!pool || !count) return fail(PA_ERR_NULL, "pool or count is NULL");
  if (!pool->table_set) return fail(PA_ERR_STATE, "no block table set");
  *count = workgroups(pool);
  return ok();
}

pa_status pa_decode_set_heads_per_workgroup(pa_kv_pool *pool, int32_t heads) {
  if (!pool) return fail(PA_ERR_NULL, "pool is NULL");
  const int32_t hmax = max_heads_per_workgroup(pool->num_kv_heads);
  if (heads != 0 && (heads < 1 || heads > hmax || (heads & (heads - 1))))
    return fail(PA_ERR_SHAPE, "heads per workgroup %d: 0 or a power of two dividing %d, at most %d",
                heads, pool->num_kv_heads, hmax);
  pool->heads_override = heads;
  return ok();
}

pa_status pa_decode_heads_per_workgroup(const pa_kv_pool *pool, int32_t *heads) {
  if (!pool || !heads) return fail(PA_ERR_NULL, "pool or heads is NULL");
  if (!pool->table_set) return fail(PA_ERR_STATE, "no block table set");
  *heads = heads_per_workgroup(pool);
  return ok();
}

pa_status pa_profile_enable(pa_kv_pool *pool, int32_t capacity) {
  if (!pool) return fail(PA_ERR_NULL, "pool is NULL");
  if (capacity < 0) return fail(PA_ERR_SHAPE, "capacity %d < 0", capacity);
  release_events(pool);
  if (capacity == 0) return ok();
  pool->prof_events.resize(2 * (size_t)capacity);
  for (auto &e : pool->prof_events) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      e = nullptr;
      release_events(pool);
      return fail(PA_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(r));
    }
  }
  pool->prof_capacity = capacity;
  return ok();
}

pa_status pa_profile_read(pa_kv_pool *pool, float *kernel_ms, int32_t capacity, int32_t *count) {
  if (!pool || !count) return fail(PA_ERR_NULL, "pool or count is NULL");
  if (pool->prof_capacity == 0) return fail(PA_ERR_STATE, "profiling not enabled");
  const int32_t n = pool->prof_count;
  *count = n;
  if (n > 0) {
    hipError_t e = hipEventSynchronize(pool->prof_events[2 * (size_t)n - 1]);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(e));
  }
  for (int32_t i = 0; i < n && i < capacity; ++i) {
    float t = 0.f;
    hipError_t e = hipEventElapsedTime(&t, pool->prof_events[2 * (size_t)i],
                                       pool->prof_events[2 * (size_t)i + 1]);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "hipEventElapsedTime: %s", hipGetErrorString(e));
    if (kernel_ms) kernel_ms[i] = t;
  }
  pool->prof_count = 0;
  return ok();
}

const char *pa_status_str(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "null pointer";
    case PA_ERR_SHAPE: return "bad shape or size";
    case PA_ERR_DTYPE: return "bad dtype";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_STATE: return "bad state";
    case PA_ERR_WORKSPACE: return "bad workspace";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_NO_BLOCKS: return "no free block";
    case PA_ERR_SEQUENCE: return "unknown or duplicate sequence";
  }
  return "unknown status";
}

const char *pa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
