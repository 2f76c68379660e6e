/*
 * pa.h -- single-token decode attention over a paged KV cache (C ABI).
 *
 * Operation.  For every sequence b and query head h of one decode step:
 *
 *     out[b][h][:] = softmax_t( scale * q[b][h][:] . K_b[t][g][:] ) V_b[t][g][:]
 *
 * over the sequence's cached tokens t = 0 .. context_lens[b]-1, where
 * g = h / (num_q_heads / num_kv_heads) is the KV head of h's group and token
 * t lives in physical block block_table[b][t / 16] at slot t % 16.
 *
 * Sources (page title and section):
 *   - attention softmax(Q K^T / sqrt(d)) V and the decode step that reuses
 *     every cached K/V of the sequence, the new token's own included:
 *     "KV Cache 深度解析:显存黑洞、PagedAttention 与三路省内存方案" (d7kj.com),
 *     sections 一 and 六;
 *   - fixed 16-token blocks and a per-sequence logical->physical block
 *     table, with blocks free to be shared between sequences: same page,
 *     section 三 (PagedAttention);
 *   - in-block layout [block_size][heads][head_dim], K and V stored apart:
 *     LLM inference-optimization notes (qingdujian.com), section 二;
 *   - query heads in groups sharing one K/V head (GQA; MHA and MQA as the
 *     two ends): "大模型推理为何这么慢？从内存带宽瓶颈到KV Cache优化的技术突围"
 *     (answer.freetools.me), section on GQA and MQA;
 *   - FP8 E4M3 KV with per-token, per-head scales: d7kj.com page, section 四.
 *
 * The pages leave open which query heads form a group; this library takes
 * contiguous groups (h / G).
 *
 * Conventions shared by every call.
 *   - Pointers named "device" point to GPU memory of the current HIP device;
 *     the caller allocates, owns and frees all of them, scratch memory
 *     included (the decode workspace).  The library owns only host-side
 *     handles: no entry point allocates or frees device memory.
 *   - Work is enqueued asynchronously on the caller's stream (a hipStream_t
 *     passed as void*; NULL is the default stream).  No call synchronises,
 *     except the debugging aids pa_block_table_validate and pa_profile_read.
 *     Device buffers must stay valid until the enqueued work completes.
 *   - Every call validates its arguments on the host before any HIP call
 *     and returns a pa_status.  On failure nothing is enqueued and
 *     pa_last_error() (thread-local) holds a one-line description.
 *   - Device-side data (block ids, context lengths) are not read by the
 *     host unless pa_block_table_validate is called.  Invalid device data
 *     give undefined *values* in out, never an out-of-bounds access: the
 *     kernels clamp lengths to max_context_len and skip block ids outside
 *     [0, num_blocks).
 *   - A handle is not thread-safe.  Runs that share a decode workspace must
 *     be ordered (one stream, or synchronised).  Distinct handles with
 *     distinct workspaces are independent.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Tokens per physical block (fixed). */
#define PA_BLOCK_SIZE 16

/* Bytes at the start of a decode workspace that hold arrival counters:
 * zero before the first run (pa_decode_workspace_clear), left zero by every
 * run.  One 32-bit counter for each of at most 65536 workgroups. */
#define PA_DECODE_COUNTER_BYTES 262144

typedef struct pa_kv_pool pa_kv_pool; /* opaque host-side handle */

typedef enum pa_dtype {
  PA_DTYPE_F32 = 0,      /* IEEE binary32                                  */
  PA_DTYPE_BF16 = 1,     /* upper 16 bits of binary32                      */
  PA_DTYPE_FP8_E4M3 = 2, /* OCP E4M3FN: bias 7, max 448, NaN = S.1111.111  */
  PA_DTYPE_INT8_KIVI = 3, /* 8-bit codes, K per channel / V per token (KIVI) */
  PA_DTYPE_INT4_KIVI = 4  /* 4-bit codes, two per byte, same grouping        */
} pa_dtype;

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL                    */
  PA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent        */
  PA_ERR_DTYPE = 3,       /* dtype unknown, or wrong for this entry point  */
  PA_ERR_UNSUPPORTED = 4, /* valid but not built: head_dim, group size     */
  PA_ERR_STATE = 5,       /* e.g. run before a block table was set         */
  PA_ERR_WORKSPACE = 6,   /* workspace missing, too small or misaligned    */
  PA_ERR_HIP = 7,         /* the HIP runtime reported an error             */
  PA_ERR_NO_BLOCKS = 8,   /* block manager: not enough free or cached blocks */
  PA_ERR_SEQUENCE = 9     /* block manager: unknown or duplicate sequence id */
} pa_status;

/*
 * pa_kv_pool_create -- describe a physical block pool (no allocation).
 *
 * k_cache, v_cache: device, [num_blocks][16][num_kv_heads][head_dim] of
 *   kv_dtype, each 16-byte aligned (the block pool of the d7kj.com page,
 *   section 三; layout of the qingdujian.com notes, section 二).  Decode
 *   runs only read them; pa_cache_append writes the new tokens' rows.
 * k_scale, v_scale: device, float32 [num_blocks][num_kv_heads][16] -- one
 *   scale per (block, KV head, slot), i.e. per token and head (d7kj.com
 *   page, section 四); the stored value is e4m3(code) * scale.  Required
 *   when kv_dtype is PA_DTYPE_FP8_E4M3, must be NULL otherwise.
 * block_size must be 16; head_dim must be 64 or 128; num_kv_heads >= 1;
 * num_blocks >= 1.
 * On success *out_pool receives a new handle (free with pa_kv_pool_destroy).
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_UNSUPPORTED.
 */
pa_status pa_kv_pool_create(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                            int32_t head_dim, pa_dtype kv_dtype, void *k_cache, void *v_cache,
                            float *k_scale, float *v_scale, pa_kv_pool **out_pool);

/*
 * pa_kv_pool_placement -- where to put the K and V pools when the caller
 * allocates both in one device buffer (the recommended layout; any
 * placement meeting pa_kv_pool_create's alignment rule works).
 *
 * For a pool of num_blocks blocks of num_kv_heads x head_dim elements of
 * kv_dtype per token (f32, bf16 or FP8 codes; scales are separate):
 *   *pool_bytes  = bytes of one pool (K or V),
 *   *v_offset    = byte offset of the V pool from the start of the buffer
 *                  (the K pool starts at offset 0),
 *   *total_bytes = size of the buffer.
 * v_offset is pool_bytes rounded up to 2 KiB, plus 256.  Why: on MI355X,
 * rows whose device addresses have bits [10:8] equal to 001 or 101 were
 * measured to stream about 18% slower than the rest, whatever the kernel
 * schedule.  With block rows of 2 KiB (8 KV heads of 256 B) one head's rows
 * all share those bits, so with K and V placed alike a (sequence, head)
 * reads only slow rows or only fast ones, and a decode step waits for the
 * slow ones.  Shifting V by 256 B puts a head's K rows and V rows in
 * different address classes (Llama-3-8B-shaped step: 91.3 -> 88.7 us).
 * This is a layout recommendation only: no kernel depends on it.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE.
 */
pa_status pa_kv_pool_placement(int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                               pa_dtype kv_dtype, size_t *pool_bytes, size_t *v_offset,
                               size_t *total_bytes);

/* pa_kv_pool_destroy -- free the handle (NULL is ignored).  Device buffers
 * are untouched.  Work already enqueued is unaffected. */
void pa_kv_pool_destroy(pa_kv_pool *pool);

/*
 * pa_block_table_set -- point the handle at this step's block tables.
 *
 * block_table: device int32 [batch][max_blocks_per_seq]; entry j of row b
 *   is the physical block holding tokens 16j .. 16j+15 of sequence b
 *   (d7kj.com page, section 三).  Entries past a sequence's last block are
 *   never read (pad them with -1).  Rows may share physical blocks (prefix
 *   sharing).
 * context_lens: device int32 [batch]; number of cached tokens each query
 *   attends to, the new token's own K/V included (d7kj.com page, section 六).
 *   0 is allowed and yields a zero output row.
 * max_context_len: host upper bound of context_lens; it sizes the launch
 *   grid and the workspace.  Must satisfy
 *   0 <= max_context_len <= 16 * max_blocks_per_seq.  Lengths above it are
 *   clamped to it by the kernels.
 * Cheap (records pointers and sizes); call it every step.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (batch < 0, max_blocks_per_seq < 1,
 *   max_context_len out of range).
 */
pa_status pa_block_table_set(pa_kv_pool *pool, const int32_t *block_table,
                             const int32_t *context_lens, int32_t batch,
                             int32_t max_blocks_per_seq, int32_t max_context_len);

/*
 * pa_block_table_validate -- debug check of the device tables (synchronous).
 *
 * Copies block_table and context_lens to the host on `stream`, waits, and
 * checks 0 <= context_lens[b] <= max_context_len and that every entry a
 * sequence uses lies in [0, num_blocks).
 * Errors: PA_ERR_STATE (no table set), PA_ERR_SHAPE (a check failed; the
 *   first offending sequence is named in pa_last_error), PA_ERR_HIP.
 */
pa_status pa_block_table_validate(pa_kv_pool *pool, void *stream);

/*
 * pa_cache_append -- write each sequence's new token into the cache.
 *
 * The decode step appends the new token's key and value to its sequence's
 * cache before attending (d7kj.com page, sections 一 and 六).  With the
 * tables set last, the token of sequence b goes to position
 * t = context_lens[b] - 1 (the new token is the last one counted; lengths
 * above max_context_len are clamped to it): physical block
 * block_table[b][t / 16], slot t % 16, one row per KV head.
 * k_new, v_new: device [batch][num_kv_heads][head_dim] of src_dtype.
 *   f32 and bf16 pools: src_dtype must be the pool's dtype; the rows are
 *   stored as they are.
 *   FP8 pool: src_dtype PA_DTYPE_F32 or PA_DTYPE_BF16; each (token, head)
 *   row is quantised (d7kj.com page, section 四): scale = absmax / 448 in
 *   float32 (1 for an all-zero row), code = nearest-even E4M3FN value of
 *   clamp(x / scale, -448, 448) (IEEE float32 division), and the scale is
 *   stored at k_scale / v_scale[block][head][slot].
 * Sequences with context_lens[b] == 0 are skipped; block ids outside
 * [0, num_blocks) are not written.  Asynchronous on `stream`; a decode run
 * enqueued after it on the same stream sees the new rows.
 * Errors: PA_ERR_NULL, PA_ERR_STATE (no table set), PA_ERR_DTYPE,
 *   PA_ERR_SHAPE, PA_ERR_HIP.
 */
pa_status pa_cache_append(pa_kv_pool *pool, const void *k_new, const void *v_new,
                          pa_dtype src_dtype, void *stream);

/*
 * pa_chunk_run -- attention of several new tokens per sequence (a chunk of
 * a prompt's prefill, or the candidate tokens of speculative verification).
 *
 * Chunked prefill cuts a long prompt into chunks run between decode steps
 * (d7kj.com page, section 五); speculative decoding checks several draft
 * tokens in one pass (freetools page, section 技术演进的未来方向).  As for a
 * decode step, the new tokens' K/V are already in the cache: with the
 * tables set last, sequence b has context_lens[b] cached tokens of which
 * the last n_b = q_start[b+1] - q_start[b] are new, so its query rows sit at
 * positions p = context_lens[b] - n_b .. context_lens[b] - 1, and the row at
 * position p attends to the cached tokens 0..p (causal; the minimal
 * implementation of the d7kj.com page, section 六, fed one position at a
 * time, gives the same outputs).  A row whose position would be negative
 * (n_b > context_lens[b]) gets zeros.
 * q: device [total_q][num_q_heads][head_dim] bf16, 16-byte aligned; rows
 *   q_start[b] .. q_start[b+1] - 1 are sequence b's, in position order.
 * q_start: device int32 [batch + 1], nondecreasing; a sequence whose rows
 *   fall outside [0, total_q) or number more than max_q_len is skipped (its
 *   output rows are not written).
 * max_q_len: host bound of n_b; it sizes the grid.
 * out: device float32 [total_q][num_q_heads][head_dim].
 * bf16 and FP8 E4M3 pools (q bf16); head_dim 64 or 128; num_q_heads /
 * num_kv_heads in {1, 2, 4, 8}.  Both products run in bf16 on the matrix
 * cores with fp32 accumulation: FP8 codes are widened to bf16 exactly, the
 * K scale multiplies the fp32 score and the V scale the softmax weight (the
 * d7kj.com page, section 四); each weight enters the PV product as the sum
 * of two bf16 values, within a relative 2^-16 of its fp32 value, and the
 * normaliser sums the same values.  No workspace; asynchronous on `stream`.
 * Errors: PA_ERR_NULL, PA_ERR_STATE (no table set), PA_ERR_DTYPE,
 *   PA_ERR_UNSUPPORTED (f32 or INT8/INT4 pool, group size), PA_ERR_SHAPE,
 *   PA_ERR_HIP.
 */
pa_status pa_chunk_run(pa_kv_pool *pool, const void *q, pa_dtype q_dtype, int32_t num_q_heads,
                       const int32_t *q_start, int32_t total_q, int32_t max_q_len, float scale,
                       float *out, void *stream);

/*
 * Block manager (host memory only; no GPU call).
 *
 * Hands out the physical blocks of one pool and keeps each sequence's block
 * table: the PagedAttention memory management of the d7kj.com page,
 * section 三 (blocks on demand, at most one partly filled block per
 * sequence, physical blocks shared between sequences) and of the
 * freetools page's PagedAttention section (blocks released when a request
 * ends), with the prefix caching of the d7kj.com page, section 五 (blocks
 * found again by hash), whose hashes chain over every earlier block so that
 * one different early token defeats reuse (section 七).
 *   - pa_bm_create: num_blocks >= 1 blocks, ids 0..num_blocks-1 (the pool's);
 *     prefix_caching != 0 turns the prefix cache on.
 *   - pa_bm_add: a new sequence (id of the caller's choice) with its prompt.
 *     *cached_tokens = leading prompt tokens whose K/V already sit in shared
 *     cached blocks (a multiple of 16, at most n_tokens - 1 rounded down to
 *     a block): the caller computes and writes only the tokens after them.
 *   - pa_bm_append: reserve the slot of one more token.  If the sequence's
 *     last block is shared and not full, it is replaced by a private copy:
 *     *n_copies = 1 and (copy_src[0], copy_dst[0]) is the copy to perform
 *     (pa_copy_blocks) before the token is written; else *n_copies = 0.
 *   - pa_bm_fork: child shares all of parent's blocks (e.g. a beam branch).
 *   - pa_bm_free: release a sequence's blocks, last block first.
 *   - pa_bm_table: host int32 table[n][max_blocks] (-1 padded) and lens[n]
 *     (tokens) of the given sequences, ready for pa_block_table_set once
 *     copied to the device.
 *   - pa_bm_stats: free blocks, cached (unreferenced, reusable) blocks and
 *     live sequences.
 * Policies: free blocks form a FIFO queue (initially 0..N-1); a registered
 * full block whose last reference goes stays cached (its K/V still valid)
 * in a least-recently-released list, and is evicted only when a block is
 * needed and the free queue is empty.  A full block is registered (16
 * tokens and a chained FNV-1a hash) when it becomes full, unless a block
 * with the same content is registered already; lookups compare tokens, so
 * a hash collision never shares data.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_SEQUENCE (unknown or duplicate
 *   id), PA_ERR_NO_BLOCKS (not enough free plus cached blocks: the call
 *   changes nothing).  A manager is not thread-safe.
 */
typedef struct pa_block_manager pa_block_manager;
pa_status pa_bm_create(int32_t num_blocks, int32_t prefix_caching, pa_block_manager **out);
void pa_bm_destroy(pa_block_manager *bm);
pa_status pa_bm_add(pa_block_manager *bm, int64_t seq, const int32_t *tokens, int32_t n_tokens,
                    int32_t *cached_tokens);
pa_status pa_bm_append(pa_block_manager *bm, int64_t seq, int32_t token, int32_t *copy_src,
                       int32_t *copy_dst, int32_t *n_copies);
pa_status pa_bm_fork(pa_block_manager *bm, int64_t parent, int64_t child);
pa_status pa_bm_free(pa_block_manager *bm, int64_t seq);
pa_status pa_bm_table(const pa_block_manager *bm, const int64_t *seqs, int32_t n,
                      int32_t max_blocks, int32_t *table, int32_t *lens);
pa_status pa_bm_stats(const pa_block_manager *bm, int32_t *free_blocks, int32_t *cached_blocks,
                      int32_t *sequences);

/*
 * INT8 / INT4 KV cache quantised the KIVI way (freetools page, section
 * "KV Cache量化：用精度换空间": Key per channel, Value per token, parameters
 * from the data, the most recent tokens kept at full precision).
 *
 * pa_kv_pool_create_kivi -- describe such a pool (no allocation).
 *   kv_dtype: PA_DTYPE_INT8_KIVI or PA_DTYPE_INT4_KIVI.
 *   k_codes, v_codes: device [num_blocks][num_kv_heads][16][head_dim * bits / 8]
 *     -- head-major, so one head's 16 rows are contiguous whole cache lines
 *     at either width (INT4: channel 2i in the low nibble of byte i, 2i+1 in
 *     the high one), 16-byte aligned; a block holds 16 quantised tokens.
 *   k_params: device fp16 [num_blocks][num_kv_heads][2][head_dim] -- per
 *     channel of the block: scale (row 0) and min (row 1); 16-byte aligned.
 *   v_params: device fp16 [num_blocks][num_kv_heads][16][2] -- per token:
 *     (scale, min); 16-byte aligned.  value = code * scale + min.
 *   Errors: PA_ERR_NULL, PA_ERR_DTYPE, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED.
 * pa_kivi_residual_set -- the bf16 rows of each sequence's partly filled
 *   last block: device [batch][16][num_kv_heads][head_dim] (row b belongs to
 *   sequence b of the tables set last; slot t % 16 holds token t), 16-byte
 *   aligned.  Tokens of full blocks are read through the table, the last
 *   context_lens % 16 tokens from here.  Errors: PA_ERR_NULL, PA_ERR_DTYPE,
 *   PA_ERR_SHAPE.
 * pa_decode_kivi_run -- one decode step over such a pool: q bf16
 *   [batch][num_q_heads][head_dim] (16-byte aligned), out float32.  No
 *   workspace.  Errors as
 *   pa_decode_run, plus PA_ERR_STATE without a residual.
 * pa_cache_append on such a pool takes bf16 rows: the new token goes to its
 *   residual row; the token that fills a block (t % 16 == 15) has the block
 *   quantised into block_table[b][t / 16]: per channel over the 16 tokens
 *   for K, per token over head_dim for V, scale = fp16((max - min) /
 *   (2^bits - 1)) in float32 (1 if zero), min = fp16(min), code =
 *   clamp(rint((x - min) / scale), 0, 2^bits - 1) in float32.
 * pa_copy_blocks copies codes and both parameter arrays.
 */
pa_status pa_kv_pool_create_kivi(int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                                 pa_dtype kv_dtype, void *k_codes, void *v_codes, void *k_params,
                                 void *v_params, pa_kv_pool **out_pool);
pa_status pa_kivi_residual_set(pa_kv_pool *pool, void *res_k, void *res_v);
pa_status pa_decode_kivi_run(pa_kv_pool *pool, const void *q, pa_dtype q_dtype,
                             int32_t num_q_heads, float scale, float *out, void *stream);

/*
 * pa_copy_blocks -- copy whole physical blocks of a pool (the copies that
 * pa_bm_append orders for copy-on-write of a shared block).
 * pairs: device int32 [n][2] of (src, dst) block ids; the K and V rows of
 * block src (and its FP8 scales) are copied to block dst.  Pairs naming a
 * block outside [0, num_blocks), or with src == dst, are skipped.  The dst
 * blocks must be distinct and none may be another pair's src.
 * Asynchronous on `stream`.  Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_HIP.
 */
pa_status pa_copy_blocks(pa_kv_pool *pool, const int32_t *pairs, int32_t n, void *stream);

/*
 * pa_chunk_tiles -- launch shape of pa_chunk_run (for tests and tuning).
 * One workgroup takes *rows_per_workgroup query rows (a row is one (query
 * token, query head) pair of one KV head's group) of one sequence and KV
 * head; *workgroups_per_head = ceil(max_q_len * G / rows_per_workgroup).
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE.
 */
pa_status pa_chunk_tiles(const pa_kv_pool *pool, int32_t num_q_heads, int32_t max_q_len,
                         int32_t *rows_per_workgroup, int32_t *workgroups_per_head);

/*
 * pa_decode_workspace_bytes -- device scratch a decode run needs.
 *
 * The kernel's workgroups take equal shares of the batch's 16-token blocks
 * (whatever the mix of context lengths), so a sequence may be split
 * between two or more workgroups.  Each piece of a split sequence leaves a
 * running max, a running sum and an unnormalised output per query head
 * (the FlashAttention state of the qingdujian.com notes, section 三),
 * combined exactly (log-sum-exp) by the workgroup that finishes last, which
 * it finds with an arrival counter.  Layout: PA_DECODE_COUNTER_BYTES of
 * counters (fixed size and place), then two records per workgroup sized for
 * the widest head chunk a run may use; the size depends on the workgroup
 * count, the head chunks (pa_decode_workgroups,
 * pa_decode_heads_per_workgroup) and num_q_heads, not on the lengths.
 * *bytes receives the size (0 with a single workgroup: nothing is split).
 * Errors: PA_ERR_NULL, PA_ERR_STATE (no table set), PA_ERR_SHAPE.
 */
pa_status pa_decode_workspace_bytes(const pa_kv_pool *pool, int32_t num_q_heads,
                                    size_t *bytes);

/*
 * pa_decode_workspace_clear -- prepare a decode workspace for its first run.
 *
 * Enqueues on `stream` a kernel that zeroes the counter region (the first
 * min(workspace_bytes, PA_DECODE_COUNTER_BYTES) bytes).  Call it once after
 * allocating a workspace (or zero the whole buffer any other way); every run
 * leaves the counters zero again, so a workspace stays ready for runs of
 * any shape that fit it.  Allocates nothing and does not wait.
 * workspace: device, 256-byte aligned (NULL allowed when workspace_bytes is 0).
 * Errors: PA_ERR_NULL, PA_ERR_WORKSPACE (misaligned), PA_ERR_HIP.
 */
pa_status pa_decode_workspace_clear(void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_decode_run -- one decode step over an f32 or bf16 pool.
 *
 * q: device [batch][num_q_heads][head_dim] of q_dtype (PA_DTYPE_F32 with an
 *   f32 pool, PA_DTYPE_BF16 with a bf16 pool).
 * num_q_heads: a multiple of num_kv_heads with group size
 *   num_q_heads/num_kv_heads in {1, 2, 4, 8}.
 * scale: softmax scale, normally 1/sqrt(head_dim) (d7kj.com page, section 一).
 * out: device float32 [batch][num_q_heads][head_dim], written in full.
 * workspace: device, 256-byte aligned, at least pa_decode_workspace_bytes,
 *   its counter region zero (pa_decode_workspace_clear once after
 *   allocation; runs leave it zero); the rest is scratch.  May be NULL when
 *   that size is 0.  Runs that overlap in time must not share a workspace.
 * stream: hipStream_t of the caller.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (also when batch * num_kv_heads *
 *   ceil(max_context_len / 16) reaches 2^30: the kernel counts its work in
 *   32-bit integers), PA_ERR_DTYPE (pool is FP8, or q_dtype does not
 *   match), PA_ERR_UNSUPPORTED (group size), PA_ERR_STATE (no table set),
 *   PA_ERR_WORKSPACE, PA_ERR_HIP (launch failed; out undefined).
 */
pa_status pa_decode_run(pa_kv_pool *pool, const void *q, pa_dtype q_dtype,
                        int32_t num_q_heads, float scale, float *out, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * pa_decode_fp8_run -- one decode step over an FP8 E4M3 pool.
 *
 * Same arguments and outputs as pa_decode_run; the pool must have been
 * created with PA_DTYPE_FP8_E4M3 and scales, and q_dtype must be
 * PA_DTYPE_BF16.  Keys and values are dequantised in registers as
 * e4m3(code) * scale (d7kj.com page, section 四); accumulation and output
 * are float32.
 * Errors: as pa_decode_run; PA_ERR_DTYPE if the pool is not FP8.
 */
pa_status pa_decode_fp8_run(pa_kv_pool *pool, const void *q, pa_dtype q_dtype,
                            int32_t num_q_heads, float scale, float *out, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * pa_decode_run_noalloc -- one decode step that allocates nothing and takes
 * no workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid it).
 *
 * Same operation, arguments and results as pa_decode_run (f32 and bf16
 * pools) and pa_decode_fp8_run (FP8 pools, chosen by the pool's dtype),
 * minus the workspace: the partial records and arrival counters live in a
 * file-scope device array of the library, 16 MiB, held on each GPU the
 * library runs on until the process ends.  The first call on a device looks
 * up that array's address (hipGetSymbolAddress); every call enqueues, before
 * the attention kernel, a small kernel that zeroes the counters it will use.
 * No hipMalloc, hipFree or wait.  All calls on one GPU share the array:
 * calls that may overlap in time on one GPU (several streams, several host
 * threads) race and give wrong results; order them.
 * Limit: launch shapes whose workspace (pa_decode_workspace_bytes) exceeds
 * 16 MiB are refused with PA_ERR_WORKSPACE (the automatic shape needs at
 * most 8.8 MiB: 256 workgroups, 32 query heads per workgroup, head_dim 128).
 * Errors: as pa_decode_run and pa_decode_fp8_run, PA_ERR_WORKSPACE as above.
 */
pa_status pa_decode_run_noalloc(pa_kv_pool *pool, const void *q, pa_dtype q_dtype,
                                int32_t num_q_heads, float scale, float *out, void *stream);

/*
 * pa_decode_set_workgroups -- override the number of workgroups.
 *
 * count: 0 restores the automatic choice (one per compute unit, 256, or
 * fewer when the batch has fewer 16-token blocks per head chunk);
 * otherwise 1 .. 65536.  Any value gives the same result up to rounding
 * (the merge of split sequences is exact); it only changes parallelism and
 * the workspace size.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE.
 */
pa_status pa_decode_set_workgroups(pa_kv_pool *pool, int32_t count);

/*
 * pa_decode_workgroups -- workgroup count the next run will use for the
 * table set last (after the automatic choice or an override).
 * Errors: PA_ERR_NULL, PA_ERR_STATE (no table set).
 */
pa_status pa_decode_workgroups(const pa_kv_pool *pool, int32_t *count);

/*
 * pa_decode_set_heads_per_workgroup -- override how many adjacent KV heads
 * one workgroup of the attention kernel takes.
 *
 * heads: 0 restores the automatic choice; otherwise a power of two that
 * divides num_kv_heads and is at most the workgroup's wave count (4).  Any
 * value gives the same result; it changes how many contiguous bytes of
 * each block one workgroup reads and how many workgroups there are.
 * Automatic choice, made on the device from the lengths: when every
 * sequence has the block count of max_context_len, the largest chunk for
 * which batch * num_kv_heads / heads is still at least 256 (each
 * workgroup's share is then whole sequences), else the largest allowed;
 * when the block counts differ, the largest allowed (shares cut across
 * sequences anyway, and fewer, longer pieces stream faster).  An override
 * fixes the chunk for both cases.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE.
 */
pa_status pa_decode_set_heads_per_workgroup(pa_kv_pool *pool, int32_t heads);

/*
 * pa_decode_heads_per_workgroup -- head chunk the next run will use for the
 * table set last if every sequence has the block count of max_context_len
 * (with differing block counts the run takes the largest allowed chunk,
 * unless an override is set).
 * Errors: PA_ERR_NULL, PA_ERR_STATE (no table set).
 */
pa_status pa_decode_heads_per_workgroup(const pa_kv_pool *pool, int32_t *heads);

/*
 * pa_profile_enable -- time the attention kernel of the next runs.
 *
 * While enabled (capacity > 0), each run records a pair of HIP events on
 * its stream, attached to the dispatch of its attention kernel (the start
 * and the end of the kernel's own execution), for up to `capacity` runs;
 * capacity 0 disables and releases the events.  Events are host-side HIP
 * objects, not device memory.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (capacity < 0), PA_ERR_HIP.
 */
pa_status pa_profile_enable(pa_kv_pool *pool, int32_t capacity);

/*
 * pa_profile_read -- per-run kernel durations recorded since enabling.
 *
 * Waits for the recorded events, writes up to `capacity` durations in
 * milliseconds to kernel_ms[i] (may be NULL) and the number of recorded
 * runs to *count, then starts a new recording.
 * Errors: PA_ERR_NULL, PA_ERR_STATE (profiling not enabled), PA_ERR_HIP.
 */
pa_status pa_profile_read(pa_kv_pool *pool, float *kernel_ms, int32_t capacity,
                          int32_t *count);

/* Static text for a status code. */
const char *pa_status_str(pa_status status);

/* Description of the last failure on this thread ("" if none). */
const char *pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
