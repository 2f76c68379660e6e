// pa_block_manager.cpp -- host-side manager of the physical blocks of a paged
// KV cache: on-demand allocation, reference-counted sharing, copy-on-write
// and hash-chained prefix caching.  Host memory only; no HIP call.
//
// What it does ("KV Cache 深度解析:显存黑洞、PagedAttention 与三路省内存方案",
// sections 三, 五 and 七; the PagedAttention sections of the other pages):
//
//  - A sequence owns a block table that grows on demand: a block is taken
//    only when the last one is full, so at most one block per sequence is
//    partly empty.  When a sequence ends its blocks are released at once.
//  - Sequences share physical blocks by reference count (branches of one
//    request via fork, requests with a common prefix via the prefix cache).
//    A shared block that must still receive a token is copied first (the
//    copy is reported to the caller, who runs pa_copy_blocks before writing).
//  - Prefix caching: a full block is registered under a hash of its 16
//    tokens chained with the hash of the block before it, so one different
//    token early in a prompt changes every later hash.  Lookups compare the
//    tokens too, so a collision never shares wrong data.
//
// Policies where the pages are silent: free blocks are a FIFO queue
// (initially 0..N-1; released blocks join the back); a registered block
// whose last reference goes stays cached in a least-recently-released list
// and is evicted (forgotten) only when a block is needed and the free queue
// is empty; a sequence releases its blocks from last to first; a new
// sequence reuses cached blocks only among the full blocks of its first
// n - 1 tokens; a request that cannot get enough blocks fails and changes
// nothing.

#include <array>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <deque>
#include <list>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

constexpr int kBlockTokens = PA_BLOCK_SIZE;
using Tokens = std::array<int32_t, kBlockTokens>;

// FNV-1a, 64 bit (Fowler, Noll, Vo), over the parent hash (8 bytes, little
// endian) and the block's 16 token ids (4 bytes each, little endian).
uint64_t block_hash(uint64_t parent, const int32_t *tok) {
  uint64_t h = 0xCBF29CE484222325ull;
  auto mix = [&](uint64_t v, int bytes) {
    for (int i = 0; i < bytes; ++i) {
      h ^= (v >> (8 * i)) & 0xFF;
      h *= 0x100000001B3ull;
    }
  };
  mix(parent, 8);
  for (int i = 0; i < kBlockTokens; ++i) mix((uint32_t)tok[i], 4);
  return h;
}

struct Sequence {
  std::vector<int32_t> table;   // physical block of each logical block
  std::vector<int32_t> tokens;  // every token so far
  std::vector<uint64_t> hashes; // chained hash of each full block
};

struct BlockInfo {
  int32_t ref = 0;
  bool registered = false;      // content known to the prefix cache
  uint64_t hash = 0;
  Tokens tokens{};
  std::list<int32_t>::iterator lru;  // valid while in the cached list
};

pa_status bm_fail(pa_status s, const char *fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return pa::record_error(s, buf);
}

}  // namespace

struct pa_block_manager {
  int32_t num_blocks = 0;
  bool caching = false;
  std::vector<BlockInfo> blocks;
  std::deque<int32_t> free_q;
  std::list<int32_t> cached;  // unreferenced registered blocks, oldest first
  std::unordered_multimap<uint64_t, int32_t> by_hash;
  std::unordered_map<int64_t, Sequence> seqs;

  int64_t available() const { return (int64_t)free_q.size() + (int64_t)cached.size(); }

  int32_t lookup(uint64_t h, const int32_t *tok) const {
    auto range = by_hash.equal_range(h);
    for (auto it = range.first; it != range.second; ++it) {
      const BlockInfo &bi = blocks[it->second];
      bool same = true;
      for (int i = 0; i < kBlockTokens && same; ++i) same = bi.tokens[i] == tok[i];
      if (same) return it->second;
    }
    return -1;
  }

  void forget(int32_t b) {
    BlockInfo &bi = blocks[b];
    auto range = by_hash.equal_range(bi.hash);
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == b) {
        by_hash.erase(it);
        break;
      }
    bi.registered = false;
  }

  // A block for new data; the caller has checked available() > 0.
  int32_t take() {
    int32_t b;
    if (!free_q.empty()) {
      b = free_q.front();
      free_q.pop_front();
    } else {
      b = cached.front();
      cached.pop_front();
      forget(b);
    }
    blocks[b].ref = 1;
    return b;
  }

  void release(int32_t b) {
    BlockInfo &bi = blocks[b];
    if (--bi.ref == 0) {
      if (bi.registered) {
        cached.push_back(b);
        bi.lru = std::prev(cached.end());
      } else {
        free_q.push_back(b);
      }
    }
  }

  // Block j of sequence s has just become full (its hash is s.hashes[j]).
  void register_full(const Sequence &s, size_t j) {
    if (!caching) return;
    const int32_t b = s.table[j];
    BlockInfo &bi = blocks[b];
    if (bi.registered) return;
    const int32_t *tok = s.tokens.data() + j * kBlockTokens;
    if (lookup(s.hashes[j], tok) >= 0) return;
    bi.registered = true;
    bi.hash = s.hashes[j];
    for (int i = 0; i < kBlockTokens; ++i) bi.tokens[i] = tok[i];
    by_hash.emplace(bi.hash, b);
  }
};

extern "C" {

pa_status pa_bm_create(int32_t num_blocks, int32_t prefix_caching, pa_block_manager **out) {
  if (!out) return bm_fail(PA_ERR_NULL, "out is NULL");
  *out = nullptr;
  if (num_blocks < 1) return bm_fail(PA_ERR_SHAPE, "num_blocks %d < 1", num_blocks);
  pa_block_manager *m = new (std::nothrow) pa_block_manager();
  if (!m) return bm_fail(PA_ERR_SHAPE, "out of host memory");
  m->num_blocks = num_blocks;
  m->caching = prefix_caching != 0;
  m->blocks.resize(num_blocks);
  for (int32_t b = 0; b < num_blocks; ++b) m->free_q.push_back(b);
  *out = m;
  pa::clear_error();
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager *bm) { delete bm; }

pa_status pa_bm_add(pa_block_manager *bm, int64_t seq, const int32_t *tokens, int32_t n_tokens,
                    int32_t *cached_tokens) {
  if (!bm || !cached_tokens || (n_tokens > 0 && !tokens))
    return bm_fail(PA_ERR_NULL, "bm, tokens or cached_tokens is NULL");
  if (n_tokens < 0) return bm_fail(PA_ERR_SHAPE, "n_tokens %d < 0", n_tokens);
  if (bm->seqs.count(seq)) return bm_fail(PA_ERR_SEQUENCE, "sequence %lld exists", (long long)seq);
  const int64_t need = (n_tokens + kBlockTokens - 1) / kBlockTokens;
  // chained hashes of the prompt's full blocks
  std::vector<uint64_t> hashes;
  uint64_t h = 0;
  for (int64_t j = 0; j < n_tokens / kBlockTokens; ++j) {
    h = block_hash(h, tokens + j * kBlockTokens);
    hashes.push_back(h);
  }
  std::vector<int32_t> matched;
  if (bm->caching && n_tokens > 0) {
    for (int64_t j = 0; j < (n_tokens - 1) / kBlockTokens; ++j) {
      const int32_t b = bm->lookup(hashes[j], tokens + j * kBlockTokens);
      if (b < 0) break;
      matched.push_back(b);
    }
  }
  int64_t revived = 0;
  for (int32_t b : matched) revived += bm->blocks[b].ref == 0;
  if (need - (int64_t)matched.size() > bm->available() - revived)
    return bm_fail(PA_ERR_NO_BLOCKS, "%lld blocks needed, %lld available",
                   (long long)(need - (int64_t)matched.size()),
                   (long long)(bm->available() - revived));
  Sequence s;
  for (int32_t b : matched) {
    BlockInfo &bi = bm->blocks[b];
    if (bi.ref == 0) bm->cached.erase(bi.lru);
    ++bi.ref;
    s.table.push_back(b);
  }
  while ((int64_t)s.table.size() < need) s.table.push_back(bm->take());
  s.tokens.assign(tokens, tokens + n_tokens);
  s.hashes = hashes;
  for (size_t j = matched.size(); j < hashes.size(); ++j) bm->register_full(s, j);
  bm->seqs.emplace(seq, std::move(s));
  *cached_tokens = (int32_t)(matched.size() * kBlockTokens);
  pa::clear_error();
  return PA_OK;
}

pa_status pa_bm_append(pa_block_manager *bm, int64_t seq, int32_t token, int32_t *copy_src,
                       int32_t *copy_dst, int32_t *n_copies) {
  if (!bm || !copy_src || !copy_dst || !n_copies) return bm_fail(PA_ERR_NULL, "NULL argument");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return bm_fail(PA_ERR_SEQUENCE, "no sequence %lld", (long long)seq);
  Sequence &s = it->second;
  const size_t t = s.tokens.size();
  *n_copies = 0;
  if (t % kBlockTokens == 0) {
    if (bm->available() < 1) return bm_fail(PA_ERR_NO_BLOCKS, "no block for the new token");
    s.table.push_back(bm->take());
  } else {
    const int32_t last = s.table.back();
    if (bm->blocks[last].ref > 1) {  // shared: copy before writing
      if (bm->available() < 1) return bm_fail(PA_ERR_NO_BLOCKS, "no block for the copy");
      const int32_t fresh = bm->take();
      bm->release(last);
      s.table.back() = fresh;
      copy_src[0] = last;
      copy_dst[0] = fresh;
      *n_copies = 1;
    }
  }
  s.tokens.push_back(token);
  if ((t + 1) % kBlockTokens == 0) {
    const size_t j = t / kBlockTokens;
    s.hashes.push_back(block_hash(j ? s.hashes[j - 1] : 0, s.tokens.data() + j * kBlockTokens));
    bm->register_full(s, j);
  }
  pa::clear_error();
  return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager *bm, int64_t parent, int64_t child) {
  if (!bm) return bm_fail(PA_ERR_NULL, "bm is NULL");
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return bm_fail(PA_ERR_SEQUENCE, "no sequence %lld", (long long)parent);
  if (bm->seqs.count(child)) return bm_fail(PA_ERR_SEQUENCE, "sequence %lld exists", (long long)child);
  Sequence c = it->second;
  for (int32_t b : c.table) ++bm->blocks[b].ref;
  bm->seqs.emplace(child, std::move(c));
  pa::clear_error();
  return PA_OK;
}

pa_status pa_bm_free(pa_block_manager *bm, int64_t seq) {
  if (!bm) return bm_fail(PA_ERR_NULL, "bm is NULL");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return bm_fail(PA_ERR_SEQUENCE, "no sequence %lld", (long long)seq);
  const std::vector<int32_t> &t = it->second.table;
  for (size_t j = t.size(); j-- > 0;) bm->release(t[j]);
  bm->seqs.erase(it);
  pa::clear_error();
  return PA_OK;
}

pa_status pa_bm_table(const pa_block_manager *bm, const int64_t *seqs, int32_t n,
                      int32_t max_blocks, int32_t *table, int32_t *lens) {
  if (!bm || (n > 0 && (!seqs || !table || !lens))) return bm_fail(PA_ERR_NULL, "NULL argument");
  if (n < 0 || max_blocks < 1) return bm_fail(PA_ERR_SHAPE, "n %d, max_blocks %d", n, max_blocks);
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end())
      return bm_fail(PA_ERR_SEQUENCE, "no sequence %lld", (long long)seqs[i]);
    if ((int64_t)it->second.table.size() > max_blocks)
      return bm_fail(PA_ERR_SHAPE, "sequence %lld holds %zu blocks > max_blocks %d",
                     (long long)seqs[i], it->second.table.size(), max_blocks);
  }
  for (int32_t i = 0; i < n; ++i) {
    const Sequence &s = bm->seqs.find(seqs[i])->second;
    int32_t *row = table + (size_t)i * max_blocks;
    for (int32_t j = 0; j < max_blocks; ++j) row[j] = j < (int32_t)s.table.size() ? s.table[j] : -1;
    lens[i] = (int32_t)s.tokens.size();
  }
  pa::clear_error();
  return PA_OK;
}

pa_status pa_bm_stats(const pa_block_manager *bm, int32_t *free_blocks, int32_t *cached_blocks,
                      int32_t *sequences) {
  if (!bm || !free_blocks || !cached_blocks || !sequences)
    return bm_fail(PA_ERR_NULL, "NULL argument");
  *free_blocks = (int32_t)bm->free_q.size();
  *cached_blocks = (int32_t)bm->cached.size();
  *sequences = (int32_t)bm->seqs.size();
  pa::clear_error();
  return PA_OK;
}

}  // extern "C"
