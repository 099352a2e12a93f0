// Host side of the pkv library: error reporting, size formulas, the block
// pool allocator and the block-table / slot-mapping builders.
//
// The allocator follows the block manager of "Reducing LLM Inference
// Latency: KV Cache Quantization and PagedAttention in vLLM" (section
// "PagedAttention: Solving VRAM Fragmentation"): a FIFO list of free
// physical blocks, a per-sequence list of physical block ids, and the
// address of token t = (table[t / p], t % p).  Appending takes a new block
// only when the token count is a multiple of p ("Optimizing LLM Inference:
// KV Cache and PagedAttention Explained", section "PagedAttention:
// Operating Systems to the Rescue").  Shared prefixes point several tables
// at the same blocks ("KV Cache Compression & Paged Attention Deep Dive",
// section "PagedAttention: Operating System-Inspired Memory Management");
// reference counts decide when a block is free again.
//
// Unlike the pages' emulation, every operation checks before it changes
// anything (all-or-nothing), allocating a live sequence is an error, and the
// free list is a ring buffer so that take/return are O(1).
//
// Copy-on-write (named with per-block reference counts in "KV Cache
// Compression & Paged Attention Deep Dive", sections "PagedAttention:
// Operating System-Inspired Memory Management" and "Implementation Details:
// PagedAttention Kernel and Page Table"): a fork may end inside a block, and
// the new sequence then shares that partly filled block too.  The first
// sequence about to write into a partly filled block that another table
// still points at takes a fresh block (before any block its append grows
// by), records the copy old -> new and moves its table entry to the new
// block.  Copies stay pending until the caller takes them (and runs them on
// the device before the same appends' tokens are written); fork and free
// are refused meanwhile, which keeps the pending copies disjoint: no
// destination is ever a source, and no block of a pending copy can return
// to the free list.
//
// Automatic prefix caching ("KV Cache Compression & Paged Attention Deep
// Dive", section "Implementation Details: PagedAttention Kernel and Page
// Table": look the hashed prefix up before allocating; "KV Cache
// Optimization: 3x Faster LLM Inference on 24GB VRAM", section "Prefix
// Caching: The Hidden Multiplier": later requests reuse the pages of a
// common prefix, pages are evicted in LRU order): every full block of a
// prompt allocated with its token ids enters a hash map under the key
// (entry id of the block before it or -1, the block's p token ids), matched
// exactly (the stored ids are compared on a hash hit).  Entry
// ids are never reused, so entries below an evicted block become
// unreachable.  A cached block whose last reference goes joins an LRU list
// instead of the free list and can still be found; blocks are taken from
// the free list first, then by evicting the least recently released cached
// block.
//
// Swapping ("Reducing LLM Inference Latency: KV Cache Quantization and
// PagedAttention in vLLM", section "Prefill Swapping and GPU Thrashing": KV
// pages move to host memory when the pool is exhausted): a pool may have a
// FIFO of host blocks.  Swap-out moves every block the sequence holds alone
// to a host block (front of the host FIFO, table order) and releases the
// device block; shared blocks keep their device reference.  Swap-in takes
// device blocks for the host entries in table order and returns the host
// blocks to the back of the host FIFO.  Each returns (device block, host
// block) pairs for pkv_swap_blocks.
#include <algorithm>
#include <cstdio>
#include <list>
#include <cstring>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pkv_internal.h"

namespace pkv {

static thread_local std::string g_last_error;

pkv_status fail(pkv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

void clear_error() { g_last_error.clear(); }

bool is_16bit_kv(int32_t kv) { return kv == PKV_F16 || kv == PKV_BF16; }

static bool is_fp8_kv(int32_t kv) {
  return kv == PKV_FP8_E4M3 || kv == PKV_FP8_E5M2 || kv == PKV_FP8_E4M3_BLOCK;
}

pkv_status validate_desc(const pkv_cache_desc* d) {
  if (!d) return fail(PKV_ERR_INVALID_ARG, "desc is NULL");
  if (!is_16bit_kv(d->kv_dtype) && !is_fp8_kv(d->kv_dtype) && d->kv_dtype != PKV_INT4_ASYM_G32)
    return fail(PKV_ERR_INVALID_ARG, "kv_dtype %d is not a cache type", d->kv_dtype);
  if (d->io_dtype != PKV_F16 && d->io_dtype != PKV_BF16 && d->io_dtype != PKV_F32)
    return fail(PKV_ERR_INVALID_ARG, "io_dtype %d must be F16, BF16 or F32", d->io_dtype);
  if (is_16bit_kv(d->kv_dtype) && d->io_dtype != PKV_F32 && d->io_dtype != d->kv_dtype)
    return fail(PKV_ERR_INVALID_ARG, "a 16-bit cache needs io_dtype equal to kv_dtype or F32");
  if (d->num_kv_heads < 1) return fail(PKV_ERR_INVALID_ARG, "num_kv_heads must be >= 1");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", d->head_dim);
  if (d->block_size != 16 && d->block_size != 32)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d (supported: 16, 32)", d->block_size);
  if (d->num_blocks < 1 || d->num_blocks > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARG, "num_blocks %lld out of range", (long long)d->num_blocks);
  return PKV_OK;
}

static size_t pool_bytes_per_chunk(const pkv_cache_desc& d) {
  const size_t pd = (size_t)d.block_size * d.head_dim;
  switch (d.kv_dtype) {
    case PKV_F16:
    case PKV_BF16: return pd * 2;
    case PKV_FP8_E4M3:
    case PKV_FP8_E5M2:
    case PKV_FP8_E4M3_BLOCK: return pd;
    default: return pd / 2;
  }
}

static size_t meta_bytes_per_chunk(const pkv_cache_desc& d) {
  switch (d.kv_dtype) {
    case PKV_FP8_E4M3:
    case PKV_FP8_E5M2:
    case PKV_FP8_E4M3_BLOCK: return (size_t)d.block_size * 4;
    case PKV_INT4_ASYM_G32: return (size_t)d.block_size * (d.head_dim / 32) * 4;
    default: return 0;
  }
}

}  // namespace pkv

using namespace pkv;

// ------------------------------------------------------------------ errors

extern "C" const char* pkv_status_str(pkv_status s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_OUT_OF_BLOCKS: return "block pool exhausted";
    case PKV_ERR_NO_SUCH_SEQ: return "no such sequence";
    case PKV_ERR_SEQ_EXISTS: return "sequence exists";
    case PKV_ERR_UNSUPPORTED: return "unsupported";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_COPIES_PENDING: return "block copies pending";
    case PKV_ERR_SEQ_SWAPPED: return "sequence swapped out";
  }
  return "unknown status";
}

extern "C" const char* pkv_last_error(void) { return g_last_error.c_str(); }

extern "C" const char* pkv_version(void) { return "pkv 0.1 gfx950"; }

// ------------------------------------------------------------------- sizes

extern "C" int64_t pkv_kv_bytes(int64_t layers, int64_t kv_heads, int64_t head_dim,
                                int64_t seq_len, int64_t batch, int64_t bytes_x2) {
  if (layers < 0 || kv_heads < 0 || head_dim < 0 || seq_len < 0 || batch < 0 || bytes_x2 < 0)
    return -1;
  // 2 (K and V) * ... * P  ==  (...) * bytes_x2.  Each partial product is
  // checked before the next multiply, so no product exceeds 2^63 * 2^63.
  const int64_t f[6] = {layers, kv_heads, head_dim, seq_len, batch, bytes_x2};
  __int128 r = 1;
  for (int i = 0; i < 6; ++i) {
    r *= f[i];
    if (r > INT64_MAX) return -1;
  }
  return (int64_t)r;
}

extern "C" pkv_status pkv_cache_bytes(const pkv_cache_desc* desc, size_t* pool_bytes,
                                      size_t* meta_bytes) {
  pkv_status s = validate_desc(desc);
  if (s != PKV_OK) return s;
  const size_t chunks = (size_t)desc->num_blocks * desc->num_kv_heads;
  if (pool_bytes) *pool_bytes = chunks * pool_bytes_per_chunk(*desc);
  if (meta_bytes) *meta_bytes = chunks * meta_bytes_per_chunk(*desc);
  return PKV_OK;
}

// ---------------------------------------------------------------- the pool

struct pkv_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ring;  // FIFO of free block ids
  int32_t head = 0;           // index of the front of the FIFO
  int32_t count = 0;          // number of free blocks
  std::vector<int32_t> ref;   // references per block (0 = free)
  struct Seq {
    std::vector<int32_t> blocks;
    int32_t ntok = 0;
    bool swapped = false;
    std::vector<char> on_host;  // when swapped: which entries are host blocks
  };
  std::unordered_map<int64_t, Seq> seqs;
  std::vector<int32_t> copies;  // pending (source, destination) pairs
  // prefix cache
  // key hash -> cached blocks with that hash; a hit also compares the
  // block's stored parent entry and token ids, so collisions cannot match
  std::unordered_multimap<uint64_t, int32_t> cache;
  std::vector<int64_t> entry_parent;               // per block: entry before it (-1: none)
  std::vector<int32_t> entry_tokens;               // per block: its p token ids
  std::vector<uint64_t> entry_hash;                // per block, for eviction
  std::vector<int64_t> entry_id;                   // per block; -1: not cached
  std::list<int32_t> lru;                          // released cached blocks, oldest first
  std::vector<std::list<int32_t>::iterator> lru_pos;
  std::vector<char> in_lru;
  int64_t next_entry = 0, hits = 0, queries = 0;
  // host blocks for swapping (FIFO ring like the device one)
  std::vector<int32_t> host_ring;
  int32_t host_head = 0, host_count = 0, num_host = 0, swapped = 0;
  int32_t host_take() {
    const int32_t h = host_ring[host_head];
    host_head = host_head + 1 == num_host ? 0 : host_head + 1;
    --host_count;
    return h;
  }
  void host_give(int32_t h) {
    int32_t tail = host_head + host_count;
    if (tail >= num_host) tail -= num_host;
    host_ring[tail] = h;
    ++host_count;
  }

  // Blocks an allocation can take: free ones and evictable cached ones.
  int64_t available() const { return (int64_t)count + (int64_t)lru.size(); }

  uint64_t hash_of(int64_t parent, const int32_t* tokens) const {
    uint64_t h = 0x9E3779B97F4A7C15ull ^ (uint64_t)parent;
    for (int32_t i = 0; i < block_size; ++i) {
      h ^= (uint32_t)tokens[i];
      h *= 0xBF58476D1CE4E5B9ull;
      h ^= h >> 31;
    }
    return h;
  }
  // The cached block under (parent, tokens), or -1.
  int32_t find_cached(int64_t parent, const int32_t* tokens, uint64_t h) const {
    auto range = cache.equal_range(h);
    for (auto it = range.first; it != range.second; ++it) {
      const int32_t b = it->second;
      if (entry_parent[b] == parent &&
          std::memcmp(&entry_tokens[(size_t)b * block_size], tokens,
                      sizeof(int32_t) * (size_t)block_size) == 0)
        return b;
    }
    return -1;
  }
  void uncache(int32_t b) {
    auto range = cache.equal_range(entry_hash[b]);
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == b) {
        cache.erase(it);
        break;
      }
    entry_id[b] = -1;
  }
  void lru_remove(int32_t b) {
    lru.erase(lru_pos[b]);
    in_lru[b] = 0;
  }
  // Drops one reference; at zero a cached block becomes evictable and any
  // other block returns to the back of the free list.
  void release(int32_t b) {
    if (--ref[b] != 0) return;
    if (entry_id[b] >= 0) {
      lru_pos[b] = lru.insert(lru.end(), b);
      in_lru[b] = 1;
    } else {
      give(b);
    }
  }

  // Whether the next token of s would land in a partly filled block that
  // another table also points at.  `released` counts references the same
  // batch has already moved off that block.
  bool needs_copy(const Seq& s, int32_t num_tokens, int32_t released = 0) const {
    return num_tokens > 0 && s.ntok % block_size != 0 &&
           ref[s.blocks.back()] - released > 1;
  }
  // Moves s off its shared last block onto a fresh one (caller checked a
  // block is free) and records the copy.
  void copy_on_write(Seq& s) {
    const int32_t old = s.blocks.back();
    s.blocks.pop_back();
    take(1, s.blocks);
    --ref[old];
    copies.push_back(old);
    copies.push_back(s.blocks.back());
  }

  int32_t blocks_for(int64_t ntok) const { return (int32_t)((ntok + block_size - 1) / block_size); }

  // Takes k blocks from the front of the FIFO, then by evicting the least
  // recently released cached blocks (caller checked available() >= k).
  void take(int32_t k, std::vector<int32_t>& out) {
    for (int32_t i = 0; i < k; ++i) {
      int32_t b;
      if (count > 0) {
        b = ring[head];
        head = head + 1 == num_blocks ? 0 : head + 1;
        --count;
      } else {
        b = lru.front();
        lru_remove(b);
        uncache(b);
      }
      ref[b] = 1;
      out.push_back(b);
    }
  }
  // Returns a block to the back of the FIFO.
  void give(int32_t b) {
    int32_t tail = head + count;
    if (tail >= num_blocks) tail -= num_blocks;
    ring[tail] = b;
    ++count;
  }
};

// The sequence, or NULL with the error recorded (NO_SUCH_SEQ, SEQ_SWAPPED).
static pkv_pool::Seq* live_seq(pkv_pool* pool, int64_t seq, pkv_status* st) {
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) {
    *st = fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld", (long long)seq);
    return nullptr;
  }
  if (it->second.swapped) {
    *st = fail(PKV_ERR_SEQ_SWAPPED, "sequence %lld is swapped out", (long long)seq);
    return nullptr;
  }
  return &it->second;
}
static const pkv_pool::Seq* live_seq(const pkv_pool* pool, int64_t seq, pkv_status* st) {
  return live_seq(const_cast<pkv_pool*>(pool), seq, st);
}

extern "C" pkv_status pkv_pool_create(int32_t num_blocks, int32_t block_size,
                                      const int32_t* free_order, pkv_pool** out) {
  if (!out) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (num_blocks < 1) return fail(PKV_ERR_INVALID_ARG, "num_blocks must be >= 1");
  if (block_size < 1) return fail(PKV_ERR_INVALID_ARG, "block_size must be >= 1");
  pkv_pool* p = new (std::nothrow) pkv_pool;
  if (!p) return fail(PKV_ERR_INVALID_ARG, "out of host memory");
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->ring.resize(num_blocks);
  p->ref.assign(num_blocks, 0);
  p->entry_id.assign(num_blocks, -1);
  p->entry_parent.assign(num_blocks, -1);
  p->entry_hash.assign(num_blocks, 0);
  p->lru_pos.resize(num_blocks);
  p->in_lru.assign(num_blocks, 0);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete p;
        return fail(PKV_ERR_INVALID_ARG, "free_order is not a permutation of 0..%d", num_blocks - 1);
      }
      seen[b] = 1;
      p->ring[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) p->ring[i] = i;
  }
  p->count = num_blocks;
  *out = p;
  return PKV_OK;
}

extern "C" void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

extern "C" pkv_status pkv_seq_allocate(pkv_pool* pool, int64_t seq, int32_t num_tokens) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (seq < 0) return fail(PKV_ERR_INVALID_ARG, "sequence ids are >= 0");
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens must be >= 0");
  if (pool->seqs.count(seq)) return fail(PKV_ERR_SEQ_EXISTS, "sequence %lld exists", (long long)seq);
  int32_t need = pool->blocks_for(num_tokens);
  if (need > pool->available())
    return fail(PKV_ERR_OUT_OF_BLOCKS, "block pool exhausted: need %d blocks, %lld free", need,
                (long long)pool->available());
  pkv_pool::Seq s;
  s.blocks.reserve(need);
  pool->take(need, s.blocks);
  s.ntok = num_tokens;
  pool->seqs.emplace(seq, std::move(s));
  return PKV_OK;
}

extern "C" pkv_status pkv_seq_append(pkv_pool* pool, int64_t seq, int32_t num_tokens,
                                     int64_t* out_slots) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens must be >= 0");
  pkv_status st;
  pkv_pool::Seq* sp = live_seq(pool, seq, &st);
  if (!sp) return st;
  pkv_pool::Seq& s = *sp;
  int64_t total = (int64_t)s.ntok + num_tokens;
  if (total > INT32_MAX) return fail(PKV_ERR_INVALID_ARG, "sequence length overflows int32");
  int32_t need = pool->blocks_for(total) - (int32_t)s.blocks.size();
  if (need < 0) need = 0;
  const bool cow = pool->needs_copy(s, num_tokens);
  if (need + (int32_t)cow > pool->available())
    return fail(PKV_ERR_OUT_OF_BLOCKS, "block pool exhausted: need %d blocks, %lld free",
                need + (int32_t)cow, (long long)pool->available());
  if (cow) pool->copy_on_write(s);
  pool->take(need, s.blocks);
  const int32_t p = pool->block_size;
  if (out_slots)
    for (int32_t i = 0; i < num_tokens; ++i) {
      int32_t t = s.ntok + i;
      out_slots[i] = (int64_t)s.blocks[t / p] * p + t % p;
    }
  s.ntok = (int32_t)total;
  return PKV_OK;
}

extern "C" pkv_status pkv_seq_append_batch(pkv_pool* pool, const int64_t* seqs, int32_t B,
                                           int32_t num_tokens, int64_t* out_slots) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (B < 0 || num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "B and num_tokens must be >= 0");
  if (B > 0 && !seqs) return fail(PKV_ERR_INVALID_ARG, "seqs is NULL");
  // check the whole batch first (existence, overflow, blocks needed,
  // copies: a later member sharing a block an earlier one copies away from
  // sees one reference less)
  std::vector<pkv_pool::Seq*> rows(B);
  std::unordered_map<int32_t, int32_t> released;
  int64_t need_total = 0;
  for (int32_t i = 0; i < B; ++i) {
    auto it = pool->seqs.find(seqs[i]);
    if (it == pool->seqs.end())
      return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld", (long long)seqs[i]);
    if (it->second.swapped)
      return fail(PKV_ERR_SEQ_SWAPPED, "sequence %lld is swapped out", (long long)seqs[i]);
    for (int32_t k = 0; k < i; ++k)
      if (rows[k] == &it->second)
        return fail(PKV_ERR_INVALID_ARG, "sequence %lld repeats in the batch", (long long)seqs[i]);
    rows[i] = &it->second;
    const int64_t total = (int64_t)it->second.ntok + num_tokens;
    if (total > INT32_MAX) return fail(PKV_ERR_INVALID_ARG, "sequence length overflows int32");
    const int32_t need = pool->blocks_for(total) - (int32_t)it->second.blocks.size();
    need_total += need > 0 ? need : 0;
    if (num_tokens > 0 && it->second.ntok % pool->block_size != 0) {
      const int32_t last = it->second.blocks.back();
      auto r = released.find(last);
      if (pool->needs_copy(it->second, num_tokens, r == released.end() ? 0 : r->second)) {
        ++need_total;
        ++released[last];
      }
    }
  }
  if (need_total > pool->available())
    return fail(PKV_ERR_OUT_OF_BLOCKS, "block pool exhausted: need %lld blocks, %lld free",
                (long long)need_total, (long long)pool->available());
  const int32_t p = pool->block_size;
  for (int32_t i = 0; i < B; ++i) {
    pkv_pool::Seq& s = *rows[i];
    const int32_t need = pool->blocks_for((int64_t)s.ntok + num_tokens) - (int32_t)s.blocks.size();
    if (pool->needs_copy(s, num_tokens)) pool->copy_on_write(s);
    if (need > 0) pool->take(need, s.blocks);
    if (out_slots)
      for (int32_t k = 0; k < num_tokens; ++k) {
        const int32_t t = s.ntok + k;
        out_slots[(int64_t)i * num_tokens + k] = (int64_t)s.blocks[t / p] * p + t % p;
      }
    s.ntok += num_tokens;
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_seq_fork(pkv_pool* pool, int64_t src, int64_t dst,
                                   int32_t prefix_tokens) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (dst < 0) return fail(PKV_ERR_INVALID_ARG, "sequence ids are >= 0");
  auto it = pool->seqs.find(src);
  if (it == pool->seqs.end())
    return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld", (long long)src);
  if (it->second.swapped)
    return fail(PKV_ERR_SEQ_SWAPPED, "sequence %lld is swapped out", (long long)src);
  if (pool->seqs.count(dst)) return fail(PKV_ERR_SEQ_EXISTS, "sequence %lld exists", (long long)dst);
  if (prefix_tokens < 0 || prefix_tokens > it->second.ntok)
    return fail(PKV_ERR_INVALID_ARG, "fork of %d tokens from a sequence of %d", prefix_tokens,
                it->second.ntok);
  if (!pool->copies.empty())
    return fail(PKV_ERR_COPIES_PENDING, "%zu block copies pending: take them before a fork",
                pool->copies.size() / 2);
  pkv_pool::Seq s;
  s.blocks.assign(it->second.blocks.begin(),
                  it->second.blocks.begin() + pool->blocks_for(prefix_tokens));
  for (int32_t b : s.blocks) ++pool->ref[b];
  s.ntok = prefix_tokens;
  pool->seqs.emplace(dst, std::move(s));
  return PKV_OK;
}

extern "C" pkv_status pkv_seq_free(pkv_pool* pool, int64_t seq) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end())
    return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld", (long long)seq);
  if (!pool->copies.empty())
    return fail(PKV_ERR_COPIES_PENDING, "%zu block copies pending: take them before a free",
                pool->copies.size() / 2);
  const auto& bl = it->second.blocks;
  const auto& oh = it->second.on_host;
  const bool sw = it->second.swapped;
  for (size_t i = 0; i < bl.size(); ++i) {
    if (sw && oh[i])
      pool->host_give(bl[i]);
    else
      pool->release(bl[i]);
  }
  if (sw) --pool->swapped;
  pool->seqs.erase(it);
  return PKV_OK;
}

extern "C" pkv_status pkv_seq_allocate_cached(pkv_pool* pool, int64_t seq, const int32_t* tokens,
                                              int32_t num_tokens, int32_t* cached_tokens) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (seq < 0) return fail(PKV_ERR_INVALID_ARG, "sequence ids are >= 0");
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens must be >= 0");
  if (num_tokens > 0 && !tokens) return fail(PKV_ERR_INVALID_ARG, "tokens is NULL");
  if (pool->seqs.count(seq)) return fail(PKV_ERR_SEQ_EXISTS, "sequence %lld exists", (long long)seq);
  const int32_t p = pool->block_size, full = num_tokens / p;
  // lookup: leading full blocks found in the cache
  std::vector<int32_t> found;
  int64_t parent = -1;
  for (int32_t i = 0; i < full; ++i) {
    const int32_t* t = tokens + (int64_t)i * p;
    const int32_t c = pool->find_cached(parent, t, pool->hash_of(parent, t));
    if (c < 0) break;
    found.push_back(c);
    parent = pool->entry_id[c];
  }
  const int32_t need = pool->blocks_for(num_tokens) - (int32_t)found.size();
  int32_t revive = 0;
  for (int32_t b : found) revive += pool->ref[b] == 0;
  if (need > pool->available() - revive)
    return fail(PKV_ERR_OUT_OF_BLOCKS, "block pool exhausted: need %d blocks, %lld free", need,
                (long long)(pool->available() - revive));
  pool->queries += full;
  pool->hits += (int64_t)found.size();
  for (int32_t b : found) {
    if (pool->in_lru[b]) pool->lru_remove(b);
    ++pool->ref[b];
  }
  pkv_pool::Seq s;
  s.blocks = found;
  pool->take(need, s.blocks);
  for (int32_t i = (int32_t)found.size(); i < full; ++i) {
    const int32_t b = s.blocks[i];
    const int32_t* t = tokens + (int64_t)i * p;
    if (pool->entry_tokens.empty())  // token ids are kept once the cache is used
      pool->entry_tokens.assign((size_t)pool->num_blocks * p, 0);
    std::memcpy(&pool->entry_tokens[(size_t)b * p], t, sizeof(int32_t) * (size_t)p);
    pool->entry_parent[b] = parent;
    pool->entry_hash[b] = pool->hash_of(parent, t);
    pool->entry_id[b] = pool->next_entry;
    pool->cache.emplace(pool->entry_hash[b], b);
    parent = pool->next_entry++;
  }
  s.ntok = num_tokens;
  pool->seqs.emplace(seq, std::move(s));
  if (cached_tokens) *cached_tokens = (int32_t)found.size() * p;
  return PKV_OK;
}

extern "C" pkv_status pkv_prefix_cache_stats(const pkv_pool* pool, int32_t* cached_blocks,
                                             int32_t* evictable_blocks, int64_t* hit_blocks,
                                             int64_t* queried_blocks) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (cached_blocks) *cached_blocks = (int32_t)pool->cache.size();
  if (evictable_blocks) *evictable_blocks = (int32_t)pool->lru.size();
  if (hit_blocks) *hit_blocks = pool->hits;
  if (queried_blocks) *queried_blocks = pool->queries;
  return PKV_OK;
}

extern "C" pkv_status pkv_seq_num_tokens(const pkv_pool* pool, int64_t seq, int32_t* num_tokens) {
  if (!pool || !num_tokens) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end())
    return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld", (long long)seq);
  *num_tokens = it->second.ntok;
  return PKV_OK;
}

extern "C" pkv_status pkv_seq_physical_address(const pkv_pool* pool, int64_t seq, int32_t token,
                                               int32_t* block, int32_t* offset) {
  if (!pool || !block || !offset) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  pkv_status st;
  const pkv_pool::Seq* sp = live_seq(pool, seq, &st);
  if (!sp) return st;
  if (token < 0 || token >= sp->ntok)
    return fail(PKV_ERR_INVALID_ARG, "token %d outside [0, %d)", token, sp->ntok);
  *block = sp->blocks[token / pool->block_size];
  *offset = token % pool->block_size;
  return PKV_OK;
}

extern "C" pkv_status pkv_pool_set_host_blocks(pkv_pool* pool, int32_t num_host_blocks) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (num_host_blocks < 0) return fail(PKV_ERR_INVALID_ARG, "num_host_blocks must be >= 0");
  if (pool->num_host - pool->host_count > 0)
    return fail(PKV_ERR_INVALID_ARG, "%d host blocks are in use",
                pool->num_host - pool->host_count);
  pool->num_host = num_host_blocks;
  pool->host_ring.resize(num_host_blocks);
  for (int32_t i = 0; i < num_host_blocks; ++i) pool->host_ring[i] = i;
  pool->host_head = 0;
  pool->host_count = num_host_blocks;
  return PKV_OK;
}

extern "C" pkv_status pkv_seq_swap_out(pkv_pool* pool, int64_t seq, int32_t* pairs,
                                       int32_t capacity, int32_t* num_pairs) {
  if (!pool || !num_pairs) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  pkv_status st;
  pkv_pool::Seq* sp = live_seq(pool, seq, &st);
  if (!sp) return st;
  if (!pool->copies.empty())
    return fail(PKV_ERR_COPIES_PENDING, "%zu block copies pending: take them before a swap",
                pool->copies.size() / 2);
  int32_t m = 0;
  for (int32_t b : sp->blocks) m += pool->ref[b] == 1;
  *num_pairs = m;
  if (m > pool->host_count)
    return fail(PKV_ERR_OUT_OF_BLOCKS, "host block pool exhausted: need %d blocks, %d free", m,
                pool->host_count);
  if (m > capacity) return fail(PKV_ERR_INVALID_ARG, "%d pairs, room for %d", m, capacity);
  if (m > 0 && !pairs) return fail(PKV_ERR_INVALID_ARG, "pairs is NULL");
  sp->on_host.assign(sp->blocks.size(), 0);
  int32_t k = 0;
  for (size_t i = 0; i < sp->blocks.size(); ++i) {
    const int32_t b = sp->blocks[i];
    if (pool->ref[b] != 1) continue;
    const int32_t h = pool->host_take();
    pairs[2 * k] = b;
    pairs[2 * k + 1] = h;
    ++k;
    pool->release(b);
    sp->blocks[i] = h;
    sp->on_host[i] = 1;
  }
  sp->swapped = true;
  ++pool->swapped;
  return PKV_OK;
}

extern "C" pkv_status pkv_seq_swap_in(pkv_pool* pool, int64_t seq, int32_t* pairs,
                                      int32_t capacity, int32_t* num_pairs) {
  if (!pool || !num_pairs) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end())
    return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld", (long long)seq);
  pkv_pool::Seq& s = it->second;
  if (!s.swapped)
    return fail(PKV_ERR_INVALID_ARG, "sequence %lld is not swapped out", (long long)seq);
  if (!pool->copies.empty())
    return fail(PKV_ERR_COPIES_PENDING, "%zu block copies pending: take them before a swap",
                pool->copies.size() / 2);
  int32_t m = 0;
  for (char f : s.on_host) m += f != 0;
  *num_pairs = m;
  if (m > pool->available())
    return fail(PKV_ERR_OUT_OF_BLOCKS, "block pool exhausted: need %d blocks, %lld free", m,
                (long long)pool->available());
  if (m > capacity) return fail(PKV_ERR_INVALID_ARG, "%d pairs, room for %d", m, capacity);
  if (m > 0 && !pairs) return fail(PKV_ERR_INVALID_ARG, "pairs is NULL");
  std::vector<int32_t> fresh;
  fresh.reserve(m);
  pool->take(m, fresh);
  int32_t k = 0;
  for (size_t i = 0; i < s.blocks.size(); ++i) {
    if (!s.on_host[i]) continue;
    const int32_t h = s.blocks[i], b = fresh[k];
    pairs[2 * k] = b;
    pairs[2 * k + 1] = h;
    ++k;
    pool->host_give(h);
    s.blocks[i] = b;
  }
  s.on_host.clear();
  s.swapped = false;
  --pool->swapped;
  return PKV_OK;
}

extern "C" pkv_status pkv_pool_swap_stats(const pkv_pool* pool, int32_t* swapped_seqs,
                                          int32_t* host_free, int32_t* host_used) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (swapped_seqs) *swapped_seqs = pool->swapped;
  if (host_free) *host_free = pool->host_count;
  if (host_used) *host_used = pool->num_host - pool->host_count;
  return PKV_OK;
}

extern "C" pkv_status pkv_pool_stats(const pkv_pool* pool, int32_t* free_blocks,
                                     int32_t* used_blocks, float* usage) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  const int32_t avail = (int32_t)pool->available();
  if (free_blocks) *free_blocks = avail;
  if (used_blocks) *used_blocks = pool->num_blocks - avail;
  if (usage) *usage = (float)(pool->num_blocks - avail) / (float)pool->num_blocks;
  return PKV_OK;
}

extern "C" pkv_status pkv_pool_num_copies(const pkv_pool* pool, int32_t* num_copies) {
  if (!pool || !num_copies) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  *num_copies = (int32_t)(pool->copies.size() / 2);
  return PKV_OK;
}

extern "C" pkv_status pkv_pool_take_copies(pkv_pool* pool, int32_t* pairs, int32_t capacity,
                                           int32_t* num_copies) {
  if (!pool || !num_copies) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  const int32_t n = (int32_t)(pool->copies.size() / 2);
  *num_copies = n;
  if (n > capacity)
    return fail(PKV_ERR_INVALID_ARG, "%d copies pending, room for %d", n, capacity);
  if (n > 0 && !pairs) return fail(PKV_ERR_INVALID_ARG, "pairs is NULL");
  std::copy(pool->copies.begin(), pool->copies.end(), pairs);
  pool->copies.clear();
  return PKV_OK;
}

extern "C" pkv_status pkv_block_refcount(const pkv_pool* pool, int32_t block, int32_t* refcount) {
  if (!pool || !refcount) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  if (block < 0 || block >= pool->num_blocks)
    return fail(PKV_ERR_INVALID_ARG, "block %d outside the pool", block);
  *refcount = pool->ref[block];
  return PKV_OK;
}

extern "C" pkv_status pkv_build_block_tables(const pkv_pool* pool, const int64_t* seqs, int32_t B,
                                             int32_t W, int32_t* tables, int32_t* ctx_lens) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (B < 0 || W < 1) return fail(PKV_ERR_INVALID_ARG, "need B >= 0 and W >= 1");
  if (B > 0 && (!seqs || !tables || !ctx_lens)) return fail(PKV_ERR_INVALID_ARG, "NULL buffer");
  std::vector<const pkv_pool::Seq*> rows(B);
  for (int32_t i = 0; i < B; ++i) {
    auto it = pool->seqs.find(seqs[i]);
    if (it == pool->seqs.end())
      return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld", (long long)seqs[i]);
    if (it->second.swapped)
      return fail(PKV_ERR_SEQ_SWAPPED, "sequence %lld is swapped out", (long long)seqs[i]);
    if ((int64_t)it->second.blocks.size() > W)
      return fail(PKV_ERR_INVALID_ARG, "sequence %lld needs %zu blocks, table width is %d",
                  (long long)seqs[i], it->second.blocks.size(), W);
    rows[i] = &it->second;
  }
  for (int32_t i = 0; i < B; ++i) {
    int32_t* row = tables + (int64_t)i * W;
    const auto& bl = rows[i]->blocks;
    std::copy(bl.begin(), bl.end(), row);
    std::fill(row + bl.size(), row + W, -1);
    ctx_lens[i] = rows[i]->ntok;
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_build_slot_mapping(const pkv_pool* pool, const int64_t* seqs,
                                             const int32_t* pos, int32_t N, int64_t* slots) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (N < 0) return fail(PKV_ERR_INVALID_ARG, "N must be >= 0");
  if (N > 0 && (!seqs || !pos || !slots)) return fail(PKV_ERR_INVALID_ARG, "NULL buffer");
  const int32_t p = pool->block_size;
  // validate everything first so that nothing is written on error
  for (int32_t i = 0; i < N; ++i) {
    if (pos[i] < 0) continue;
    auto it = pool->seqs.find(seqs[i]);
    if (it == pool->seqs.end())
      return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld", (long long)seqs[i]);
    if (it->second.swapped)
      return fail(PKV_ERR_SEQ_SWAPPED, "sequence %lld is swapped out", (long long)seqs[i]);
    if (pos[i] >= it->second.ntok)
      return fail(PKV_ERR_INVALID_ARG, "position %d past the length %d of sequence %lld", pos[i],
                  it->second.ntok, (long long)seqs[i]);
  }
  for (int32_t i = 0; i < N; ++i) {
    if (pos[i] < 0) {
      slots[i] = -1;
      continue;
    }
    const auto& s = pool->seqs.find(seqs[i])->second;
    slots[i] = (int64_t)s.blocks[pos[i] / p] * p + pos[i] % p;
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_check_slot_mapping(const int64_t* slots, int32_t N, int64_t num_slots) {
  if (N < 0 || (N > 0 && !slots)) return fail(PKV_ERR_INVALID_ARG, "bad slot array");
  std::unordered_set<int64_t> seen;
  seen.reserve((size_t)N * 2);
  for (int32_t i = 0; i < N; ++i) {
    int64_t s = slots[i];
    if (s == -1) continue;
    if (s < 0 || s >= num_slots)
      return fail(PKV_ERR_INVALID_ARG, "slot %lld at index %d outside [0, %lld)", (long long)s, i,
                  (long long)num_slots);
    if (!seen.insert(s).second)
      return fail(PKV_ERR_INVALID_ARG, "slot %lld repeats (index %d)", (long long)s, i);
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_check_block_appends(const int64_t* slots, int32_t N, int64_t num_slots,
                                              int32_t block_size) {
  pkv_status st = pkv_check_slot_mapping(slots, N, num_slots);
  if (st != PKV_OK) return st;
  if (block_size < 1) return fail(PKV_ERR_INVALID_ARG, "block_size must be >= 1");
  std::unordered_set<int64_t> blocks;
  blocks.reserve((size_t)N * 2);
  for (int32_t i = 0; i < N; ++i)
    if (slots[i] >= 0 && !blocks.insert(slots[i] / block_size).second)
      return fail(PKV_ERR_INVALID_ARG, "two slots in block %lld (index %d)",
                  (long long)(slots[i] / block_size), i);
  return PKV_OK;
}
