/*
 * pkv -- paged KV-cache decode attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every function is extern "C"; arguments are plain pointers and
 * sizes.  Functions that can fail return pkv_status; the message of the last
 * failure on the calling thread is pkv_last_error().  No exception or abort
 * crosses this boundary.
 *
 * Ownership.  The caller allocates every device buffer (pools, tables,
 * queries, outputs, workspace) and every stream; the library never
 * allocates or frees device memory and never synchronises a stream.  Device
 * entry points only enqueue work on the given stream (NULL = the default
 * stream); pointers must stay valid until that work has finished.  Host
 * pool objects are owned by the library between pkv_pool_create and
 * pkv_pool_destroy; one pool must not be used from two threads at once,
 * distinct pools are independent.
 *
 * The method (from the pages this library follows):
 *  - A KV cache is split into fixed-size blocks of 16 or 32 tokens drawn
 *    from one pre-allocated pool; a per-sequence block table maps logical
 *    block t / p to a physical block and token t sits at offset t % p
 *    ("Reducing LLM Inference Latency: KV Cache Quantization and
 *    PagedAttention in vLLM", section "PagedAttention: Solving VRAM
 *    Fragmentation").
 *  - The attention kernel receives the query, the block table, the pool and
 *    the number of tokens, and resolves each block's physical address on the
 *    fly ("KV Cache Compression & Paged Attention Deep Dive", section
 *    "Implementation Details: PagedAttention Kernel and Page Table").
 *  - K/V may be quantised before they are stored and dequantised during
 *    attention (same pages, sections "KV Cache Quantization: Shrinking the
 *    Memory Footprint" and "KV Cache Quantization: Squeezing 2-4x More
 *    Sequences").
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A HIP stream (hipStream_t has this exact type); NULL is the default stream. */
typedef struct ihipStream_t* pkv_stream_t;

/*
 * Status codes.  The pages' block manager raises an error when the pool of
 * free blocks is exhausted and names swapping or preemption as the way out
 * ("Reducing LLM Inference Latency: KV Cache Quantization and
 * PagedAttention in vLLM", section "PagedAttention: Solving VRAM
 * Fragmentation", block-manager emulation; section "Prefill Swapping and GPU
 * Thrashing"): that error is PKV_ERR_OUT_OF_BLOCKS, reported with nothing
 * changed so that the caller can swap or preempt and retry.  The other codes
 * are this library's own argument and state checks.
 */
typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,   /* bad pointer, size, dtype or shape; nothing was done */
  PKV_ERR_OUT_OF_BLOCKS = 2, /* the block pool cannot satisfy the request; state unchanged */
  PKV_ERR_NO_SUCH_SEQ = 3,
  PKV_ERR_SEQ_EXISTS = 4,
  PKV_ERR_UNSUPPORTED = 5,   /* valid request this library version does not implement */
  PKV_ERR_HIP = 6,           /* a HIP runtime call failed (launch error) */
  PKV_ERR_COPIES_PENDING = 7, /* fork, free or swap while block copies wait to be taken */
  PKV_ERR_SEQ_SWAPPED = 8     /* the sequence is swapped out (swap it in or free it) */
} pkv_status;

typedef enum pkv_dtype {
  PKV_F16 = 0,
  PKV_BF16 = 1,
  PKV_FP8_E4M3 = 2,      /* OCP E4M3 ("fn"), one fp32 absmax scale per (token, KV head) */
  PKV_INT4_ASYM_G32 = 3, /* 4-bit codes, fp16 (scale, zero) per (token, KV head, 32 channels) */
  PKV_F32 = 4,           /* io only: fp32 queries/outputs/new K,V (diagnostic) */
  PKV_FP8_E5M2 = 5,      /* OCP E5M2, one fp32 absmax scale per (token, KV head) */
  PKV_FP8_E4M3_BLOCK = 6 /* OCP E4M3, one fp32 absmax scale per (block, KV head) */
} pkv_dtype;

/*
 * One layer's cache.
 *   kv_dtype   : storage type (PKV_F16, PKV_BF16, PKV_FP8_E4M3, PKV_FP8_E5M2,
 *                PKV_FP8_E4M3_BLOCK, PKV_INT4_ASYM_G32)
 *   io_dtype   : type of Q, of the output and of the new K/V given to
 *                pkv_reshape_and_cache (PKV_F16, PKV_BF16 or PKV_F32).  A
 *                16-bit cache requires io_dtype == kv_dtype or PKV_F32.
 *   num_kv_heads, head_dim (64 or 128), block_size (16 or 32), num_blocks.
 *
 * Pool layouts.  Each pool is [num_blocks][Hkv][chunk]: one chunk holds one
 * block of p tokens for one KV head, and chunks are stored block-major, so
 * all heads of a block are adjacent.  Inside a chunk the order is the one
 * the decode kernel's matrix-core operands are consumed in, so that every
 * lane of a wave receives its share of 16 tokens with 16-byte loads.
 * Notation: token t of the block = 16 u + 4 g + r (unit u < p/16,
 * g < 4, r < 4); channel d = 32 c + 8 g' + e (e < 8) = 16 T + j (j < 16).
 *   F16/BF16  K: [p][D] 16-bit, token rows.
 *             V: [p/16][D/32][16 j][4 g][2 (T % 2)][4 r] 16-bit.
 *   FP8_E4M3, FP8_E5M2 and FP8_E4M3_BLOCK (same layouts; the block type
 *   keeps its block scale in each of the block's p scale entries)
 *             K: [p/16][D/64][16 j][4 g'][2 (c % 2)][8 e] u8 codes, token
 *                16 u + j of channel 32 c + 8 g' + e (with c / 2 the second
 *                index; each 1 KB run is one load).
 *             V: [p/16][D/64][16 j][4 g][4 (T % 4)][4 r] u8 codes.
 *             k_meta, v_meta: [p] fp32 scales.
 *   INT4      K: [p][4 g'][D/32 c][4 bytes] u8 (token rows); byte e/2
 *                holds channel 32 c + 8 g' + e, even e in the low nibble.
 *             V: [p/16][16 j][4 g][D/32 T/2] 32-bit words; the word holds
 *                tokens 4 g + r of channels 16 T + j for T = 2 (T/2) and
 *                2 (T/2) + 1, the nibble of token r of tile parity T % 2 at
 *                bit 16 (r % 2) + 8 (r / 2) + 4 (T % 2).
 *             k_meta, v_meta: [p/16][4 g][D/32 groups][4 r] (scale, zero)
 *                fp16 pairs, scale in the low half of each 32-bit word.
 * Every layout is a fixed permutation of the logical one (K [token][channel],
 * V [channel][token]) inside a chunk; pkv_reshape_and_cache writes it.
 */
typedef struct pkv_cache_desc {
  int32_t kv_dtype;
  int32_t io_dtype;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int64_t num_blocks;
} pkv_cache_desc;

typedef struct pkv_pool pkv_pool;

/* ----------------------------------------------------------------- errors */

/* Short text of a status code ("ok", "block pool exhausted", ...);
 * "unknown status" for any other value. */
const char* pkv_status_str(pkv_status s);
/* Message of the last failing call on this thread ("" if none). */
const char* pkv_last_error(void);
const char* pkv_version(void);

/* ------------------------------------------------------------------ sizes */

/*
 * KV-cache bytes of the closed form 2 * layers * kv_heads * head_dim *
 * seq_len * batch * P with P the bytes per element, given here as
 * bytes_x2 = 2 * P (4 for FP16/BF16, 2 for FP8/INT8, 1 for INT4) so the
 * result stays an integer ("Reducing LLM Inference Latency...", section
 * "Understanding the Bottleneck"; "Optimizing KV-Cache Memory Footprint in
 * High-Throughput LLM Serving", section 2).  Scales and zero points are not
 * included.  Returns -1 on negative arguments or overflow.
 */
int64_t pkv_kv_bytes(int64_t layers, int64_t kv_heads, int64_t head_dim, int64_t seq_len,
                     int64_t batch, int64_t bytes_x2);

/* Bytes of one K (or V) pool and of one K (or V) metadata array for `desc`
 * (metadata is 0 for 16-bit caches).  INVALID_ARG on a bad descriptor. */
pkv_status pkv_cache_bytes(const pkv_cache_desc* desc, size_t* pool_bytes, size_t* meta_bytes);

/* --------------------------------------------------- block pool (host) */

/*
 * Host-side block allocator ("Reducing LLM Inference Latency...", section
 * "PagedAttention: Solving VRAM Fragmentation", block-manager emulation;
 * appending follows "Optimizing LLM Inference: KV Cache and PagedAttention
 * Explained", section "PagedAttention: Operating Systems to the Rescue").
 * The free list is FIFO: blocks are taken from its front and returned to its
 * back.  free_order (num_blocks entries, a permutation of 0..num_blocks-1)
 * is its initial order; NULL means 0, 1, ..., num_blocks-1.  Every
 * operation is all-or-nothing: on error nothing changes.
 */
pkv_status pkv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                           pkv_pool** out);
void pkv_pool_destroy(pkv_pool* pool);

/* New sequence `seq` (>= 0) holding num_tokens tokens: ceil(num_tokens/p)
 * blocks.  SEQ_EXISTS if seq is live; OUT_OF_BLOCKS if the pool is short. */
pkv_status pkv_seq_allocate(pkv_pool* pool, int64_t seq, int32_t num_tokens);

/* Append num_tokens tokens; a block is taken only when the token count is a
 * multiple of p.  out_slots (may be NULL) receives the num_tokens new slots
 * (physical block * p + offset).
 * Copy-on-write: if the sequence's last block is partly filled and another
 * sequence's table also points at it, the append first takes a fresh block
 * from the front of the free list (before any block it grows by), moves its
 * table entry there, drops one reference to the old block and records the
 * copy (old, new); see pkv_pool_take_copies.  That block counts toward
 * OUT_OF_BLOCKS like any other. */
pkv_status pkv_seq_append(pkv_pool* pool, int64_t seq, int32_t num_tokens, int64_t* out_slots);

/* Append num_tokens tokens to each of B sequences (one decode step of a
 * batch when num_tokens is 1), with the same result as B pkv_seq_append
 * calls in order (copies included).  out_slots (may be NULL) receives B *
 * num_tokens slots, sequence-major.  All-or-nothing over the whole batch:
 * if the pool cannot hold every new block, nothing changes. */
pkv_status pkv_seq_append_batch(pkv_pool* pool, const int64_t* seqs, int32_t B,
                                int32_t num_tokens, int64_t* out_slots);

/* New sequence dst sharing the first prefix_tokens tokens of src ("KV Cache
 * Compression & Paged Attention Deep Dive", section "PagedAttention:
 * Operating System-Inspired Memory Management": sequences with a common
 * prefix point at the same physical blocks; copy-on-write makes forks such
 * as beam-search candidates safe).  0 <= prefix_tokens <= src's length
 * (INVALID_ARG otherwise); dst shares the ceil(prefix_tokens / p) blocks
 * holding the prefix, each gaining a reference.  A partly filled last block
 * is copied by whichever sharer writes into it first (pkv_seq_append).
 * COPIES_PENDING while copies wait to be taken. */
pkv_status pkv_seq_fork(pkv_pool* pool, int64_t src, int64_t dst, int32_t prefix_tokens);

/* Drop a sequence; each of its blocks loses a reference and returns to the
 * back of the free list (in table order) when none is left ("Reducing LLM
 * Inference Latency...", section "PagedAttention: Solving VRAM
 * Fragmentation": the block manager's free returns a sequence's blocks to
 * the free list; "KV Cache Compression & Paged Attention Deep Dive",
 * section "PagedAttention: Operating System-Inspired Memory Management for
 * LLMs": a finished sequence's pages are freed one by one and can go to any
 * new sequence).  NO_SUCH_SEQ for an unknown sequence.
 * COPIES_PENDING while copies wait to be taken. */
pkv_status pkv_seq_free(pkv_pool* pool, int64_t seq);

/* Number of block copies recorded by copy-on-write and not yet taken. */
pkv_status pkv_pool_num_copies(const pkv_pool* pool, int32_t* num_copies);

/*
 * Take the pending copies: pairs [capacity][2] int32 (host) receives
 * (source block, destination block) in the order they were recorded, and
 * *num_copies their number; the pool forgets them.  If capacity is too
 * small, INVALID_ARG with *num_copies set and nothing taken.  The caller
 * runs them with pkv_copy_blocks on the device before the tokens of the
 * appends that recorded them are written.  The pairs of one take are
 * disjoint (no block is both a source and a destination, no destination
 * repeats), because fork and free are refused while copies are pending.
 */
pkv_status pkv_pool_take_copies(pkv_pool* pool, int32_t* pairs, int32_t capacity,
                                int32_t* num_copies);

/*
 * Automatic prefix caching ("KV Cache Compression & Paged Attention Deep
 * Dive", section "Implementation Details: PagedAttention Kernel and Page
 * Table": the prefix is hashed and a cached block is looked up before new
 * blocks are allocated; "KV Cache Optimization: 3x Faster LLM Inference on
 * 24GB VRAM", section "Prefix Caching: The Hidden Multiplier").  New
 * sequence `seq` for a prompt of num_tokens token ids (host int32).  Its
 * leading full blocks are looked up in order under the exact key (the cache
 * entry of the block before, the block's p token ids) and every one found
 * is shared (a reference more) until the first miss; the remaining blocks
 * are taken as by pkv_seq_allocate, and each new full block of the prompt
 * is entered in the cache.  *cached_tokens (may be NULL) receives the
 * number of leading tokens whose K/V are already in the pool (a multiple of
 * p): the caller computes and writes only the tokens after them.
 * A cached block whose last reference is dropped is not freed: it stays
 * findable and becomes evictable; every allocation takes blocks from the
 * free list first, then evicts the least recently released cached block
 * (its cache entry is removed, and entries that followed it can no longer
 * be reached).  pkv_pool_stats counts evictable blocks as free.  Blocks
 * filled by later appends are not cached.  SEQ_EXISTS, OUT_OF_BLOCKS
 * (nothing changes) as pkv_seq_allocate.
 */
pkv_status pkv_seq_allocate_cached(pkv_pool* pool, int64_t seq, const int32_t* tokens,
                                   int32_t num_tokens, int32_t* cached_tokens);

/* Prefix cache counters: cached blocks (findable), of which evictable (no
 * reference), full prompt blocks found by lookups, and full prompt blocks
 * looked up since the pool was created.  Any output may be NULL. */
pkv_status pkv_prefix_cache_stats(const pkv_pool* pool, int32_t* cached_blocks,
                                  int32_t* evictable_blocks, int64_t* hit_blocks,
                                  int64_t* queried_blocks);

/* Tokens held by `seq` (the token count of the pages' BlockTable,
 * "Optimizing LLM Inference: KV Cache and PagedAttention Explained", section
 * "PagedAttention: Operating Systems to the Rescue"). */
pkv_status pkv_seq_num_tokens(const pkv_pool* pool, int64_t seq, int32_t* num_tokens);

/* (physical block, offset) of token `token` of `seq`: block = the table's
 * entry t / p, offset = t % p ("Reducing LLM Inference Latency...", section
 * "PagedAttention: Solving VRAM Fragmentation", the block manager's
 * get_physical_address; its worked example maps token 34 of a fresh
 * 35-token sequence to block 2, offset 2).  INVALID_ARG if token is outside
 * [0, length); NO_SUCH_SEQ; SEQ_SWAPPED for a swapped-out sequence. */
pkv_status pkv_seq_physical_address(const pkv_pool* pool, int64_t seq, int32_t token,
                                    int32_t* block, int32_t* offset);

/*
 * Swapping ("Reducing LLM Inference Latency...", section "Prefill Swapping
 * and GPU Thrashing": when the pool is exhausted, KV pages move to host
 * memory over PCIe; the number of swapped requests is a monitored metric).
 * pkv_pool_set_host_blocks gives the pool num_host_blocks host blocks
 * (ids 0..n-1 in a FIFO); INVALID_ARG while any is in use.
 *
 * pkv_seq_swap_out moves every block `seq` holds alone (reference count 1)
 * to a host block taken from the front of the host FIFO, in table order,
 * and releases the device block (a cached one becomes evictable); blocks
 * another table also points at stay on the device with their reference.
 * pairs [capacity][2] (host) receives the (device block, host block) pairs,
 * *num_pairs their number.  The caller moves the data with pkv_swap_blocks
 * (to_host = 1) before any later write to the pool.  A swapped sequence can
 * only be swapped in or freed (others: SEQ_SWAPPED).
 * pkv_seq_swap_in takes a device block for each host entry, in table
 * order (free list first, then eviction), returns the host blocks to the
 * back of the host FIFO and gives the pairs the same way; the caller moves
 * the data (to_host = 0) before the sequence is read.
 * Both are all-or-nothing: OUT_OF_BLOCKS if the host (out) or device (in)
 * side is short, INVALID_ARG with *num_pairs set if capacity is too small,
 * COPIES_PENDING while copy-on-write copies wait to be taken.
 */
pkv_status pkv_pool_set_host_blocks(pkv_pool* pool, int32_t num_host_blocks);
pkv_status pkv_seq_swap_out(pkv_pool* pool, int64_t seq, int32_t* pairs, int32_t capacity,
                            int32_t* num_pairs);
pkv_status pkv_seq_swap_in(pkv_pool* pool, int64_t seq, int32_t* pairs, int32_t capacity,
                           int32_t* num_pairs);
/* Swapped-out sequences, free and used host blocks.  Outputs may be NULL. */
pkv_status pkv_pool_swap_stats(const pkv_pool* pool, int32_t* swapped_seqs, int32_t* host_free,
                               int32_t* host_used);

/* Free and used block counts and the usage factor used / num_blocks, the
 * fraction of physical blocks allocated ("Reducing LLM Inference
 * Latency...", section "Monitoring and Alerting in Production": the
 * gpu_cache_usage_factor health metric).  Evictable cached blocks count as
 * free.  Any output may be NULL. */
pkv_status pkv_pool_stats(const pkv_pool* pool, int32_t* free_blocks, int32_t* used_blocks,
                          float* usage);

/* Reference count of one physical block (0 = free) ("KV Cache Compression
 * & Paged Attention Deep Dive", section "Implementation Details:
 * PagedAttention Kernel and Page Table": page-table entries carry reference
 * counts for copy-on-write).  INVALID_ARG for an id outside the pool. */
pkv_status pkv_block_refcount(const pkv_pool* pool, int32_t block, int32_t* refcount);

/*
 * Block tables for B sequences into caller-owned host buffers:
 * tables [B][W] int32 (unused entries -1), ctx_lens [B] int32 (the token
 * counts).  The attention kernel is given the block table and the pool
 * instead of a contiguous cache tensor ("Reducing LLM Inference
 * Latency...", section "PagedAttention: Solving VRAM Fragmentation", the
 * paragraph after the block manager); each entry is a 32-bit physical
 * block id and the table lives in GPU memory, updated by the scheduler
 * ("KV Cache Compression & Paged Attention Deep Dive", section
 * "Implementation Details: PagedAttention Kernel and Page Table"): the
 * caller copies these buffers to the device.  INVALID_ARG if a sequence
 * needs more than W blocks; NO_SUCH_SEQ; SEQ_SWAPPED.
 */
pkv_status pkv_build_block_tables(const pkv_pool* pool, const int64_t* seqs, int32_t B,
                                  int32_t W, int32_t* tables, int32_t* ctx_lens);

/* Slots of (seqs[i], pos[i]) into slots [N] int64: slot = physical block
 * * p + offset, with (block, offset) as pkv_seq_physical_address gives them
 * ("Reducing LLM Inference Latency...", section "PagedAttention: Solving
 * VRAM Fragmentation", get_physical_address), i.e. the flat token index in
 * the pool that pkv_reshape_and_cache writes.  pos[i] < 0 gives -1 (skip).
 * INVALID_ARG if a position is past the sequence's length. */
pkv_status pkv_build_slot_mapping(const pkv_pool* pool, const int64_t* seqs, const int32_t* pos,
                                  int32_t N, int64_t* slots);

/* Host check of a slot mapping (a guard of this library, not a step of the
 * method): every slot is -1 or in [0, num_slots) and no non-negative slot
 * repeats (a repeat would race on the device).  pkv_reshape_and_cache does
 * not run it itself: slot mappings normally live in device memory, and
 * checking them there would cost a synchronisation per call. */
pkv_status pkv_check_slot_mapping(const int64_t* slots, int32_t N, int64_t num_slots);

/* The same, and no two slots in one block of block_size tokens (the rule of
 * one call of pkv_reshape_and_cache for PKV_FP8_E4M3_BLOCK caches). */
pkv_status pkv_check_block_appends(const int64_t* slots, int32_t N, int64_t num_slots,
                                   int32_t block_size);

/* ------------------------------------------------------- device kernels */

/*
 * Write N new tokens' K and V into the cache, quantising on the way for
 * FP8/INT4 caches ("Reducing LLM Inference Latency...", sections "KV Cache
 * Quantization: Shrinking the Memory Footprint" -- quantise before storing
 * -- and "Block-Wise Scaling Factors" -- absmax / 448 scale, here one per
 * (token, KV head); E5M2 (section "FP8 (Float8) vs INT8 / INT4
 * Quantization") the same with its largest finite value 57344 in place of
 * 448; INT4 per 32 channels: s = fp16((max - min) / 15),
 * z = fp16(min), code = clamp(rne((x - z) / s), 0, 15), 0 when s == 0).
 *
 *   k, v          device [N][Hkv][D] in desc->io_dtype
 *   slot_mapping  device [N] int64; -1 skips the token; slots outside
 *                 [0, num_blocks * p) are skipped by the kernel (validate on
 *                 the host with pkv_check_slot_mapping)
 *   k_pool, v_pool, k_meta, v_meta   device, layouts as in pkv_cache_desc
 *                 (metas NULL for 16-bit caches)
 * Asynchronous on `stream`.  Slots must be distinct within one call.
 */
/*
 * PKV_FP8_E4M3_BLOCK follows the page's block-wise scaling (section
 * "Block-Wise Scaling Factors": one absmax scale for a block's tokens) for
 * tokens arriving one at a time: a token at offset 0 opens its block with
 * its own scale max(absmax / 448, 1e-12); a token at a later offset raises
 * the block scale to max(block scale, its own) and, if it grows, first
 * requantises the block's tokens at offsets below it from their codes:
 * code' = e4m3(fp32(fp32(code * s_old) / s_new)) (NaN codes kept).  The
 * scale is written to every entry of the block's metadata.  One call may
 * write at most one token per block (decode steps do; a prompt is written
 * in rounds of one offset), and a block's tokens must arrive in offset
 * order (appends do); pkv_check_block_appends checks the first rule.
 */
pkv_status pkv_reshape_and_cache(const pkv_cache_desc* desc, const void* k, const void* v,
                                 int32_t N, const int64_t* slot_mapping, void* k_pool,
                                 void* v_pool, void* k_meta, void* v_meta, pkv_stream_t stream);

/*
 * Copy-on-write on the device: for each of the n (source, destination)
 * physical block pairs in `pairs` (device [n][2] int32, as taken by
 * pkv_pool_take_copies), every KV head's chunk of the source block replaces
 * the destination's in k_pool and v_pool, and so do its scales or (scale,
 * zero) pairs in k_meta and v_meta for quantised caches ("KV Cache
 * Compression & Paged Attention Deep Dive", copy-on-write of shared
 * blocks).  The chunk layouts are the ones in pkv_cache_desc, copied
 * byte for byte.
 *   k_pool, v_pool, k_meta, v_meta  device, 16-byte aligned (metas NULL for
 *                 16-bit caches)
 * Pairs with an id outside [0, num_blocks) or with source == destination
 * are skipped.  The pairs of one call must be disjoint (no block both a
 * source and a destination, no repeated destination): they are copied in
 * parallel.  Asynchronous on `stream`.
 */
pkv_status pkv_copy_blocks(const pkv_cache_desc* desc, const int32_t* pairs, int32_t n,
                           void* k_pool, void* v_pool, void* k_meta, void* v_meta,
                           pkv_stream_t stream);

/* Bytes of one block in a host pool for pkv_swap_blocks: the block's K
 * pool chunks of all KV heads, then its V pool chunks, then (quantised
 * caches) its K and V metadata, each exactly as in the device arrays.
 * 0 on a bad descriptor. */
size_t pkv_swap_block_bytes(const pkv_cache_desc* desc);

/*
 * Move whole blocks between the device arrays and a host pool
 * ([num_host_blocks][pkv_swap_block_bytes] bytes, pinned host memory for
 * asynchronous copies) for the (device block, host block) pairs [n][2]
 * (host memory) given by pkv_seq_swap_out / pkv_seq_swap_in; to_host 1
 * copies device -> host, 0 host -> device.  A kernel gathers the device
 * blocks into `staging` (device, staging_bytes >= one block, 16-byte
 * aligned) in pair order, and hipMemcpyAsync moves every run of
 * consecutive host blocks in one copy (or the reverse, then a scatter);
 * more pairs than staging holds are moved in rounds, ordered on `stream`.
 * Ids are checked on the host: INVALID_ARG for an id out of range or a
 * repeated device or host block.  Asynchronous on `stream`.
 */
pkv_status pkv_swap_blocks(const pkv_cache_desc* desc, const int32_t* pairs, int32_t n,
                           int32_t to_host, void* k_pool, void* v_pool, void* k_meta,
                           void* v_meta, void* host_pool, int64_t num_host_blocks, void* staging,
                           size_t staging_bytes, pkv_stream_t stream);

typedef struct pkv_decode_args {
  void* out;                   /* device [B][Hq][D] in io_dtype */
  const void* q;               /* device [B][Hq][D] in io_dtype */
  const void* k_pool;          /* device pools and metadata as in pkv_cache_desc */
  const void* v_pool;
  const void* k_meta;
  const void* v_meta;
  const int32_t* block_tables; /* device [B][W] */
  const int32_t* ctx_lens;     /* device [B]: tokens per sequence, including the new one */
  int32_t num_seqs;            /* B */
  int32_t num_q_heads;         /* Hq, a multiple of Hkv with Hq / Hkv <= 16 */
  int32_t table_width;         /* W */
  int32_t max_ctx;             /* upper bound of ctx_lens, <= W * p (longer contexts are cut here) */
  float scale;                 /* softmax scale, normally 1 / sqrt(D) */
  int32_t partition;           /* 0: balanced split (below); -1: one pass per sequence;
                                  > 0: tokens per split-K partition, a multiple of p */
  void* workspace;             /* device scratch for split-K partial results */
  size_t workspace_bytes;
  int32_t flags;               /* 0 or an OR of PKV_DECODE_SKIP_MERGE, PKV_DECODE_OUT_F32 */
  int32_t* bad_blocks;         /* optional device int32 (NULL: not reported): the kernels add
                                  the number of 16-token units whose block-table entry lies
                                  outside [0, num_blocks); the caller zeroes it beforehand and
                                  reads it after the stream work (4-byte aligned) */
} pkv_decode_args;

/*
 * How the work is split.  partition > 0: each (sequence, KV head) is cut
 * into partitions of that many tokens, one workgroup each.  partition -1:
 * one workgroup per (sequence, KV head).  partition 0 (batches of up to
 * 4096 sequences; larger ones use partitions of 32 blocks): the balanced
 * split.  Every (sequence, KV head) is a run of ceil(n / 16) units of 16
 * tokens, the runs are laid end to end (sequence-major, then KV head), and
 * each of the NW waves of a grid sized to the GPU's resident workgroups
 * takes an equal share of that line, NW being at most (total units) / 8.
 * A run cut by share boundaries leaves one part per wave that touches it.
 *
 * Workspace bytes pkv_paged_decode needs for these sizes (0 for one pass).
 * Layout in 4-byte words, with P parts per (sequence, query head) and
 * nm = B * Hq * P; P = ceil(max_ctx / partition) for partition > 0 and
 * ceil(max_ctx / 16) / 8 + 2 for the balanced split:
 *   balanced split only: B * Hkv int32 part counts, one per (sequence, KV
 *   head) run (0 for an empty sequence), padded to a multiple of 4 words;
 *   then
 *   m [B][Hq][P], l [B][Hq][P] (nm words each), and acc [B][Hq][P][D]
 *   starting at the next multiple of 4 words.
 * Part k of a (sequence, head) split into several holds a reference score
 * m (units of the scaled score; at most the part's largest score and at
 * least that score minus 8 ln 2), the sum l = sum exp(s - m) and the
 * unnormalised acc = sum exp(s - m) v.  Returns 0 for invalid arguments.
 */
size_t pkv_decode_workspace_bytes(const pkv_cache_desc* desc, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t max_ctx, int32_t partition);

/* Tokens per partition the call would use for these sizes: 0 for the
 * balanced split, -1 for one pass, else the partition (a batch too large
 * for the balanced split resolves 0 to 32 blocks). */
int32_t pkv_decode_partition(const pkv_cache_desc* desc, int32_t num_seqs, int32_t num_q_heads,
                             int32_t max_ctx, int32_t partition);

/* pkv_decode_args.flags */
#define PKV_DECODE_SKIP_MERGE 1 /* leave split partitions in the workspace; run
                                   pkv_lse_reduce afterwards on the same args */
#define PKV_DECODE_OUT_F32 2    /* out is fp32 [B][Hq][D]; every step before the final
                                   store is that of the io type (queries, operands,
                                   accumulation), so fp32 output measures the arithmetic
                                   without the output rounding.  pkv_lse_reduce must be
                                   given the same flag */

/*
 * Paged decode attention: for each sequence b and query head h (KV head
 * h / (Hq / Hkv)), out[b][h] = softmax(scale * q[b][h] . K^T) V over tokens
 * 0..ctx_lens[b]-1, K/V gathered through block_tables[b] and dequantised
 * on the fly ("KV Cache Optimization: 3x Faster LLM Inference on 24GB VRAM",
 * section "Why Standard Approaches Fail", for the formula and grouped-query
 * heads).  Scores and the softmax are fp32; P.V accumulates in fp32.  With
 * split runs or partitions, each part's (m, l, acc) goes to the workspace and a
 * second kernel merges them: M = max m_k, out = sum e^(m_k - M) acc_k /
 * sum e^(m_k - M) l_k.  A sequence with ctx_lens[b] <= 0 gets zeros.  Block
 * table entries outside [0, num_blocks) are never dereferenced: their
 * tokens are left out of the softmax, and every 16-token unit this happens
 * to is counted in *bad_blocks when that pointer is given.  Errors
 * (nothing is enqueued): INVALID_ARG for a bad descriptor, NULL or
 * misaligned pointers (16 bytes for q, out, pools, metadata and workspace),
 * Hq not a multiple of Hkv, max_ctx outside [0, W * p], a non-positive or
 * non-finite scale, a partition that is not -1, 0 or a multiple of p, a
 * workspace smaller than pkv_decode_workspace_bytes, unknown flags;
 * UNSUPPORTED for groups over 16 heads; HIP_ERROR for a failed launch.
 */
pkv_status pkv_paged_decode(const pkv_cache_desc* desc, const pkv_decode_args* args,
                            pkv_stream_t stream);

/*
 * The merge step alone: for every (sequence, query head) whose context was
 * split into several parts, combine the parts' (m, l, acc) left in the
 * workspace by pkv_paged_decode with PKV_DECODE_SKIP_MERGE into the output
 * (log-sum-exp merge as above).  Same arguments as that call; a no-op when
 * the call needed a single partition.  (Empty sequences get their zeros
 * from pkv_paged_decode itself.)
 */
pkv_status pkv_lse_reduce(const pkv_cache_desc* desc, const pkv_decode_args* args,
                          pkv_stream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * decode as pkv_paged_decode, with its split-K partial results in a
 * device array owned by the library (64 MiB on each GPU it runs on, held
 * from the library's load until the process ends) instead of a caller
 * workspace.  args->workspace must be NULL and workspace_bytes 0;
 * PKV_DECODE_SKIP_MERGE is refused (the merge runs in this call).  Sizes
 * whose pkv_decode_workspace_bytes exceeds 64 MiB are refused with
 * INVALID_ARG before anything is enqueued.  Nothing is allocated or freed.
 * Every call on one GPU shares that GPU's array and overwrites what it
 * needs before reading it (no clearing is needed); calls that overlap on
 * one GPU (several streams or threads) race on it and must be serialised
 * by the caller.
 */
pkv_status pkv_paged_decode_noalloc(const pkv_cache_desc* desc, const pkv_decode_args* args,
                                    pkv_stream_t stream);

/* ------------------------------------------------- measurement helpers */

/* Overwrite `bytes` (multiple of 16) of device memory with a pattern; used
 * to evict caches between timed launches. */
pkv_status pkv_bench_flush(void* buf, size_t bytes, pkv_stream_t stream);

/* Read `bytes` (multiple of 16) of device memory with 128-bit loads and
 * write one 32-bit checksum per workgroup to sink (>= 8192 entries):
 * the achievable streaming-read bandwidth.  Four workgroups of four waves
 * per compute unit; each wave reads its own range of 1 KB runs (one load
 * instruction each) with four loads in flight. */
pkv_status pkv_bench_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                                 pkv_stream_t stream);

/* Plain 128-bit copy of `bytes` (multiple of 16) from `src` to `dst`, both
 * 16-byte aligned device addresses: a kernel of known traffic for calibrating
 * hardware byte counters.  `src` may also be the device address of pinned
 * host memory (hipHostGetDevicePointer); the benchmark uploads each step's
 * slots, lengths and block tables this way, in the launching stream. */
pkv_status pkv_bench_copy(void* dst, const void* src, size_t bytes, pkv_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
