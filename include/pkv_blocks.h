/*
 * pkv_blocks.h — host-side block manager with prefix caching (C ABI, part of libpkv).
 *
 * It decides which physical block of the pools (include/pkv.h) holds which tokens of which
 * sequence, and produces the int32 block tables and positions the append / decode / prefill
 * calls take. Host memory and host integers only: no HIP call, nothing on a GPU.
 *
 * Source: page "makarna/pkg/kvcache/paged_cache.go" — the PagedKVCache methods
 * ensureCapacityLocked, AppendToken, AllocateForTokens, Commit, Truncate, Free, SeqLen, and the
 * BlockPool calls they make (AllocateBlocks, FreeBlocks, FindCachedBlocks, TouchBlocks,
 * CacheBlocks, ComputeBlockHash(es)). The pool's own code is not on the page; its behaviour
 * here is read off those call sites:
 *   - a block has a reference count: a sequence holding it (owned or borrowed) counts once;
 *     freeing a sequence gives back one reference per block (the page frees borrowed and owned
 *     blocks alike, so borrowing must take a reference);
 *   - blocks whose count drops to 0 join the end of a free list; allocation takes blocks from
 *     its front (least recently freed first), all requested blocks or none;
 *   - a block is cached under the hash of its tokens when a Commit completes it; a cached block
 *     stays findable after it is freed, until allocation hands it out again (then its entry is
 *     dropped); a hash already cached keeps its first block;
 *   - a block's hash is FNV-1a (64-bit) over the previous block's hash (8 bytes, little-endian;
 *     absent for block 0) followed by the block's token ids (4 bytes each, little-endian), so
 *     equal hashes mean equal whole prefixes (up to 64-bit collisions). A prompt's last block
 *     may be partial: it is hashed over the tokens it has, and replaced by the full block's hash
 *     when pkv_seq_append_token completes it.
 *
 * One id space for every layer: the page keeps a block list per layer, but every layer's list
 * has the same length and the same borrowed / owned pattern (allocations succeed for all layers
 * or are rolled back). Here a block id names the same block index in every layer's pool, so a
 * sequence has one table row for all layers.
 *
 * Ownership: pkv_pool_create / pkv_seq_create return objects the caller destroys
 * (pkv_seq_destroy before pkv_pool_destroy). Arrays passed in are the caller's; the library
 * copies what it keeps. Errors: PKV_ERR_INVALID_ARG with pkv_last_error() set; a failed call
 * changes nothing. Thread safety: every call on a pool or on a sequence of it is serialised by
 * the pool's lock.
 */
#ifndef PKV_BLOCKS_H
#define PKV_BLOCKS_H

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_block_pool pkv_block_pool;
typedef struct pkv_seq_cache pkv_seq_cache;

typedef struct {
    int64_t num_blocks;
    int block_size;
    int64_t num_free;    /* blocks with no reference (cached or not) */
    int64_t num_cached;  /* blocks findable by hash */
    int64_t live_seqs;   /* sequences created on the pool and not destroyed */
} pkv_pool_info;

typedef struct {
    int num_computed;  /* tokens whose K/V are computed = position of the next token (SeqLen) */
    int num_written;   /* tokens written, may run ahead of num_computed within a step */
    int num_tokens;    /* token ids known (prompt + pkv_seq_append_token) */
    int num_blocks;    /* blocks held */
    int num_hashes;    /* block hashes known */
    int num_dropped;   /* leading blocks given back by pkv_seq_drop_before (ids -1) */
} pkv_seq_state;

/* A pool of num_blocks ids (1 .. 2^31-1), all free, none cached; block_size > 0 tokens. */
pkv_status pkv_pool_create(int64_t num_blocks, int block_size, pkv_block_pool** out);
/* Destroys the pool; INVALID_ARG while sequences created on it still exist. NULL is a no-op. */
pkv_status pkv_pool_destroy(pkv_block_pool* pool);
pkv_status pkv_pool_stats(pkv_block_pool* pool, pkv_pool_info* info);
/* Per-block state, each array (host) of num_blocks entries or NULL: reference counts, cached
 * flags, cached hashes (0 when not cached); free_order receives the free list front to back
 * (num_free entries). */
pkv_status pkv_pool_block_state(pkv_block_pool* pool, int32_t* refcounts, uint8_t* cached,
                                uint64_t* hashes, int32_t* free_order);

/* The block hash described above: tokens[0..n) chained to *parent (NULL for block 0). */
uint64_t pkv_block_hash(const int32_t* tokens, int n, const uint64_t* parent);

/* A sequence on `pool` with no blocks; max_seq_len 0 = no limit. */
pkv_status pkv_seq_create(pkv_block_pool* pool, int max_seq_len, pkv_seq_cache** out);
/* Frees the sequence's blocks and the sequence. NULL is a no-op. */
void pkv_seq_destroy(pkv_seq_cache* seq);

/*
 * Prompt admission (AllocateForTokens). The n prompt tokens are hashed block by block
 * (ceil(n / block_size) blocks); the longest run of leading blocks found in the cache is
 * borrowed (a reference each), blocks for the rest are allocated. The sequence's computed count
 * becomes the borrowed blocks' tokens, but at most n - 1: the last prompt token is always
 * computed again (its block may then be a borrowed one: the step rewrites the same values).
 * *cached_tokens (may be NULL) receives that count = the position the caller's prefill starts
 * at. Errors: n > max_seq_len, the sequence already holds blocks (free it first), not enough
 * free blocks (nothing is taken).
 */
pkv_status pkv_seq_allocate_for_tokens(pkv_seq_cache* seq, const int32_t* tokens, int n,
                                       int* cached_tokens);

/* Room for new_tokens more tokens after the computed ones (Append's capacity growth): blocks
 * are added until ceil((num_computed + new_tokens) / block_size) are held, all or none;
 * num_written advances to num_computed + new_tokens. *start_pos (may be NULL) receives
 * num_computed, the position of the first new token. Errors: past max_seq_len, not enough
 * free blocks. */
pkv_status pkv_seq_reserve(pkv_seq_cache* seq, int new_tokens, int* start_pos);

/* Token history (AppendToken): appends one id; when it completes a block, that block's hash is
 * computed (chained to the previous one) and a block is added if the sequence holds too few
 * (INVALID_ARG if none is free; the token and hash are recorded all the same, as on the page). */
pkv_status pkv_seq_append_token(pkv_seq_cache* seq, int32_t token);

/* Commit: num_computed += new_tokens; every block that this completes and whose hash is known is
 * cached under that hash. */
pkv_status pkv_seq_commit(pkv_seq_cache* seq, int new_tokens);

/* Truncate: rewinds num_computed (and num_written) to seq_len when it is smaller; blocks, token
 * ids and hashes are kept, as on the page (a rewind across a committed block leaves that block
 * cached under its old tokens' hash, so callers rewind only within the uncommitted tail).
 * INVALID_ARG if seq_len falls inside blocks given back by pkv_seq_drop_before. */
pkv_status pkv_seq_truncate(pkv_seq_cache* seq, int seq_len);

/* Free: gives back every block (one reference each), clears tokens, hashes and counts. */
pkv_status pkv_seq_free(pkv_seq_cache* seq);

pkv_status pkv_seq_info(pkv_seq_cache* seq, pkv_seq_state* state);

/* The sequence's block ids (-1 for blocks given back by pkv_seq_drop_before), owned flags (0 =
 * borrowed from the cache, or given back) and known hashes, into host arrays of `capacity`
 * entries (any may be NULL); INVALID_ARG if capacity is too small. */
pkv_status pkv_seq_blocks(pkv_seq_cache* seq, int32_t* block_ids, uint8_t* owned,
                          uint64_t* hashes, int capacity);

/* Sliding-window layers (page "soft3/glia/run/arch/decoder/forward.rs", forward_layer: a sliding layer keeps
 * a ring of cache_seq slots, so a token older than the window is overwritten and never read
 * again). In a paged pool the same reuse happens one block at a time: every block held whose
 * tokens all lie before first_pos (block index < first_pos / block_size) is given back (one
 * reference, as pkv_seq_free does) and its entry becomes -1; the table keeps its logical
 * indexing, so the kernels address tokens as before and pkv_fill_block_tables writes pad_block
 * for these entries. A decode step of window W attending L tokens reads from max(0, L - W) on,
 * so first_pos = num_computed + 1 - W is safe before the step. Hashes and token ids are kept
 * (later blocks' hashes chain through them). *num_dropped (may be NULL) receives the number of
 * leading entries given back so far. Errors: first_pos < 0 or > num_computed. */
pkv_status pkv_seq_drop_before(pkv_seq_cache* seq, int first_pos, int* num_dropped);

/* Batch tables for the paged calls: row b of block_tables (host int32 [B, max_blocks_per_seq])
 * = seqs[b]'s block ids, padded with pad_block (also in place of entries given back by
 * pkv_seq_drop_before); positions[b] (host int32 [B], may be NULL) = its num_computed.
 * INVALID_ARG if a sequence holds more than max_blocks_per_seq entries. */
pkv_status pkv_fill_block_tables(pkv_seq_cache* const* seqs, int B, int max_blocks_per_seq,
                                 int32_t pad_block, int32_t* block_tables, int32_t* positions);

/* One decode (or chunk) step for a batch, host side: for every sequence in order, when
 * window > 0, pkv_seq_drop_before(seqs[b], max(0, num_computed + 1 - window)) (the first key
 * the step's first new token attends under a sliding window of that many tokens), then
 * pkv_seq_reserve(seqs[b], new_tokens); then (block_tables non-NULL) pkv_fill_block_tables. On a
 * failed reserve the sequences before it keep their room; the error names the sequence. */
pkv_status pkv_batch_prepare(pkv_seq_cache* const* seqs, int B, int new_tokens, int window,
                             int max_blocks_per_seq, int32_t pad_block, int32_t* block_tables,
                             int32_t* positions);

/* After the step: for every sequence, its new_tokens token ids (host int32 [B, new_tokens], or
 * NULL to record none) through pkv_seq_append_token, then pkv_seq_commit(new_tokens). Stops at
 * the first failure. */
pkv_status pkv_batch_commit(pkv_seq_cache* const* seqs, int B, int new_tokens,
                            const int32_t* token_ids);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCKS_H */
