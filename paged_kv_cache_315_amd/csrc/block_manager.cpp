// block_manager.cpp — host-side block manager with prefix caching: the allocator that produces
// the block tables the paged kernels read. Declared in include/pkv_blocks.h. Plain C++ (no HIP):
// it only hands out integer block ids.
//
// Page "makarna/pkg/kvcache/paged_cache.go":
//   ensureCapacityLocked — grow the block list to the required count, all or nothing;
//   AppendToken          — extend the token history, hash each block as it completes, chained
//                          to the previous block's hash;
//   AllocateForTokens    — MaxSeqLen check, hash the prompt's blocks, take the longest cached
//                          prefix (borrowed blocks, reference taken), allocate the rest, undo on
//                          failure, never report the last token as cached;
//   Commit               — advance the computed count and cache the blocks it completed;
//   Truncate / Free      — rewind the computed count / give every block back.
// The pool's own code (BlockPool: AllocateBlocks, FreeBlocks, FindCachedBlocks, TouchBlocks,
// CacheBlocks, ComputeBlockHash) is not on the page; what it does here is read off those call
// sites: reference counts, a least-recently-freed order for reuse, a hash -> block map that
// keeps a freed block findable until it is handed out again.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv_blocks.h"

namespace pkv {
pkv_status fail(pkv_status st, const char* fmt, ...);  // pkv_api.hip: thread-local message
}

using pkv::fail;

namespace {

// FNV-1a, 64-bit (Fowler, Noll, Vo): h = offset basis; per byte h = (h ^ byte) * prime.
constexpr uint64_t kFnvBasis = 0xcbf29ce484222325ULL;
constexpr uint64_t kFnvPrime = 0x100000001b3ULL;

uint64_t fnv_bytes(uint64_t h, const unsigned char* p, size_t n) {
    for (size_t i = 0; i < n; ++i) h = (h ^ p[i]) * kFnvPrime;
    return h;
}

// Hash of one block of token ids: the parent's hash (8 bytes, little-endian) when there is a
// previous block, then each id as 4 little-endian bytes.
uint64_t block_hash(const int32_t* tok, int n, const uint64_t* parent) {
    uint64_t h = kFnvBasis;
    unsigned char buf[8];
    if (parent) {
        for (int i = 0; i < 8; ++i) buf[i] = (unsigned char)(*parent >> (8 * i));
        h = fnv_bytes(h, buf, 8);
    }
    for (int j = 0; j < n; ++j) {
        const uint32_t u = (uint32_t)tok[j];
        for (int i = 0; i < 4; ++i) buf[i] = (unsigned char)(u >> (8 * i));
        h = fnv_bytes(h, buf, 4);
    }
    return h;
}

}  // namespace

struct pkv_block_pool {
    int64_t num_blocks = 0;
    int block_size = 0;
    std::vector<int32_t> ref;        // references per block (sequences holding it)
    std::vector<uint64_t> hash;      // hash the block is cached under (valid when cached[i])
    std::vector<uint8_t> cached;
    std::vector<int64_t> prev, next; // free list (ref == 0), head is handed out first
    int64_t head = -1, tail = -1, nfree = 0;
    std::unordered_map<uint64_t, int64_t> by_hash;
    int64_t live_seqs = 0;
    std::mutex mu;

    void push_free(int64_t b) {
        prev[b] = tail;
        next[b] = -1;
        if (tail >= 0) next[tail] = b; else head = b;
        tail = b;
        ++nfree;
    }
    void unlink_free(int64_t b) {
        if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
        if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
        prev[b] = next[b] = -1;
        --nfree;
    }
    // n blocks from the head of the free list, or none at all
    bool allocate(int64_t n, std::vector<int32_t>& out) {
        if (n > nfree) return false;
        for (int64_t i = 0; i < n; ++i) {
            const int64_t b = head;
            unlink_free(b);
            if (cached[b]) {  // reused: its old contents are gone, so is its cache entry
                by_hash.erase(hash[b]);
                cached[b] = 0;
            }
            ref[b] = 1;
            out.push_back((int32_t)b);
        }
        return true;
    }
    void release(int32_t b) {
        if (ref[b] > 0 && --ref[b] == 0) push_free(b);
    }
    void touch(int32_t b) {
        if (ref[b] == 0) unlink_free(b);
        ++ref[b];
    }
    void cache(int32_t b, uint64_t h) {
        if (cached[b] || by_hash.count(h)) return;  // first block cached under a hash keeps it
        by_hash.emplace(h, b);
        hash[b] = h;
        cached[b] = 1;
    }
};

struct pkv_seq_cache {
    pkv_block_pool* pool = nullptr;
    int max_seq_len = 0;
    std::vector<int32_t> tokens;
    std::vector<int32_t> blocks;
    std::vector<uint8_t> owned;
    std::vector<uint64_t> hashes;
    int num_computed = 0;
    int num_written = 0;
    int dropped = 0;  // leading entries given back behind a sliding window (id -1 in `blocks`)

    // grow the block list to `required` blocks, all or nothing
    bool ensure_capacity(int64_t required) {
        if (required <= (int64_t)blocks.size()) return true;
        std::vector<int32_t> fresh;
        if (!pool->allocate(required - (int64_t)blocks.size(), fresh)) return false;
        blocks.insert(blocks.end(), fresh.begin(), fresh.end());
        owned.insert(owned.end(), fresh.size(), 1);
        return true;
    }
    void release_all() {
        for (int32_t b : blocks)
            if (b >= 0) pool->release(b);
        blocks.clear();
        owned.clear();
        dropped = 0;
    }
    // give back every held block whose tokens all lie before first_pos
    void drop_before(int first_pos) {
        const int bs = pool->block_size;
        const int upto = std::min((int)blocks.size(), first_pos / bs);
        for (; dropped < upto; ++dropped) {
            pool->release(blocks[dropped]);
            blocks[dropped] = -1;
            owned[dropped] = 0;
        }
    }
};

extern "C" {

pkv_status pkv_pool_create(int64_t num_blocks, int block_size, pkv_block_pool** out) {
    if (!out) return fail(PKV_ERR_INVALID_ARG, "pkv_pool_create: out is NULL");
    *out = nullptr;
    if (num_blocks <= 0 || num_blocks > INT32_MAX || block_size <= 0)
        return fail(PKV_ERR_INVALID_ARG,
                    "pkv_pool_create: num_blocks %lld (need 1..2^31-1), block_size %d (need > 0)",
                    (long long)num_blocks, block_size);
    pkv_block_pool* p = new (std::nothrow) pkv_block_pool;
    if (!p) return fail(PKV_ERR_INVALID_ARG, "pkv_pool_create: out of host memory");
    try {
        p->num_blocks = num_blocks;
        p->block_size = block_size;
        p->ref.assign(num_blocks, 0);
        p->hash.assign(num_blocks, 0);
        p->cached.assign(num_blocks, 0);
        p->prev.assign(num_blocks, -1);
        p->next.assign(num_blocks, -1);
    } catch (const std::bad_alloc&) {
        delete p;
        return fail(PKV_ERR_INVALID_ARG, "pkv_pool_create: out of host memory");
    }
    for (int64_t b = 0; b < num_blocks; ++b) p->push_free(b);
    *out = p;
    return PKV_OK;
}

pkv_status pkv_pool_destroy(pkv_block_pool* pool) {
    if (!pool) return PKV_OK;
    {
        std::lock_guard<std::mutex> lk(pool->mu);
        if (pool->live_seqs)
            return fail(PKV_ERR_INVALID_ARG, "pkv_pool_destroy: %lld sequences still use the pool",
                        (long long)pool->live_seqs);
    }
    delete pool;
    return PKV_OK;
}

pkv_status pkv_pool_stats(pkv_block_pool* pool, pkv_pool_info* info) {
    if (!pool || !info) return fail(PKV_ERR_INVALID_ARG, "pkv_pool_stats: NULL argument");
    std::lock_guard<std::mutex> lk(pool->mu);
    info->num_blocks = pool->num_blocks;
    info->block_size = pool->block_size;
    info->num_free = pool->nfree;
    info->num_cached = (int64_t)pool->by_hash.size();
    info->live_seqs = pool->live_seqs;
    return PKV_OK;
}

pkv_status pkv_pool_block_state(pkv_block_pool* pool, int32_t* refcounts, uint8_t* cached,
                                uint64_t* hashes, int32_t* free_order) {
    if (!pool) return fail(PKV_ERR_INVALID_ARG, "pkv_pool_block_state: pool is NULL");
    std::lock_guard<std::mutex> lk(pool->mu);
    for (int64_t b = 0; b < pool->num_blocks; ++b) {
        if (refcounts) refcounts[b] = pool->ref[b];
        if (cached) cached[b] = pool->cached[b];
        if (hashes) hashes[b] = pool->cached[b] ? pool->hash[b] : 0;
    }
    if (free_order) {
        int64_t i = 0;
        for (int64_t b = pool->head; b >= 0; b = pool->next[b]) free_order[i++] = (int32_t)b;
    }
    return PKV_OK;
}

uint64_t pkv_block_hash(const int32_t* tokens, int n, const uint64_t* parent) {
    return block_hash(tokens, n < 0 ? 0 : n, parent);
}

pkv_status pkv_seq_create(pkv_block_pool* pool, int max_seq_len, pkv_seq_cache** out) {
    if (!out) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_create: out is NULL");
    *out = nullptr;
    if (!pool) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_create: pool is NULL");
    if (max_seq_len < 0) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_create: max_seq_len < 0");
    pkv_seq_cache* s = new (std::nothrow) pkv_seq_cache;
    if (!s) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_create: out of host memory");
    s->pool = pool;
    s->max_seq_len = max_seq_len;
    std::lock_guard<std::mutex> lk(pool->mu);
    ++pool->live_seqs;
    *out = s;
    return PKV_OK;
}

void pkv_seq_destroy(pkv_seq_cache* s) {
    if (!s) return;
    {
        std::lock_guard<std::mutex> lk(s->pool->mu);
        s->release_all();
        --s->pool->live_seqs;
    }
    delete s;
}

pkv_status pkv_seq_allocate_for_tokens(pkv_seq_cache* s, const int32_t* tokens, int n,
                                       int* cached_tokens) {
    if (!s || (n > 0 && !tokens) || n < 0)
        return fail(PKV_ERR_INVALID_ARG, "pkv_seq_allocate_for_tokens: NULL sequence or tokens, or n < 0");
    if (cached_tokens) *cached_tokens = 0;
    pkv_block_pool* p = s->pool;
    std::lock_guard<std::mutex> lk(p->mu);
    if (!s->blocks.empty())
        return fail(PKV_ERR_INVALID_ARG,
                    "pkv_seq_allocate_for_tokens: the sequence already holds %zu blocks (free it first)",
                    s->blocks.size());
    if (s->max_seq_len > 0 && n > s->max_seq_len)
        return fail(PKV_ERR_INVALID_ARG, "pkv_seq_allocate_for_tokens: prompt length %d exceeds max_seq_len %d",
                    n, s->max_seq_len);
    const int bs = p->block_size;
    const int nblk = (n + bs - 1) / bs;
    std::vector<uint64_t> hashes(nblk);
    for (int i = 0; i < nblk; ++i) {
        const int len = (i + 1) * bs <= n ? bs : n - i * bs;
        hashes[i] = block_hash(tokens + (size_t)i * bs, len, i ? &hashes[i - 1] : nullptr);
    }
    // longest cached prefix: stop at the first block whose hash is not in the cache
    std::vector<int32_t> hit;
    for (int i = 0; i < nblk; ++i) {
        auto it = p->by_hash.find(hashes[i]);
        if (it == p->by_hash.end()) break;
        hit.push_back((int32_t)it->second);
    }
    for (int32_t b : hit) p->touch(b);
    std::vector<int32_t> fresh;
    if (!p->allocate(nblk - (int64_t)hit.size(), fresh)) {
        for (int32_t b : hit) p->release(b);  // undo the references just taken
        return fail(PKV_ERR_INVALID_ARG,
                    "pkv_seq_allocate_for_tokens: %lld free blocks, %lld needed",
                    (long long)p->nfree, (long long)(nblk - (int64_t)hit.size()));
    }
    s->tokens.assign(tokens, tokens + n);
    s->hashes = hashes;
    s->blocks = hit;
    s->owned.assign(hit.size(), 0);
    s->blocks.insert(s->blocks.end(), fresh.begin(), fresh.end());
    s->owned.insert(s->owned.end(), fresh.size(), 1);
    int computed = (int)hit.size() * bs;
    if (computed >= n) computed = n > 0 ? n - 1 : 0;  // the last token is always recomputed
    s->num_computed = s->num_written = computed;
    if (cached_tokens) *cached_tokens = computed;
    return PKV_OK;
}

pkv_status pkv_seq_reserve(pkv_seq_cache* s, int new_tokens, int* start_pos) {
    if (!s || new_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_reserve: NULL sequence or new_tokens < 0");
    std::lock_guard<std::mutex> lk(s->pool->mu);
    const int64_t end = (int64_t)s->num_computed + new_tokens;
    if (s->max_seq_len > 0 && end > s->max_seq_len)
        return fail(PKV_ERR_INVALID_ARG, "pkv_seq_reserve: %d + %d tokens exceed max_seq_len %d",
                    s->num_computed, new_tokens, s->max_seq_len);
    const int bs = s->pool->block_size;
    if (!s->ensure_capacity((end + bs - 1) / bs))
        return fail(PKV_ERR_INVALID_ARG, "pkv_seq_reserve: %lld free blocks, not enough for %lld tokens",
                    (long long)s->pool->nfree, (long long)end);
    if (start_pos) *start_pos = s->num_computed;
    if (s->num_written < end) s->num_written = (int)end;
    return PKV_OK;
}

pkv_status pkv_seq_append_token(pkv_seq_cache* s, int32_t token) {
    if (!s) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_append_token: sequence is NULL");
    pkv_block_pool* p = s->pool;
    std::lock_guard<std::mutex> lk(p->mu);
    s->tokens.push_back(token);
    const int bs = p->block_size;
    const size_t n = s->tokens.size();
    if (n % bs) return PKV_OK;
    const size_t blk = n / bs - 1;
    pkv_status st = PKV_OK;
    if (!s->ensure_capacity((int64_t)blk + 1))
        st = fail(PKV_ERR_INVALID_ARG, "pkv_seq_append_token: no free block for block %zu", blk);
    const uint64_t* parent = blk >= 1 && blk - 1 < s->hashes.size() ? &s->hashes[blk - 1] : nullptr;
    const uint64_t h = block_hash(s->tokens.data() + blk * bs, bs, parent);
    if (blk < s->hashes.size()) s->hashes[blk] = h;
    else {
        s->hashes.resize(blk, 0);
        s->hashes.push_back(h);
    }
    return st;
}

pkv_status pkv_seq_commit(pkv_seq_cache* s, int new_tokens) {
    if (!s || new_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_commit: NULL sequence or new_tokens < 0");
    pkv_block_pool* p = s->pool;
    std::lock_guard<std::mutex> lk(p->mu);
    const int old_computed = s->num_computed;
    s->num_computed += new_tokens;
    if (s->num_written < s->num_computed) s->num_written = s->num_computed;
    const int bs = p->block_size;
    size_t lo = old_computed / bs, hi = s->num_computed / bs;
    hi = std::min(hi, std::min(s->hashes.size(), s->blocks.size()));
    for (size_t i = lo; i < hi; ++i)
        if (s->blocks[i] >= 0) p->cache(s->blocks[i], s->hashes[i]);
    return PKV_OK;
}

pkv_status pkv_seq_truncate(pkv_seq_cache* s, int seq_len) {
    if (!s) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_truncate: sequence is NULL");
    std::lock_guard<std::mutex> lk(s->pool->mu);
    if (seq_len < 0) seq_len = 0;
    if (seq_len >= s->num_computed) return PKV_OK;
    if (seq_len < s->dropped * s->pool->block_size)
        return fail(PKV_ERR_INVALID_ARG, "pkv_seq_truncate: tokens before %d were given back (pkv_seq_drop_before)",
                    s->dropped * s->pool->block_size);
    s->num_computed = seq_len;
    if (s->num_written > s->num_computed) s->num_written = s->num_computed;
    return PKV_OK;
}

pkv_status pkv_seq_free(pkv_seq_cache* s) {
    if (!s) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_free: sequence is NULL");
    std::lock_guard<std::mutex> lk(s->pool->mu);
    s->release_all();
    s->tokens.clear();
    s->hashes.clear();
    s->num_computed = s->num_written = 0;
    return PKV_OK;
}

pkv_status pkv_seq_info(pkv_seq_cache* s, pkv_seq_state* st) {
    if (!s || !st) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_info: NULL argument");
    std::lock_guard<std::mutex> lk(s->pool->mu);
    st->num_computed = s->num_computed;
    st->num_written = s->num_written;
    st->num_tokens = (int)s->tokens.size();
    st->num_blocks = (int)s->blocks.size();
    st->num_hashes = (int)s->hashes.size();
    st->num_dropped = s->dropped;
    return PKV_OK;
}

pkv_status pkv_seq_blocks(pkv_seq_cache* s, int32_t* block_ids, uint8_t* owned, uint64_t* hashes,
                          int capacity) {
    if (!s || capacity < 0) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_blocks: NULL sequence or capacity < 0");
    std::lock_guard<std::mutex> lk(s->pool->mu);
    if (capacity < (int)s->blocks.size() || ((hashes && capacity < (int)s->hashes.size())))
        return fail(PKV_ERR_INVALID_ARG, "pkv_seq_blocks: capacity %d < %zu blocks / %zu hashes", capacity,
                    s->blocks.size(), s->hashes.size());
    for (size_t i = 0; i < s->blocks.size(); ++i) {
        if (block_ids) block_ids[i] = s->blocks[i];
        if (owned) owned[i] = s->owned[i];
    }
    if (hashes)
        for (size_t i = 0; i < s->hashes.size(); ++i) hashes[i] = s->hashes[i];
    return PKV_OK;
}

pkv_status pkv_fill_block_tables(pkv_seq_cache* const* seqs, int B, int max_blocks_per_seq,
                                 int32_t pad_block, int32_t* block_tables, int32_t* positions) {
    if (B < 0 || (B > 0 && (!seqs || !block_tables)) || max_blocks_per_seq <= 0)
        return fail(PKV_ERR_INVALID_ARG, "pkv_fill_block_tables: NULL argument, B < 0 or max_blocks_per_seq <= 0");
    for (int b = 0; b < B; ++b) {
        pkv_seq_cache* s = seqs[b];
        if (!s) return fail(PKV_ERR_INVALID_ARG, "pkv_fill_block_tables: sequence %d is NULL", b);
        std::lock_guard<std::mutex> lk(s->pool->mu);
        if ((int64_t)s->blocks.size() > max_blocks_per_seq)
            return fail(PKV_ERR_INVALID_ARG, "pkv_fill_block_tables: sequence %d holds %zu blocks > %d", b,
                        s->blocks.size(), max_blocks_per_seq);
        int32_t* row = block_tables + (size_t)b * max_blocks_per_seq;
        for (int i = 0; i < max_blocks_per_seq; ++i)
            row[i] = i < (int)s->blocks.size() && s->blocks[i] >= 0 ? s->blocks[i] : pad_block;
        if (positions) positions[b] = s->num_computed;
    }
    return PKV_OK;
}

pkv_status pkv_seq_drop_before(pkv_seq_cache* s, int first_pos, int* num_dropped) {
    if (!s) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_drop_before: sequence is NULL");
    std::lock_guard<std::mutex> lk(s->pool->mu);
    if (first_pos < 0 || first_pos > s->num_computed)
        return fail(PKV_ERR_INVALID_ARG, "pkv_seq_drop_before: first_pos %d outside [0, %d]", first_pos,
                    s->num_computed);
    s->drop_before(first_pos);
    if (num_dropped) *num_dropped = s->dropped;
    return PKV_OK;
}

pkv_status pkv_batch_prepare(pkv_seq_cache* const* seqs, int B, int new_tokens, int window,
                             int max_blocks_per_seq, int32_t pad_block, int32_t* block_tables,
                             int32_t* positions) {
    if (B < 0 || (B > 0 && !seqs) || new_tokens < 0 || window < 0)
        return fail(PKV_ERR_INVALID_ARG, "pkv_batch_prepare: NULL sequences, B < 0, new_tokens < 0 or window < 0");
    for (int b = 0; b < B; ++b) {
        if (window > 0 && seqs[b]) {
            pkv_seq_cache* s = seqs[b];
            std::lock_guard<std::mutex> lk(s->pool->mu);
            s->drop_before(std::max(0, s->num_computed + 1 - window));
        }
        const pkv_status st = pkv_seq_reserve(seqs[b], new_tokens, nullptr);
        if (st != PKV_OK) {
            char msg[512];
            snprintf(msg, sizeof(msg), "%s", pkv_last_error());
            return fail(st, "pkv_batch_prepare: sequence %d: %s", b, msg);
        }
    }
    if (!block_tables) return PKV_OK;
    return pkv_fill_block_tables(seqs, B, max_blocks_per_seq, pad_block, block_tables, positions);
}

pkv_status pkv_batch_commit(pkv_seq_cache* const* seqs, int B, int new_tokens,
                            const int32_t* token_ids) {
    if (B < 0 || (B > 0 && !seqs) || new_tokens < 0)
        return fail(PKV_ERR_INVALID_ARG, "pkv_batch_commit: NULL sequences, B < 0 or new_tokens < 0");
    for (int b = 0; b < B; ++b) {
        if (!seqs[b]) return fail(PKV_ERR_INVALID_ARG, "pkv_batch_commit: sequence %d is NULL", b);
        if (token_ids)
            for (int i = 0; i < new_tokens; ++i) {
                const pkv_status st = pkv_seq_append_token(seqs[b], token_ids[(size_t)b * new_tokens + i]);
                if (st != PKV_OK) return st;
            }
        const pkv_status st = pkv_seq_commit(seqs[b], new_tokens);
        if (st != PKV_OK) return st;
    }
    return PKV_OK;
}

}  // extern "C"
