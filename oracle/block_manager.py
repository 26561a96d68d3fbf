"""Oracle of the host block manager (test infrastructure: only tests/, smoke() and bench.py's
CPU baseline use anything under oracle/).

A plain, slow model in Python lists and dicts of what page "makarna/pkg/kvcache/paged_cache.go"
does with its blocks, written from the PagedKVCache methods in the page's order:
  AllocateForTokens — check MaxSeqLen; hash the prompt's blocks; find the cached prefix;
                      borrow it (take a reference); allocate the rest, undoing everything on
                      failure; report the cached tokens, never all of them;
  ensureCapacityLocked (Append's growth) — add blocks up to the required count, all or none;
  AppendToken       — record the token; when a block completes, hash it chained to the
                      previous block's hash and add a block if needed;
  Commit            — advance the computed count; cache the blocks it completed;
  Truncate, Free, SeqLen;
and, for sliding-window layers (page "soft3/glia/run/arch/decoder/forward.rs", forward_layer:
a sliding layer's cache is a ring whose slots older than the window are reused), drop_before
gives back the blocks whose tokens all precede the window's first key (entries become -1).
The pool (BlockPool) is not on the page; this model follows the reading its call sites
support: reference counts; a free list handed out front first and refilled at the back; a
hash -> block map; a freed cached block stays findable until it is handed out again; a hash
already cached keeps its first block. The block hash is FNV-1a 64 (Fowler, Noll, Vo) over the
parent hash's 8 little-endian bytes (block 0: none) and then each token id's 4 little-endian
bytes.

One id space serves every layer (the page's per-layer lists always agree in length and in which
blocks are borrowed), so each sequence has one block list.
"""
from __future__ import annotations

import struct

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


class BlockError(Exception):
    """A call the page answers with an error; the model's state is unchanged."""


def fnv1a64(data: bytes) -> int:
    h = FNV_OFFSET
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def block_hash(tokens, parent=None) -> int:
    data = b"" if parent is None else struct.pack("<Q", parent)
    for t in tokens:
        data += struct.pack("<i", t)
    return fnv1a64(data)


def prompt_hashes(tokens, block_size):
    """ComputeBlockHashes: one hash per block of the prompt, the last one possibly partial."""
    hashes = []
    for start in range(0, len(tokens), block_size):
        parent = hashes[-1] if hashes else None
        hashes.append(block_hash(tokens[start:start + block_size], parent))
    return hashes


class Pool:
    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks <= 0 or block_size <= 0:
            raise BlockError("pool sizes must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.ref = [0] * num_blocks
        self.free = list(range(num_blocks))   # front is handed out first
        self.cache = {}                        # hash -> block
        self.cached_hash = {}                  # block -> hash
        self.live_seqs = 0

    def allocate(self, n):
        if n > len(self.free):
            raise BlockError(f"{len(self.free)} free blocks, {n} needed")
        out = []
        for _ in range(n):
            b = self.free.pop(0)
            if b in self.cached_hash:          # reused block: drop its cache entry
                del self.cache[self.cached_hash.pop(b)]
            self.ref[b] = 1
            out.append(b)
        return out

    def release(self, blocks):
        for b in blocks:
            if b < 0:                          # already given back (drop_before)
                continue
            if self.ref[b] > 0:
                self.ref[b] -= 1
                if self.ref[b] == 0:
                    self.free.append(b)

    def find_cached(self, hashes):
        out = []
        for h in hashes:
            if h not in self.cache:
                break
            out.append(self.cache[h])
        return out

    def touch(self, blocks):
        for b in blocks:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1

    def cache_blocks(self, blocks, hashes):
        for b, h in zip(blocks, hashes):
            if b in self.cached_hash or h in self.cache:
                continue
            self.cache[h] = b
            self.cached_hash[b] = h


class Seq:
    def __init__(self, pool: Pool, max_seq_len: int = 0):
        self.pool = pool
        self.max_seq_len = max_seq_len
        self.tokens = []
        self.blocks = []
        self.owned = []
        self.hashes = []
        self.num_computed = 0
        self.num_written = 0
        self.dropped = 0
        pool.live_seqs += 1

    def allocate_for_tokens(self, tokens):
        bs = self.pool.block_size
        if self.blocks:
            raise BlockError("sequence already holds blocks")
        if self.max_seq_len > 0 and len(tokens) > self.max_seq_len:
            raise BlockError("prompt longer than max_seq_len")
        hashes = prompt_hashes(tokens, bs)
        hit = self.pool.find_cached(hashes)
        self.pool.touch(hit)
        try:
            fresh = self.pool.allocate(len(hashes) - len(hit))
        except BlockError:
            self.pool.release(hit)
            raise
        self.tokens = list(tokens)
        self.hashes = hashes
        self.blocks = hit + fresh
        self.owned = [False] * len(hit) + [True] * len(fresh)
        computed = len(hit) * bs
        if computed >= len(tokens):
            computed = max(len(tokens) - 1, 0)
        self.num_computed = self.num_written = computed
        return computed

    def _ensure(self, required):
        if required > len(self.blocks):
            fresh = self.pool.allocate(required - len(self.blocks))
            self.blocks += fresh
            self.owned += [True] * len(fresh)

    def reserve(self, new_tokens):
        bs = self.pool.block_size
        end = self.num_computed + new_tokens
        if self.max_seq_len > 0 and end > self.max_seq_len:
            raise BlockError("past max_seq_len")
        self._ensure(-(-end // bs))
        self.num_written = max(self.num_written, end)
        return self.num_computed

    def append_token(self, token):
        """Returns False when the block the token completes could not be allocated."""
        bs = self.pool.block_size
        self.tokens.append(token)
        if len(self.tokens) % bs:
            return True
        blk = len(self.tokens) // bs - 1
        ok = True
        try:
            self._ensure(blk + 1)
        except BlockError:
            ok = False
        parent = self.hashes[blk - 1] if 1 <= blk <= len(self.hashes) else None
        h = block_hash(self.tokens[blk * bs:(blk + 1) * bs], parent)
        if blk < len(self.hashes):
            self.hashes[blk] = h
        else:
            self.hashes += [0] * (blk - len(self.hashes)) + [h]
        return ok

    def commit(self, new_tokens):
        bs = self.pool.block_size
        old = self.num_computed
        self.num_computed += new_tokens
        self.num_written = max(self.num_written, self.num_computed)
        lo = old // bs
        hi = min(self.num_computed // bs, len(self.hashes), len(self.blocks))
        for i in range(lo, hi):
            if self.blocks[i] >= 0:
                self.pool.cache_blocks([self.blocks[i]], [self.hashes[i]])

    def drop_before(self, first_pos):
        """Blocks 0 .. first_pos // block_size - 1 go back to the pool (one reference each);
        their entries become -1. Only computed tokens can be dropped."""
        if first_pos < 0 or first_pos > self.num_computed:
            raise BlockError("first_pos outside [0, num_computed]")
        upto = min(len(self.blocks), first_pos // self.pool.block_size)
        for i in range(upto):
            if self.blocks[i] >= 0:
                self.pool.release([self.blocks[i]])
                self.blocks[i] = -1
                self.owned[i] = False
        self.dropped = max(self.dropped, upto)
        return self.dropped

    def truncate(self, seq_len):
        seq_len = max(seq_len, 0)
        if seq_len < self.num_computed and seq_len < self.dropped * self.pool.block_size:
            raise BlockError("tokens before the dropped blocks' end are gone")
        if seq_len < self.num_computed:
            self.num_computed = seq_len
            self.num_written = min(self.num_written, seq_len)

    def free(self):
        self.pool.release(self.blocks)
        self.blocks, self.owned, self.tokens, self.hashes = [], [], [], []
        self.num_computed = self.num_written = 0
        self.dropped = 0

    def destroy(self):
        self.free()
        self.pool.live_seqs -= 1


def fill_tables(seqs, max_blocks_per_seq, pad_block):
    """Row b = seqs[b]'s block ids padded with pad_block; positions[b] = its computed count."""
    rows, positions = [], []
    for s in seqs:
        if len(s.blocks) > max_blocks_per_seq:
            raise BlockError("more blocks than the table row holds")
        rows.append([b if b >= 0 else pad_block for b in s.blocks]
                    + [pad_block] * (max_blocks_per_seq - len(s.blocks)))
        positions.append(s.num_computed)
    return rows, positions
