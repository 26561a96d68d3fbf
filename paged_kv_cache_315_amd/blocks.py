"""Python handles on the host block manager of libpkv (include/pkv_blocks.h).

Marshalling only: every decision (reference counts, free list, prefix cache, hashes, table
rows) is made by the C++ block manager in libpkv.so.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _lib


class PoolInfo(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int64), ("block_size", ctypes.c_int),
                ("num_free", ctypes.c_int64), ("num_cached", ctypes.c_int64),
                ("live_seqs", ctypes.c_int64)]


class SeqState(ctypes.Structure):
    _fields_ = [("num_computed", ctypes.c_int), ("num_written", ctypes.c_int),
                ("num_tokens", ctypes.c_int), ("num_blocks", ctypes.c_int),
                ("num_hashes", ctypes.c_int), ("num_dropped", ctypes.c_int)]


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def block_hash(tokens, parent: int | None = None) -> int:
    t = _i32(tokens)
    par = ctypes.byref(ctypes.c_uint64(parent)) if parent is not None else None
    return int(_lib.load().pkv_block_hash(t.ctypes.data, len(t), par))


class BlockPool:
    """num_blocks physical block ids of block_size tokens, shared by every layer's pools."""

    def __init__(self, num_blocks: int, block_size: int):
        self._lib = _lib.load()
        h = ctypes.c_void_p()
        _lib.check(self._lib.pkv_pool_create(num_blocks, block_size, ctypes.byref(h)),
                   "pkv_pool_create")
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    @property
    def handle(self):
        return self._h

    def stats(self) -> PoolInfo:
        info = PoolInfo()
        _lib.check(self._lib.pkv_pool_stats(self._h, ctypes.byref(info)), "pkv_pool_stats")
        return info

    def block_state(self):
        """(refcounts int32[n], cached uint8[n], hashes uint64[n], free list front to back)."""
        n = self.num_blocks
        ref = np.zeros(n, np.int32)
        cached = np.zeros(n, np.uint8)
        hashes = np.zeros(n, np.uint64)
        order = np.zeros(n, np.int32)
        _lib.check(self._lib.pkv_pool_block_state(self._h, ref.ctypes.data, cached.ctypes.data,
                                                  hashes.ctypes.data, order.ctypes.data),
                   "pkv_pool_block_state")
        return ref, cached, hashes, order[:self.stats().num_free]

    def close(self):
        if self._h:
            _lib.check(self._lib.pkv_pool_destroy(self._h), "pkv_pool_destroy")
            self._h = None


class SeqCache:
    """One sequence's block list, token history and computed count on a BlockPool."""

    def __init__(self, pool: BlockPool, max_seq_len: int = 0):
        self._lib = pool._lib
        self.pool = pool
        h = ctypes.c_void_p()
        _lib.check(self._lib.pkv_seq_create(pool.handle, max_seq_len, ctypes.byref(h)),
                   "pkv_seq_create")
        self._h = h

    @property
    def handle(self):
        return self._h

    def allocate_for_tokens(self, tokens) -> int:
        t = _i32(tokens)
        cached = ctypes.c_int()
        _lib.check(self._lib.pkv_seq_allocate_for_tokens(self._h, t.ctypes.data, len(t),
                                                         ctypes.byref(cached)),
                   "pkv_seq_allocate_for_tokens")
        return cached.value

    def reserve(self, new_tokens: int) -> int:
        start = ctypes.c_int()
        _lib.check(self._lib.pkv_seq_reserve(self._h, new_tokens, ctypes.byref(start)),
                   "pkv_seq_reserve")
        return start.value

    def append_token(self, token: int):
        _lib.check(self._lib.pkv_seq_append_token(self._h, int(token)), "pkv_seq_append_token")

    def commit(self, new_tokens: int):
        _lib.check(self._lib.pkv_seq_commit(self._h, new_tokens), "pkv_seq_commit")

    def truncate(self, seq_len: int):
        _lib.check(self._lib.pkv_seq_truncate(self._h, seq_len), "pkv_seq_truncate")

    def drop_before(self, first_pos: int) -> int:
        """Give back the blocks whose tokens all lie before first_pos (sliding window); returns
        how many leading entries are given back so far."""
        n = ctypes.c_int(0)
        _lib.check(self._lib.pkv_seq_drop_before(self._h, first_pos, ctypes.byref(n)),
                   "pkv_seq_drop_before")
        return n.value

    def free(self):
        _lib.check(self._lib.pkv_seq_free(self._h), "pkv_seq_free")

    def state(self) -> SeqState:
        st = SeqState()
        _lib.check(self._lib.pkv_seq_info(self._h, ctypes.byref(st)), "pkv_seq_info")
        return st

    def blocks(self):
        """(block ids int32 (-1 where given back by drop_before), owned bool, hashes uint64)."""
        st = self.state()
        cap = max(st.num_blocks, st.num_hashes, 1)
        ids = np.zeros(cap, np.int32)
        owned = np.zeros(cap, np.uint8)
        hashes = np.zeros(cap, np.uint64)
        _lib.check(self._lib.pkv_seq_blocks(self._h, ids.ctypes.data, owned.ctypes.data,
                                            hashes.ctypes.data, cap), "pkv_seq_blocks")
        return ids[:st.num_blocks], owned[:st.num_blocks].astype(bool), hashes[:st.num_hashes]

    def destroy(self):
        if self._h:
            self._lib.pkv_seq_destroy(self._h)
            self._h = None


def fill_block_tables(seqs, max_blocks_per_seq: int, pad_block: int):
    """Host int32 tables [B, max_blocks_per_seq] and positions [B] for the paged calls."""
    B = len(seqs)
    tables = np.zeros((B, max_blocks_per_seq), np.int32)
    positions = np.zeros(B, np.int32)
    arr = (ctypes.c_void_p * max(B, 1))(*[s.handle.value for s in seqs])
    _lib.check(_lib.load().pkv_fill_block_tables(arr, B, max_blocks_per_seq, pad_block,
                                                 tables.ctypes.data, positions.ctypes.data),
               "pkv_fill_block_tables")
    return tables, positions


class Batch:
    """A fixed list of sequences driven together: one C call per step for room + tables and one
    for the commit (the per-sequence calls cost a Python round trip each)."""

    def __init__(self, seqs, max_blocks_per_seq: int, pad_block: int):
        self.seqs = list(seqs)
        self.B = len(self.seqs)
        self._arr = (ctypes.c_void_p * max(self.B, 1))(*[s.handle.value for s in self.seqs])
        self.max_blocks = max_blocks_per_seq
        self.pad = pad_block
        self.tables = np.zeros((self.B, max_blocks_per_seq), np.int32)
        self.positions = np.zeros(self.B, np.int32)
        self._lib = _lib.load()

    def prepare(self, new_tokens: int = 1, window: int = 0):
        """Room for new_tokens per sequence (after giving back the blocks wholly behind a sliding
        window of `window` tokens, when > 0); returns (tables, positions), host int32 arrays
        reused by every call."""
        _lib.check(self._lib.pkv_batch_prepare(self._arr, self.B, new_tokens, window,
                                               self.max_blocks,
                                               self.pad, self.tables.ctypes.data,
                                               self.positions.ctypes.data), "pkv_batch_prepare")
        return self.tables, self.positions

    def commit(self, new_tokens: int = 1, token_ids=None):
        ids = None if token_ids is None else _i32(token_ids)
        if ids is not None:
            assert ids.size == self.B * new_tokens
        _lib.check(self._lib.pkv_batch_commit(self._arr, self.B, new_tokens,
                                              None if ids is None else ids.ctypes.data),
                   "pkv_batch_commit")

