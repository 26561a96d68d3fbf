"""The host block manager driving the GPU path: prompts admitted with a shared prefix, their
uncached tokens prefilled, then decode steps, all over the tables the manager produces
(page "makarna/pkg/kvcache/paged_cache.go": AllocateForTokens borrows the cached prefix, Append
grows the block list, Commit caches completed blocks).

Every phase runs on the GPU (C ABI) and in the oracle on the same inputs and tables: pools
bit-identical over the whole pool, outputs within 1e-3 abs + 2e-3 rel (tests/gpu_util.py).
The pool starts as quiet-NaN codes, so a borrowed block read before anyone wrote it, or a
padded table entry read, would turn the outputs into NaN.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_315_amd as pkv
from paged_kv_cache_315_amd.blocks import BlockPool, SeqCache, fill_block_tables
from gpu_util import assert_close, assert_pools_equal, log, pool_host

pytestmark = pytest.mark.gpu

HQ, HKV, D, BS, NB, MAXB = 8, 2, 64, 16, 48, 8
THETA, DTYPE = 1e4, "fp16"
SCALE = float(np.float32(1.0 / np.sqrt(D)))
PAD = NB                       # one spare block past the managed ones: table padding
NAN16 = 0x7E00


class Both:
    """The same pools on the GPU (torch) and in host memory (oracle)."""

    def __init__(self):
        self.k = np.full((NB + 1, BS, HKV, D), NAN16, np.uint16)
        self.v = self.k.copy()
        self.kd = torch.from_numpy(self.k.view(np.int16).copy()).cuda()
        self.vd = torch.from_numpy(self.v.view(np.int16).copy()).cuda()

    def check_pools(self, what):
        assert_pools_equal(pool_host(self.kd), self.k, f"{what}: k_pool")
        assert_pools_equal(pool_host(self.vd), self.v, f"{what}: v_pool")


def _inputs(rng, n):
    f = lambda *s: rng.standard_normal(s, dtype=np.float32)
    return f(n, HQ, D), f(n, HKV, D), f(n, HKV, D)


def _prefill(both, seqs, chunks, rng, what, window=0):
    """Reserve and prefill chunks[b] new tokens of seqs[b] (from their computed count on)."""
    starts = np.array([s.reserve(c) for s, c in zip(seqs, chunks)], np.int32)
    tables, pos = fill_block_tables(seqs, MAXB, PAD)
    assert (pos == starts).all()
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q, k, v = _inputs(rng, int(cu[-1]))
    q_ref = oracle.prefill_append(q, k, v, both.k, both.v, tables, cu, starts, None, None, 1e-6,
                                  THETA, DTYPE)
    out_ref = oracle.paged_attn_prefill(q_ref, both.k, both.v, tables, cu, starts, SCALE, DTYPE,
                                        window=window)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q_out, out = pkv.prefill_step(t(q), t(k), t(v), both.kd, both.vd, t(tables), t(cu), t(starts),
                                  int(max(chunks)), int((starts + np.array(chunks)).max()),
                                  theta=THETA, scale=SCALE, dtype=DTYPE, window=window)
    torch.cuda.synchronize()
    both.check_pools(what)
    assert_close(q_out.cpu().numpy(), q_ref, f"{what}: q_out")
    assert_close(out.cpu().numpy(), out_ref, f"{what}: out")
    for s, c in zip(seqs, chunks):
        s.commit(c)
    return q, k, v


def _decode(both, seqs, rng, what, kv=None, window=0):
    for s in seqs:
        if window:
            s.drop_before(max(0, s.state().num_computed + 1 - window))
        s.reserve(1)
    tables, pos = fill_block_tables(seqs, MAXB, PAD)
    q, k, v = _inputs(rng, len(seqs))
    if kv is not None:
        k, v = kv
    q_ref = oracle.kv_append(q, k, v, both.k, both.v, tables, pos, None, None, 1e-6, THETA, DTYPE)
    out_ref = oracle.paged_attn_decode(q_ref, both.k, both.v, tables, pos + 1, SCALE, DTYPE,
                                       window=window)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q_out, out = pkv.decode_step(t(q), t(k), t(v), both.kd, both.vd, t(tables), t(pos),
                                 theta=THETA, scale=SCALE, dtype=DTYPE, window=window)
    torch.cuda.synchronize()
    both.check_pools(what)
    assert_close(q_out.cpu().numpy(), q_ref, f"{what}: q_out")
    assert_close(out.cpu().numpy(), out_ref, f"{what}: out")
    for s in seqs:
        s.commit(1)
    return tables


def test_shared_prefix_prefill_then_decode():
    rng = np.random.default_rng(315)
    both = Both()
    pool = BlockPool(NB, BS)
    prompt = rng.integers(0, 32000, 40).tolist()

    log("block manager: cold prompt of 40 tokens")
    a = SeqCache(pool, max_seq_len=MAXB * BS)
    assert a.allocate_for_tokens(prompt) == 0
    _, cold_k, cold_v = _prefill(both, [a], [40], rng, "cold prefill")
    assert pool.stats().num_cached == 2                     # blocks of tokens 0..31

    log("block manager: three prompts, two sharing the first 32 tokens")
    b = SeqCache(pool, max_seq_len=MAXB * BS)
    c = SeqCache(pool, max_seq_len=MAXB * BS)
    d = SeqCache(pool, max_seq_len=MAXB * BS)
    pb = prompt[:32] + rng.integers(0, 32000, 10).tolist()
    pc = prompt[:32] + rng.integers(0, 32000, 27).tolist()
    pd = rng.integers(0, 32000, 19).tolist()
    assert b.allocate_for_tokens(pb) == 32
    assert c.allocate_for_tokens(pc) == 32
    assert d.allocate_for_tokens(pd) == 0
    ids_a, _, _ = a.blocks()
    for s in (b, c):
        ids, owned, _ = s.blocks()
        assert ids[:2].tolist() == ids_a[:2].tolist() and not owned[:2].any() and owned[2:].all()
    assert pool.block_state()[0][ids_a[:2]].tolist() == [3, 3]
    _prefill(both, [b, c, d], [10, 27, 19], rng, "prefill over borrowed blocks")

    log("block manager: decode steps over the shared tables")
    seqs = [a, b, c, d]
    for step in range(3):
        tables = _decode(both, seqs, rng, f"decode step {step}")
    assert (tables[:3, :2] == tables[0, :2]).all()          # one physical prefix, three rows

    log("block manager: a prompt equal to a cached one borrows all but the recomputed token")
    e = SeqCache(pool, max_seq_len=MAXB * BS)
    assert e.allocate_for_tokens(prompt[:32]) == 31
    k_before, v_before = both.k.copy(), both.v.copy()
    # the recomputed token has the K/V it had when the prefix was first computed, so writing it
    # into the borrowed block leaves the shared block's bits as they were
    _decode(both, [e], rng, "decode rewriting a borrowed block's last slot",
            kv=(cold_k[31:32].copy(), cold_v[31:32].copy()))
    assert np.array_equal(both.k, k_before) and np.array_equal(both.v, v_before)

    for s in seqs + [e]:
        s.destroy()
    assert pool.stats().num_free == NB
    pool.close()


def test_sliding_window_blocks_reused_by_another_sequence():
    """Sliding-window layer (window 24, blocks of 16) on a pool of six blocks: sequence A's
    first block falls behind its window and goes back to the pool (drop_before), sequence B's
    admission takes it and B's prefill overwrites it, and A keeps decoding over a table whose
    given-back entries are the NaN padding block. Pools bit-identical to the oracle's at every
    phase (so B's writes land where the manager put them), outputs within tolerance (so A never
    reads a given-back entry: it would read NaN)."""
    W = 24
    rng = np.random.default_rng(316)
    both = Both()
    pool = BlockPool(6, BS)

    log("sliding window: A prefills 40 tokens")
    a = SeqCache(pool)
    assert a.allocate_for_tokens(rng.integers(0, 32000, 40).tolist()) == 0
    _prefill(both, [a], [40], rng, "window prefill A", window=W)
    first_a = int(a.blocks()[0][0])

    log("sliding window: A decodes; its first block goes back")
    _decode(both, [a], rng, "window decode A", window=W)
    assert a.state().num_dropped == 1 and a.blocks()[0][0] == -1
    assert pool.block_state()[0][first_a] == 0

    log("sliding window: B takes the given-back block and prefills over it")
    b = SeqCache(pool)
    assert b.allocate_for_tokens(rng.integers(0, 32000, 60).tolist()) == 0
    assert b.blocks()[0].tolist()[-1] == first_a           # the last of the four free blocks
    _prefill(both, [b], [60], rng, "window prefill B over A's old block", window=W)

    log("sliding window: A and B decode together")
    for step in range(16):
        tables = _decode(both, [a, b], rng, f"window decode A+B {step}", window=W)
        assert tables[0, 0] == PAD
    # A attended 57 tokens last (keys 33..56: two blocks behind), B 76 (keys 52..75: three)
    assert a.state().num_dropped == 2 and b.state().num_dropped == 3
    for s in (a, b):
        s.destroy()
    assert pool.stats().num_free == 6
    pool.close()
