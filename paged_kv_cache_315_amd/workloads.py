"""Seeded synthetic inputs for the paged-KV decode step.

This module only DRAWS inputs: context lengths, block tables, pre-filled pools, new-token
Q/K/V and norm weights. It holds none of the step's arithmetic, and it is the one module that
both the HIP path's tests/bench and the CPU oracle read (the oracle receives these arrays as
arguments). Pre-filled 16-bit pool values come from library casts (numpy ``float16``,
torch ``bfloat16``); they are inputs, any valid codes would do.

Every named input has its own PCG64 stream, seeded ``[workload_id, stream_id]``, so a workload
is a pure function of its parameters.

Workload shapes follow the five decode workloads the method is measured on (and, for chunked
prefill, ``make_prefill_workload`` with the same head shapes):
  1 tiny        B=2, cached 37 / 50 tokens, 4/2 heads, D=64, bs=16, 16-block pool, fp16, theta 1e4
  2 llama3-8b   B=32, cached U{512..4096}, 32/8 heads, D=128, bs=16, bf16, theta 5e5
  3 qwen3-norm  B=64, cached 8192, 32/8 heads, D=128, bs=16, fp16, QK-RMSNorm eps 1e-6,
                weights U(0.5, 1.5), theta 1e6, edge values in 0.1 % of the new K/V
  4 long-gqa8   B=8, cached 32768, 64/8 heads, D=128, bs=32, bf16 pool N(0,1)*0.5, theta 5e5
  5 prefix      B=128, 128 shared prefix blocks (2048 tokens) + private tail U{0..1024},
                32/8 heads, D=128, bs=16, fp16, theta 5e5
"""
from __future__ import annotations

import math

import numpy as np

# stream ids
S_CTX, S_PERM, S_KPOOL, S_VPOOL, S_Q, S_KNEW, S_VNEW, S_NORM, S_EDGE_POS, S_EDGE_VAL = range(10)

# quiet-NaN codes used to poison every pool element that no valid token owns (f32 pools hold
# the float bits themselves, as uint32)
POISON = {"f16": 0x7E00, "bf16": 0x7FC0, "f32": 0x7FC00000}
POOL_NP = {"f16": np.uint16, "bf16": np.uint16, "f32": np.uint32}

EDGE_VALUES = np.array([70000.0, -70000.0, 1e-7, np.nan], dtype=np.float32)


def _rng(wid: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(wid), int(stream)])


def _to_codes(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> pool codes: 16-bit with a library cast, or the float bits (inputs only)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def _fill_pool(rng: np.random.Generator, shape, dtype: str, std: float) -> np.ndarray:
    """N(0, std^2) codes, drawn in chunks of blocks to bound host memory."""
    pool = np.empty(shape, dtype=POOL_NP[dtype])
    nb = shape[0]
    per_block = int(np.prod(shape[1:]))
    chunk = max(1, (1 << 24) // per_block)
    for b0 in range(0, nb, chunk):
        b1 = min(nb, b0 + chunk)
        x = rng.standard_normal((b1 - b0) * per_block, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        pool[b0:b1] = _to_codes(x, dtype).reshape((b1 - b0,) + tuple(shape[1:]))
    return pool


def make_workload(wid: int, cached, Hq: int, Hkv: int, D: int, bs: int, dtype: str,
                  theta: float, *, qk_norm: bool = False, eps: float = 1e-6,
                  pool_std: float = 1.0, new_kv_std: float = 1.0, spare_blocks: int = 1,
                  shared_prefix_blocks: int = 0, edge_fraction: float = 0.0,
                  extra_table_cols: int = 0, name: str | None = None) -> dict:
    """Draw one decode-step workload.

    cached[b] = tokens already in the cache for sequence b = the position the new token is
    appended at; the attended length is cached[b] + 1.
    shared_prefix_blocks: the first n logical blocks of every sequence map to the same n
    physical blocks (a shared prefix; every cached[b] must be >= n * bs).
    spare_blocks: unassigned physical blocks (poisoned); the first one also pads the tables.
    """
    cached = np.asarray(cached, dtype=np.int64)
    B = int(cached.shape[0])
    assert Hq % Hkv == 0 and D % 2 == 0
    lens = cached + 1
    need = (lens + bs - 1) // bs                      # logical blocks per sequence
    if shared_prefix_blocks:
        assert np.all(cached >= shared_prefix_blocks * bs), "prefix must be full blocks"
    private = need - shared_prefix_blocks
    n_assigned = int(shared_prefix_blocks + private.sum())
    NB = n_assigned + int(spare_blocks)
    perm = _rng(wid, S_PERM).permutation(NB).astype(np.int32)
    shared_ids = perm[:shared_prefix_blocks]
    max_blocks = int(need.max()) if B else 1
    max_blocks += int(extra_table_cols)
    spare_ids = perm[n_assigned:]
    pad_id = int(spare_ids[0]) if len(spare_ids) else int(perm[0])
    tables = np.full((B, max_blocks), pad_id, dtype=np.int32)
    cur = shared_prefix_blocks
    for b in range(B):
        tables[b, :shared_prefix_blocks] = shared_ids
        n = int(private[b])
        tables[b, shared_prefix_blocks:shared_prefix_blocks + n] = perm[cur:cur + n]
        cur += n

    shape = (NB, bs, Hkv, D)
    k_pool = _fill_pool(_rng(wid, S_KPOOL), shape, dtype, pool_std)
    v_pool = _fill_pool(_rng(wid, S_VPOOL), shape, dtype, pool_std)
    poison = POISON[dtype]
    # poison: spare blocks, and in each sequence's last block the new token's slot and after
    for pid in spare_ids:
        k_pool[pid] = poison
        v_pool[pid] = poison
    for b in range(B):
        last = tables[b, int(cached[b]) // bs]
        s0 = int(cached[b]) % bs
        k_pool[last, s0:] = poison
        v_pool[last, s0:] = poison

    q = _rng(wid, S_Q).standard_normal((B, Hq, D), dtype=np.float32)
    k_new = _rng(wid, S_KNEW).standard_normal((B, Hkv, D), dtype=np.float32)
    v_new = _rng(wid, S_VNEW).standard_normal((B, Hkv, D), dtype=np.float32)
    if new_kv_std != 1.0:
        k_new *= np.float32(new_kv_std)
        v_new *= np.float32(new_kv_std)
    q_norm_w = k_norm_w = None
    if qk_norm:
        rn = _rng(wid, S_NORM)
        q_norm_w = rn.uniform(0.5, 1.5, D).astype(np.float32)
        k_norm_w = rn.uniform(0.5, 1.5, D).astype(np.float32)
    edges = {}
    if edge_fraction > 0 and B > 0:
        rp = _rng(wid, S_EDGE_POS)
        rv = _rng(wid, S_EDGE_VAL)
        for nm, arr in (("k_new", k_new), ("v_new", v_new)):
            n = arr.size
            cnt = int(math.ceil(edge_fraction * n))
            idx = rp.permutation(n)[:cnt]
            val = EDGE_VALUES[rv.integers(0, len(EDGE_VALUES), cnt)]
            arr.reshape(-1)[idx] = val
            edges[nm] = (idx, val)

    return {
        "name": name or f"w{wid}", "wid": wid, "B": B, "Hq": Hq, "Hkv": Hkv, "D": D, "bs": bs,
        "dtype": dtype, "theta": float(theta), "eps": float(eps),
        "positions": cached.astype(np.int32), "context_lens": lens.astype(np.int32),
        "max_context_len": int(lens.max()) if B else 0,
        "tables": tables, "max_blocks": max_blocks, "num_blocks": NB,
        "k_pool": k_pool, "v_pool": v_pool, "q": q, "k_new": k_new, "v_new": v_new,
        "q_norm_w": q_norm_w, "k_norm_w": k_norm_w,
        "scale": float(np.float32(1.0 / math.sqrt(D))),
        "spare_ids": spare_ids, "shared_ids": shared_ids, "edges": edges,
    }


def config(cfg_id: int) -> dict:
    """The five decode workloads (see module docstring)."""
    if cfg_id == 1:
        return make_workload(1, [37, 50], 4, 2, 64, 16, "f16", 1e4, spare_blocks=9,
                             name="tiny")
    if cfg_id == 2:
        cached = _rng(2, S_CTX).integers(512, 4096, size=32, endpoint=True)
        return make_workload(2, cached, 32, 8, 128, 16, "bf16", 5e5, name="llama3-8b")
    if cfg_id == 3:
        return make_workload(3, [8192] * 64, 32, 8, 128, 16, "f16", 1e6, qk_norm=True,
                             eps=1e-6, edge_fraction=0.001, name="qwen3-qknorm")
    if cfg_id == 4:
        return make_workload(4, [32768] * 8, 64, 8, 128, 32, "bf16", 5e5, pool_std=0.5,
                             new_kv_std=0.5, name="long-gqa8")
    if cfg_id == 5:
        tails = _rng(5, S_CTX).integers(0, 1024, size=128, endpoint=True)
        return make_workload(5, 2048 + tails, 32, 8, 128, 16, "f16", 5e5,
                             shared_prefix_blocks=128, name="prefix-shared")
    raise ValueError(f"unknown workload {cfg_id}")


CONFIG_NAMES = {1: "tiny", 2: "llama3-8b", 3: "qwen3-qknorm", 4: "long-gqa8", 5: "prefix-shared"}


def kv_bytes(wl: dict) -> int:
    """K+V bytes a decode step must read: sum over sequences of L_b * 2 * Hkv * D * 2."""
    return int(wl["context_lens"].astype(np.int64).sum()) * 2 * wl["Hkv"] * wl["D"] * 2


def unique_kv_bytes(wl: dict) -> int:
    """K+V bytes of distinct (block, slot) rows read (a shared prefix counted once)."""
    bs = wl["bs"]
    rows = {}
    for b in range(wl["B"]):
        L = int(wl["context_lens"][b])
        for j in range((L + bs - 1) // bs):
            blk = int(wl["tables"][b, j])
            rows[blk] = max(rows.get(blk, 0), min(bs, L - j * bs))
    return sum(rows.values()) * 2 * wl["Hkv"] * wl["D"] * 2


def make_prefill_workload(wid: int, cached, chunk, Hq: int, Hkv: int, D: int, bs: int,
                          dtype: str, theta: float, *, qk_norm: bool = False, eps: float = 1e-6,
                          pool_std: float = 1.0, spare_blocks: int = 1,
                          extra_table_cols: int = 0, name: str | None = None) -> dict:
    """Draw one chunked-prefill workload: sequence b has cached[b] tokens in the cache and
    chunk[b] new tokens (token-major rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of q / k_new /
    v_new) at positions cached[b] .. cached[b] + chunk[b] - 1. Pool slots from position
    cached[b] on, and spare blocks, are poisoned."""
    cached = np.asarray(cached, dtype=np.int64)
    chunk = np.asarray(chunk, dtype=np.int64)
    B = int(cached.shape[0])
    assert chunk.shape == cached.shape and np.all(chunk >= 0)
    assert Hq % Hkv == 0 and D % 2 == 0
    total = cached + chunk
    need = np.maximum((total + bs - 1) // bs, 1)
    n_assigned = int(need.sum())
    NB = n_assigned + int(spare_blocks)
    perm = _rng(wid, S_PERM).permutation(NB).astype(np.int32)
    max_blocks = (int(need.max()) if B else 1) + int(extra_table_cols)
    spare_ids = perm[n_assigned:]
    pad_id = int(spare_ids[0]) if len(spare_ids) else int(perm[0])
    tables = np.full((B, max_blocks), pad_id, dtype=np.int32)
    cur = 0
    for b in range(B):
        n = int(need[b])
        tables[b, :n] = perm[cur:cur + n]
        cur += n
    shape = (NB, bs, Hkv, D)
    k_pool = _fill_pool(_rng(wid, S_KPOOL), shape, dtype, pool_std)
    v_pool = _fill_pool(_rng(wid, S_VPOOL), shape, dtype, pool_std)
    poison = POISON[dtype]
    for pid in spare_ids:
        k_pool[pid] = poison
        v_pool[pid] = poison
    for b in range(B):
        c0 = int(cached[b])
        for j in range(c0 // bs, int(need[b])):
            s0 = c0 % bs if j == c0 // bs else 0
            k_pool[tables[b, j], s0:] = poison
            v_pool[tables[b, j], s0:] = poison
    N = int(chunk.sum())
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(chunk)
    q = _rng(wid, S_Q).standard_normal((N, Hq, D), dtype=np.float32)
    k_new = _rng(wid, S_KNEW).standard_normal((N, Hkv, D), dtype=np.float32)
    v_new = _rng(wid, S_VNEW).standard_normal((N, Hkv, D), dtype=np.float32)
    q_norm_w = k_norm_w = None
    if qk_norm:
        rn = _rng(wid, S_NORM)
        q_norm_w = rn.uniform(0.5, 1.5, D).astype(np.float32)
        k_norm_w = rn.uniform(0.5, 1.5, D).astype(np.float32)
    # per query token: the sequence it belongs to and the number of tokens it attends
    tok_seq = np.repeat(np.arange(B, dtype=np.int32), chunk)
    tok_len = (np.repeat(cached, chunk) + np.concatenate(
        [np.arange(int(c)) for c in chunk] or [np.zeros(0, np.int64)]) + 1).astype(np.int32)
    return {
        "name": name or f"p{wid}", "wid": wid, "B": B, "N": N, "Hq": Hq, "Hkv": Hkv, "D": D,
        "bs": bs, "dtype": dtype, "theta": float(theta), "eps": float(eps),
        "start_pos": cached.astype(np.int32), "chunk": chunk.astype(np.int32),
        "cu_seqlens": cu, "tok_seq": tok_seq, "tok_len": tok_len,
        "max_chunk": int(chunk.max()) if B else 0,
        "max_context_len": int(total.max()) if B else 0,
        "tables": tables, "max_blocks": max_blocks, "num_blocks": NB,
        "k_pool": k_pool, "v_pool": v_pool, "q": q, "k_new": k_new, "v_new": v_new,
        "q_norm_w": q_norm_w, "k_norm_w": k_norm_w,
        "scale": float(np.float32(1.0 / math.sqrt(D))), "spare_ids": spare_ids,
    }


def prefill_config(cfg_id: int) -> dict:
    """Chunked-prefill workloads with the decode workloads' head shapes:
      1 tiny        B=3, cached 0 / 21 / 40, chunks 7 / 30 / 1, 4/2 heads, D=64, bs=16, fp16
      2 llama3-8b   B=4, cached U{0..2048}, chunks of 512, 32/8 heads, D=128, bs=16, bf16
      3 spec-decode B=32, cached U{512..4096}, 4 new tokens each (draft verification), as 2
    """
    if cfg_id == 1:
        return make_prefill_workload(101, [0, 21, 40], [7, 30, 1], 4, 2, 64, 16, "f16", 1e4,
                                     spare_blocks=3, name="prefill-tiny")
    if cfg_id == 2:
        cached = _rng(102, S_CTX).integers(0, 2048, size=4, endpoint=True)
        return make_prefill_workload(102, cached, [512] * 4, 32, 8, 128, 16, "bf16", 5e5,
                                     name="prefill-llama3-8b")
    if cfg_id == 3:
        cached = _rng(103, S_CTX).integers(512, 4096, size=32, endpoint=True)
        return make_prefill_workload(103, cached, [4] * 32, 32, 8, 128, 16, "bf16", 5e5,
                                     name="spec-decode-4")
    raise ValueError(f"unknown prefill workload {cfg_id}")


def prefill_kv_bytes(wl: dict) -> int:
    """K+V bytes the per-token reading of a prefill step reads: sum over query tokens of
    their attended lengths * 2 * Hkv * D * 2 (each token reading its own prefix)."""
    return int(wl["tok_len"].astype(np.int64).sum()) * 2 * wl["Hkv"] * wl["D"] * 2


def prefill_unique_kv_bytes(wl: dict) -> int:
    """K+V bytes of the distinct rows a prefill step reads: per sequence its
    cached + chunk tokens, once."""
    tot = (wl["start_pos"].astype(np.int64) + wl["chunk"]).sum()
    return int(tot) * 2 * wl["Hkv"] * wl["D"] * 2
