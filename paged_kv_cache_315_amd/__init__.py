"""paged_kv_cache_315_amd — the paged-KV decode step on AMD Instinct MI355X (gfx950).

Python face of the C ABI in include/pkv.h (libpkv.so, hand-written HIP kernels). torch is
used only for device memory and streams: every function takes torch tensors that already live
on the GPU, passes their pointers to libpkv and enqueues the kernels on the current stream.

    kv_append(...)          new token per sequence: QK-norm (optional), RoPE, fp16/bf16
                            round-to-nearest-even, scatter into the block pools
    paged_attn_decode(...)  softmax(scale q.K^T).V over each sequence's block list (GQA)
    decode_step(...)        both, as one decoder layer's attention step (one kernel launch)
"""
from __future__ import annotations

import ctypes

from . import _lib
from ._lib import PKV_BF16, PKV_F16, PKV_F32, PkvError

__all__ = ["PKV_F16", "PKV_BF16", "PKV_F32", "kv_append", "paged_attn_decode", "decode_step",
           "decode_workspace_bytes", "decode_schedule_split",
           "prefill_append", "paged_attn_prefill", "prefill_workspace_bytes", "prefill_step",
           "decode_step_workspace_bytes", "decode_step_noalloc", "decode_step_noalloc_scratch_bytes",
           "append_then_decode", "decode_split_tokens", "validate_tables", "version",
           "PkvError", "pool_dtype_code"]


def _torch():
    import torch
    return torch


def version() -> str:
    return _lib.load().pkv_version().decode()


def pool_dtype_code(pool, dtype=None) -> int:
    """PKV_F16 / PKV_BF16 / PKV_F32 from an explicit name or from the pool tensor's dtype."""
    torch = _torch()
    if dtype is not None:
        return {"f16": PKV_F16, "fp16": PKV_F16, "bf16": PKV_BF16, "f32": PKV_F32}[dtype]
    if pool.dtype == torch.float16:
        return PKV_F16
    if pool.dtype == torch.bfloat16:
        return PKV_BF16
    if pool.dtype == torch.float32:
        return PKV_F32
    raise ValueError("pool dtype must be float16, bfloat16 or float32, or pass "
                     "dtype='f16'|'bf16'|'f32'")


def _pool_elem(pool, dtype) -> int:
    """Bytes per pool element the call expects: 4 for float32 pools, else 2."""
    return 4 if pool_dtype_code(pool, dtype) == PKV_F32 else 2


def _dev_ptr(t, name, *, dtype=None, ndim=None, elem_size=None):
    """Device pointer of a contiguous CUDA(HIP) tensor, after shape/dtype checks."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if elem_size is not None and t.element_size() != elem_size:
        raise ValueError(f"{name} must have {elem_size}-byte elements")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def kv_append(q_in, k_in, v_in, k_pool, v_pool, block_tables, positions, *, theta: float,
              q_norm_w=None, k_norm_w=None, eps: float = 1e-6, q_out=None, dtype=None,
              rope_dim: int = 0, v_norm: bool = False, rope_on_read: bool = False,
              stream=None):
    """Append one token per sequence; returns q_out ([B, Hq, D] float32, normed + rotated).

    q_in [B,Hq,D], k_in / v_in [B,Hkv,D] float32; k_pool / v_pool [NB,bs,Hkv,D] 16-bit;
    block_tables [B,max_blocks] int32; positions [B] int32 (write slot = RoPE position).
    rope_dim: rotary dims (0 = D; partial rotary below D); v_norm: RMS-normalise each new V
    head vector before it is stored; rope_on_read: rotate nothing (the decode rotates at read).
    """
    torch = _torch()
    B, Hq, D = q_in.shape
    Hkv = k_in.shape[1]
    NB, bs = k_pool.shape[0], k_pool.shape[1]
    if q_out is None:
        q_out = torch.empty_like(q_in)
    f32 = torch.float32
    args = (
        _dev_ptr(q_in, "q_in", dtype=f32, ndim=3), _dev_ptr(k_in, "k_in", dtype=f32, ndim=3),
        _dev_ptr(v_in, "v_in", dtype=f32, ndim=3), _dev_ptr(q_out, "q_out", dtype=f32, ndim=3),
        _dev_ptr(k_pool, "k_pool", ndim=4, elem_size=_pool_elem(k_pool, dtype)),
        _dev_ptr(v_pool, "v_pool", ndim=4, elem_size=_pool_elem(k_pool, dtype)),
        _dev_ptr(block_tables, "block_tables", dtype=torch.int32, ndim=2), block_tables.shape[1],
        _dev_ptr(positions, "positions", dtype=torch.int32, ndim=1),
        _dev_ptr(q_norm_w, "q_norm_w", dtype=f32), _dev_ptr(k_norm_w, "k_norm_w", dtype=f32),
        float(eps), float(theta), B, Hq, Hkv, D, bs, NB, pool_dtype_code(k_pool, dtype),
        _lib.variant(rope_dim, v_norm, rope_on_read=rope_on_read), _stream(stream))
    _lib.check(_lib.load().pkv_kv_append(*args), "pkv_kv_append")
    return q_out


def decode_split_tokens(B, Hq, Hkv, D, block_size, max_context_len) -> int:
    return _lib.load().pkv_decode_split_tokens(B, Hq, Hkv, D, block_size, max_context_len)


def decode_workspace_bytes(B, Hq, Hkv, D, block_size, max_context_len,
                           split_tokens: int = 0) -> int:
    return _lib.load().pkv_decode_workspace_bytes(B, Hq, Hkv, D, block_size, max_context_len,
                                                  split_tokens)


def decode_schedule_split(B, Hq, Hkv, D, block_size, max_context_len, dtype_code: int,
                          rope_on_read: bool = False, rope_dim: int = 0) -> int:
    """split_tokens to size a decode workspace with when the call passes split_tokens = 0:
    0 (the library picks the schedule pkv_decode_workspace_bytes sizes for), except for rotation
    at read or float32 pools where the library runs the partitioned vector-ALU kernel with
    min(pkv_decode_split_tokens(...), 576) tokens per partition: shapes the matrix-core tile does not
    serve (head_dim other than 64 / 128, or rotated dims not a multiple of 64), and small query
    groups, where the vector ALU is faster (G = Hq / Hkv below 3, or G = 1 for float32 pools
    without rotation)."""
    read_dim = (rope_dim or D) if rope_on_read else 0
    special = rope_on_read or dtype_code == PKV_F32
    G = Hq // Hkv if Hkv else 0
    tile_ok = D in (64, 128) and read_dim % 64 == 0
    pays = G >= 3 or (dtype_code == PKV_F32 and read_dim == 0 and G == 2)
    if special and not (tile_ok and pays):
        # the library's partition length for that kernel (kValuSplitMax in pkv_api.hip)
        return min(decode_split_tokens(B, Hq, Hkv, D, block_size, max_context_len), 576)
    return 0


def paged_attn_decode(q, k_pool, v_pool, block_tables, context_lens, max_context_len: int,
                      scale: float, *, out=None, workspace=None, split_tokens: int = 0,
                      dtype=None, window: int = 0, rope_on_read: bool = False,
                      read_theta: float = 0.0, rope_dim: int = 0, stream=None):
    """Decode attention for one query token per sequence; returns out [B, Hq, D] float32.

    window: 0, or W > 0 to attend only the last W of each sequence's context_lens tokens.
    rope_on_read: the pool holds un-rotated keys; the query is rotated to position L - 1 and
    key t to position t (base read_theta, rotary dims rope_dim, 0 = D) inside the kernel.
    workspace: uint8 GPU tensor of >= decode_workspace_bytes(...) bytes, zero-filled before its
    first use (the library keeps its counters zero); allocated here (zeroed) if None.
    """
    torch = _torch()
    B, Hq, D = q.shape
    NB, bs, Hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    if out is None:
        out = torch.empty_like(q)
    if not split_tokens and B and max_context_len:
        split_tokens = decode_schedule_split(B, Hq, Hkv, D, bs, max_context_len,
                                             pool_dtype_code(k_pool, dtype), rope_on_read,
                                             rope_dim)
    need = decode_workspace_bytes(B, Hq, Hkv, D, bs, max_context_len, split_tokens) if B else 0
    if workspace is None and need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev_ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    f32 = torch.float32
    args = (
        _dev_ptr(q, "q", dtype=f32, ndim=3),
        _dev_ptr(k_pool, "k_pool", ndim=4, elem_size=_pool_elem(k_pool, dtype)),
        _dev_ptr(v_pool, "v_pool", ndim=4, elem_size=_pool_elem(k_pool, dtype)),
        _dev_ptr(block_tables, "block_tables", dtype=torch.int32, ndim=2), block_tables.shape[1],
        _dev_ptr(context_lens, "context_lens", dtype=torch.int32, ndim=1), int(max_context_len),
        float(scale), _dev_ptr(out, "out", dtype=f32, ndim=3), ws_ptr, ws_bytes,
        int(split_tokens), B, Hq, Hkv, D, bs, NB, pool_dtype_code(k_pool, dtype),
        _lib.variant(rope_dim=rope_dim, window=window, rope_on_read=rope_on_read,
                     read_theta=read_theta), _stream(stream))
    _lib.check(_lib.load().pkv_paged_attn_decode(*args), "pkv_paged_attn_decode")
    return out


def decode_step_workspace_bytes(B, Hq, Hkv, D, block_size, max_blocks_per_seq) -> int:
    return _lib.load().pkv_decode_step_workspace_bytes(B, Hq, Hkv, D, block_size,
                                                       max_blocks_per_seq)


def decode_step(q_in, k_in, v_in, k_pool, v_pool, block_tables, positions, *, theta: float,
                scale: float, q_norm_w=None, k_norm_w=None, eps: float = 1e-6, q_out=None,
                out=None, workspace=None, dtype=None, rope_dim: int = 0, v_norm: bool = False,
                window: int = 0, stream=None):
    """One layer's decode step in one launch: append the new token of every sequence, then
    attend over positions + 1 tokens. Returns (q_out, out), both [B, Hq, D] float32.
    rope_dim / v_norm as for kv_append, window as for paged_attn_decode.

    workspace: uint8 GPU tensor of >= decode_step_workspace_bytes(...) bytes, zero-filled before
    its first use; allocated here (zeroed) if None.
    """
    torch = _torch()
    B, Hq, D = q_in.shape
    Hkv = k_in.shape[1]
    NB, bs = k_pool.shape[0], k_pool.shape[1]
    if q_out is None:
        q_out = torch.empty_like(q_in)
    if out is None:
        out = torch.empty_like(q_in)
    need = decode_step_workspace_bytes(B, Hq, Hkv, D, bs, block_tables.shape[1]) if B else 0
    if workspace is None and need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q_in.device)
    ws_ptr = _dev_ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    f32 = torch.float32
    args = (
        _dev_ptr(q_in, "q_in", dtype=f32, ndim=3), _dev_ptr(k_in, "k_in", dtype=f32, ndim=3),
        _dev_ptr(v_in, "v_in", dtype=f32, ndim=3), _dev_ptr(q_out, "q_out", dtype=f32, ndim=3),
        _dev_ptr(k_pool, "k_pool", ndim=4, elem_size=_pool_elem(k_pool, dtype)),
        _dev_ptr(v_pool, "v_pool", ndim=4, elem_size=_pool_elem(k_pool, dtype)),
        _dev_ptr(block_tables, "block_tables", dtype=torch.int32, ndim=2), block_tables.shape[1],
        _dev_ptr(positions, "positions", dtype=torch.int32, ndim=1),
        _dev_ptr(q_norm_w, "q_norm_w", dtype=f32), _dev_ptr(k_norm_w, "k_norm_w", dtype=f32),
        float(eps), float(theta), float(scale), _dev_ptr(out, "out", dtype=f32, ndim=3),
        ws_ptr, ws_bytes, B, Hq, Hkv, D, bs, NB, pool_dtype_code(k_pool, dtype),
        _lib.variant(rope_dim, v_norm, window), _stream(stream))
    _lib.check(_lib.load().pkv_decode_step(*args), "pkv_decode_step")
    return q_out, out


def decode_step_noalloc(q_in, k_in, v_in, k_pool, v_pool, block_tables, positions, *,
                        theta: float, scale: float, q_out, out, q_norm_w=None, k_norm_w=None,
                        eps: float = 1e-6, dtype=None, rope_dim: int = 0, v_norm: bool = False,
                        window: int = 0, stream=None):
    """decode_step without a workspace: the library's own per-GPU scratch array holds the
    merge counters and partial pieces, and nothing is allocated (q_out and out are the
    caller's). Calls that overlap in time on one GPU race. Returns (q_out, out)."""
    torch = _torch()
    B, Hq, D = q_in.shape
    Hkv = k_in.shape[1]
    NB, bs = k_pool.shape[0], k_pool.shape[1]
    f32 = torch.float32
    args = (
        _dev_ptr(q_in, "q_in", dtype=f32, ndim=3), _dev_ptr(k_in, "k_in", dtype=f32, ndim=3),
        _dev_ptr(v_in, "v_in", dtype=f32, ndim=3), _dev_ptr(q_out, "q_out", dtype=f32, ndim=3),
        _dev_ptr(k_pool, "k_pool", ndim=4, elem_size=_pool_elem(k_pool, dtype)),
        _dev_ptr(v_pool, "v_pool", ndim=4, elem_size=_pool_elem(k_pool, dtype)),
        _dev_ptr(block_tables, "block_tables", dtype=torch.int32, ndim=2), block_tables.shape[1],
        _dev_ptr(positions, "positions", dtype=torch.int32, ndim=1),
        _dev_ptr(q_norm_w, "q_norm_w", dtype=f32), _dev_ptr(k_norm_w, "k_norm_w", dtype=f32),
        float(eps), float(theta), float(scale), _dev_ptr(out, "out", dtype=f32, ndim=3),
        B, Hq, Hkv, D, bs, NB, pool_dtype_code(k_pool, dtype),
        _lib.variant(rope_dim, v_norm, window), _stream(stream))
    _lib.check(_lib.load().pkv_decode_step_noalloc(*args), "pkv_decode_step_noalloc")
    return q_out, out


def decode_step_noalloc_scratch_bytes() -> int:
    return _lib.load().pkv_decode_step_noalloc_scratch_bytes()


def append_then_decode(q_in, k_in, v_in, k_pool, v_pool, block_tables, positions, context_lens,
                       max_context_len: int, *, theta: float, scale: float, q_norm_w=None,
                       k_norm_w=None, eps: float = 1e-6, q_out=None, out=None, workspace=None,
                       split_tokens: int = 0, dtype=None, rope_dim: int = 0,
                       v_norm: bool = False, window: int = 0, stream=None):
    """The same step as two calls (kv_append, then paged_attn_decode). Returns (q_out, out)."""
    q_out = kv_append(q_in, k_in, v_in, k_pool, v_pool, block_tables, positions, theta=theta,
                      q_norm_w=q_norm_w, k_norm_w=k_norm_w, eps=eps, q_out=q_out, dtype=dtype,
                      rope_dim=rope_dim, v_norm=v_norm, stream=stream)
    out = paged_attn_decode(q_out, k_pool, v_pool, block_tables, context_lens, max_context_len,
                            scale, out=out, workspace=workspace, split_tokens=split_tokens,
                            dtype=dtype, window=window, stream=stream)
    return q_out, out


def validate_tables(block_tables, positions, context_lens, block_size: int, num_blocks: int,
                    max_context_len: int) -> None:
    """Host-side precondition check (numpy int32 arrays or None); raises PkvError."""
    import numpy as np

    def ptr(a):
        return None if a is None else np.ascontiguousarray(a, dtype=np.int32)

    t, p, c = ptr(block_tables), ptr(positions), ptr(context_lens)
    B = next(len(x) for x in (t, p, c) if x is not None)
    st = _lib.load().pkv_validate_tables(
        None if t is None else t.ctypes.data, t.shape[1] if t is not None else 1,
        None if p is None else p.ctypes.data, None if c is None else c.ctypes.data, B,
        block_size, num_blocks, max_context_len)
    _lib.check(st, "pkv_validate_tables")


def prefill_append(q_in, k_in, v_in, k_pool, v_pool, block_tables, cu_seqlens, start_pos, *,
                   theta: float, q_norm_w=None, k_norm_w=None, eps: float = 1e-6, q_out=None,
                   dtype=None, rope_dim: int = 0, v_norm: bool = False, stream=None):
    """Append a chunk of tokens per sequence; returns q_out ([N, Hq, D] float32).

    q_in [N,Hq,D], k_in / v_in [N,Hkv,D] float32 token-major; cu_seqlens [B+1] int32 (rows of
    sequence b are cu_seqlens[b] .. cu_seqlens[b+1]-1); start_pos [B] int32 (position of the
    chunk's first token). rope_dim / v_norm as for kv_append.
    """
    torch = _torch()
    N, Hq, D = q_in.shape
    Hkv = k_in.shape[1]
    B = start_pos.shape[0]
    NB, bs = k_pool.shape[0], k_pool.shape[1]
    if q_out is None:
        q_out = torch.empty_like(q_in)
    f32 = torch.float32
    args = (
        _dev_ptr(q_in, "q_in", dtype=f32, ndim=3), _dev_ptr(k_in, "k_in", dtype=f32, ndim=3),
        _dev_ptr(v_in, "v_in", dtype=f32, ndim=3), _dev_ptr(q_out, "q_out", dtype=f32, ndim=3),
        _dev_ptr(k_pool, "k_pool", ndim=4, elem_size=_pool_elem(k_pool, dtype)),
        _dev_ptr(v_pool, "v_pool", ndim=4, elem_size=_pool_elem(k_pool, dtype)),
        _dev_ptr(block_tables, "block_tables", dtype=torch.int32, ndim=2), block_tables.shape[1],
        _dev_ptr(cu_seqlens, "cu_seqlens", dtype=torch.int32, ndim=1),
        _dev_ptr(start_pos, "start_pos", dtype=torch.int32, ndim=1),
        _dev_ptr(q_norm_w, "q_norm_w", dtype=f32), _dev_ptr(k_norm_w, "k_norm_w", dtype=f32),
        float(eps), float(theta), B, N, Hq, Hkv, D, bs, NB, pool_dtype_code(k_pool, dtype),
        _lib.variant(rope_dim, v_norm), _stream(stream))
    _lib.check(_lib.load().pkv_prefill_append(*args), "pkv_prefill_append")
    return q_out


def prefill_workspace_bytes(B, Hq, Hkv, D, block_size, max_chunk, max_context_len) -> int:
    return _lib.load().pkv_prefill_workspace_bytes(B, Hq, Hkv, D, block_size, max_chunk,
                                                   max_context_len)


def paged_attn_prefill(q, k_pool, v_pool, block_tables, cu_seqlens, start_pos, max_chunk: int,
                       max_context_len: int, scale: float, *, out=None, workspace=None,
                       dtype=None, window: int = 0, stream=None):
    """Causal attention of a chunk of query tokens per sequence; returns out [N, Hq, D].
    window: 0, or W > 0 so that the row at position p attends positions p - W + 1 .. p only.

    workspace: uint8 GPU tensor of >= prefill_workspace_bytes(...) bytes, zero-filled before
    its first use; allocated here (zeroed) if None and needed.
    """
    torch = _torch()
    N, Hq, D = q.shape
    B = start_pos.shape[0]
    NB, bs, Hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    if out is None:
        out = torch.empty_like(q)
    need = prefill_workspace_bytes(B, Hq, Hkv, D, bs, max_chunk, max_context_len) \
        if B and N and max_chunk and max_context_len else 0
    if workspace is None and need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev_ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    f32 = torch.float32
    args = (
        _dev_ptr(q, "q", dtype=f32, ndim=3),
        _dev_ptr(k_pool, "k_pool", ndim=4, elem_size=_pool_elem(k_pool, dtype)),
        _dev_ptr(v_pool, "v_pool", ndim=4, elem_size=_pool_elem(k_pool, dtype)),
        _dev_ptr(block_tables, "block_tables", dtype=torch.int32, ndim=2), block_tables.shape[1],
        _dev_ptr(cu_seqlens, "cu_seqlens", dtype=torch.int32, ndim=1),
        _dev_ptr(start_pos, "start_pos", dtype=torch.int32, ndim=1), int(max_chunk),
        int(max_context_len), float(scale), _dev_ptr(out, "out", dtype=f32, ndim=3), ws_ptr,
        ws_bytes, B, N, Hq, Hkv, D, bs, NB, pool_dtype_code(k_pool, dtype),
        _lib.variant(window=window), _stream(stream))
    _lib.check(_lib.load().pkv_paged_attn_prefill(*args), "pkv_paged_attn_prefill")
    return out


def prefill_step(q_in, k_in, v_in, k_pool, v_pool, block_tables, cu_seqlens, start_pos,
                 max_chunk: int, max_context_len: int, *, theta: float, scale: float,
                 q_norm_w=None, k_norm_w=None, eps: float = 1e-6, q_out=None, out=None,
                 workspace=None, dtype=None, rope_dim: int = 0, v_norm: bool = False,
                 window: int = 0, stream=None):
    """pkv_prefill_append then pkv_paged_attn_prefill on the same stream; returns
    (q_out, out)."""
    q_out = prefill_append(q_in, k_in, v_in, k_pool, v_pool, block_tables, cu_seqlens,
                           start_pos, theta=theta, q_norm_w=q_norm_w, k_norm_w=k_norm_w,
                           eps=eps, q_out=q_out, dtype=dtype, rope_dim=rope_dim, v_norm=v_norm,
                           stream=stream)
    out = paged_attn_prefill(q_out, k_pool, v_pool, block_tables, cu_seqlens, start_pos,
                             max_chunk, max_context_len, scale, out=out, workspace=workspace,
                             dtype=dtype, window=window, stream=stream)
    return q_out, out
