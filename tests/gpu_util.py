"""Helpers for the GPU parity tests: upload a workload, run the HIP path through the C ABI,
compare with the oracle.

Tolerance (fp32 outputs): |gpu - ref| <= 1e-3 + 2e-3 * |ref| elementwise on finite references;
non-finite references must match in kind (NaN <-> NaN, +Inf <-> +Inf, -Inf <-> -Inf).
Stored pools: bit-identical over the whole pool.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import paged_kv_cache_315_amd as pkv

ATOL = 1e-3
RTOL = 2e-3


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def upload(wl: dict, device="cuda:0") -> dict:
    def t(a, dt=None):
        return torch.from_numpy(np.ascontiguousarray(a if dt is None else a.view(dt))).to(device)

    d = {
        "q": t(wl["q"]), "k_new": t(wl["k_new"]), "v_new": t(wl["v_new"]),
        "k_pool": t(wl["k_pool"], np.int16), "v_pool": t(wl["v_pool"], np.int16),
        "tables": t(wl["tables"]), "positions": t(wl["positions"]),
        "context_lens": t(wl["context_lens"]),
        "q_norm_w": None if wl["q_norm_w"] is None else t(wl["q_norm_w"]),
        "k_norm_w": None if wl["k_norm_w"] is None else t(wl["k_norm_w"]),
    }
    return d


def gpu_step(wl: dict, dev: dict, split_tokens: int = 0, fused: bool = False):
    """One decode step on the GPU; returns (q_out, out) as host arrays (pools stay in dev).
    fused: the one-launch pkv_decode_step; otherwise pkv_kv_append then pkv_paged_attn_decode
    (split_tokens 0 = balanced schedule, > 0 = partitions of that many tokens)."""
    if fused:
        q_out, out = pkv.decode_step(
            dev["q"], dev["k_new"], dev["v_new"], dev["k_pool"], dev["v_pool"], dev["tables"],
            dev["positions"], theta=wl["theta"], scale=wl["scale"], q_norm_w=dev["q_norm_w"],
            k_norm_w=dev["k_norm_w"], eps=wl["eps"], dtype=wl["dtype"])
    else:
        q_out, out = pkv.append_then_decode(
            dev["q"], dev["k_new"], dev["v_new"], dev["k_pool"], dev["v_pool"], dev["tables"],
            dev["positions"], dev["context_lens"], wl["max_context_len"], theta=wl["theta"],
            scale=wl["scale"], q_norm_w=dev["q_norm_w"], k_norm_w=dev["k_norm_w"], eps=wl["eps"],
            split_tokens=split_tokens, dtype=wl["dtype"])
    torch.cuda.synchronize()
    return q_out.cpu().numpy(), out.cpu().numpy()


def pool_host(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def assert_close(got: np.ndarray, ref: np.ndarray, what: str):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    fin = np.isfinite(ref)
    # non-finite pattern
    assert np.array_equal(np.isnan(got), np.isnan(ref)), \
        f"{what}: NaN pattern differs ({np.isnan(got).sum()} vs {np.isnan(ref).sum()})"
    inf = np.isinf(ref)
    assert np.array_equal(got[inf], ref[inf]), f"{what}: Inf pattern differs"
    assert np.all(np.isfinite(got[fin])), f"{what}: non-finite where the oracle is finite"
    err = np.abs(got[fin].astype(np.float64) - ref[fin].astype(np.float64))
    bound = ATOL + RTOL * np.abs(ref[fin].astype(np.float64))
    bad = err > bound
    if bad.any():
        i = np.argmax(err - bound)
        raise AssertionError(f"{what}: {bad.sum()} of {fin.sum()} outside tolerance; worst "
                             f"got={got[fin][i]} ref={ref[fin][i]} err={err[i]:.3g}")


def assert_pools_equal(got: np.ndarray, ref: np.ndarray, what: str):
    if not np.array_equal(got, ref):
        diff = np.argwhere(got != ref)
        raise AssertionError(f"{what}: {len(diff)} codes differ, first at {tuple(diff[0])}: "
                             f"got {got[tuple(diff[0])]:#06x} ref {ref[tuple(diff[0])]:#06x}")
