"""Benchmark of one decode step (KV append + paged-attention decode) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 2] [--copies R] [--no-cpu-baseline]

A step is one pass of the whole path over one batch: pkv_decode_step (the append of every
sequence's new token and the paged-attention decode, in one kernel launch), on the
Llama-3-8B-shaped workload by default (32 sequences, cached
lengths U{512..4096}, 32 query / 8 KV heads, head_dim 128, block_size 16, bf16 pool,
RoPE theta 5e5). Inputs are seeded synthetic data resident in HBM before timing starts.
The pools exist in R identical copies and step i uses copy i % R, so the K/V stream of one
step is not still in the 256 MB last-level cache from the previous step.

Prints ONE JSON line. `value` is the step's algorithmic bytes over the step time (GB/s); the
step is one kernel launch, so `roofline` reports that kernel (HIP events on its stream around
the timed steps); `decode_only` times pkv_paged_attn_decode alone on the same inputs; `cpu_baseline` is the single-threaded CPU oracle on one full step of the same
workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ("paged_kv_cache_315_amd/csrc/decode_balanced.hip",
                  "paged_kv_cache_315_amd/csrc/pkv_device.h",
                  "paged_kv_cache_315_amd/csrc/pkv_internal.h")


def profiled_traffic(workload: str):
    """HBM bytes per launch of the step kernel measured with rocprofv3 counters
    (profiles/decode_step_<workload>.md), or None when there is no such profile or the kernel
    sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"decode_step_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", " ")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if fields.get("kernel_sources_sha256") != h.hexdigest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(wl: dict) -> dict:
    """Bytes the step must move (each input read once, each output written once)."""
    B, Hq, Hkv, D, bs = wl["B"], wl["Hq"], wl["Hkv"], wl["D"], wl["bs"]
    L = wl["context_lens"].astype(np.int64)
    kv = int(L.sum()) * 2 * Hkv * D * 2
    tables = int(((L + bs - 1) // bs).sum()) * 4
    decode = kv + B * Hq * D * 4 * 2 + tables + B * 4
    norm = 2 * D * 4 if wl["q_norm_w"] is not None else 0
    append = B * (Hq + 2 * Hkv) * D * 4 + B * Hq * D * 4 + 2 * B * Hkv * D * 2 + B * 4 * 2 + norm
    return {"kv": kv, "decode": decode, "append": append, "step": decode + append}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--copies", type=int, default=0, help="pool copies (0: enough for >= 1 GB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy a 1 GiB device buffer 5 times (a known-size kernel that the "
                         "HBM byte counters are scaled by)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the decode step "
              "has no multi-GPU path in this library", file=sys.stderr)
        return 2

    import torch
    import paged_kv_cache_315_amd as pkv
    from paged_kv_cache_315_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": 1 << 30,
                          "bytes_written_per_copy": 1 << 30, "copies": 5}))
        return 0
    pkv._lib.load()  # fail loudly before any work if the HIP library is missing

    wl = W.config(args.config)
    nbytes = algorithmic_bytes(wl)
    dev = torch.device("cuda:0")

    def t(a, dt=None):
        return torch.from_numpy(np.ascontiguousarray(a if dt is None else a.view(dt))).to(dev)

    q, k_new, v_new = t(wl["q"]), t(wl["k_new"]), t(wl["v_new"])
    tables, positions, ctx = t(wl["tables"]), t(wl["positions"]), t(wl["context_lens"])
    qn = None if wl["q_norm_w"] is None else t(wl["q_norm_w"])
    kn = None if wl["k_norm_w"] is None else t(wl["k_norm_w"])
    pool_bytes = 2 * wl["k_pool"].nbytes
    copies = args.copies or max(2, int(np.ceil(1.0e9 / pool_bytes)))
    k0, v0 = t(wl["k_pool"], np.int16), t(wl["v_pool"], np.int16)
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(copies - 1)]
    B, Hq, Hkv, D = wl["B"], wl["Hq"], wl["Hkv"], wl["D"]
    split = args.split_tokens
    ws_bytes = max(pkv.decode_workspace_bytes(B, Hq, Hkv, D, wl["bs"], wl["max_context_len"], split),
                   pkv.decode_step_workspace_bytes(B, Hq, Hkv, D, wl["bs"], wl["max_blocks"]))
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    q_out = torch.empty_like(q)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def step(i):
        kp, vp = pools[i % copies]
        pkv.decode_step(q, k_new, v_new, kp, vp, tables, positions, theta=wl["theta"],
                        scale=wl["scale"], q_norm_w=qn, k_norm_w=kn, eps=wl["eps"], q_out=q_out,
                        out=out, workspace=ws, dtype=wl["dtype"], stream=stream)

    def decode_only(i):
        kp, vp = pools[i % copies]
        pkv.paged_attn_decode(q_out, kp, vp, tables, ctx, wl["max_context_len"], wl["scale"],
                              out=out, workspace=ws, split_tokens=split, dtype=wl["dtype"],
                              stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # the paged-decode call alone, back to back over the pool copies
    for i in range(args.warmup):
        decode_only(i)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        decode_only(i)
    e1.record(stream)
    torch.cuda.synchronize()
    decode_ms = e0.elapsed_time(e1) / args.steps

    step_gbs = nbytes["step"] / (ms_per_step * 1e-3) / 1e9
    traffic_bytes = profiled_traffic(wl["name"]) if args.split_tokens == 0 else None
    tokens_per_s = B / (ms_per_step * 1e-3)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.load()
        c0 = time.perf_counter()
        oracle.decode_step(wl)
        cpu_s = time.perf_counter() - c0
        cpu = {"value": round(nbytes["step"] / cpu_s / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"one full step of the {wl['name']} workload ({B} sequences), "
                         f"{cpu_s:.2f} s single-threaded; {B / cpu_s:.2f} tokens/s"}

    line = {
        "metric": "paged-attn decode achieved HBM GB/s (% of peak) + tokens/s, B=32 ctx<=4K",
        "value": round(step_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl["dtype"],
        "data": "synthetic",
        "pct_of_peak": round(100 * step_gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(tokens_per_s, 1),
        "config": {
            "workload": wl["name"], "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv,
            "head_dim": D, "block_size": wl["bs"], "kv_dtype": wl["dtype"],
            "context_tokens": int(wl["context_lens"].sum()),
            "max_context_len": wl["max_context_len"], "rope_theta": wl["theta"],
            "qk_norm": wl["q_norm_w"] is not None, "pool_copies": copies,
            "split_tokens": split or pkv.decode_split_tokens(B, Hq, Hkv, D, wl["bs"],
                                                             wl["max_context_len"]),
            "bytes_per_step": nbytes["step"], "kv_bytes": nbytes["kv"],
        },
        # the step is one launch of the fused kernel, so the step time is its launch time;
        # traffic = rocprofv3-measured HBM bytes per launch over the same launch time
        "roofline": {
            "bound": "hbm", "kernel": "decode_balanced_kernel (append fused, pkv_decode_step)",
            "achieved": round(step_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(step_gbs / HBM_PEAK_GBS, 4),
            "traffic": (None if traffic_bytes is None
                        else round(traffic_bytes / (ms_per_step * 1e-3) / 1e9, 2)),
            "traffic_bytes_per_launch": traffic_bytes,
            "bytes_per_launch": nbytes["step"], "avg_launch_us": round(ms_per_step * 1e3, 3),
        },
        "decode_only": {"kernel": "pkv_paged_attn_decode", "avg_launch_us": round(decode_ms * 1e3, 3),
                        "gb_per_s": round(nbytes["decode"] / (decode_ms * 1e-3) / 1e9, 2)},
        "cpu_baseline": cpu,
        "wall_ms_timed_steps": round(wall_ms, 2),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
