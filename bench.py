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
                  "paged_kv_cache_315_amd/csrc/decode_tile.h",
                  "paged_kv_cache_315_amd/csrc/pkv_device.h",
                  "paged_kv_cache_315_amd/csrc/pkv_internal.h")


def host_cpu() -> dict:
    """The host's logical core count and CPU model (for the CPU baseline's context)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"of_cores": os.cpu_count(), "cpu_model": model}


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


def algorithmic_bytes(wl: dict, window: int = 0) -> dict:
    """Bytes the step must move (each input read once, each output written once); with a
    sliding window only the last `window` tokens of each sequence are read."""
    B, Hq, Hkv, D, bs = wl["B"], wl["Hq"], wl["Hkv"], wl["D"], wl["bs"]
    L = wl["context_lens"].astype(np.int64)
    if window:
        L = np.minimum(L, window)
    E = 4 if wl["dtype"] == "f32" else 2           # bytes per pool element
    kv = int(L.sum()) * 2 * Hkv * D * E
    tables = int(((L + bs - 1) // bs).sum()) * 4
    decode = kv + B * Hq * D * 4 * 2 + tables + B * 4
    norm = 2 * D * 4 if wl["q_norm_w"] is not None else 0
    append = B * (Hq + 2 * Hkv) * D * 4 + B * Hq * D * 4 + 2 * B * Hkv * D * E + B * 4 * 2 + norm
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
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="--workload rope|f32: KV heads of the workload (query heads kept; "
                         "0: the workload's own), to compare group sizes")
    ap.add_argument("--window", type=int, default=0,
                    help="decode step with a sliding window of this many tokens (layer variant)")
    ap.add_argument("--rope-dim", type=int, default=0,
                    help="decode step with partial rotary over this many dims (layer variant)")
    ap.add_argument("--v-norm", action="store_true",
                    help="decode step with per-head V normalisation (layer variant)")
    ap.add_argument("--workload", choices=["decode", "prefill", "spec", "rope", "f32", "blocks"],
                    default="decode",
                    help="decode: the decode step (default); prefill / spec: chunked prefill "
                         "(4 x 512-token chunks) / 4 draft tokens per sequence, append + "
                         "causal paged attention; rope: the decode step with RoPE applied at "
                         "read (un-rotated pool), append + decode; f32: the decode step over "
                         "float32 pools, append + decode; blocks: the host block manager "
                         "(admission with a shared prefix, per-step growth and tables)")
    ap.add_argument("--timeline", action="store_true",
                    help="decode workloads: per-workgroup phase stamps of the fused step from the "
                         "profiling build libpkv_timeline.so (python -m "
                         "paged_kv_cache_315_amd.build --timeline); prints the start / stream / "
                         "tail breakdown instead of the bench line")
    ap.add_argument("--pool-offset", default="0,0",
                    help="K,V: bytes by which each pool copy starts past a 4 KiB-aligned "
                         "allocation (the caller's pool placement; decode workloads)")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="only time a plain streaming read (torch's float32 sum) of the step's "
                         "K/V byte count and of 2 GiB, over rotating buffers: context for the "
                         "decode's rate, not a figure of this library")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy a 1 GiB device buffer 5 times (a known-size kernel that the "
                         "HBM byte counters are scaled by)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the decode step "
              "has no multi-GPU path in this library", file=sys.stderr)
        return 2

    if args.workload == "blocks":
        return run_blocks(args)
    if args.timeline:
        os.environ.setdefault("PKV_LIBRARY", os.path.join(ROOT, "paged_kv_cache_315_amd",
                                                          "libpkv_timeline.so"))

    import torch
    import paged_kv_cache_315_amd as pkv
    from paged_kv_cache_315_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.read_ceiling:
        res = {}
        for name, nbytes_ in (("llama3-8b K/V (296 MB)", 296108032), ("2 GiB", 1 << 31)):
            n = nbytes_ // 4
            copies = max(2, int(np.ceil(1.2e9 / nbytes_)))
            bufs = [torch.ones(n, dtype=torch.float32, device="cuda:0") for _ in range(copies)]
            for i in range(5):
                bufs[i % copies].sum()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 50
            e0.record()
            for i in range(reps):
                bufs[i % copies].sum()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            res[name] = {"us": round(us, 2), "GB_per_s": round(nbytes_ / (us * 1e-6) / 1e9, 1)}
            del bufs
        print(json.dumps({"read_ceiling": "torch float32 sum over rotating buffers", **res}))
        return 0
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
    if args.workload in ("rope", "f32"):
        return run_rope(args, torch, pkv, W)
    if args.workload != "decode":
        return run_prefill(args, torch, pkv, W)

    wl = W.config(args.config)
    nbytes = algorithmic_bytes(wl, args.window)
    variant = dict(rope_dim=args.rope_dim, v_norm=args.v_norm, window=args.window)
    has_variant = bool(args.window or args.rope_dim or args.v_norm)
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
    k_off, v_off = (int(x) for x in args.pool_offset.split(","))

    def placed(x, off_bytes):
        """A copy of pool x starting off_bytes past a 4 KiB-aligned allocation."""
        if off_bytes == 0:
            return x.clone()
        assert off_bytes % 16 == 0, "pool offsets must keep 16-byte rows aligned"
        n = x.numel() + (4096 + off_bytes) // 2
        buf = torch.empty(n, dtype=x.dtype, device=x.device)
        skip = ((-buf.data_ptr()) % 4096 + off_bytes) // 2
        y = buf[skip:skip + x.numel()].view(x.shape)
        y.copy_(x)
        return y

    if k_off or v_off:
        pools = [(placed(k0, k_off), placed(v0, v_off)) for _ in range(copies)]
    else:
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
                        out=out, workspace=ws, dtype=wl["dtype"], stream=stream, **variant)

    if args.timeline:
        return run_timeline(args, torch, pkv, wl, step)

    def decode_only(i):
        kp, vp = pools[i % copies]
        pkv.paged_attn_decode(q_out, kp, vp, tables, ctx, wl["max_context_len"], wl["scale"],
                              out=out, workspace=ws, split_tokens=split, dtype=wl["dtype"],
                              window=args.window, stream=stream)

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

    # per-launch distribution of the step: one event pair around each of 200 launches (a
    # separate pass; the timed K steps above are back to back with no events between them)
    n_lat = min(200, max(args.steps, 1))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_lat)]
    for i in range(n_lat):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    lat_us = np.array([s.elapsed_time(e) * 1e3 for s, e in ev])
    lat = {"p10": round(float(np.percentile(lat_us, 10)), 2),
           "p50": round(float(np.percentile(lat_us, 50)), 2),
           "p90": round(float(np.percentile(lat_us, 90)), 2), "launches": n_lat}

    step_gbs = nbytes["step"] / (ms_per_step * 1e-3) / 1e9
    traffic_bytes = (profiled_traffic(wl["name"]) if args.split_tokens == 0 and not has_variant
                     else None)
    tokens_per_s = B / (ms_per_step * 1e-3)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.load()
        c0 = time.perf_counter()
        oracle.decode_step(wl, rope_dim=args.rope_dim or None, v_norm=args.v_norm,
                           window=args.window)
        cpu_s = time.perf_counter() - c0
        cpu = {"value": round(nbytes["step"] / cpu_s / 1e9, 4), "unit": "GB/s", "cores": 1,
               **host_cpu(), "kind": "oracle",
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
            "workload": wl["name"] + ("-variant" if has_variant else ""), "batch": B,
            "num_q_heads": Hq, "num_kv_heads": Hkv, "window": args.window,
            "rope_dim": args.rope_dim or D, "v_norm": args.v_norm,
            "head_dim": D, "block_size": wl["bs"], "kv_dtype": wl["dtype"],
            "context_tokens": int(wl["context_lens"].sum()),
            "max_context_len": wl["max_context_len"], "rope_theta": wl["theta"],
            "qk_norm": wl["q_norm_w"] is not None, "pool_copies": copies,
            "schedule": "partitioned" if split else "balanced", "split_tokens": split,
            "pool_offset_bytes": args.pool_offset,
            "bytes_per_step": nbytes["step"], "kv_bytes": nbytes["kv"],
        },
        # the step is one launch of the fused kernel, so the step time is its launch time;
        # traffic = rocprofv3-measured HBM bytes per launch over the same launch time
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_balanced_kernel (append fused, pkv_decode_step" +
                      (", variant fields read at run time)" if has_variant else ")"),
            "achieved": round(step_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(step_gbs / HBM_PEAK_GBS, 4),
            "traffic": (None if traffic_bytes is None
                        else round(traffic_bytes / (ms_per_step * 1e-3) / 1e9, 2)),
            "traffic_bytes_per_launch": traffic_bytes,
            "bytes_per_launch": nbytes["step"], "avg_launch_us": round(ms_per_step * 1e3, 3),
        },
        "step_launch_us": lat,
        "decode_only": {"kernel": "pkv_paged_attn_decode", "avg_launch_us": round(decode_ms * 1e3, 3),
                        "gb_per_s": round(nbytes["decode"] / (decode_ms * 1e-3) / 1e9, 2)},
        "cpu_baseline": cpu,
        "wall_ms_timed_steps": round(wall_ms, 2),
    }
    print(json.dumps(line), flush=True)
    return 0


def run_timeline(args, torch, pkv, wl, step) -> int:
    """Per-workgroup phase stamps of the fused step (profiling build): where a launch's time
    goes between the first workgroup's start and the last one's end."""
    import ctypes
    lib = pkv._lib.load()
    lib.pkv_timeline_set.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.pkv_timeline_set.restype = None
    n_wg_max, n_st = 2048, 10
    buf = torch.zeros(n_wg_max * n_st, dtype=torch.int64, device="cuda:0")
    lib.pkv_timeline_set(buf.data_ptr(), 0)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    launches = max(1, min(args.steps, 200))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per = []
    ev_us = []
    for i in range(launches):
        buf.zero_()
        e0.record()
        step(i)
        e1.record()
        torch.cuda.synchronize()
        ev_us.append(e0.elapsed_time(e1) * 1e3)
        per.append(buf.cpu().numpy().reshape(n_wg_max, n_st).copy())
    # the same launches with the tile ranges dealt out rotated by a third of the grid: if a
    # workgroup id stays slow it is where it runs; if a range stays slow it is the data
    rot = None
    per_rot = []
    n_wg = int((per[0][:, 0] != 0).sum())
    if n_wg > 2:
        rot = n_wg // 3
        lib.pkv_timeline_set(buf.data_ptr(), rot)
        for i in range(launches):
            buf.zero_()
            step(i)
            torch.cuda.synchronize()
            per_rot.append(buf.cpu().numpy().reshape(n_wg_max, n_st).copy())
    lib.pkv_timeline_set(None, 0)
    tick_us = 0.01  # the real-time counter runs at 100 MHz

    def pct(x, q):
        return float(np.percentile(x, q))

    rows = []
    for t in per:
        t = t[t[:, 0] != 0]
        t0 = t[:, 0].min()
        rel = (t[:, :7].astype(np.float64) - t0) * tick_us
        work = t[:, 8] > 0
        w = rel[work]
        exit_ = rel[:, 6]
        rows.append({
            "span": exit_.max(), "entry_p50": pct(rel[:, 0], 50), "entry_max": rel[:, 0].max(),
            "lengths_p50": pct(w[:, 1] - w[:, 0], 50),
            "prefix_p50": pct(w[:, 2] - w[:, 1], 50),
            "query_p50": pct(w[:, 3] - w[:, 2], 50),
            "first_tile_p50": pct(w[:, 4] - w[:, 3], 50),
            "stream_p10": pct(w[:, 5] - w[:, 4], 10), "stream_p50": pct(w[:, 5] - w[:, 4], 50),
            "stream_p90": pct(w[:, 5] - w[:, 4], 90),
            "merge_p50": pct(w[:, 6] - w[:, 5], 50),
            "exit_p10": pct(exit_[work], 10), "exit_p50": pct(exit_[work], 50),
            "exit_p90": pct(exit_[work], 90), "exit_max": exit_.max(),
            "tail": exit_.max() - pct(exit_[work], 50),
            "units_max": int(t[work, 7].max()), "units_mean": float(t[work, 7].mean()),
            "tiles_per_wg": int(t[work, 8].max()), "workgroups": int(len(t)),
        })
    med = {k: round(float(np.median([r[k] for r in rows])), 2) for k in rows[0]}
    # is a workgroup slow because of where it runs (the same workgroups every launch) or at
    # random? Stream time per workgroup id, its correlation between launches, and by XCD
    # (workgroup ids are dealt round-robin over the 8 XCDs)
    n = min(len(t[t[:, 0] != 0]) for t in per)
    dur = np.array([(t[:n, 5] - t[:n, 4]).astype(np.float64) * tick_us for t in per])
    work = per[0][:n, 8] > 0
    dur = dur[:, work]
    ids = np.arange(n)[work]
    ranks = np.argsort(np.argsort(dur, axis=1), axis=1).astype(np.float64)
    corr = [float(np.corrcoef(ranks[i], ranks[i + 1])[0, 1]) for i in range(len(ranks) - 1)]
    mean_dur = dur.mean(axis=0)
    by_xcd = [round(float(np.median(mean_dur[ids % 8 == x])), 2) for x in range(8)]
    # range of workgroup w (the kernel's XCD-aware deal): per = n // 8 ranges per XCD
    per_x, rem_x = n // 8, n % 8
    rng_of = (ids % 8) * per_x + np.minimum(ids % 8, rem_x) + ids // 8
    by_range_mod8 = [round(float(np.median(mean_dur[rng_of % 8 == k])), 2) for k in range(8)]
    # stream time by the number of units (segment pieces) a workgroup streams
    units = per[0][:n, 7][work].astype(np.int64)
    by_units = {int(u): [int((units == u).sum()), round(float(np.median(mean_dur[units == u])), 2)]
                for u in np.unique(units)}
    half = [round(float(np.median(mean_dur[ids < n // 2])), 2),
            round(float(np.median(mean_dur[ids >= n // 2])), 2)]
    rot_corr = None
    if per_rot:
        d_rot = np.array([(t[:n, 5] - t[:n, 4]).astype(np.float64) * tick_us
                          for t in per_rot])[:, work].mean(axis=0)
        # workgroup ids[i] ran range (ids[i] + rot) % n in the rotated launches
        by_wg = float(np.corrcoef(mean_dur, d_rot)[0, 1])
        by_range = None
        if len(ids) == n:   # every workgroup had a range: range r ran on workgroup r - rot
            same_range = d_rot[(np.arange(n) - rot) % n]
            by_range = round(float(np.corrcoef(mean_dur, same_range)[0, 1]), 3)
        rot_corr = {"rotation": rot, "corr_same_workgroup": round(by_wg, 3),
                    "corr_same_range": by_range}
    print(json.dumps({"timeline": wl["name"], "launches": launches, "rotated": rot_corr,
                      "event_us_median": round(float(np.median(ev_us)), 2),
                      "median_over_launches_us": med,
                      "stream_rank_corr_between_launches": round(float(np.median(corr)), 3)
                      if corr else None,
                      "stream_us_by_xcd": by_xcd, "stream_us_first_second_half_of_ids": half,
                      "stream_us_by_range_mod8": by_range_mod8,
                      "workgroups_and_stream_us_by_units": by_units,
                      "stream_us_mean_per_wg_p10_p50_p90": [
                          round(float(np.percentile(mean_dur, q)), 2) for q in (10, 50, 90)]}),
          flush=True)
    return 0


def run_rope(args, torch, pkv, W) -> int:
    """Decode step over un-rotated or float32 pools (decode_rope_mfma.hip, the float32
    matrix-core tile on the balanced schedule), append + decode: with RoPE
    applied at read (--workload rope: pkv_kv_append storing un-rotated keys, the decode rotating
    query and keys), or over float32 pools (--workload f32: the same lengths and shapes with
    float32 K/V, rotation by the append). HBM-bound like the plain decode."""
    rope = args.workload == "rope"
    wl = W.config(args.config)
    hkv = args.kv_heads or wl["Hkv"]
    if wl["Hq"] % hkv:
        print(f"--kv-heads {hkv} does not divide {wl['Hq']} query heads", file=sys.stderr)
        return 2
    if not rope or hkv != wl["Hkv"]:
        wl = W.make_workload(wl["wid"], wl["positions"], wl["Hq"], hkv, wl["D"], wl["bs"],
                             wl["dtype"] if rope else "f32", wl["theta"],
                             name=wl["name"] + ("" if rope else "-f32") +
                             ("" if hkv == W.config(args.config)["Hkv"] else f"-kv{hkv}"))
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
    pool_view = np.int16 if rope else np.int32
    k0, v0 = t(wl["k_pool"], pool_view), t(wl["v_pool"], pool_view)
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(copies - 1)]
    B, Hq, Hkv, D, bs = wl["B"], wl["Hq"], wl["Hkv"], wl["D"], wl["bs"]
    split = args.split_tokens or pkv.decode_schedule_split(
        B, Hq, Hkv, D, bs, wl["max_context_len"], pkv.pool_dtype_code(None, wl["dtype"]),
        rope_on_read=rope)
    ws = torch.zeros(max(pkv.decode_workspace_bytes(B, Hq, Hkv, D, bs, wl["max_context_len"],
                                                    split), 1), dtype=torch.uint8, device=dev)
    q_out = torch.empty_like(q)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def append(i):
        kp, vp = pools[i % copies]
        pkv.kv_append(q, k_new, v_new, kp, vp, tables, positions, theta=wl["theta"],
                      q_norm_w=qn, k_norm_w=kn, eps=wl["eps"], q_out=q_out, dtype=wl["dtype"],
                      rope_on_read=rope, stream=stream)

    def attend(i):
        kp, vp = pools[i % copies]
        pkv.paged_attn_decode(q_out, kp, vp, tables, ctx, wl["max_context_len"], wl["scale"],
                              out=out, workspace=ws, split_tokens=split, dtype=wl["dtype"],
                              rope_on_read=rope, read_theta=wl["theta"], stream=stream)

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    t0 = time.perf_counter()
    step_ms = timed(lambda i: (append(i), attend(i)))
    wall_ms = (time.perf_counter() - t0) * 1e3
    attn_ms = timed(attend)
    append_ms = timed(append)
    step_gbs = nbytes["step"] / (step_ms * 1e-3) / 1e9
    attn_gbs = nbytes["decode"] / (attn_ms * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.load()
        kp, vp = wl["k_pool"].copy(), wl["v_pool"].copy()
        q_ref = oracle.kv_append(wl["q"], wl["k_new"], wl["v_new"], kp, vp, wl["tables"],
                                 wl["positions"], wl["q_norm_w"], wl["k_norm_w"], wl["eps"],
                                 wl["theta"], wl["dtype"], rope_on_read=rope)
        mask = np.zeros(B, dtype=np.uint8)
        mask[::4] = 1
        c0 = time.perf_counter()
        if rope:
            oracle.paged_attn_decode_rope(q_ref, kp, vp, wl["tables"], wl["context_lens"],
                                          wl["theta"], wl["scale"], wl["dtype"], row_mask=mask)
        else:
            oracle.paged_attn_decode(q_ref, kp, vp, wl["tables"], wl["context_lens"],
                                     wl["scale"], wl["dtype"], row_mask=mask)
        cpu_s = time.perf_counter() - c0
        L = wl["context_lens"].astype(np.int64)
        E = 4 if wl["dtype"] == "f32" else 2
        kv_sample = int(L[mask.astype(bool)].sum()) * 2 * Hkv * D * E
        cpu = {"value": round(kv_sample / cpu_s / 1e9, 4), "unit": "GB/s", "cores": 1, **host_cpu(),
               "kind": "oracle",
               "sample": f"attention of {int(mask.sum())} of the {B} sequences (every 4th), "
                         f"{cpu_s:.2f} s single-threaded"}

    line = {
        "metric": ("paged-attn decode with RoPE applied at read, achieved HBM GB/s" if rope
                   else "paged-attn decode over float32 KV pools, achieved HBM GB/s"),
        "value": round(step_gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl["dtype"], "data": "synthetic",
        "tokens_per_s": round(B / (step_ms * 1e-3), 1),
        "config": {"workload": wl["name"] + ("-rope-at-read" if rope else ""), "batch": B,
                   "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": D, "block_size": bs,
                   "kv_dtype": wl["dtype"], "context_tokens": int(wl["context_lens"].sum()),
                   "max_context_len": wl["max_context_len"], "rope_theta": wl["theta"],
                   "pool_copies": copies, "split_tokens": split,
                   "bytes_per_step": nbytes["step"]},
        "roofline": {"bound": "hbm", "kernel": ("decode_rope_balanced_kernel" if split == 0 else
                                                "decode_rope_kernel")
                     + " (pkv_paged_attn_decode)",
                     "achieved": round(attn_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": nbytes["decode"],
                     "avg_launch_us": round(attn_ms * 1e3, 3)},
        "append": {"kernel": "pkv_kv_append" + (" (no rotation)" if rope else " (float32 rows)"),
                   "avg_launch_us": round(append_ms * 1e3, 3)},
        "cpu_baseline": cpu,
        "wall_ms_timed_steps": round(wall_ms, 2),
    }
    print(json.dumps(line), flush=True)
    return 0


def run_blocks(args) -> int:
    """Host block manager (include/pkv_blocks.h) on the prefix-shared decode workload's shape:
    128 sequences whose prompts share 2048 tokens plus a private tail of U{0..1024}, block size
    16. Timed: admission of the batch (the first prompt cold and committed, the others borrowing
    its 128 prefix blocks), then decode steps (room for one token, the table rows and positions
    filled for the batch, one token committed and recorded per sequence: pkv_batch_prepare and
    pkv_batch_commit). Host code only; the baseline is the Python oracle model doing the same
    per sequence."""
    from paged_kv_cache_315_amd import blocks as BM
    rng = np.random.default_rng([5, 99])
    B, bs, prefix_len = 128, 16, 2048
    prefix = rng.integers(0, 32000, prefix_len).tolist()
    tails = rng.integers(0, 1025, B)
    prompts = [prefix + rng.integers(0, 32000, int(t)).tolist() for t in tails]
    max_blocks = (prefix_len + 1024 + args.steps + bs - 1) // bs + 1
    nb = 128 + B * (1024 // bs + 2) + B * (args.steps // bs + 2)
    steps = max(args.steps, 1)

    def run(make_pool, make_seq, fill):
        pool = make_pool(nb, bs)
        seqs = [make_seq(pool) for _ in range(B)]
        t0 = time.perf_counter()
        seqs[0].allocate_for_tokens(prompts[0])
        seqs[0].commit(len(prompts[0]))
        for s, p in zip(seqs[1:], prompts[1:]):
            s.allocate_for_tokens(p)
        t_admit = time.perf_counter() - t0
        t0 = time.perf_counter()
        for i in range(steps):
            for s in seqs:
                s.reserve(1)
            fill(seqs)
            for s in seqs:
                s.commit(1)
                s.append_token(i)
        return t_admit, (time.perf_counter() - t0) / steps

    # native: one C call per step for room + tables and one for the commit (Batch)
    pool = BM.BlockPool(nb, bs)
    seqs = [BM.SeqCache(pool, 0) for _ in range(B)]
    t0 = time.perf_counter()
    seqs[0].allocate_for_tokens(prompts[0])
    seqs[0].commit(len(prompts[0]))
    for s, p in zip(seqs[1:], prompts[1:]):
        s.allocate_for_tokens(p)
    t_admit = time.perf_counter() - t0
    batch = BM.Batch(seqs, max_blocks, 0)
    ids = np.zeros(B, np.int32)
    t0 = time.perf_counter()
    for i in range(steps):
        batch.prepare(1)
        ids[:] = i
        batch.commit(1, ids)
    native = (t_admit, (time.perf_counter() - t0) / steps)
    for s in seqs:
        s.destroy()
    pool.close()
    cpu = None
    if not args.no_cpu_baseline:
        import oracle.block_manager as OB
        ref = run(lambda n, b: OB.Pool(n, b), lambda p: OB.Seq(p, 0),
                  lambda ss: OB.fill_tables(ss, max_blocks, 0))
        cpu = {"value": round(ref[1] * 1e6, 1), "unit": "us per decode step", "cores": 1, **host_cpu(),
               "kind": "oracle",
               "sample": f"the same {steps} steps on the Python oracle model "
                         f"(admission {ref[0] * 1e3:.1f} ms)"}
    line = {
        "metric": "host block manager: us per decode step (128 sequences, tables + growth)",
        "value": round(native[1] * 1e6, 2), "unit": "us", "n_gpus": 0, "steps": steps,
        "warmup": 0, "ms_per_step": round(native[1] * 1e3, 5), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": "prefix-shared-blocks", "batch": B, "block_size": bs,
                   "shared_prefix_tokens": prefix_len, "tail_tokens": "U{0..1024}",
                   "pool_blocks": nb, "max_blocks_per_seq": max_blocks},
        "admission_ms": round(native[0] * 1e3, 3),
        "roofline": None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


MFMA_BF16_PEAK_TFLOPS = 2500.0


def run_prefill(args, torch, pkv, W) -> int:
    """Chunked-prefill step (pkv_prefill_append + pkv_paged_attn_prefill) on one of the prefill
    workloads; roofline of the attention kernel: matrix cores for long chunks (prefill), HBM
    for a few tokens per sequence (spec)."""
    wl = W.prefill_config(2 if args.workload == "prefill" else 3)
    dev = torch.device("cuda:0")

    def t(a, dt=None):
        return torch.from_numpy(np.ascontiguousarray(a if dt is None else a.view(dt))).to(dev)

    q, k_new, v_new = t(wl["q"]), t(wl["k_new"]), t(wl["v_new"])
    tables, cu, start = t(wl["tables"]), t(wl["cu_seqlens"]), t(wl["start_pos"])
    pool_bytes = 2 * wl["k_pool"].nbytes
    copies = args.copies or max(2, int(np.ceil(1.0e9 / pool_bytes)))
    k0, v0 = t(wl["k_pool"], np.int16), t(wl["v_pool"], np.int16)
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(copies - 1)]
    B, N, Hq, Hkv, D, bs = wl["B"], wl["N"], wl["Hq"], wl["Hkv"], wl["D"], wl["bs"]
    need = pkv.prefill_workspace_bytes(B, Hq, Hkv, D, bs, wl["max_chunk"], wl["max_context_len"])
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    q_out = torch.empty_like(q)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def append(i):
        kp, vp = pools[i % copies]
        pkv.prefill_append(q, k_new, v_new, kp, vp, tables, cu, start, theta=wl["theta"],
                           q_out=q_out, dtype=wl["dtype"], stream=stream)

    def attend(i):
        kp, vp = pools[i % copies]
        pkv.paged_attn_prefill(q_out, kp, vp, tables, cu, start, wl["max_chunk"],
                               wl["max_context_len"], wl["scale"], out=out, workspace=ws,
                               dtype=wl["dtype"], stream=stream)

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    t0 = time.perf_counter()
    step_ms = timed(lambda i: (append(i), attend(i)))
    wall_ms = (time.perf_counter() - t0) * 1e3
    attn_ms = timed(attend)
    append_ms = timed(append)

    tok_len = wl["tok_len"].astype(np.int64)
    flops = 4 * D * Hq * int(tok_len.sum())            # QK^T and PV, 2 flops per MAC
    uniq = W.prefill_unique_kv_bytes(wl)
    io = N * Hq * D * 4 * 2 + int(((wl["start_pos"] + wl["chunk"] + bs - 1) // bs).sum()) * 4
    attn_bytes = uniq + io
    if args.workload == "prefill":
        achieved = flops / (attn_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "prefill_attn_shared_kernel (pkv_paged_attn_prefill)",
                "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": None, "flops_per_launch": flops,
                "avg_launch_us": round(attn_ms * 1e3, 3)}
        metric = "chunked-prefill causal paged attention TFLOP/s (4 x 512-token chunks)"
        value, unit = achieved, "TFLOP/s"
    else:
        achieved = attn_bytes / (attn_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "prefill_balanced_kernel (pkv_paged_attn_prefill)",
                "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "bytes_per_launch": attn_bytes, "avg_launch_us": round(attn_ms * 1e3, 3)}
        metric = "draft-verification paged attention GB/s (32 sequences x 4 tokens)"
        value, unit = achieved, "GB/s"

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.load()
        kp = wl["k_pool"].copy()
        vp = wl["v_pool"].copy()
        q_ref = oracle.prefill_append(wl["q"], wl["k_new"], wl["v_new"], kp, vp, wl["tables"],
                                      wl["cu_seqlens"], wl["start_pos"], None, None, wl["eps"],
                                      wl["theta"], wl["dtype"])
        stride = 16 if args.workload == "prefill" else 1
        mask = np.zeros(N, dtype=np.uint8)
        mask[::stride] = 1
        c0 = time.perf_counter()
        oracle.paged_attn_prefill(q_ref, kp, vp, wl["tables"], wl["cu_seqlens"],
                                  wl["start_pos"], wl["scale"], wl["dtype"], row_mask=mask)
        cpu_s = time.perf_counter() - c0
        sel = mask.astype(bool)
        if args.workload == "prefill":
            cpu_val = 4 * D * Hq * int(tok_len[sel].sum()) / cpu_s / 1e12
        else:
            cpu_val = attn_bytes / cpu_s / 1e9
        cpu = {"value": round(cpu_val, 6), "unit": unit, "cores": 1, **host_cpu(), "kind": "oracle",
               "sample": f"causal attention of {int(sel.sum())} of the {N} query tokens "
                         f"(every {stride}th), {cpu_s:.2f} s single-threaded"}

    line = {
        "metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl["dtype"], "data": "synthetic",
        "config": {"workload": wl["name"], "batch": B, "query_tokens": N, "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": D, "block_size": bs,
                   "kv_dtype": wl["dtype"], "max_chunk": wl["max_chunk"],
                   "max_context_len": wl["max_context_len"], "pool_copies": copies,
                   "attended_keys": int(tok_len.sum()), "unique_kv_bytes": uniq},
        "roofline": roof,
        "append": {"kernel": "pkv_prefill_append", "avg_launch_us": round(append_ms * 1e3, 3)},
        "cpu_baseline": cpu,
        "wall_ms_timed_steps": round(wall_ms, 2),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
