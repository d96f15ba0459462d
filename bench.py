"""Benchmark: fixed-m attention forward on one MI355X.

One step = the whole hot path for one ring rank: fixedm_bounds, run init, then one
fixedm_attn_fwd_final over the visiting K/V chunks in ring order 0, 3, 2, 1 (the chunks
folded with the accumulators resident in registers, and the output written as bf16 by the
same launch).  With --per-chunk a step is instead one call per chunk, as a ring rank
receiving one chunk at a time would run it: fixedm_attn_fwd for each chunk but the last,
and fixedm_attn_fwd_final for the last one (which writes the output).
Inputs are seeded synthetic tensors at the Wan2.2 720p rank-share shape (40 heads,
head_dim 128, 18,900 resident queries, 75,600 keys in 4 chunks), resident in HBM before
the timed region starts.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--config 3] [--per-chunk] [--no-cpu-baseline]
                    [--fallback none|all|FRACTION]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 4096 dense bf16 flop/clk x 2.4 GHz
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


KERNEL_SOURCES = ("attn_bf16.hip", "fixed_loop.inc")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "dit_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, fused: bool, fallback: str, q_block_default: bool):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary, or None
    when this run is not the launch the counters were taken on (another workload, the
    per-chunk calls, a fallback mode, another q_block) or the kernel source has changed
    since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    if not (fused and fallback == "none" and q_block_default
            and str(t.get("workload", "")).split(" ")[0] == workload):
        return None
    return t.get("hbm_bytes_per_launch")


def to_dev(arr, dtype, torch, np):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def cpu_baseline(inp, seconds: float):
    """The oracle as it stands, timed on the host on a bounded sample of the same workload:
    whole 256-row q-blocks of successive heads against all N keys, until `seconds` pass or
    every block has been timed (then the sample is the whole workload)."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    wl = inp.wl
    K = [c for c in inp.k_store]
    V = [c for c in inp.v_store]
    f32 = inp._f32
    flops = 0.0
    rows_done = 0
    heads_used = set()
    t0 = time.perf_counter()
    elapsed = 0.0
    h = 0
    beta = 0
    n_blocks = -(-wl.sq // 256)
    while elapsed < seconds and beta < n_blocks:
        kh = np.concatenate([f32(c[:, :, h:h + 1]) for c in K], axis=1)
        vh = np.concatenate([f32(c[:, :, h:h + 1]) for c in V], axis=1)
        qh = f32(inp.q_store[:, :, h:h + 1])
        lo = beta * 256
        hi = min(lo + 256, wl.sq)
        ts = time.perf_counter()
        O.attention(qh[:, lo:hi], kh, vh, wl.scale)
        elapsed += time.perf_counter() - ts
        flops += 4.0 * (hi - lo) * wl.sk * wl.head_dim
        rows_done += hi - lo
        heads_used.add(h)
        h = (h + 1) % wl.heads
        if h == 0:
            beta += 1
    wall = time.perf_counter() - t0
    return {
        "value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{rows_done} query rows (whole 256-row q-blocks over {len(heads_used)} heads) x "
                   f"all {wl.sk} keys, fp64 numpy oracle, {elapsed:.1f} s timed "
                   f"({wall:.1f} s with input upcasts)"),
        "host_cpus_visible": len(os.sched_getaffinity(0)),
    }


def apply_fallback(inp, mode: str, q_block: int, np, WL):
    """Edits the drawn inputs so that some q-blocks fail the gate and take the online-softmax
    body (for timing that body).  Returns the number of (b, h, q-block) pairs scaled, or None."""
    if mode == "none":
        return None
    wl = inp.wl

    def put(store, x):
        return WL.bf16_bits_from_f32(x) if wl.dtype == "bf16" else x.astype(np.float32)

    if mode == "all":
        v0 = inp._f32(inp.v_store[0]).copy()
        v0[0, 0, 0, 0] = 300.0
        inp.v_store[0] = put(inp.v_store[0], v0)
        return None
    frac = float(mode)
    if not 0.0 < frac <= 1.0:
        raise SystemExit(f"bench.py: --fallback {mode}: expected none, all or a fraction in (0, 1]")
    every = max(1, int(round(1.0 / frac)))
    nqb = -(-wl.sq // q_block)
    qf = inp._f32(inp.q_store).copy()
    n = 0
    for b in range(wl.batch):
        for h in range(wl.heads):
            for beta in range(nqb):
                if ((b * wl.heads + h) * nqb + beta) % every == 0:
                    lo, hi = beta * q_block, min((beta + 1) * q_block, wl.sq)
                    qf[b, lo:hi, h] *= np.float32(8.0)
                    n += 1
    inp.q_store = put(inp.q_store, qf)
    return n


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--per-chunk", action="store_true",
                    help="one call per ring chunk (fixedm_attn_fwd, then fixedm_attn_fwd_final for "
                         "the last) instead of one fixedm_attn_fwd_final over all chunks")
    ap.add_argument("--fallback", default="none",
                    help="which q-blocks take the online-softmax body: 'none' (the workload as "
                         "drawn), 'all' (one V element set to 300 fails the |v| <= 256 check, so "
                         "every block falls back), or a fraction such as 0.01 (that share of the "
                         "(head, q-block) pairs, every 1/fraction-th, gets its queries scaled by 8, "
                         "which lifts its bound above the gate)")
    ap.add_argument("--q-block", type=int, default=None,
                    help="rows per shift/eligibility block (default: the workload's, 256); 64 puts "
                         "four blocks in one workgroup, so a loud block shares it with fixed-m waves")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB fp32 read+write kernel (3 times): the reference "
                         "dispatch for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the fixed-m benchmark runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the multi-GPU ring is described, not implemented.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": 1 << 30, "calibrate_copy_bytes_written": 1 << 30}),
              flush=True)
        return

    from dit_amd import fixedm as F
    from dit_amd import workloads as WL

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    F.lib()
    wl = WL.get(args.config)
    log(f"bench: drawing inputs for config {wl.cid} ({wl.name})")
    inp = WL.make_inputs(wl.cid)
    q_block = args.q_block or wl.q_block
    loud_blocks = apply_fallback(inp, args.fallback, q_block, np, WL)
    q = to_dev(inp.q_store, wl.dtype, torch, np)
    ks = [to_dev(c, wl.dtype, torch, np) for c in inp.k_store]
    vs = [to_dev(c, wl.dtype, torch, np) for c in inp.v_store]
    km = torch.from_numpy(inp.k_mean).cuda() if inp.k_mean is not None else None
    order = [0] + list(range(len(ks) - 1, 0, -1))        # rank 0's ring visit order
    ks, vs = [ks[i] for i in order], [vs[i] for i in order]

    p = F.make_problem(wl.dtype, wl.batch, wl.heads, wl.head_dim, wl.sq, wl.sk, q_block,
                       0.0, wl.center)
    buf = torch.empty(F.bounds_bytes(p), dtype=torch.uint8, device="cuda")
    ws = F.alloc_workspace(p, q.device)
    out_dtype = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    out = torch.empty((wl.batch, wl.sq, wl.heads, wl.head_dim), dtype=out_dtype, device="cuda")
    stream = torch.cuda.current_stream()
    fused = not args.per_chunk
    n_attn = 1 if fused else len(ks)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps * n_attn)]
    ev_b = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(args.steps)]

    def step(timed_idx=None):
        if timed_idx is not None:
            ev_b[timed_idx][0].record(stream)
        desc, _ = F.bounds(p, q, ks, vs, k_mean=km, buf=buf, stream=stream)
        if timed_idx is not None:
            ev_b[timed_idx][1].record(stream)
        run = F.run_init(desc)
        if fused:
            if timed_idx is not None:
                ev[timed_idx][0].record(stream)
            F.attn_fwd_final(desc, run, q, ks, vs, ws, out, None, stream=stream)
            if timed_idx is not None:
                ev[timed_idx][1].record(stream)
            return desc
        for c in range(n_attn):
            if timed_idx is not None:
                ev[timed_idx * n_attn + c][0].record(stream)
            if c + 1 < n_attn:
                F.attn_fwd(desc, run, q, [ks[c]], [vs[c]], ws, stream=stream)
            else:
                F.attn_fwd_final(desc, run, q, [ks[c]], [vs[c]], ws, out, None, stream=stream)
            if timed_idx is not None:
                ev[timed_idx * n_attn + c][1].record(stream)
        return desc

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        desc = step()
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps")
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        desc = step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in ev]
    attn_avg = sum(attn_ms) / len(attn_ms)
    bounds_avg = sum(a.elapsed_time(b) for a, b in ev_b) / len(ev_b)
    # the bounds pass reads Q once, K twice when the key mean is computed (the mean, then the
    # centred norms), else once, and V once
    esz = 2 if wl.dtype == "bf16" else 4
    kv_bytes = wl.batch * wl.sk * wl.heads * wl.head_dim * esz
    q_bytes = wl.batch * wl.sq * wl.heads * wl.head_dim * esz
    bounds_bytes = q_bytes + kv_bytes * (3 if wl.center == "compute" else 2)

    flops = wl.flops
    value = flops / (ms_per_step * 1e-3) / 1e12
    per_launch_flops = flops / n_attn
    achieved = per_launch_flops / (attn_avg * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS

    gb = F.read_bounds(desc, buf)
    elig_frac = float(gb["elig"].float().mean().item())
    log(f"bench: {ms_per_step:.3f} ms/step, attention launch avg {attn_avg:.3f} ms, "
        f"eligible fraction {elig_frac:.4f}")

    result = {
        "metric": "fixed-m attn fwd TFLOP/s (4*B*H*Sq*Sk*D / t) + % bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "frac_of_peak": round(value / peak, 4),
        "config": {
            "workload": wl.name, "batch": wl.batch, "heads": wl.heads, "head_dim": wl.head_dim,
            "sq": wl.sq, "sk": wl.sk, "chunks": list(wl.chunks), "ring_order": order,
            "q_block": q_block, "centering": wl.center, "eligible_fraction": elig_frac,
            "fallback": args.fallback, "loud_qblocks": loud_blocks,
            "step": (f"bounds + attn_fwd_final over the {len(ks)} ring chunks (output written by "
                     "the attention launch)" if fused else
                     f"bounds + {len(ks) - 1} x attn_fwd + attn_fwd_final (one call per ring chunk)"),
        },
        "roofline": {
            "kernel": "attn_bf16_d128_kernel" if wl.dtype == "bf16" else "attn_f32_kernel",
            "bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": measured_traffic(wl.name, fused, args.fallback, q_block == wl.q_block),
            "launch_ms": round(attn_avg, 4), "launches_per_step": n_attn,
            "flops_per_launch": per_launch_flops,
            "timed_call": ("fixedm_attn_fwd_final: the attention launch plus the finalize of "
                           "the split tail tiles" if fused else "fixedm_attn_fwd (one launch)"),
        },
    }
    result["bounds"] = {
        "ms": round(bounds_avg, 4), "algorithmic_bytes": bounds_bytes,
        "GB/s": round(bounds_bytes / (bounds_avg * 1e-3) / 1e9, 1), "bound": "hbm",
        "frac_of_hbm_peak": round(bounds_bytes / (bounds_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "terms": "Q + K (key mean) + K (centred norms) + V (magnitude check), one read each",
    }
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on the host (bounded sample)")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
