"""Throughput of the TTT-layer forward pass (libttt_la) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-others] [--no-cpu] [--flush-mb 512]

A step is one ttt_la_forward call over one batch of synthetic inputs that
are already resident in HBM.  Before every step a 512 MB buffer is
overwritten so the 256 MB last-level cache and the L2s hold none of the
inputs; each step is timed with HIP events on the stream the kernels run
on, and the K steps are bracketed by device synchronisation.  Prints ONE
JSON line (the headline workload, plus sub-records for the other
workloads of the method under "workloads").
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

import workloads  # noqa: E402

METRIC = "tokens/s and % of bf16 MFMA peak for TTT-linear-attn fwd, 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector


def algorithmic(s: dict) -> tuple[int, float]:
    """Bytes the method must move and flops it must do for one forward pass.

    Bytes: read Q, K, V, eta once, write O once, read W0 and write W_out.
    Flops per token-head: per-token mode 4 d_k d_v (rank-1 update + read)
    plus (C+1)(d_k+d_v) for the causal half of the intra-chunk products;
    large-chunk linear 4 d^2 plus 3 d^2 per chunk for the normalisation;
    SwiGLU 18 d d_h (Q read 6, K forward 4, four gradient products 8)."""
    B, H, T, dk, dv, dh, C = s["B"], s["H"], s["T"], s["d_k"], s["d_v"], s["d_h"], s["chunk"]
    es = 2 if s["dtype"] == "bf16" else 4
    n = B * H * T
    state = B * H * (3 * dk * dh if s["mode"] == "large_chunk_swiglu" else dk * dv) * 4
    nbytes = n * (2 * dk + 2 * dv) * es + n * 4 + 2 * state
    if s["mode"] == "per_token_linear":
        flops = n * (4 * dk * dv + (C + 1) * (dk + dv))
    elif s["mode"] == "large_chunk_linear":
        flops = n * 4 * dk * dv + B * H * (-(-T // C)) * 3 * dk * dv
    else:
        flops = n * 18 * dk * dh
    return nbytes, float(flops)


def run_workload(name: str, steps: int, warmup: int, flush_mb: int):
    import torch
    import linear_attention_ttt_amd as la

    s = workloads.spec(name)
    x = workloads.generate(s, seed=0)
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if s["dtype"] == "bf16" else torch.float32
    t = {k: torch.from_numpy(x[k]).to(dev) for k in ("Q", "K", "V", "eta", "W0")}
    for k in ("Q", "K", "V"):
        t[k] = t[k].to(dt)
    del x
    B, H, T, dv = s["B"], s["H"], s["T"], s["d_v"]
    O = torch.empty((B, H, T, dv), dtype=dt, device=dev)
    Wout = torch.empty_like(t["W0"])
    desc = la.make_desc(B, H, T, s["d_k"], dv, s["d_h"], la.BF16 if dt == torch.bfloat16 else la.FP32)
    nws = la.workspace_bytes(desc, s["chunk"], s["mode"])
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    flush = torch.empty(flush_mb << 20, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        la.forward(t["Q"], t["K"], t["V"], t["eta"], t["W0"], s["chunk"], s["mode"], out=O, W_out=Wout,
                   workspace=ws)

    for _ in range(warmup):
        flush.fill_(1)
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(steps):
        flush.fill_(i & 0xFF)
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    nbytes, flops = algorithmic(s)
    mean_s = float(ms.mean()) * 1e-3
    rec = dict(workload=name, mode=s["mode"], B=B, H=H, T=T, d=s["d_k"], d_h=s["d_h"], chunk=s["chunk"],
               dtype=s["dtype"], ms_per_step=float(ms.mean()), ms_min=float(ms.min()), ms_median=float(np.median(ms)),
               tokens_per_s=B * T / mean_s, token_heads_per_s=B * H * T / mean_s,
               algorithmic_bytes=nbytes, algorithmic_flops=flops,
               hbm_GBps=nbytes / mean_s / 1e9, hbm_frac=nbytes / mean_s / 1e9 / HBM_PEAK_GBS,
               bf16_mfma_TFLOPs=flops / mean_s / 1e12, bf16_mfma_frac=flops / mean_s / 1e12 / BF16_PEAK_TFLOPS,
               wall_s_including_flush=wall)
    del t, O, Wout, ws, flush
    torch.cuda.empty_cache()
    return rec


def cpu_baseline(name: str, target_s: float = 12.0):
    """Time the fp64 oracle on a bounded sample of the workload: whole
    sequences of a subset of the (independent) heads, scaled to the full
    workload's tokens/s."""
    import oracle

    s = workloads.spec(name)
    x = workloads.generate(s, seed=0)
    BH = s["B"] * s["H"]

    def heads(idx):
        return {k: x[k].reshape((BH,) + x[k].shape[2:])[idx][None] for k in ("Q", "K", "V", "eta", "W0")}

    # calibrate on one head, then size the sample to about target_s seconds
    h1 = heads([0])
    c0, w0 = time.process_time(), time.perf_counter()
    oracle.forward(h1["Q"], h1["K"], h1["V"], h1["eta"], h1["W0"], s["chunk"], s["mode"], d_h=s["d_h"])
    one = time.perf_counter() - w0
    nh = int(max(1, min(BH, target_s / max(one, 1e-3))))
    hs = heads(list(range(nh)))
    c0, w0 = time.process_time(), time.perf_counter()
    oracle.forward(hs["Q"], hs["K"], hs["V"], hs["eta"], hs["W0"], s["chunk"], s["mode"], d_h=s["d_h"])
    wall = time.perf_counter() - w0
    cpu = time.process_time() - c0
    full_s = wall * BH / nh
    return {"value": s["B"] * s["T"] / full_s, "unit": "tokens/s",
            "cores": max(1, round(cpu / wall)),
            "kind": "oracle",
            "sample": f"{nh} of {BH} heads of {name}, full T={s['T']}; {wall:.1f} s wall, {cpu:.1f} s CPU; "
                      f"scaled by {BH}/{nh} (heads are independent)",
            "host_cpus_available": len(os.sched_getaffinity(0))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=workloads.HEADLINE)
    ap.add_argument("--no-others", action="store_true", help="skip the other workloads' sub-records")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--flush-mb", type=int, default=512)
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every (b,h) recurrence is independent; sharding B*H across GPUs needs no communication)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    head = run_workload(a.workload, a.steps, a.warmup, a.flush_mb)
    others = {}
    if not a.no_others:
        for name in workloads.WORKLOADS:
            if name == a.workload:
                continue
            try:
                others[name] = run_workload(name, max(3, a.steps // 4), 2, a.flush_mb)
            except Exception as e:  # a mode not built yet is reported, not fatal
                others[name] = {"error": str(e)[:200]}
    s = workloads.spec(a.workload)
    nbytes, flops = head["algorithmic_bytes"], head["algorithmic_flops"]
    kernel_s = head["ms_per_step"] * 1e-3
    roof = {"kernel": "per_token_bf16_kernel" if s["mode"] == "per_token_linear" else s["mode"],
            "bound": "hbm", "achieved": nbytes / kernel_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": nbytes / kernel_s / 1e9 / HBM_PEAK_GBS, "traffic": None,
            "algorithmic_bytes_per_launch": nbytes}
    if s["mode"] == "large_chunk_swiglu":
        roof.update(bound="mfma", achieved=flops / kernel_s / 1e12, peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=flops / kernel_s / 1e12 / BF16_PEAK_TFLOPS)
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s["dtype"],
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": a.workload, "mode": s["mode"], "B": s["B"], "H": s["H"], "T": s["T"],
                   "d_k": s["d_k"], "d_v": s["d_v"], "d_h": s["d_h"], "chunk": s["chunk"]},
        "bf16_mfma_frac": head["bf16_mfma_frac"],
        "token_heads_per_s": head["token_heads_per_s"],
        "roofline": roof,
        "cpu_baseline": None if a.no_cpu else cpu_baseline(a.workload),
        "workloads": others,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
