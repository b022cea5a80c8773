"""Throughput of the TTT-layer forward pass (libttt_la) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-others] [--no-cpu] [--no-backward] [--flush-mb 512]
                    [--calibrate-copy-mb N] [--mode M] [--other-order] [--momentum B]

A step is one ttt_la_forward call over one batch of synthetic inputs that
are already resident in HBM.  Each workload is timed three ways:

* flushed (the headline ``value`` and ``ms_per_step``): before every step a
  512 MB buffer is overwritten and another 512 MB buffer read, so the 256 MB
  last-level cache and the L2s hold none of the inputs and no dirty lines;
  each step is bracketed by HIP events on the stream the kernels run on and
  the K steps by device synchronisation;
* steady state: K calls back to back, rotating over copies of the inputs
  and outputs whose total exceeds the caches, timed as a whole, so the
  write-back of one call's outputs falls inside the timed window of the
  next (no eviction between calls);
* dominant kernel: the library records fence-free events around it
  (ttt_la_forward_timed), for the roofline.

Prints ONE JSON line: the headline workload (the largest per-token one),
with sub-records for the other workloads under "workloads" (each with its
own roofline, counter traffic and CPU baseline) and backward records under
"backward".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "tokens/s and % of bf16 MFMA peak for TTT-linear-attn fwd, 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
CEILINGS = {}                  # practical ceilings measured on this GPU at the start of the run (practical_ceilings)
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector

# each method's other read order (exclusive per-token read, update-then-read chunks): same kernels and work
OTHER_ORDER = {"per_token_linear": "per_token_linear_exclusive",
               "large_chunk_linear": "large_chunk_linear_update_first",
               "large_chunk_swiglu": "large_chunk_swiglu_update_first"}

# kernel source each workload's dominant kernel is built from (counter summaries are keyed to its hash)
KERNEL_SOURCE = {"per_token_linear": "per_token.hip", "large_chunk_linear": "large_chunk_linear.hip",
                 "large_chunk_swiglu": "large_chunk_swiglu.hip", "large_chunk_swiglu_last_layer": "large_chunk_swiglu.hip"}


def method_of(mode: str) -> str:
    for base, other in OTHER_ORDER.items():
        if mode == other:
            return base
    return mode


def o_size(s: dict) -> int:
    return 4 if s.get("o_dtype", s["dtype"]) == "fp32" else (2 if s["dtype"] == "bf16" else 4)


def algorithmic(s: dict) -> tuple[int, float]:
    """Bytes the method must move and flops it must do for one forward pass.

    Bytes: read Q, K, V, eta once, write O once (in its element type), read
    W0 and write W_out.  Flops per token-head: per-token mode 4 d_k d_v
    (rank-1 update + read) plus (C+1)(d_k+d_v) for the causal half of the
    intra-chunk products; large-chunk linear 4 d^2 plus 3 d^2 per chunk for
    the normalisation; SwiGLU 18 d d_h (Q read 6, K forward 4, four
    gradient products 8)."""
    B, H, T, dk, dv, dh, C = s["B"], s["H"], s["T"], s["d_k"], s["d_v"], s["d_h"], s["chunk"]
    es = 2 if s["dtype"] == "bf16" else 4
    n = B * H * T
    m = method_of(s["mode"])
    state = B * H * (3 * dk * dh if m.startswith("large_chunk_swiglu") else dk * dv) * 4
    nbytes = n * (2 * dk + dv) * es + n * dv * o_size(s) + n * 4 + 2 * state
    if m == "per_token_linear":
        flops = n * (4 * dk * dv + (C + 1) * (dk + dv))
    elif m == "large_chunk_linear":
        flops = n * 4 * dk * dv + B * H * (-(-T // C)) * 3 * dk * dv
    elif m == "large_chunk_swiglu_last_layer":
        flops = n * 12 * dk * dh       # Q read 6, K features 4, W2 gradient 2
    else:
        flops = n * 18 * dk * dh
    return nbytes, float(flops)


def dominant_kernel(s: dict) -> tuple[str, float, str]:
    """The kernel ttt_la_forward_timed brackets for this mode, the algorithmic
    units it processes per launch (bytes for an HBM-bound kernel, flops for
    an MFMA-bound one) and its bound.

    per-token: the chunked-form pass over the sequence moves all of the
      method's bytes (reads Q, K, V, eta, W0; writes O, W_out).
    large-chunk linear: the chunk update reads K, V and eta.
    SwiGLU: the recurrence does the K forward (4 d d_h) and the four
      gradient products (8 d d_h) of every token-head."""
    B, H, T, dk, dv, dh = s["B"], s["H"], s["T"], s["d_k"], s["d_v"], s["d_h"]
    es = 2 if s["dtype"] == "bf16" else 4
    n = B * H * T
    m = method_of(s["mode"])
    if m == "per_token_linear":
        return ("pt_seg_kernel (output pass)" if s["dtype"] == "bf16" else "per_token_fp32_kernel",
                float(algorithmic(s)[0]), "hbm")
    if m == "large_chunk_linear":
        return "lact_delta_kernel (chunk update)", float(n * ((dk + dv) * es + 4)), "hbm"
    if m == "large_chunk_swiglu_last_layer":
        return "swiglu_recur_kernel (recurrence)", float(n * 6 * dk * dh), "mfma"
    return "swiglu_recur_kernel (recurrence)", float(n * 12 * dk * dh), "mfma"


def traffic_per_launch(name: str, s: dict):
    """HBM bytes per launch of the workload's dominant kernel from the
    committed counter summary ``profiles/traffic_<workload>.md``
    (FETCH_SIZE + WRITE_SIZE, calibrated against a copy of known size), or
    None when there is none, it was taken in another mode or output dtype,
    or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9]+)", text)
    m_mode = re.search(r"mode:\s*(\S+)", text)
    m_odt = re.search(r"o_dtype:\s*(\S+)", text)
    if not (m_sha and m_bytes and m_mode and m_odt):
        return None
    if m_mode.group(1) != s["mode"] or m_odt.group(1) != s.get("o_dtype", s["dtype"]):
        return None
    src = os.path.join(ROOT, "linear_attention_ttt_amd", "csrc", KERNEL_SOURCE[method_of(s["mode"])])
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != m_sha.group(1):
        return None
    return int(m_bytes.group(1))


def run_workload(name: str, steps: int, warmup: int, flush_mb: int, other_order: bool = False, mode=None,
                 momentum=None, muon=None):
    import torch
    import linear_attention_ttt_amd as la

    s = workloads.spec(name)
    if other_order:
        s["mode"] = OTHER_ORDER[s["mode"]]
    if mode:
        s["mode"] = mode
    x = workloads.generate(s, seed=0)
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if s["dtype"] == "bf16" else torch.float32
    odt = torch.float32 if s["o_dtype"] == "fp32" else dt
    B, H, T, dv = s["B"], s["H"], s["T"], s["d_v"]
    desc = la.make_desc(B, H, T, s["d_k"], dv, s["d_h"], la.BF16 if dt == torch.bfloat16 else la.FP32,
                        la.O_FP32 if odt != dt else la.O_AS_INPUT)
    nws = la.muon_workspace_bytes(desc, s["chunk"], s["mode"]) if muon is not None else \
        la.workspace_bytes(desc, s["chunk"], s["mode"])
    nbytes, flops = algorithmic(s)
    # copies of the inputs and outputs for the steady-state loop: enough that their total exceeds the
    # caches (256 MB last-level cache) several times over
    nsets = int(min(8, max(2, -(-(768 << 20) // max(nbytes, 1)))))
    sets = []
    for i in range(nsets):
        t = {k: torch.from_numpy(np.ascontiguousarray(x[k])).to(dev) for k in ("Q", "K", "V", "eta", "W0")}
        for k in ("Q", "K", "V"):
            t[k] = t[k].to(dt)
        t["O"] = torch.empty((B, H, T, dv), dtype=odt, device=dev)
        t["Wout"] = torch.empty_like(t["W0"])
        t["M"] = torch.zeros_like(t["W0"]) if momentum is not None else None   # (Muon with momentum too)
        sets.append(t)
    del x
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    # cache eviction before every flushed step, outside the timed region: overwrite one buffer, then read
    # another, so that the last-level cache and the L2s hold neither the inputs nor dirty lines whose
    # write-back would otherwise land in the next timed step
    flush = torch.empty(flush_mb << 20, dtype=torch.uint8, device=dev)
    flush_rd = torch.ones((flush_mb << 20) // 4, dtype=torch.float32, device=dev)   # fp32: summed without a copy

    def evict(v):
        flush.fill_(v)
        flush_rd.sum()

    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    # arguments prepared once: each step is one library call (no Python-side checks inside the timed region)
    def step(i=0, timing=None):
        t = sets[i % nsets]
        ptrs = [t[k].data_ptr() for k in ("Q", "K", "V", "eta", "W0")]
        if muon is not None:       # no timed form either
            if timing is not None:
                timing[0].record(sptr)
            mp = t["M"].data_ptr() if t["M"] is not None else None
            st = la.forward_muon_raw(*ptrs, mp, momentum or 0.0, muon, s["chunk"], s["mode"], desc, t["O"].data_ptr(),
                                     t["Wout"].data_ptr(), mp, ws.data_ptr(), ws.numel(), sptr)
            if timing is not None:
                timing[1].record(sptr)
        elif momentum is not None:   # ttt_la_forward_momentum has no timed form: events around the whole call
            if timing is not None:
                timing[0].record(sptr)
            st = la.forward_momentum_raw(*ptrs, t["M"].data_ptr(), momentum, s["chunk"], s["mode"], desc,
                                         t["O"].data_ptr(), t["Wout"].data_ptr(), t["M"].data_ptr(), ws.data_ptr(),
                                         ws.numel(), sptr)
            if timing is not None:
                timing[1].record(sptr)
        elif timing is None:
            st = la.forward_raw(*ptrs, s["chunk"], s["mode"], desc, t["O"].data_ptr(), t["Wout"].data_ptr(),
                                ws.data_ptr(), ws.numel(), sptr)
        else:
            st = la.forward_timed_raw(*ptrs, s["chunk"], s["mode"], desc, t["O"].data_ptr(), t["Wout"].data_ptr(),
                                      ws.data_ptr(), ws.numel(), sptr, timing[0].handle, timing[1].handle)
        if st != 0:
            raise RuntimeError(f"ttt_la_forward failed: {la.status_string(st)}")

    # reference call through the checked binding (also validates the raw arguments above)
    t0 = sets[0]
    if muon is None and momentum is None:
        la.forward(t0["Q"], t0["K"], t0["V"], t0["eta"], t0["W0"], s["chunk"], s["mode"], out=t0["O"],
                   W_out=t0["Wout"], workspace=ws, out_dtype=odt)

    for _ in range(warmup):
        evict(1)
        step()
    torch.cuda.synchronize()
    # 1. flushed steps, each between events on the stream with nothing recorded inside the call
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(steps):
        evict(i & 0xFF)
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    # 2. steady state: back-to-back calls over the rotating copies, one pair of events around them all
    for i in range(nsets):
        step(i)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(steps):
        step(i)
    b.record(stream)
    torch.cuda.synchronize()
    ss_ms = a.elapsed_time(b) / steps
    # 3. the dominant kernel, between fence-free events the library records around it (the two extra queue
    # packets lengthen a step by a few microseconds, so the step time is not taken from this loop)
    kstarts = [la.TimingEvent() for _ in range(steps)]
    kends = [la.TimingEvent() for _ in range(steps)]
    for i in range(steps):
        evict(i & 0xFF)
        step(timing=(kstarts[i], kends[i]))
    torch.cuda.synchronize()
    kms = np.array([a_.elapsed_ms(b_) for a_, b_ in zip(kstarts, kends)])
    kname, kunits, kbound = dominant_kernel(s)
    kmean_s = float(kms.mean()) * 1e-3
    mean_s = float(ms.mean()) * 1e-3
    peak = HBM_PEAK_GBS if kbound == "hbm" else BF16_PEAK_TFLOPS
    achieved = kunits / kmean_s / (1e9 if kbound == "hbm" else 1e12)
    plain = not (other_order or mode or momentum is not None or muon is not None)
    roof = {"bound": kbound, "achieved": achieved, "peak": peak, "unit": "GB/s" if kbound == "hbm" else "TFLOP/s",
            "frac": achieved / peak, "traffic": traffic_per_launch(name, s) if plain else None,
            "kernel": kname, "kernel_ms": float(kms.mean()), "kernel_ms_min": float(kms.min()),
            "units_per_launch": kunits,
            "step_frac": (nbytes / mean_s / 1e9 / HBM_PEAK_GBS) if kbound == "hbm"
            else (flops / mean_s / 1e12 / BF16_PEAK_TFLOPS),
            "steady_state_step_frac": (nbytes / (ss_ms * 1e-3) / 1e9 / HBM_PEAK_GBS) if kbound == "hbm"
            else (flops / (ss_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS)}
    if CEILINGS:
        prac = CEILINGS["copy_GBps"] if kbound == "hbm" else CEILINGS["bf16_gemm_TFLOPs"]
        roof["practical_peak"] = prac
        roof["practical_frac"] = achieved / prac
    if not plain:
        roof["kernel"] += " (whole call: the update-rule entries have no timed form)" if (
            momentum is not None or muon is not None) else ""
    rec = dict(workload=name, mode=s["mode"], B=B, H=H, T=T, d=s["d_k"], d_h=s["d_h"], chunk=s["chunk"],
               update_rule=("muon %g" % muon if muon is not None else "") +
               (" momentum %g" % momentum if momentum is not None else "") or "descent",
               dtype=s["dtype"], o_dtype=s["o_dtype"], ms_per_step=float(ms.mean()), ms_min=float(ms.min()),
               ms_median=float(np.median(ms)), tokens_per_s=B * T / mean_s, token_heads_per_s=B * H * T / mean_s,
               steady_state=dict(ms_per_step=ss_ms, tokens_per_s=B * T / (ss_ms * 1e-3), input_sets=nsets,
                                 note="back-to-back calls over rotating copies of the inputs and outputs, "
                                      "no eviction between calls"),
               algorithmic_bytes=nbytes, algorithmic_flops=flops,
               hbm_GBps=nbytes / mean_s / 1e9, hbm_frac=nbytes / mean_s / 1e9 / HBM_PEAK_GBS,
               bf16_mfma_TFLOPs=flops / mean_s / 1e12, bf16_mfma_frac=flops / mean_s / 1e12 / BF16_PEAK_TFLOPS,
               wall_s_including_flush=wall, roofline=roof)
    del sets, ws, flush, flush_rd
    torch.cuda.empty_cache()
    return rec


def run_backward(name: str, steps: int, warmup: int, flush_mb: int, mode: str):
    """Time ttt_la_backward (the workload's mode: per-token, large-chunk linear or SwiGLU) on its inputs and
    seeded upstream gradients, each call bracketed by events with the caches
    flushed in between, as for the forward.  Algorithmic bytes: read Q, K,
    V, dO (bf16), eta, W0, dW; write dQ, dK, dV (fp32), deta, dW0."""
    import torch
    import linear_attention_ttt_amd as la

    s = workloads.spec(name, mode=mode)
    x = workloads.generate(s, seed=0)
    gr = workloads.generate_grads(s, seed=0)
    dev = torch.device("cuda:0")
    t = {k: torch.from_numpy(x[k]).to(dev) for k in ("Q", "K", "V", "eta", "W0")}
    for k in ("Q", "K", "V"):
        t[k] = t[k].to(torch.bfloat16)
    dO = torch.from_numpy(gr["dO"]).to(dev).to(torch.bfloat16)
    dW = torch.from_numpy(gr["dW"]).to(dev)
    del x, gr
    B, H, T, d = s["B"], s["H"], s["T"], s["d_k"]
    desc = la.make_desc(B, H, T, d, d, s["d_h"], la.BF16)
    ws = torch.empty(la.backward_workspace_bytes(desc, s["chunk"], s["mode"]), dtype=torch.uint8, device=dev)
    outs = [torch.empty((B, H, T, d), dtype=torch.float32, device=dev) for _ in range(3)]
    deta = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    dW0 = torch.empty_like(t["W0"])
    flush = torch.empty(flush_mb << 20, dtype=torch.uint8, device=dev)
    flush_rd = torch.ones((flush_mb << 20) // 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    ptrs = [t[k].data_ptr() for k in ("Q", "K", "V", "eta", "W0")]

    def step():
        st = la.backward_raw(*ptrs, dO.data_ptr(), dW.data_ptr(), s["chunk"], s["mode"], desc,
                             *[o.data_ptr() for o in outs], deta.data_ptr(), dW0.data_ptr(), ws.data_ptr(),
                             ws.numel(), stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"ttt_la_backward failed: {la.status_string(st)}")

    for _ in range(warmup):
        flush.fill_(1)
        flush_rd.sum()
        step()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        flush.fill_(i & 0xFF)
        flush_rd.sum()
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    n = B * H * T
    state = int(np.prod(workloads.state_shape(s))) * 4
    nbytes = n * (4 * d * 2 + 4) + n * (3 * d * 4 + 4) + 3 * state
    mean_s = float(ms.mean()) * 1e-3
    rec = dict(workload=name, mode=s["mode"], ms_per_step=float(ms.mean()), ms_min=float(ms.min()),
               tokens_per_s=B * T / mean_s, algorithmic_bytes=nbytes, hbm_GBps=nbytes / mean_s / 1e9,
               hbm_frac=nbytes / mean_s / 1e9 / HBM_PEAK_GBS,
               note="float32 gradients")
    if method_of(s["mode"]).startswith("large_chunk_swiglu"):
        # per token-head: the step's vector-Jacobian product 30 d d_h, the read's gradients 16 d d_h, the
        # recomputed recurrence 12 d d_h (all as bf16 MFMA products; the hi + lo splits not counted)
        flops = n * 58 * d * s["d_h"]
        rec.update(algorithmic_flops=flops, bf16_mfma_TFLOPs=flops / mean_s / 1e12,
                   bf16_mfma_frac=flops / mean_s / 1e12 / BF16_PEAK_TFLOPS)
    del t, dO, dW, ws, outs, deta, dW0, flush, flush_rd
    torch.cuda.empty_cache()
    return rec


def practical_ceilings(reps: int = 5):
    """Measured practical ceilings of this GPU, next to the published peaks: a 1 GiB device copy (bytes read +
    written per second) and an 8192^3 bf16 matrix product (dense FLOP/s of the vendor library).  Best of
    `reps` runs each, timed with events."""
    import torch

    def best(fn):
        fn()
        ts = []
        for _ in range(reps):
            a0, b0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record()
            fn()
            b0.record()
            torch.cuda.synchronize()
            ts.append(a0.elapsed_time(b0) * 1e-3)
        return min(ts)

    n = 1 << 28                                   # 2^28 floats = 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t_copy = best(lambda: dst.copy_(src))
    del src, dst
    m = 8192
    x = torch.randn((m, m), dtype=torch.bfloat16, device="cuda")
    y = torch.randn((m, m), dtype=torch.bfloat16, device="cuda")
    t_mm = best(lambda: torch.matmul(x, y))
    del x, y
    torch.cuda.empty_cache()
    return {"copy_GBps": 2 * 4 * n / t_copy / 1e9, "bf16_gemm_TFLOPs": 2 * m ** 3 / t_mm / 1e12,
            "how": "best of 5: 1 GiB fp32 device copy (read + write bytes), 8192^3 bf16 torch.matmul; "
                   "roofline.practical_frac = achieved / (copy_GBps for HBM-bound kernels, bf16_gemm_TFLOPs for "
                   "MFMA-bound ones)"}


def host_info():
    """The host the oracle baseline runs on: CPU model, core counts, BLAS threads."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = [{"api": i.get("internal_api"), "threads": i.get("num_threads")} for i in threadpool_info()]
    except Exception:  # threadpoolctl missing: reported as unknown
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "blas": blas}


def cpu_baseline(name: str, mode: str, target_s: float = 12.0):
    """Time the fp64 oracle on a bounded sample of the workload: whole
    sequences of a subset of the (independent) heads, scaled to the full
    workload's tokens/s."""
    import oracle

    s = workloads.spec(name, mode=mode)
    x = workloads.generate(s, seed=0)
    BH = s["B"] * s["H"]

    def heads(idx):
        return {k: x[k].reshape((BH,) + x[k].shape[2:])[idx][None] for k in ("Q", "K", "V", "eta", "W0")}

    # calibrate on one head, then size the sample to about target_s seconds
    h1 = heads([0])
    w0 = time.perf_counter()
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
            "host_cpus_available": len(os.sched_getaffinity(0)), "host": host_info()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=workloads.HEADLINE)
    ap.add_argument("--no-others", action="store_true", help="skip the other workloads' sub-records")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baselines")
    ap.add_argument("--flush-mb", type=int, default=512)
    ap.add_argument("--no-backward", action="store_true", help="skip the backward sub-records")
    ap.add_argument("--momentum", type=float, default=None,
                    help="large-chunk linear workloads: run ttt_la_forward_momentum with this coefficient (the "
                         "kernel-timing loop then times whole calls); implies --no-others --no-backward")
    ap.add_argument("--muon", type=float, default=None,
                    help="SwiGLU workloads: run ttt_la_forward_muon with this scale (with --momentum too if given); "
                         "implies --no-others --no-backward")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the update-rule records (momentum, Muon) of the large-chunk workloads")
    ap.add_argument("--mode", default=None,
                    help="run the workload in this mode instead of its own (same shapes; e.g. "
                         "large_chunk_swiglu_last_layer on the SwiGLU workload); implies --no-others")
    ap.add_argument("--other-order", action="store_true",
                    help="run every workload in its method's other read order (exclusive per-token read, "
                         "update-then-read chunks)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="first copy a buffer of this size 3 times (untimed), as a known-size reference for "
                         "FETCH_SIZE / WRITE_SIZE counter runs")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: libttt_la has no multi-GPU path "
              "(every (b,h) recurrence is independent; sharding B*H across GPUs needs no communication)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if a.calibrate_copy_mb > 0:
        src = torch.ones(a.calibrate_copy_mb << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    CEILINGS.update(practical_ceilings())
    if a.mode:
        a.no_others = True
    if a.momentum is not None or a.muon is not None:
        a.no_others = a.no_backward = a.no_variants = True
    if a.mode or a.other_order:
        a.no_variants = True
    head = run_workload(a.workload, a.steps, a.warmup, a.flush_mb, a.other_order, a.mode, a.momentum, a.muon)
    if not a.no_cpu:
        head["cpu_baseline"] = cpu_baseline(a.workload, head["mode"], target_s=15.0)
    print(f"# {a.workload}: {head['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)
    others = {}
    if not a.no_others:
        for name in workloads.WORKLOADS:
            if name == a.workload:
                continue
            try:
                rec = run_workload(name, max(10, a.steps // 2), 3, a.flush_mb, a.other_order)
                if not a.no_cpu:
                    rec["cpu_baseline"] = cpu_baseline(name, rec["mode"], target_s=8.0)
                others[name] = rec
                print(f"# {name}: {rec['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)
            except Exception as e:  # a mode not built yet is reported, not fatal
                others[name] = {"error": str(e)[:200]}
    # the other update rules the LaCT review compares (momentum, Muon) on the large-chunk workloads
    variants = {}
    if not a.no_variants:
        for key, name, mom, mu in (
                ("linear momentum 0.9", "large_chunk_linear_bf16_B1H12T196608_d64_c4096", 0.9, None),
                ("swiglu momentum 0.9", "large_chunk_swiglu_bf16_B2H8T32768_d128_dh256_c2048", 0.9, None),
                ("swiglu muon 0.05", "large_chunk_swiglu_bf16_B2H8T32768_d128_dh256_c2048", None, 0.05),
                ("swiglu muon 0.05 momentum 0.9", "large_chunk_swiglu_bf16_B2H8T32768_d128_dh256_c2048", 0.9, 0.05)):
            try:
                rec = run_workload(name, max(10, a.steps // 2), 3, a.flush_mb, momentum=mom, muon=mu)
                variants[key] = {k: rec[k] for k in ("workload", "mode", "update_rule", "ms_per_step", "ms_min",
                                                     "tokens_per_s", "steady_state", "hbm_frac", "bf16_mfma_frac")}
                print(f"# {key}: {rec['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)
            except Exception as e:  # reported, not fatal
                variants[key] = {"error": str(e)[:200]}
    # backward records: the headline workload, and (with the other workloads) every bf16 workload
    backward = {}
    if not a.no_backward:
        names = [a.workload] + ([] if a.no_others else [n for n in workloads.WORKLOADS if n != a.workload])
        for name in names:
            sw = workloads.spec(name)
            mode = a.mode or (OTHER_ORDER[sw["mode"]] if a.other_order else sw["mode"])
            if sw["dtype"] != "bf16":
                continue
            try:
                backward[name] = run_backward(name, max(10, a.steps // 2), 3, a.flush_mb, mode)
            except Exception as e:  # reported, not fatal
                backward[name] = {"error": str(e)[:200]}
    s = workloads.spec(a.workload, mode=head["mode"])
    roof = head.pop("roofline")
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
                   "d_k": s["d_k"], "d_v": s["d_v"], "d_h": s["d_h"], "chunk": s["chunk"],
                   "o_dtype": s["o_dtype"]},
        "bf16_mfma_frac": head["bf16_mfma_frac"],
        "token_heads_per_s": head["token_heads_per_s"],
        "steady_state": head["steady_state"],
        "roofline": roof,
        "practical_ceilings": CEILINGS,
        "cpu_baseline": head.get("cpu_baseline"),
        "workloads": others,
        "update_rules": variants,
        "backward": backward,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
