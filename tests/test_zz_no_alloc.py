"""ttt_la_forward_noalloc (the library's own device scratch, no workspace
argument) against ttt_la_forward with a caller workspace: the same kernels,
so the same outputs bit for bit, on two calls in a row per method, the
second smaller (the scratch keeps the first call's contents)."""
import pytest
import torch

from helpers import la, out_dtype, to_device, workloads


def _desc(s):
    return la.make_desc(s["B"], s["H"], s["T"], s["d_k"], s["d_v"], s["d_h"],
                        la.BF16 if s["dtype"] == "bf16" else la.FP32,
                        la.O_FP32 if s["o_dtype"] == "fp32" and s["dtype"] == "bf16" else la.O_AS_INPUT)


def _noalloc(t, s):
    O = torch.empty((s["B"], s["H"], s["T"], s["d_v"]), dtype=out_dtype(s), device="cuda")
    W = torch.empty_like(t["W0"])
    st = la.forward_noalloc_raw(t["Q"].data_ptr(), t["K"].data_ptr(), t["V"].data_ptr(), t["eta"].data_ptr(),
                                t["W0"].data_ptr(), s["chunk"], s["mode"], _desc(s), O.data_ptr(), W.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    assert st == 0, la.status_string(st)
    return O, W


PAIRS = [
    # (first call, second call): per method, the second smaller
    (workloads.make_spec("per_token_linear", 1, 4, 2000, 128, chunk=64, dtype="bf16", eta="sigmoid"),
     workloads.make_spec("per_token_linear", 1, 2, 500, 128, chunk=64, dtype="bf16", eta="sigmoid")),
    (workloads.make_spec("per_token_linear", 1, 4, 2000, 128, chunk=64, dtype="bf16", eta="sigmoid", o_dtype="fp32"),
     workloads.make_spec("per_token_linear_exclusive", 1, 1, 300, 64, chunk=64, dtype="bf16", eta="sigmoid")),
    (workloads.make_spec("per_token_linear", 1, 2, 300, 64, chunk=32, dtype="fp32"),
     workloads.make_spec("per_token_linear", 1, 1, 100, 64, chunk=32, dtype="fp32")),
    (workloads.make_spec("large_chunk_linear", 1, 3, 3000, 64, chunk=512, dtype="bf16", eta_scale=0.05),
     workloads.make_spec("large_chunk_linear_update_first", 1, 2, 700, 64, chunk=128, dtype="bf16", eta_scale=0.05)),
    (workloads.make_spec("large_chunk_swiglu", 1, 2, 700, 128, d_h=256, chunk=256, dtype="bf16", eta_scale=0.02),
     workloads.make_spec("large_chunk_swiglu", 1, 1, 300, 128, d_h=256, chunk=128, dtype="bf16", eta_scale=0.02)),
    (workloads.make_spec("large_chunk_swiglu_last_layer", 1, 1, 700, 128, d_h=256, chunk=128, dtype="bf16",
                         eta_scale=0.02),
     workloads.make_spec("large_chunk_swiglu_update_first", 1, 1, 200, 128, d_h=256, chunk=64, dtype="bf16",
                         eta_scale=0.02)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("first,second", PAIRS, ids=lambda s: f"{s['mode']}-{s['H']}x{s['T']}")
def test_noalloc_matches_forward(first, second):
    for k, s in enumerate((first, second)):
        x = workloads.generate(s, seed=30 + k)
        t = to_device(x, s)
        O1, W1 = la.forward(t["Q"], t["K"], t["V"], t["eta"], t["W0"], s["chunk"], s["mode"], out_dtype=out_dtype(s))
        O2, W2 = _noalloc(t, s)
        torch.cuda.synchronize()
        eq = (O1.view(torch.int16) if O1.dtype == torch.bfloat16 else O1).equal(
            O2.view(torch.int16) if O2.dtype == torch.bfloat16 else O2)
        print(f"[noalloc {s['mode']} {s['H']}x{s['T']}] workspace {la.workspace_bytes(_desc(s), s['chunk'], s['mode'])}"
              f" bytes, outputs equal: {eq}", flush=True)
        assert eq and torch.equal(W1, W2)


def test_noalloc_rejects_problems_beyond_its_scratch():
    # 1024 chunks of a SwiGLU head need 384 MB of stored states: refused before any HIP call
    d = la.make_desc(1, 1, 1 << 20, 128, 128, 256, la.BF16)
    assert la.workspace_bytes(d, 1024, "large_chunk_swiglu") > la.NOALLOC_SCRATCH_BYTES
    base = 1 << 40
    st = la.forward_noalloc_raw(base, base + (1 << 34), base + (2 << 34), base + (3 << 34), base + (4 << 34), 1024,
                                "large_chunk_swiglu", d, base + (5 << 34), base + (6 << 34), None)
    assert st == 10 and "scratch" in la.status_string(st)
