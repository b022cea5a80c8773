"""GPU parity of the large-chunk linear backward against the fp64 oracle (through the C ABI)."""
import pytest

from helpers import workloads, to_device
from test_gpu_per_token_backward import check_backward, grads_to_device, run_backward

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", ["large_chunk_linear", "large_chunk_linear_update_first"])
@pytest.mark.parametrize("B,H,T,d,chunk", [
    (1, 2, 300, 64, 128),     # ragged last chunk
    (1, 3, 1000, 128, 300),   # chunk not a multiple of the token blocks
    (1, 1, 2500, 64, 2048),   # several parts of a chunk, ragged
    (1, 2, 97, 64, 1),        # one token per chunk
    (1, 2, 100, 64, 4096),    # one chunk longer than the sequence
    (2, 2, 512, 128, 64),
])
def test_large_chunk_linear_backward_small(mode, B, H, T, d, chunk):
    s = workloads.make_spec(mode, B, H, T, d, chunk=chunk, dtype="bf16", eta_scale=0.05)
    x = workloads.generate(s, seed=21)
    gr = workloads.generate_grads(s, seed=21)
    out = run_backward(to_device(x, s), grads_to_device(gr), s)
    check_backward(s, x, gr, out, label=f"{B},{H},{T},{d},c{chunk}")


def test_large_chunk_linear_backward_empty():
    s = workloads.make_spec("large_chunk_linear", 1, 2, 0, 64, chunk=64, dtype="bf16")
    x = workloads.generate(s, seed=0)
    gr = workloads.generate_grads(s, seed=0)
    dQ, dK, dV, deta, dW0 = run_backward(to_device(x, s), grads_to_device(gr), s)
    import torch
    assert torch.equal(dW0.cpu(), torch.from_numpy(gr["dW"]))


@pytest.mark.parametrize("mode", ["large_chunk_linear", "large_chunk_linear_update_first"])
def test_large_chunk_linear_backward_workload_sampled_heads(mode):
    s = workloads.spec("large_chunk_linear_bf16_B1H12T196608_d64_c4096", mode=mode)
    x = workloads.generate(s, seed=0)
    gr = workloads.generate_grads(s, seed=0)
    out = run_backward(to_device(x, s), grads_to_device(gr), s)
    check_backward(s, x, gr, out, heads=[2, 11], label="B1H12T196608 heads 2,11")
