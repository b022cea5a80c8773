"""C-ABI tests that need no GPU: the library loads, exports every declared
symbol, and rejects invalid arguments before touching the device."""
import ctypes
import os
import re

import pytest

import linear_attention_ttt_amd as la

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ttt_la.h")

needs_lib = pytest.mark.skipif(not os.path.exists(la.library_path), reason="libttt_la.so not built")

# Fake, non-overlapping device addresses: validation never dereferences them.
BASE = 1 << 40
GAP = 1 << 34


def ptr(i):
    return BASE + i * GAP


def call(Q=ptr(0), K=ptr(1), V=ptr(2), eta=ptr(3), W0=ptr(4), chunk=64, mode=0, desc=None, O=ptr(5),
         W_out=ptr(6), ws=ptr(7), ws_bytes=1 << 33):
    if desc is None:
        desc = la.make_desc(1, 2, 128, 64, 64, 0, la.BF16)
    return la.forward_raw(Q, K, V, eta, W0, chunk, mode, desc, O, W_out, ws, ws_bytes, None)


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(ttt_la_[a-z_]+)\s*\(", src)))


@needs_lib
def test_exports_every_declared_symbol():
    L = la.lib()
    names = declared_functions()
    assert {"ttt_la_forward", "ttt_la_workspace_bytes", "ttt_la_status_string", "ttt_la_abi_version",
            "ttt_la_event_create", "ttt_la_event_record", "ttt_la_event_elapsed_ms",
            "ttt_la_event_destroy", "ttt_la_backward", "ttt_la_backward_workspace_bytes",
            "ttt_la_forward_momentum"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} not exported"


@needs_lib
def test_version_and_status_strings():
    assert la.lib().ttt_la_abi_version() == 7
    for s in range(10):
        assert la.status_string(s) and la.status_string(s) != "unknown status"
    assert la.status_string(99) == "unknown status"


@needs_lib
@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), 1), (dict(K=None), 1), (dict(V=None), 1), (dict(eta=None), 1), (dict(O=None), 1),
    (dict(W0=None), 1), (dict(W_out=None), 1),
    (dict(chunk=0), 3), (dict(chunk=-5), 3),
    (dict(mode=7), 5), (dict(mode=-1), 5),
])
def test_invalid_arguments(kw, code):
    assert call(**kw) == code


@needs_lib
def test_null_desc():
    L = la.lib()
    r = L.ttt_la_forward(ptr(0), ptr(1), ptr(2), ptr(3), ptr(4), 64, 0, None, ptr(5), ptr(6), None, 0, None)
    assert r == 1
    assert L.ttt_la_workspace_bytes(None, 64, 0) == 0


@needs_lib
@pytest.mark.parametrize("desc,mode,code", [
    (la.make_desc(0, 1, 8, 64, 64), 0, 2),
    (la.make_desc(1, 0, 8, 64, 64), 0, 2),
    (la.make_desc(1, 1, -1, 64, 64), 0, 2),
    (la.make_desc(1, 1, 8, 0, 64), 0, 2),
    (la.make_desc(1, 1, 8, 64, 0), 0, 2),
    (la.make_desc(1, 1, 8, 128, 64, 256), 2, 2),       # SwiGLU needs d_k == d_v
    (la.make_desc(1, 1, 8, 128, 128, 0), 2, 2),        # SwiGLU needs d_h
    (la.make_desc(1, 1, 8, 128, 64, 256), 5, 2),       # so does its update-first variant
    (la.make_desc(1, 1, 8, 128, 128, 0), 5, 2),
    (la.make_desc(1, 1, 8, 64, 64, 0, 7), 0, 4),       # bad dtype
    (la.make_desc(1, 1, 8, 96, 96), 0, 6),             # d not compiled
    (la.make_desc(1, 1, 8, 64, 128), 0, 6),            # d_k != d_v not compiled
    (la.make_desc(1, 1, 0, 2**62, 2**62, 256), 2, 2),  # sizes that overflow 64 bits (no tokens)
    (la.make_desc(1, 1, 0, 128, 128, 2**62), 2, 2),
])
def test_invalid_shapes(desc, mode, code):
    assert call(desc=desc, mode=mode) == code


@needs_lib
@pytest.mark.parametrize("o_dtype", [2, -1, 7])
def test_output_dtype_outside_enum(o_dtype):
    assert call(desc=la.make_desc(1, 1, 8, 64, 64, 0, la.BF16, o_dtype)) == 4


@needs_lib
def test_float32_output_range_checked_for_aliasing():
    # with float32 O the output spans twice the bytes of a bf16 one: it reaches into K placed just after
    desc = la.make_desc(1, 2, 128, 64, 64, 0, la.BF16, la.O_FP32)
    obytes16 = 1 * 2 * 128 * 64 * 2
    assert call(O=ptr(1) - obytes16, desc=desc) == 7
    # just clear of K it passes the alias check and stops at the (missing) workspace, before any HIP call
    assert la.workspace_bytes(desc, 64, 0) > 0
    assert call(O=ptr(1) - 2 * obytes16 - 256, desc=desc, ws=None, ws_bytes=0, chunk=64) == 8


@needs_lib
def test_backward_needs_output_in_input_dtype():
    d = la.make_desc(1, 2, 256, 128, 128, 0, la.BF16, la.O_FP32)
    assert la.backward_workspace_bytes(d, 64, "per_token_linear") == 0
    r = la.backward_raw(ptr(0), ptr(1), ptr(2), ptr(3), ptr(4), ptr(5), ptr(6), 64, "per_token_linear", d, ptr(7),
                        ptr(8), ptr(9), ptr(10), ptr(11), ptr(12), 1 << 33, None)
    assert r == 6


@needs_lib
def test_float32_output_workspace():
    # per-token: float32 rows cap a segment at 2^21 tokens, so a long sequence may take more segments
    for o in (la.O_AS_INPUT, la.O_FP32):
        d = la.make_desc(1, 32, 32768, 128, 128, 0, la.BF16, o)
        assert la.workspace_bytes(d, 128, "per_token_linear") > 0
    one = la.make_desc(1, 1, 1 << 22, 128, 128, 0, la.BF16, la.O_AS_INPUT)
    one32 = la.make_desc(1, 1, 1 << 22, 128, 128, 0, la.BF16, la.O_FP32)
    assert la.workspace_bytes(one32, 64, 0) >= la.workspace_bytes(one, 64, 0)
    # the large-chunk modes' workspace does not depend on the output dtype
    for mode, dd, chunk in ((1, la.make_desc(1, 12, 196608, 64, 64, 0, la.BF16), 4096),
                            (2, la.make_desc(2, 8, 32768, 128, 128, 256, la.BF16), 2048)):
        d32 = la.make_desc(dd.B, dd.H, dd.T, dd.d_k, dd.d_v, dd.d_h, la.BF16, la.O_FP32)
        assert la.workspace_bytes(d32, chunk, mode) == la.workspace_bytes(dd, chunk, mode)


@needs_lib
@pytest.mark.parametrize("chunk,dtype,code", [(48, la.BF16, 6), (256, la.BF16, 6), (128, la.FP32, 6)])
def test_unsupported_per_token_chunk(chunk, dtype, code):
    assert call(chunk=chunk, desc=la.make_desc(1, 1, 64, 64, 64, 0, dtype)) == code


@needs_lib
def test_overflowing_sizes_rejected():
    assert call(desc=la.make_desc(1 << 40, 1 << 40, 8, 64, 64)) == 2


@needs_lib
def test_aliasing_rejected():
    desc = la.make_desc(1, 2, 128, 64, 64)
    qbytes = 1 * 2 * 128 * 64 * 2
    assert call(O=ptr(0), desc=desc) == 7                      # O == Q
    assert call(O=ptr(1) + qbytes - 2, desc=desc) == 7         # O overlaps the tail of K
    assert call(W_out=ptr(2) + 16, desc=desc) == 7             # W_out inside V
    assert call(W_out=ptr(4) + 4, desc=desc) == 7              # partial overlap with W0
    assert call(W_out=ptr(5), desc=desc) == 7                  # W_out overlaps O
    # (an adjacent, non-overlapping layout is valid and would launch: not tested here)


@needs_lib
def test_workspace_query_and_check():
    d = la.make_desc(1, 12, 196608, 64, 64, 0, la.BF16)
    n = la.workspace_bytes(d, 4096, "large_chunk_linear")
    if n == 0:
        pytest.skip("large-chunk linear needs no workspace for this problem")
    assert call(desc=d, mode=1, chunk=4096, ws=None, ws_bytes=0) == 8
    assert call(desc=d, mode=1, chunk=4096, ws_bytes=n - 1) == 8


@needs_lib
def test_ordering_variants_share_support_and_workspace():
    # modes 3, 4, 5 are the other read orders of modes 0, 1, 2: same shapes, support and workspace
    for base, var, desc, chunk in [
            (0, 3, la.make_desc(4, 16, 4096, 128, 128, 0, la.BF16), 64),
            (0, 3, la.make_desc(1, 1, 256, 64, 64, 0, la.FP32), 64),
            (1, 4, la.make_desc(1, 12, 196608, 64, 64, 0, la.BF16), 4096),
            (2, 5, la.make_desc(2, 8, 32768, 128, 128, 256, la.BF16), 2048)]:
        assert la.workspace_bytes(desc, chunk, var) == la.workspace_bytes(desc, chunk, base)
    assert la.MODES["per_token_linear_exclusive"] == 3
    assert la.MODES["large_chunk_linear_update_first"] == 4
    assert la.MODES["large_chunk_swiglu_update_first"] == 5
    assert la.MODES["large_chunk_swiglu_last_layer"] == 6
    d6 = la.make_desc(2, 8, 32768, 128, 128, 256, la.BF16)
    assert la.workspace_bytes(d6, 2048, 6) == la.workspace_bytes(d6, 2048, 2)
    assert call(desc=la.make_desc(1, 1, 8, 128, 128, 0), mode=6) == 2      # needs d_h
    assert call(desc=la.make_desc(1, 1, 8, 96, 96), mode=3) == 6


def test_per_token_workspace():
    # fp32 needs none; bf16 splits a head's sequence into segments of whole
    # 64-token tiles so that heads x segments reach 256 workgroups, and keeps
    # one fp32 d_k x d_v state per segment when there is more than one
    assert la.workspace_bytes(la.make_desc(4, 16, 4096, 128, 128, 0, la.FP32), 64, "per_token_linear") == 0
    assert la.workspace_bytes(la.make_desc(16, 16, 4096, 128, 128, 0, la.BF16), 64, "per_token_linear") == 0
    assert la.workspace_bytes(la.make_desc(1, 1, 64, 64, 64, 0, la.BF16), 64, "per_token_linear") == 0
    d = la.make_desc(4, 16, 4096, 128, 128, 0, la.BF16)        # 64 heads x 4 segments of 16 tiles
    n = la.workspace_bytes(d, 64, "per_token_linear")
    assert n == 4 * 64 * 128 * 128 * 4
    assert la.workspace_bytes(la.make_desc(1, 32, 32768, 128, 128, 0, la.BF16), 128, "per_token_linear") == \
        8 * 32 * 128 * 128 * 4                                  # 32 heads x 8 segments
    assert la.workspace_bytes(la.make_desc(1, 1, 300, 64, 64, 0, la.BF16), 64, "per_token_linear") == \
        5 * 64 * 64 * 4                                         # 5 tiles -> 5 segments of one tile
    # enough heads for one segment each, but a segment holds at most 2^22 tokens (32-bit byte offsets)
    assert la.workspace_bytes(la.make_desc(256, 1, 1 << 22, 128, 128, 0, la.BF16), 64, "per_token_linear") == 0
    assert la.workspace_bytes(la.make_desc(256, 1, (1 << 22) + 64, 128, 128, 0, la.BF16), 64, "per_token_linear") == \
        2 * 256 * 128 * 128 * 4
    assert call(desc=d, mode=0, chunk=64, ws=None, ws_bytes=0) == 8
    assert call(desc=d, mode=0, chunk=64, ws_bytes=n - 1) == 8


@needs_lib
def test_event_helpers_reject_null():
    # argument checks happen before any HIP call, so they run without a GPU
    L = la.lib()
    assert L.ttt_la_event_create(None) == 1
    assert L.ttt_la_event_record(None, None) == 1
    assert L.ttt_la_event_elapsed_ms(None, None, None) == 1
    assert L.ttt_la_event_destroy(None) == 0


def bcall(desc=None, mode=0, chunk=64, ws_bytes=1 << 34, **kw):
    if desc is None:
        desc = la.make_desc(1, 2, 128, 64, 64, 0, la.BF16)
    p = dict(Q=ptr(0), K=ptr(1), V=ptr(2), eta=ptr(3), W0=ptr(4), dO=ptr(5), dW=ptr(6), dQ=ptr(7), dK=ptr(8),
             dV=ptr(9), deta=ptr(10), dW0=ptr(11), ws=ptr(12))
    p.update(kw)
    return la.backward_raw(p["Q"], p["K"], p["V"], p["eta"], p["W0"], p["dO"], p["dW"], chunk, mode, desc, p["dQ"],
                           p["dK"], p["dV"], p["deta"], p["dW0"], p["ws"], ws_bytes, None)


@needs_lib
@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), 1), (dict(dO=None), 1), (dict(dW=None), 1), (dict(dQ=None), 1), (dict(deta=None), 1),
    (dict(dW0=None), 1), (dict(ws=None), 1), (dict(W0=None), 1),
    (dict(mode=2), 2), (dict(mode=7), 5), (dict(chunk=0), 3),
    (dict(mode=2, desc=la.make_desc(1, 2, 128, 128, 128, 256, la.FP32)), 6),    # SwiGLU backward: bf16 only
    (dict(mode=2, desc=la.make_desc(1, 2, 128, 128, 128, 256, la.BF16), ws_bytes=1024), 8),   # its workspace
    (dict(mode=5, desc=la.make_desc(1, 2, 128, 128, 128, 256, la.BF16, la.O_FP32)), 6),   # dO has io_dtype
    (dict(mode=6, desc=la.make_desc(1, 2, 128, 128, 128, 128, la.BF16)), 6),     # d_h = 128 not compiled
    (dict(mode=1, desc=la.make_desc(1, 2, 128, 64, 64, 0, la.FP32)), 6),
    (dict(desc=la.make_desc(1, 2, 128, 96, 96, 0, la.BF16)), 6),
    (dict(chunk=256), 6),
    (dict(ws_bytes=0), 8),
    (dict(dQ=ptr(0)), 7), (dict(dK=ptr(5) + 64), 7), (dict(dW0=ptr(6)), 7), (dict(deta=ptr(7) + 4), 7),
    (dict(dW0=ptr(4) + 8), 7), (dict(dV=ptr(12)), 7),
])
def test_backward_invalid_arguments(kw, code):
    assert bcall(**kw) == code


@needs_lib
def test_backward_workspace():
    # segment slots (4 segments per head here, as in the forward), W0^T, dW^T, a discarded memory and the
    # u pass's partial dots (B H T d/16 floats)
    d = la.make_desc(4, 16, 4096, 128, 128, 0, la.BF16)
    st = 64 * 128 * 128 * 4
    n = la.workspace_bytes(d, 64, "per_token_linear") + 3 * st + 4 * 16 * 4096 * 8 * 4
    assert la.backward_workspace_bytes(d, 64, "per_token_linear") == n
    assert la.backward_workspace_bytes(d, 64, "per_token_linear_exclusive") == n
    # large-chunk linear: two sets of chunk updates (K^T diag(eta) V and Q^T dO), the memories and the
    # normalisation gradients of every chunk, unit rates, a discarded final memory
    dl = la.make_desc(1, 12, 196608, 64, 64, 0, la.BF16)
    m, nc = 64 * 64 * 4, 48
    nsplit = la.workspace_bytes(dl, 4096, "large_chunk_linear") // (12 * nc * m) - 1
    assert la.backward_workspace_bytes(dl, 4096, "large_chunk_linear") == \
        12 * nc * m * (2 * nsplit + 2) + 12 * 196608 * 4 + 12 * m
    assert la.backward_workspace_bytes(dl, 4096, "large_chunk_linear_update_first") == \
        la.backward_workspace_bytes(dl, 4096, "large_chunk_linear")
    # float32 per-token: the transposed states and the discarded memory (one segment, no slots); the
    # partial-dot rows are laid out in every case
    assert la.backward_workspace_bytes(la.make_desc(1, 1, 64, 64, 64, 0, la.FP32), 64, 0) == \
        3 * 64 * 64 * 4 + 64 * 4 * 4
    assert bcall(desc=d, ws_bytes=n - 1) == 8
    # a backward segment holds at most 2^21 tokens (float32 rows addressed below 2^31 bytes)
    d1 = la.make_desc(256, 1, 1 << 22, 128, 128, 0, la.BF16)
    st1 = 256 * 128 * 128 * 4
    assert la.backward_workspace_bytes(d1, 64, 0) == 2 * st1 + 3 * st1 + 256 * (1 << 22) * 8 * 4


def mcall(mode=1, momentum=0.9, M0=ptr(8), M_out=ptr(9), desc=None, **kw):
    if desc is None:
        desc = la.make_desc(1, 2, 128, 64, 64, 0, la.BF16)
    p = dict(Q=ptr(0), K=ptr(1), V=ptr(2), eta=ptr(3), W0=ptr(4), O=ptr(5), W_out=ptr(6), ws=ptr(7))
    p.update(kw)
    return la.forward_momentum_raw(p["Q"], p["K"], p["V"], p["eta"], p["W0"], M0, momentum, 64, mode, desc, p["O"],
                                   p["W_out"], M_out, p["ws"], 1 << 33, None)


@needs_lib
@pytest.mark.parametrize("kw,code", [
    (dict(mode=0), 6), (dict(mode=6, desc=la.make_desc(1, 2, 128, 128, 128, 256, la.BF16)), 6), (dict(mode=3), 6),
    (dict(mode=2, desc=la.make_desc(1, 2, 128, 128, 128, 256, la.BF16), M_out=None), 1),   # SwiGLU needs M_out
    (dict(mode=7), 5), (dict(momentum=float("nan")), 2), (dict(momentum=float("inf")), 2),
    (dict(W0=None), 1),
    (dict(M_out=ptr(0)), 7),                  # M_out over Q
    (dict(M_out=ptr(6)), 7),                  # M_out over W_out
    (dict(M_out=ptr(8) + 4), 7),              # partly over M0
    (dict(M0=ptr(5)), 7),                     # M0 over O
])
def test_momentum_invalid_arguments(kw, code):
    assert mcall(**kw) == code


def muoncall(mode=2, momentum=0.9, scale=0.1, M0=ptr(8), M_out=ptr(9), desc=None, ws_bytes=1 << 33, **kw):
    if desc is None:
        desc = la.make_desc(1, 2, 128, 128, 128, 256, la.BF16)
    p = dict(Q=ptr(0), K=ptr(1), V=ptr(2), eta=ptr(3), W0=ptr(4), O=ptr(5), W_out=ptr(6), ws=ptr(7))
    p.update(kw)
    return la.forward_muon_raw(p["Q"], p["K"], p["V"], p["eta"], p["W0"], M0, momentum, scale, 64, mode, desc,
                               p["O"], p["W_out"], M_out, p["ws"], ws_bytes, None)


@needs_lib
@pytest.mark.parametrize("kw,code", [
    (dict(mode=0, desc=la.make_desc(1, 2, 128, 64, 64, 0, la.BF16)), 6),
    (dict(mode=1, desc=la.make_desc(1, 2, 128, 64, 64, 0, la.BF16)), 6),
    (dict(mode=6), 6), (dict(mode=9), 5),
    (dict(scale=float("nan")), 2), (dict(momentum=float("inf")), 2),
    (dict(M_out=None), 1),                            # momentum without a buffer
    (dict(M_out=None, momentum=0.0), 1),              # M0 given without a buffer
    (dict(W0=None), 1), (dict(O=None), 1),
    (dict(M_out=ptr(4) + 4), 7),                      # buffer over W0
    (dict(ws_bytes=1024), 8),                         # workspace too small
])
def test_muon_invalid_arguments(kw, code):
    assert muoncall(**kw) == code


@needs_lib
def test_muon_workspace_holds_the_exchange():
    d = la.make_desc(2, 8, 32768, 128, 128, 256, la.BF16)
    plain = la.workspace_bytes(d, 2048, "large_chunk_swiglu")
    muon = la.muon_workspace_bytes(d, 2048, "large_chunk_swiglu")
    per_head = (16 + 1) * 3 * 128 * 128 * 4            # partial Gram matrices and their sums
    assert plain > 0 and muon >= plain + 16 * per_head
    assert la.muon_workspace_bytes(d, 2048, "large_chunk_swiglu_update_first") == muon
    assert la.muon_workspace_bytes(d, 2048, "large_chunk_swiglu_last_layer") == 0
    assert la.muon_workspace_bytes(la.make_desc(1, 2, 128, 64, 64, 0, la.BF16), 64, "large_chunk_linear") == 0


@needs_lib
def test_swiglu_backward_workspace():
    d = la.make_desc(2, 8, 32768, 128, 128, 256, la.BF16)
    n = la.backward_workspace_bytes(d, 2048, "large_chunk_swiglu")
    # at least: the recomputation's float32 weights of every chunk (16 heads x 16 chunks x 384 KB)
    assert n > 16 * 16 * 3 * 128 * 256 * 4
    assert la.backward_workspace_bytes(d, 2048, "large_chunk_swiglu_update_first") == n
    assert la.backward_workspace_bytes(d, 2048, "large_chunk_swiglu_last_layer") == n
    assert la.backward_workspace_bytes(la.make_desc(2, 8, 32768, 128, 128, 256, la.BF16, la.O_FP32), 2048, 2) == 0
