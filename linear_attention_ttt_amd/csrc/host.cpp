// C-ABI entry points of libttt_la: argument validation, workspace sizing
// and dispatch to the gfx950 kernels.  Every check runs before the first
// HIP call, so an invalid call enqueues nothing and writes nothing.
#include <cmath>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ttt_la.h"
#include "kernels.h"

namespace {

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range(const void* p, size_t bytes) {
  uintptr_t a = (uintptr_t)p;
  return Range{a, a + (p ? bytes : 0)};
}

bool overlap(Range a, Range b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

// The three methods, and whether the mode is the method's other read order (exclusive per-token read,
// update-then-read chunks).  -1 for an unknown mode.
int32_t method_of(int32_t mode) {
  switch (mode) {
    case TTT_LA_PER_TOKEN_LINEAR:
    case TTT_LA_PER_TOKEN_LINEAR_EXCLUSIVE: return TTT_LA_PER_TOKEN_LINEAR;
    case TTT_LA_LARGE_CHUNK_LINEAR:
    case TTT_LA_LARGE_CHUNK_LINEAR_UPDATE_FIRST: return TTT_LA_LARGE_CHUNK_LINEAR;
    case TTT_LA_LARGE_CHUNK_SWIGLU:
    case TTT_LA_LARGE_CHUNK_SWIGLU_UPDATE_FIRST:
    case TTT_LA_LARGE_CHUNK_SWIGLU_LAST_LAYER: return TTT_LA_LARGE_CHUNK_SWIGLU;
  }
  return -1;
}
bool other_order(int32_t mode) {
  return mode == TTT_LA_PER_TOKEN_LINEAR_EXCLUSIVE || mode == TTT_LA_LARGE_CHUNK_LINEAR_UPDATE_FIRST ||
         mode == TTT_LA_LARGE_CHUNK_SWIGLU_UPDATE_FIRST;
}

// 1 when O is float32 (asked for, or the inputs are float32 already)
int o_f32(const ttt_la_desc& d) { return d.o_dtype == TTT_LA_O_FP32 || d.io_dtype == TTT_LA_FP32 ? 1 : 0; }

int64_t state_elems(const ttt_la_desc& d, int method) {
  if (method == TTT_LA_LARGE_CHUNK_SWIGLU) return d.B * d.H * 3 * d.d_k * d.d_h;
  return d.B * d.H * d.d_k * d.d_v;
}

// Shape, mode, dtype and chunk checks shared by forward and workspace sizing.
int check_problem(const ttt_la_desc* d, int64_t chunk, int32_t mode) {
  if (!d) return TTT_LA_ERR_NULL;
  const int32_t method = method_of(mode);
  if (method < 0) return TTT_LA_ERR_MODE;
  if (d->io_dtype != TTT_LA_FP32 && d->io_dtype != TTT_LA_BF16) return TTT_LA_ERR_DTYPE;
  if (d->o_dtype != TTT_LA_O_AS_INPUT && d->o_dtype != TTT_LA_O_FP32) return TTT_LA_ERR_DTYPE;
  if (d->B < 1 || d->H < 1 || d->T < 0 || d->d_k < 1 || d->d_v < 1) return TTT_LA_ERR_SHAPE;
  if (method == TTT_LA_LARGE_CHUNK_SWIGLU && (d->d_h < 1 || d->d_k != d->d_v)) return TTT_LA_ERR_SHAPE;
  int64_t x;
  const int64_t dmax = d->d_k > d->d_v ? d->d_k : d->d_v;
  if (!mul_ok(d->B, d->H, &x) || !mul_ok(x, d->T, &x) || !mul_ok(x, dmax, &x) || !mul_ok(x, 4, &x))
    return TTT_LA_ERR_SHAPE;
  int64_t y;
  if (method == TTT_LA_LARGE_CHUNK_SWIGLU &&
      (!mul_ok(3, d->d_k, &y) || !mul_ok(d->B * d->H, y, &x) || !mul_ok(x, d->d_h, &x) || !mul_ok(x, 4, &x)))
    return TTT_LA_ERR_SHAPE;
  if (chunk < 1) return TTT_LA_ERR_CHUNK;
  return TTT_LA_OK;
}

bool supported(const ttt_la_desc& d, int64_t chunk, int32_t mode) {
  if (d.T > INT32_MAX || d.B * d.H > (int64_t)1 << 24) return false;
  switch (method_of(mode)) {
    case TTT_LA_PER_TOKEN_LINEAR:
      return ttt::per_token_supported(d.d_k, d.d_v, chunk, d.io_dtype);
    case TTT_LA_LARGE_CHUNK_LINEAR:
      return ttt::large_chunk_linear_supported(d.d_k, d.d_v, chunk, d.io_dtype);
    case TTT_LA_LARGE_CHUNK_SWIGLU:
      return ttt::large_chunk_swiglu_supported(d.d_k, d.d_h, chunk, d.io_dtype);
  }
  return false;
}

size_t workspace_for(const ttt_la_desc& d, int64_t chunk, int32_t mode) {
  switch (method_of(mode)) {
    case TTT_LA_PER_TOKEN_LINEAR:
      return ttt::per_token_workspace(d.B, d.H, d.T, d.d_k, d.d_v, d.io_dtype, o_f32(d));
    case TTT_LA_LARGE_CHUNK_LINEAR:
      return ttt::large_chunk_linear_workspace(d.B, d.H, d.T, d.d_k, d.d_v, chunk);
    case TTT_LA_LARGE_CHUNK_SWIGLU:
      return ttt::large_chunk_swiglu_workspace(d.B, d.H, d.T, d.d_k, d.d_h, chunk);
  }
  return 0;
}

size_t muon_workspace_for(const ttt_la_desc& d, int64_t chunk) {
  return ttt::large_chunk_swiglu_workspace(d.B, d.H, d.T, d.d_k, d.d_h, chunk, 1);
}

bool swiglu_rule_mode(int32_t mode) {
  return mode == TTT_LA_LARGE_CHUNK_SWIGLU || mode == TTT_LA_LARGE_CHUNK_SWIGLU_UPDATE_FIRST;
}

}  // namespace

extern "C" {

int ttt_la_abi_version(void) { return TTT_LA_ABI_VERSION; }

const char* ttt_la_status_string(int s) {
  switch (s) {
    case TTT_LA_OK: return "ok";
    case TTT_LA_ERR_NULL: return "a required pointer is NULL";
    case TTT_LA_ERR_SHAPE: return "invalid shape";
    case TTT_LA_ERR_CHUNK: return "chunk must be >= 1";
    case TTT_LA_ERR_DTYPE: return "io_dtype is not TTT_LA_FP32 or TTT_LA_BF16, or o_dtype is not TTT_LA_O_AS_INPUT or TTT_LA_O_FP32";
    case TTT_LA_ERR_MODE: return "unknown mode";
    case TTT_LA_ERR_UNSUPPORTED: return "no compiled kernel supports this shape, dtype or chunk";
    case TTT_LA_ERR_ALIAS: return "an output overlaps an input or another output";
    case TTT_LA_ERR_WORKSPACE: return "workspace too small";
    case TTT_LA_ERR_HIP: return "HIP kernel launch failed";
    case TTT_LA_ERR_SCRATCH: return "the problem needs more workspace than the allocation-free entry point's scratch";
  }
  return "unknown status";
}

size_t ttt_la_workspace_bytes(const ttt_la_desc* desc, int64_t chunk, int32_t mode) {
  if (check_problem(desc, chunk, mode) != TTT_LA_OK) return 0;
  if (!supported(*desc, chunk, mode)) return 0;
  return workspace_for(*desc, chunk, mode);
}

static int forward_impl(const void* Q, const void* K, const void* V, const float* eta, const float* W0,
                        int64_t chunk, int32_t mode, const ttt_la_desc* desc, void* O, float* W_out,
                        void* workspace, size_t workspace_bytes, void* stream, void* ev_start, void* ev_stop,
                        const float* M0, float* M_out, float momentum, int muon = 0, float muon_scale = 0.f) {
  int st = check_problem(desc, chunk, mode);
  if (st != TTT_LA_OK) return st;
  const ttt_la_desc d = *desc;
  const bool have_tokens = d.T > 0;
  if (!W0 || !W_out) return TTT_LA_ERR_NULL;
  if (have_tokens && (!Q || !K || !V || !eta || !O)) return TTT_LA_ERR_NULL;
  if (!supported(d, chunk, mode)) return TTT_LA_ERR_UNSUPPORTED;
  const size_t need = muon ? muon_workspace_for(d, chunk) : workspace_for(d, chunk, mode);
  if (need > 0 && (!workspace || workspace_bytes < need)) return TTT_LA_ERR_WORKSPACE;

  const size_t es = d.io_dtype == TTT_LA_BF16 ? 2 : 4;
  const size_t ntok = (size_t)(d.B * d.H * d.T);
  const Range rQ = range(Q, ntok * d.d_k * es), rK = range(K, ntok * d.d_k * es);
  const Range rV = range(V, ntok * d.d_v * es), rE = range(eta, ntok * 4);
  const int32_t method = method_of(mode);
  const Range rW0 = range(W0, (size_t)state_elems(d, method) * 4);
  const Range rO = range(O, ntok * d.d_v * (o_f32(d) ? 4 : es));
  const Range rWo = range(W_out, (size_t)state_elems(d, method) * 4);
  const Range rWs = range(workspace, need);
  const Range ins[5] = {rQ, rK, rV, rE, rW0};
  for (const Range& in : ins) {
    if (overlap(rO, in) || overlap(rWs, in)) return TTT_LA_ERR_ALIAS;
  }
  for (int i = 0; i < 4; ++i)
    if (overlap(rWo, ins[i])) return TTT_LA_ERR_ALIAS;
  if (overlap(rWo, rW0) && W_out != W0) return TTT_LA_ERR_ALIAS;
  if (overlap(rO, rWo) || overlap(rO, rWs) || overlap(rWo, rWs)) return TTT_LA_ERR_ALIAS;
  // momentum buffers (large-chunk modes): M0 is an input, M_out an output; M_out == M0 in place
  const Range rM0 = range(M0, (size_t)state_elems(d, method) * 4);
  const Range rMo = range(M_out, (size_t)state_elems(d, method) * 4);
  for (const Range& in : ins)
    if (overlap(rMo, in)) return TTT_LA_ERR_ALIAS;
  if (overlap(rO, rM0) || overlap(rWo, rM0) || overlap(rWs, rM0)) return TTT_LA_ERR_ALIAS;
  if (overlap(rMo, rM0) && M_out != M0) return TTT_LA_ERR_ALIAS;
  if (overlap(rMo, rO) || overlap(rMo, rWo) || overlap(rMo, rWs)) return TTT_LA_ERR_ALIAS;

  hipStream_t s = (hipStream_t)stream;
  ttt::Timing tm;
  tm.start = (hipEvent_t)ev_start;
  tm.stop = (hipEvent_t)ev_stop;
  hipError_t e = hipSuccess;
  const int other = other_order(mode) ? 1 : 0;
  if (method == TTT_LA_PER_TOKEN_LINEAR) {
    ttt::PerTokenArgs a{Q, K, V, eta, W0, O, W_out, workspace, d.B, d.H, d.T, d.d_k, d.d_v, chunk, d.io_dtype,
                        other, o_f32(d)};
    e = ttt::launch_per_token(a, s, tm);
  } else {
    ttt::LargeChunkArgs a{Q, K, V, eta, W0, O, W_out, workspace, d.B, d.H, d.T, d.d_k, d.d_v, d.d_h, chunk, d.io_dtype,
                          other, mode == TTT_LA_LARGE_CHUNK_SWIGLU_LAST_LAYER ? 1 : 0, M0, M_out, momentum,
                          o_f32(d), muon, muon_scale};
    e = method == TTT_LA_LARGE_CHUNK_LINEAR ? ttt::launch_large_chunk_linear(a, s, tm)
                                            : ttt::launch_large_chunk_swiglu(a, s, tm);
  }
  return e == hipSuccess ? TTT_LA_OK : TTT_LA_ERR_HIP;
}

int ttt_la_forward_timed(const void* Q, const void* K, const void* V, const float* eta, const float* W0,
                         int64_t chunk, int32_t mode, const ttt_la_desc* desc, void* O, float* W_out,
                         void* workspace, size_t workspace_bytes, void* stream, void* ev_start, void* ev_stop) {
  return forward_impl(Q, K, V, eta, W0, chunk, mode, desc, O, W_out, workspace, workspace_bytes, stream, ev_start,
                      ev_stop, nullptr, nullptr, 0.f);
}

int ttt_la_forward_momentum(const void* Q, const void* K, const void* V, const float* eta, const float* W0,
                            const float* M0, float momentum, int64_t chunk, int32_t mode, const ttt_la_desc* desc,
                            void* O, float* W_out, float* M_out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  const int st = check_problem(desc, chunk, mode);
  if (st != TTT_LA_OK) return st;
  if (method_of(mode) != TTT_LA_LARGE_CHUNK_LINEAR && !swiglu_rule_mode(mode)) return TTT_LA_ERR_UNSUPPORTED;
  if (!std::isfinite(momentum)) return TTT_LA_ERR_SHAPE;
  if (swiglu_rule_mode(mode) && !M_out) return TTT_LA_ERR_NULL;   // the SwiGLU buffers live in M_out
  return forward_impl(Q, K, V, eta, W0, chunk, mode, desc, O, W_out, workspace, workspace_bytes, stream, nullptr,
                      nullptr, M0, M_out, momentum);
}

size_t ttt_la_muon_workspace_bytes(const ttt_la_desc* desc, int64_t chunk, int32_t mode) {
  if (check_problem(desc, chunk, mode) != TTT_LA_OK || !swiglu_rule_mode(mode) || !supported(*desc, chunk, mode))
    return 0;
  return muon_workspace_for(*desc, chunk);
}

int ttt_la_forward_muon(const void* Q, const void* K, const void* V, const float* eta, const float* W0,
                        const float* M0, float momentum, float muon_scale, int64_t chunk, int32_t mode,
                        const ttt_la_desc* desc, void* O, float* W_out, float* M_out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  const int st = check_problem(desc, chunk, mode);
  if (st != TTT_LA_OK) return st;
  if (!swiglu_rule_mode(mode)) return TTT_LA_ERR_UNSUPPORTED;
  if (!std::isfinite(momentum) || !std::isfinite(muon_scale)) return TTT_LA_ERR_SHAPE;
  if ((momentum != 0.f || M0) && !M_out) return TTT_LA_ERR_NULL;   // the buffers live in M_out
  return forward_impl(Q, K, V, eta, W0, chunk, mode, desc, O, W_out, workspace, workspace_bytes, stream, nullptr,
                      nullptr, M0, M_out, momentum, 1, muon_scale);
}

int ttt_la_forward(const void* Q, const void* K, const void* V, const float* eta, const float* W0,
                   int64_t chunk, int32_t mode, const ttt_la_desc* desc, void* O, float* W_out,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return ttt_la_forward_timed(Q, K, V, eta, W0, chunk, mode, desc, O, W_out, workspace, workspace_bytes, stream,
                              nullptr, nullptr);
}

static bool backward_ok(const ttt_la_desc& d, int64_t chunk, int32_t mode) {
  if (!supported(d, chunk, mode)) return false;
  if (d.o_dtype != TTT_LA_O_AS_INPUT) return false;   // dO has io_dtype
  switch (method_of(mode)) {
    case TTT_LA_PER_TOKEN_LINEAR: return ttt::per_token_backward_supported(d.d_k, d.d_v, chunk, d.io_dtype);
    case TTT_LA_LARGE_CHUNK_LINEAR: return d.io_dtype == TTT_LA_BF16;
    case TTT_LA_LARGE_CHUNK_SWIGLU: return d.io_dtype == TTT_LA_BF16;   // (supported: d = 128, d_h = 256)
  }
  return false;
}

static size_t backward_workspace(const ttt_la_desc& d, int64_t chunk, int32_t mode) {
  switch (method_of(mode)) {
    case TTT_LA_PER_TOKEN_LINEAR: return ttt::per_token_backward_workspace(d.B, d.H, d.T, d.d_k);
    case TTT_LA_LARGE_CHUNK_LINEAR: return ttt::large_chunk_linear_backward_workspace(d.B, d.H, d.T, d.d_k, chunk);
  }
  return ttt::large_chunk_swiglu_backward_workspace(d.B, d.H, d.T, chunk);
}

size_t ttt_la_backward_workspace_bytes(const ttt_la_desc* desc, int64_t chunk, int32_t mode) {
  if (check_problem(desc, chunk, mode) != TTT_LA_OK || !backward_ok(*desc, chunk, mode)) return 0;
  return backward_workspace(*desc, chunk, mode);
}

int ttt_la_backward(const void* Q, const void* K, const void* V, const float* eta, const float* W0,
                    const void* dO, const float* dW_out, int64_t chunk, int32_t mode, const ttt_la_desc* desc,
                    void* dQ, void* dK, void* dV, float* deta, float* dW0, void* workspace, size_t workspace_bytes,
                    void* stream) {
  int st = check_problem(desc, chunk, mode);
  if (st != TTT_LA_OK) return st;
  const ttt_la_desc d = *desc;
  if (!W0 || !dW_out || !dW0 || !workspace) return TTT_LA_ERR_NULL;
  if (d.T > 0 && (!Q || !K || !V || !eta || !dO || !dQ || !dK || !dV || !deta)) return TTT_LA_ERR_NULL;
  if (!backward_ok(d, chunk, mode)) return TTT_LA_ERR_UNSUPPORTED;
  const size_t need = backward_workspace(d, chunk, mode);
  if (workspace_bytes < need) return TTT_LA_ERR_WORKSPACE;

  const size_t es = d.io_dtype == TTT_LA_BF16 ? 2 : 4;
  const size_t ntok = (size_t)(d.B * d.H * d.T);
  const size_t st_bytes = (size_t)state_elems(d, method_of(mode)) * 4;
  const Range ins[7] = {range(Q, ntok * d.d_k * es), range(K, ntok * d.d_k * es), range(V, ntok * d.d_v * es),
                        range(eta, ntok * 4), range(W0, st_bytes), range(dO, ntok * d.d_v * es),
                        range(dW_out, st_bytes)};
  const Range outs[6] = {range(dQ, ntok * d.d_k * 4), range(dK, ntok * d.d_k * 4), range(dV, ntok * d.d_v * 4),
                         range(deta, ntok * 4), range(dW0, st_bytes), range(workspace, need)};
  for (int i = 0; i < 6; ++i) {
    for (const Range& in : ins)
      if (overlap(outs[i], in)) return TTT_LA_ERR_ALIAS;
    for (int j = i + 1; j < 6; ++j)
      if (overlap(outs[i], outs[j])) return TTT_LA_ERR_ALIAS;
  }

  ttt::BackwardArgs a{Q,  K,  V,    eta, W0,        dO,  dW_out, dQ,  dK,  dV,          deta,
                         dW0, workspace, d.B, d.H, d.T, d.d_k, d.d_v, chunk, d.io_dtype, other_order(mode) ? 1 : 0};
  hipError_t e;
  switch (method_of(mode)) {
    case TTT_LA_PER_TOKEN_LINEAR: e = ttt::launch_per_token_backward(a, (hipStream_t)stream); break;
    case TTT_LA_LARGE_CHUNK_LINEAR: e = ttt::launch_large_chunk_linear_backward(a, (hipStream_t)stream); break;
    default:
      e = ttt::launch_large_chunk_swiglu_backward(a, mode == TTT_LA_LARGE_CHUNK_SWIGLU_LAST_LAYER ? 1 : 0,
                                                  (hipStream_t)stream);
  }
  return e == hipSuccess ? TTT_LA_OK : TTT_LA_ERR_HIP;
}

int ttt_la_event_create(void** event) {
  if (!event) return TTT_LA_ERR_NULL;
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return TTT_LA_ERR_HIP;
  *event = (void*)e;
  return TTT_LA_OK;
}

int ttt_la_event_record(void* event, void* stream) {
  if (!event) return TTT_LA_ERR_NULL;
  return hipEventRecord((hipEvent_t)event, (hipStream_t)stream) == hipSuccess ? TTT_LA_OK : TTT_LA_ERR_HIP;
}

int ttt_la_event_elapsed_ms(void* start, void* stop, float* ms) {
  if (!start || !stop || !ms) return TTT_LA_ERR_NULL;
  return hipEventElapsedTime(ms, (hipEvent_t)start, (hipEvent_t)stop) == hipSuccess ? TTT_LA_OK : TTT_LA_ERR_HIP;
}

int ttt_la_event_destroy(void* event) {
  if (!event) return TTT_LA_OK;
  return hipEventDestroy((hipEvent_t)event) == hipSuccess ? TTT_LA_OK : TTT_LA_ERR_HIP;
}

}  // extern "C"
