// Internal interface between the C-ABI host layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ttt {

// Events recorded on the launch stream immediately before and after the
// dominant kernel of a forward call (either may be null).
struct Timing {
  hipEvent_t start = nullptr, stop = nullptr;
};
inline hipError_t mark(hipEvent_t e, hipStream_t s) { return e ? hipEventRecord(e, s) : hipSuccess; }

struct PerTokenArgs {
  const void* Q;
  const void* K;
  const void* V;
  const float* eta;
  const float* W0;
  void* O;
  float* W_out;
  void* ws;
  int64_t B, H, T, DK, DV, chunk;
  int dtype;      // 0 = fp32, 1 = bf16
  int exclusive;  // 1: a query reads before its own token's step
  int o_f32;      // 1: O is float32 (bf16 inputs; float32 inputs always give float32 O)
};

// Sequence segments of the bf16 per-token path (segments per head, tokens per segment).
struct SegPlan {
  int nseg, seg_len;
};
// a segment holds at most max_seg_tokens tokens (its views are addressed with 32-bit offsets)
SegPlan per_token_seg_plan(int64_t BH, int64_t T, int64_t dk, int64_t max_seg_tokens = (int64_t)1 << 22);
bool per_token_supported(int64_t dk, int64_t dv, int64_t chunk, int dtype);
size_t per_token_workspace(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int dtype, int o_f32);
hipError_t launch_per_token(const PerTokenArgs& a, hipStream_t stream, const Timing& tm);

// Backward (bf16 inputs): gradients of O and of the final memory in, float32 gradients of Q, K, V,
// eta and W0 out.  other_order: the exclusive per-token read, or update-then-read chunks.
struct BackwardArgs {
  const void* Q;
  const void* K;
  const void* V;
  const float* eta;
  const float* W0;
  const void* dO;
  const float* dW;
  void* dQ;
  void* dK;
  void* dV;
  float* deta;
  float* dW0;
  void* ws;
  int64_t B, H, T, DK, DV, chunk;
  int dtype;
  int other_order;
};
bool per_token_backward_supported(int64_t dk, int64_t dv, int64_t chunk, int dtype);
size_t per_token_backward_workspace(int64_t B, int64_t H, int64_t T, int64_t dk);
hipError_t launch_per_token_backward(const BackwardArgs& a, hipStream_t stream);

struct LargeChunkArgs {
  const void* Q;
  const void* K;
  const void* V;
  const float* eta;
  const float* W0;
  void* O;
  float* W_out;
  void* ws;
  int64_t B, H, T, DK, DV, DH, chunk;
  int dtype;
  int update_first;  // 1: a chunk takes its step, then its queries read the result
  int last_layer_only = 0;  // SwiGLU: only W2 is updated, and nothing is normalised
  // large-chunk linear: momentum buffer M_c = momentum M_{c-1} + dW_c (from M0, zeros when null;
  // the final buffer into M_out when not null)
  const float* M0 = nullptr;
  float* M_out = nullptr;
  float momentum = 0.f;
  int o_f32 = 0;  // 1: O is float32
  // SwiGLU: Muon (the step of each matrix replaced by muon_scale * NS5(step)); momentum needs M_out
  int muon = 0;
  float muon_scale = 0.f;
};

bool large_chunk_linear_supported(int64_t dk, int64_t dv, int64_t chunk, int dtype);
size_t large_chunk_linear_workspace(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t chunk);
hipError_t launch_large_chunk_linear(const LargeChunkArgs& a, hipStream_t stream, const Timing& tm);
size_t large_chunk_linear_backward_workspace(int64_t B, int64_t H, int64_t T, int64_t d, int64_t chunk);
hipError_t launch_large_chunk_linear_backward(const BackwardArgs& a, hipStream_t stream);

bool large_chunk_swiglu_supported(int64_t d, int64_t dh, int64_t chunk, int dtype);
size_t large_chunk_swiglu_workspace(int64_t B, int64_t H, int64_t T, int64_t d, int64_t dh, int64_t chunk,
                                    int muon = 0);
hipError_t launch_large_chunk_swiglu(const LargeChunkArgs& a, hipStream_t stream, const Timing& tm);
// the recurrence again with every chunk's float32 weights into dump [BH][nchunks][3 d d_h] and the column
// norms before each normalisation into dnorm [BH][nchunks][640]; a.ws is a forward workspace of
// swiglu_forward_workspace_plain(BH, nchunks) bytes; a.W_out receives the final weights
hipError_t launch_swiglu_recur_dump(const LargeChunkArgs& a, float* dump, float* dnorm, hipStream_t stream);
size_t swiglu_forward_workspace_plain(int64_t BH, int64_t nchunks);
// backward of the SwiGLU modes (2, 5, 6): recomputation, then the reverse chunk loop
size_t large_chunk_swiglu_backward_workspace(int64_t B, int64_t H, int64_t T, int64_t chunk);
hipError_t launch_large_chunk_swiglu_backward(const BackwardArgs& a, int last_layer_only, hipStream_t stream);

}  // namespace ttt
