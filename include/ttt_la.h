/*
 * libttt_la - forward pass of a test-time-training (TTT) layer with
 * key-value binding, its backward pass, and the large-chunk forms with the
 * momentum and Muon update rules, for AMD Instinct MI355X (gfx950).
 *
 * The method (pages on "Test-Time Training with KV Binding Is Secretly
 * Linear Attention", paper summary technical sections 2B and 3, and the
 * LaCT review "Test-Time Training Done Right", sections on fast weights,
 * non-linear memory and read order):
 *
 *   A fast weight W (a linear map, or a SwiGLU MLP) is trained at inference
 *   time by gradient descent on the binding loss -<f_W(k_i), v_i> with a
 *   per-token learning rate eta_i, and read by queries q_i.
 *
 *   TTT_LA_PER_TOKEN_LINEAR: one step per token, read after the step:
 *       o_t = q_t (W0 + sum_{i<=t} eta_i k_i^T v_i),
 *       W_out = W0 + sum_i eta_i k_i^T v_i.
 *     This is causal linear attention without softmax or scaling; it is
 *     computed in chunked parallel form.  `chunk` only selects the tile
 *     length of that form: results do not depend on it beyond rounding.
 *
 *   TTT_LA_LARGE_CHUNK_LINEAR: for each chunk of `chunk` tokens (the last
 *     may be shorter): O_c = Q_c W; W <- W + K_c^T diag(eta_c) V_c; then
 *     every column of W (one output unit's fan-in) is divided by
 *     max(||column||_2, 1e-12).  W0 itself is not normalised.
 *
 *   TTT_LA_LARGE_CHUNK_SWIGLU: f_W(x) = (silu(x W1) * (x W3)) W2.  For each
 *     chunk: O_c = f_W(Q_c); the gradient G of sum_{i in c} eta_i
 *     (-<f_W(k_i), v_i>) is taken at those same weights; W <- W - G for
 *     W1, W3, W2; then columns of W1 and W3 (over d) and of W2 (over d_h)
 *     are divided by max(norm, 1e-12).
 *
 *   Ordering variants (the other read orders the pages describe):
 *   TTT_LA_PER_TOKEN_LINEAR_EXCLUSIVE: a query reads before its own token's
 *     step: o_t = q_t (W0 + sum_{i<t} eta_i k_i^T v_i); W_out as above.
 *   TTT_LA_LARGE_CHUNK_LINEAR_UPDATE_FIRST, TTT_LA_LARGE_CHUNK_SWIGLU_UPDATE_FIRST:
 *     each chunk first takes its step (gradient at the weights before it)
 *     and is normalised, then its queries read the result (the update-then-
 *     read order of the LaCT review's read-order section, applied chunk by
 *     chunk).  W_out is the same as in the read-first mode.
 *
 *   TTT_LA_LARGE_CHUNK_SWIGLU_LAST_LAYER: the SwiGLU memory with only its
 *     last layer trained and no normalisation (the paper summary's ablation
 *     ladder, technical section 4: update only the last layer, then drop the
 *     weight normalisation).  W1 and W3 stay as given, so with
 *     phi(x) = silu(x W1) * (x W3) this is block-causal linear attention in
 *     that feature space: O_c = phi(Q_c) W2; W2 <- W2 + phi(K_c)^T diag(eta_c) V_c.
 *     Same shapes, support and workspace as TTT_LA_LARGE_CHUNK_SWIGLU;
 *     W_out holds W1 and W3 unchanged and the final W2.
 *
 * Conventions: row vectors, W stored [d_in, d_out] row-major; every tensor
 * contiguous with the last dimension fastest.
 *
 * Threading and ownership: every pointer is caller-owned device memory
 * (except `desc`, host memory, read during the call only).  The library
 * allocates nothing, frees nothing and never synchronises: work is enqueued
 * on `stream` and the call returns.  It keeps no global state and may be
 * called from several host threads.
 */
#ifndef TTT_LA_H
#define TTT_LA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
    TTT_LA_OK = 0,
    TTT_LA_ERR_NULL = 1,        /* a required pointer is NULL                        */
    TTT_LA_ERR_SHAPE = 2,       /* negative or zero size where one is required,       */
                                /* or d_k != d_v where the mode needs them equal      */
    TTT_LA_ERR_CHUNK = 3,       /* chunk < 1                                          */
    TTT_LA_ERR_DTYPE = 4,       /* io_dtype or o_dtype is not one of its enum values  */
    TTT_LA_ERR_MODE = 5,        /* mode is not one of ttt_la_mode                     */
    TTT_LA_ERR_UNSUPPORTED = 6, /* valid arguments that no compiled kernel covers     */
    TTT_LA_ERR_ALIAS = 7,       /* an output overlaps an input or another output      */
    TTT_LA_ERR_WORKSPACE = 8,   /* workspace smaller than ttt_la_workspace_bytes()    */
    TTT_LA_ERR_HIP = 9,         /* a kernel launch failed (hipGetLastError)           */
    TTT_LA_ERR_SCRATCH = 10     /* ttt_la_forward_noalloc: the problem needs more     */
                                /* workspace than the library's scratch holds         */
};

/* Modes. */
enum {
    TTT_LA_PER_TOKEN_LINEAR = 0,
    TTT_LA_LARGE_CHUNK_LINEAR = 1,
    TTT_LA_LARGE_CHUNK_SWIGLU = 2,
    TTT_LA_PER_TOKEN_LINEAR_EXCLUSIVE = 3,
    TTT_LA_LARGE_CHUNK_LINEAR_UPDATE_FIRST = 4,
    TTT_LA_LARGE_CHUNK_SWIGLU_UPDATE_FIRST = 5,
    TTT_LA_LARGE_CHUNK_SWIGLU_LAST_LAYER = 6
};

/* Element type of Q, K and V (and, by default, of O).  eta and the
 * fast-weight state are always float32. */
enum {
    TTT_LA_FP32 = 0,
    TTT_LA_BF16 = 1
};

/* Element type of O (ttt_la_desc.o_dtype). */
enum {
    TTT_LA_O_AS_INPUT = 0, /* O has io_dtype                                          */
    TTT_LA_O_FP32 = 1      /* O is float32 whatever io_dtype is: the kernels keep      */
                           /* float32 accumulators, so this only drops the final       */
                           /* rounding of a bf16 output, which alone costs up to half  */
                           /* a bf16 ulp of max|o| (over 2% of the output RMS when the */
                           /* outputs are heavy-tailed, e.g. 32 heads of 32K tokens)   */
};

/* Problem description.  d_h is the SwiGLU hidden width (ignored by the
 * linear modes).  io_dtype is TTT_LA_FP32 or TTT_LA_BF16; o_dtype is
 * TTT_LA_O_AS_INPUT or TTT_LA_O_FP32 (any other value is ERR_DTYPE). */
typedef struct ttt_la_desc {
    int64_t B, H, T, d_k, d_v, d_h;
    int32_t io_dtype;
    int32_t o_dtype;
} ttt_la_desc;

/*
 * ttt_la_forward(Q, K, V, eta, W0, chunk, mode) -> (O, W_out)
 *
 *   Q, K   [B,H,T,d_k]  io_dtype, device
 *   V      [B,H,T,d_v]  io_dtype, device
 *   eta    [B,H,T]      float32,  device; any sign (negative = ascent)
 *   W0     initial fast weights, float32, device:
 *            linear modes  [B,H,d_k,d_v]
 *            SwiGLU        [B,H, d*d_h + d*d_h + d_h*d] = W1 [d,d_h] | W3 [d,d_h] | W2 [d_h,d]
 *                          per (b,h), with d = d_k = d_v
 *   chunk  tokens per chunk (>= 1)
 *   mode   TTT_LA_PER_TOKEN_LINEAR | TTT_LA_LARGE_CHUNK_LINEAR | TTT_LA_LARGE_CHUNK_SWIGLU,
 *          or an ordering variant (3 | 4 | 5: same shapes, support and workspace as
 *          modes 0 | 1 | 2), or TTT_LA_LARGE_CHUNK_SWIGLU_LAST_LAYER (6, as mode 2)
 *   desc   sizes and io_dtype (host pointer)
 *   O      [B,H,T,d_v]  io_dtype (float32 with o_dtype TTT_LA_O_FP32), device (written)
 *   W_out  same layout as W0, float32, device (written); W_out == W0 (in
 *          place) is allowed, any other overlap between an output and an
 *          input, or between O, W_out and the workspace, is ERR_ALIAS
 *   workspace, workspace_bytes
 *          device scratch of at least ttt_la_workspace_bytes(desc, chunk,
 *          mode) bytes (may be NULL when that is 0); its contents on entry
 *          do not matter and are undefined on return
 *   stream hipStream_t to enqueue on (NULL = the default stream)
 *
 * Supported set (ERR_UNSUPPORTED otherwise):
 *   per-token:    d_k = d_v in {64, 128}; bf16 or fp32; chunk in
 *                 {16, 32, 64, 128} (the bf16 kernels always work in
 *                 64-token tiles, the fp32 kernel in tiles of `chunk`
 *                 tokens and needs chunk <= 64).  bf16 cuts each head's
 *                 sequence into segments of whole tiles and keeps one fp32
 *                 d_k x d_v state per segment in the workspace (none when
 *                 each head is one segment);
 *   large-chunk linear: d_k = d_v in {64, 128}; bf16; any chunk;
 *   large-chunk SwiGLU: d = 128, d_h = 256; bf16; any chunk.
 *   T = 0 is accepted: O is empty and W_out = W0.
 *
 * Every argument is checked before anything is enqueued: on any error
 * nothing is written and no HIP call is made, except that ERR_HIP reports
 * a failed launch after earlier kernels of the same call were enqueued.
 */
int ttt_la_forward(const void* Q, const void* K, const void* V, const float* eta,
                   const float* W0, int64_t chunk, int32_t mode, const ttt_la_desc* desc,
                   void* O, float* W_out, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * ttt_la_forward_timed: ttt_la_forward (same arguments, checks, results and
 * status codes) that additionally records two HIP events on `stream`
 * immediately before and after the dominant kernel of the call, for
 * measuring that kernel alone:
 *   per-token      the chunked-form kernel over the sequence (bf16: the
 *                  output pass over the segments; fp32: the whole kernel)
 *   large-chunk    the chunk-update kernel (streams K and V)
 *   SwiGLU         the recurrence over the chunks
 * ev_start, ev_stop: hipEvent_t created by the caller (ttt_la_event_create
 * for fence-free timestamps, or hipEventCreate), or NULL to skip; the
 * library only records them.  Nothing is recorded when
 * the call returns an error before enqueueing, nor by large-chunk linear
 * with T = 0 (no chunk to update).
 */
int ttt_la_forward_timed(const void* Q, const void* K, const void* V, const float* eta,
                         const float* W0, int64_t chunk, int32_t mode, const ttt_la_desc* desc,
                         void* O, float* W_out, void* workspace, size_t workspace_bytes,
                         void* stream, void* ev_start, void* ev_stop);

/*
 * ttt_la_forward_momentum: the large-chunk modes (linear: TTT_LA_LARGE_CHUNK_LINEAR and its
 * update-first variant; SwiGLU: TTT_LA_LARGE_CHUNK_SWIGLU and its update-first variant) with
 * momentum in the inner loop, one of the update rules the LaCT review's non-linear-memory
 * section compares.  Each chunk's step S_c (linear: K_c^T diag(eta_c) V_c; SwiGLU: minus the
 * gradient of each of W1, W3, W2, at the weights that read the chunk) goes into a buffer
 * M_c = momentum * M_{c-1} + S_c, and W takes M_c instead, then the column normalisation:
 *     W_c = colnorm(W_{c-1} + M_c)   (per matrix for SwiGLU).
 * momentum = 0 with M0 = NULL gives ttt_la_forward's O and W_out bit for bit.
 *   M0         float32, device, the layout of W0: the buffer before the first chunk (NULL = zeros),
 *              e.g. the M_out of a call on the preceding tokens
 *   momentum   the coefficient (finite; ERR_SHAPE otherwise)
 *   M_out      float32, device, the layout of W0: the buffer after the last chunk; linear: NULL =
 *              not written; SwiGLU: required (ERR_NULL), the buffers are kept there during the
 *              call; M_out == M0 in place is allowed, any other overlap is ERR_ALIAS
 * Other arguments, workspace, checks and status codes as ttt_la_forward; ERR_UNSUPPORTED
 * for the other modes.  ttt_la_backward has no momentum form.
 */
int ttt_la_forward_momentum(const void* Q, const void* K, const void* V, const float* eta,
                            const float* W0, const float* M0, float momentum, int64_t chunk,
                            int32_t mode, const ttt_la_desc* desc, void* O, float* W_out,
                            float* M_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ttt_la_forward_muon: the SwiGLU modes (TTT_LA_LARGE_CHUNK_SWIGLU and its update-first
 * variant) with Muon as the update rule (LaCT review, non-linear-memory section: Muon
 * transforms the matrix gradients by Newton-Schulz iterations; the L2 normalisation follows
 * the update).  For each chunk and each of W1, W3, W2 the step S (minus the gradient at the
 * weights that read the chunk; with momentum != 0 or M0 given, the buffer
 * M_c = momentum * M_{c-1} + S) is replaced by
 *     muon_scale * NS5(S),
 * NS5 being the quintic Newton-Schulz iteration of the Muon optimizer (K. Jordan et al.,
 * 2024): X = S / (||S||_F + 1e-7), taken transposed when it has more rows than columns (W2),
 * then five times X <- 3.4445 X + (-4.7750 A + 2.0315 A A) X with A = X X^T, transposed back;
 * then W <- colnorm(W + muon_scale * NS5(S)).  The orthogonalised step has singular values
 * near 1 whatever the rates, so muon_scale is its size (the pages fix none).
 *   M0, momentum, M_out  as ttt_la_forward_momentum; M_out may be NULL only when
 *              momentum = 0 and M0 = NULL (no buffer; ERR_NULL otherwise)
 *   muon_scale finite (ERR_SHAPE otherwise)
 *   workspace  at least ttt_la_muon_workspace_bytes(desc, chunk, mode) bytes: ttt_la_forward's
 *              plus 3.3 MB per head for the iteration's exchange between the workgroups of a head
 * Other arguments, checks and status codes as ttt_la_forward; ERR_UNSUPPORTED for the other
 * modes.
 */
int ttt_la_forward_muon(const void* Q, const void* K, const void* V, const float* eta,
                        const float* W0, const float* M0, float momentum, float muon_scale,
                        int64_t chunk, int32_t mode, const ttt_la_desc* desc, void* O,
                        float* W_out, float* M_out, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Bytes of device workspace ttt_la_forward_muon needs (0 for invalid or unsupported
 * arguments). */
size_t ttt_la_muon_workspace_bytes(const ttt_la_desc* desc, int64_t chunk, int32_t mode);

/* Timing events for ttt_la_forward_timed and for timing calls on a stream.
 * ttt_la_event_create makes a hipEvent_t (returned through *event) that
 * records a timestamp without the system-scope memory fence an ordinary
 * event performs (that fence writes back and invalidates caches, which costs
 * several microseconds between two kernels and perturbs the work after it).
 * Such an event only serves timing: wait for the stream (or a fenced event)
 * before reading it with ttt_la_event_elapsed_ms.
 *   ttt_la_event_create     event != NULL; TTT_LA_ERR_NULL otherwise,
 *                           TTT_LA_ERR_HIP if HIP fails.  The caller owns
 *                           the event and frees it with ttt_la_event_destroy.
 *   ttt_la_event_record     records `event` on `stream` (hipStream_t, NULL =
 *                           the null stream).
 *   ttt_la_event_elapsed_ms *ms = time from `start` to `stop` in
 *                           milliseconds; both must have completed.
 *   ttt_la_event_destroy    frees an event from ttt_la_event_create (NULL
 *                           is ignored). */
int ttt_la_event_create(void** event);
int ttt_la_event_record(void* event, void* stream);
int ttt_la_event_elapsed_ms(void* start, void* stop, float* ms);
int ttt_la_event_destroy(void* event);

/*
 * ttt_la_backward(Q, K, V, eta, W0, dO, dW_out, chunk, mode) -> (dQ, dK, dV, deta, dW0)
 *
 * Gradients of a scalar loss through ttt_la_forward in every mode that
 * trains the memory, for training the model around the layer (the paper
 * summary reports the parallel form's speed-up for training as well as
 * inference, technical section 4; the LaCT review, language section, reports
 * training throughput).
 *   Per-token: with G_t = dW_out + sum of q_j^T dO_j over the reads j at or
 *   after token t (strictly after it for TTT_LA_PER_TOKEN_LINEAR_EXCLUSIVE),
 *   and S_t the memory token t's query reads:
 *     dq_t = dO_t S_t^T,   dk_t = eta_t v_t G_t^T,   dv_t = eta_t k_t G_t,
 *     deta_t = k_t G_t v_t^T,   dW0 = dW_out + sum_t q_t^T dO_t.
 *   Large-chunk linear: chunk c forms P_c = W_{c-1} + K_c^T diag(eta_c) V_c
 *   and W_c = P_c / n_c per column; its queries read R_c (W_{c-1}, or W_c
 *   for TTT_LA_LARGE_CHUNK_LINEAR_UPDATE_FIRST).  From the last chunk back,
 *   with G = dW_out at the end and A_c = Q_c^T dO_c: (update-first) G += A_c;
 *   dP_c = (G - w (w . G)) / n_c per column (G / 1e-12 when the norm is at
 *   the floor); G = dP_c; (read-first) G += A_c.  Then dQ_c = dO_c R_c^T,
 *   dK_c = diag(eta) V_c dP_c^T, dV_c = diag(eta) K_c dP_c,
 *   deta_t = k_t dP_c v_t^T, and dW0 = G.
 *   SwiGLU (LaCT review, non-linear-memory and read-order sections): chunk c
 *   forms U_c = W_{c-1} + S(W_{c-1}), S the eta-weighted descent step of the
 *   binding loss, and W_c = U_c normalised per column (W1, W3 over d, W2 over
 *   d_h); from the last chunk back the read's gradient enters G before
 *   (update-first) or after (read-first) the chunk's step, the normalisation's
 *   backward is (G - w (w . G)) / n per column, and the step's vector-Jacobian
 *   product (through the gradient of the binding loss, so with silu's second
 *   derivative) gives dK, dV, deta of the chunk and the weight term added to
 *   the previous weights' gradient.  TTT_LA_LARGE_CHUNK_SWIGLU_LAST_LAYER has
 *   no normalisation and no W1 / W3 step.  dW0 = G at the start.
 *
 *   Q, K, V, eta, W0, chunk, desc   as passed to ttt_la_forward (the forward
 *                  outputs are not needed: the memories are recomputed)
 *   mode           any mode of ttt_la_forward: TTT_LA_PER_TOKEN_LINEAR,
 *                  TTT_LA_PER_TOKEN_LINEAR_EXCLUSIVE, TTT_LA_LARGE_CHUNK_LINEAR,
 *                  TTT_LA_LARGE_CHUNK_LINEAR_UPDATE_FIRST, TTT_LA_LARGE_CHUNK_SWIGLU,
 *                  TTT_LA_LARGE_CHUNK_SWIGLU_UPDATE_FIRST, TTT_LA_LARGE_CHUNK_SWIGLU_LAST_LAYER
 *   dO             [B,H,T,d_v] io_dtype, device: gradient of O
 *   dW_out         float32, device, W_out's shape ([B,H,d_k,d_v], or the packed
 *                  W1 | W3 | W2 per head in the SwiGLU modes): gradient of W_out
 *                  (pass zeros if the final memory does not reach the loss)
 *   dQ, dK         [B,H,T,d_k] float32, device (written)
 *   dV             [B,H,T,d_v] float32, device (written)
 *                  (float32 whatever io_dtype is: rounding these heavy-tailed
 *                  gradients to bf16 alone would use up the accuracy budget)
 *   deta           [B,H,T] float32, device (written)
 *   dW0            float32, device, W0's shape (written)
 *   workspace, workspace_bytes
 *                  at least ttt_la_backward_workspace_bytes(desc, chunk, mode)
 *                  bytes of device scratch (contents on entry do not matter)
 *   stream         hipStream_t (NULL = the default stream)
 *
 * Supported set: per-token as ttt_la_forward (bf16 or fp32, d_k = d_v in
 * {64, 128}); large-chunk linear bf16, d_k = d_v in {64, 128}, any chunk;
 * SwiGLU bf16, d = 128, d_h = 256, any chunk, o_dtype TTT_LA_O_AS_INPUT.
 * dO has io_dtype.
 * Every pointer is required (ERR_NULL), except that the per-token arrays
 * may be NULL when T = 0 (then dW0 = dW_out); no output may overlap an input,
 * another output or the workspace (ERR_ALIAS).  Checks, ownership and
 * enqueue-only behaviour are those of ttt_la_forward.
 */
int ttt_la_backward(const void* Q, const void* K, const void* V, const float* eta,
                    const float* W0, const void* dO, const float* dW_out, int64_t chunk,
                    int32_t mode, const ttt_la_desc* desc, void* dQ, void* dK, void* dV,
                    float* deta, float* dW0, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * ttt_la_forward_noalloc: ttt_la_forward for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results, checks and
 * status codes as ttt_la_forward, without the workspace: the call uses a
 * device scratch array of TTT_LA_NOALLOC_SCRATCH_BYTES that the library
 * holds itself (one per GPU, in the library's code object, from the first
 * use on that GPU until the process ends; its address is looked up on the
 * calling thread's current device, which must be the device of `stream`).
 * The call allocates and frees nothing.
 *   TTT_LA_ERR_SCRATCH  the problem needs more than TTT_LA_NOALLOC_SCRATCH_BYTES
 *                       of workspace (ttt_la_workspace_bytes); nothing is enqueued
 *   TTT_LA_ERR_HIP      the scratch address could not be obtained
 * Every call on a GPU shares that GPU's scratch: calls that may overlap in
 * time on one GPU (on different streams, or from several host threads)
 * race on it and must be ordered by the caller.  Whatever the kernels need
 * zeroed is cleared by the call itself, on `stream`.
 */
#define TTT_LA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int ttt_la_forward_noalloc(const void* Q, const void* K, const void* V, const float* eta,
                           const float* W0, int64_t chunk, int32_t mode, const ttt_la_desc* desc,
                           void* O, float* W_out, void* stream);

/* Bytes of device workspace ttt_la_backward needs (0 for invalid or
 * unsupported arguments). */
size_t ttt_la_backward_workspace_bytes(const ttt_la_desc* desc, int64_t chunk, int32_t mode);

/* Bytes of device workspace ttt_la_forward needs for this problem (0 if
 * none).  Returns 0 as well for invalid arguments (ttt_la_forward reports
 * those). */
size_t ttt_la_workspace_bytes(const ttt_la_desc* desc, int64_t chunk, int32_t mode);

/* Static, NUL-terminated description of a status code. */
const char* ttt_la_status_string(int status);

/* ABI version of this header (incremented on incompatible change). */
int ttt_la_abi_version(void);

#define TTT_LA_ABI_VERSION 7

#ifdef __cplusplus
}
#endif

#endif /* TTT_LA_H */
