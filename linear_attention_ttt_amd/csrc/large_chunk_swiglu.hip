// LaCT large-chunk TTT with a SwiGLU fast-weight MLP (LaCT review "Test-Time
// Training Done Right": the usual memory is a SwiGLU MLP with three
// matrices; the chunk's gradients of the negative inner-product loss are
// summed with per-token rates; the weights are L2-normalised after the
// update; a chunk reads the memory of earlier chunks, then updates it):
//     f_W(x) = (silu(x W1) * (x W3)) W2
//     O_c    = f_{W_{c-1}}(Q_c)
//     W_c    = normalise(W_{c-1} - grad_W sum_{i in c} eta_i (-<f_W(k_i), v_i>))
// With G = diag(eta) V, A = K W1, B = K W3, H = silu(A) * B, the descent
// step is  dW2 = H^T G,  dH = G W2^T,  dW1 = K^T (dH * B * silu'(A)),
// dW3 = K^T (dH * silu(A)); columns of W1, W3 (over d) and of W2 (over
// d_h) are then divided by max(norm, 1e-12).
//
// Two kernels:
//  * swiglu_recur_kernel (sequential over chunks; every workgroup of a
//    launch resident at once, see launch_large_chunk_swiglu): a head's
//    hidden units are split into NSL slices of NS units, one workgroup per
//    slice.  With that split dW1[:, s], dW3[:, s], dW2[s, :] and the W1/W3
//    normalisation are local to the slice; only the W2 column norms need a
//    128-float sum across the head's workgroups, exchanged through global
//    memory with a counter (device-scope atomics).  Within a workgroup each wave
//    streams its own 32-token groups of the chunk (private LDS ring, no
//    barriers) and keeps its partial gradients in registers; the waves'
//    partials are added at the chunk end.  Each workgroup stores the
//    weights every chunk reads (bf16 hi + lo planes, transposed for the
//    read kernel's operands).
//  * swiglu_read_kernel (fully parallel): O_c = f_{W_{c-1}}(Q_c) for every
//    (head, chunk, 128-token tile), hidden units in 32-unit slices staged
//    through LDS; products use the bf16 hi + lo split of the weights and of
//    H so the only visible rounding is that of the bf16 output.
#include <algorithm>
#include <cstdlib>

#include "device_common.h"
#include "kernels.h"

namespace ttt {

namespace {

constexpr int SW_D = 128;
constexpr int SW_DH = 256;
constexpr int SW_NS = 16;                 // hidden units per recurrence workgroup
constexpr int SW_NSL = SW_DH / SW_NS;     // workgroups per head
constexpr int SW_TT = 256;                // tokens per read workgroup (4 waves x 64)
constexpr int SW_US = 32;                 // hidden units per read slice
constexpr int SW_SPIN_LIMIT = 1 << 24;
constexpr size_t SW_STATE = (size_t)6 * SW_D * SW_DH;  // bf16 elements per stored state

// Recurrence: each wave streams its own 32-token groups of the chunk through
// a private 2-stage LDS ring and keeps its partial chunk gradients in
// registers; the 4 waves' partials are added at the chunk end.
constexpr int SW_WAVES = 4;
constexpr int SW_GT = 32;                 // tokens per wave step
constexpr int SW_KROW = SW_D * 2;         // bf16 row of K / V in LDS (swizzled 16-byte pieces)
constexpr int SW_STAGE = SW_GT * SW_KROW; // one matrix of one stage
constexpr int SW_LOADS = 2 * SW_STAGE / 1024 + 1;   // direct-to-LDS loads per wave per stage: K, V, eta

struct RecurLds {
  unsigned char kv[SW_WAVES][2][2][SW_STAGE];   // [wave][stage][K, V]
  float eta[SW_WAVES][2][64];               // one value per lane copied; the first SW_GT are the stage's
  float w1[SW_D * SW_NS];   // W1[d][u] at w13i(d, u)
  float w3[SW_D * SW_NS];   // W3[d][u] at w13i(d, u)
  float w2[SW_NS * SW_D];   // W2[u][d] at w2i(u, d)
};
static_assert(sizeof(RecurLds) <= 160 * 1024, "recurrence LDS exceeds 160 KB");

// Position of the 16-byte piece of a 256-byte K/V row in LDS: piece c of row
// r sits at c ^ sw_swz(r & 15), a map chosen by measuring LDS throughput on
// gfx950: the row-wise 16-byte operand reads (16 rows, one piece) and the
// transposed 8-byte reads (4 rows x 32 bytes per 16 lanes) are both free of
// bank conflicts.
__device__ __forceinline__ int sw_swz(int row) { return (int)((0x159DAE2673FBC840ull >> (4 * (row & 15))) & 15); }
// The slice's fp32 weights in LDS are kept in the MFMA accumulator order of
// the gradients, so a wave adds its partial chunk gradient with one 16-byte
// read-modify-write per 4 values: W1[d][u], W3[d][u] at ((d/4)*16 + u)*4 + d%4
// and W2[u][d] at (((d/16)*4 + u/4)*16 + d%16)*4 + u%4.
__device__ __forceinline__ int w13i(int d, int u) { return ((d >> 2) * 16 + u) * 4 + (d & 3); }
__device__ __forceinline__ int w2i(int u, int d) { return (((d >> 4) * 4 + (u >> 2)) * 16 + (d & 15)) * 4 + (u & 3); }

// One matrix of a recurrence stage: 8 direct-to-LDS loads of 16 bytes per lane, load j into LDS
// lds + 1024 j + 16 lane.  The loads keep the ordinary cache policy: every slice workgroup of a head reads
// the same K and V rows, so the lines should stay in L2 for the others (measured: ~1.5 % faster than
// non-temporal loads).  The instruction offset (1024 (j % 4)) is added to both the global and the LDS
// address, so four loads share one M0 and off[j] is the global offset less it.  Written as one asm statement
// (M0 set twice instead of per load); the compiler does not see these loads, so the caller counts them in
// its vmcnt waits, as with dma16.
__device__ __forceinline__ void stage_dma(__amdgpu_buffer_rsrc_t r, const unsigned (&off)[8], const void* lds) {
  unsigned saved;
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds);
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %4, %1, 0 offen lds\n\t"
      "buffer_load_dwordx4 %5, %1, 0 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %6, %1, 0 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %7, %1, 0 offen offset:3072 lds\n\t"
      "s_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %8, %1, 0 offen lds\n\t"
      "buffer_load_dwordx4 %9, %1, 0 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %10, %1, 0 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %11, %1, 0 offen offset:3072 lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(r), "s"(base), "s"(base + 4096u), "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "v"(off[4]),
        "v"(off[5]), "v"(off[6]), "v"(off[7]));
}
// logistic function with the hardware reciprocal (about 1 ulp): its value
// only feeds bf16 operands or a bf16 hi + lo pair, so a correctly rounded
// division buys nothing here
__device__ __forceinline__ float sigmoid_fast(float a) { return __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

__device__ __forceinline__ void split_store8(bf16* hi, bf16* lo, const float* f) {
  bf16x8 h, l;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    h[j] = (bf16)f[j];
    l[j] = (bf16)(f[j] - (float)h[j]);
  }
  *(bf16x8*)hi = h;
  *(bf16x8*)lo = l;
}

__global__ void zero_u32_kernel(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Update rules of the recurrence (compile-time RULE of swiglu_recur_kernel):
//   0  plain descent: W <- W + dW (dW = minus the chunk's eta-weighted gradient);
//   1  momentum: M <- beta M + dW, W <- W + M;
//   2  Muon: the step (dW, or M <- beta M + dW with momentum) is replaced by
//      muon_scale * NS5(step) for each matrix, NS5 the quintic Newton-Schulz
//      iteration of the Muon optimizer (five steps X <- a X + (b A + c A^2) X,
//      A = X X^T, from X = step / (||step||_F + 1e-7); W2's step is taken
//      transposed, so all three are d x d_h).
// The column normalisation follows in every rule.
constexpr float NS_A = 3.4445f, NS_B = -4.7750f, NS_C = 2.0315f, NS_EPS = 1e-7f;
constexpr int NS_STEPS = 5;
struct SwRule {
  const float* M0;   // momentum buffers before the first chunk, state layout (null: zeros)
  float* Mout;       // momentum buffers, updated at every chunk end (null: no momentum)
  float beta;        // momentum coefficient
  float muon_scale;  // scale of the orthogonalised step (RULE 2)
  float* ns;         // RULE 2: per head [NSL][3][d][d] partial Gram matrices, then [3][d][d] their sums
  // DUMP (the backward's recomputation): after chunk c, the float32 weights (packed W1 | W3 | W2) into
  // dump[head][c], and the column norms before the normalisation into dnorm[head][c][W1 256 | W3 256 | W2 128]
  float* dump;
  float* dnorm;
};
constexpr size_t NS_HEAD_FLOATS = (size_t)(SW_NSL + 1) * 3 * SW_D * SW_D;

// Barrier of the NSL workgroups of head bh (their counter; the k-th barrier waits for NSL * k arrivals).
// Bounded: on giving up the call's error flag is raised (the read kernel then fills every output with
// NaN) and the workgroup carries on, so every kernel still ends.  Stores that the other workgroups read
// after it must be complete (wait_vm<0>) before it.
__device__ __forceinline__ void head_barrier_wait(unsigned* counters, unsigned* errflag, int bh, unsigned& nbar,
                                                  int spin_limit, unsigned target_extra) {
  __syncthreads();
  ++nbar;
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(&counters[bh], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned target = (unsigned)SW_NSL * nbar + target_extra;
    int spins = 0;
    while (__hip_atomic_load(&counters[bh], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > spin_limit) {
        __hip_atomic_store(errflag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

// RULE 2 at the end of chunk c: replace the step of the three matrices by muon_scale * NS5(step).  On
// entry S.w* hold W + dW and the LDS of the K/V stages (every copy into it has landed) holds, after
// 3 d NS floats, the weights before the update in the layout of S.w*.  The steps (with momentum:
// M <- beta M + dW, kept in R.Mout) are the columns of three d x d_h matrices X (W2's transposed), split
// by hidden unit over the head's NSL workgroups; the iteration needs A = X X^T = the sum over workgroups
// of X_s X_s^T.  Per step each workgroup writes its three partial Gram matrices, sums 8 rows of each over
// the NSL partials, and after a second barrier reads the full sums back; wave w then updates rows
// 32w .. 32w + 31 of its workgroup's columns, X_s <- a X_s + b A X_s + c A (A X_s) (bf16 hi + lo
// products, float32 accumulation).  The Frobenius normalisation comes from trace(X X^T) of the first
// step.  LDS of the stages: X [3][d][NS] float32, Y [3][d][NS] (A X), then wave w's rows of A as bf16
// [hi, lo][32][d].  Kept out of line: its registers are not the recurrence's.
__device__ __attribute__((noinline)) void swiglu_muon_steps(RecurLds& S, const SwRule& R, int bh, int sl, int u0,
                                                           int c, unsigned* counters, unsigned* errflag,
                                                           unsigned& nbar, int spin_limit, unsigned target_extra) {
  constexpr int D = SW_D, DH = SW_DH, NS = SW_NS, G = D * D, NT = SW_WAVES * 64;
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto head_barrier = [&]() { head_barrier_wait(counters, errflag, bh, nbar, spin_limit, target_extra); };
  float* X = (float*)&S.kv[0][0][0][0];
  float* Y = X + 3 * D * NS;
  unsigned char* Aw = (unsigned char*)(Y + 3 * D * NS) + w * (2 * 32 * D * 2);
  const bool mom = R.Mout != nullptr;
  const float* Msrc = c == 0 ? R.M0 : R.Mout;
  const float* Mi = mom && Msrc ? Msrc + (size_t)bh * 3 * D * DH : nullptr;
  float* Mh = mom ? R.Mout + (size_t)bh * 3 * D * DH : nullptr;
  for (int k = 0; k < 8; ++k) {
    const int i = tid + NT * k, d = i >> 4, u = i & 15, u2 = i >> 7, d2 = i & 127;
    const int li3[3] = {w13i(d, u), w13i(d, u), w2i(u2, d2)};
    float* e[3] = {S.w1 + li3[0], S.w3 + li3[1], S.w2 + li3[2]};
    const size_t go[3] = {(size_t)d * DH + u0 + u, (size_t)D * DH + (size_t)d * DH + u0 + u,
                          2 * (size_t)D * DH + (size_t)(u0 + u2) * D + d2};
    const int xi[3] = {d * NS + u, D * NS + d * NS + u, 2 * D * NS + d2 * NS + u2};
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const float before = Y[j * D * NS + li3[j]];
      const float m = Mi ? __hip_atomic_load(Mi + go[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.f;
      const float st = (*e[j] - before) + (mom ? R.beta * m : 0.f);
      if (mom) __hip_atomic_store(Mh + go[j], st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *e[j] = before;
      X[xi[j]] = st;
    }
  }
  if (mom) wait_vm<0>();
  __syncthreads();
  float* nsh = R.ns + (size_t)bh * NS_HEAD_FLOATS;   // [NSL][3][d][d] partials, then [3][d][d] sums
  const __amdgpu_buffer_rsrc_t rn = make_rsrc(nsh, (long long)NS_HEAD_FLOATS * 4);
  constexpr unsigned SUMS = (unsigned)SW_NSL * 3 * G;   // float offset of the sums
  float f[3] = {1.f, 1.f, 1.f};
  for (int it = 0; it < NS_STEPS; ++it) {
    // this workgroup's partial Gram matrices G = X_s X_s^T; wave w: row tiles 2w, 2w+1 (stored
    // transposed: G is symmetric up to rounding)
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      const float* Xm = X + m * D * NS;
      bf16x4 ah[2], al[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const floatx4 x = *(const floatx4*)(Xm + (16 * (2 * w + tt) + li) * NS + 4 * g);
        const uint2 s0 = split2(x[0], x[1]), s1 = split2(x[2], x[3]);
        ah[tt] = __builtin_bit_cast(bf16x4, uint2{s0.x, s1.x});
        al[tt] = __builtin_bit_cast(bf16x4, uint2{s0.y, s1.y});
      }
#pragma unroll
      for (int tj = 0; tj < 8; ++tj) {
        const floatx4 x = *(const floatx4*)(Xm + (16 * tj + li) * NS + 4 * g);
        const uint2 s0 = split2(x[0], x[1]), s1 = split2(x[2], x[3]);
        const bf16x4 bh = __builtin_bit_cast(bf16x4, uint2{s0.x, s1.x});
        const bf16x4 bl = __builtin_bit_cast(bf16x4, uint2{s0.y, s1.y});
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          acc = mfma16k16(ah[tt], bh, acc);
          acc = mfma16k16(ah[tt], bl, acc);
          acc = mfma16k16(al[tt], bh, acc);
          const unsigned off = ((((unsigned)sl * 3 + m) * D + 16 * tj + li) * D + 16 * (2 * w + tt) + 4 * g) * 4;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), rn, off, 0, 16);
        }
      }
    }
    wait_vm<0>();
    head_barrier();
    // rows 8 sl .. 8 sl + 7 of the three sums, over the NSL partials in a fixed order (three 16-byte pieces
    // per thread; the partials' loads are issued in groups of 8 so that they are in flight together)
    {
      constexpr int RS = 3 * 8 * (D / 4) / NT;
      static_assert(RS * NT == 3 * 8 * (D / 4), "reduce-scatter items per thread");
      floatx4 acc[RS];
      unsigned src[RS], dst[RS];
#pragma unroll
      for (int k = 0; k < RS; ++k) {
        const int q = tid + NT * k;
        const int m = q / (8 * (D / 4)), row = 8 * sl + (q / (D / 4)) % 8, c4 = q % (D / 4);
        acc[k] = floatx4{0.f, 0.f, 0.f, 0.f};
        src[k] = (((unsigned)m * D + row) * D + 4 * c4) * 4;
        dst[k] = (SUMS + ((unsigned)m * D + row) * D + 4 * c4) * 4;
      }
#pragma unroll
      for (int s0 = 0; s0 < SW_NSL; s0 += 8) {
        floatx4 v[8][RS];
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int k = 0; k < RS; ++k)
            v[j][k] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rn, src[k] + (unsigned)(s0 + j) * 3 * G * 4, 0, 16));
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int k = 0; k < RS; ++k) acc[k] += v[j][k];
      }
#pragma unroll
      for (int k = 0; k < RS; ++k)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[k]), rn, dst[k], 0, 16);
    }
    wait_vm<0>();
    head_barrier();
#pragma unroll 1
    for (int m = 0; m < 3; ++m) {
      float* Xm = X + m * D * NS;
      float* Ym = Y + m * D * NS;
      const unsigned abase = SUMS + (unsigned)m * G;
      if (it == 0) {   // 1 / (||X||_F + eps), with ||X||_F^2 = trace(X X^T)
        const float t = __hip_atomic_load(nsh + abase + l * (D + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) +
                        __hip_atomic_load(nsh + abase + (l + 64) * (D + 1), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        f[m] = 1.0f / (sqrtf(wave_sum(t)) + NS_EPS);
      }
      const float fx = it == 0 ? f[m] : 1.f, f2 = fx * fx;   // A of the normalised X is f^2 A
      // this wave's rows 32w .. 32w + 31 of f^2 A as bf16 hi + lo, 16-byte pieces swizzled by row
      {
        constexpr int AG = 32 * (D / 4) / 64;   // 16-byte pieces per lane, loaded together
        floatx4 av[AG];
#pragma unroll
        for (int k = 0; k < AG; ++k) {
          const int q = l + 64 * k, row = q / (D / 4), c4 = q % (D / 4);
          av[k] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rn, (abase + (32u * w + row) * D + 4 * c4) * 4, 0, 16));
        }
#pragma unroll
        for (int k = 0; k < AG; ++k) {
          const int q = l + 64 * k, row = q / (D / 4), c4 = q % (D / 4);
          const floatx4 a = f2 * av[k];
          const uint2 s0 = split2(a[0], a[1]), s1 = split2(a[2], a[3]);
          const int off = row * (2 * D) + (((c4 >> 1) ^ (row & 15)) << 4) + (c4 & 1) * 8;
          *(uint2*)(Aw + off) = uint2{s0.x, s1.x};
          *(uint2*)(Aw + 32 * D * 2 + off) = uint2{s0.y, s1.y};
        }
      }
      // P = A' B for B = X or Y (d x NS in LDS): rows 32w + 16tt + 4g + r, column li of the lane
      auto prod = [&](const float* Bm, floatx4 (&acc)[2]) {
        acc[0] = acc[1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          floatx4 b0, b1;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            b0[j] = Bm[(32 * ks + 8 * g + j) * NS + li];
            b1[j] = Bm[(32 * ks + 8 * g + 4 + j) * NS + li];
          }
          bf16x8 bh, bl;
          split8(b0, b1, bh, bl);
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int row = 16 * tt + li, off = row * (2 * D) + (((4 * ks + g) ^ (row & 15)) << 4);
            const bf16x8 ah = *(const bf16x8*)(Aw + off), al = *(const bf16x8*)(Aw + 32 * D * 2 + off);
            acc[tt] = mfma16(ah, bh, acc[tt]);
            acc[tt] = mfma16(ah, bl, acc[tt]);
            acc[tt] = mfma16(al, bh, acc[tt]);
          }
        }
      };
      floatx4 y[2], z[2];
      prod(Xm, y);                    // A' X; A' (f X) = f A' X
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          y[tt][r] *= fx;
          Ym[(32 * w + 16 * tt + 4 * g + r) * NS + li] = y[tt][r];
        }
      __syncthreads();                // every row of A' X is in LDS; every wave is done reading X
      prod(Ym, z);                    // A' (A' X)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* xp = Xm + (32 * w + 16 * tt + 4 * g + r) * NS + li;
          *xp = NS_A * fx * *xp + NS_B * y[tt][r] + NS_C * z[tt][r];
        }
    }
    __syncthreads();                  // every row of the new X before its next use
  }
  // W <- W + muon_scale * NS5(step) (W was put back to its value before the update above)
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int i = tid + NT * k, d = i >> 4, u = i & 15, u2 = i >> 7, d2 = i & 127;
    S.w1[w13i(d, u)] += R.muon_scale * X[d * NS + u];
    S.w3[w13i(d, u)] += R.muon_scale * X[D * NS + d * NS + u];
    S.w2[w2i(u2, d2)] += R.muon_scale * X[2 * D * NS + d2 * NS + u2];
  }
  __syncthreads();
}

template <int RULE, bool DUMP = false>
__global__ __launch_bounds__(SW_WAVES * 64, 1) void swiglu_recur_kernel(
    const bf16* __restrict__ K, const bf16* __restrict__ V, const float* __restrict__ eta,
    const float* __restrict__ W0, float* __restrict__ Wout, bf16* __restrict__ states,
    unsigned long long* __restrict__ ss2,
    unsigned* __restrict__ counters, unsigned* __restrict__ errflag, int T_in, int chunk, int nchunks_in, int head0,
    int update_first, int last_only, int par_nchunks, int spin_limit, unsigned target_extra, SwRule R) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  RecurLds& S = *reinterpret_cast<RecurLds*>(smem_raw);
  constexpr int NT = SW_WAVES * 64;
  const int nblocks = gridDim.x;
  const int logical = (nblocks % 8 == 0) ? xcd_logical_block(blockIdx.x, nblocks) : blockIdx.x;
  // par_nchunks > 0 (only with last_only): the chunks are independent, since the W2 gradient does not
  // depend on W2 and W1, W3 stay fixed.  Workgroup (head, chunk, slice) then computes that chunk's W2
  // update alone, as a one-chunk sequence starting from W2 = 0, and writes it instead of the weights.
  const int par = par_nchunks > 0;
  const int bhc = logical / SW_NSL;
  const int bh = par ? bhc / par_nchunks : head0 + bhc;
  const int cpar = par ? bhc % par_nchunks : 0;
  const int sl = logical % SW_NSL;
  const int T = par ? min(chunk, T_in - cpar * chunk) : T_in;
  const int nchunks = par ? 1 : nchunks_in;
  const int u0 = sl * SW_NS;
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int D = SW_D, DH = SW_DH, NS = SW_NS;

  const size_t tok0 = (size_t)bh * T_in + (size_t)cpar * chunk;
  const bf16* Kh = K + tok0 * D;
  const bf16* Vh = V + tok0 * D;
  const float* Eh = eta + tok0;
  const float* W0h = W0 + (size_t)bh * 3 * D * DH;
  bf16* St = states + (size_t)bh * nchunks * SW_STATE;

  // ---- load this slice of the initial weights ----
  for (int i = tid; i < D * NS; i += NT) {
    const int d = i / NS, u = i % NS;
    S.w1[w13i(d, u)] = W0h[(size_t)d * DH + u0 + u];
    S.w3[w13i(d, u)] = W0h[(size_t)D * DH + (size_t)d * DH + u0 + u];
  }
  for (int i = tid; i < NS * D; i += NT) {
    const int u = i / D, d = i % D;
    S.w2[w2i(u, d)] = par ? 0.f : W0h[(size_t)2 * D * DH + (size_t)(u0 + u) * D + d];
  }
  __syncthreads();

  // the weights chunk `slot` reads: W1^T, W3^T [DH][D] and W2^T [D][DH], bf16 hi + lo
  auto store_state = [&](int slot) {
    if (tid >= 256) return;
    bf16* base = St + (size_t)slot * SW_STATE;
    const size_t P = (size_t)D * DH;
    {
      const int idx = tid * 8;               // 8 consecutive d of one unit
      const int u = idx / D, d = idx % D;
      float f1[8], f3[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        f1[j] = S.w1[w13i(d + j, u)];
        f3[j] = S.w3[w13i(d + j, u)];
      }
      const size_t o = (size_t)(u0 + u) * D + d;
      split_store8(base + o, base + P + o, f1);
      split_store8(base + 2 * P + o, base + 3 * P + o, f3);
    }
    {
      const int idx = tid * 8;               // 8 consecutive units of one output dim
      const int n = idx / NS, u = idx % NS;
      float f2[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) f2[j] = S.w2[w2i(u + j, n)];
      const size_t o = (size_t)n * DH + u0 + u;
      split_store8(base + 4 * P + o, base + 5 * P + o, f2);
    }
  };
  // state slot c holds the weights chunk c reads: W_{c-1} (W0 for chunk 0), or W_c when a chunk updates first
  if (nchunks > 0 && !update_first && !par) store_state(0);

  // ---- this wave's 32-token groups: in chunk c, groups w + 4k for k < count(c) ----
  // All slices of a head walk a chunk in the same order, so they request the
  // same lines at about the same time (measured on gfx950: faster than
  // spreading the slices over the chunk, which raises L2 misses).
  auto count = [&](int c) {
    const int ng = (min(c * chunk + chunk, T) - c * chunk + SW_GT - 1) / SW_GT;
    return ng > w ? (ng - w + SW_WAVES - 1) / SW_WAVES : 0;
  };
  // next step of this wave (c == nchunks: none left); kn caches count(c)
  auto advance = [&](int& c, int& k, int& kn) {
    ++k;
    while (c < nchunks && k >= kn) {
      ++c;
      k = 0;
      kn = c < nchunks ? count(c) : 0;
    }
  };
  auto group_of = [&](int c, int k) {
    (void)c;
    return w + SW_WAVES * k;
  };
  // per-lane byte offsets: direct-to-LDS rows (4 per load), row-wise operand reads (row 16tt + li,
  // piece 4ks + g) and transposed reads (rows 16tt + 4g .. + 3, columns 16m + li)
  // (load j of a stage: LDS bytes 1024 j + 16 lane; the instruction offset 1024 (j % 4) applies to both the
  // global and the LDS address, so four loads share one LDS base and dma_off[j] is the global offset less it)
  unsigned dma_off[SW_STAGE / 1024];
#pragma unroll
  for (int j = 0; j < SW_STAGE / 1024; ++j) {
    const int row = 4 * j + (l >> 4);
    dma_off[j] = (unsigned)(row * SW_KROW + (((l & 15) ^ sw_swz(row)) << 4) - 1024 * (j & 3));
  }
  unsigned fwd_off[4], tr_off[8];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) fwd_off[ks] = (unsigned)(li * SW_KROW + (((4 * ks + g) ^ sw_swz(li)) << 4));
  const int trow = 4 * g + (li >> 2);
#pragma unroll
  for (int m = 0; m < 8; ++m)
    tr_off[m] = (unsigned)(trow * SW_KROW + (((2 * m + ((li >> 1) & 1)) ^ sw_swz(trow)) << 4) + (li & 1) * 8);

  int last_c = -1, last_gi = 0, last_slot = 0;   // the latest stage issued (RULE 2 re-issues it)
  auto issue = [&](int c, int gi, int slot) {
    last_c = c;
    last_gi = gi;
    last_slot = slot;
    const int t0 = c * chunk + gi * SW_GT;
    const int n = min(c * chunk + chunk, T) - t0;   // valid tokens; rows beyond read as 0
    // (1 <= n <= SW_GT: the sizes need no clamping)
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(Kh + (size_t)t0 * D), (short)0,
                                                                        n * SW_KROW, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(Vh + (size_t)t0 * D), (short)0,
                                                                        n * SW_KROW, 0x00020000);
    const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc((void*)(Eh + t0), (short)0, n * 4, 0x00020000);
    stage_dma(rk, dma_off, S.kv[w][slot][0]);
    stage_dma(rv, dma_off, S.kv[w][slot][1]);
    dma4<true>(re, (unsigned)(l * 4), S.eta[w][slot]);    // lanes past the group read 0
  };

  unsigned nbar = 0;   // head barriers passed (the Newton-Schulz exchange's, RULE 2; see head_barrier_wait)

  // RULE 2 at a chunk end (see swiglu_muon_steps); the stage whose copy was in flight when the iteration
  // took the LDS of the stages is copied again afterwards
  auto muon_phase = [&](int c) {
    swiglu_muon_steps(S, R, bh, sl, u0, c, counters, errflag, nbar, spin_limit, target_extra);
    if (last_c > c) issue(last_c, last_gi, last_slot);
  };

  // Momentum (RULE 1): weight k (0..7) of matrix j (W1, W3, W2) kept by this thread (the mapping is given
  // at the chunk end): its place in the LDS copy and its float offset in the head's buffer [W1 | W3 | W2]
  auto mom_elem = [&](int k, int j) -> float* {
    const int i = tid + NT * k;
    return j == 0 ? S.w1 + w13i(i >> 4, i & 15) : j == 1 ? S.w3 + w13i(i >> 4, i & 15) : S.w2 + w2i(i >> 7, i & 127);
  };
  auto mom_off = [&](int k, int j) -> size_t {
    const int i = tid + NT * k;
    return j < 2 ? (size_t)j * D * DH + (size_t)(i >> 4) * DH + u0 + (i & 15)
                 : 2 * (size_t)D * DH + (size_t)(u0 + (i >> 7)) * D + (i & 127);
  };

  bf16x8 w1op[4], w3op[4], w2op[4];
  floatx4 dW1[8], dW3[8], dW2[8];
  int ic = 0, ik = -1, ikn = nchunks > 0 ? count(0) : 0;   // issue cursor: chunk, step within it, count
  advance(ic, ik, ikn);
  int cc = ic, ck = ik, ckn = ikn;           // compute cursor
  int step = 0;
  if (ic < nchunks) {
    issue(ic, group_of(ic, ik), 0);
    advance(ic, ik, ikn);
  }

  for (int c = 0; c < nchunks; ++c) {
    // operands of this chunk's weights (B operands: col = unit li, k = 8 consecutive d)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = 32 * ks + 8 * g + j;
        w1op[ks][j] = (bf16)S.w1[w13i(d, li)];
        w3op[ks][j] = (bf16)S.w3[w13i(d, li)];
        w2op[ks][j] = (bf16)S.w2[w2i(li, d)];
      }
#pragma unroll
    for (int m = 0; m < 8; ++m) dW1[m] = dW3[m] = dW2[m] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (; cc == c; advance(cc, ck, ckn), ++step) {
      const int slot = step & 1;
      // the next stage goes into the one read during the previous step; this step's stage has
      // landed once only the next stage's loads are outstanding
      if (ic < nchunks) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue(ic, group_of(ic, ik), slot ^ 1);
        advance(ic, ik, ikn);
        wait_vm<SW_LOADS>();
      } else {
        wait_vm<0>();
      }
      // K of the stage at kb, V at kb + SW_STAGE; each lane's offset is added first so that the
      // constant parts (V, token tile) become instruction offsets
      const unsigned char* kb = S.kv[w][slot][0];

      // ---- forward of the 32 tokens: A = K W1, B = K W3, Dh = V W2^T (rows: tokens 16tt + 4g + r) ----
      floatx4 A[2], Bv[2], Dh[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) A[tt] = Bv[tt] = Dh[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
      bf16x8 kop[4][2], vop[4][2];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          kop[ks][tt] = *(const bf16x8*)(kb + fwd_off[ks] + tt * 16 * SW_KROW);
          vop[ks][tt] = *(const bf16x8*)(kb + fwd_off[ks] + SW_STAGE + tt * 16 * SW_KROW);
        }
      // transposed operands of the gradient products (k slot (g, j) = token 16(j/4) + 4g + j%4),
      // read while the forward products run
      bf16x4 ktr[8][2], vtr[8][2];
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          ktr[m][tt] = lds_read_tr16(kb + tr_off[m] + tt * 16 * SW_KROW);
          vtr[m][tt] = lds_read_tr16(kb + tr_off[m] + SW_STAGE + tt * 16 * SW_KROW);
        }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          A[tt] = mfma16(kop[ks][tt], w1op[ks], A[tt]);
          Bv[tt] = mfma16(kop[ks][tt], w3op[ks], Bv[tt]);
          Dh[tt] = mfma16(vop[ks][tt], w2op[ks], Dh[tt]);
        }
      // ---- elementwise: the operands of the gradient products ----
      bf16x8 daop, dbop, ehop;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const floatx4 e4 = *(const floatx4*)(&S.eta[w][slot][16 * tt + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = A[tt][r], b = Bv[tt][r];
          const float sg = sigmoid_fast(a);
          const float sa = a * sg;
          const float dh = e4[r] * Dh[tt][r];
          daop[4 * tt + r] = (bf16)(dh * b * sg * (1.0f + a * (1.0f - sg)));
          dbop[4 * tt + r] = (bf16)(dh * sa);
          ehop[4 * tt + r] = (bf16)(e4[r] * sa * b);
        }
      }
      // ---- partial chunk gradients over the 32 tokens ----
      // dW1[d][u] += K^T da, dW3[d][u] += K^T db, dW2[u][d] += eh^T V
      if (!last_only) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const bf16x8 kt = join(ktr[m][0], ktr[m][1]);
          const bf16x8 vt = join(vtr[m][0], vtr[m][1]);
          dW1[m] = mfma16(kt, daop, dW1[m]);
          dW3[m] = mfma16(kt, dbop, dW3[m]);
          dW2[m] = mfma16(ehop, vt, dW2[m]);
        }
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) dW2[m] = mfma16(ehop, join(vtr[m][0], vtr[m][1]), dW2[m]);
      }
    }

    // ---- end of chunk ----
    // Momentum and Muon: each thread keeps 8 weights of each matrix (W1, W3 element (d, u) = (i/16,
    // i%16), W2 element (u, d) = (i/128, i%128), i = tid + 256 k): their values before the update and
    // their momentum buffers (read at device scope: other chunks' values were written by this thread
    // through the L2)
    if constexpr (RULE == 1) {
      // momentum: W + beta M goes into LDS before the partial gradients are added, so the adds leave
      // W + beta M + dW; W itself is parked in M_out, and M <- beta M + dW is their difference after the
      // adds.  The buffers are read at device scope (this thread wrote them through the L2).
      const float* Msrc = c == 0 ? R.M0 : R.Mout;
      const float* Mi = Msrc ? Msrc + (size_t)bh * 3 * D * DH : nullptr;
      float* Mh = R.Mout + (size_t)bh * 3 * D * DH;
      // (the thread's 24 buffer values are loaded 12 at a time: two memory round trips instead of 24;
      // all 24 at once would push the wave past its registers)
#pragma unroll 1
      for (int k0 = 0; k0 < 8; k0 += 4) {
        float mv[4][3];
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int j = 0; j < 3; ++j)
            mv[k][j] = Mi ? __hip_atomic_load(Mi + mom_off(k0 + k, j), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                          : 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int j = 0; j < 3; ++j) {
            float* e = mom_elem(k0 + k, j);
            const float wo = *e;
            __hip_atomic_store(Mh + mom_off(k0 + k, j), wo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *e = wo + R.beta * mv[k][j];
          }
      }
      wait_vm<0>();
      __syncthreads();   // every value moved before any wave adds its partial gradient
    } else if constexpr (RULE == 2) {
      // the weights before the update, copied into the LDS of the K/V stages (the stage in flight is
      // copied again after the Newton-Schulz iteration, which uses that LDS too)
      wait_vm<0>();
      __syncthreads();
      float* Wb = (float*)&S.kv[0][0][0][0] + 3 * D * NS;
      for (int i = tid; i < 3 * D * NS / 4; i += NT)
        ((floatx4*)Wb)[i] = i < D * NS / 4 ? ((const floatx4*)S.w1)[i]
                            : i < 2 * D * NS / 4 ? ((const floatx4*)S.w3)[i - D * NS / 4]
                                                 : ((const floatx4*)S.w2)[i - 2 * D * NS / 4];
      __syncthreads();
    }
    // The waves add their partial gradients in a fixed order, then normalise.
    // dW1 lane layout: [d = 16m + 4g + r][u = li]; dW2: [u = 4g + r][d = 16m + li].  Every weight is
    // updated as (((W + P0) + P1) + P2) + P3 (P_k: wave k's partial), pipelined over quarters of the
    // weights: in pass p wave k adds its partial to quarter p - k (row tiles 2q, 2q+1 of the three
    // matrices), so the 4 adds of a quarter stay in wave order and 7 short passes replace 4 full ones.
#pragma unroll
    for (int p = 0; p < SW_WAVES + 3; ++p) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q != p - w) continue;        // wave-uniform
        floatx4 o1[2], o3[2], o2[2];
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const int f = (((2 * q + mm) * 4 + g) * 16 + li) * 4;   // = w13i(16m + 4g, li) = w2i(4g, 16m + li)
          o1[mm] = *(const floatx4*)(S.w1 + f);
          o3[mm] = *(const floatx4*)(S.w3 + f);
          o2[mm] = *(const floatx4*)(S.w2 + f);
        }
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const int f = (((2 * q + mm) * 4 + g) * 16 + li) * 4;
          if (!last_only) {
            *(floatx4*)(S.w1 + f) = o1[mm] + dW1[2 * q + mm];
            *(floatx4*)(S.w3 + f) = o3[mm] + dW3[2 * q + mm];
          }
          *(floatx4*)(S.w2 + f) = o2[mm] + dW2[2 * q + mm];
        }
      }
      __syncthreads();
    }
    if constexpr (RULE == 1) {
      float* Mh = R.Mout + (size_t)bh * 3 * D * DH;
      // M <- (W + beta M + dW) - W: the parked values loaded 12 at a time, then the differences stored
#pragma unroll 1
      for (int k0 = 0; k0 < 8; k0 += 4) {
        float wv[4][3];
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int j = 0; j < 3; ++j)
            wv[k][j] = __hip_atomic_load(Mh + mom_off(k0 + k, j), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int j = 0; j < 3; ++j)
            __hip_atomic_store(Mh + mom_off(k0 + k, j), *mom_elem(k0 + k, j) - wv[k][j], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      }
      wait_vm<0>();
      __syncthreads();   // every updated weight read before the normalisation rewrites it
    } else if constexpr (RULE == 2) {
      muon_phase(c);
    }
    // W1, W3: unit columns over d, local (waves 0 and 1).  With only the last layer updated there is
    // no normalisation (every slice of a head takes the same branch, so none waits on the exchange).
    if (last_only) {
      // nothing: W1 and W3 stay as they are, W2 is not normalised
    } else if (w < 2) {
      float* Wm = w == 0 ? S.w1 : S.w3;
      const int u = l & 15, r0 = (l >> 4) * 32;
      // rows r0 .. r0+31 of unit u as 8 groups of 4 consecutive rows (16 bytes each in this layout)
      floatx4 x[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = *(const floatx4*)(Wm + w13i(r0 + 4 * k, u));
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j) ss = fmaf(x[k][j], x[k][j], ss);
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      const float inv = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
      if constexpr (DUMP) {
        if (l < 16) R.dnorm[((size_t)bh * nchunks + c) * 640 + w * DH + u0 + u] = sqrtf(ss);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) *(floatx4*)(Wm + w13i(r0 + 4 * k, u)) = x[k] * inv;
    } else if (w < 4) {
      // W2 column d: partial sum of squares over this slice's units
      const int d = (w - 2) * 64 + l;
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < NS / 4; ++k) {   // units 4k .. 4k+3 of column d: 16 bytes in this layout
        const floatx4 x = *(const floatx4*)(S.w2 + w2i(4 * k, d));
#pragma unroll
        for (int j = 0; j < 4; ++j) ss = fmaf(x[j], x[j], ss);
      }
      // The partial norms are the only data exchanged.  Each goes out with its chunk number in one
      // 64-bit device-scope atomic (single-copy atomic, so the number vouches for the value it travels
      // with), and the readers poll the slots themselves: a store and a load per exchange, instead of
      // waiting for the store, raising a counter, polling it and then loading the values.  The slots
      // of chunk c are reused at chunk c + 2, by which time every slice has read them (it wrote its
      // chunk c + 1 partial after using chunk c's); the call clears them before the launch.
      unsigned long long* slots = ss2 + ((size_t)bh * 2 + (c & 1)) * SW_NSL * D + d;
      const unsigned want = (unsigned)(c + 1);
      __hip_atomic_store(slots + (size_t)sl * D, ((unsigned long long)want << 32) | __float_as_uint(ss),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // every slice's partial of this chunk (bounded: on giving up the error flag is raised)
      unsigned long long v[SW_NSL];
      for (int spins = 0;; ++spins) {
#pragma unroll
        for (int s2 = 0; s2 < SW_NSL; ++s2)
          v[s2] = __hip_atomic_load(slots + (size_t)s2 * D, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        bool all = true;
#pragma unroll
        for (int s2 = 0; s2 < SW_NSL; ++s2) all = all && (unsigned)(v[s2] >> 32) == want + target_extra;
        if (all) break;
        if (spins >= spin_limit) {
          __hip_atomic_store(errflag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      ss = 0.f;
      for (int s2 = 0; s2 < SW_NSL; ++s2) ss += __uint_as_float((unsigned)v[s2]);
      const float inv = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
      if constexpr (DUMP) {
        if (sl == 0) R.dnorm[((size_t)bh * nchunks + c) * 640 + 2 * DH + d] = sqrtf(ss);
      }
#pragma unroll
      for (int k = 0; k < NS / 4; ++k) *(floatx4*)(S.w2 + w2i(4 * k, d)) *= inv;
    }
    __syncthreads();
    if constexpr (DUMP) {   // the weights after this chunk's update
      float* Wd = R.dump + ((size_t)bh * nchunks + c) * 3 * D * DH;
      for (int i = tid; i < D * NS; i += NT) {
        const int d = i / NS, u = i % NS;
        Wd[(size_t)d * DH + u0 + u] = S.w1[w13i(d, u)];
        Wd[(size_t)D * DH + (size_t)d * DH + u0 + u] = S.w3[w13i(d, u)];
      }
      for (int i = tid; i < NS * D; i += NT) {
        const int u = i / D, d = i % D;
        Wd[2 * (size_t)D * DH + (size_t)(u0 + u) * D + d] = S.w2[w2i(u, d)];
      }
    }
    if (update_first)
      store_state(c);
    else if (c + 1 < nchunks)
      store_state(c + 1);
  }
  wait_vm<0>();
  if constexpr (RULE >= 1) {
    if (nchunks == 0 && R.Mout) {   // no chunk: the buffers pass through (zeros without M0)
      const size_t hb = (size_t)bh * 3 * D * DH;
      for (int i = tid; i < D * NS; i += NT) {
        const int d = i / NS, u = i % NS;
        for (int j = 0; j < 2; ++j) {
          const size_t o = hb + (size_t)j * D * DH + (size_t)d * DH + u0 + u;
          R.Mout[o] = R.M0 ? R.M0[o] : 0.f;
        }
        const size_t o2 = hb + 2 * (size_t)D * DH + (size_t)(u0 + i / D) * D + i % D;
        R.Mout[o2] = R.M0 ? R.M0[o2] : 0.f;
      }
    }
  }

  if (par) {   // this chunk's W2 update, [d][u] fp32, into Wout (the caller's per-chunk buffer)
    float* inc = Wout + ((size_t)bh * par_nchunks + cpar) * SW_STATE / 2;
    for (int i = tid; i < NS * D; i += NT) {
      const int u = i % NS, d = i / NS;
      inc[(size_t)d * DH + u0 + u] = S.w2[w2i(u, d)];
    }
    return;
  }
  // ---- final weights, packed W1 | W3 | W2 ----
  float* Wo = Wout + (size_t)bh * 3 * D * DH;
  for (int i = tid; i < D * NS; i += NT) {
    const int d = i / NS, u = i % NS;
    Wo[(size_t)d * DH + u0 + u] = S.w1[w13i(d, u)];
    Wo[(size_t)D * DH + (size_t)d * DH + u0 + u] = S.w3[w13i(d, u)];
  }
  for (int i = tid; i < NS * D; i += NT) {
    const int u = i / D, d = i % D;
    Wo[(size_t)2 * D * DH + (size_t)(u0 + u) * D + d] = S.w2[w2i(u, d)];
  }
}

// Last-layer mode, after the per-chunk W2 updates: chunk c's state slot gets
// W2_{c-1} = W2_0 + sum_{c' < c} dW2_c' (planes 4, 5: W2^T hi + lo), and W_out
// the final W2 with W1, W3 as given.  dW2_c was written (fp32 [d][u]) into the
// first bytes of slot c, which this kernel reads before anything overwrites
// them.  One thread per (head, d, 8 consecutive units).
__global__ __launch_bounds__(256) void swiglu_ll_prefix_kernel(const float* __restrict__ W0, bf16* __restrict__ states,
                                                               float* __restrict__ Wout, int BH, int nchunks) {
  constexpr int D = SW_D, DH = SW_DH, G = DH / 8;
  const long long f = (long long)blockIdx.x * 256 + threadIdx.x;
  if (f >= (long long)BH * D * G) return;
  const int bh = (int)(f / (D * G)), d = (int)((f / G) % D), u = (int)(f % G) * 8;
  const float* W0h = W0 + (size_t)bh * 3 * D * DH;
  const size_t P = (size_t)D * DH;
  float run[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) run[j] = W0h[2 * P + (size_t)(u + j) * D + d];
  for (int c = 0; c < nchunks; ++c) {
    bf16* slot = states + ((size_t)bh * nchunks + c) * SW_STATE;
    const float* inc = (const float*)slot + (size_t)d * DH + u;
    const floatx4 i0 = *(const floatx4*)inc, i1 = *(const floatx4*)(inc + 4);
    split_store8(slot + 4 * P + (size_t)d * DH + u, slot + 5 * P + (size_t)d * DH + u, run);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      run[j] += i0[j];
      run[4 + j] += i1[j];
    }
  }
  float* Wo = Wout + (size_t)bh * 3 * P;
#pragma unroll
  for (int j = 0; j < 8; ++j) Wo[2 * P + (size_t)(u + j) * D + d] = run[j];
}

// Last-layer mode: W1^T and W3^T (planes 0..3, bf16 hi + lo) of every chunk's
// slot, and W1, W3 of W_out, from W0.  One thread per (head, unit, 8
// consecutive d).  Runs after swiglu_ll_prefix_kernel has read the updates.
__global__ __launch_bounds__(256) void swiglu_ll_fill_kernel(const float* __restrict__ W0, bf16* __restrict__ states,
                                                             float* __restrict__ Wout, int BH, int nchunks) {
  constexpr int D = SW_D, DH = SW_DH, G = D / 8;
  const long long f = (long long)blockIdx.x * 256 + threadIdx.x;
  if (f >= (long long)BH * DH * G) return;
  const int bh = (int)(f / (DH * G)), u = (int)((f / G) % DH), d = (int)(f % G) * 8;
  const float* W0h = W0 + (size_t)bh * 3 * D * DH;
  const size_t P = (size_t)D * DH;
  float w1[8], w3[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    w1[j] = W0h[(size_t)(d + j) * DH + u];
    w3[j] = W0h[P + (size_t)(d + j) * DH + u];
  }
  for (int c = 0; c < nchunks; ++c) {
    bf16* slot = states + ((size_t)bh * nchunks + c) * SW_STATE + (size_t)u * D + d;
    split_store8(slot, slot + P, w1);
    split_store8(slot + 2 * P, slot + 3 * P, w3);
  }
  float* Wo = Wout + (size_t)bh * 3 * P;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    Wo[(size_t)(d + j) * DH + u] = w1[j];
    Wo[P + (size_t)(d + j) * DH + u] = w3[j];
  }
}

// ---------------------------------------------------------------------------
// read: O = f_{W_{c-1}}(Q_c), computed transposed (tokens on the lanes'
// column index) so that H^T from one product is directly the B operand of
// the next.
// ---------------------------------------------------------------------------
// Weight slices in LDS without padding: a W1T/W3T row (one unit, 256 bytes)
// has its 16-byte pieces at c ^ sw_swz(row); a W2T row (32 units, 64 bytes)
// has its 16-byte pieces at c ^ ((row >> 2) & 3).  Both make the operand reads
// (16 rows per 16 lanes) conflict-free, and both are written by direct-to-LDS
// copies (the permutation is applied to the global addresses).
struct ReadLds {
  unsigned char w13[2][4][SW_US * SW_D * 2];   // W1T hi, W1T lo, W3T hi, W3T lo: [32 units][128 d]
  unsigned char w2[2][2][SW_D * SW_US * 2];    // W2T hi, lo: [n][32 units]
  unsigned char q[SW_TT * SW_D * 2];           // the queries of a tile: [token][d], pieces at c ^ sw_swz(token)
};
static_assert(sizeof(ReadLds) <= 160 * 1024, "read kernel LDS");
constexpr int RW13_ROW = SW_D * 2;
constexpr int RW2_ROW = SW_US * 2;
__device__ __forceinline__ int w2_swz(int row) { return (row >> 2) & 3; }

// Two waves per SIMD, 32 tokens per wave (measured against one wave per SIMD
// with 64 tokens each, which halves the LDS reads of the weights per token:
// ~6 % slower, the lone wave waits on its own LDS reads).
constexpr int SW_RW = 8;                  // waves per read workgroup
constexpr int SW_RT = SW_TT / SW_RW;      // tokens per wave (2 tiles of 16)
constexpr int SW_RSTORES = SW_RT / 16 * 8;   // output stores per wave per tile
// Persistent over tiles: the tiles (head, chunk, 256-token tile) in the order in which the tiles of a
// chunk are adjacent are dealt to the XCDs in 8 contiguous shares, and workgroup r of an XCD takes tiles
// r, r + step, ... of its share (step = workgroups per XCD), so the tiles of a chunk run at about the same
// time on one XCD and its weights are fetched into one L2.  While a tile is computed, the next tile's
// queries are copied into LDS and its first weight slice follows the current tile's last; the current
// tile's output stores drain while the next one starts.  With a grid of one workgroup per tile this is
// the plain one-tile-per-workgroup form.
// OF32: float32 outputs (16 bytes per lane: 4 consecutive columns of one token).
// errflag: raised by the recurrence when a cross-workgroup wait gave up; then every output of the call
// and every head's final weights are filled with NaN instead.
template <bool OF32>
__global__ __launch_bounds__(SW_RW * 64, 1) void swiglu_read_kernel(const bf16* __restrict__ Q,
                                                                    const bf16* __restrict__ states,
                                                                    void* __restrict__ O, int T, int chunk,
                                                                    int nchunks, int tiles, int ntiles,
                                                                    const unsigned* __restrict__ errflag,
                                                                    float* __restrict__ Wout) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  ReadLds& L = *reinterpret_cast<ReadLds*>(smem_raw);
  constexpr int D = SW_D, DH = SW_DH, NTH = SW_RW * 64, TT = SW_RT / 16;
  constexpr int OES = OF32 ? 4 : 2;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, li = l & 15;
  const size_t P = (size_t)D * DH;
  // this workgroup's k-th tile (logical index, tiles of a chunk adjacent), or -1 past its last
  const bool by_xcd = (ntiles & 7) == 0 && (gridDim.x & 7) == 0;
  const int per = by_xcd ? ntiles >> 3 : ntiles;
  const int xcd = by_xcd ? (int)(blockIdx.x & 7) : 0;
  const int r0 = by_xcd ? (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  const int step = by_xcd ? (int)(gridDim.x >> 3) : (int)gridDim.x;
  auto tile_at = [&](int k) -> int {
    const int i = r0 + step * k;
    return i < per ? xcd * per + i : -1;
  };
  struct Tile {
    int bh, c, tile, t0, cend;
  };
  auto decode = [&](int lb) {
    Tile t;
    t.tile = lb % tiles;
    t.c = (lb / tiles) % nchunks;
    t.bh = lb / (tiles * nchunks);
    t.cend = min((t.c + 1) * chunk, T);
    t.t0 = t.c * chunk + t.tile * SW_TT;
    return t;
  };
  if (__hip_atomic_load(errflag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
    // the recurrence could not complete: no output of this call is valid
    const float nan = __builtin_nanf("");
    for (int k = 0; tile_at(k) >= 0; ++k) {
      const Tile t = decode(tile_at(k));
      if (t.t0 < t.cend) {
        unsigned char* Ot = (unsigned char*)O + ((size_t)t.bh * T + t.t0) * D * OES;
        const int n = (t.cend - t.t0 < SW_TT ? t.cend - t.t0 : SW_TT) * D;
        for (int i = threadIdx.x; i < n; i += NTH) {
          if constexpr (OF32)
            ((float*)Ot)[i] = nan;
          else
            ((bf16*)Ot)[i] = (bf16)nan;
        }
      }
      if (t.c == 0 && t.tile == 0)
        for (int i = threadIdx.x; i < 3 * (int)P; i += NTH) Wout[(size_t)t.bh * 3 * P + i] = nan;
    }
    return;
  }
  // the next tile at or after k with tokens (tiles past a short last chunk's end have none), or -1
  auto next_tile = [&](int k) -> int {
    for (;; ++k) {
      const int lb = tile_at(k);
      if (lb < 0) return -1;
      const Tile t = decode(lb);
      if (t.t0 < t.cend) return k;
    }
  };

  // a tile's queries -> L.q by direct-to-LDS copies: each wave copies 8 KB (rows 32 w .. 32 w + 31);
  // rows past the chunk's end read 0
  constexpr int JQ = SW_TT * D * 2 / 1024 / SW_RW;
  unsigned offq[JQ];
#pragma unroll
  for (int j = 0; j < JQ; ++j) {
    const int b = (w * JQ + j) * 1024 + 16 * l, row = b >> 8, q = (b & 255) >> 4;
    offq[j] = (unsigned)(row * D * 2 + ((q ^ sw_swz(row)) << 4));
  }
  auto load_q = [&](const Tile& t) {
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(Q + ((size_t)t.bh * T + t.t0) * D, ((long long)t.cend - t.t0) * D * 2);
#pragma unroll
    for (int j = 0; j < JQ; ++j) dma16<true>(rq, offq[j], L.q + (w * JQ + j) * 1024);
  };
  // weight slice sl of a tile's chunk -> LDS buffer buf: each wave copies 4 KB of the W1T/W3T planes
  // (4 x 1 KB) and 2 KB of the W2T planes (2 x 1 KB)
  constexpr int J13 = 4 * SW_US * SW_D * 2 / 1024 / SW_RW, J2 = 2 * SW_D * SW_US * 2 / 1024 / SW_RW;
  unsigned off13[J13], off2[J2];
#pragma unroll
  for (int j = 0; j < J13; ++j) {
    const int k = w * J13 + j, plane = k >> 3, b = (k & 7) * 1024 + 16 * l, row = b >> 8, q = (b & 255) >> 4;
    off13[j] = (unsigned)(((size_t)plane * P + (size_t)row * D + ((q ^ sw_swz(row)) << 3)) * 2);
  }
#pragma unroll
  for (int j = 0; j < J2; ++j) {
    const int k2 = w * J2 + j, plane = k2 >> 3, b = (k2 & 7) * 1024 + 16 * l, n = b >> 6, q = (b & 63) >> 4;
    off2[j] = (unsigned)(((size_t)(4 + plane) * P + (size_t)n * DH + ((q ^ w2_swz(n)) << 3)) * 2);
  }
  auto load_slice = [&](const Tile& t, int sl, int buf) {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(states + ((size_t)t.bh * nchunks + t.c) * SW_STATE, (long long)SW_STATE * 2);
    const unsigned u13 = (unsigned)(SW_US * sl * D * 2), u2 = (unsigned)(SW_US * sl * 2);
#pragma unroll
    for (int j = 0; j < J13; ++j) {
      const int k = w * J13 + j;
      dma16<false>(rs, u13 + off13[j], L.w13[buf][k >> 3] + (k & 7) * 1024);
    }
#pragma unroll
    for (int j = 0; j < J2; ++j) {
      const int k2 = w * J2 + j;
      dma16<false>(rs, u2 + off2[j], L.w2[buf][k2 >> 3] + (k2 & 7) * 1024);
    }
  };

  constexpr int NSLICE = DH / SW_US;
  static_assert(NSLICE % 2 == 0, "a tile's first slice goes into buffer 0");
  int k = next_tile(0);
  if (k < 0) return;   // uniform over the workgroup, before any barrier
  Tile cur = decode(tile_at(k));
  load_q(cur);
  load_slice(cur, 0, 0);
  for (bool first = true;; first = false) {
    // this tile's queries and first slice have landed, every wave is done with the previous tile (only
    // its output stores, issued after the first slice's copy, may be outstanding)
    if (first)
      wait_vm_barrier<0>();
    else
      wait_vm_barrier<SW_RSTORES>();
    // this wave's queries as B operands (col = token, k = 8 consecutive d)
    bf16x8 qop[TT][4];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int row = SW_RT * w + 16 * tt + li;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qop[tt][ks] = *(const bf16x8*)(L.q + row * D * 2 + (((4 * ks + g) ^ sw_swz(row)) << 4));
    }
    const int kn = next_tile(k + 1);
    const Tile nxt = decode(kn >= 0 ? tile_at(kn) : 0);
    barrier();   // every wave holds its queries: the buffer takes the next tile's
    if (kn >= 0) load_q(nxt);

    floatx4 oacc[8][TT];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) oacc[nt][tt] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int s = 0; s < NSLICE; ++s) {
      const int buf = s & 1;
      // slice s has landed and every wave is done with slice s - 1, whose buffer the next copy reuses
      // (at s = 1 this also completes the next tile's query copy and the previous tile's stores)
      if (s > 0) wait_vm_barrier<0>();
      if (s + 1 < NSLICE)
        load_slice(cur, s + 1, buf ^ 1);
      else if (kn >= 0)
        load_slice(nxt, 0, buf ^ 1);
      // H^T = silu(A^T) * B^T as bf16 hi + lo, k-slot order of the 32 units: 4g..4g+3 of unit tile 0,
      // then of unit tile 1
      bf16x8 hh[TT], hl[TT];
#pragma unroll
      for (int ut = 0; ut < 2; ++ut) {
        // A^T, B^T [unit][token] for one 16-unit tile x the wave's token tiles
        floatx4 at[TT], bt[TT];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) at[tt] = bt[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int off = (16 * ut + li) * RW13_ROW + (((4 * ks + g) ^ sw_swz(16 * ut + li)) << 4);
          const bf16x8 w1h = *(const bf16x8*)(L.w13[buf][0] + off);
          const bf16x8 w1l = *(const bf16x8*)(L.w13[buf][1] + off);
          const bf16x8 w3h = *(const bf16x8*)(L.w13[buf][2] + off);
          const bf16x8 w3l = *(const bf16x8*)(L.w13[buf][3] + off);
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            at[tt] = mfma16(w1h, qop[tt][ks], at[tt]);
            at[tt] = mfma16(w1l, qop[tt][ks], at[tt]);
            bt[tt] = mfma16(w3h, qop[tt][ks], bt[tt]);
            bt[tt] = mfma16(w3l, qop[tt][ks], bt[tt]);
          }
        }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float a = at[tt][r];
            const float h = a * sigmoid_fast(a) * bt[tt][r];
            const bf16 hb = (bf16)h;
            hh[tt][4 * ut + r] = hb;
            hl[tt][4 * ut + r] = (bf16)(h - (float)hb);
          }
      }
      // O^T[n][t] += W2^T[n][units] H^T[units][t]
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const unsigned char* rowh = L.w2[buf][0] + (16 * nt + li) * RW2_ROW;
        const unsigned char* rowl = L.w2[buf][1] + (16 * nt + li) * RW2_ROW;
        // units 4g..4g+3 and 16+4g..16+4g+3: halves of the 16-byte pieces g/2 and 2+g/2
        const int p0 = (((g >> 1) ^ w2_swz(16 * nt + li)) << 4) + (g & 1) * 8;
        const int p1 = (((2 + (g >> 1)) ^ w2_swz(16 * nt + li)) << 4) + (g & 1) * 8;
        const bf16x8 w2h = join(*(const bf16x4*)(rowh + p0), *(const bf16x4*)(rowh + p1));
        const bf16x8 w2l = join(*(const bf16x4*)(rowl + p0), *(const bf16x4*)(rowl + p1));
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          oacc[nt][tt] = mfma16(w2h, hh[tt], oacc[nt][tt]);
          oacc[nt][tt] = mfma16(w2h, hl[tt], oacc[nt][tt]);
          oacc[nt][tt] = mfma16(w2l, hh[tt], oacc[nt][tt]);
        }
      }
    }
    unsigned char* Oh = (unsigned char*)O + (size_t)cur.bh * T * D * OES;
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(Oh + (size_t)cur.t0 * D * OES, ((long long)cur.cend - cur.t0) * D * OES);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const unsigned off = (unsigned)(((SW_RT * w + 16 * tt + li) * D + 16 * nt + 4 * g) * OES);
        if constexpr (OF32) {
          buf_store16(ro, off, __builtin_bit_cast(u32x4, oacc[nt][tt]));
        } else {
          const bf16x4 o = to_bf16x4(oacc[nt][tt][0], oacc[nt][tt][1], oacc[nt][tt][2], oacc[nt][tt][3]);
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(uint2v, o), ro, off, 0, 0);
        }
      }
    if (kn < 0) break;
    k = kn;
    cur = nxt;
  }
}

struct SwLayout {
  size_t states, ss2, counters, err, ns, total;
};

// muon: room for the Newton-Schulz exchange (partial Gram matrices and their sums, per head)
SwLayout sw_layout(int64_t BH, int64_t nchunks, int muon) {
  SwLayout L;
  L.states = 0;
  size_t off = (size_t)BH * nchunks * SW_STATE * 2;
  off = (off + 255) & ~(size_t)255;
  L.ss2 = off;
  off += (size_t)BH * 2 * SW_NSL * SW_D * 8;   // 64-bit slots: chunk number | partial norm
  off = (off + 255) & ~(size_t)255;
  L.counters = off;
  off += (size_t)BH * 4;
  L.err = off;
  off += 4;
  off = (off + 255) & ~(size_t)255;
  L.ns = off;
  if (muon) off += (size_t)BH * NS_HEAD_FLOATS * 4;
  L.total = (off + 255) & ~(size_t)255;
  return L;
}

}  // namespace

bool large_chunk_swiglu_supported(int64_t d, int64_t dh, int64_t chunk, int dtype) {
  (void)chunk;
  return dtype == 1 && d == SW_D && dh == SW_DH;
}

size_t large_chunk_swiglu_workspace(int64_t B, int64_t H, int64_t T, int64_t d, int64_t dh, int64_t chunk, int muon) {
  (void)d;
  (void)dh;
  return sw_layout(B * H, (T + chunk - 1) / chunk, muon).total;
}

// The backward's recomputation of the recurrence (plain descent): the weights after every chunk and the
// column norms before each normalisation, into dump / dnorm (see SwRule); no outputs are read.  The
// forward workspace (states, counters) is that of ttt_la_forward for the same problem.
static void spin_params(int* limit, unsigned* extra);
hipError_t launch_swiglu_recur_dump(const LargeChunkArgs& a, float* dump, float* dnorm, hipStream_t stream) {
  const int BH = (int)(a.B * a.H);
  const int T = (int)a.T, chunk = (int)a.chunk;
  const int nchunks = (int)((a.T + a.chunk - 1) / a.chunk);
  const SwLayout lay = sw_layout(BH, nchunks, 0);
  unsigned char* ws = (unsigned char*)a.ws;
  bf16* states = (bf16*)(ws + lay.states);
  auto* ss2 = (unsigned long long*)(ws + lay.ss2);
  unsigned* counters = (unsigned*)(ws + lay.counters);
  unsigned* err = (unsigned*)(ws + lay.err);
  // the norm-exchange slots, the counters and the error flag start at zero (they are contiguous)
  const int nz = (int)((lay.err + 4 - lay.ss2) / 4);
  hipLaunchKernelGGL(zero_u32_kernel, dim3((nz + 255) / 256), dim3(256), 0, stream, (unsigned*)ss2, nz);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto krec = swiglu_recur_kernel<0, true>;
  const size_t lds_r = sizeof(RecurLds);
  if ((e = hipFuncSetAttribute((const void*)krec, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_r)) !=
      hipSuccess)
    return e;
  int dev = 0, ncu = 0, per_cu = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)krec, SW_WAVES * 64, lds_r)) != hipSuccess)
    return e;
  const int heads_per_launch = (per_cu * ncu) / SW_NSL;
  if (heads_per_launch < 1) return hipErrorLaunchOutOfResources;
  int spin_limit;
  unsigned spin_extra;
  spin_params(&spin_limit, &spin_extra);
  const SwRule R{nullptr, nullptr, 0.f, 0.f, nullptr, dump, dnorm};
  for (int h0 = 0; h0 < BH; h0 += heads_per_launch) {
    const int nh = std::min(heads_per_launch, BH - h0);
    hipLaunchKernelGGL(krec, dim3(nh * SW_NSL), dim3(SW_WAVES * 64), lds_r, stream, (const bf16*)a.K,
                       (const bf16*)a.V, a.eta, a.W0, a.W_out, states, ss2, counters, err, T, chunk, nchunks, h0,
                       0, a.last_layer_only ? 1 : 0, 0, spin_limit, spin_extra, R);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

size_t swiglu_forward_workspace_plain(int64_t BH, int64_t nchunks) { return sw_layout(BH, nchunks, 0).total; }

// O_c = f_{W_{c-1}}(Q_c) for every chunk, from the stored states
static hipError_t launch_read(const LargeChunkArgs& a, const bf16* states, int nchunks, const unsigned* err,
                              hipStream_t stream) {
  const size_t lds_o = sizeof(ReadLds);
  auto kread = a.o_f32 ? swiglu_read_kernel<true> : swiglu_read_kernel<false>;
  hipError_t e = hipFuncSetAttribute((const void*)kread, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_o);
  if (e != hipSuccess) return e;
  int dev = 0, ncu = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  const int chunk = (int)a.chunk, tiles = (chunk + SW_TT - 1) / SW_TT;
  const long long ntiles = (long long)(a.B * a.H) * nchunks * tiles;
  if (ntiles > INT32_MAX) return hipErrorInvalidValue;
  // one workgroup per CU (a multiple of 8, so the tiles of a chunk stay on one XCD) walking the tiles, or
  // one per tile when there are fewer tiles or they do not split evenly over the XCDs
  const long long grid = ntiles > ncu && ntiles % 8 == 0 && ncu >= 8 ? ncu / 8 * 8 : ntiles;
  hipLaunchKernelGGL(kread, dim3((unsigned)grid), dim3(SW_RW * 64), lds_o, stream, (const bf16*)a.Q, states, a.O,
                     (int)a.T, chunk, nchunks, tiles, (int)ntiles, err, a.W_out);
  return hipGetLastError();
}

// Test hook: with TTT_LA_TEST_SPIN_GIVEUP set to a nonzero integer in the environment, every
// cross-workgroup wait of the recurrence waits for a count that never arrives and gives up after that
// many sleeps, so the error path (NaN outputs) can be checked while every kernel still ends.
static void spin_params(int* limit, unsigned* extra) {
  *limit = SW_SPIN_LIMIT;
  *extra = 0u;
  const char* v = getenv("TTT_LA_TEST_SPIN_GIVEUP");
  if (v && atoi(v) > 0) {
    *limit = atoi(v) < 4096 ? atoi(v) : 4096;
    *extra = 1u << 30;
  }
}

hipError_t launch_large_chunk_swiglu(const LargeChunkArgs& a, hipStream_t stream, const Timing& tm) {
  const int BH = (int)(a.B * a.H);
  const int T = (int)a.T, chunk = (int)a.chunk;
  const int nchunks = (int)((a.T + a.chunk - 1) / a.chunk);
  const SwLayout lay = sw_layout(BH, nchunks, a.muon);
  unsigned char* ws = (unsigned char*)a.ws;
  bf16* states = (bf16*)(ws + lay.states);
  auto* ss2 = (unsigned long long*)(ws + lay.ss2);
  unsigned* counters = (unsigned*)(ws + lay.counters);
  unsigned* err = (unsigned*)(ws + lay.err);

  // the norm-exchange slots, the counters and the error flag start at zero (they are contiguous)
  const int nz = (int)((lay.err + 4 - lay.ss2) / 4);
  hipLaunchKernelGGL(zero_u32_kernel, dim3((nz + 255) / 256), dim3(256), 0, stream, (unsigned*)ss2, nz);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // the update rule: plain descent, momentum (M_out given), Muon (with or without momentum)
  const int rule = a.muon ? 2 : (a.M_out ? 1 : 0);
  auto krec = rule == 2 ? swiglu_recur_kernel<2> : rule == 1 ? swiglu_recur_kernel<1> : swiglu_recur_kernel<0>;
  const SwRule R{a.M0, a.M_out, a.momentum, a.muon_scale, (float*)(ws + lay.ns), nullptr, nullptr};
  // the recurrence needs every workgroup of a head resident at once
  const size_t lds_r = sizeof(RecurLds);
  e = hipFuncSetAttribute((const void*)krec, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_r);
  if (e != hipSuccess) return e;
  int dev = 0, ncu = 0, per_cu = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)krec, SW_WAVES * 64, lds_r)) != hipSuccess)
    return e;
  const int heads_per_launch = (per_cu * ncu) / SW_NSL;
  if (heads_per_launch < 1) return hipErrorLaunchOutOfResources;
  if (rule == 0 && a.last_layer_only && !a.update_first && nchunks > 1 && BH * SW_NSL < ncu) {
    // The fully parallel form: every (head, chunk) W2 update at once, a prefix over chunks, the reads.
    // Taken only when the heads alone leave compute units idle: the total work is the same as the
    // recurrence's, and at one workgroup per CU or more the recurrence measured faster (B2 H8 T32768:
    // 0.67 against 0.72 ms per call; it has no prefix pass and no state copies).
    if ((e = mark(tm.start, stream)) != hipSuccess) return e;
    hipLaunchKernelGGL(swiglu_recur_kernel<0>, dim3(BH * nchunks * SW_NSL), dim3(SW_WAVES * 64), lds_r, stream,
                       (const bf16*)a.K, (const bf16*)a.V, a.eta, a.W0, (float*)states, states, ss2, counters, err, T,
                       chunk, nchunks, 0, 0, 1, nchunks, SW_SPIN_LIMIT, 0u, R);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = mark(tm.stop, stream)) != hipSuccess) return e;
    const long long np = (long long)BH * SW_D * (SW_DH / 8);
    hipLaunchKernelGGL(swiglu_ll_prefix_kernel, dim3((unsigned)((np + 255) / 256)), dim3(256), 0, stream, a.W0, states,
                       a.W_out, BH, nchunks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const long long nf = (long long)BH * SW_DH * (SW_D / 8);
    hipLaunchKernelGGL(swiglu_ll_fill_kernel, dim3((unsigned)((nf + 255) / 256)), dim3(256), 0, stream, a.W0, states,
                       a.W_out, BH, nchunks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_read(a, states, nchunks, err, stream);
  }
  const bf16* Kp = (const bf16*)a.K;
  const bf16* Vp = (const bf16*)a.V;
  const float* Ep = a.eta;
  const float* W0p = a.W0;
  float* Wo = a.W_out;
  int spin_limit;
  unsigned spin_extra;
  spin_params(&spin_limit, &spin_extra);
  if ((e = mark(tm.start, stream)) != hipSuccess) return e;   // the recurrence: the sequential part
  // The slices of a head wait for each other at every chunk end, so all workgroups of a launch must be
  // resident together: a launch holds at most as many workgroups as the compute units hold at once (the
  // occupancy query above; one workgroup per CU with this LDS size), which every workgroup of an ordinary
  // launch on an otherwise idle device then is.  If other work held compute units for longer than the
  // bounded wait, the wait gives up and the call's outputs become NaN (see swiglu_read_kernel) instead
  // of hanging.  (An ordinary launch, unlike a cooperative one, can also be captured in a HIP graph.)
  for (int h0 = 0; h0 < BH; h0 += heads_per_launch) {
    const int nh = std::min(heads_per_launch, BH - h0);
    hipLaunchKernelGGL(krec, dim3(nh * SW_NSL), dim3(SW_WAVES * 64), lds_r, stream, Kp, Vp, Ep, W0p, Wo, states, ss2,
                       counters, err, T, chunk, nchunks, h0, a.update_first ? 1 : 0, a.last_layer_only ? 1 : 0, 0,
                       spin_limit, spin_extra, R);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = mark(tm.stop, stream)) != hipSuccess) return e;
  if (nchunks == 0) return hipSuccess;
  return launch_read(a, states, nchunks, err, stream);
}

}  // namespace ttt
