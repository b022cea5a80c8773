// Backward of the LaCT SwiGLU memory (LaCT review "Test-Time Training Done
// Right", non-linear memory and read-order sections): the gradients of a
// scalar loss with respect to Q, K, V, eta and the initial weights, given the
// gradients of O and of the final weights.
//
// Chunk c forms U_c = W_{c-1} + S(W_{c-1}), S the eta-weighted descent step of
// the binding loss, then W_c = U_c normalised per column; its queries read
// R_c = W_{c-1} (W_c when a chunk updates first).  From the last chunk back,
// with G the gradient of the newest weights:
//   update-first: G += the read's weight gradient at W_c (and dQ_c);
//   dU = (G - w (w . G)) / n per column (w the normalised column, n its norm
//        before normalising; G / 1e-12 at the floor); the last-layer mode has
//        no normalisation and no W1/W3 step, so dU = (0, 0, G2);
//   the step's vector-Jacobian product with dU: with a = k W1, b = k W3,
//        s = silu(a), h = s b, adot = k dU1, bdot = k dU3,
//        hdot = silu'(a) adot b + s bdot, g = v W2^T, r = v dU2^T,
//        ydot = hdot W2 + h dU2:
//        dV = eta ydot, deta = <ydot, v>,
//        Pa = silu''(a) adot b g + silu'(a) (bdot g + b r),
//        Pb = silu'(a) adot g + s r, Padot = silu'(a) b g, Pbdot = s g,
//        dK = eta (Pa W1^T + Pb W3^T + Padot dU1^T + Pbdot dU3^T),
//        J = (K^T eta Pa, K^T eta Pb, (eta hdot)^T V);
//   G = dU + J (G + J for a matrix the loop does not update);
//   read-first: G += the read's weight gradient at W_{c-1} (and dQ_c).
// dW0 = G.  The read's gradients at weights R: a = Q R1, b = Q R3,
// dh = dO R2^T, da = dh b silu'(a), db = dh silu(a): dQ = da R1^T + db R3^T,
// (Q^T da, Q^T db, (silu(a) b)^T dO).
//
// Every chunk's weights and column norms come from running the recurrence
// again with a float32 dump (launch_swiglu_recur_dump).  Each step above is a
// batched product over the heads on bf16 MFMA with float32 operands split
// into bf16 hi + lo (three products: hi hi, hi lo, lo hi) and float32
// accumulation, or an elementwise kernel; the host walks the chunks.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace ttt {

namespace {

constexpr int BD = 128;            // d
constexpr int BDH = 256;           // d_h
constexpr long long BP = (long long)BD * BDH;   // elements of one d x d_h matrix
constexpr float BNORM_EPS = 1e-12f;

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }

// ---------------------------------------------------------------------------
// C = A B (+ beta C) over a batch, with the contraction optionally split:
// blockIdx.z = batch * nsplit + split, split s covering k in [s kper,
// min(K, (s + 1) kper)) and writing its partial product to C + s bCs.  A is
// M x K, B is K x N, addressed by element strides; one stride of each operand
// is 1.  An operand whose contraction index is contiguous (A: sAk = 1, B:
// sBk = 1) is staged in LDS as [row][k] and read as 16-byte MFMA fragments;
// otherwise (ATR / BTR) it is staged as [k][row] in its own order and read
// with the transposed LDS read.  Float32 operands are split into bf16 hi +
// lo planes on the way into LDS (three products per pair, float32
// accumulation); bf16 operands are exact and have no lo plane.
// 128 x 128 tiles, 32-deep steps, 4 waves of 64 x 64 (4 x 4 16x16x32 MFMA
// tiles each); the next step's tiles are loaded into registers while the
// current one is multiplied.  Requirements (checked by the host): the
// contiguous extent of every operand is a whole number of tiles (M, N
// multiples of 128 where they are contiguous, K a multiple of 32 where it
// is); the strided extent may be ragged (rows past it read as zero).
// ---------------------------------------------------------------------------
struct GemmArgs {
  const void* A;
  const void* B;
  float* C;
  int M, N, K;
  long long sAm, sAk, sBk, sBn, sCm;
  long long bA, bB, bC;
  float beta;
  int nsplit, kper;
  long long bCs;
};
constexpr int GT = 128, GK = 32;
constexpr int PLANE_ROW = GK * 2 + 16;          // [row][k] plane: 64 bytes of k + 16 bytes of padding
constexpr int PLANE_TR_ROW = GT * 2 + 32;       // [k][row] plane: 256 bytes of rows + 32 bytes of padding
constexpr int PLANE_BYTES = GT * PLANE_ROW;     // 10240 >= GK * PLANE_TR_ROW = 9216

template <typename T>
struct GemmOperand {
  static constexpr bool F32 = sizeof(T) == 4;
  static constexpr int LOADS = F32 ? 4 : 2;     // 16-byte loads per thread per tile
};

// One operand tile (rows r0.., k in [k0, kend)) into registers: 16-byte pieces, zeros past the ragged extent.
template <typename T, bool TR>
__device__ __forceinline__ void gemm_load(u32x4 (&v)[GemmOperand<T>::LOADS], const T* P, long long s_row,
                                          long long s_k, int r0, int rend, int k0, int kend) {
  constexpr bool F32 = GemmOperand<T>::F32;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < GemmOperand<T>::LOADS; ++q) {
    const int idx = tid + 256 * q;
    bool ok;
    const T* src;
    if (!TR) {      // [row][k]: F32 8 pieces of 4 per row, bf16 4 pieces of 8
      const int row = F32 ? idx >> 3 : idx >> 2, pc = F32 ? idx & 7 : idx & 3;
      ok = r0 + row < rend;
      src = P + (long long)(r0 + row) * s_row + (k0 + pc * (F32 ? 4 : 8));
    } else {        // [k][row]: F32 32 pieces of 4 per k, bf16 16 pieces of 8
      const int kr = F32 ? idx >> 5 : idx >> 4, pc = F32 ? idx & 31 : idx & 15;
      ok = k0 + kr < kend;
      src = P + (long long)(k0 + kr) * s_k + (r0 + pc * (F32 ? 4 : 8));
    }
    v[q] = ok ? *(const u32x4*)src : u32x4{0u, 0u, 0u, 0u};
  }
}

// The registers of gemm_load into the hi (and lo) planes.
template <typename T, bool TR>
__device__ __forceinline__ void gemm_store(const u32x4 (&v)[GemmOperand<T>::LOADS], unsigned char* hi,
                                           unsigned char* lo) {
  constexpr bool F32 = GemmOperand<T>::F32;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < GemmOperand<T>::LOADS; ++q) {
    const int idx = tid + 256 * q;
    int off;
    if (!TR) {
      const int row = F32 ? idx >> 3 : idx >> 2, pc = F32 ? idx & 7 : idx & 3;
      off = row * PLANE_ROW + pc * (F32 ? 8 : 16);
    } else {
      const int kr = F32 ? idx >> 5 : idx >> 4, pc = F32 ? idx & 31 : idx & 15;
      off = kr * PLANE_TR_ROW + pc * (F32 ? 8 : 16);
    }
    if (F32) {
      const floatx4 f = __builtin_bit_cast(floatx4, v[q]);
      const uint2 s0 = split2(f[0], f[1]), s1 = split2(f[2], f[3]);
      *(uint2*)(hi + off) = uint2{s0.x, s1.x};
      *(uint2*)(lo + off) = uint2{s0.y, s1.y};
    } else {
      *(u32x4*)(hi + off) = v[q];
    }
  }
}

// MFMA fragment of rows rb .. rb + 15 (lane: row rb + l % 16, k = 8 (l / 16) .. + 7) from a plane.
template <bool TR>
__device__ __forceinline__ bf16x8 gemm_frag(const unsigned char* plane, int rb) {
  const int l = threadIdx.x & 63, g = l >> 4, i = l & 15;
  if (!TR) return *(const bf16x8*)(plane + (rb + i) * PLANE_ROW + g * 16);
  const unsigned char* p = plane + (8 * g + (i >> 2)) * PLANE_TR_ROW + (rb + 4 * (i & 3)) * 2;
  const bf16x4 a = lds_read_tr16(p), b = lds_read_tr16(p + 4 * PLANE_TR_ROW);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <typename TA, typename TB, bool ATR, bool BTR>
__global__ __launch_bounds__(256, 2) void sw_gemm_kernel(GemmArgs g) {
  constexpr bool AF = GemmOperand<TA>::F32, BF = GemmOperand<TB>::F32;
  __shared__ __attribute__((aligned(16))) unsigned char lds[4 * PLANE_BYTES];
  unsigned char* ahi = lds;
  unsigned char* alo = lds + PLANE_BYTES;
  unsigned char* bhi = lds + 2 * PLANE_BYTES;
  unsigned char* blo = lds + 3 * PLANE_BYTES;
  const int nsplit = g.nsplit;
  const long long bz = blockIdx.z / nsplit;
  const int split = blockIdx.z % nsplit;
  const TA* A = (const TA*)g.A + bz * g.bA;
  const TB* B = (const TB*)g.B + bz * g.bB;
  float* C = g.C + bz * g.bC + split * g.bCs;
  const int m0 = blockIdx.y * GT, n0 = blockIdx.x * GT;
  const int kbeg = split * g.kper, kend = min(g.K, kbeg + g.kper);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, gq = l >> 4, li = l & 15;
  const int wm = w >> 1, wn = w & 1;
  // operand A rows are m (row stride sAm, k stride sAk); operand B rows are n (sBn, sBk)
  const long long a_row = g.sAm, a_k = g.sAk, b_row = g.sBn, b_k = g.sBk;
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  u32x4 va[GemmOperand<TA>::LOADS], vb[GemmOperand<TB>::LOADS];
  if (kbeg < kend) {
    gemm_load<TA, ATR>(va, A, a_row, a_k, m0, g.M, kbeg, kend);
    gemm_load<TB, BTR>(vb, B, b_row, b_k, n0, g.N, kbeg, kend);
  }
  for (int k0 = kbeg; k0 < kend; k0 += GK) {
    gemm_store<TA, ATR>(va, ahi, alo);
    gemm_store<TB, BTR>(vb, bhi, blo);
    __syncthreads();
    if (k0 + GK < kend) {
      gemm_load<TA, ATR>(va, A, a_row, a_k, m0, g.M, k0 + GK, kend);
      gemm_load<TB, BTR>(vb, B, b_row, b_k, n0, g.N, k0 + GK, kend);
    }
    bf16x8 bh[4], bl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bh[j] = gemm_frag<BTR>(bhi, 64 * wn + 16 * j);
      if (BF) bl[j] = gemm_frag<BTR>(blo, 64 * wn + 16 * j);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x8 ah = gemm_frag<ATR>(ahi, 64 * wm + 16 * i);
      bf16x8 al;
      if (AF) al = gemm_frag<ATR>(alo, 64 * wm + 16 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = mfma16(ah, bh[j], acc[i][j]);
        if (BF) acc[i][j] = mfma16(ah, bl[j], acc[i][j]);
        if (AF) acc[i][j] = mfma16(al, bh[j], acc[i][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 64 * wm + 16 * i + 4 * gq + r;
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + 64 * wn + 16 * j + li;
        float* p = C + (long long)m * g.sCm + n;
        *p = g.beta != 0.f ? acc[i][j][r] + g.beta * *p : acc[i][j][r];
      }
    }
}

// Launch with the operand orientations taken from the strides; nsplit > 1 splits the contraction into
// pieces of kper (a multiple of GK) whose partial products go to C + s bCs.
template <typename TA, typename TB>
hipError_t gemm(GemmArgs g, int batch, hipStream_t stream, int nsplit = 1, long long bCs = 0) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const bool atr = g.sAk != 1, btr = g.sBk != 1;
  // the contiguous extent of each operand must be whole tiles (or whole k steps)
  if ((atr ? (g.sAm != 1 || g.M % GT) : (g.K % GK)) || (btr ? (g.sBn != 1 || g.N % GT) : (g.K % GK)) || g.N % GT)
    return hipErrorInvalidValue;
  if (nsplit < 1) nsplit = 1;
  g.kper = (((g.K + nsplit - 1) / nsplit) + GK - 1) / GK * GK;
  g.nsplit = nsplit;
  g.bCs = bCs;
  const dim3 grid((unsigned)(g.N / GT), (unsigned)((g.M + GT - 1) / GT), (unsigned)(batch * nsplit));
  if (atr && btr)
    hipLaunchKernelGGL((sw_gemm_kernel<TA, TB, true, true>), grid, dim3(256), 0, stream, g);
  else if (atr)
    hipLaunchKernelGGL((sw_gemm_kernel<TA, TB, true, false>), grid, dim3(256), 0, stream, g);
  else if (btr)
    hipLaunchKernelGGL((sw_gemm_kernel<TA, TB, false, true>), grid, dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL((sw_gemm_kernel<TA, TB, false, false>), grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

__device__ __forceinline__ float sigm(float a) { return 1.0f / (1.0f + expf(-a)); }

// The step's elementwise part for chunk tokens t < Cc, units u < d_h (one thread each; grid.y = head):
// Z1 [t][a | b | adot | bdot], Z2 [t][g | r] -> E1 [t][eta Pa | eta Pb | eta Padot | eta Pbdot],
// E2 [t][hdot | h], E3 [t][eta hdot].
__global__ __launch_bounds__(256) void sw_bwd_step_elem(const float* __restrict__ Z1, const float* __restrict__ Z2,
                                                        const float* __restrict__ eta, float* __restrict__ E1,
                                                        float* __restrict__ E2, float* __restrict__ E3, int Cc,
                                                        long long ldz, int T, int c0) {
  const long long h = blockIdx.y;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)Cc * BDH) return;
  const long long t = i / BDH;
  const int u = (int)(i % BDH);
  const float* z1 = Z1 + h * ldz * 4 * BDH + t * 4 * BDH;
  const float* z2 = Z2 + h * ldz * 2 * BDH + t * 2 * BDH;
  const float a = z1[u], b = z1[BDH + u], ad = z1[2 * BDH + u], bd = z1[3 * BDH + u];
  const float gg = z2[u], r = z2[BDH + u];
  const float e = eta[h * T + c0 + t];
  const float sg = sigm(a), s = a * sg, s1 = sg * (1.0f + a * (1.0f - sg));
  const float s2 = sg * (1.0f - sg) * (2.0f + a * (1.0f - 2.0f * sg));
  const float hh = s * b, hd = s1 * ad * b + s * bd;
  float* e1 = E1 + h * ldz * 4 * BDH + t * 4 * BDH;
  e1[u] = e * (s2 * ad * b * gg + s1 * (bd * gg + b * r));
  e1[BDH + u] = e * (s1 * ad * gg + s * r);
  e1[2 * BDH + u] = e * (s1 * b * gg);
  e1[3 * BDH + u] = e * (s * gg);
  float* e2 = E2 + h * ldz * 2 * BDH + t * 2 * BDH;
  e2[u] = hd;
  e2[BDH + u] = hh;
  E3[h * ldz * BDH + t * BDH + u] = e * hd;
}

// The read's elementwise part: Zq [t][a | b], Dh [t][dh] -> Eq [t][da | db], Hq [t][silu(a) b].
__global__ __launch_bounds__(256) void sw_bwd_read_elem(const float* __restrict__ Zq, const float* __restrict__ Dh,
                                                        float* __restrict__ Eq, float* __restrict__ Hq, int Cc,
                                                        long long ldz) {
  const long long h = blockIdx.y;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)Cc * BDH) return;
  const long long t = i / BDH;
  const int u = (int)(i % BDH);
  const float* zq = Zq + h * ldz * 2 * BDH + t * 2 * BDH;
  const float a = zq[u], b = zq[BDH + u];
  const float dh = Dh[h * ldz * BDH + t * BDH + u];
  const float sg = sigm(a), s = a * sg, s1 = sg * (1.0f + a * (1.0f - sg));
  float* eq = Eq + h * ldz * 2 * BDH + t * 2 * BDH;
  eq[u] = dh * b * s1;
  eq[BDH + u] = dh * s;
  Hq[h * ldz * BDH + t * BDH + u] = s * b;
}

// Per head, one wave per column: the normalisation's backward dU of G (packed W1 | W3 | W2) at the chunk's
// normalised weights Wc and norms nrm, and the operand blocks of the step at the weights before it (Wp):
// Wcat [d][W1 | W3 | dU1 | dU3] (d x 4 d_h), W2cat [W2 ; dU2] (2 d_h x d).  Columns 0..255: W1, 256..511:
// W3, 512..639: W2.  last_only: dU1 = dU3 = 0, dU2 = G2.
__global__ __launch_bounds__(256) void sw_bwd_prep(const float* __restrict__ G, const float* __restrict__ Wc,
                                                   long long wc_stride, const float* __restrict__ nrm,
                                                   long long nrm_stride, const float* __restrict__ Wp,
                                                   long long wp_stride, float* __restrict__ Wcat,
                                                   float* __restrict__ W2cat, int last_only) {
  const long long h = blockIdx.y;
  const int col = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  const float* g = G + h * 3 * BP;
  const float* wc = Wc + h * wc_stride;
  const float* wp = Wp + h * wp_stride;
  float* wcat = Wcat + h * BD * 4 * BDH;
  float* w2cat = W2cat + h * 2 * BDH * BD;
  if (col < 2 * BDH) {              // a column of W1 or W3: d = l, l + 64
    const int m = col / BDH, u = col % BDH;
    const long long base = m * BP;
    float gv[2], wv[2], dot = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int d = l + 64 * j;
      gv[j] = g[base + (long long)d * BDH + u];
      wv[j] = wc[base + (long long)d * BDH + u];
      dot += gv[j] * wv[j];
      wcat[(long long)d * 4 * BDH + m * BDH + u] = wp[base + (long long)d * BDH + u];
    }
    dot = wave_sum(dot);
    const float n = nrm[h * nrm_stride + col];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int d = l + 64 * j;
      const float du = last_only ? 0.f : (n > BNORM_EPS ? (gv[j] - wv[j] * dot) / n : gv[j] / BNORM_EPS);
      wcat[(long long)d * 4 * BDH + (2 + m) * BDH + u] = du;
    }
  } else {                          // a column of W2: units u = l, l + 64, l + 128, l + 192
    const int dcol = col - 2 * BDH;
    float gv[4], wv[4], dot = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = l + 64 * j;
      gv[j] = g[2 * BP + (long long)u * BD + dcol];
      wv[j] = wc[2 * BP + (long long)u * BD + dcol];
      dot += gv[j] * wv[j];
      w2cat[(long long)u * BD + dcol] = wp[2 * BP + (long long)u * BD + dcol];
    }
    dot = wave_sum(dot);
    const float n = last_only ? 0.f : nrm[h * nrm_stride + col];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = l + 64 * j;
      const float du = last_only ? gv[j] : (n > BNORM_EPS ? (gv[j] - wv[j] * dot) / n : gv[j] / BNORM_EPS);
      w2cat[(long long)(BDH + u) * BD + dcol] = du;
    }
  }
}

// G (packed W1 | W3 | W2 per head) from the chunk's terms, each the sum of its split partials in a fixed order
// (J13, A13: s13 partials of [BH][d][2 d_h]; J2, A2: s2 partials of [BH][d_h][d]):
//   add_read_only: G += A (the read's weight gradient: A13 [d][W1 | W3 parts], A2 [d_h][d]);
//   otherwise: G = base + J (+ A when with_read), base = dU (from Wcat / W2cat) for an updated matrix, G
//   itself for a matrix the loop does not update (W1, W3 in the last-layer mode).
__global__ __launch_bounds__(256) void sw_bwd_gupdate(float* __restrict__ G, const float* __restrict__ Wcat,
                                                      const float* __restrict__ W2cat, const float* __restrict__ J13,
                                                      const float* __restrict__ J2, const float* __restrict__ A13,
                                                      const float* __restrict__ A2, int s13, int s2,
                                                      int add_read_only, int with_read, int last_only) {
  const long long h = blockIdx.y, BH = gridDim.y;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= 3 * BP) return;
  float* g = G + h * 3 * BP + i;
  auto psum = [](const float* P, int n, long long stride, long long off) {
    float x = 0.f;
    for (int s = 0; s < n; ++s) x += P[s * stride + off];
    return x;
  };
  float a, j, base;
  if (i < 2 * BP) {
    const int m = (int)(i / BP);
    const long long k = i % BP, d = k / BDH, u = k % BDH;
    const long long off = h * BD * 2 * BDH + d * 2 * BDH + m * BDH + u, stride = BH * BD * 2 * BDH;
    a = A13 ? psum(A13, s13, stride, off) : 0.f;
    if (add_read_only) {
      *g += a;
      return;
    }
    j = psum(J13, s13, stride, off);
    base = last_only ? *g : Wcat[h * BD * 4 * BDH + d * 4 * BDH + (2 + m) * BDH + u];
  } else {
    const long long k = i - 2 * BP;
    a = A2 ? psum(A2, s2, BH * BP, h * BP + k) : 0.f;
    if (add_read_only) {
      *g += a;
      return;
    }
    j = psum(J2, s2, BH * BP, h * BP + k);
    base = W2cat[h * 2 * BP + BP + k];
  }
  *g = base + j + (with_read ? a : 0.f);
}

// dV = eta ydot (ydot computed into dV), deta = <ydot, v>: one wave per token.
__global__ __launch_bounds__(256) void sw_bwd_finish_v(float* __restrict__ dV, float* __restrict__ deta,
                                                       const bf16* __restrict__ V, const float* __restrict__ eta,
                                                       int T, int c0, int Cc) {
  const long long h = blockIdx.y;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (t >= Cc) return;
  const long long row = h * T + c0 + t;
  float* y = dV + row * BD;
  const bf16* v = V + row * BD;
  const float e = eta[row];
  const float y0 = y[l], y1 = y[l + 64];
  const float dot = wave_sum(y0 * (float)v[l] + y1 * (float)v[l + 64]);
  y[l] = e * y0;
  y[l + 64] = e * y1;
  if (l == 0) deta[row] = dot;
}

__global__ __launch_bounds__(256) void sw_bwd_copy(float* __restrict__ dst, const float* __restrict__ src, long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

struct BwdSwLayout {
  size_t fws, wfin, dump, dnorm, wcat, w2cat, z1, e1, z2, e2, e3, j13, j2, a13, a2, total;
};
size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
// Split of the products that contract over a chunk's tokens: enough workgroups (about 512) for the chip, at
// least 128 tokens per split, at most 16 splits.
int token_split(int tiles_per_head, int64_t BH, int64_t Cc) {
  const int64_t want = 512 / std::max<int64_t>(1, tiles_per_head * BH);
  const int64_t most = std::max<int64_t>(1, Cc / 128);
  return (int)std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(want, most), 16));
}
constexpr int TILES13 = (BD / GT) * (2 * BDH / GT);   // a [d][2 d_h] product
constexpr int TILES2 = (BDH / GT) * (BD / GT);        // a [d_h][d] product

BwdSwLayout bwd_sw_layout(int64_t BH, int64_t T, int64_t chunk) {
  BwdSwLayout L;
  const int64_t nch = (T + chunk - 1) / chunk, Cc = std::min<int64_t>(chunk, T);
  const int64_t s13 = token_split(TILES13, BH, Cc), s2 = token_split(TILES2, BH, Cc);
  size_t o = 0;
  L.fws = o; o += al256(swiglu_forward_workspace_plain(BH, nch));
  L.wfin = o; o += al256((size_t)BH * 3 * BP * 4);
  L.dump = o; o += al256((size_t)BH * nch * 3 * BP * 4);
  L.dnorm = o; o += al256((size_t)BH * nch * 640 * 4);
  L.wcat = o; o += al256((size_t)BH * BD * 4 * BDH * 4);
  L.w2cat = o; o += al256((size_t)BH * 2 * BDH * BD * 4);
  L.z1 = o; o += al256((size_t)BH * Cc * 4 * BDH * 4);
  L.e1 = o; o += al256((size_t)BH * Cc * 4 * BDH * 4);
  L.z2 = o; o += al256((size_t)BH * Cc * 2 * BDH * 4);
  L.e2 = o; o += al256((size_t)BH * Cc * 2 * BDH * 4);
  L.e3 = o; o += al256((size_t)BH * Cc * BDH * 4);
  L.j13 = o; o += al256((size_t)s13 * BH * BD * 2 * BDH * 4);
  L.j2 = o; o += al256((size_t)s2 * BH * BP * 4);
  L.a13 = o; o += al256((size_t)s13 * BH * BD * 2 * BDH * 4);
  L.a2 = o; o += al256((size_t)s2 * BH * BP * 4);
  L.total = o;
  return L;
}

GemmArgs gargs(const void* A, long long sAm, long long sAk, long long bA, const void* B, long long sBk, long long sBn,
               long long bB, float* C, long long sCm, long long bC, int M, int N, int K, float beta = 0.f) {
  GemmArgs g;
  g.A = A; g.B = B; g.C = C;
  g.M = M; g.N = N; g.K = K;
  g.sAm = sAm; g.sAk = sAk; g.sBk = sBk; g.sBn = sBn; g.sCm = sCm;
  g.bA = bA; g.bB = bB; g.bC = bC;
  g.beta = beta;
  g.nsplit = 1; g.kper = K; g.bCs = 0;
  return g;
}

}  // namespace

size_t large_chunk_swiglu_backward_workspace(int64_t B, int64_t H, int64_t T, int64_t chunk) {
  return bwd_sw_layout(B * H, T, chunk).total;
}

hipError_t launch_large_chunk_swiglu_backward(const BackwardArgs& a, int last_only, hipStream_t stream) {
  const int BH = (int)(a.B * a.H);
  const long long T = a.T, C = a.chunk;
  const int nch = (int)((T + C - 1) / C);
  const BwdSwLayout L = bwd_sw_layout(BH, T, C);
  unsigned char* ws = (unsigned char*)a.ws;
  float* wfin = (float*)(ws + L.wfin);
  float* dump = (float*)(ws + L.dump);
  float* dnorm = (float*)(ws + L.dnorm);
  float* Wcat = (float*)(ws + L.wcat);
  float* W2cat = (float*)(ws + L.w2cat);
  float* Z1 = (float*)(ws + L.z1);
  float* E1 = (float*)(ws + L.e1);
  float* Z2 = (float*)(ws + L.z2);
  float* E2 = (float*)(ws + L.e2);
  float* E3 = (float*)(ws + L.e3);
  float* J13 = (float*)(ws + L.j13);
  float* J2 = (float*)(ws + L.j2);
  float* A13 = (float*)(ws + L.a13);
  float* A2 = (float*)(ws + L.a2);
  float* G = a.dW0;                 // the running gradient lives in the output
  const bf16* Q = (const bf16*)a.Q;
  const bf16* K = (const bf16*)a.K;
  const bf16* V = (const bf16*)a.V;
  const bf16* dO = (const bf16*)a.dO;
  float* dQ = (float*)a.dQ;
  float* dK = (float*)a.dK;
  float* dV = (float*)a.dV;
  const long long SP = 3 * BP;      // elements of a packed state
  const long long cap = std::min<long long>(C, T);   // leading dimension (tokens) of the chunk buffers
  const int s13 = token_split(TILES13, BH, cap), s2 = token_split(TILES2, BH, cap);
  const long long p13 = (long long)BH * BD * 2 * BDH, p2 = (long long)BH * BP;   // partial strides
  hipError_t e;
  const long long ncopy = (long long)BH * SP;
  hipLaunchKernelGGL(sw_bwd_copy, dim3((unsigned)((ncopy + 255) / 256)), dim3(256), 0, stream, G, a.dW, ncopy);
  if ((e = hipGetLastError()) != hipSuccess || nch == 0) return e;

  // every chunk's weights and norms (the state sequence is the same in both read orders)
  LargeChunkArgs fa{a.Q, a.K, a.V, a.eta, a.W0, nullptr, wfin, ws + L.fws, a.B, a.H, a.T, BD, BD, BDH, a.chunk, 1, 0};
  fa.last_layer_only = last_only;
  if ((e = launch_swiglu_recur_dump(fa, dump, dnorm, stream)) != hipSuccess) return e;

  const bool read_first = !a.other_order;
  auto read_phase = [&](const float* R, long long rstride, long long c0, int Cc) -> hipError_t {
    hipError_t e2;
    const bf16* Qc = Q + c0 * BD;
    const bf16* dOc = dO + c0 * BD;
    float* Zq = Z1;    // [Cc][a | b]        (Z1's room)
    float* Dh = Z2;    // [Cc][dh]           (Z2's room)
    float* Eq = E1;    // [Cc][da | db]      (E1's room)
    float* Hq = E2;    // [Cc][silu(a) b]    (E2's room)
    // a = Q R1, b = Q R3
    for (int m = 0; m < 2; ++m)
      if ((e2 = gemm<bf16, float>(gargs(Qc, BD, 1, T * BD, R + m * BP, BDH, 1, rstride, Zq + m * BDH, 2 * BDH,
                                        cap * 2 * BDH, Cc, BDH, BD), BH, stream)) != hipSuccess)
        return e2;
    // dh = dO R2^T
    if ((e2 = gemm<bf16, float>(gargs(dOc, BD, 1, T * BD, R + 2 * BP, 1, BD, rstride, Dh, BDH, cap * BDH, Cc, BDH, BD),
                                BH, stream)) != hipSuccess)
      return e2;
    hipLaunchKernelGGL(sw_bwd_read_elem, dim3((unsigned)(((long long)Cc * BDH + 255) / 256), BH), dim3(256), 0, stream,
                       Zq, Dh, Eq, Hq, Cc, cap);
    if ((e2 = hipGetLastError()) != hipSuccess) return e2;
    // dQ = da R1^T + db R3^T
    for (int m = 0; m < 2; ++m)
      if ((e2 = gemm<float, float>(gargs(Eq + m * BDH, 2 * BDH, 1, cap * 2 * BDH, R + m * BP, 1, BDH, rstride,
                                         dQ + c0 * BD, BD, T * BD, Cc, BD, BDH, m == 0 ? 0.f : 1.f), BH, stream)) !=
          hipSuccess)
        return e2;
    // (Q^T da | Q^T db), (silu(a) b)^T dO
    if ((e2 = gemm<bf16, float>(gargs(Qc, 1, BD, T * BD, Eq, 2 * BDH, 1, cap * 2 * BDH, A13, 2 * BDH, BD * 2 * BDH,
                                      BD, 2 * BDH, Cc), BH, stream, s13, p13)) != hipSuccess)
      return e2;
    return gemm<float, bf16>(gargs(Hq, 1, BDH, cap * BDH, dOc, BD, 1, T * BD, A2, BD, BP, BDH, BD, Cc), BH, stream, s2,
                             p2);
  };

  for (int c = nch - 1; c >= 0; --c) {
    const long long c0 = (long long)c * C;
    const int Cc = (int)std::min<long long>(C, T - c0);
    const float* Wp = c == 0 ? a.W0 : dump + (long long)(c - 1) * SP;   // weights before the chunk
    const long long wp_stride = c == 0 ? SP : (long long)nch * SP;
    const float* Wc = dump + (long long)c * SP;                       // after it
    const long long wc_stride = (long long)nch * SP;
    if (!read_first) {   // the chunk's queries read W_c: their gradient reaches G before the normalisation
      if ((e = read_phase(Wc, wc_stride, c0, Cc)) != hipSuccess) return e;
      hipLaunchKernelGGL(sw_bwd_gupdate, dim3((unsigned)((3 * BP + 255) / 256), BH), dim3(256), 0, stream, G, Wcat,
                         W2cat, J13, J2, A13, A2, s13, s2, 1, 0, last_only);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sw_bwd_prep, dim3(640 / 4, BH), dim3(256), 0, stream, G, Wc, wc_stride, dnorm + (long long)c * 640,
                       (long long)nch * 640, Wp, wp_stride, Wcat, W2cat, last_only);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const bf16* Kc = K + c0 * BD;
    const bf16* Vc = V + c0 * BD;
    // Z1 = K [W1 | W3 | dU1 | dU3], Z2 = V [W2 ; dU2]^T
    if ((e = gemm<bf16, float>(gargs(Kc, BD, 1, T * BD, Wcat, 4 * BDH, 1, BD * 4 * BDH, Z1, 4 * BDH, cap * 4 * BDH, Cc,
                                     4 * BDH, BD), BH, stream)) != hipSuccess)
      return e;
    if ((e = gemm<bf16, float>(gargs(Vc, BD, 1, T * BD, W2cat, 1, BD, 2 * BP, Z2, 2 * BDH, cap * 2 * BDH, Cc, 2 * BDH,
                                     BD), BH, stream)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(sw_bwd_step_elem, dim3((unsigned)(((long long)Cc * BDH + 255) / 256), BH), dim3(256), 0, stream,
                       Z1, Z2, a.eta, E1, E2, E3, Cc, cap, (int)T, (int)c0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // dK = E1 [W1 | W3 | dU1 | dU3]^T
    if ((e = gemm<float, float>(gargs(E1, 4 * BDH, 1, cap * 4 * BDH, Wcat, 1, 4 * BDH, BD * 4 * BDH, dK + c0 * BD, BD,
                                      T * BD, Cc, BD, 4 * BDH), BH, stream)) != hipSuccess)
      return e;
    // ydot = E2 [W2 ; dU2] (into dV), then dV = eta ydot and deta = <ydot, v>
    if ((e = gemm<float, float>(gargs(E2, 2 * BDH, 1, cap * 2 * BDH, W2cat, BD, 1, 2 * BP, dV + c0 * BD, BD, T * BD, Cc,
                                      BD, 2 * BDH), BH, stream)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(sw_bwd_finish_v, dim3((unsigned)((Cc + 3) / 4), BH), dim3(256), 0, stream, dV, a.deta, V, a.eta,
                       (int)T, (int)c0, Cc);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // J13 = K^T (eta Pa | eta Pb), J2 = (eta hdot)^T V
    if ((e = gemm<bf16, float>(gargs(Kc, 1, BD, T * BD, E1, 4 * BDH, 1, cap * 4 * BDH, J13, 2 * BDH, BD * 2 * BDH, BD,
                                     2 * BDH, Cc), BH, stream, s13, p13)) != hipSuccess)
      return e;
    if ((e = gemm<float, bf16>(gargs(E3, 1, BDH, cap * BDH, Vc, BD, 1, T * BD, J2, BD, BP, BDH, BD, Cc), BH, stream, s2,
                               p2)) != hipSuccess)
      return e;
    if (read_first && (e = read_phase(Wp, wp_stride, c0, Cc)) != hipSuccess) return e;
    hipLaunchKernelGGL(sw_bwd_gupdate, dim3((unsigned)((3 * BP + 255) / 256), BH), dim3(256), 0, stream, G, Wcat, W2cat,
                       J13, J2, A13, A2, s13, s2, 0, read_first ? 1 : 0, last_only);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ttt
