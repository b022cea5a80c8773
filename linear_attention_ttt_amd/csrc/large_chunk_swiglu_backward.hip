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
// again with a float32 dump (launch_swiglu_recur_dump).  The products are
// batched over the heads on bf16 MFMA with float32 accumulation; a float32
// weight operand is split into bf16 hi + lo (three products: hi hi, hi lo,
// lo hi; two when the other operand is bf16 input).  The products of the
// tokens with the weights run fused with the elementwise factors they feed and
// the products of those factors with the weights (sw_bwd_step_kernel,
// sw_bwd_read_step_kernel); the factors that the weight gradients contract
// over the chunk's tokens (E1a, E3, Eq, Hq) go to memory rounded to bf16, like
// the token inputs they meet there, and those products take one bf16 product
// each.  The host walks the chunks.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace ttt {

namespace {

constexpr int BD = 128;            // d
constexpr int BDH = 256;           // d_h
constexpr long long BP = (long long)BD * BDH;   // elements of one d x d_h matrix
constexpr float BNORM_EPS = 1e-12f;


// ---------------------------------------------------------------------------
// C = A B over a batch, with the contraction optionally split:
// blockIdx.z = batch * nsplit + split, split s covering k in [s kper,
// min(K, (s + 1) kper)) and writing its partial product to C + s bCs.  A is
// M x K, B is K x N, addressed by element strides; one stride of each operand
// is 1.  An operand whose contraction index is contiguous (A: sAk = 1, B:
// sBk = 1) is staged in LDS as [row][k] and read as 16-byte MFMA fragments;
// otherwise (ATR / BTR) it is staged as [k][row] in its own order and read
// with the transposed LDS read.  Both operands are bf16 (float32
// accumulation).  BM x 128 tiles (BM = 128 or 64), 32-deep steps, 4 waves of
// BM/2 x 64 (BM/32 x 4 16x16x32 MFMA tiles each); the tiles of the next two
// steps are in flight in registers while the current one is multiplied.
// Requirements (checked by the host): the contiguous extent of every operand
// is a whole number of tiles (M a multiple of BM and N of 128 where they are
// contiguous, K a multiple of 32 where k is); the strided extent may be
// ragged (rows past it read as zero).
// ---------------------------------------------------------------------------
struct GemmArgs {
  const void* A;
  const void* B;
  float* C;
  int M, N, K;
  long long sAm, sAk, sBk, sBn, sCm;
  long long bA, bB, bC;
  int nsplit, kper;
  long long bCs;
};
constexpr int GT = 128, GK = 32;
constexpr int PLANE_ROW = GK * 2 + 16;          // [row][k] plane: 64 bytes of k + 16 bytes of padding
constexpr int PLANE_TR_ROW = GT * 2 + 32;       // [k][row] plane (128 rows): 256 bytes + 32 bytes of padding
constexpr int PLANE_BYTES = GT * PLANE_ROW;     // 10240 >= GK * PLANE_TR_ROW = 9216

template <typename T, int ROWS = GT>
struct GemmOperand {
  static_assert(sizeof(T) == 2, "bf16 operands");
  static constexpr int PER = 8;                               // elements per 16-byte piece
  static constexpr int LOADS = ROWS * GK / PER / 256;         // 16-byte loads per thread per tile
  static constexpr int KPC = GK / PER;                        // [row][k]: pieces per row
  static constexpr int RPC = ROWS / PER;                      // [k][row]: pieces per k
  static constexpr int TR_ROW = ROWS * 2 + 32;                // [k][row] plane row stride
};

// One operand tile (ROWS rows from r0, k in [k0, kend)) into registers: 16-byte pieces, zeros past the
// ragged extent.  Buffer loads over the valid region
// (rows below rend, or k below kend for a transposed operand; byte offsets below 2^31): a piece past it
// reads 0 without a branch, so the compiler can count the loads in flight.
template <typename T, bool TR, int ROWS>
__device__ __forceinline__ void gemm_load(u32x4 (&v)[(GemmOperand<T, ROWS>::LOADS)], const T* P, long long s_row,
                                          long long s_k, int r0, int rend, int k0, int kend) {
  using O = GemmOperand<T, ROWS>;
  const int tid = threadIdx.x;
  const long long nvalid = TR ? (long long)kend * s_k : (long long)rend * s_row;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(P, nvalid * (long long)sizeof(T));
#pragma unroll
  for (int q = 0; q < O::LOADS; ++q) {
    const int idx = tid + 256 * q;
    long long off;
    if (!TR) {
      const int row = idx / O::KPC, pc = idx % O::KPC;
      off = (long long)(r0 + row) * s_row + (k0 + pc * O::PER);
    } else {
      const int kr = idx / O::RPC, pc = idx % O::RPC;
      off = (long long)(k0 + kr) * s_k + (r0 + pc * O::PER);
    }
    v[q] = buf_load16(rs, (unsigned)(off * (long long)sizeof(T)));
  }
}

// The registers of gemm_load into the LDS plane.
template <typename T, bool TR, int ROWS>
__device__ __forceinline__ void gemm_store(const u32x4 (&v)[(GemmOperand<T, ROWS>::LOADS)], unsigned char* plane) {
  using O = GemmOperand<T, ROWS>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < O::LOADS; ++q) {
    const int idx = tid + 256 * q;
    const int off = !TR ? (idx / O::KPC) * PLANE_ROW + (idx % O::KPC) * 16 : (idx / O::RPC) * O::TR_ROW + (idx % O::RPC) * 16;
    *(u32x4*)(plane + off) = v[q];
  }
}

// MFMA fragment of rows rb .. rb + 15 (lane: row rb + l % 16, k = 8 (l / 16) .. + 7) from a plane whose
// transposed form has row stride tr_row.
template <bool TR>
__device__ __forceinline__ bf16x8 gemm_frag(const unsigned char* plane, int rb, int tr_row = PLANE_TR_ROW) {
  const int l = threadIdx.x & 63, g = l >> 4, i = l & 15;
  if (!TR) return *(const bf16x8*)(plane + (rb + i) * PLANE_ROW + g * 16);
  const unsigned char* p = plane + (8 * g + (i >> 2)) * tr_row + (rb + 4 * (i & 3)) * 2;
  const bf16x4 a = lds_read_tr16(p), b = lds_read_tr16(p + 4 * tr_row);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// One output tile (column tile bx, row tile by, batch entry and contraction split bz) of a product.
template <typename TA, typename TB, bool ATR, bool BTR, int BM>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, int bx, int by, int bzs, unsigned char* lds) {
  using OA = GemmOperand<TA, BM>;
  using OB = GemmOperand<TB, GT>;
  constexpr int MI = BM / 32;             // row tiles per wave
  unsigned char* ap = lds;
  unsigned char* bp = lds + PLANE_BYTES;
  const int nsplit = g.nsplit;
  const long long bz = bzs / nsplit;
  const int split = bzs % nsplit;
  const TA* A = (const TA*)g.A + bz * g.bA;
  const TB* B = (const TB*)g.B + bz * g.bB;
  float* C = g.C + bz * g.bC + split * g.bCs;
  const int m0 = by * BM, n0 = bx * GT;
  const int kbeg = split * g.kper, kend = min(g.K, kbeg + g.kper);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, gq = l >> 4, li = l & 15;
  const int wm = w >> 1, wn = w & 1;
  // operand A rows are m (row stride sAm, k stride sAk); operand B rows are n (sBn, sBk)
  const long long a_row = g.sAm, a_k = g.sAk, b_row = g.sBn, b_k = g.sBk;
  floatx4 acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  // two steps' tiles in flight in registers, in two sets used alternately (no copies between them, so
  // each set's loads have two steps to arrive): set 0 holds the even steps from kbeg, set 1 the odd
  u32x4 va0[OA::LOADS], vb0[OB::LOADS], va1[OA::LOADS], vb1[OB::LOADS];
  auto load = [&](u32x4 (&va)[OA::LOADS], u32x4 (&vb)[OB::LOADS], int k) {
    gemm_load<TA, ATR, BM>(va, A, a_row, a_k, m0, g.M, k, kend);
    gemm_load<TB, BTR, GT>(vb, B, b_row, b_k, n0, g.N, k, kend);
  };
  // one step: the set's tiles into LDS, the set reloaded with the step two ahead, the products
  auto step = [&](u32x4 (&va)[OA::LOADS], u32x4 (&vb)[OB::LOADS], int k0) {
    gemm_store<TA, ATR, BM>(va, ap);
    gemm_store<TB, BTR, GT>(vb, bp);
    __syncthreads();
    load(va, vb, k0 + 2 * GK);   // unconditional (past the end it reads zeros or unused values), so that
                                 // the loads in flight are the same on every path
    bf16x8 bf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = gemm_frag<BTR>(bp, 64 * wn + 16 * j, OB::TR_ROW);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const bf16x8 af = gemm_frag<ATR>(ap, (BM / 2) * wm + 16 * i, OA::TR_ROW);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(af, bf[j], acc[i][j]);
    }
    __syncthreads();
  };
  load(va0, vb0, kbeg);
  asm volatile("" ::: "memory");   // set 0's loads stay the older ones, as in every later step
  load(va1, vb1, kbeg + GK);
  // pairs of steps, then an odd last step: the loop has no exit between its two steps, so on every path
  // into a step of set 0 the loads of set 1 are the newer ones
  const int nsteps = kend > kbeg ? (kend - kbeg + GK - 1) / GK : 0;
  int k0 = kbeg;
  for (int p = 0; p < nsteps / 2; ++p, k0 += 2 * GK) {
    step(va0, vb0, k0);
    step(va1, vb1, k0 + GK);
  }
  if (nsteps & 1) step(va0, vb0, k0);
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + (BM / 2) * wm + 16 * i + 4 * gq + r;
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + 64 * wn + 16 * j + li;
        float* p = C + (long long)m * g.sCm + n;
        *p = acc[i][j][r];
      }
    }
}

template <typename TA, typename TB, bool ATR, bool BTR, int BM>
__global__ __launch_bounds__(256, 2) void sw_gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * PLANE_BYTES];
  gemm_tile<TA, TB, ATR, BTR, BM>(g, blockIdx.x, blockIdx.y, blockIdx.z, lds);
}

// Up to four independent products of the same orientation and tile height in one launch: workgroups
// [first[i], first[i + 1]) compute product i (grid gx[i] x gy[i] x batch splits), so that no product's
// tail leaves compute units idle and the group costs one launch.
constexpr int GEMM_GROUP = 4;
struct GemmGroup {
  GemmArgs g[GEMM_GROUP];
  int first[GEMM_GROUP + 1];
  int gx[GEMM_GROUP], gy[GEMM_GROUP];
};
template <typename TA, typename TB, bool ATR, bool BTR, int BM>
__global__ __launch_bounds__(256, 2) void sw_gemmg_kernel(GemmGroup G) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * PLANE_BYTES];
  const int b = blockIdx.x;
#pragma unroll
  for (int i = 0; i < GEMM_GROUP; ++i) {
    if (b >= G.first[i] && b < G.first[i + 1]) {   // uniform over the workgroup
      const int lb = b - G.first[i];
      gemm_tile<TA, TB, ATR, BTR, BM>(G.g[i], lb % G.gx[i], (lb / G.gx[i]) % G.gy[i], lb / (G.gx[i] * G.gy[i]), lds);
      return;
    }
  }
}

template <typename TA, typename TB, int BM>
void gemm_launch(const GemmArgs& g, dim3 grid, bool atr, bool btr, hipStream_t stream) {
  if (atr && btr)
    hipLaunchKernelGGL((sw_gemm_kernel<TA, TB, true, true, BM>), grid, dim3(256), 0, stream, g);
  else if (atr)
    hipLaunchKernelGGL((sw_gemm_kernel<TA, TB, true, false, BM>), grid, dim3(256), 0, stream, g);
  else if (btr)
    hipLaunchKernelGGL((sw_gemm_kernel<TA, TB, false, true, BM>), grid, dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL((sw_gemm_kernel<TA, TB, false, false, BM>), grid, dim3(256), 0, stream, g);
}

// Launch with the operand orientations taken from the strides; nsplit > 1 splits the contraction into
// pieces of kper (a multiple of GK) whose partial products go to C + s bCs.  Products with few column tiles
// use 64-row tiles, so that the grid still has several workgroups per CU.
// Orientation, tile height and grid of a product (nsplit and bCs folded into g); false if its shape does not
// fit the kernel.
struct GemmPlan {
  bool atr, btr;
  int bm;
  dim3 grid;
};
static bool gemm_plan(GemmArgs& g, int batch, int nsplit, long long bCs, GemmPlan& pl) {
  pl.atr = g.sAk != 1;
  pl.btr = g.sBk != 1;
  pl.bm = (!pl.atr && g.N <= GT) ? 64 : GT;
  // the contiguous extent of each operand must be whole tiles (or whole k steps)
  if ((pl.atr ? (g.sAm != 1 || g.M % pl.bm) : (g.K % GK)) || (pl.btr ? (g.sBn != 1 || g.N % GT) : (g.K % GK)) ||
      g.N % GT)
    return false;
  if (nsplit < 1) nsplit = 1;
  g.kper = (((g.K + nsplit - 1) / nsplit) + GK - 1) / GK * GK;
  g.nsplit = nsplit;
  g.bCs = bCs;
  pl.grid = dim3((unsigned)(g.N / GT), (unsigned)((g.M + pl.bm - 1) / pl.bm), (unsigned)(batch * nsplit));
  return true;
}

template <typename TA, typename TB>
hipError_t gemm(GemmArgs g, int batch, hipStream_t stream, int nsplit = 1, long long bCs = 0) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  GemmPlan pl;
  if (!gemm_plan(g, batch, nsplit, bCs, pl)) return hipErrorInvalidValue;
  const bool atr = pl.atr, btr = pl.btr;
  const int bm = pl.bm;
  const dim3 grid = pl.grid;
  if (bm == 64)
    gemm_launch<TA, TB, 64>(g, grid, atr, btr, stream);
  else
    gemm_launch<TA, TB, GT>(g, grid, atr, btr, stream);
  return hipGetLastError();
}

// Independent products (at most GEMM_GROUP) in one launch when they all have both operands transposed and
// 128-row tiles, else one launch each.
struct GemmJob {
  GemmArgs g;
  int batch, nsplit;
  long long bCs;
};
template <typename TA, typename TB>
hipError_t gemm_group(const GemmJob* jobs, int n, hipStream_t stream) {
  GemmGroup G;
  int m = 0;
  long long total = 0;
  bool one_launch = n <= GEMM_GROUP;
  for (int i = 0; i < n && one_launch; ++i) {
    GemmArgs h = jobs[i].g;
    if (h.M <= 0 || h.N <= 0) continue;
    GemmPlan pl;
    if (!gemm_plan(h, jobs[i].batch, jobs[i].nsplit, jobs[i].bCs, pl)) return hipErrorInvalidValue;
    if (!pl.atr || !pl.btr || pl.bm != GT) {
      one_launch = false;
      break;
    }
    G.g[m] = h;
    G.first[m] = (int)total;
    G.gx[m] = (int)pl.grid.x;
    G.gy[m] = (int)pl.grid.y;
    total += (long long)pl.grid.x * pl.grid.y * pl.grid.z;
    ++m;
  }
  if (!one_launch || total > INT32_MAX) {
    for (int i = 0; i < n; ++i) {
      const hipError_t e = gemm<TA, TB>(jobs[i].g, jobs[i].batch, stream, jobs[i].nsplit, jobs[i].bCs);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (m == 0) return hipSuccess;
  for (int i = m; i <= GEMM_GROUP; ++i) G.first[i] = (int)total;   // empty ranges
  for (int i = m; i < GEMM_GROUP; ++i) {
    G.g[i] = G.g[0];
    G.gx[i] = G.gy[i] = 1;
  }
  hipLaunchKernelGGL((sw_gemmg_kernel<TA, TB, true, true, GT>), dim3((unsigned)total), dim3(256), 0, stream, G);
  return hipGetLastError();
}

__device__ __forceinline__ float sigm(float a) { return 1.0f / (1.0f + expf(-a)); }

// Column of the concatenated step operand Wcat ([d][1024] per head) holding part p (0: the weights, 1: their
// tangents dU) of matrix m (0: W1, 1: W3) at hidden unit u: 16-unit slices of 64 columns (W1, W3, dU1, dU3).
__device__ __forceinline__ int wcat_col(int p, int m, int u) { return (u >> 4) * 64 + (2 * p + m) * 16 + (u & 15); }
// A bf16 store into a buffer: a store past the buffer's end is dropped, so the factor stores of a tile's
// ragged last rows need no branch (branches around stores keep the compiler from counting them, and it
// would then wait for every store before each load of the next weight slice).
__device__ __forceinline__ void st_bf16(__amdgpu_buffer_rsrc_t r, unsigned off, float x) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16)x), r, off, 0, 0);
}
// Column of E1a ([t][512]: eta Pa, eta Pb) and of J13 = K^T E1a ([d][512]) for matrix m at unit u.
__device__ __forceinline__ int j13_col(int m, int u) { return (u >> 4) * 32 + m * 16 + (u & 15); }

// ---------------------------------------------------------------------------
// The step's vector-Jacobian product for a 128-token tile of one head, all of
// it but the two products that contract over the chunk's tokens (K^T E1a and
// E3^T V): 8 waves of 16 tokens each; the 256 hidden units are visited in 16
// slices of 16, and per slice
//   Z1 = k [W1 | W3 | dU1 | dU3]_slice (a, b, adot, bdot: 64 columns),
//   Z2 = v [W2 ; dU2]_slice^T (g, r: 32 columns),
//   the elementwise factors eta Pa, eta Pb, eta Padot, eta Pbdot, hdot, h,
//   E1a = (eta Pa, eta Pb) and E3 = eta hdot to memory (for the weight
//   gradient), and
//   dK += [eta Pa | eta Pb | eta Padot | eta Pbdot] [W1 | W3 | dU1 | dU3]_slice^T,
//   ydot += [hdot | h] [W2 ; dU2]_slice,
// then dK, dV = eta ydot and deta = <ydot, v> are written.  The k and v rows
// of a wave's tokens stay in registers as MFMA operands for all slices; a
// slice's weights (fp32) are staged once per workgroup as bf16 hi + lo planes
// that serve both products they enter ([d][64 columns] read transposed for Z1
// and directly for dK; [32 rows][d] read directly for Z2 and transposed for
// ydot), the next slice's loaded into registers meanwhile; a wave's factors
// pass through its own LDS planes ([column][token], read transposed as the A
// operand), so the slice needs no barrier between its two halves.
// ---------------------------------------------------------------------------
struct StepArgs {
  const bf16* K;        // [BH][T][d], offset to the chunk
  const bf16* V;
  const float* eta;     // [BH][T]
  const float* Wcat;    // [BH][d][1024] (wcat_col order)
  const float* W2cat;   // [BH][2 d_h][d]
  bf16* E1a;            // [BH][cap][512] (j13_col order)
  bf16* E3;             // [BH][cap][d_h]
  float* dK;            // [BH][T][d], offset to the chunk
  float* dV;
  float* deta;          // [BH][T], offset to the chunk
  int T, c0, Cc;
  long long cap;
};
constexpr int ST_WAVES = 8, ST_TOK = 16 * ST_WAVES, ST_NT = 64 * ST_WAVES;
constexpr int ST_WC_ROW = 64 * 2 + 32;         // [d][64 columns] bf16 plane row: 160 bytes
constexpr int ST_W2_ROW = BD * 2 + 32;         // [32 rows][d] plane row: 288 bytes
constexpr int ST_WC_PLANE = BD * ST_WC_ROW;    // 20480
constexpr int ST_W2_PLANE = 32 * ST_W2_ROW;    // 9216
constexpr int ST_E1_PLANE = 64 * 32;           // [64 columns][16 tokens] bf16
constexpr int ST_E2_PLANE = 32 * 32;           // [32 rows][16 tokens]
constexpr int ST_WAVE_BYTES = 2 * ST_E1_PLANE + 2 * ST_E2_PLANE;
constexpr int ST_LDS = 2 * ST_WC_PLANE + 2 * ST_W2_PLANE + ST_WAVES * ST_WAVE_BYTES;   // 108544

// Transposed fragment (rows m = rb + l % 16 of the MFMA operand, k = 8 (l / 16) .. + 7) of a [k][m] plane.
__device__ __forceinline__ bf16x8 frag_tr(const unsigned char* plane, int row_bytes, int k0, int rb) {
  const int l = threadIdx.x & 63, g = l >> 4, i = l & 15;
  const unsigned char* p = plane + (k0 + 8 * g + (i >> 2)) * row_bytes + (rb + 4 * (i & 3)) * 2;
  const bf16x4 x = lds_read_tr16(p), y = lds_read_tr16(p + 4 * row_bytes);
  return bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}
// Direct fragment (rows rb + l % 16, k = k0 + 8 (l / 16) .. + 7) of a [m][k] plane.
__device__ __forceinline__ bf16x8 frag_dir(const unsigned char* plane, int row_bytes, int k0, int rb) {
  const int l = threadIdx.x & 63, g = l >> 4, i = l & 15;
  return *(const bf16x8*)(plane + (rb + i) * row_bytes + (k0 + 8 * g) * 2);
}

__global__ __launch_bounds__(ST_WAVES * 64, 1) void sw_bwd_step_kernel(StepArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char st_lds[];
  unsigned char* wch = st_lds;
  unsigned char* wcl = wch + ST_WC_PLANE;
  unsigned char* w2h = wcl + ST_WC_PLANE;
  unsigned char* w2l = w2h + ST_W2_PLANE;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, gq = l >> 4, li = l & 15;
  unsigned char* e1h = w2l + ST_W2_PLANE + w * ST_WAVE_BYTES;
  unsigned char* e1l = e1h + ST_E1_PLANE;
  unsigned char* e2h = e1l + ST_E1_PLANE;
  unsigned char* e2l = e2h + ST_E2_PLANE;
  const long long bh = blockIdx.y;
  const int t0 = blockIdx.x * ST_TOK + 16 * w;     // this wave's first token (chunk-relative)
  const int Cc = a.Cc;
  const float* Wc = a.Wcat + bh * BD * 4 * BDH;
  const float* W2 = a.W2cat + bh * 2 * BP;
  const long long trow = bh * (long long)a.T;      // row of token 0 of the chunk in [BH][T]
  // k and v rows of the wave's tokens as MFMA A operands (row li, d = 32 ks + 8 gq ..)
  bf16x8 kf[4], vf[4];
  {
    const int t = t0 + li;
    const bool ok = t < Cc;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const long long o = (trow + t) * BD + 32 * ks + 8 * gq;
      kf[ks] = ok ? *(const bf16x8*)(a.K + o) : bf16x8{};
      vf[ks] = ok ? *(const bf16x8*)(a.V + o) : bf16x8{};
    }
  }
  float er[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = t0 + 4 * gq + r;
    er[r] = t < Cc ? a.eta[trow + a.c0 + t] : 0.f;
  }
  // a slice's weights: Wcat [d][64 columns] (4 pieces of 4 floats per thread), W2cat 32 rows (2 pieces)
  u32x4 pw[4], p2[2];
  auto load = [&](int s) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 512 * q, d = idx >> 4, pc = idx & 15;
      pw[q] = *(const u32x4*)(Wc + (long long)d * 4 * BDH + 64 * s + 4 * pc);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = tid + 512 * q, row = idx >> 5, pc = idx & 31;
      const int srow = (row >> 4) * BDH + 16 * s + (row & 15);
      p2[q] = *(const u32x4*)(W2 + (long long)srow * BD + 4 * pc);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 512 * q, d = idx >> 4, pc = idx & 15;
      const floatx4 f = __builtin_bit_cast(floatx4, pw[q]);
      const uint2 s0 = split2(f[0], f[1]), s1 = split2(f[2], f[3]);
      *(uint2*)(wch + d * ST_WC_ROW + pc * 8) = uint2{s0.x, s1.x};
      *(uint2*)(wcl + d * ST_WC_ROW + pc * 8) = uint2{s0.y, s1.y};
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = tid + 512 * q, row = idx >> 5, pc = idx & 31;
      const floatx4 f = __builtin_bit_cast(floatx4, p2[q]);
      const uint2 s0 = split2(f[0], f[1]), s1 = split2(f[2], f[3]);
      *(uint2*)(w2h + row * ST_W2_ROW + pc * 8) = uint2{s0.x, s1.x};
      *(uint2*)(w2l + row * ST_W2_ROW + pc * 8) = uint2{s0.y, s1.y};
    }
  };
  floatx4 dk[8], yd[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) dk[j] = yd[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  constexpr int NSLICE = BDH / 16;
  load(0);
  store();
  load(1);
  __syncthreads();
  for (int s = 0; s < NSLICE; ++s) {
    // Z1 (a, b, adot, bdot) and Z2 (g, r) of the wave's 16 tokens and the slice's 16 units
    floatx4 z1[4], z2[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) z1[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    z2[0] = z2[1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        z1[j] = mfma16(kf[ks], frag_tr(wch, ST_WC_ROW, 32 * ks, 16 * j), z1[j]);
        z1[j] = mfma16(kf[ks], frag_tr(wcl, ST_WC_ROW, 32 * ks, 16 * j), z1[j]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        z2[j] = mfma16(vf[ks], frag_dir(w2h, ST_W2_ROW, 32 * ks, 16 * j), z2[j]);
        z2[j] = mfma16(vf[ks], frag_dir(w2l, ST_W2_ROW, 32 * ks, 16 * j), z2[j]);
      }
    }
    // the elementwise factors: lane (gq, li) holds tokens t0 + 4 gq + r of unit 16 s + li
    const int u = 16 * s + li;
    float f1[4][4], f2[2][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float av = z1[0][r], bv = z1[1][r], ad = z1[2][r], bd = z1[3][r], gg = z2[0][r], rr = z2[1][r];
      const float e = er[r];
      const float sg = sigm(av), sv = av * sg, s1 = sg * (1.0f + av * (1.0f - sg));
      const float s2 = sg * (1.0f - sg) * (2.0f + av * (1.0f - 2.0f * sg));
      const float hd = s1 * ad * bv + sv * bd;
      f1[0][r] = e * (s2 * ad * bv * gg + s1 * (bd * gg + bv * rr));
      f1[1][r] = e * (s1 * ad * gg + sv * rr);
      f1[2][r] = e * (s1 * bv * gg);
      f1[3][r] = e * (sv * gg);
      f2[0][r] = hd;
      f2[1][r] = sv * bv;
      const int t = t0 + 4 * gq + r;
      if (t < Cc) {
        const long long orow = bh * a.cap + t;
        a.E1a[orow * 2 * BDH + j13_col(0, u)] = (bf16)f1[0][r];
        a.E1a[orow * 2 * BDH + j13_col(1, u)] = (bf16)f1[1][r];
        a.E3[orow * BDH + u] = (bf16)(e * hd);
      }
    }
    // the factors into the wave's [column][token] planes (4 consecutive tokens per lane and column)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint2 s0 = split2(f1[q][0], f1[q][1]), s1 = split2(f1[q][2], f1[q][3]);
      const int off = (16 * q + li) * 32 + 8 * gq;
      *(uint2*)(e1h + off) = uint2{s0.x, s1.x};
      *(uint2*)(e1l + off) = uint2{s0.y, s1.y};
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint2 s0 = split2(f2[q][0], f2[q][1]), s1 = split2(f2[q][2], f2[q][3]);
      const int off = (16 * q + li) * 32 + 8 * gq;
      *(uint2*)(e2h + off) = uint2{s0.x, s1.x};
      *(uint2*)(e2l + off) = uint2{s0.y, s1.y};
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    // dK += E1 Wcat_slice^T (k = the slice's 64 columns), ydot += E2 W2cat_slice (k = its 32 rows)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 ah = frag_tr(e1h, 32, 32 * ks, 0), al = frag_tr(e1l, 32, 32 * ks, 0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bf16x8 bh = frag_dir(wch, ST_WC_ROW, 32 * ks, 16 * j), bl = frag_dir(wcl, ST_WC_ROW, 32 * ks, 16 * j);
        dk[j] = mfma16(ah, bh, dk[j]);
        dk[j] = mfma16(ah, bl, dk[j]);
        dk[j] = mfma16(al, bh, dk[j]);
      }
    }
    {
      const bf16x8 ah = frag_tr(e2h, 32, 0, 0), al = frag_tr(e2l, 32, 0, 0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bf16x8 bh = frag_tr(w2h, ST_W2_ROW, 0, 16 * j), bl = frag_tr(w2l, ST_W2_ROW, 0, 16 * j);
        yd[j] = mfma16(ah, bh, yd[j]);
        yd[j] = mfma16(ah, bl, yd[j]);
        yd[j] = mfma16(al, bh, yd[j]);
      }
    }
    __syncthreads();                 // every wave is done with the slice's weight planes
    if (s + 1 < NSLICE) {
      store();
      // unconditional (the last slice again at the end, unused), so that the loads in flight are the
      // same on every path and the wait for them does not also wait for the factor stores
      load(s + 2 < NSLICE ? s + 2 : NSLICE - 1);
      __syncthreads();
    }
  }
  // dK, dV = eta ydot, deta = <ydot, v>: lane (gq, li) holds tokens t0 + 4 gq + r, d = 16 j + li
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = t0 + 4 * gq + r;
    const bool ok = t < Cc;
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int d = 16 * j + li;
      if (ok) {
        const long long o = (trow + t) * BD + d;
        a.dK[o] = dk[j][r];
        a.dV[o] = er[r] * yd[j][r];
        dot += yd[j][r] * (float)a.V[o];
      }
    }
    dot += __shfl_xor(dot, 1);
    dot += __shfl_xor(dot, 2);
    dot += __shfl_xor(dot, 4);
    dot += __shfl_xor(dot, 8);
    if (ok && li == 0) a.deta[trow + t] = dot;
  }
}

// ---------------------------------------------------------------------------
// The read's gradients for a 128-token tile of one head at read weights R
// (packed W1 | W3 | W2): 8 waves of 16 tokens, the 256 hidden units in 16
// slices of 16, and per slice
//   a = q R1_slice, b = q R3_slice (32 columns), dh = dO R2_slice^T (16),
//   da = dh b silu'(a), db = dh silu(a), h = silu(a) b,
//   Eq = (da, db) and Hq = h to memory (the operands of the weight terms
//   Q^T Eq and Hq^T dO), and dQ += [da | db] [R1 | R3]_slice^T,
// then dQ is written.  Structure as sw_bwd_step_kernel: q and dO rows in
// registers, the slice's weights staged once per workgroup as bf16 hi + lo
// planes ([d][32 columns]: read transposed for a, b and directly for dQ;
// [16 rows][d] read directly for dh), each wave's factors through its own
// [column][token] planes.
// ---------------------------------------------------------------------------
struct ReadStepArgs {
  const bf16* Q;        // [BH][T][d], offset to the chunk
  const bf16* dO;
  const float* R;       // read weights, per head + bh * sR
  long long sR;
  bf16* Eq;             // [BH][cap][2 d_h]
  bf16* Hq;             // [BH][cap][d_h]
  float* dQ;            // [BH][T][d], offset to the chunk
  int T, Cc;
  long long cap;
};
constexpr int RS_W13_ROW = 32 * 2 + 32;         // [d][32 columns] bf16 plane row: 96 bytes
constexpr int RS_W13_PLANE = BD * RS_W13_ROW;   // 12288
constexpr int RS_W2_PLANE = 16 * ST_W2_ROW;     // [16 rows][d]: 4608
constexpr int RS_E_PLANE = 32 * 32;             // [32 columns][16 tokens] bf16
constexpr int RS_WAVE_BYTES = 2 * RS_E_PLANE;
constexpr int RS_LDS = 2 * RS_W13_PLANE + 2 * RS_W2_PLANE + ST_WAVES * RS_WAVE_BYTES;   // 50176
constexpr int RS_PW = BD * 32 / 4 / ST_NT, RS_P2 = 16 * BD / 4 / ST_NT;               // 16-byte pieces per thread

__global__ __launch_bounds__(ST_NT, 1) void sw_bwd_read_step_kernel(ReadStepArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[RS_LDS];
  unsigned char* wh = lds;
  unsigned char* wl = wh + RS_W13_PLANE;
  unsigned char* w2h = wl + RS_W13_PLANE;
  unsigned char* w2l = w2h + RS_W2_PLANE;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, gq = l >> 4, li = l & 15;
  unsigned char* eh = w2l + RS_W2_PLANE + w * RS_WAVE_BYTES;
  unsigned char* el = eh + RS_E_PLANE;
  const long long bh = blockIdx.y;
  const int t0 = blockIdx.x * ST_TOK + 16 * w;
  const int Cc = a.Cc;
  const float* R = a.R + bh * a.sR;
  const long long trow = bh * (long long)a.T;
  const __amdgpu_buffer_rsrc_t req = make_rsrc(a.Eq + bh * a.cap * 2 * BDH, (long long)Cc * 2 * BDH * 2);
  const __amdgpu_buffer_rsrc_t rhq = make_rsrc(a.Hq + bh * a.cap * BDH, (long long)Cc * BDH * 2);
  bf16x8 qf[4], of[4];
  {
    const int t = t0 + li;
    const bool ok = t < Cc;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const long long o = (trow + t) * BD + 32 * ks + 8 * gq;
      qf[ks] = ok ? *(const bf16x8*)(a.Q + o) : bf16x8{};
      of[ks] = ok ? *(const bf16x8*)(a.dO + o) : bf16x8{};
    }
  }
  // a slice's weights: R1, R3 columns 16 s .. 16 s + 15 ([d][32 columns]: 8 pieces of 4 floats per d), R2 rows
  // 16 s .. 16 s + 15 (32 pieces each)
  u32x4 pw[RS_PW], p2[RS_P2];
  auto load = [&](int s) {
#pragma unroll
    for (int q = 0; q < RS_PW; ++q) {
      const int idx = tid + ST_NT * q, d = idx >> 3, pc = idx & 7;
      pw[q] = *(const u32x4*)(R + (long long)(pc >> 2) * BP + (long long)d * BDH + 16 * s + 4 * (pc & 3));
    }
#pragma unroll
    for (int q = 0; q < RS_P2; ++q) {
      const int idx = tid + ST_NT * q, row = idx >> 5, pc = idx & 31;
      p2[q] = *(const u32x4*)(R + 2 * BP + (long long)(16 * s + row) * BD + 4 * pc);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int q = 0; q < RS_PW; ++q) {
      const int idx = tid + ST_NT * q, d = idx >> 3, pc = idx & 7;
      const floatx4 f = __builtin_bit_cast(floatx4, pw[q]);
      const uint2 s0 = split2(f[0], f[1]), s1 = split2(f[2], f[3]);
      *(uint2*)(wh + d * RS_W13_ROW + pc * 8) = uint2{s0.x, s1.x};
      *(uint2*)(wl + d * RS_W13_ROW + pc * 8) = uint2{s0.y, s1.y};
    }
#pragma unroll
    for (int q = 0; q < RS_P2; ++q) {
      const int idx = tid + ST_NT * q, row = idx >> 5, pc = idx & 31;
      const floatx4 f = __builtin_bit_cast(floatx4, p2[q]);
      const uint2 s0 = split2(f[0], f[1]), s1 = split2(f[2], f[3]);
      *(uint2*)(w2h + row * ST_W2_ROW + pc * 8) = uint2{s0.x, s1.x};
      *(uint2*)(w2l + row * ST_W2_ROW + pc * 8) = uint2{s0.y, s1.y};
    }
  };
  floatx4 dq[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) dq[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  constexpr int NSLICE = BDH / 16;
  load(0);
  store();
  load(1);
  __syncthreads();
  for (int s = 0; s < NSLICE; ++s) {
    floatx4 z1[2], z2 = {0.f, 0.f, 0.f, 0.f};
    z1[0] = z1[1] = z2;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        z1[j] = mfma16(qf[ks], frag_tr(wh, RS_W13_ROW, 32 * ks, 16 * j), z1[j]);
        z1[j] = mfma16(qf[ks], frag_tr(wl, RS_W13_ROW, 32 * ks, 16 * j), z1[j]);
      }
      z2 = mfma16(of[ks], frag_dir(w2h, ST_W2_ROW, 32 * ks, 0), z2);
      z2 = mfma16(of[ks], frag_dir(w2l, ST_W2_ROW, 32 * ks, 0), z2);
    }
    // the elementwise step: lane (gq, li) holds tokens t0 + 4 gq + r of unit 16 s + li
    const int u = 16 * s + li;
    float f1[2][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float av = z1[0][r], bv = z1[1][r], dh = z2[r];
      const float sg = sigm(av), sv = av * sg, s1 = sg * (1.0f + av * (1.0f - sg));
      f1[0][r] = dh * bv * s1;
      f1[1][r] = dh * sv;
      const int t = t0 + 4 * gq + r;   // rows past Cc fall outside the buffers: their stores are dropped
      st_bf16(req, (unsigned)((t * 2 * BDH + u) * 2), f1[0][r]);
      st_bf16(req, (unsigned)((t * 2 * BDH + BDH + u) * 2), f1[1][r]);
      st_bf16(rhq, (unsigned)((t * BDH + u) * 2), sv * bv);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint2 s0 = split2(f1[q][0], f1[q][1]), s1 = split2(f1[q][2], f1[q][3]);
      const int off = (16 * q + li) * 32 + 8 * gq;
      *(uint2*)(eh + off) = uint2{s0.x, s1.x};
      *(uint2*)(el + off) = uint2{s0.y, s1.y};
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    // dQ += [da | db] [R1 | R3]_slice^T (k = the slice's 32 columns)
    {
      const bf16x8 ah = frag_tr(eh, 32, 0, 0), al = frag_tr(el, 32, 0, 0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bf16x8 bh = frag_dir(wh, RS_W13_ROW, 0, 16 * j), bl = frag_dir(wl, RS_W13_ROW, 0, 16 * j);
        dq[j] = mfma16(ah, bh, dq[j]);
        dq[j] = mfma16(ah, bl, dq[j]);
        dq[j] = mfma16(al, bh, dq[j]);
      }
    }
    __syncthreads();                 // every wave is done with the slice's weight planes
    if (s + 1 < NSLICE) {
      store();
      // unconditional (the last slice again at the end, unused), so that the loads in flight are the
      // same on every path and the wait for them does not also wait for the factor stores
      load(s + 2 < NSLICE ? s + 2 : NSLICE - 1);
      __syncthreads();
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = t0 + 4 * gq + r;
    if (t < Cc) {
#pragma unroll
      for (int j = 0; j < 8; ++j) a.dQ[(trow + t) * BD + 16 * j + li] = dq[j][r];
    }
  }
}

// Per head: the normalisation's backward dU of G (packed W1 | W3 | W2) at the chunk's normalised weights Wc and
// norms nrm, and the step's operands at the weights before it (Wp): Wcat [d][1024] in wcat_col order (part 0:
// W1, W3; part 1: dU1, dU3), W2cat [W2 ; dU2] (2 d_h x d).  Block (matrix m, group of 16 columns): 64 row
// groups x 4 column quads, each thread holding 4 columns (16-byte accesses) of 2 rows of W1 / W3 or 4 rows of
// W2 and summing w . G over them; the 64 partials of a column are added in a fixed order through LDS.
// Norm columns: 0..255 W1, 256..511 W3, 512..639 W2.  last_only: dU1 = dU3 = 0, dU2 = G2.
__global__ __launch_bounds__(256) void sw_bwd_prep(const float* __restrict__ G, const float* __restrict__ Wc,
                                                   long long wc_stride, const float* __restrict__ nrm,
                                                   long long nrm_stride, const float* __restrict__ Wp,
                                                   long long wp_stride, float* __restrict__ Wcat,
                                                   float* __restrict__ W2cat, int last_only) {
  __shared__ float part[64][17];
  __shared__ float dots[16];
  const long long h = blockIdx.y;
  const int grp = blockIdx.x, m = grp < 16 ? 0 : grp < 32 ? 1 : 2;
  const int cq = threadIdx.x & 3, rg = threadIdx.x >> 2;      // column quad, row group
  const int col0 = (m < 2 ? (grp & 15) : grp - 32) * 16, col = col0 + 4 * cq;
  const int ld = m < 2 ? BDH : BD;
  constexpr int PER_MAX = 4;
  const int per = m < 2 ? BD / 64 : BDH / 64;                 // rows per thread: 2 or 4
  const long long base = (long long)m * BP;
  const float* g = G + h * 3 * BP + base;
  const float* wc = Wc + h * wc_stride + base;
  const float* wp = Wp + h * wp_stride + base;
  floatx4 gv[PER_MAX], wv[PER_MAX];
  floatx4 dot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < PER_MAX; ++k)
    if (k < per) {
      const long long o = (long long)(rg + 64 * k) * ld + col;
      gv[k] = *(const floatx4*)(g + o);
      wv[k] = *(const floatx4*)(wc + o);
      dot += gv[k] * wv[k];
    }
#pragma unroll
  for (int j = 0; j < 4; ++j) part[rg][4 * cq + j] = dot[j];
  __syncthreads();
  if (threadIdx.x < 16) {
    float x = 0.f;
    for (int r = 0; r < 64; ++r) x += part[r][threadIdx.x];
    dots[threadIdx.x] = x;
  }
  __syncthreads();
  floatx4 dt, n;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    dt[j] = dots[4 * cq + j];
    n[j] = nrm[h * nrm_stride + (m < 2 ? m * BDH : 2 * BDH) + col + j];
  }
  float* wcat = Wcat + h * BD * 4 * BDH;
  float* w2cat = W2cat + h * 2 * BP;
#pragma unroll
  for (int k = 0; k < PER_MAX; ++k)
    if (k < per) {
      const int r = rg + 64 * k;
      const long long o = (long long)r * ld + col;
      floatx4 du;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        du[j] = n[j] > BNORM_EPS ? (gv[k][j] - wv[k][j] * dt[j]) / n[j] : gv[k][j] / BNORM_EPS;
      const floatx4 w0 = *(const floatx4*)(wp + o);
      if (m < 2) {
        if (last_only) du = floatx4{0.f, 0.f, 0.f, 0.f};
        *(floatx4*)(wcat + (long long)r * 4 * BDH + wcat_col(0, m, col)) = w0;
        *(floatx4*)(wcat + (long long)r * 4 * BDH + wcat_col(1, m, col)) = du;
      } else {
        if (last_only) du = gv[k];
        *(floatx4*)(w2cat + o) = w0;
        *(floatx4*)(w2cat + BP + o) = du;
      }
    }
}

// G (packed W1 | W3 | W2 per head) from the chunk's terms, each the sum of its split partials in a fixed order
// (J13: s13 partials of [BH][d][2 d_h] in j13_col order; A13: s13 partials of [BH][d][W1 part | W3
// part]; J2, A2: s2 partials of [BH][d_h][d]); four consecutive elements per thread:
//   add_read_only: G += A (the read's weight gradient);
//   otherwise: G = base + J (+ A when with_read), base = dU (from Wcat / W2cat) for an updated matrix, G
//   itself for a matrix the loop does not update (W1, W3 in the last-layer mode).
__global__ __launch_bounds__(256) void sw_bwd_gupdate(float* __restrict__ G, const float* __restrict__ Wcat,
                                                      const float* __restrict__ W2cat, const float* __restrict__ J13,
                                                      const float* __restrict__ J2, const float* __restrict__ A13,
                                                      const float* __restrict__ A2, int s13, int s2,
                                                      int add_read_only, int with_read, int last_only) {
  const long long h = blockIdx.y, BH = gridDim.y;
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= 3 * BP) return;
  floatx4* g = (floatx4*)(G + h * 3 * BP + i);
  auto psum = [](const float* P, int n, long long stride, long long off) {
    floatx4 x = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < n; ++s) x += *(const floatx4*)(P + s * stride + off);
    return x;
  };
  floatx4 av = {0.f, 0.f, 0.f, 0.f}, jv, base;
  if (i < 2 * BP) {
    const int m = (int)(i / BP);
    const long long k = i % BP, d = k / BDH;
    const int u = (int)(k % BDH);
    const long long stride = BH * BD * 2 * BDH, hoff = h * BD * 2 * BDH + d * 2 * BDH;
    if (A13) av = psum(A13, s13, stride, hoff + m * BDH + u);
    if (add_read_only) {
      *g += av;
      return;
    }
    jv = psum(J13, s13, stride, hoff + j13_col(m, u));
    base = last_only ? *g : *(const floatx4*)(Wcat + h * BD * 4 * BDH + d * 4 * BDH + wcat_col(1, m, u));
  } else {
    const long long k = i - 2 * BP;
    if (A2) av = psum(A2, s2, BH * BP, h * BP + k);
    if (add_read_only) {
      *g += av;
      return;
    }
    jv = psum(J2, s2, BH * BP, h * BP + k);
    base = *(const floatx4*)(W2cat + h * 2 * BP + BP + k);
  }
  *g = base + jv + (with_read ? av : floatx4{0.f, 0.f, 0.f, 0.f});
}

__global__ __launch_bounds__(256) void sw_bwd_copy(float* __restrict__ dst, const float* __restrict__ src, long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

struct BwdSwLayout {
  size_t fws, wfin, dump, dnorm, wcat, w2cat, e1, eq, e2, e3, j13, j2, a13, a2, total;
};
size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
// Split of the products that contract over a chunk's tokens: enough workgroups (about 256) for the chip, at
// least 128 tokens per split, at most 16 splits.
int token_split(int tiles_per_head, int64_t BH, int64_t Cc) {
  const int64_t want = 256 / std::max<int64_t>(1, tiles_per_head * BH);
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
  L.e1 = o; o += al256((size_t)BH * Cc * 2 * BDH * 2);     // E1a (bf16)
  L.eq = o; o += al256((size_t)BH * Cc * 2 * BDH * 2);     // the read's Eq (bf16)
  L.e2 = o; o += al256((size_t)BH * Cc * BDH * 2);         // the read's Hq (bf16)
  L.e3 = o; o += al256((size_t)BH * Cc * BDH * 2);         // E3 (bf16)
  L.j13 = o; o += al256((size_t)s13 * BH * BD * 2 * BDH * 4);
  L.j2 = o; o += al256((size_t)s2 * BH * BP * 4);
  L.a13 = o; o += al256((size_t)s13 * BH * BD * 2 * BDH * 4);
  L.a2 = o; o += al256((size_t)s2 * BH * BP * 4);
  L.total = o;
  return L;
}

GemmArgs gargs(const void* A, long long sAm, long long sAk, long long bA, const void* B, long long sBk, long long sBn,
               long long bB, float* C, long long sCm, long long bC, int M, int N, int K) {
  GemmArgs g;
  g.A = A; g.B = B; g.C = C;
  g.M = M; g.N = N; g.K = K;
  g.sAm = sAm; g.sAk = sAk; g.sBk = sBk; g.sBn = sBn; g.sCm = sCm;
  g.bA = bA; g.bB = bB; g.bC = bC;
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
  bf16* E1 = (bf16*)(ws + L.e1);
  bf16* EQ = (bf16*)(ws + L.eq);
  bf16* E2 = (bf16*)(ws + L.e2);
  bf16* E3 = (bf16*)(ws + L.e3);
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

  if ((e = hipFuncSetAttribute((const void*)sw_bwd_step_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, ST_LDS)) !=
      hipSuccess)
    return e;
  const bool read_first = !a.other_order;
  // the read's two token-contraction products of a chunk: (Q^T da | Q^T db) and (silu(a) b)^T dO
  auto read_job13 = [&](long long c0, int Cc) {
    return GemmJob{gargs(Q + c0 * BD, 1, BD, T * BD, EQ, 2 * BDH, 1, cap * 2 * BDH, A13, 2 * BDH, BD * 2 * BDH, BD,
                         2 * BDH, Cc), BH, s13, p13};
  };
  auto read_job2 = [&](long long c0, int Cc) {
    return GemmJob{gargs(E2, 1, BDH, cap * BDH, dO + c0 * BD, BD, 1, T * BD, A2, BD, BP, BDH, BD, Cc), BH, s2, p2};
  };
  auto read_phase = [&](const float* R, long long rstride, long long c0, int Cc, bool with_products) -> hipError_t {
    hipError_t e2;
    const bf16* Qc = Q + c0 * BD;
    const bf16* dOc = dO + c0 * BD;
    bf16* Eq = EQ;     // [Cc][da | db]
    bf16* Hq = E2;     // [Cc][silu(a) b]      (E2's room)
    // the read's factors and dQ
    const ReadStepArgs ra{Qc, dOc, R, rstride, Eq, Hq, dQ + c0 * BD, (int)T, Cc, cap};
    hipLaunchKernelGGL(sw_bwd_read_step_kernel, dim3((unsigned)((Cc + ST_TOK - 1) / ST_TOK), BH), dim3(ST_NT), 0,
                       stream, ra);
    if ((e2 = hipGetLastError()) != hipSuccess) return e2;
    if (!with_products) return hipSuccess;
    // (Q^T da | Q^T db), (silu(a) b)^T dO
    const GemmJob jobs[2] = {read_job13(c0, Cc), read_job2(c0, Cc)};
    return gemm_group<bf16, bf16>(jobs, 2, stream);
  };

  for (int c = nch - 1; c >= 0; --c) {
    const long long c0 = (long long)c * C;
    const int Cc = (int)std::min<long long>(C, T - c0);
    const float* Wp = c == 0 ? a.W0 : dump + (long long)(c - 1) * SP;   // weights before the chunk
    const long long wp_stride = c == 0 ? SP : (long long)nch * SP;
    const float* Wc = dump + (long long)c * SP;                       // after it
    const long long wc_stride = (long long)nch * SP;
    if (!read_first) {   // the chunk's queries read W_c: their gradient reaches G before the normalisation
      if ((e = read_phase(Wc, wc_stride, c0, Cc, true)) != hipSuccess) return e;
      hipLaunchKernelGGL(sw_bwd_gupdate, dim3((unsigned)((3 * BP / 4 + 255) / 256), BH), dim3(256), 0, stream, G, Wcat,
                         W2cat, J13, J2, A13, A2, s13, s2, 1, 0, last_only);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sw_bwd_prep, dim3(40, BH), dim3(256), 0, stream, G, Wc, wc_stride, dnorm + (long long)c * 640,
                       (long long)nch * 640, Wp, wp_stride, Wcat, W2cat, last_only);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const bf16* Kc = K + c0 * BD;
    const bf16* Vc = V + c0 * BD;
    // the step's vector-Jacobian product except the weight terms: dK, dV, deta, and E1a, E3 for those
    const StepArgs sa{Kc, Vc, a.eta, Wcat, W2cat, E1, E3, dK + c0 * BD, dV + c0 * BD, a.deta + c0, (int)T, (int)c0, Cc,
                      cap};
    hipLaunchKernelGGL(sw_bwd_step_kernel, dim3((unsigned)((Cc + ST_TOK - 1) / ST_TOK), BH), dim3(ST_WAVES * 64),
                       ST_LDS, stream, sa);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // J13 = K^T (eta Pa | eta Pb), J2 = (eta hdot)^T V; with the read first, the read's factors are formed
    // before them and its two products join the same launch
    if (read_first && (e = read_phase(Wp, wp_stride, c0, Cc, false)) != hipSuccess) return e;
    const GemmJob jobs[4] = {
        {gargs(Kc, 1, BD, T * BD, E1, 2 * BDH, 1, cap * 2 * BDH, J13, 2 * BDH, BD * 2 * BDH, BD, 2 * BDH, Cc), BH, s13,
         p13},
        {gargs(E3, 1, BDH, cap * BDH, Vc, BD, 1, T * BD, J2, BD, BP, BDH, BD, Cc), BH, s2, p2},
        read_job13(c0, Cc), read_job2(c0, Cc)};
    if ((e = gemm_group<bf16, bf16>(jobs, read_first ? 4 : 2, stream)) != hipSuccess) return e;
    hipLaunchKernelGGL(sw_bwd_gupdate, dim3((unsigned)((3 * BP / 4 + 255) / 256), BH), dim3(256), 0, stream, G, Wcat, W2cat,
                       J13, J2, A13, A2, s13, s2, 0, read_first ? 1 : 0, last_only);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ttt
