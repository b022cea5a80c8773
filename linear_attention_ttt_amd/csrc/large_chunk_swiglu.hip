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
//  * swiglu_recur_kernel (cooperative, sequential over chunks): a head's
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
  float eta[SW_WAVES][2][SW_GT];
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

__global__ __launch_bounds__(SW_WAVES * 64, 1) void swiglu_recur_kernel(
    const bf16* __restrict__ K, const bf16* __restrict__ V, const float* __restrict__ eta,
    const float* __restrict__ W0, float* __restrict__ Wout, bf16* __restrict__ states, float* __restrict__ ss2,
    unsigned* __restrict__ counters, unsigned* __restrict__ errflag, int T_in, int chunk, int nchunks_in, int head0,
    int update_first, int last_only, int par_nchunks) {
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
  auto advance = [&](int& c, int& k) {       // next step of this wave (c == nchunks: none left)
    ++k;
    while (c < nchunks && k >= count(c)) {
      ++c;
      k = 0;
    }
  };
  auto group_of = [&](int c, int k) {
    (void)c;
    return w + SW_WAVES * k;
  };
  // per-lane byte offsets: direct-to-LDS rows (4 per load), row-wise operand reads (row 16tt + li,
  // piece 4ks + g) and transposed reads (rows 16tt + 4g .. + 3, columns 16m + li)
  unsigned dma_off[SW_STAGE / 1024];
#pragma unroll
  for (int j = 0; j < SW_STAGE / 1024; ++j) {
    const int row = 4 * j + (l >> 4);
    dma_off[j] = (unsigned)(row * SW_KROW + (((l & 15) ^ sw_swz(row)) << 4));
  }
  unsigned fwd_off[4], tr_off[8];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) fwd_off[ks] = (unsigned)(li * SW_KROW + (((4 * ks + g) ^ sw_swz(li)) << 4));
  const int trow = 4 * g + (li >> 2);
#pragma unroll
  for (int m = 0; m < 8; ++m)
    tr_off[m] = (unsigned)(trow * SW_KROW + (((2 * m + ((li >> 1) & 1)) ^ sw_swz(trow)) << 4) + (li & 1) * 8);

  auto issue = [&](int c, int gi, int slot) {
    const int t0 = c * chunk + gi * SW_GT;
    const int n = min(c * chunk + chunk, T) - t0;   // valid tokens; rows beyond read as 0
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + (size_t)t0 * D, (long long)n * SW_KROW);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh + (size_t)t0 * D, (long long)n * SW_KROW);
    const __amdgpu_buffer_rsrc_t re = make_rsrc(Eh + t0, (long long)n * 4);
#pragma unroll
    for (int j = 0; j < SW_STAGE / 1024; ++j) dma16<true>(rk, dma_off[j], S.kv[w][slot][0] + j * 1024);
#pragma unroll
    for (int j = 0; j < SW_STAGE / 1024; ++j) dma16<true>(rv, dma_off[j], S.kv[w][slot][1] + j * 1024);
    if (l < SW_GT) dma4<true>(re, (unsigned)(l * 4), S.eta[w][slot]);
  };

  bf16x8 w1op[4], w3op[4], w2op[4];
  floatx4 dW1[8], dW3[8], dW2[8];
  int ic = 0, ik = -1;                       // issue cursor: chunk, step within the chunk
  advance(ic, ik);
  int cc = ic, ck = ik;                      // compute cursor
  int step = 0;
  if (ic < nchunks) {
    issue(ic, group_of(ic, ik), 0);
    advance(ic, ik);
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

    for (; cc == c; advance(cc, ck), ++step) {
      const int slot = step & 1;
      // the next stage goes into the one read during the previous step; this step's stage has
      // landed once only the next stage's loads are outstanding
      if (ic < nchunks) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue(ic, group_of(ic, ik), slot ^ 1);
        advance(ic, ik);
        wait_vm<SW_LOADS>();
      } else {
        wait_vm<0>();
      }
      const unsigned char* kb = S.kv[w][slot][0];
      const unsigned char* vb = S.kv[w][slot][1];

      // ---- forward of the 32 tokens: A = K W1, B = K W3, Dh = V W2^T (rows: tokens 16tt + 4g + r) ----
      floatx4 A[2], Bv[2], Dh[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) A[tt] = Bv[tt] = Dh[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
      bf16x8 kop[4][2], vop[4][2];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          kop[ks][tt] = *(const bf16x8*)(kb + tt * 16 * SW_KROW + fwd_off[ks]);
          vop[ks][tt] = *(const bf16x8*)(vb + tt * 16 * SW_KROW + fwd_off[ks]);
        }
      // transposed operands of the gradient products (k slot (g, j) = token 16(j/4) + 4g + j%4),
      // read while the forward products run
      bf16x4 ktr[8][2], vtr[8][2];
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          ktr[m][tt] = lds_read_tr16(kb + tt * 16 * SW_KROW + tr_off[m]);
          vtr[m][tt] = lds_read_tr16(vb + tt * 16 * SW_KROW + tr_off[m]);
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
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const bf16x8 kt = join(ktr[m][0], ktr[m][1]);
        const bf16x8 vt = join(vtr[m][0], vtr[m][1]);
        if (!last_only) {
          dW1[m] = mfma16(kt, daop, dW1[m]);
          dW3[m] = mfma16(kt, dbop, dW3[m]);
        }
        dW2[m] = mfma16(ehop, vt, dW2[m]);
      }
    }

    // ---- end of chunk: the waves add their partial gradients in a fixed order, then normalise ----
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
      __hip_atomic_store(&ss2[(((size_t)bh * 2 + (c & 1)) * SW_NSL + sl) * D + d], ss, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      // The partial norms are the only data exchanged, and every access to them is a device-scope
      // atomic (coherent on its own).  Waiting for the stores to complete before the count goes up
      // orders them before it; release/acquire on the count would in addition write back and
      // invalidate the whole L2 at every chunk end (measured: ~9% of the recurrence).
      wait_vm<0>();
    }
    __syncthreads();
    if (tid == 0 && !last_only) {
      __hip_atomic_fetch_add(&counters[bh], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned target = (unsigned)SW_NSL * (unsigned)(c + 1);
      int spins = 0;
      while (__hip_atomic_load(&counters[bh], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > SW_SPIN_LIMIT) {
          __hip_atomic_store(errflag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    __syncthreads();
    if (!last_only && w >= 2 && w < 4) {
      const int d = (w - 2) * 64 + l;
      float ss = 0.f;
      for (int s = 0; s < SW_NSL; ++s)
        ss += __hip_atomic_load(&ss2[(((size_t)bh * 2 + (c & 1)) * SW_NSL + s) * D + d], __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
      const float inv = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
#pragma unroll
      for (int k = 0; k < NS / 4; ++k) *(floatx4*)(S.w2 + w2i(4 * k, d)) *= inv;
    }
    __syncthreads();
    if (update_first)
      store_state(c);
    else if (c + 1 < nchunks)
      store_state(c + 1);
  }
  wait_vm<0>();

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
};
constexpr int RW13_ROW = SW_D * 2;
constexpr int RW2_ROW = SW_US * 2;
__device__ __forceinline__ int w2_swz(int row) { return (row >> 2) & 3; }

// Two waves per SIMD, 32 tokens per wave (measured against one wave per SIMD
// with 64 tokens each, which halves the LDS reads of the weights per token:
// ~6 % slower, the lone wave waits on its own LDS reads).
constexpr int SW_RW = 8;                  // waves per read workgroup
constexpr int SW_RT = SW_TT / SW_RW;      // tokens per wave (2 tiles of 16)
__global__ __launch_bounds__(SW_RW * 64, 1) void swiglu_read_kernel(const bf16* __restrict__ Q,
                                                                    const bf16* __restrict__ states,
                                                                    bf16* __restrict__ O, int T, int chunk,
                                                                    int nchunks, int tiles) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  ReadLds& L = *reinterpret_cast<ReadLds*>(smem_raw);
  constexpr int D = SW_D, DH = SW_DH, NTH = SW_RW * 64, TT = SW_RT / 16;
  // the token tiles of one chunk run on one XCD, so its weights are fetched into one L2
  const int lb = (gridDim.x & 7) == 0 ? xcd_logical_block(blockIdx.x, gridDim.x) : blockIdx.x;
  const int tile = lb % tiles;
  const int c = (lb / tiles) % nchunks;
  const int bh = lb / (tiles * nchunks);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, li = l & 15;
  const int cend = min((c + 1) * chunk, T);
  const int t0 = c * chunk + tile * SW_TT;
  if (t0 >= cend) return;   // uniform over the workgroup, before any barrier
  const bf16* st = states + ((size_t)bh * nchunks + c) * SW_STATE;
  const size_t P = (size_t)D * DH;

  // this wave's queries as B operands (col = token, k = 8 consecutive d)
  const bf16* Qh = Q + (size_t)bh * T * D;
  bf16x8 qop[TT][4];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int t = min(t0 + SW_RT * w + 16 * tt + li, cend - 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qop[tt][ks] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const u32x4*)(Qh + (size_t)t * D + 32 * ks + 8 * g)));
  }

  // weight slice s -> LDS buffer buf by direct-to-LDS copies: each wave copies 4 KB of the W1T/W3T
  // planes (4 x 1 KB) and 2 KB of the W2T planes (2 x 1 KB)
  constexpr int J13 = 4 * SW_US * SW_D * 2 / 1024 / SW_RW, J2 = 2 * SW_D * SW_US * 2 / 1024 / SW_RW;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(st, (long long)SW_STATE * 2);
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
  auto load_slice = [&](int sl, int buf) {
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

  floatx4 oacc[8][TT];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) oacc[nt][tt] = floatx4{0.f, 0.f, 0.f, 0.f};

  constexpr int NSLICE = DH / SW_US;
  load_slice(0, 0);
  for (int s = 0; s < NSLICE; ++s) {
    const int buf = s & 1;
    // slice s has landed and every wave is done with slice s-1, whose buffer the next copy reuses
    // (the query loads issued before the first copy are complete too)
    wait_vm_barrier<0>();
    if (s + 1 < NSLICE) load_slice(s + 1, buf ^ 1);
    // H^T = silu(A^T) * B^T as bf16 hi + lo, k-slot order of the 32 units: 4g..4g+3 of unit tile 0,
    // then of unit tile 1
    bf16x8 hh[TT], hl[TT];
#pragma unroll
    for (int ut = 0; ut < 2; ++ut) {
      // A^T, B^T [unit][token] for one 16-unit tile x the wave's 4 token tiles
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
  bf16* Oh = O + (size_t)bh * T * D;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(Oh + (size_t)t0 * D, ((long long)cend - t0) * D * 2);
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const bf16x4 o = to_bf16x4(oacc[nt][tt][0], oacc[nt][tt][1], oacc[nt][tt][2], oacc[nt][tt][3]);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(uint2v, o), ro,
                                            (unsigned)((SW_RT * w + 16 * tt + li) * D * 2 + (16 * nt + 4 * g) * 2), 0, 0);
    }
}

struct SwLayout {
  size_t states, ss2, counters, err, total;
};

SwLayout sw_layout(int64_t BH, int64_t nchunks) {
  SwLayout L;
  L.states = 0;
  size_t off = (size_t)BH * nchunks * SW_STATE * 2;
  off = (off + 255) & ~(size_t)255;
  L.ss2 = off;
  off += (size_t)BH * 2 * SW_NSL * SW_D * 4;
  off = (off + 255) & ~(size_t)255;
  L.counters = off;
  off += (size_t)BH * 4;
  L.err = off;
  off += 4;
  L.total = (off + 255) & ~(size_t)255;
  return L;
}

}  // namespace

bool large_chunk_swiglu_supported(int64_t d, int64_t dh, int64_t chunk, int dtype) {
  (void)chunk;
  return dtype == 1 && d == SW_D && dh == SW_DH;
}

size_t large_chunk_swiglu_workspace(int64_t B, int64_t H, int64_t T, int64_t d, int64_t dh, int64_t chunk) {
  (void)d;
  (void)dh;
  return sw_layout(B * H, (T + chunk - 1) / chunk).total;
}

hipError_t launch_large_chunk_swiglu(const LargeChunkArgs& a, hipStream_t stream, const Timing& tm) {
  const int BH = (int)(a.B * a.H);
  const int T = (int)a.T, chunk = (int)a.chunk;
  const int nchunks = (int)((a.T + a.chunk - 1) / a.chunk);
  const SwLayout lay = sw_layout(BH, nchunks);
  unsigned char* ws = (unsigned char*)a.ws;
  bf16* states = (bf16*)(ws + lay.states);
  float* ss2 = (float*)(ws + lay.ss2);
  unsigned* counters = (unsigned*)(ws + lay.counters);
  unsigned* err = (unsigned*)(ws + lay.err);

  const int nz = BH + 1;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((nz + 255) / 256), dim3(256), 0, stream, counters, nz);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // the recurrence needs every workgroup of a head resident at once
  const size_t lds_r = sizeof(RecurLds);
  e = hipFuncSetAttribute((const void*)swiglu_recur_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_r);
  if (e != hipSuccess) return e;
  int dev = 0, ncu = 0, per_cu = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)swiglu_recur_kernel, SW_WAVES * 64, lds_r)) !=
      hipSuccess)
    return e;
  const int heads_per_launch = (per_cu * ncu) / SW_NSL;
  if (heads_per_launch < 1) return hipErrorCooperativeLaunchTooLarge;
  if (a.last_layer_only && !a.update_first && nchunks > 1 && BH * SW_NSL < ncu) {
    // The fully parallel form: every (head, chunk) W2 update at once, a prefix over chunks, the reads.
    // Taken only when the heads alone leave compute units idle: the total work is the same as the
    // recurrence's, and at one workgroup per CU or more the recurrence measured faster (B2 H8 T32768:
    // 0.67 against 0.72 ms per call; it has no prefix pass and no state copies).
    if ((e = mark(tm.start, stream)) != hipSuccess) return e;
    hipLaunchKernelGGL(swiglu_recur_kernel, dim3(BH * nchunks * SW_NSL), dim3(SW_WAVES * 64), lds_r, stream,
                       (const bf16*)a.K, (const bf16*)a.V, a.eta, a.W0, (float*)states, states, ss2, counters, err, T,
                       chunk, nchunks, 0, 0, 1, nchunks);
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
    const size_t lds_o = sizeof(ReadLds);
    e = hipFuncSetAttribute((const void*)swiglu_read_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_o);
    if (e != hipSuccess) return e;
    const int tiles = (chunk + SW_TT - 1) / SW_TT;
    hipLaunchKernelGGL(swiglu_read_kernel, dim3(BH * nchunks * tiles), dim3(SW_RW * 64), lds_o, stream,
                       (const bf16*)a.Q, (const bf16*)states, (bf16*)a.O, T, chunk, nchunks, tiles);
    return hipGetLastError();
  }
  const bf16* Kp = (const bf16*)a.K;
  const bf16* Vp = (const bf16*)a.V;
  const float* Ep = a.eta;
  const float* W0p = a.W0;
  float* Wo = a.W_out;
  if ((e = mark(tm.start, stream)) != hipSuccess) return e;   // the recurrence: the sequential part
  for (int h0 = 0; h0 < BH; h0 += heads_per_launch) {
    const int nh = std::min(heads_per_launch, BH - h0);
    int Ti = T, ci = chunk, nci = nchunks, hi = h0, uf = a.update_first ? 1 : 0, lo = a.last_layer_only ? 1 : 0;
    int pn = 0;
    void* args[] = {(void*)&Kp, (void*)&Vp, (void*)&Ep, (void*)&W0p, (void*)&Wo, (void*)&states, (void*)&ss2,
                    (void*)&counters, (void*)&err, (void*)&Ti, (void*)&ci, (void*)&nci, (void*)&hi, (void*)&uf,
                    (void*)&lo, (void*)&pn};
    e = hipLaunchCooperativeKernel((const void*)swiglu_recur_kernel, dim3(nh * SW_NSL), dim3(SW_WAVES * 64), args,
                                   (unsigned)lds_r, stream);
    if (e != hipSuccess) return e;
  }
  if ((e = mark(tm.stop, stream)) != hipSuccess) return e;
  if (nchunks == 0) return hipSuccess;
  const size_t lds_o = sizeof(ReadLds);
  e = hipFuncSetAttribute((const void*)swiglu_read_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_o);
  if (e != hipSuccess) return e;
  const int tiles = (chunk + SW_TT - 1) / SW_TT;
  hipLaunchKernelGGL(swiglu_read_kernel, dim3(BH * nchunks * tiles), dim3(SW_RW * 64), lds_o, stream, (const bf16*)a.Q,
                     (const bf16*)states, (bf16*)a.O, T, chunk, nchunks, tiles);
  return hipGetLastError();
}

}  // namespace ttt
