// LaCT large-chunk TTT with a linear fast weight (LaCT review "Test-Time
// Training Done Right": fast-weights section - one update per large chunk;
// non-linear-memory section - chunk gradients summed with per-token rates
// and L2 normalisation after the update; read-order section - a chunk
// reads the memory left by earlier chunks, then updates it):
//     O_c = Q_c W_{c-1}
//     W_c = colnorm(W_{c-1} + K_c^T diag(eta_c) V_c),   W_0 = W0 (not normalised)
// colnorm divides each column (one output unit's fan-in) by
// max(||column||_2, 1e-12).
//
// The update K_c^T diag(eta_c) V_c does not depend on W, so it is computed
// for every chunk in parallel; the normalisation acts on each column of W
// separately, so the sequential part is a scan per column:
//   1. lact_delta_kernel - partial updates over token slices of every chunk
//                          (bf16 MFMA, diag(eta) V split into bf16 hi + lo),
//                          written transposed [out][in]
//   2. lact_scan_kernel  - one wave per (head, column): sums the slices,
//                          adds, normalises, and keeps W_{c-1} of every
//                          chunk (transposed, fp32)
//   3. lact_read_kernel  - O_c = Q_c W_{c-1}, a quarter chunk per workgroup,
//                          W staged once in LDS as bf16 hi + lo, queries
//                          streamed per wave through a direct-to-LDS ring
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace ttt {

namespace {

constexpr int LC_STEP = 64;       // tokens per LDS step in the update kernel
constexpr int LC_MAXSPLIT = 4;    // token slices per chunk
constexpr int LC_WG_TARGET = 512;  // update workgroups wanted: about two per CU

// Token slices per chunk of the update kernel: as few as give about two
// workgroups per CU (each slice writes a d x d partial, so fewer slices move
// fewer bytes: at the 196K-token workload one slice per 4096-token chunk ran
// 101 us against 108 us with two and 113 us with four), at most LC_MAXSPLIT,
// each at least one 64-token step.
inline int64_t nsplit_of(int64_t BH, int64_t nchunks, int64_t chunk) {
  const int64_t units = BH * nchunks > 0 ? BH * nchunks : 1;
  int64_t n = (LC_WG_TARGET + units - 1) / units;
  const int64_t steps = (chunk + LC_STEP - 1) / LC_STEP;
  n = n > LC_MAXSPLIT ? LC_MAXSPLIT : n;
  n = n > steps ? steps : n;
  return n < 1 ? 1 : n;
}
inline int64_t slice_of(int64_t BH, int64_t nchunks, int64_t chunk) {
  const int64_t n = nsplit_of(BH, nchunks, chunk);
  return ((chunk + n - 1) / n + LC_STEP - 1) / LC_STEP * LC_STEP;
}

// ---------------------------------------------------------------------------
// 1. partial dW = sum_{t in slice} k_t^T (eta_t v_t), one slice per workgroup
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, D == 64 ? 4 : 2) void lact_delta_kernel(const bf16* __restrict__ K, const bf16* __restrict__ V,
                                                            const float* __restrict__ eta, float* __restrict__ part,
                                                            int T, int chunk, int nchunks, int nsplit, int slice) {
  constexpr int ROW = D * 2 + 32;              // padded LDS row (bytes)
  constexpr int PIECES = LC_STEP * D / 8;      // 16-byte pieces per tile
  constexpr int PPT = PIECES / 256;            // pieces per thread
  constexpr int QW = D / 2;                    // quadrant width per wave
  constexpr int TW = QW / 32;                  // 32x32 tiles per quadrant side
  __shared__ __attribute__((aligned(16))) unsigned char lds[3 * LC_STEP * ROW];
  unsigned char* ks = lds;
  unsigned char* vh = lds + LC_STEP * ROW;
  unsigned char* vl = lds + 2 * LC_STEP * ROW;
  static_assert(64 * (D + 1) * 4 <= 3 * LC_STEP * ROW, "transpose buffer");

  const int split = blockIdx.x % nsplit;
  const int c = (blockIdx.x / nsplit) % nchunks;
  const int bh = blockIdx.x / (nsplit * nchunks);
  const int cstart = c * chunk;
  const int cend = min(cstart + chunk, T);
  const int s0 = cstart + split * slice;
  const int s1 = min(s0 + slice, cend);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, G = l >> 4, L = l & 15;
  const bf16* Kh = K + (size_t)bh * T * D;
  const bf16* Vh = V + (size_t)bh * T * D;
  const float* Eh = eta + (size_t)bh * T;

  uint4 kreg[PPT], vreg[PPT];
  float ereg[PPT];
  auto load = [&](int t0) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int p = k * 256 + tid;
      const int row = p / (D / 8), col = (p % (D / 8)) * 8;
      const int t = t0 + row;
      const int tc = min(t, s1 - 1);
      kreg[k] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)(Kh + (size_t)tc * D + col)));
      vreg[k] = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)(Vh + (size_t)tc * D + col)));
      ereg[k] = t < s1 ? Eh[tc] : 0.f;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int p = k * 256 + tid;
      const int row = p / (D / 8), col = (p % (D / 8)) * 8;
      *(uint4*)(ks + row * ROW + col * 2) = kreg[k];
      const bf16x8 v = __builtin_bit_cast(bf16x8, vreg[k]);
      bf16x8 hi, lo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float f = ereg[k] * (float)v[j];
        hi[j] = (bf16)f;
        lo[j] = (bf16)(f - (float)hi[j]);
      }
      *(bf16x8*)(vh + row * ROW + col * 2) = hi;
      *(bf16x8*)(vl + row * ROW + col * 2) = lo;
    }
  };

  floatx16 acc[TW][TW];
#pragma unroll
  for (int i = 0; i < TW; ++i)
#pragma unroll
    for (int j = 0; j < TW; ++j) acc[i][j] = floatx16{};
  const int a0 = (w >> 1) * QW, b0 = (w & 1) * QW;
  const int nsteps = s1 > s0 ? (s1 - s0 + LC_STEP - 1) / LC_STEP : 0;
  if (nsteps > 0) load(s0);
  for (int st = 0; st < nsteps; ++st) {
    if (st > 0) __syncthreads();               // everyone is done with the previous tile
    store();
    __syncthreads();
    if (st + 1 < nsteps) load(s0 + (st + 1) * LC_STEP);
#pragma unroll
    for (int k0 = 0; k0 < LC_STEP; k0 += 16) {
      // operands with tokens as the contraction index, via transposed reads
      const int r0 = k0 + 8 * (G >> 1) + (L >> 2);
      bf16x8 A[TW], Bh[TW], Bl[TW];
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        const int ca = a0 + 32 * i + 16 * (G & 1) + 4 * (L & 3);
        A[i] = join(lds_read_tr16(ks + r0 * ROW + ca * 2), lds_read_tr16(ks + (r0 + 4) * ROW + ca * 2));
        const int cb = b0 + 32 * i + 16 * (G & 1) + 4 * (L & 3);
        Bh[i] = join(lds_read_tr16(vh + r0 * ROW + cb * 2), lds_read_tr16(vh + (r0 + 4) * ROW + cb * 2));
        Bl[i] = join(lds_read_tr16(vl + r0 * ROW + cb * 2), lds_read_tr16(vl + (r0 + 4) * ROW + cb * 2));
      }
#pragma unroll
      for (int i = 0; i < TW; ++i)
#pragma unroll
        for (int j = 0; j < TW; ++j) {
          acc[i][j] = mfma32(A[i], Bh[j], acc[i][j]);
          acc[i][j] = mfma32(A[i], Bl[j], acc[i][j]);
        }
    }
  }
  // transpose through LDS, 64 output columns b at a time (fp32 [b][a], padded),
  // so the partial is written [out][in] with coalesced stores
  float* P = part + (((size_t)bh * nchunks + c) * nsplit + split) * D * D;
  float* tr = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int bp = 0; bp < D / 64; ++bp) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
      for (int j = 0; j < TW; ++j) {
        const int b = b0 + 32 * j + (l & 31);
        if (b / 64 != bp) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int a = a0 + 32 * i + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
          tr[(b - 64 * bp) * (D + 1) + a] = acc[i][j][r];
        }
      }
    __syncthreads();
    for (int i = tid; i < 64 * D; i += 256) P[(size_t)(64 * bp) * D + i] = tr[(i / D) * (D + 1) + (i % D)];
  }
}

// ---------------------------------------------------------------------------
// 2. normalise-scan: one wave per (head, column j).  Lane l holds rows
//    l, l+64, ... of the column.  The updates do not depend on W, so those of
//    the next window of chunks are loaded while the current window is
//    scanned (two register buffers); the column norm is a DPP wave sum.
// ---------------------------------------------------------------------------
// With momentum beta the step applied is the buffer M_c = beta M_{c-1} + dW_c (M from M0, or
// zeros when M0 is null; written to Mout when it is not null).  beta = 0 without M0 gives the
// plain step bit for bit (0 * 0 + dW = dW).
template <int D, bool UF>
__global__ __launch_bounds__(256) void lact_scan_kernel(const float* __restrict__ W0, const float* __restrict__ part,
                                                        float* __restrict__ wprev_t, float* __restrict__ Wout,
                                                        int nchunks, int nsplit, const float* M0, float* Mout,
                                                        float beta) {
  constexpr int RPL = D / 64;
  constexpr int WIN = D == 64 ? 12 : 6;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int j = (blockIdx.x % (D / 4)) * 4 + w;
  const int bh = blockIdx.x / (D / 4);
  float Wc[RPL], Mc[RPL];
  const float* W0h = W0 + (size_t)bh * D * D;
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    Wc[r] = W0h[(size_t)(l + 64 * r) * D + j];
    Mc[r] = M0 ? M0[(size_t)bh * D * D + (size_t)(l + 64 * r) * D + j] : 0.f;
  }
  // slice updates of chunks c0 .. c0+WIN-1, loaded unconditionally (indices clamped) so that every window
  // issues the same loads and the waits for one window never cover the next one's
  auto issue = [&](int c0, float (&raw)[LC_MAXSPLIT][WIN][RPL]) {
#pragma unroll
    for (int s = 0; s < LC_MAXSPLIT; ++s) {
      const int sc = min(s, nsplit - 1);
#pragma unroll
      for (int i = 0; i < WIN; ++i) {
        const int cc = min(c0 + i, nchunks - 1);
        const float* Pc = part + ((((size_t)bh * nchunks + cc) * nsplit + sc) * D + j) * D;
#pragma unroll
        for (int r = 0; r < RPL; ++r) raw[s][i][r] = Pc[l + 64 * r];
      }
    }
  };
  auto scan_win = [&](int c0, const float (&raw)[LC_MAXSPLIT][WIN][RPL]) {
#pragma unroll
    for (int i = 0; i < WIN; ++i) {
      const int c = c0 + i;
      if (c >= nchunks) break;
      // the state chunk c reads, transposed: W_{c-1}, or W_c when a chunk updates first
      float* Wt = wprev_t + (((size_t)bh * nchunks + c) * D + j) * D;
      float ss = 0.f;
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        float d = raw[0][i][r];
#pragma unroll
        for (int s = 1; s < LC_MAXSPLIT; ++s) d += s < nsplit ? raw[s][i][r] : 0.f;
        if (!UF) Wt[l + 64 * r] = Wc[r];
        Mc[r] = fmaf(beta, Mc[r], d);
        Wc[r] += Mc[r];
        ss = fmaf(Wc[r], Wc[r], ss);
      }
      const float inv = 1.0f / fmaxf(sqrtf(wave_sum(ss)), 1e-12f);
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        Wc[r] *= inv;
        if (UF) Wt[l + 64 * r] = Wc[r];
      }
    }
  };
  // two register buffers: the next window is in flight while the current one is scanned
  float ra[LC_MAXSPLIT][WIN][RPL], rb[LC_MAXSPLIT][WIN][RPL];
  if (nchunks > 0) {
    issue(0, ra);
    for (int c0 = 0;;) {
      issue(c0 + WIN, rb);
      __builtin_amdgcn_sched_barrier(0);
      scan_win(c0, ra);
      if ((c0 += WIN) >= nchunks) break;
      issue(c0 + WIN, ra);
      __builtin_amdgcn_sched_barrier(0);
      scan_win(c0, rb);
      if ((c0 += WIN) >= nchunks) break;
    }
  }
  float* Wo = Wout + (size_t)bh * D * D;
#pragma unroll
  for (int r = 0; r < RPL; ++r) Wo[(size_t)(l + 64 * r) * D + j] = Wc[r];
  if (Mout) {
#pragma unroll
    for (int r = 0; r < RPL; ++r) Mout[(size_t)bh * D * D + (size_t)(l + 64 * r) * D + j] = Mc[r];
  }
}

// ---------------------------------------------------------------------------
// 3. O_c = Q_c W_{c-1}.  One workgroup per (head, chunk, part of a chunk);
//    W_{c-1} staged once in LDS as bf16 hi + lo (rows = output unit); each
//    wave streams its own 16-token rows of every 64-token tile through a
//    private direct-to-LDS ring and computes O^T = W^T Q^T for them.
// ---------------------------------------------------------------------------
constexpr int LR_STAGES = 4;
template <int D>
struct LactReadCfg {
  static constexpr int ROWB = D * 2;
  static constexpr int W_BYTES = D * D * 2;                  // one bf16 plane of W^T, swizzled
  static constexpr int QW_BYTES = 16 * ROWB;                 // one wave's 16 rows of a tile
  static constexpr int QI = QW_BYTES / 1024;                 // DMA instructions per wave per tile
  static constexpr int LDS = 2 * W_BYTES + 4 * LR_STAGES * QW_BYTES;
  static constexpr int KT = D / 32;
  static constexpr int MT = D / 16;
  static constexpr int SWZ = D / 8 >= 16 ? 15 : D / 8 - 1;
};

// OF32: float32 outputs, stored straight from the accumulators (16 bytes per lane: 4 columns of one token).
template <int D, bool OF32>
__global__ __launch_bounds__(256, 2) void lact_read_kernel(const bf16* __restrict__ Q, const float* __restrict__ wprev_t,
                                                           void* __restrict__ O, int T, int chunk, int nchunks,
                                                           int parts, int part_len) {
  using Cfg = LactReadCfg<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // the parts of one chunk run on one XCD, so its W is fetched into one L2
  const int lb = (gridDim.x & 7) == 0 ? xcd_logical_block(blockIdx.x, gridDim.x) : blockIdx.x;
  const int part = lb % parts;
  const int c = (lb / parts) % nchunks;
  const int bh = lb / (parts * nchunks);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, li = l & 15;
  const int cend = min((c + 1) * chunk, T);
  const int t0 = c * chunk + part * part_len;
  const int t1 = min(t0 + part_len, cend);
  if (t0 >= t1) return;

  // per-lane offsets: natural operand reads (row 16*blk + li, k = 32ks + 8g)
  int nat[Cfg::KT];
#pragma unroll
  for (int ks = 0; ks < Cfg::KT; ++ks) nat[ks] = li * Cfg::ROWB + (((4 * ks + g) ^ (li & Cfg::SWZ)) << 4);
  // this wave's DMA: 16 rows of a tile = QI instructions; slot (lane) -> (row, piece)
  unsigned qoff[Cfg::QI];
#pragma unroll
  for (int k = 0; k < Cfg::QI; ++k) {
    const int s = k * 64 + l;
    const int row = s / (D / 8);
    qoff[k] = (unsigned)((16 * w + row) * Cfg::ROWB + (((s % (D / 8)) ^ (row & Cfg::SWZ)) << 4));
  }
  unsigned char* ring = smem + 2 * Cfg::W_BYTES + w * LR_STAGES * Cfg::QW_BYTES;
  const bf16* Qh = Q + (size_t)bh * T * D;
  const size_t oes = OF32 ? 4 : 2;
  unsigned char* Oh = (unsigned char*)O + (size_t)bh * T * D * oes;
  const int ntiles = (t1 - t0 + 63) / 64;
  // one buffer view of this part's queries and outputs (rows past its end read 0 / are dropped)
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qh + (size_t)t0 * D, (long long)(t1 - t0) * Cfg::ROWB);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(Oh + (size_t)t0 * D * oes, (long long)(t1 - t0) * D * oes);
  constexpr int ST = OF32 ? Cfg::MT : Cfg::QI;    // output stores per wave per tile
  auto issue = [&](int i) {
    unsigned char* dst = ring + (i % LR_STAGES) * Cfg::QW_BYTES;
    const unsigned t = (unsigned)i * 64 * Cfg::ROWB;
#pragma unroll
    for (int k = 0; k < Cfg::QI; ++k) buf2lds16<true>(rq, t + qoff[k], dst + k * 1024);
  };
  // the first query tiles are in flight while W is staged
#pragma unroll
  for (int i = 0; i < LR_STAGES - 1; ++i) issue(i);
  // ---- W^T of this chunk as bf16 hi + lo planes [n][a], 16-byte pieces swizzled by n ----
  const float* Wt = wprev_t + ((size_t)bh * nchunks + c) * D * D;
  for (int p = tid; p < D * D / 8; p += 256) {
    const int n = p / (D / 8), pc = p % (D / 8);
    const floatx4 x0 = *(const floatx4*)(Wt + (size_t)n * D + pc * 8);
    const floatx4 x1 = *(const floatx4*)(Wt + (size_t)n * D + pc * 8 + 4);
    bf16x8 hi, lo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float f = j < 4 ? x0[j] : x1[j - 4];
      hi[j] = (bf16)f;
      lo[j] = (bf16)(f - (float)hi[j]);
    }
    const int off = n * Cfg::ROWB + ((pc ^ (n & Cfg::SWZ)) << 4);
    *(bf16x8*)(smem + off) = hi;
    *(bf16x8*)(smem + Cfg::W_BYTES + off) = lo;
  }
  __syncthreads();                                  // W planes complete
  const unsigned char* wh = smem;
  const unsigned char* wl = smem + Cfg::W_BYTES;
  for (int i = 0; i < ntiles; ++i) {
    // This wave's rows of tile i have landed once only later operations are outstanding: the copies of
    // tiles i+1 and i+2 and the output stores of up to three earlier tiles (issued after tile i's copy).
    if (i == 0)
      wait_vm<2 * Cfg::QI>();
    else if (i == 1)
      wait_vm<2 * Cfg::QI + ST>();
    else if (i == 2)
      wait_vm<2 * Cfg::QI + 2 * ST>();
    else
      wait_vm<2 * Cfg::QI + 3 * ST>();
    issue(i + LR_STAGES - 1);
    unsigned char* qs = ring + (i % LR_STAGES) * Cfg::QW_BYTES;   // this wave's 16 rows
    bf16x8 qop[Cfg::KT];
#pragma unroll
    for (int ks = 0; ks < Cfg::KT; ++ks) qop[ks] = *(const bf16x8*)(qs + nat[ks]);
    // O^T = W^T Q^T: lane holds O[16w + li][16m + 4g .. +3], staged over the dead query rows (same
    // swizzled layout) and written out as whole rows, 16 bytes per lane
#pragma unroll
    for (int m = 0; m < Cfg::MT; ++m) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < Cfg::KT; ++ks) {
        acc = mfma16(*(const bf16x8*)(wh + m * 16 * Cfg::ROWB + nat[ks]), qop[ks], acc);
        acc = mfma16(*(const bf16x8*)(wl + m * 16 * Cfg::ROWB + nat[ks]), qop[ks], acc);
      }
      if constexpr (OF32) {
        buf_store16(ro, (unsigned)(((i * 64 + 16 * w + li) * D + 16 * m + 4 * g) * 4), __builtin_bit_cast(u32x4, acc));
      } else {
        const int piece = 2 * m + (g >> 1);
        *(bf16x4*)(qs + li * Cfg::ROWB + ((piece ^ (li & Cfg::SWZ)) << 4) + (g & 1) * 8) =
            to_bf16x4(acc[0], acc[1], acc[2], acc[3]);
      }
    }
    if constexpr (!OF32) {
      const unsigned t = (unsigned)i * 64 * Cfg::ROWB;
      u32x4 v[Cfg::QI];
#pragma unroll
      for (int k = 0; k < Cfg::QI; ++k) v[k] = *(const u32x4*)(qs + k * 1024 + 16 * l);
#pragma unroll
      for (int k = 0; k < Cfg::QI; ++k) buf_store16(ro, t + qoff[k], v[k]);
    }
  }
  wait_vm<0>();
}

template <int D>
hipError_t launch_lact(const LargeChunkArgs& a, hipStream_t stream, const Timing& tm) {
  const int T = (int)a.T, chunk = (int)a.chunk;
  const int nchunks = (int)((a.T + a.chunk - 1) / a.chunk);
  const int nsplit = (int)nsplit_of(a.B * a.H, nchunks, a.chunk);
  const int slice = (int)slice_of(a.B * a.H, nchunks, a.chunk);
  const int BH = (int)(a.B * a.H);
  float* part = (float*)a.ws;
  float* wprev = part + (size_t)BH * nchunks * nsplit * D * D;
  if (nchunks > 0) {
    hipError_t e = mark(tm.start, stream);   // the update kernel streams K and V: the largest share of the bytes
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lact_delta_kernel<D>, dim3(BH * nchunks * nsplit), dim3(256), 0, stream, (const bf16*)a.K,
                       (const bf16*)a.V, a.eta, part, T, chunk, nchunks, nsplit, slice);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = mark(tm.stop, stream)) != hipSuccess) return e;
  }
  auto kscan = a.update_first ? lact_scan_kernel<D, true> : lact_scan_kernel<D, false>;
  hipLaunchKernelGGL(kscan, dim3(BH * D / 4), dim3(256), 0, stream, a.W0, part, wprev, a.W_out, nchunks, nsplit, a.M0,
                     a.M_out, a.momentum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nchunks == 0) return e;
  using Cfg = LactReadCfg<D>;
  auto kread = a.o_f32 ? lact_read_kernel<D, true> : lact_read_kernel<D, false>;
  e = hipFuncSetAttribute((const void*)kread, hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS);
  if (e != hipSuccess) return e;
  // about a quarter chunk (at least 256 tokens) per workgroup
  int part_len = (chunk + 3) / 4;
  part_len = part_len < 256 ? 256 : part_len;
  part_len = (part_len + 63) / 64 * 64;
  part_len = part_len > (1 << 20) ? (1 << 20) : part_len;   // 32-bit byte offsets within a part
  const int parts = (chunk + part_len - 1) / part_len;
  hipLaunchKernelGGL(kread, dim3(BH * nchunks * parts), dim3(256), Cfg::LDS, stream, (const bf16*)a.Q, wprev, a.O, T,
                     chunk, nchunks, parts, part_len);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Backward.  Chunk c forms P_c = W_{c-1} + dW_c and W_c = P_c / n_c per column
// (n_c = max(||column||, 1e-12)); its queries read R_c = W_{c-1} (W_c when a
// chunk updates first).  With G the gradient of the newest memory (dW_T at
// the end), from the last chunk back:
//   update-first: G += A_c                (A_c = Q_c^T dO_c)
//   dP_c = (G - w (w . G)) / n_c per column (G / 1e-12 under the floor)
//   G = dP_c, and read-first: G += A_c
// and dW0 = G.  Then, for every chunk in parallel,
//   dQ_c = dO_c R_c^T,  u = K_c dP_c,  dK_c = diag(eta) V_c dP_c^T,
//   dV_c = diag(eta) u,  deta_t = <u_t, v_t>.
// The dW_c and A_c come from lact_delta_kernel (A_c with unit rates); the
// memories R_c from lact_scan_kernel, as in the forward.
// ---------------------------------------------------------------------------

// One wave per (head, column j), lanes over rows, as lact_scan_kernel.
// dpt: dP_c transposed ([c][j][i]); dW, dW0 natural [i][j].
template <int D, bool UF>
__global__ __launch_bounds__(256) void lact_bwd_scan_kernel(const float* __restrict__ W0, const float* __restrict__ dW,
                                                            const float* __restrict__ partA,
                                                            const float* __restrict__ partB,
                                                            const float* __restrict__ wprev_t, float* __restrict__ dpt,
                                                            float* __restrict__ dW0, int nchunks, int nsplit) {
  constexpr int RPL = D / 64;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int j = (blockIdx.x % (D / 4)) * 4 + w;
  const int bh = blockIdx.x / (D / 4);
  float G[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) G[r] = dW[(size_t)bh * D * D + (size_t)(l + 64 * r) * D + j];
  for (int c = nchunks - 1; c >= 0; --c) {
    float dw[RPL], a[RPL], wp[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      dw[r] = 0.f;
      a[r] = 0.f;
    }
    for (int sp = 0; sp < nsplit; ++sp) {
      const size_t o = ((((size_t)bh * nchunks + c) * nsplit + sp) * D + j) * D;
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        dw[r] += partA[o + l + 64 * r];
        a[r] += partB[o + l + 64 * r];
      }
    }
    // W_{c-1}: what chunk c reads when it reads first, else the memory chunk c-1 read (W0 for c = 0)
    if (!UF || c > 0) {
      const float* Wt = wprev_t + (((size_t)bh * nchunks + (UF ? c - 1 : c)) * D + j) * D;
#pragma unroll
      for (int r = 0; r < RPL; ++r) wp[r] = Wt[l + 64 * r];
    } else {
#pragma unroll
      for (int r = 0; r < RPL; ++r) wp[r] = W0[(size_t)bh * D * D + (size_t)(l + 64 * r) * D + j];
    }
    if (UF) {
#pragma unroll
      for (int r = 0; r < RPL; ++r) G[r] += a[r];
    }
    float p[RPL], ss = 0.f;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      p[r] = wp[r] + dw[r];
      ss = fmaf(p[r], p[r], ss);
    }
    const float nrm = sqrtf(wave_sum(ss));
    const float inv = 1.0f / fmaxf(nrm, 1e-12f);
    float wg = 0.f;
#pragma unroll
    for (int r = 0; r < RPL; ++r) wg = fmaf(p[r] * inv, G[r], wg);
    const float proj = nrm > 1e-12f ? wave_sum(wg) : 0.f;   // the floor's branch is linear: no projection
    float* out = dpt + (((size_t)bh * nchunks + c) * D + j) * D;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      G[r] = (G[r] - p[r] * inv * proj) * inv;
      out[l + 64 * r] = G[r];
      if (!UF) G[r] += a[r];
    }
  }
#pragma unroll
  for (int r = 0; r < RPL; ++r) dW0[(size_t)bh * D * D + (size_t)(l + 64 * r) * D + j] = G[r];
}

// Per (head, chunk, part of the chunk): dQ = dO R^T, u = K dP, w = V dP^T for
// the part's tokens, then dV = eta u, dK = eta w, deta = <u, v>, all float32.
// The matrices are staged once in LDS as the MFMA A operands M^T (rows =
// output column) in bf16 hi + lo; each wave takes 16-token blocks and reads
// its B operands (token rows) straight from HBM.  WHICH selects the products
// (1: dQ, 2: u and w, 3: all): at d = 128 the three matrices do not fit in
// LDS together, so dQ runs as a launch of its own.
template <int D, int WHICH>
struct LactBwdCfg {
  static constexpr int ROWB = 2 * D + 16;             // padded LDS row of M^T (bytes)
  static constexpr int PLANE = D * ROWB;
  static constexpr int NPL = 2;                       // hi, lo
  static constexpr int MAT = NPL * PLANE;
  static constexpr int OFF_U = (WHICH & 1) ? MAT : 0;  // dP^T and dP after R when both are staged
  static constexpr int LDS = ((WHICH & 1) ? MAT : 0) + ((WHICH & 2) ? 2 * MAT : 0);
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <int D, int WHICH>
__global__ __launch_bounds__(256) void lact_bwd_prod_kernel(const bf16* __restrict__ K, const bf16* __restrict__ V,
                                                            const bf16* __restrict__ dO, const float* __restrict__ eta,
                                                            const float* __restrict__ wprev_t,
                                                            const float* __restrict__ dpt, float* __restrict__ dQ,
                                                            float* __restrict__ dK, float* __restrict__ dV,
                                                            float* __restrict__ deta, int T, int chunk, int nchunks,
                                                            int parts, int part_len) {
  using Cfg = LactBwdCfg<D, WHICH>;
  constexpr bool DQ = WHICH & 1, UW = WHICH & 2;
  constexpr int MT = D / 16, KP = D / 32;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int bh = blockIdx.x / (nchunks * parts);
  const int c = (blockIdx.x / parts) % nchunks, pi = blockIdx.x % parts;
  const long long cs = (long long)c * chunk, ce = min(cs + chunk, (long long)T);
  const long long t0 = cs + (long long)pi * part_len;
  const long long t1 = min(t0 + part_len, ce);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, li = l & 15;

  // stage M^T of the three products: R_c (dQ), dP_c^T (u) and dP_c (w); source layouts are transposed
  // ([j][i] = M[i][j]), so M^T[n][k] is src[k][n] for R and dP, src[n][k] for dP^T
  const float* Rt = wprev_t + ((size_t)bh * nchunks + c) * D * D;
  const float* Pt = dpt + ((size_t)bh * nchunks + c) * D * D;
  auto stage = [&](int off, float v, int n, int k) {
    const bf16 h = (bf16)v;
    unsigned char* row = smem + off + n * Cfg::ROWB + 2 * k;
    *(bf16*)row = h;
    *(bf16*)(row + Cfg::PLANE) = (bf16)(v - (float)h);
  };
  for (int idx = tid; idx < D * D; idx += 256) {
    const int n = idx / D, k = idx % D;
    if constexpr (DQ) stage(0, Rt[(size_t)k * D + n], n, k);
    if constexpr (UW) {
      stage(Cfg::OFF_U, Pt[(size_t)n * D + k], n, k);
      stage(Cfg::OFF_U + Cfg::MAT, Pt[(size_t)k * D + n], n, k);
    }
  }
  __syncthreads();
  if (t1 <= t0) return;

  const long long ntok = t1 - t0;
  const size_t base = (size_t)bh * T + t0;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + base * D, ntok * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + base * D, ntok * D * 2);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(dO + base * D, ntok * D * 2);
  const __amdgpu_buffer_rsrc_t re = make_rsrc(eta + base, ntok * 4);
  const __amdgpu_buffer_rsrc_t rq32 = make_rsrc(dQ + base * D, ntok * D * 4);
  const __amdgpu_buffer_rsrc_t rk32 = make_rsrc(dK + base * D, ntok * D * 4);
  const __amdgpu_buffer_rsrc_t rv32 = make_rsrc(dV + base * D, ntok * D * 4);
  const __amdgpu_buffer_rsrc_t rde = make_rsrc(deta + base, ntok * 4);
  const int nblk = (int)((ntok + 15) / 16);
  // several 16-token blocks per wave and step: the loads of all are issued before any is computed
  struct Ops {
    bf16x8 xd[KP], xk[KP], xv[KP];
    uint2v vc[MT];
    float e;
  };
  auto load = [&](int b, Ops& x) {
    const unsigned trow = (unsigned)(16 * b + li);
#pragma unroll
    for (int p = 0; p < KP; ++p) {
      const unsigned o = trow * (D * 2) + (unsigned)(32 * p + 8 * g) * 2;
      if constexpr (DQ) x.xd[p] = __builtin_bit_cast(bf16x8, buf_load16(rdo, o));
      if constexpr (UW) {
        x.xk[p] = __builtin_bit_cast(bf16x8, buf_load16(rk, o));
        x.xv[p] = __builtin_bit_cast(bf16x8, buf_load16(rv, o));
      }
    }
    if constexpr (UW) {
      x.e = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(re, trow * 4, 0, 0));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        x.vc[mt] = __builtin_amdgcn_raw_buffer_load_b64(rv, trow * (D * 2) + (unsigned)(16 * mt + 4 * g) * 2, 0, 0);
    }
  };
  auto compute = [&](int b, const Ops& x) {
    const unsigned trow = (unsigned)(16 * b + li);
    float dot = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      floatx4 aq = {0.f, 0.f, 0.f, 0.f}, au = aq, aw = aq;
#pragma unroll
      for (int p = 0; p < KP; ++p) {
        const int ao = (16 * mt + li) * Cfg::ROWB + (32 * p + 8 * g) * 2;
#pragma unroll
        for (int pl = 0; pl < Cfg::NPL; ++pl) {
          if constexpr (DQ) aq = mfma16(*(const bf16x8*)(smem + pl * Cfg::PLANE + ao), x.xd[p], aq);
          if constexpr (UW) {
            const unsigned char* b0 = smem + Cfg::OFF_U + pl * Cfg::PLANE + ao;
            au = mfma16(*(const bf16x8*)(b0), x.xk[p], au);
            aw = mfma16(*(const bf16x8*)(b0 + Cfg::MAT), x.xv[p], aw);
          }
        }
      }
      // lane (g, li) holds columns 16mt + 4g .. +3 of token 16b + li
      const unsigned col = (unsigned)(16 * mt + 4 * g);
      const unsigned o32 = trow * (D * 4) + col * 4;
      if constexpr (DQ) buf_store16(rq32, o32, __builtin_bit_cast(u32x4, aq));
      if constexpr (UW) {
        buf_store16(rv32, o32, __builtin_bit_cast(u32x4, x.e * au));
        buf_store16(rk32, o32, __builtin_bit_cast(u32x4, x.e * aw));
        const uint2v vv = x.vc[mt];
        dot = fmaf(au[0], bf16lo_f(vv[0]), dot);
        dot = fmaf(au[1], bf16hi_f(vv[0]), dot);
        dot = fmaf(au[2], bf16lo_f(vv[1]), dot);
        dot = fmaf(au[3], bf16hi_f(vv[1]), dot);
      }
    }
    if constexpr (UW) {
      dot += __shfl_xor(dot, 16);
      dot += __shfl_xor(dot, 32);
      if (g == 0) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, dot), rde, trow * 4, 0, 0);
    }
  };
  constexpr int NBW = 2;            // blocks per wave and step (4 measured no faster)
  for (int b = w; b < nblk; b += 4 * NBW) {
    Ops x[NBW];
#pragma unroll
    for (int k = 0; k < NBW; ++k)
      if (b + 4 * k < nblk) load(b + 4 * k, x[k]);   // wave-uniform
#pragma unroll
    for (int k = 0; k < NBW; ++k)
      if (b + 4 * k < nblk) compute(b + 4 * k, x[k]);
  }
}

__global__ __launch_bounds__(256) void lact_fill_ones_kernel(float* __restrict__ p, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) p[i] = 1.0f;
}

struct LactBwdLayout {
  size_t partA, partB, wprev, dpt, ones, junk, total;
};
inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
inline LactBwdLayout lact_bwd_layout(int64_t BH, int64_t T, int64_t D, int64_t chunk) {
  const int64_t nchunks = (T + chunk - 1) / chunk;
  const size_t mat = (size_t)D * D * 4, nsplit = (size_t)nsplit_of(BH, nchunks, chunk);
  LactBwdLayout L;
  size_t o = 0;
  L.partA = o; o += al256(BH * nchunks * nsplit * mat);
  L.partB = o; o += al256(BH * nchunks * nsplit * mat);
  L.wprev = o; o += al256(BH * nchunks * mat);
  L.dpt = o; o += al256(BH * nchunks * mat);
  L.ones = o; o += al256((size_t)BH * T * 4);
  L.junk = o; o += al256(BH * mat);
  L.total = o;
  return L;
}

template <int D>
hipError_t launch_lact_bwd(const BackwardArgs& a, hipStream_t stream) {
  const int T = (int)a.T, chunk = (int)a.chunk, BH = (int)(a.B * a.H);
  const int nchunks = (int)((a.T + a.chunk - 1) / a.chunk);
  const int nsplit = (int)nsplit_of(BH, nchunks, a.chunk);
  const int slice = (int)slice_of(BH, nchunks, a.chunk);
  const LactBwdLayout L = lact_bwd_layout(BH, a.T, D, a.chunk);
  char* ws = (char*)a.ws;
  float *partA = (float*)(ws + L.partA), *partB = (float*)(ws + L.partB), *wprev = (float*)(ws + L.wprev);
  float *dpt = (float*)(ws + L.dpt), *ones = (float*)(ws + L.ones), *junk = (float*)(ws + L.junk);
  const bool uf = a.other_order != 0;
  hipError_t e;
  const long long ntok = (long long)BH * T;
  if (nchunks > 0) {
    hipLaunchKernelGGL(lact_fill_ones_kernel, dim3((unsigned)std::min<long long>((ntok + 255) / 256, 2048)), dim3(256),
                       0, stream, ones, ntok);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(lact_delta_kernel<D>, dim3(BH * nchunks * nsplit), dim3(256), 0, stream, (const bf16*)a.K,
                       (const bf16*)a.V, a.eta, partA, T, chunk, nchunks, nsplit, slice);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(lact_delta_kernel<D>, dim3(BH * nchunks * nsplit), dim3(256), 0, stream, (const bf16*)a.Q,
                       (const bf16*)a.dO, (const float*)ones, partB, T, chunk, nchunks, nsplit, slice);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  auto kscan = uf ? lact_scan_kernel<D, true> : lact_scan_kernel<D, false>;
  hipLaunchKernelGGL(kscan, dim3(BH * D / 4), dim3(256), 0, stream, a.W0, partA, wprev, junk, nchunks, nsplit,
                     (const float*)nullptr, (float*)nullptr, 0.0f);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  auto kb = uf ? lact_bwd_scan_kernel<D, true> : lact_bwd_scan_kernel<D, false>;
  hipLaunchKernelGGL(kb, dim3(BH * D / 4), dim3(256), 0, stream, a.W0, a.dW, partA, partB, wprev, dpt, a.dW0, nchunks,
                     nsplit);
  if ((e = hipGetLastError()) != hipSuccess || nchunks == 0) return e;
  int part_len = (chunk + 3) / 4;
  part_len = part_len < 256 ? 256 : part_len;
  part_len = (part_len + 63) / 64 * 64;
  part_len = part_len > (1 << 20) ? (1 << 20) : part_len;   // float32 rows of a part stay below 2^31 bytes
  const int parts = (chunk + part_len - 1) / part_len;
  auto prod = [&](auto kern, int lds) -> hipError_t {
    hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(BH * nchunks * parts), dim3(256), lds, stream, (const bf16*)a.K, (const bf16*)a.V,
                       (const bf16*)a.dO, a.eta, wprev, dpt, (float*)a.dQ, (float*)a.dK, (float*)a.dV, a.deta, T,
                       chunk, nchunks, parts, part_len);
    return hipGetLastError();
  };
  if constexpr (D == 64) return prod(lact_bwd_prod_kernel<D, 3>, LactBwdCfg<D, 3>::LDS);
  if ((e = prod(lact_bwd_prod_kernel<D, 1>, LactBwdCfg<D, 1>::LDS)) != hipSuccess) return e;
  return prod(lact_bwd_prod_kernel<D, 2>, LactBwdCfg<D, 2>::LDS);
}

}  // namespace

bool large_chunk_linear_supported(int64_t dk, int64_t dv, int64_t chunk, int dtype) {
  (void)chunk;
  return dtype == 1 && dk == dv && (dk == 64 || dk == 128);
}

size_t large_chunk_linear_workspace(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t chunk) {
  const int64_t nchunks = (T + chunk - 1) / chunk;
  return (size_t)(B * H * nchunks * (nsplit_of(B * H, nchunks, chunk) + 1) * dk * dv * 4);
}

hipError_t launch_large_chunk_linear(const LargeChunkArgs& a, hipStream_t stream, const Timing& tm) {
  if (a.DK == 64) return launch_lact<64>(a, stream, tm);
  return launch_lact<128>(a, stream, tm);
}

size_t large_chunk_linear_backward_workspace(int64_t B, int64_t H, int64_t T, int64_t d, int64_t chunk) {
  return lact_bwd_layout(B * H, T, d, chunk).total;
}

hipError_t launch_large_chunk_linear_backward(const BackwardArgs& a, hipStream_t stream) {
  return a.DK == 64 ? launch_lact_bwd<64>(a, stream) : launch_lact_bwd<128>(a, stream);
}

}  // namespace ttt
