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
// for every chunk in parallel; only the normalise-scan is sequential:
//   1. lact_delta_kernel  - partial dW over token slices of every chunk
//                           (bf16 MFMA, diag(eta) V split into bf16 hi+lo)
//   2. lact_scan_kernel   - per head: sum the partials, add, normalise,
//                           keep W_{c-1} of every chunk (transposed, fp32)
//   3. lact_read_kernel   - O_c = Q_c W_{c-1} for all chunks in parallel
//                           (W split into bf16 hi+lo)
#include "device_common.h"
#include "kernels.h"

namespace ttt {

namespace {

constexpr int LC_STEP = 64;     // tokens per LDS step in the update kernel
constexpr int LC_SLICE = 1024;  // tokens per workgroup slice of a chunk
constexpr int LC_READ_TILE = 64;

inline int64_t nsplit_of(int64_t chunk) { return (chunk + LC_SLICE - 1) / LC_SLICE; }

// ---------------------------------------------------------------------------
// 1. partial dW = sum_{t in slice} k_t^T (eta_t v_t), one slice per workgroup
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void lact_delta_kernel(const bf16* __restrict__ K, const bf16* __restrict__ V,
                                                         const float* __restrict__ eta, float* __restrict__ part,
                                                         int T, int chunk, int nchunks, int nsplit) {
  constexpr int ROW = D * 2 + 32;              // padded LDS row (bytes)
  constexpr int PIECES = LC_STEP * D / 8;      // 16-byte pieces per tile
  constexpr int PPT = PIECES / 256;            // pieces per thread
  constexpr int QW = D / 2;                    // quadrant width per wave
  constexpr int TW = QW / 32;                  // 32x32 tiles per quadrant side
  __shared__ __attribute__((aligned(16))) unsigned char ks[2][LC_STEP * ROW];
  __shared__ __attribute__((aligned(16))) unsigned char vh[2][LC_STEP * ROW];
  __shared__ __attribute__((aligned(16))) unsigned char vl[2][LC_STEP * ROW];

  const int split = blockIdx.x % nsplit;
  const int c = (blockIdx.x / nsplit) % nchunks;
  const int bh = blockIdx.x / (nsplit * nchunks);
  const int cstart = c * chunk;
  const int cend = min(cstart + chunk, T);
  const int s0 = cstart + split * LC_SLICE;
  const int s1 = min(s0 + LC_SLICE, cend);
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
      kreg[k] = *(const uint4*)(Kh + (size_t)tc * D + col);
      vreg[k] = *(const uint4*)(Vh + (size_t)tc * D + col);
      ereg[k] = t < s1 ? Eh[tc] : 0.f;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int p = k * 256 + tid;
      const int row = p / (D / 8), col = (p % (D / 8)) * 8;
      *(uint4*)(ks[buf] + row * ROW + col * 2) = kreg[k];
      const bf16x8 v = __builtin_bit_cast(bf16x8, vreg[k]);
      bf16x8 hi, lo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float f = ereg[k] * (float)v[j];
        hi[j] = (bf16)f;
        lo[j] = (bf16)(f - (float)hi[j]);
      }
      *(bf16x8*)(vh[buf] + row * ROW + col * 2) = hi;
      *(bf16x8*)(vl[buf] + row * ROW + col * 2) = lo;
    }
  };

  floatx16 acc[TW][TW];
#pragma unroll
  for (int i = 0; i < TW; ++i)
#pragma unroll
    for (int j = 0; j < TW; ++j) acc[i][j] = floatx16{};
  const int a0 = (w >> 1) * QW, b0 = (w & 1) * QW;
  const int nsteps = (s1 - s0 + LC_STEP - 1) / LC_STEP;
  if (nsteps > 0) {
    load(s0);
    store(0);
  }
  __syncthreads();
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    if (st + 1 < nsteps) load(s0 + (st + 1) * LC_STEP);
#pragma unroll
    for (int k0 = 0; k0 < LC_STEP; k0 += 16) {
      // operands with tokens as the contraction index, via transposed reads
      const int r0 = k0 + 8 * (G >> 1) + (L >> 2);
      bf16x8 A[TW], Bh[TW], Bl[TW];
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        const int ca = a0 + 32 * i + 16 * (G & 1) + 4 * (L & 3);
        A[i] = join(lds_read_tr16(ks[buf] + r0 * ROW + ca * 2), lds_read_tr16(ks[buf] + (r0 + 4) * ROW + ca * 2));
        const int cb = b0 + 32 * i + 16 * (G & 1) + 4 * (L & 3);
        Bh[i] = join(lds_read_tr16(vh[buf] + r0 * ROW + cb * 2), lds_read_tr16(vh[buf] + (r0 + 4) * ROW + cb * 2));
        Bl[i] = join(lds_read_tr16(vl[buf] + r0 * ROW + cb * 2), lds_read_tr16(vl[buf] + (r0 + 4) * ROW + cb * 2));
      }
#pragma unroll
      for (int i = 0; i < TW; ++i)
#pragma unroll
        for (int j = 0; j < TW; ++j) {
          acc[i][j] = mfma32(A[i], Bh[j], acc[i][j]);
          acc[i][j] = mfma32(A[i], Bl[j], acc[i][j]);
        }
    }
    if (st + 1 < nsteps) store(buf ^ 1);
    __syncthreads();
  }
  float* P = part + (((size_t)bh * nchunks + c) * nsplit + split) * D * D;
#pragma unroll
  for (int i = 0; i < TW; ++i)
#pragma unroll
    for (int j = 0; j < TW; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int a = a0 + 32 * i + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        const int b = b0 + 32 * j + (l & 31);
        P[(size_t)a * D + b] = acc[i][j][r];
      }
}

// ---------------------------------------------------------------------------
// 2. normalise-scan, one workgroup per (b,h).  Wave w owns columns
//    [w*D/4, (w+1)*D/4); a column's rows are spread over 64/(D/4) lanes.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void lact_scan_kernel(const float* __restrict__ W0, const float* __restrict__ part,
                                                        float* __restrict__ wprev_t, float* __restrict__ Wout,
                                                        int nchunks, int nsplit) {
  constexpr int CPW = D / 4;          // columns per wave
  constexpr int LPC = 64 / CPW;       // lanes per column
  constexpr int RPL = D / LPC;        // rows per lane
  const int bh = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int col = w * CPW + (l % CPW);
  const int rbase = (l / CPW) * RPL;
  float Wr[RPL];
  const float* W0h = W0 + (size_t)bh * D * D;
#pragma unroll
  for (int r = 0; r < RPL; ++r) Wr[r] = W0h[(size_t)(rbase + r) * D + col];
  float nxt[RPL];
  auto fetch = [&](int c) {
#pragma unroll
    for (int r = 0; r < RPL; ++r) nxt[r] = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float* P = part + (((size_t)bh * nchunks + c) * nsplit + s) * D * D;
#pragma unroll
      for (int r = 0; r < RPL; ++r) nxt[r] += P[(size_t)(rbase + r) * D + col];
    }
  };
  if (nchunks > 0) fetch(0);
  for (int c = 0; c < nchunks; ++c) {
    // keep W_{c-1} for the read kernel, transposed: wprev_t[c][col][row]
    float* Wt = wprev_t + ((size_t)bh * nchunks + c) * D * D + (size_t)col * D + rbase;
#pragma unroll
    for (int r = 0; r < RPL; r += 4) *(floatx4*)(Wt + r) = floatx4{Wr[r], Wr[r + 1], Wr[r + 2], Wr[r + 3]};
    float d[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) d[r] = nxt[r];
    if (c + 1 < nchunks) fetch(c + 1);
    float ss = 0.f;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      Wr[r] += d[r];
      ss = fmaf(Wr[r], Wr[r], ss);
    }
#pragma unroll
    for (int m = CPW; m < 64; m <<= 1) ss += __shfl_xor(ss, m);
    const float inv = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
#pragma unroll
    for (int r = 0; r < RPL; ++r) Wr[r] *= inv;
  }
  float* Wo = Wout + (size_t)bh * D * D;
#pragma unroll
  for (int r = 0; r < RPL; ++r) Wo[(size_t)(rbase + r) * D + col] = Wr[r];
}

// ---------------------------------------------------------------------------
// 3. O_c = Q_c W_{c-1}.  One workgroup per 64-token tile of a chunk; wave w
//    computes output columns [w*D/4, (w+1)*D/4) as O^T = W^T Q^T with W in
//    bf16 hi+lo.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void lact_read_kernel(const bf16* __restrict__ Q, const float* __restrict__ wprev_t,
                                                        bf16* __restrict__ O, int T, int chunk, int nchunks,
                                                        int tiles_per_chunk) {
  constexpr int MTW = D / 64;   // 16-row M tiles (output columns) per wave
  constexpr int KS = D / 32;
  const int tile = blockIdx.x % tiles_per_chunk;
  const int c = (blockIdx.x / tiles_per_chunk) % nchunks;
  const int bh = blockIdx.x / (tiles_per_chunk * nchunks);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, li = l & 15;
  const int cend = min((c + 1) * chunk, T);
  const int t0 = c * chunk + tile * LC_READ_TILE;
  if (t0 >= cend) return;
  const float* Wt = wprev_t + ((size_t)bh * nchunks + c) * D * D;
  bf16x8 wh[MTW][KS], wl[MTW][KS];
#pragma unroll
  for (int m = 0; m < MTW; ++m)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const float* p = Wt + (size_t)(w * (D / 4) + 16 * m + li) * D + 32 * s + 8 * g;
      const floatx4 x0 = *(const floatx4*)p, x1 = *(const floatx4*)(p + 4);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float f = j < 4 ? x0[j] : x1[j - 4];
        wh[m][s][j] = (bf16)f;
        wl[m][s][j] = (bf16)(f - (float)wh[m][s][j]);
      }
    }
  const bf16* Qh = Q + (size_t)bh * T * D;
  bf16* Oh = O + (size_t)bh * T * D;
#pragma unroll
  for (int nt = 0; nt < LC_READ_TILE / 16; ++nt) {
    const int t = t0 + 16 * nt + li;
    const int tc = min(t, cend - 1);
    bf16x8 qop[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qop[s] = *(const bf16x8*)(Qh + (size_t)tc * D + 32 * s + 8 * g);
#pragma unroll
    for (int m = 0; m < MTW; ++m) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        acc = mfma16(wh[m][s], qop[s], acc);
        acc = mfma16(wl[m][s], qop[s], acc);
      }
      if (t < cend) *(bf16x4*)(Oh + (size_t)t * D + w * (D / 4) + 16 * m + 4 * g) = to_bf16x4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
}

template <int D>
hipError_t launch_lact(const LargeChunkArgs& a, hipStream_t stream) {
  const int T = (int)a.T, chunk = (int)a.chunk;
  const int nchunks = (int)((a.T + a.chunk - 1) / a.chunk);
  const int nsplit = (int)nsplit_of(a.chunk);
  const int BH = (int)(a.B * a.H);
  float* part = (float*)a.ws;
  float* wprev = part + (size_t)BH * nchunks * nsplit * D * D;
  if (nchunks > 0) {
    hipLaunchKernelGGL(lact_delta_kernel<D>, dim3(BH * nchunks * nsplit), dim3(256), 0, stream,
                       (const bf16*)a.K, (const bf16*)a.V, a.eta, part, T, chunk, nchunks, nsplit);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(lact_scan_kernel<D>, dim3(BH), dim3(256), 0, stream, a.W0, part, wprev, a.W_out, nchunks,
                     nsplit);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nchunks == 0) return e;
  const int tiles = (chunk + LC_READ_TILE - 1) / LC_READ_TILE;
  hipLaunchKernelGGL(lact_read_kernel<D>, dim3(BH * nchunks * tiles), dim3(256), 0, stream, (const bf16*)a.Q, wprev,
                     (bf16*)a.O, T, chunk, nchunks, tiles);
  return hipGetLastError();
}

}  // namespace

bool large_chunk_linear_supported(int64_t dk, int64_t dv, int64_t chunk, int dtype) {
  (void)chunk;
  return dtype == 1 && dk == dv && (dk == 64 || dk == 128);
}

size_t large_chunk_linear_workspace(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t chunk) {
  const int64_t nchunks = (T + chunk - 1) / chunk;
  return (size_t)(B * H * nchunks * (nsplit_of(chunk) + 1) * dk * dv * 4);
}

hipError_t launch_large_chunk_linear(const LargeChunkArgs& a, hipStream_t stream) {
  if (a.DK == 64) return launch_lact<64>(a, stream);
  return launch_lact<128>(a, stream);
}

}  // namespace ttt
