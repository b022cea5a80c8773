// Per-token TTT with a linear fast weight, chunked parallel form.
//
// Method: one gradient step per token on the binding loss -<k_t W, v_t>
// with rate eta_t, read by q_t after the step, is exactly causal linear
// attention ("Test-Time Training with KV Binding Is Secretly Linear
// Attention", paper summary technical section 2B; podcast at 7:50-8:26):
//     o_t = q_t (W0 + sum_{i<=t} eta_i k_i^T v_i).
// Associativity gives the chunked form (technical section 3 item 4,
// podcast at 13:41): for chunk c of C tokens, with S_0 = W0,
//     O_c = tril(Q_c K_c^T) (diag(eta_c) V_c) + Q_c S_{c-1}
//     S_c = S_{c-1} + K_c^T diag(eta_c) V_c.
//
// bf16 kernel design (gfx950):
//  * one workgroup = one (b,h) pair x one TV-wide tile of d_v; the columns
//    of S are independent, so tiles need no communication.  The tiles of a
//    head are placed on one XCD so their repeated Q/K reads hit that XCD's
//    L2.  The chunk loop is sequential inside the workgroup; S (fp32) lives
//    in MFMA accumulators for the whole sequence.
//  * 4 waves.  Wave w owns i-blocks (16 query tokens) of the chunk for the
//    output and a DK/4-row slab of S for the state update.  A bf16 copy of
//    S is exchanged through LDS (double-buffered) for the Q S product.
//  * Q, K, V, eta of a chunk are streamed HBM -> LDS with asynchronous
//    direct-to-LDS loads through a STAGES-deep ring; waits are explicit
//    vmcnt counts.  Q and K rows are XOR-swizzled in 16-byte units.
//  * Products contracting over tokens (A V and K^T V) read their operands
//    with the LDS transpose read; eta is applied to V when it is read
//    (diag(eta) V rounded once to bf16 and used by both products).
//  * The outputs go LDS -> HBM as 16-byte row pieces one chunk later.
#include "device_common.h"
#include "kernels.h"

namespace ttt {

template <int DK, int C, int TV, int STAGES>
struct PerTokenCfg {
  static constexpr int NW = 4;
  static constexpr int THREADS = NW * WAVE;
  static constexpr int IB = C / 16;
  static constexpr int IBW = IB / NW;
  static constexpr int NT = TV / 16;
  static constexpr int KT = DK / 32;
  static constexpr int KC = C / 32;
  static constexpr int SROWS = DK / NW;
  static constexpr int MT = SROWS / 16;
  static constexpr int CPR = DK / 8;          // 16-byte pieces per Q/K row
  static constexpr int Q_BYTES = C * DK * 2;
  static constexpr int V_BYTES = C * TV * 2;
  static constexpr int E_BYTES = C * 4;
  static constexpr int STAGE_BYTES = 2 * Q_BYTES + V_BYTES + E_BYTES;
  static constexpr int S_ROW = DK * 2 + 16;   // padded bf16 row of S^T
  static constexpr int S_BYTES = TV * S_ROW;
  static constexpr int O_ROW = TV * 2 + 16;
  static constexpr int O_BYTES = C * O_ROW;
  // S^T is exchanged as a pair of bf16 planes (hi + lo), double-buffered
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES + 4 * S_BYTES + 2 * O_BYTES;
  // per-wave memory instructions per chunk
  static constexpr int QI = Q_BYTES / 1024 / NW;
  static constexpr int VPW = C * TV / 8 / NW;   // 16-byte V pieces per wave
  static constexpr int VI = (VPW + 63) / 64;
  static constexpr int LOADS = 2 * QI + VI + 1;
  static constexpr int OI = VI;                 // O pieces per wave equal V pieces
  static constexpr int STEADY_VMCNT = (STAGES - 2) * (LOADS + OI);
  static_assert(IB % NW == 0, "C must be a multiple of 64");
  static_assert(Q_BYTES % (1024 * NW) == 0, "Q tile must split into whole wave loads");
  static_assert(C / NW / 4 <= 64, "eta split");
  static_assert(STEADY_VMCNT < 64, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <int DK, int C, int TV, int STAGES>
__global__ __launch_bounds__(256, 1) void per_token_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const float* __restrict__ eta, const float* __restrict__ W0, bf16* __restrict__ O,
    float* __restrict__ Wout, int T, int DV) {
  using Cfg = PerTokenCfg<DK, C, TV, STAGES>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int NV = DV / TV;
  const int nblocks = gridDim.x;
  const int logical = (nblocks % 8 == 0) ? xcd_logical_block(blockIdx.x, nblocks) : blockIdx.x;
  const int bh = logical / NV;
  const int tv0 = (logical % NV) * TV;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int g = l >> 4;
  const int li = l & 15;
  const int nchunks = (T + C - 1) / C;

  const bf16* Qh = Q + (size_t)bh * T * DK;
  const bf16* Kh = K + (size_t)bh * T * DK;
  const bf16* Vh = V + (size_t)bh * T * DV;
  const float* Eh = eta + (size_t)bh * T;
  bf16* Oh = O + (size_t)bh * T * DV;

  unsigned char* stage_base = smem;
  unsigned char* s_lds = smem + STAGES * Cfg::STAGE_BYTES;
  unsigned char* o_lds = s_lds + 4 * Cfg::S_BYTES;

  // ---- issue the asynchronous loads of one chunk into one stage ----
  auto issue_loads = [&](int c, int stage) {
    unsigned char* st = stage_base + stage * Cfg::STAGE_BYTES;
    const int t0 = c * C;
    // Q and K: slot s (16 B) -> row s / CPR, physical piece s % CPR, logical piece p ^ (row & 7)
#pragma unroll
    for (int k = 0; k < Cfg::QI; ++k) {
      const int s = (w * Cfg::QI + k) * 64 + l;
      const int row = s / Cfg::CPR;
      const int lp = (s % Cfg::CPR) ^ (row & 7);
      const int t = min(t0 + row, T - 1);
      g2lds16(Qh + (size_t)t * DK + lp * 8, st + (w * Cfg::QI + k) * 1024);
    }
#pragma unroll
    for (int k = 0; k < Cfg::QI; ++k) {
      const int s = (w * Cfg::QI + k) * 64 + l;
      const int row = s / Cfg::CPR;
      const int lp = (s % Cfg::CPR) ^ (row & 7);
      const int t = min(t0 + row, T - 1);
      g2lds16(Kh + (size_t)t * DK + lp * 8, st + Cfg::Q_BYTES + (w * Cfg::QI + k) * 1024);
    }
    // V tile: pieces in row-major order, TV/8 pieces per row
#pragma unroll
    for (int k = 0; k < Cfg::VI; ++k) {
      const int pw = k * 64 + l;
      if (pw < Cfg::VPW) {
        const int p = w * Cfg::VPW + pw;
        const int row = p / (TV / 8);
        const int col = (p % (TV / 8)) * 8;
        const int t = min(t0 + row, T - 1);
        g2lds16(Vh + (size_t)t * DV + tv0 + col, st + 2 * Cfg::Q_BYTES + (w * Cfg::VPW + k * 64) * 16);
      }
    }
    // eta: C/4 tokens per wave, 4 bytes per lane
    if (l < C / Cfg::NW) {
      const int t = min(t0 + w * (C / Cfg::NW) + l, T - 1);
      g2lds4(Eh + t, st + 2 * Cfg::Q_BYTES + Cfg::V_BYTES + w * (C / Cfg::NW) * 4);
    }
  };

  // ---- state: S[mt][nt] holds rows w*SROWS + 16mt + 4g + r, column 16nt + li ----
  floatx4 S[Cfg::MT][Cfg::NT];
  const float* W0h = W0 + (size_t)bh * DK * DV;
#pragma unroll
  for (int mt = 0; mt < Cfg::MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < Cfg::NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S[mt][nt][r] = W0h[(size_t)(w * Cfg::SROWS + 16 * mt + 4 * g + r) * DV + tv0 + 16 * nt + li];

  // bf16 hi/lo planes of S^T: S = hi + lo up to 2^-16 relative
  auto write_s_lds = [&](int buf) {
    unsigned char* sb = s_lds + buf * 2 * Cfg::S_BYTES;
#pragma unroll
    for (int mt = 0; mt < Cfg::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < Cfg::NT; ++nt) {
        bf16x4 hi, lo;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          hi[r] = (bf16)S[mt][nt][r];
          lo[r] = (bf16)(S[mt][nt][r] - (float)hi[r]);
        }
        const int off = (16 * nt + li) * Cfg::S_ROW + (w * Cfg::SROWS + 16 * mt + 4 * g) * 2;
        *(bf16x4*)(sb + off) = hi;
        *(bf16x4*)(sb + Cfg::S_BYTES + off) = lo;
      }
  };
  write_s_lds(0);

  auto store_o = [&](int c) {
    const unsigned char* ob = o_lds + (c & 1) * Cfg::O_BYTES;
    const int t0 = c * C;
#pragma unroll
    for (int k = 0; k < Cfg::OI; ++k) {
      const int pw = k * 64 + l;
      if (pw < Cfg::VPW) {
        const int p = w * Cfg::VPW + pw;
        const int row = p / (TV / 8);
        const int col = (p % (TV / 8)) * 8;
        const uint4 v = *(const uint4*)(ob + row * Cfg::O_ROW + col * 2);
        if (t0 + row < T) *(uint4*)(Oh + (size_t)(t0 + row) * DV + tv0 + col) = v;
      }
    }
  };

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nchunks) issue_loads(s, s);

  for (int c = 0; c < nchunks; ++c) {
    if (c >= STAGES - 1 && c + STAGES - 1 <= nchunks)
      wait_vm_barrier<Cfg::STEADY_VMCNT>();
    else
      wait_vm_barrier<0>();
    if (c >= 1) store_o(c - 1);
    if (c + STAGES - 1 < nchunks) issue_loads(c + STAGES - 1, (c + STAGES - 1) % STAGES);

    const unsigned char* st = stage_base + (c % STAGES) * Cfg::STAGE_BYTES;
    const unsigned char* qst = st;
    const unsigned char* kst = st + Cfg::Q_BYTES;
    const unsigned char* vs = st + 2 * Cfg::Q_BYTES;
    const float* es = (const float*)(st + 2 * Cfg::Q_BYTES + Cfg::V_BYTES);
    const unsigned char* sb = s_lds + (c & 1) * 2 * Cfg::S_BYTES;
    const int t0 = c * C;

    // eta of every token row this lane touches (zero past the end of the
    // sequence), raw V operands for A V, and hi/lo bf16 pairs of diag(eta) V
    // for the state update.  Row order of a 32-token step: rows 4g..4g+3
    // then 16+4g..16+4g+3 (the transposed-read order).
    float e[Cfg::KC][2][4];
    bf16x8 vop[Cfg::KC][Cfg::NT], evh[Cfg::KC][Cfg::NT], evl[Cfg::KC][Cfg::NT];
#pragma unroll
    for (int kc = 0; kc < Cfg::KC; ++kc) {
      bf16x4 half[2][Cfg::NT];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rb = 32 * kc + 16 * h + 4 * g;
        const floatx4 e4 = *(const floatx4*)(es + rb);
#pragma unroll
        for (int r = 0; r < 4; ++r) e[kc][h][r] = (t0 + rb + r < T) ? e4[r] : 0.0f;
#pragma unroll
        for (int nt = 0; nt < Cfg::NT; ++nt) {
          const int row = rb + (li >> 2);
          half[h][nt] = lds_read_tr16(vs + row * (TV * 2) + (16 * nt + 4 * (li & 3)) * 2);
        }
      }
#pragma unroll
      for (int nt = 0; nt < Cfg::NT; ++nt) {
        vop[kc][nt] = join(half[0][nt], half[1][nt]);
        bf16x8 hi, lo;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float f = e[kc][h][r] * (float)half[h][nt][r];
            hi[4 * h + r] = (bf16)f;
            lo[4 * h + r] = (bf16)(f - (float)hi[4 * h + r]);
          }
        evh[kc][nt] = hi;
        evl[kc][nt] = lo;
      }
    }

    // outputs of this wave's i-blocks
#pragma unroll
    for (int ibw = 0; ibw < Cfg::IBW; ++ibw) {
      const int ib = (ibw == 0) ? w : (Cfg::IB - 1 - w);
      bf16x8 qop[Cfg::KT];
#pragma unroll
      for (int ks = 0; ks < Cfg::KT; ++ks) {
        const int row = 16 * ib + li;
        const int piece = (4 * ks + g) ^ (row & 7);
        qop[ks] = *(const bf16x8*)(qst + row * (DK * 2) + piece * 16);
      }
      floatx4 acc[Cfg::NT];
#pragma unroll
      for (int nt = 0; nt < Cfg::NT; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
      // intra-chunk: P^T tiles (key rows j, query columns i) for j-blocks
      // 0..ib, scaled by eta_j, causally masked, split into bf16 hi + lo
#pragma unroll
      for (int kc = 0; kc < Cfg::KC; ++kc) {
        if (32 * kc > 16 * ib + 15) break;
        bf16x4 ph[2], pl[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int jb = 2 * kc + h;
          if (jb > ib) {
            ph[h] = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
            pl[h] = ph[h];
            continue;
          }
          floatx4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < Cfg::KT; ++ks) {
            const int row = 16 * jb + li;
            const int piece = (4 * ks + g) ^ (row & 7);
            const bf16x8 kop = *(const bf16x8*)(kst + row * (DK * 2) + piece * 16);
            p = mfma16(kop, qop[ks], p);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float f = p[r] * e[kc][h][r];
            if (jb == ib && 4 * g + r > li) f = 0.f;
            ph[h][r] = (bf16)f;
            pl[h][r] = (bf16)(f - (float)ph[h][r]);
          }
        }
        const bf16x8 ah = join(ph[0], ph[1]);
        const bf16x8 al = join(pl[0], pl[1]);
#pragma unroll
        for (int nt = 0; nt < Cfg::NT; ++nt) {
          acc[nt] = mfma16(ah, vop[kc][nt], acc[nt]);
          acc[nt] = mfma16(al, vop[kc][nt], acc[nt]);
        }
      }
      // inter-chunk: Q (S_hi + S_lo)
#pragma unroll
      for (int nt = 0; nt < Cfg::NT; ++nt)
#pragma unroll
        for (int ks = 0; ks < Cfg::KT; ++ks) {
          const int off = (16 * nt + li) * Cfg::S_ROW + (32 * ks + 8 * g) * 2;
          const bf16x8 sh = *(const bf16x8*)(sb + off);
          const bf16x8 sl = *(const bf16x8*)(sb + Cfg::S_BYTES + off);
          acc[nt] = mfma16(qop[ks], sh, acc[nt]);
          acc[nt] = mfma16(qop[ks], sl, acc[nt]);
        }
      // stage the outputs (bf16) for the coalesced store one chunk later
      unsigned char* ob = o_lds + (c & 1) * Cfg::O_BYTES;
#pragma unroll
      for (int nt = 0; nt < Cfg::NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *(bf16*)(ob + (16 * ib + 4 * g + r) * Cfg::O_ROW + (16 * nt + li) * 2) = (bf16)acc[nt][r];
    }

    // state update: S += K^T diag(eta) V on this wave's rows
#pragma unroll
    for (int mt = 0; mt < Cfg::MT; ++mt) {
      const int m0 = w * Cfg::SROWS + 16 * mt;
#pragma unroll
      for (int kc = 0; kc < Cfg::KC; ++kc) {
        bf16x4 kh[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int row = 32 * kc + 16 * h + 4 * g + (li >> 2);
          const int col = m0 + 4 * (li & 3);
          const int piece = (col >> 3) ^ (row & 7);
          kh[h] = lds_read_tr16(kst + row * (DK * 2) + piece * 16 + (col & 7) * 2);
        }
        const bf16x8 a = join(kh[0], kh[1]);
#pragma unroll
        for (int nt = 0; nt < Cfg::NT; ++nt) {
          S[mt][nt] = mfma16(a, evh[kc][nt], S[mt][nt]);
          S[mt][nt] = mfma16(a, evl[kc][nt], S[mt][nt]);
        }
      }
    }
    write_s_lds((c + 1) & 1);
  }

  wait_vm_barrier<0>();
  if (nchunks > 0) store_o(nchunks - 1);
  float* Wh = Wout + (size_t)bh * DK * DV;
#pragma unroll
  for (int mt = 0; mt < Cfg::MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < Cfg::NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Wh[(size_t)(w * Cfg::SROWS + 16 * mt + 4 * g + r) * DV + tv0 + 16 * nt + li] = S[mt][nt][r];
}

// ---------------------------------------------------------------------------
// fp32 kernel: same chunked form on the vector ALUs, everything staged in
// LDS.  Used for float32 inputs where bf16 rounding would exceed the fp32
// accuracy budget.  One workgroup per (b,h) x 32-column tile of d_v.
// ---------------------------------------------------------------------------
template <int DK, int C>
__global__ __launch_bounds__(256) void per_token_fp32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ eta, const float* __restrict__ W0, float* __restrict__ O,
    float* __restrict__ Wout, int T, int DV) {
  constexpr int TV = 32;
  constexpr int QP = DK + 1;  // padded rows
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* q = (float*)smem;              // [C][QP]
  float* k = q + C * QP;                // [C][QP]
  float* v = k + C * QP;                // [C][TV]
  float* e = v + C * TV;                // [C]
  float* p = e + C;                     // [C][C+1]
  float* s = p + C * (C + 1);           // [DK][TV]
  const int NV = DV / TV;
  const int bh = blockIdx.x / NV;
  const int tv0 = (blockIdx.x % NV) * TV;
  const int tid = threadIdx.x;
  const float* Qh = Q + (size_t)bh * T * DK;
  const float* Kh = K + (size_t)bh * T * DK;
  const float* Vh = V + (size_t)bh * T * DV;
  const float* Eh = eta + (size_t)bh * T;
  float* Oh = O + (size_t)bh * T * DV;
  for (int i = tid; i < DK * TV; i += 256) s[i] = W0[(size_t)bh * DK * DV + (size_t)(i / TV) * DV + tv0 + i % TV];
  const int nchunks = (T + C - 1) / C;
  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * C;
    __syncthreads();
    for (int i = tid; i < C * DK; i += 256) {
      const int r = i / DK, a = i % DK;
      const bool ok = t0 + r < T;
      q[r * QP + a] = ok ? Qh[(size_t)(t0 + r) * DK + a] : 0.f;
      k[r * QP + a] = ok ? Kh[(size_t)(t0 + r) * DK + a] : 0.f;
    }
    for (int i = tid; i < C * TV; i += 256) {
      const int r = i / TV, n = i % TV;
      v[i] = (t0 + r < T) ? Vh[(size_t)(t0 + r) * DV + tv0 + n] : 0.f;
    }
    for (int i = tid; i < C; i += 256) e[i] = (t0 + i < T) ? Eh[t0 + i] : 0.f;
    __syncthreads();
    // scores with the causal mask (diagonal included) and eta of the key token
    for (int idx = tid; idx < C * C; idx += 256) {
      const int i = idx / C, j = idx % C;
      float acc = 0.f;
      if (j <= i) {
        for (int a = 0; a < DK; ++a) acc = fmaf(q[i * QP + a], k[j * QP + a], acc);
        acc *= e[j];
      }
      p[i * (C + 1) + j] = acc;
    }
    __syncthreads();
    for (int idx = tid; idx < C * TV; idx += 256) {
      const int i = idx / TV, n = idx % TV;
      float acc = 0.f;
      for (int j = 0; j <= i; ++j) acc = fmaf(p[i * (C + 1) + j], v[j * TV + n], acc);
      for (int a = 0; a < DK; ++a) acc = fmaf(q[i * QP + a], s[a * TV + n], acc);
      if (t0 + i < T) Oh[(size_t)(t0 + i) * DV + tv0 + n] = acc;
    }
    __syncthreads();
    for (int idx = tid; idx < DK * TV; idx += 256) {
      const int a = idx / TV, n = idx % TV;
      float acc = s[idx];
      for (int j = 0; j < C; ++j) acc = fmaf(k[j * QP + a] * e[j], v[j * TV + n], acc);
      s[idx] = acc;
    }
  }
  __syncthreads();
  for (int i = tid; i < DK * TV; i += 256) Wout[(size_t)bh * DK * DV + (size_t)(i / TV) * DV + tv0 + i % TV] = s[i];
}

template <int DK, int C>
static size_t fp32_lds_bytes() {
  return sizeof(float) * (2 * C * (DK + 1) + C * 32 + C + C * (C + 1) + DK * 32);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int DK, int C, int TV, int STAGES>
static hipError_t launch_bf16(const PerTokenArgs& a, hipStream_t stream) {
  using Cfg = PerTokenCfg<DK, C, TV, STAGES>;
  auto kern = per_token_bf16_kernel<DK, C, TV, STAGES>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int grid = (int)(a.B * a.H * (a.DV / TV));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(Cfg::THREADS), Cfg::LDS_BYTES, stream,
                     (const bf16*)a.Q, (const bf16*)a.K, (const bf16*)a.V, a.eta, a.W0, (bf16*)a.O, a.W_out,
                     (int)a.T, (int)a.DV);
  return hipGetLastError();
}

template <int DK, int C>
static hipError_t launch_fp32(const PerTokenArgs& a, hipStream_t stream) {
  auto kern = per_token_fp32_kernel<DK, C>;
  const size_t lds = fp32_lds_bytes<DK, C>();
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int grid = (int)(a.B * a.H * (a.DV / 32));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, stream, (const float*)a.Q, (const float*)a.K,
                     (const float*)a.V, a.eta, a.W0, (float*)a.O, a.W_out, (int)a.T, (int)a.DV);
  return hipGetLastError();
}

bool per_token_supported(int64_t dk, int64_t dv, int64_t chunk, int dtype) {
  if (dk != dv || (dk != 64 && dk != 128)) return false;
  if (chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128) return false;
  if (dtype == 0 && chunk > 64) return false;
  return true;
}

// Tile plan for the bf16 kernel: enough workgroups to cover the CUs while
// keeping the per-tile recomputation of Q K^T small.
int per_token_bf16_tv(int64_t BH, int64_t dv) {
  if (BH * (dv / 32) < 256) return 16;
  if (dv == 64 && BH * (dv / 64) >= 512) return 64;
  return 32;
}

hipError_t launch_per_token(const PerTokenArgs& a, hipStream_t stream) {
  if (a.dtype == 0) {
    const int c = a.chunk <= 16 ? 16 : a.chunk <= 32 ? 32 : 64;
    if (a.DK == 64) return c == 16 ? launch_fp32<64, 16>(a, stream) : c == 32 ? launch_fp32<64, 32>(a, stream) : launch_fp32<64, 64>(a, stream);
    return c == 16 ? launch_fp32<128, 16>(a, stream) : c == 32 ? launch_fp32<128, 32>(a, stream) : launch_fp32<128, 64>(a, stream);
  }
  const int tv = per_token_bf16_tv(a.B * a.H, a.DV);
  if (a.DK == 128) {
    if (tv == 16) return launch_bf16<128, 64, 16, 3>(a, stream);
    return launch_bf16<128, 64, 32, 3>(a, stream);
  }
  if (tv == 16) return launch_bf16<64, 64, 16, 4>(a, stream);
  if (tv == 64) return launch_bf16<64, 64, 64, 4>(a, stream);
  return launch_bf16<64, 64, 32, 4>(a, stream);
}

}  // namespace ttt
