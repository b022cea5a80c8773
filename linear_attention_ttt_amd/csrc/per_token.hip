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
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace ttt {

// bf16 kernel, one 64-token tile per step, two phases per step:
//   phase 1: the 10 score tiles P^T(jb, ib) = K_jb Q_ib^T (jb <= ib) are
//            spread evenly over the 4 waves, scaled by eta_j, masked and
//            split into bf16 hi + lo in LDS; each wave w starts its outputs
//            O_w^T = S_{c-1}^T Q_w^T for the queries 16w..16w+15; the
//            diag(eta) V planes of the next tile are prepared.
//   phase 2: O_w^T += V^T A_w^T (A from the score tiles), stored to HBM;
//            S += K^T (diag(eta) V) on the wave's DK/4-row slab; the new S is
//            written to LDS for the next step.
// Outputs are computed transposed so one lane holds 4 consecutive output
// columns of one token: an 8-byte store per lane.  Each wave runs its own
// instantiation of the program (the wave index is a template parameter) so
// every tile index and LDS offset is a compile-time constant added to a
// handful of per-lane offsets computed once.
template <int DK, int TV, int NW_>
struct PerTokenCfg {
  static constexpr int C = 64;                 // tokens per tile
  static constexpr int NW = NW_;               // 4 waves, or 8 (two per SIMD) when there are >= 2 column tiles
  static constexpr int THREADS = NW * WAVE;
  static constexpr int QKSTAGES = 3;           // Q and K rings
  static constexpr int VSTAGES = 4;            // V / eta ring: prefetched one tile further
  static constexpr int NT = TV / 16;
  static constexpr int GW = NW / 4;            // waves sharing one query block / state slab
  static constexpr int NTW = NT / GW;          // 16-column tiles per wave
  static constexpr int KT = DK / 32;
  static constexpr int MTW = DK / 64;          // 16-row m-tiles of S per wave
  static constexpr int CPR = DK / 8;           // 16-byte pieces per Q/K row
  static constexpr int SWZ = CPR >= 16 ? 15 : CPR - 1;  // XOR swizzle of 16-byte pieces by row
  static constexpr int ROWB = DK * 2;
  static constexpr int QK_BYTES = C * ROWB;
  static constexpr int V_BYTES = C * TV * 2;
  static constexpr int E_BYTES = C * 4;
  static constexpr int S_BYTES = TV * ROWB;    // one bf16 plane of S^T [TV][DK], swizzled like Q/K
  static constexpr int P_BYTES = 10 * 64 * 8;  // one plane of the 10 score tiles, 8 bytes per lane
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_K = OFF_Q + QKSTAGES * QK_BYTES;
  static constexpr int OFF_V = OFF_K + QKSTAGES * QK_BYTES;
  static constexpr int OFF_E = OFF_V + VSTAGES * V_BYTES;
  static constexpr int OFF_EV = OFF_E + VSTAGES * E_BYTES;   // [2 buffers][hi, lo]
  static constexpr int OFF_S = OFF_EV + 4 * V_BYTES;         // [hi, lo]
  static constexpr int OFF_P = OFF_S + 2 * S_BYTES;          // [hi, lo]
  static constexpr int LDS_BYTES = OFF_P + 2 * P_BYTES;
  // per-wave vector-memory instructions issued every step
  static constexpr int QI = QK_BYTES / 1024 / NW;
  static constexpr int VPW = C * TV / 8 / NW;  // 16-byte V pieces per wave
  static constexpr int VI = (VPW + 63) / 64;
  static constexpr int OPS = 2 * QI + VI + 1 /*eta*/ + NTW /*O stores*/;
  static_assert(NT % GW == 0, "column tiles must split evenly over the waves of a block");
  static_assert(QK_BYTES % (1024 * NW) == 0, "Q/K tile must split into whole wave loads");
  static_assert(OPS < 64, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// score tile t (0..9) <-> (jb, ib), jb <= ib; wave w owns tiles [tile_begin(w), tile_begin(w+1))
__host__ __device__ constexpr int ptile_jb(int t) { return t < 1 ? 0 : t < 3 ? t - 1 : t < 6 ? t - 3 : t - 6; }
__host__ __device__ constexpr int ptile_ib(int t) { return t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3; }
__host__ __device__ constexpr int ptile_index(int jb, int ib) { return ib * (ib + 1) / 2 + jb; }
__host__ __device__ constexpr int tile_begin4(int w) { return w == 0 ? 0 : w == 1 ? 3 : w == 2 ? 6 : w == 3 ? 8 : 10; }
__host__ __device__ constexpr int tile_begin8(int w) { return w <= 3 ? 2 * w : w <= 7 ? w + 3 : 10; }
template <int NW>
__host__ __device__ constexpr int tile_begin(int w) { return NW == 4 ? tile_begin4(w) : tile_begin8(w); }

struct PerTokenPtrs {
  const bf16* Qh;
  const bf16* Kh;
  const bf16* Vh;
  const float* Eh;
  bf16* Oh;
  const float* W0h;
  float* Wh;
  int T, DV, tv0;
};

template <int DK, int TV, int NW, int W>
__device__ __forceinline__ void per_token_wave(const PerTokenPtrs& P, unsigned char* smem, int l) {
  using Cfg = PerTokenCfg<DK, TV, NW>;
  constexpr int C = Cfg::C;
  constexpr int ROWB = Cfg::ROWB;
  constexpr int SWZ = Cfg::SWZ;
  constexpr int IB = W / Cfg::GW;              // this wave's query block (16 queries)
  constexpr int NT0 = (W % Cfg::GW) * Cfg::NTW;  // first of this wave's column tiles
  constexpr int SLAB = DK / 4 * IB;            // first state row of this wave
  const int g = l >> 4;
  const int li = l & 15;
  const int tid = W * 64 + l;
  const int T = P.T, DV = P.DV, tv0 = P.tv0;
  const int nchunks = (T + C - 1) / C;

  // ---- per-lane byte offsets, fixed for the whole sequence ----
  unsigned qkoff[Cfg::QI];                     // DMA: global offset of LDS slot (W*QI + k)*64 + l
#pragma unroll
  for (int k = 0; k < Cfg::QI; ++k) {
    const int s = (W * Cfg::QI + k) * 64 + l;
    const int row = s / Cfg::CPR;
    qkoff[k] = (unsigned)(row * ROWB + (((s % Cfg::CPR) ^ (row & SWZ)) << 4));
  }
  unsigned voff[Cfg::VI];
#pragma unroll
  for (int k = 0; k < Cfg::VI; ++k) {
    const int p = W * Cfg::VPW + k * 64 + l;
    voff[k] = (unsigned)((p / (TV / 8)) * DV * 2 + (tv0 + (p % (TV / 8)) * 8) * 2);
  }
  // natural 16-byte operand reads: row 16*blk + li, d = 32*ks + 8g  ->  blk*16*ROWB + nat[ks]
  int nat[Cfg::KT];
#pragma unroll
  for (int ks = 0; ks < Cfg::KT; ++ks) nat[ks] = li * ROWB + ((((4 * ks + g) ^ (li & SWZ))) << 4);
  // S^T plane writes: row n = 16nt + li, d_k = SLAB + 16j + 4g  ->  nt*16*ROWB + swr[j]
  int swr[Cfg::MTW];
#pragma unroll
  for (int j = 0; j < Cfg::MTW; ++j) {
    const int k = SLAB + 16 * j + 4 * g;
    swr[j] = li * ROWB + ((((k >> 3) ^ (li & SWZ))) << 4) + (k & 7) * 2;
  }
  // transposed K reads for the state update: rows 32kc + 16h + 4g + li/4, cols SLAB + 16j + 4(li%4)
  int ktr[Cfg::MTW];
#pragma unroll
  for (int j = 0; j < Cfg::MTW; ++j) {
    const int r = 4 * g + (li >> 2), col = SLAB + 16 * j + 4 * (li & 3);
    ktr[j] = r * ROWB + ((((col >> 3) ^ (r & SWZ))) << 4) + (col & 7) * 2;
  }
  const int vtr = (4 * g + (li >> 2)) * (TV * 2) + 4 * (li & 3) * 2;   // + (32kc + 16h)*TV*2 + 32nt
  const unsigned ooff = (unsigned)((16 * IB + li) * DV * 2 + (tv0 + 16 * NT0 + 4 * g) * 2);

  auto issue_qk = [&](int c, int slot) {
    const long long rem = (long long)T - (long long)c * C;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(P.Qh + (size_t)c * C * DK, rem * ROWB);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(P.Kh + (size_t)c * C * DK, rem * ROWB);
    unsigned char* dq = smem + Cfg::OFF_Q + slot * Cfg::QK_BYTES + W * Cfg::QI * 1024;
    unsigned char* dk = smem + Cfg::OFF_K + slot * Cfg::QK_BYTES + W * Cfg::QI * 1024;
#pragma unroll
    for (int k = 0; k < Cfg::QI; ++k) buf2lds16(rq, qkoff[k], dq + k * 1024);
#pragma unroll
    for (int k = 0; k < Cfg::QI; ++k) buf2lds16(rk, qkoff[k], dk + k * 1024);
  };
  auto issue_ve = [&](int c, int slot) {
    const long long rem = (long long)T - (long long)c * C;
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(P.Vh + (size_t)c * C * DV, rem * DV * 2);
    unsigned char* dst = smem + Cfg::OFF_V + slot * Cfg::V_BYTES + W * Cfg::VPW * 16;
#pragma unroll
    for (int k = 0; k < Cfg::VI; ++k)
      if (k * 64 + l < Cfg::VPW) buf2lds16(rv, voff[k], dst + k * 1024);
    const __amdgpu_buffer_rsrc_t re = make_rsrc(P.Eh + (size_t)c * C, rem * 4);
    if (l < C / Cfg::NW)
      buf2lds4(re, (unsigned)((W * (C / Cfg::NW) + l) * 4), smem + Cfg::OFF_E + slot * Cfg::E_BYTES + W * (C / Cfg::NW) * 4);
  };
  // diag(eta) V of one tile as bf16 hi + lo planes (same layout as the V tile)
  auto convert_ev = [&](int vslot, int buf) {
    const unsigned char* vs = smem + Cfg::OFF_V + vslot * Cfg::V_BYTES;
    const float* es = (const float*)(smem + Cfg::OFF_E + vslot * Cfg::E_BYTES);
    unsigned char* eh = smem + Cfg::OFF_EV + buf * 2 * Cfg::V_BYTES;
#pragma unroll
    for (int p0 = 0; p0 < C * TV / 8; p0 += Cfg::THREADS) {
      const int p = p0 + tid;
      if (p < C * TV / 8) {
        const bf16x8 v = *(const bf16x8*)(vs + p * 16);
        const float e = es[p / (TV / 8)];
        bf16x8 hi, lo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float f = e * (float)v[j];
          hi[j] = (bf16)f;
          lo[j] = (bf16)(f - (float)hi[j]);
        }
        *(bf16x8*)(eh + p * 16) = hi;
        *(bf16x8*)(eh + Cfg::V_BYTES + p * 16) = lo;
      }
    }
  };

  // ---- state: S[j][n] holds rows SLAB + 16j + 4g + r, column 16(NT0 + n) + li ----
  floatx4 S[Cfg::MTW][Cfg::NTW];
#pragma unroll
  for (int j = 0; j < Cfg::MTW; ++j)
#pragma unroll
    for (int n = 0; n < Cfg::NTW; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S[j][n][r] = P.W0h[(size_t)(SLAB + 16 * j + 4 * g + r) * DV + tv0 + 16 * (NT0 + n) + li];
  auto write_s_lds = [&]() {
    unsigned char* sb = smem + Cfg::OFF_S;
#pragma unroll
    for (int j = 0; j < Cfg::MTW; ++j)
#pragma unroll
      for (int n = 0; n < Cfg::NTW; ++n) {
        const int nt = NT0 + n;
        bf16x4 hi, lo;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          hi[r] = (bf16)S[j][n][r];
          lo[r] = (bf16)(S[j][n][r] - (float)hi[r]);
        }
        *(bf16x4*)(sb + nt * 16 * ROWB + swr[j]) = hi;
        *(bf16x4*)(sb + Cfg::S_BYTES + nt * 16 * ROWB + swr[j]) = lo;
      }
  };

  if (nchunks > 0) {
    write_s_lds();
    issue_qk(0, 0);
    issue_ve(0, 0);
    issue_qk(1, 1);
    issue_ve(1, 1);
    issue_ve(2, 2);
    wait_vm_barrier<0>();
    convert_ev(0, 0);
  }

  int qslot = 0, vslot = 0;
  for (int c = 0; c < nchunks; ++c) {
    // loads of tile c landed, and V/eta of tile c+1; all of step c-1 done
    if (c >= 1)
      wait_vm_barrier<Cfg::OPS>();
    else
      wait_vm_barrier<0>();
    const int qslot2 = qslot == 0 ? 2 : qslot - 1;          // (c + 2) % 3
    const int vslot1 = (vslot + 1) & 3, vslot3 = (vslot + 3) & 3;
    // prefetch: Q/K of tile c+2, V/eta of tile c+3 (past the end: empty resources)
    issue_qk(c + 2, qslot2);
    issue_ve(c + 3, vslot3);

    const unsigned char* qst = smem + Cfg::OFF_Q + qslot * Cfg::QK_BYTES;
    const unsigned char* kst = smem + Cfg::OFF_K + qslot * Cfg::QK_BYTES;
    const unsigned char* vs = smem + Cfg::OFF_V + vslot * Cfg::V_BYTES;
    const float* es = (const float*)(smem + Cfg::OFF_E + vslot * Cfg::E_BYTES);
    const unsigned char* evb = smem + Cfg::OFF_EV + (c & 1) * 2 * Cfg::V_BYTES;
    const unsigned char* sb = smem + Cfg::OFF_S;
    unsigned char* pb = smem + Cfg::OFF_P;

    // ---- phase 1a: this wave's score tiles ----
#pragma unroll
    for (int t = tile_begin<NW>(W); t < tile_begin<NW>(W + 1); ++t) {
      const int jb = ptile_jb(t), ib = ptile_ib(t);
      floatx4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < Cfg::KT; ++ks) {
        const bf16x8 kop = *(const bf16x8*)(kst + jb * 16 * ROWB + nat[ks]);
        const bf16x8 qop = *(const bf16x8*)(qst + ib * 16 * ROWB + nat[ks]);
        p = mfma16(kop, qop, p);
      }
      const floatx4 e4 = *(const floatx4*)(es + 16 * jb + 4 * g);
      bf16x4 hi, lo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float f = p[r] * e4[r];
        if (jb == ib && 4 * g + r > li) f = 0.f;
        hi[r] = (bf16)f;
        lo[r] = (bf16)(f - (float)hi[r]);
      }
      *(bf16x4*)(pb + t * 512 + l * 8) = hi;
      *(bf16x4*)(pb + Cfg::P_BYTES + t * 512 + l * 8) = lo;
    }
    // ---- phase 1b: O_w^T = S^T Q_w^T (S as bf16 hi + lo) ----
    bf16x8 qop[Cfg::KT];
#pragma unroll
    for (int ks = 0; ks < Cfg::KT; ++ks) qop[ks] = *(const bf16x8*)(qst + IB * 16 * ROWB + nat[ks]);
    floatx4 acc[Cfg::NTW];
#pragma unroll
    for (int n = 0; n < Cfg::NTW; ++n) {
      const int nt = NT0 + n;
      acc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < Cfg::KT; ++ks) {
        acc[n] = mfma16(*(const bf16x8*)(sb + nt * 16 * ROWB + nat[ks]), qop[ks], acc[n]);
        acc[n] = mfma16(*(const bf16x8*)(sb + Cfg::S_BYTES + nt * 16 * ROWB + nat[ks]), qop[ks], acc[n]);
      }
    }
    // ---- phase 1c: diag(eta) V planes of tile c+1 ----
    if (c + 1 < nchunks) convert_ev(vslot1, (c + 1) & 1);
    barrier();

    // ---- phase 2a: O_w^T += V^T A_w^T over key blocks 0..IB ----
    constexpr int NKC = IB / 2 + 1;
    bf16x4 vtr_[NKC * Cfg::NTW * 2];
    {
      unsigned ad[NKC * Cfg::NTW * 2];
      const unsigned vb0 = lds_addr(vs) + vtr;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int n = 0; n < Cfg::NTW; ++n) {
          const unsigned o0 = vb0 + 32 * kc * TV * 2 + 32 * (NT0 + n);
          ad[(kc * Cfg::NTW + n) * 2] = o0;
          ad[(kc * Cfg::NTW + n) * 2 + 1] = o0 + 16 * TV * 2;
        }
      lds_tr16_batch<NKC * Cfg::NTW * 2>(vtr_, ad);
    }
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int t0i = ptile_index(2 * kc, IB);
      const bf16x4 h0 = *(const bf16x4*)(pb + t0i * 512 + l * 8);
      const bf16x4 l0 = *(const bf16x4*)(pb + Cfg::P_BYTES + t0i * 512 + l * 8);
      bf16x4 h1 = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f}, l1 = h1;
      if (2 * kc + 1 <= IB) {
        const int t1i = ptile_index(2 * kc + 1, IB);
        h1 = *(const bf16x4*)(pb + t1i * 512 + l * 8);
        l1 = *(const bf16x4*)(pb + Cfg::P_BYTES + t1i * 512 + l * 8);
      }
      const bf16x8 bh_ = join(h0, h1), bl_ = join(l0, l1);
#pragma unroll
      for (int n = 0; n < Cfg::NTW; ++n) {
        const bf16x8 vt = join(vtr_[(kc * Cfg::NTW + n) * 2], vtr_[(kc * Cfg::NTW + n) * 2 + 1]);
        acc[n] = mfma16(vt, bh_, acc[n]);
        acc[n] = mfma16(vt, bl_, acc[n]);
      }
    }
    {
      const long long rem = (long long)T - (long long)c * C;
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(P.Oh + (size_t)c * C * DV, rem * DV * 2);
#pragma unroll
      for (int n = 0; n < Cfg::NTW; ++n) {
        const bf16x4 o = to_bf16x4(acc[n][0], acc[n][1], acc[n][2], acc[n][3]);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(uint2v, o), ro, ooff + n * 32, 0, 0);
      }
    }
    // ---- phase 2b: S += K^T (diag(eta) V)_hi + K^T (diag(eta) V)_lo on this wave's slab ----
    // operands of both 32-token halves: per half, diag(eta)V hi/lo (2 reads
    // each per column tile) then K^T (2 reads per m-tile)
    constexpr int NE = 4 * Cfg::NTW, NKR = 2 * Cfg::MTW, NH = NE + NKR;
    bf16x4 opb[2 * NH];
    {
      unsigned ad[2 * NH];
      const unsigned eb0 = lds_addr(evb) + vtr, kb0 = lds_addr(kst);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
        for (int n = 0; n < Cfg::NTW; ++n) {
          const unsigned o0 = eb0 + 32 * kc * TV * 2 + 32 * (NT0 + n), o1 = o0 + 16 * TV * 2;
          ad[kc * NH + 4 * n + 0] = o0;
          ad[kc * NH + 4 * n + 1] = o1;
          ad[kc * NH + 4 * n + 2] = o0 + Cfg::V_BYTES;
          ad[kc * NH + 4 * n + 3] = o1 + Cfg::V_BYTES;
        }
#pragma unroll
        for (int j = 0; j < Cfg::MTW; ++j) {
          const unsigned o0 = kb0 + ktr[j] + 32 * kc * ROWB;
          ad[kc * NH + NE + 2 * j] = o0;
          ad[kc * NH + NE + 2 * j + 1] = o0 + 16 * ROWB;
        }
      }
      lds_tr16_batch<2 * NH>(opb, ad);
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
      for (int j = 0; j < Cfg::MTW; ++j) {
        const bf16x8 a = join(opb[kc * NH + NE + 2 * j], opb[kc * NH + NE + 2 * j + 1]);
#pragma unroll
        for (int n = 0; n < Cfg::NTW; ++n) {
          const bf16x8 evh = join(opb[kc * NH + 4 * n], opb[kc * NH + 4 * n + 1]);
          const bf16x8 evl = join(opb[kc * NH + 4 * n + 2], opb[kc * NH + 4 * n + 3]);
          S[j][n] = mfma16(a, evh, S[j][n]);
          S[j][n] = mfma16(a, evl, S[j][n]);
        }
      }
    }
    write_s_lds();
    qslot = qslot == 2 ? 0 : qslot + 1;
    vslot = vslot1;
  }

  wait_vm_barrier<0>();
#pragma unroll
  for (int j = 0; j < Cfg::MTW; ++j)
#pragma unroll
    for (int n = 0; n < Cfg::NTW; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        P.Wh[(size_t)(SLAB + 16 * j + 4 * g + r) * DV + tv0 + 16 * (NT0 + n) + li] = S[j][n][r];
}

template <int DK, int TV, int NW>
__global__ __launch_bounds__(NW * 64, 1) void per_token_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const float* __restrict__ eta, const float* __restrict__ W0, bf16* __restrict__ O,
    float* __restrict__ Wout, int T, int DV) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int NV = DV / TV;
  const int nblocks = gridDim.x;
  const int logical = (nblocks % 8 == 0) ? xcd_logical_block(blockIdx.x, nblocks) : blockIdx.x;
  const int bh = logical / NV;
  PerTokenPtrs P;
  P.Qh = Q + (size_t)bh * T * DK;
  P.Kh = K + (size_t)bh * T * DK;
  P.Vh = V + (size_t)bh * T * DV;
  P.Eh = eta + (size_t)bh * T;
  P.Oh = O + (size_t)bh * T * DV;
  P.W0h = W0 + (size_t)bh * DK * DV;
  P.Wh = Wout + (size_t)bh * DK * DV;
  P.T = T;
  P.DV = DV;
  P.tv0 = (logical % NV) * TV;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if constexpr (NW == 4) {
    switch (w) {
      case 0: per_token_wave<DK, TV, NW, 0>(P, smem, l); break;
      case 1: per_token_wave<DK, TV, NW, 1>(P, smem, l); break;
      case 2: per_token_wave<DK, TV, NW, 2>(P, smem, l); break;
      default: per_token_wave<DK, TV, NW, 3>(P, smem, l); break;
    }
  } else {
    switch (w) {
      case 0: per_token_wave<DK, TV, NW, 0>(P, smem, l); break;
      case 1: per_token_wave<DK, TV, NW, 1>(P, smem, l); break;
      case 2: per_token_wave<DK, TV, NW, 2>(P, smem, l); break;
      case 3: per_token_wave<DK, TV, NW, 3>(P, smem, l); break;
      case 4: per_token_wave<DK, TV, NW, 4>(P, smem, l); break;
      case 5: per_token_wave<DK, TV, NW, 5>(P, smem, l); break;
      case 6: per_token_wave<DK, TV, NW, 6>(P, smem, l); break;
      default: per_token_wave<DK, TV, NW, 7>(P, smem, l); break;
    }
  }
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
template <int DK, int TV, int NW = (TV >= 32 ? 8 : 4)>
static hipError_t launch_bf16(const PerTokenArgs& a, hipStream_t stream) {
  using Cfg = PerTokenCfg<DK, TV, NW>;
  auto kern = per_token_bf16_kernel<DK, TV, NW>;
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
  if (a.DK == 128) return tv == 16 ? launch_bf16<128, 16>(a, stream) : launch_bf16<128, 32>(a, stream);
  if (tv == 16) return launch_bf16<64, 16>(a, stream);
  if (tv == 64) return launch_bf16<64, 64>(a, stream);
  return launch_bf16<64, 32>(a, stream);
}

}  // namespace ttt
