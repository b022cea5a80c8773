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
// bf16 design (gfx950): the sequence of each head is cut into P segments of
// whole 64-token tiles so that heads x segments cover the compute units.
//  1. pt_incr_kernel<D>: for every segment but the last, its state
//     increment dS_s = K_s^T diag(eta_s) V_s (fp32) into the workspace;
//     pt_seg_scan_kernel<D> turns them into start states in place;
//  2. pt_seg_kernel<D>: segment s starts from
//     S = W0 + sum_{s' < s} dS_s' and runs the chunked form over its tiles;
//     the last segment writes W_out.
// A workgroup has D/16 waves; wave w owns columns 16w..16w+15 of S and O for
// all D rows of S, which stay in MFMA accumulators for the whole segment, so
// no state is exchanged between waves.  Q, K, V and eta go HBM -> LDS with
// asynchronous direct-to-LDS loads through a 3-stage ring (explicit vmcnt
// waits).  Per 64-token tile:
//   phase 1: the 10 causal score tiles P^T(jb, ib) = K_jb Q_ib^T (jb <= ib),
//            spread over the waves, scaled by eta of the key, masked and
//            split bf16 hi + lo into LDS; the wave's V columns (transposed
//            reads) scaled by eta and split hi + lo, and the first K^T
//            operands of the state update;
//   phase 2: O_w^T = S_w^T Q^T with S_w as bf16 hi + lo built in registers
//            from the accumulators (the contraction index follows the
//            accumulator row order and Q is read in the same order), plus
//            V_w^T A^T from the score tiles; then S_w += K^T diag(eta) V_w.
// Outputs are computed transposed, so a lane holds 4 consecutive columns of
// one token; they are staged as whole rows in the tile's dead V region and
// leave with 16-byte stores after the next barrier.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace ttt {

// Q, K, V and eta are streamed with non-temporal loads in both passes.  On
// gfx950 this keeps their throughput when the caches hold many dirty lines
// (measured: about 1.2x faster for the two passes together), and costs about
// 3% when the caches are clean, where the output pass would otherwise find
// some K/V lines the increment pass left behind.
constexpr bool PT_STREAM = true;

// score tile t (0..9) <-> (jb, ib), jb <= ib; wave w owns tiles [tile_begin(w), tile_begin(w+1))
__host__ __device__ constexpr int ptile_jb(int t) { return t < 1 ? 0 : t < 3 ? t - 1 : t < 6 ? t - 3 : t - 6; }
__host__ __device__ constexpr int ptile_ib(int t) { return t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3; }
__host__ __device__ constexpr int ptile_index(int jb, int ib) { return ib * (ib + 1) / 2 + jb; }
// LDS slot of the score-tile pair (2kc, 2kc+1) of query block ib: the pairs of all query blocks in order
// (ib + 2) / 2 pairs for block ib); a pair whose second tile lies above the diagonal keeps zeros there
__host__ __device__ constexpr int ppair_slot(int ib, int kc) { return (ib / 2) * (ib / 2 + 1) + (ib & 1) * (ib / 2 + 1) + kc; }
__host__ __device__ constexpr int tile_begin4(int w) { return w == 0 ? 0 : w == 1 ? 3 : w == 2 ? 6 : w == 3 ? 8 : 10; }
__host__ __device__ constexpr int tile_begin8(int w) { return w <= 3 ? 2 * w : w <= 7 ? w + 3 : 10; }
template <int NW>
__host__ __device__ constexpr int tile_begin(int w) { return NW == 4 ? tile_begin4(w) : tile_begin8(w); }

// Tile length of the output pass.  The wave program also supports 32-token
// tiles, whose workgroups take under half a CU's LDS (two workgroups, 4 waves
// per SIMD, per CU); at d = 128 that measured slower overall on gfx950 (the
// per-token split and barrier costs double and more segments are needed).
template <int D>
__host__ __device__ constexpr int seg_tile() { return 64; }

template <int D, int CT>
struct SegCfg {
  static constexpr int C = CT;                   // tokens per tile
  static constexpr int NB = C / 16;              // 16-token blocks per tile
  static constexpr int NT = NB * (NB + 1) / 2;   // causal score tiles per tile
  static constexpr int KC = C / 32;              // 32-key halves of the state update
  static constexpr int NW = D / 16;              // waves; wave w owns columns 16w..16w+15
  static constexpr int THREADS = NW * WAVE;
  static constexpr int MT = D / 16;              // 16-row tiles of S per wave
  static constexpr int KP = D / 32;              // 32-deep contraction steps over d
  static constexpr int ROWB = D * 2;             // bytes per token row of Q, K, V, O
  static constexpr int MAT = C * ROWB;           // one matrix of a tile
  // ring slot: Q, K, V (reused for the tile's outputs), eta
  static constexpr int STAGES = 3;
  static constexpr int OFF_K = MAT;
  static constexpr int OFF_V = OFF_K + MAT;
  static constexpr int OFF_E = OFF_V + MAT;
  static constexpr int STAGE = 3 * MAT + C * 4;
  // The score tiles come first, so that their addresses (lane offset plus constants below 64 KB) take
  // the LDS instructions' immediate offsets instead of one address add per read.  They are stored as
  // pairs (2kc, 2kc+1) of one query block, 16 bytes per lane, so that each operand of the intra-tile
  // product is one 16-byte read.
  static constexpr int NPAIR = ppair_slot(NB, 0);  // pair slots (6 for 64-token tiles)
  static constexpr int OFF_P = 0;                 // score pairs [hi, lo][NPAIR][64 lanes x 16 bytes]
  static constexpr int P_PLANE = NPAIR * 1024;
  static constexpr int OFF_RING = 2 * P_PLANE;
  static constexpr int LDS_BYTES = OFF_RING + STAGES * STAGE;
  static constexpr int WG_PER_CU = (160 * 1024) / LDS_BYTES >= 2 ? 2 : 1;
  static constexpr int WAVES_PER_SIMD = NW * WG_PER_CU / 4;
  static constexpr int EPW = C / NW;             // eta values loaded by each wave
  static constexpr int MAT_LOADS = MAT / 1024 / NW;  // 16-byte direct-to-LDS loads per wave per matrix
  static constexpr int LOADS = 3 * MAT_LOADS + 1;
  static constexpr int OUT_STORES = MAT_LOADS;   // 16-byte output stores per wave per tile
  static_assert(C == 32 || C == 64, "tile length");
  static_assert(MAT % (1024 * NW) == 0, "tile matrix must split into whole wave loads");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(LDS_BYTES >= D * D * 4, "W0 is staged through the ring");
};
// wave w computes score tiles [seg_tile_begin(w), seg_tile_begin(w+1))
template <class Cfg>
__device__ __forceinline__ int seg_tile_begin(int w) {
  if constexpr (Cfg::C == 64) return tile_begin<Cfg::NW>(w);
  else return min(w, Cfg::NT);
}

// Row order of the state held in MFMA accumulators: accumulator row 4g + r
// of row tile m = 2p + h holds row d = 32p + 8g + 4h + r of S.  Then tiles
// 2p and 2p + 1 of a lane together hold 8 consecutive rows 32p + 8g .. + 7,
// so the products that contract over d (scores, Q S) read their Q and K
// operands as one 16-byte piece per lane in natural order.
__host__ __device__ constexpr int seg_srow(int m, int g, int r) { return 32 * (m >> 1) + 8 * g + 4 * (m & 1) + r; }

// LDS layout of the tiles: row-major, with 16-byte piece c of row r stored
// at piece c ^ seg_swz(r).  For d = 128 the map (a linear map of the row's
// low 4 bits, as a table) was chosen by measuring LDS throughput on gfx950
// so that the 16-byte operand reads (16 rows, one piece), the transposed
// reads of K for the state update (4 rows x 4 pieces 16 bytes apart, one
// half) and of V (4 rows x 32 bytes) all run without bank conflicts; simple
// XOR maps of the row leave one or the other 2-way conflicted.
template <int D>
__host__ __device__ constexpr int seg_swz(int r) {
  return D == 128 ? (int)((0x159DAE2673FBC840ull >> (4 * (r & 15))) & 15) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}
// LDS byte offset, within a tile matrix, of the transposed read that gives
// lane (g, li) its A operand of the state update for row tile m: key row
// 4g + li/4, the 4 columns 32p + 8(li%4) + 4h .. + 3 (m = 2p + h)
template <int D>
__host__ __device__ constexpr unsigned seg_ktr(int m, int g, int li) {
  return (unsigned)((4 * g + (li >> 2)) * 2 * D + (((4 * (m >> 1) + (li & 3)) ^ seg_swz<D>(4 * g + (li >> 2))) << 4) +
                    8 * (m & 1));
}

// S_w += K^T diag(eta) V_w over the tile's keys, in pieces that can be
// placed on either side of a barrier: A operand rows seg_srow(m, li/4, li%4) of K^T with keys
// 16kb + 4g + j (transposed reads, one key half at a time); B operand
// diag(eta) V_w built from the V_w fragments vt (same key order), split bf16
// hi + lo.
template <class Cfg>
struct SegUpdate {
  bf16x8 evh[Cfg::KC], evl[Cfg::KC];  // diag(eta) V_w, keys of half kc, bf16 hi + lo
};
template <class Cfg>
__device__ __forceinline__ void seg_update_eta(SegUpdate<Cfg>& U, const float* es, const bf16x4 (&vt)[Cfg::NB], int g) {
#pragma unroll
  for (int kc = 0; kc < Cfg::KC; ++kc) {
    const floatx4 e0 = *(const floatx4*)(es + 32 * kc + 4 * g);
    const floatx4 e1 = *(const floatx4*)(es + 32 * kc + 16 + 4 * g);
    const uint2 v0 = __builtin_bit_cast(uint2, vt[2 * kc]), v1 = __builtin_bit_cast(uint2, vt[2 * kc + 1]);
    split8(floatx4{e0[0] * bf16lo_f(v0.x), e0[1] * bf16hi_f(v0.x), e0[2] * bf16lo_f(v0.y), e0[3] * bf16hi_f(v0.y)},
           floatx4{e1[0] * bf16lo_f(v1.x), e1[1] * bf16hi_f(v1.x), e1[2] * bf16lo_f(v1.y), e1[3] * bf16hi_f(v1.y)},
           U.evh[kc], U.evl[kc]);
  }
}
// the same without rates: V_w itself (bf16, so no lo part)
template <class Cfg>
__device__ __forceinline__ void seg_update_unit(SegUpdate<Cfg>& U, const bf16x4 (&vt)[Cfg::NB]) {
#pragma unroll
  for (int kc = 0; kc < Cfg::KC; ++kc) U.evh[kc] = join(vt[2 * kc], vt[2 * kc + 1]);
}
// transposed K operands of key half kc: rows seg_srow(m, li/4, li%4) of K^T, keys 32kc + 16h + 4g + j
template <class Cfg>
__device__ __forceinline__ void seg_update_k(bf16x8 (&a)[Cfg::MT], const unsigned char* ks,
                                             const unsigned (&ktr)[Cfg::MT], int kc) {
#pragma unroll
  for (int m = 0; m < Cfg::MT; ++m)
    a[m] = join(lds_read_tr16(ks + (2 * kc) * 16 * Cfg::ROWB + ktr[m]),
                lds_read_tr16(ks + (2 * kc + 1) * 16 * Cfg::ROWB + ktr[m]));
}
// hi products of every m-tile before the lo products: consecutive MFMAs never depend on each other
template <class Cfg, bool LO = true>
__device__ __forceinline__ void seg_update_mfma(floatx4 (&S)[Cfg::MT], const bf16x8 (&a)[Cfg::MT],
                                                const SegUpdate<Cfg>& U, int kc) {
#pragma unroll
  for (int m = 0; m < Cfg::MT; ++m) S[m] = mfma16(a[m], U.evh[kc], S[m]);
  if constexpr (LO) {
#pragma unroll
    for (int m = 0; m < Cfg::MT; ++m) S[m] = mfma16(a[m], U.evl[kc], S[m]);
  }
}

struct SegArgs {
  const bf16* Q;
  const bf16* K;
  const bf16* V;
  const float* eta;
  const float* W0;
  floatx4* part;
  bf16* O;
  float* Wout;
  int T, nseg, seg_len;             // segment s covers tokens [s*seg_len, (s+1)*seg_len), whole tiles of both passes
  int start_transposed = 0;         // 1: segment s > 0 starts from the transpose of the state in slot s
  const bf16* aux = nullptr;        // DOT: the rows each output row is dotted with ([B,H,T,D], original order)
  float* dpart = nullptr;           // DOT: per-wave partial dots, [B,H,T][D / 16] (original order)
};

// The program of wave W (wave-uniform).  One program for all waves keeps the
// code within the instruction cache.
// REV runs the same recurrence over the head's sequence in reverse token
// order (the backward pass's suffix sums): the segment of reversed tokens
// [tok0, seg_end) is the original range [T - seg_end, T - tok0), and row r
// of tile i is original segment row seg_toks - 1 - (C i + r).  A row before
// the segment's start gets the offset 2^31, past any view's size, so it
// reads 0 and its store is dropped, as a row past the end does in forward
// order.
// EM places the rates: 0 on the keys (the method's recurrence); 1 on the
// queries (keys unit-rate, each output row scaled by its own token's rate);
// 2 nowhere (unit rates; eta is still streamed but unused).
// OF32: the outputs are float32 (A.O points to floats) and leave straight
// from the accumulators, 16 bytes per lane (4 columns of one token), instead
// of as bf16 rows staged in LDS.
// DOT (with OF32): each output row o_t (before the rate of EM 1 scales it)
// is also dotted with row t of A.aux over the wave's 16 columns, and the
// partial goes to A.dpart[t][W] (the backward's rate gradient <u_t, v_t>
// without a pass of its own over u).
template <int D, int CT, bool EXCL, bool REV, int EM, bool OF32, bool DOT = false>
__device__ __forceinline__ void seg_wave(const SegArgs& A, unsigned char* smem, int bh, int s, int W, int l) {
  static_assert(!DOT || OF32, "the partial dots are taken from the float32 output path");
  using Cfg = SegCfg<D, CT>;
  constexpr int NB = Cfg::NB;
  constexpr int C = Cfg::C, ROWB = Cfg::ROWB, MT = Cfg::MT, KP = Cfg::KP, NW = Cfg::NW;
  constexpr int LOADS = Cfg::LOADS;
  const int g = l >> 4, li = l & 15;
  const int T = A.T, nseg = A.nseg;
  const int nchunks = (int)(((long long)T + C - 1) / C);
  const int seg_tiles = A.seg_len / C;
  const int c0 = s * seg_tiles, c1 = min(c0 + seg_tiles, nchunks);
  const int nt = c1 > c0 ? c1 - c0 : 0;
  const long long seg_end = min((long long)c1 * C, (long long)T);
  const bf16* Qh = A.Q + (size_t)bh * T * D;
  const bf16* Kh = A.K + (size_t)bh * T * D;
  const bf16* Vh = A.V + (size_t)bh * T * D;
  const float* Eh = A.eta + (size_t)bh * T;
  bf16* Oh = A.O + (size_t)bh * T * D;

  // ---- per-lane byte offsets, fixed for the whole segment ----
  // this wave's share of a tile matrix: LDS bytes [W*MAT_LOADS*1024, +MAT_LOADS*1024), i.e. whole rows
  unsigned gofs[Cfg::MAT_LOADS];    // global offset of the 16 bytes lane l moves per load (forward order)
  int grow[Cfg::MAT_LOADS];         // REV: their tile row and byte offset within the row
  unsigned gpc[Cfg::MAT_LOADS];
  unsigned lofs[Cfg::MAT_LOADS];    // their (swizzled) LDS offset
#pragma unroll
  for (int k = 0; k < Cfg::MAT_LOADS; ++k) {
    const int b = (W * Cfg::MAT_LOADS + k) * 1024 + 16 * l;
    const int row = b / ROWB, ph = (b % ROWB) >> 4;
    gofs[k] = (unsigned)(row * ROWB + ((ph ^ seg_swz<D>(row)) << 4));
    grow[k] = row;
    gpc[k] = (unsigned)((ph ^ seg_swz<D>(row)) << 4);
    lofs[k] = (unsigned)b;
  }
  unsigned ksb[KP];                 // operand reads: row li, d = 32p + 8g .. + 7
#pragma unroll
  for (int p = 0; p < KP; ++p) ksb[p] = (unsigned)(li * ROWB + (((4 * p + g) ^ seg_swz<D>(li)) << 4));
  const int trow = 4 * g + (li >> 2);   // transposed reads: rows 4g..4g+3, column 16m + li
  unsigned ktr[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) ktr[m] = seg_ktr<D>(m, g, li);
  const unsigned vtr = (unsigned)(trow * ROWB + (((2 * W + ((li >> 1) & 1)) ^ seg_swz<D>(trow)) << 4) + (li & 1) * 8);
  // output fragment (row 16ib + li, columns 16W + 4g..+3) in the swizzled staging rows
  const unsigned ofr = (unsigned)(li * ROWB + (((2 * W + (g >> 1)) ^ seg_swz<D>(li)) << 4) + (g & 1) * 8);

  // One buffer view per matrix for the whole segment (rows past its end read 0, stores there are
  // dropped); a tile is addressed by its 32-bit offset.
  const long long tok0 = (long long)c0 * C;
  const long long seg_toks = seg_end > tok0 ? seg_end - tok0 : 0;
  const long long first = nt > 0 ? (REV ? (long long)T - seg_end : tok0) : 0;   // first original token
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qh + first * D, seg_toks * ROWB);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + first * D, seg_toks * ROWB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh + first * D, seg_toks * ROWB);
  const __amdgpu_buffer_rsrc_t re = make_rsrc(Eh + first, seg_toks * 4);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(Oh + first * D, seg_toks * ROWB);
  const __amdgpu_buffer_rsrc_t ro32 =
      make_rsrc((float*)(void*)A.O + ((size_t)bh * T + first) * D, OF32 ? seg_toks * D * 4 : 0);
  // DOT: the aux rows (bf16) and the partial dots of the segment, addressed like the outputs
  const __amdgpu_buffer_rsrc_t raux =
      make_rsrc(DOT ? (const void*)(A.aux + ((size_t)bh * T + first) * D) : nullptr, DOT ? seg_toks * ROWB : 0);
  const __amdgpu_buffer_rsrc_t rdp =
      make_rsrc(DOT ? (const void*)(A.dpart + ((size_t)bh * T + first) * NW) : nullptr, DOT ? seg_toks * NW * 4 : 0);
  const int erow = W * Cfg::EPW + l;   // the tile row whose eta lane l moves
  constexpr unsigned OOB = 0x80000000u;
  // byte offset in the segment's views of load k of tile i (of its eta value)
  auto mat_ofs = [&](int i, int k) -> unsigned {
    if constexpr (REV) {
      const long long r = seg_toks - 1 - (long long)i * C - grow[k];
      return r >= 0 ? (unsigned)(r * ROWB) + gpc[k] : OOB;
    } else {
      return (unsigned)i * Cfg::MAT + gofs[k];
    }
  };
  // OF32: byte offset of lane (g, li)'s 16 output bytes of token 16ib + li of tile i
  auto out32_ofs = [&](int i, int ib) -> unsigned {
    const int row = 16 * ib + li;
    const unsigned col = (unsigned)(16 * W + 4 * g) * 4;
    if constexpr (REV) {
      const long long r = seg_toks - 1 - (long long)i * C - row;
      return r >= 0 ? (unsigned)(r * D * 4) + col : OOB;
    } else {
      return (unsigned)(((long long)i * C + row) * D * 4) + col;
    }
  };
  // DOT: segment row of output row 16ib + li of tile i (OOB before the segment in reverse order)
  auto seg_row = [&](int i, int ib) -> long long {
    const int row = 16 * ib + li;
    if constexpr (REV)
      return seg_toks - 1 - (long long)i * C - row;
    else
      return (long long)i * C + row;
  };
  auto aux_ofs = [&](int i, int ib) -> unsigned {
    const long long r = seg_row(i, ib);
    return r >= 0 ? (unsigned)(r * ROWB) + (unsigned)((16 * W + 4 * g) * 2) : OOB;
  };
  auto dpart_ofs = [&](int i, int ib) -> unsigned {
    const long long r = seg_row(i, ib);
    return r >= 0 ? (unsigned)(r * NW + W) * 4u : OOB;
  };
  auto eta_ofs = [&](int i) -> unsigned {
    if constexpr (REV) {
      const long long r = seg_toks - 1 - (long long)i * C - erow;
      return r >= 0 ? (unsigned)(r * 4) : OOB;
    } else {
      return (unsigned)i * (C * 4) + (unsigned)(erow * 4);
    }
  };
  // Tile i of the segment into ring slot i % STAGES (empty past the segment), in two parts: Q, and
  // K, V, eta.  The parts are issued at different points of a tile so that the workgroup's vector
  // memory instructions do not all queue at the tile boundary.
  auto issue_q = [&](int i) {
    unsigned char* st = smem + Cfg::OFF_RING + (i % Cfg::STAGES) * Cfg::STAGE + W * Cfg::MAT_LOADS * 1024;
#pragma unroll
    for (int k = 0; k < Cfg::MAT_LOADS; ++k) dma16<PT_STREAM>(rq, mat_ofs(i, k), st + k * 1024);
  };
  auto issue_kve = [&](int i) {
    unsigned char* st = smem + Cfg::OFF_RING + (i % Cfg::STAGES) * Cfg::STAGE + W * Cfg::MAT_LOADS * 1024;
#pragma unroll
    for (int k = 0; k < Cfg::MAT_LOADS; ++k) dma16<PT_STREAM>(rk, mat_ofs(i, k), st + Cfg::OFF_K + k * 1024);
#pragma unroll
    for (int k = 0; k < Cfg::MAT_LOADS; ++k) dma16<PT_STREAM>(rv, mat_ofs(i, k), st + Cfg::OFF_V + k * 1024);
    unsigned char* ed = smem + Cfg::OFF_RING + (i % Cfg::STAGES) * Cfg::STAGE + Cfg::OFF_E + W * Cfg::EPW * 4;
    if (l < Cfg::EPW) dma4<PT_STREAM>(re, eta_ofs(i), ed);
  };
  // rows of tile i's outputs staged in its (dead) V region -> HBM, 16 bytes per lane, whole rows
  auto write_out = [&](int i) {
    const unsigned char* st = smem + Cfg::OFF_RING + (i % Cfg::STAGES) * Cfg::STAGE + Cfg::OFF_V;
    u32x4 v[Cfg::MAT_LOADS];
#pragma unroll
    for (int k = 0; k < Cfg::MAT_LOADS; ++k) v[k] = *(const u32x4*)(st + lofs[k]);
#pragma unroll
    for (int k = 0; k < Cfg::MAT_LOADS; ++k) buf_store16(ro, mat_ofs(i, k), v[k]);
  };

  // The first two tiles go out to LDS first; the loads of the start state
  // (one workspace slot, registers only) follow, so both are in flight together.  (Compiler-issued
  // loads after the asynchronous copies only make its own waits conservative.)
#pragma unroll
  for (int k = 0; k < Cfg::STAGES - 1; ++k)
    if (nt > 0) {
      issue_q(k);
      issue_kve(k);
    }

  // ---- state: S[m][r] = S[seg_srow(m, g, r)][16W + li] ----
  floatx4 S[MT];
  const floatx4* pp = A.part + ((size_t)bh * nseg * NW + W) * MT * 64 + l;   // slot 0 of this head
  constexpr int SLOT = NW * MT * 64;                                         // floatx4 per slot
  if (s > 0 && A.start_transposed) {
    // the transpose of the slot's state: element (row x, column y) of the slot sits in wave y/16,
    // lane 16g + y%16 and row tile m, register r of seg_srow(m, g, r) = x
    const float* ps = (const float*)(A.part + ((size_t)bh * nseg + s) * SLOT);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int y = seg_srow(m, g, r), x = 16 * W + li;
        const int mx = 2 * (x >> 5) + ((x >> 2) & 1), gx = (x >> 3) & 3, rx = x & 3;
        S[m][r] = ps[((size_t)((y >> 4) * MT + mx) * 64 + 16 * gx + (y & 15)) * 4 + rx];
      }
  } else if (s > 0) {
    // start state of this segment, prepared by pt_seg_scan_kernel in the same fragment layout
#pragma unroll
    for (int m = 0; m < MT; ++m) S[m] = pp[(size_t)s * SLOT + m * 64];
  } else {                        // the first segment starts from W0
    const float* W0h = A.W0 + (size_t)bh * D * D;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[m][r] = W0h[seg_srow(m, g, r) * D + 16 * W + li];
  }

  // second halves of the pair slots that hold a single tile (an even query block's diagonal tile):
  // zero once, never written again (visible to every wave after the first barrier of the loop)
  if (W == 0) {
#pragma unroll
    for (int ib = 0; ib < NB; ib += 2) {
      const int po = ppair_slot(ib, ib / 2) * 1024 + 8 + l * 16;
      *(uint2*)(smem + Cfg::OFF_P + po) = uint2{0u, 0u};
      *(uint2*)(smem + Cfg::OFF_P + Cfg::P_PLANE + po) = uint2{0u, 0u};
    }
  }

  static_assert(Cfg::STAGES == 3, "the vmcnt waits below count the loads of two tiles in flight");
  for (int i = 0; i < nt; ++i) {
    // Tile i has landed once only later-issued loads (and output stores) may be outstanding: per
    // wave the order is stores(i-2), Q(i+1) [tile i-1 start], K/V/eta(i+1) [tile i-1 middle].
    // With OF32 a tile's NB stores follow its K/V/eta issue: after tile i's loads come
    // stores(i-2), Q(i+1), K/V/eta(i+1), stores(i-1).
    // DOT: its NB aux loads come right after Q(i+2) and are complete before the tile's stores (the wait
    // before them), and each tile stores NB partial dots after its outputs.
    constexpr int NBS = DOT ? 2 * NB : NB;   // stores per tile
    if constexpr (OF32) {
      if (i == 0)
        wait_vm_barrier<LOADS>();
      else if (i == 1)
        wait_vm_barrier<LOADS + NBS>();
      else
        wait_vm_barrier<LOADS + 2 * NBS>();
    } else if (i < 2) {
      wait_vm_barrier<LOADS>();
    } else {
      wait_vm_barrier<LOADS + Cfg::OUT_STORES>();
    }
    if (!OF32 && i >= 1) {
      write_out(i - 1);           // from the slot the next load overwrites: read it first
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    issue_q(i + Cfg::STAGES - 1);   // into the slot read during tile i-1
    u32x2 vd[NB];                   // DOT: aux row 16ib + li, columns 16W + 4g .. + 3 (bf16)
    if constexpr (DOT) {
#pragma unroll
      for (int ib = 0; ib < NB; ++ib)
        vd[ib] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(raux, aux_ofs(i, ib), 0, 0));
    }
    const unsigned char* st = smem + Cfg::OFF_RING + (i % Cfg::STAGES) * Cfg::STAGE;
    const unsigned char* ks = st + Cfg::OFF_K;
    const unsigned char* vs = st + Cfg::OFF_V;
    const float* es = (const float*)(st + Cfg::OFF_E);

    const unsigned char* qs = st;
    unsigned char* pb = smem + Cfg::OFF_P;
    floatx4 acc[NB];
    bf16x4 vt[NB];                 // vt[kb][j] = V[16kb + 4g + j][16W + li]
    SegUpdate<Cfg> U;
    // Q operand of block ib, step p (k order of the S accumulators)
    auto qop = [&](int p, int ib) {
      const unsigned char* qrow = qs + ib * 16 * ROWB;
      return *(const bf16x8*)(qrow + ksb[p]);
    };
    // this wave's score tiles P^T(jb, ib) = K_jb Q_ib^T, scaled by eta of the key, masked, bf16 hi + lo
    auto scores = [&]() {
      const int tb = seg_tile_begin<Cfg>(W), te = seg_tile_begin<Cfg>(W + 1);
#pragma unroll
      for (int t = 0; t < Cfg::NT; ++t) {
        if (t < tb || t >= te) continue;    // wave-uniform
        const int jb = ptile_jb(t), ib = ptile_ib(t);
        floatx4 p = {0.f, 0.f, 0.f, 0.f};
        const unsigned char* krow = ks + jb * 16 * ROWB;
#pragma unroll
        for (int kk = 0; kk < KP; ++kk) {
          const bf16x8 ka = *(const bf16x8*)(krow + ksb[kk]);
          p = mfma16(ka, qop(kk, ib), p);
        }
        const floatx4 e4 = EM == 0 ? *(const floatx4*)(es + 16 * jb + 4 * g) : floatx4{1.f, 1.f, 1.f, 1.f};
        floatx4 f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // key 16jb + 4g + r against query 16ib + li: a key after the query (or the query's own key,
          // for the read before the token's step) is masked
          const bool masked = jb == ib && (EXCL ? 4 * g + r >= li : 4 * g + r > li);
          f[r] = masked ? 0.f : p[r] * e4[r];
        }
        const uint2 s01 = split2(f[0], f[1]), s23 = split2(f[2], f[3]);
        const int po = ppair_slot(ib, jb >> 1) * 1024 + (jb & 1) * 8 + l * 16;
        *(uint2*)(pb + po) = uint2{s01.x, s23.x};
        *(uint2*)(pb + Cfg::P_PLANE + po) = uint2{s01.y, s23.y};
      }
    };
    // O_W^T = S_W^T Q^T with S_W as bf16 hi + lo
    auto qs_mfma = [&]() {
      // the split of step p + 1 is interleaved with the MFMAs of step p
      bf16x8 ah[2], al[2], qv[2][NB];
      split8(S[0], S[1], ah[0], al[0]);
#pragma unroll
      for (int ib = 0; ib < NB; ++ib) qv[0][ib] = qop(0, ib);
#pragma unroll
      for (int p = 0; p < KP; ++p) {
        const int c = p & 1, n = c ^ 1;
        if (p + 1 < KP) {
#pragma unroll
          for (int ib = 0; ib < NB; ++ib) qv[n][ib] = qop(p + 1, ib);
          split8(S[2 * p + 2], S[2 * p + 3], ah[n], al[n]);
        }
#pragma unroll
        for (int ib = 0; ib < NB; ++ib) acc[ib] = mfma16(ah[c], qv[c][ib], acc[ib]);
#pragma unroll
        for (int ib = 0; ib < NB; ++ib) acc[ib] = mfma16(al[c], qv[c][ib], acc[ib]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // operands of phase 2 that do not depend on the score tiles
    bf16x8 ka0[MT];               // transposed K operands of the first key half
    auto load_update = [&]() {
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) vt[kb] = lds_read_tr16(vs + kb * 16 * ROWB + vtr);
      if constexpr (EM == 0)
        seg_update_eta<Cfg>(U, es, vt, g);
      else
        seg_update_unit<Cfg>(U, vt);
      if constexpr (Cfg::KC == 2) seg_update_k<Cfg>(ka0, ks, ktr, 0);
    };
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) acc[ib] = floatx4{0.f, 0.f, 0.f, 0.f};
    auto av_mfma = [&]() {        // O_W^T += V_W^T A^T over key blocks 0..ib
#pragma unroll
    for (int ib = 0; ib < NB; ++ib)
#pragma unroll
      for (int kc = 0; 2 * kc <= ib; ++kc) {
        const int po = ppair_slot(ib, kc) * 1024 + l * 16;
        const bf16x8 bh_ = *(const bf16x8*)(pb + po);
        const bf16x8 bl_ = *(const bf16x8*)(pb + Cfg::P_PLANE + po);
        const bf16x8 av = join(vt[2 * kc], vt[2 * kc + 1]);
        acc[ib] = mfma16(av, bh_, acc[ib]);
        acc[ib] = mfma16(av, bl_, acc[ib]);
      }
    };
    // phase 1: score tiles and the operands of the state update; phase 2: the
    // two waves of a SIMD take Q S and the intra-tile product in opposite
    // orders so that one issues MFMAs while the other waits on LDS
    scores();
    load_update();
    barrier();                    // score tiles visible; V of this tile read by everyone
    // The two waves of a SIMD take Q S and the intra-tile product in opposite orders, and issue the
    // next K/V/eta copies at different points (measured on gfx950: with all eight waves issuing them
    // right after the barrier, the second wave of each SIMD stalled ~1000 cycles on the issue)
    if (W < NW / 2) {
      issue_kve(i + Cfg::STAGES - 1);
      qs_mfma();
      av_mfma();
    } else {
      av_mfma();
      qs_mfma();
      issue_kve(i + Cfg::STAGES - 1);
    }
    // outputs into the V region of this slot (written out after the next barrier), or straight out
    unsigned char* ob = smem + Cfg::OFF_RING + (i % Cfg::STAGES) * Cfg::STAGE + Cfg::OFF_V;
    // DOT: the aux loads have landed once only K/V/eta(i+2) may be outstanding (in both issue orders
    // that copy comes after them)
    if constexpr (DOT) wait_vm<2 * Cfg::MAT_LOADS + 1>();
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) {
      const float eq = EM == 1 ? es[16 * ib + li] : 1.f;   // rate of the output row's own token
      if constexpr (OF32)
        buf_store16(ro32, out32_ofs(i, ib), __builtin_bit_cast(u32x4, eq * acc[ib]));
      else
        *(bf16x4*)(ob + ib * 16 * ROWB + ofr) = to_bf16x4(eq * acc[ib][0], eq * acc[ib][1], eq * acc[ib][2],
                                                          eq * acc[ib][3]);
    }
    if constexpr (DOT) {
#pragma unroll
      for (int ib = 0; ib < NB; ++ib) {
        float dot = acc[ib][0] * bf16lo_f(vd[ib].x) + acc[ib][1] * bf16hi_f(vd[ib].x) +
                    acc[ib][2] * bf16lo_f(vd[ib].y) + acc[ib][3] * bf16hi_f(vd[ib].y);
        dot += __shfl_xor(dot, 16);     // the four column groups of the row: lanes li + 16 g
        dot += __shfl_xor(dot, 32);
        // one store per block (lanes g = 0 carry it), so every wave issues the same count
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, dot), rdp,
                                              g == 0 ? dpart_ofs(i, ib) : OOB, 0, 0);
      }
    }
    if constexpr (Cfg::KC == 2) {
      bf16x8 ka1[MT];
      seg_update_k<Cfg>(ka1, ks, ktr, 1);
      seg_update_mfma<Cfg, EM == 0>(S, ka0, U, 0);
      seg_update_mfma<Cfg, EM == 0>(S, ka1, U, 1);
    } else {                      // one key half: its K operands are read here, within the register budget
      seg_update_k<Cfg>(ka0, ks, ktr, 0);
      seg_update_mfma<Cfg, EM == 0>(S, ka0, U, 0);
    }

  }
  if (!OF32 && nt > 0) {
    wait_vm_barrier<0>();
    write_out(nt - 1);
  }

  wait_vm<0>();

  if (s == nseg - 1) {
    float* Wh = A.Wout + (size_t)bh * D * D;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) Wh[(size_t)seg_srow(m, g, r) * D + 16 * W + li] = S[m][r];
  }

}

// Outputs of segment s of head bh (grid BH x nseg), starting from W0 plus
// the increments of the earlier segments of the head.
template <int D, int CT, bool EXCL, bool REV, int EM, bool OF32, bool DOT = false>
__global__ __attribute__((amdgpu_flat_work_group_size(1, D / 16 * WAVE),
                          amdgpu_waves_per_eu(SegCfg<D, CT>::WAVES_PER_SIMD))) void pt_seg_kernel(SegArgs A) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int bh = blockIdx.x / A.nseg, s = blockIdx.x % A.nseg;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  seg_wave<D, CT, EXCL, REV, EM, OF32, DOT>(A, smem, bh, s, w, threadIdx.x & 63);
}

// Segment increments dS_s = K_s^T diag(eta_s) V_s for every segment but the
// last of each head (grid BH x (nseg - 1)), in the fragment layout the
// output pass reads.  2*D/16 waves, 4 per SIMD: wave w takes column tile
// c = w / 2 of the increment over key half kc = w % 2 of every tile, for all
// D rows, so each wave scales and splits only its own 32 keys of diag(eta) V;
// the two key halves of a column tile are added once, at the end.  K, V and
// eta stream through a 4-stage direct-to-LDS ring.
template <int D>
struct IncrCfg {
  static constexpr int C = 64;
  static constexpr int NC = D / 16;              // column tiles
  static constexpr int NW = 2 * NC;              // waves
  static constexpr int THREADS = NW * WAVE;
  static constexpr int MT = D / 16;              // row tiles
  static constexpr int ROWB = D * 2;
  static constexpr int MAT = C * ROWB;
  static constexpr int STAGES = 4;
  static constexpr int STAGE = 2 * MAT + C * 4;  // K, V, eta
  static constexpr int LDS_BYTES = STAGES * STAGE;
  static constexpr int MAT_LOADS = MAT / 1024 / NW;
  static constexpr int EPW = C / NW;
  static constexpr int LOADS = 2 * MAT_LOADS + 1;
  static_assert(MAT % (1024 * NW) == 0, "tile matrix must split into whole wave loads");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(LDS_BYTES >= NC * MT * WAVE * 16, "the key-half reduction is staged through the ring");
};

// REV: segment s holds the reversed tokens [s*seg_len, ...), i.e. the original range
// [T - seg_end, T - seg_begin); the sum over its tokens does not depend on their order.
// UNIT: unit rates, K_s^T V_s.
template <int D, bool REV, bool UNIT>
__global__ __launch_bounds__(2 * D / 16 * WAVE, 1) void pt_incr_kernel(SegArgs A) {
  using Cfg = IncrCfg<D>;
  constexpr int C = Cfg::C, ROWB = Cfg::ROWB, MT = Cfg::MT, NC = Cfg::NC, MAT = Cfg::MAT;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int nseg = A.nseg, T = A.T;
  const int bh = blockIdx.x / (nseg - 1), s = blockIdx.x % (nseg - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63, g = l >> 4, li = l & 15;
  const int c = w >> 1, kc = w & 1;
  const long long seg_begin = (long long)s * A.seg_len;
  const long long seg_end = min(seg_begin + A.seg_len, (long long)T);
  const long long seg_toks = seg_end > seg_begin ? seg_end - seg_begin : 0;
  const int nt = (int)((seg_toks + C - 1) / C);
  const long long first = seg_toks > 0 ? (REV ? (long long)T - seg_end : seg_begin) : 0;
  // one buffer view per matrix for the whole segment: rows past its end read 0
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(A.K + ((size_t)bh * T + first) * D, seg_toks * ROWB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(A.V + ((size_t)bh * T + first) * D, seg_toks * ROWB);
  const __amdgpu_buffer_rsrc_t re = make_rsrc(A.eta + (size_t)bh * T + first, seg_toks * 4);

  unsigned gofs[Cfg::MAT_LOADS];
#pragma unroll
  for (int k = 0; k < Cfg::MAT_LOADS; ++k) {
    const int b = (w * Cfg::MAT_LOADS + k) * 1024 + 16 * l;
    const int row = b / ROWB, ph = (b % ROWB) >> 4;
    gofs[k] = (unsigned)(row * ROWB + ((ph ^ seg_swz<D>(row)) << 4));
  }
  const unsigned eofs = (unsigned)((w * Cfg::EPW + l) * 4);
  // transposed reads of this wave's key half: K rows 32kc + 4g + li/4 (+16), V likewise
  const int trow = 4 * g + (li >> 2);
  const unsigned khalf = (unsigned)(2 * kc * 16 * ROWB);
  unsigned ktr[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) ktr[m] = khalf + seg_ktr<D>(m, g, li);
  const unsigned vtr =
      khalf + (unsigned)(trow * ROWB + (((2 * c + ((li >> 1) & 1)) ^ seg_swz<D>(trow)) << 4) + (li & 1) * 8);

  auto issue = [&](int i) {
    unsigned char* st = smem + (i % Cfg::STAGES) * Cfg::STAGE;
    const unsigned t = (unsigned)i * MAT;
#pragma unroll
    for (int k = 0; k < Cfg::MAT_LOADS; ++k) dma16<PT_STREAM>(rk, t + gofs[k], st + (w * Cfg::MAT_LOADS + k) * 1024);
#pragma unroll
    for (int k = 0; k < Cfg::MAT_LOADS; ++k)
      dma16<PT_STREAM>(rv, t + gofs[k], st + MAT + (w * Cfg::MAT_LOADS + k) * 1024);
    if (l < Cfg::EPW) dma4<PT_STREAM>(re, (unsigned)i * (C * 4) + eofs, st + 2 * MAT + w * Cfg::EPW * 4);
  };

  floatx4 S[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) S[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < Cfg::STAGES - 1; ++k)
    if (nt > 0) issue(k);
  for (int i = 0; i < nt; ++i) {
    wait_vm_barrier<(Cfg::STAGES - 2) * Cfg::LOADS>();   // tile i landed; slot of tile i-1 free
    issue(i + Cfg::STAGES - 1);
    const unsigned char* st = smem + (i % Cfg::STAGES) * Cfg::STAGE;
    const unsigned char* ks = st;
    const unsigned char* vs = st + MAT;
    const float* es = (const float*)(st + 2 * MAT);
    // diag(eta) V for keys 32kc + 4g + j (first 16) and 32kc + 16 + 4g + j, column 16c + li
    const uint2 v0 = __builtin_bit_cast(uint2, lds_read_tr16(vs + vtr));
    const uint2 v1 = __builtin_bit_cast(uint2, lds_read_tr16(vs + 16 * ROWB + vtr));
    bf16x8 evh, evl;
    if constexpr (UNIT) {
      evh = join(__builtin_bit_cast(bf16x4, v0), __builtin_bit_cast(bf16x4, v1));
    } else {
      const floatx4 e0 = *(const floatx4*)(es + 32 * kc + 4 * g);
      const floatx4 e1 = *(const floatx4*)(es + 32 * kc + 16 + 4 * g);
      split8(floatx4{e0[0] * bf16lo_f(v0.x), e0[1] * bf16hi_f(v0.x), e0[2] * bf16lo_f(v0.y), e0[3] * bf16hi_f(v0.y)},
             floatx4{e1[0] * bf16lo_f(v1.x), e1[1] * bf16hi_f(v1.x), e1[2] * bf16lo_f(v1.y), e1[3] * bf16hi_f(v1.y)},
             evh, evl);
    }
    bf16x8 a[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) a[m] = join(lds_read_tr16(ks + ktr[m]), lds_read_tr16(ks + 16 * ROWB + ktr[m]));
#pragma unroll
    for (int m = 0; m < MT; ++m) S[m] = mfma16(a[m], evh, S[m]);
    if constexpr (!UNIT) {
#pragma unroll
      for (int m = 0; m < MT; ++m) S[m] = mfma16(a[m], evl, S[m]);
    }
  }
  // key half 1 of each column tile -> LDS (the ring is idle once every copy has landed), half 0 adds it
  wait_vm_barrier<0>();
  floatx4* red = (floatx4*)smem + (size_t)c * MT * WAVE + l;
  if (kc == 1) {
#pragma unroll
    for (int m = 0; m < MT; ++m) red[m * WAVE] = S[m];
  }
  barrier();
  if (kc == 0) {
    floatx4* pp = A.part + (((size_t)bh * nseg + s) * NC + c) * MT * 64 + l;
#pragma unroll
    for (int m = 0; m < MT; ++m) __builtin_nontemporal_store(S[m] + red[m * WAVE], pp + m * 64);
  }
}

// Start states of the segments of one head, in place: slot s holds dS_s
// (s < nseg-1) on entry and S_start(s) = W0 + sum_{s' < s} dS_s' on exit,
// for s >= 1 (the first segment reads W0 itself, slot 0 is left as it is).
// Non-temporal stores: the states are read once, by the output pass.
// Layout of a slot: [wave W][m-tile][lane][4] floats, lane (g, li) of wave W
// holding rows seg_srow(m, g, r), column 16W + li.  One thread per 4 floats.
template <int D>
__global__ __launch_bounds__(256) void pt_seg_scan_kernel(const float* __restrict__ W0, floatx4* __restrict__ part,
                                                          int nseg) {
  constexpr int MT = D / 16, PER = D * D / 4;   // floatx4 per slot
  const int per_head_blocks = PER / 256;
  const int bh = blockIdx.x / per_head_blocks;
  const int f = (blockIdx.x % per_head_blocks) * 256 + threadIdx.x;
  const int W = f / (MT * 64), m = (f / 64) % MT, l = f % 64, g = l >> 4, li = l & 15;
  const float* W0h = W0 + (size_t)bh * D * D;
  floatx4 run;
#pragma unroll
  for (int r = 0; r < 4; ++r) run[r] = W0h[(size_t)seg_srow(m, g, r) * D + 16 * W + li];
  floatx4* ph = part + (size_t)bh * nseg * PER + f;
  // up to 8 increments are loaded before any slot is rewritten (one memory round trip per 8 segments)
  for (int s0 = 0; s0 < nseg - 1; s0 += 8) {
    const int n = min(8, nseg - 1 - s0);
    floatx4 d[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) d[k] = ph[(size_t)(s0 + min(k, n - 1)) * PER];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < n) {
        if (s0 + k > 0) __builtin_nontemporal_store(run, ph + (size_t)(s0 + k) * PER);
        run += d[k];
      }
  }
  __builtin_nontemporal_store(run, ph + (size_t)(nseg - 1) * PER);
}

// ---------------------------------------------------------------------------
// fp32 kernel: same chunked form on the vector ALUs, everything staged in
// LDS.  Used for float32 inputs where bf16 rounding would exceed the fp32
// accuracy budget.  One workgroup per (b,h) x 32-column tile of d_v.  Each
// product is register-blocked (a thread owns a small block of its result and
// reads its operands as 16-byte pieces), so the inner loops issue one LDS
// read per 4 FMAs or better, with independent accumulators.
// ---------------------------------------------------------------------------
template <int DK, int C>
struct Fp32Cfg {
  static constexpr int TV = 32;                 // state / output columns per workgroup
  static constexpr int QP = DK + 4;             // padded rows of q, k (16-byte aligned, conflict-free blocks)
  static constexpr int PP = C + 4;              // padded rows of the score tile
  static constexpr int SB = C / 16;             // score block per thread: SB x SB (256 threads cover C x C)
  static constexpr int OFF_K = C * QP;
  static constexpr int OFF_V = 2 * C * QP;
  static constexpr int OFF_E = OFF_V + C * TV;
  static constexpr int OFF_P = OFF_E + C;
  static constexpr int OFF_S = OFF_P + C * PP;
  static constexpr int FLOATS = OFF_S + DK * TV;
  static_assert(C % 16 == 0 && DK % 32 == 0, "tile shape");
};

// REV and EM as for the bf16 output pass: REV walks the head's sequence in
// reverse (chunk row r of chunk c is original token T - 1 - (cC + r)); EM
// places the rates on the keys (0), on the outputs (1) or nowhere (2).
// PAR (short sequences, few heads): one workgroup per (head, column tile,
// chunk) instead of per (head, column tile): the workgroup of chunk c adds
// the state updates of the tokens before the chunk itself (each thread its
// own state entries, token by token in order as the chunk loop does, reading
// keys, values and rates straight from memory with no barrier in between)
// and then computes chunk c's outputs, so the chunks' score and output
// phases run in parallel; only the last chunk's workgroup takes its own
// state update and writes W_out.
template <int DK, int C, bool EXCL, bool REV = false, int EM = 0, bool PAR = false>
__global__ __launch_bounds__(256) void per_token_fp32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ eta, const float* __restrict__ W0, float* __restrict__ O,
    float* __restrict__ Wout, int T, int DV) {
  using Cfg = Fp32Cfg<DK, C>;
  constexpr int TV = Cfg::TV, QP = Cfg::QP, PP = Cfg::PP, SB = Cfg::SB;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* q = (float*)smem;              // [C][QP]
  float* k = q + Cfg::OFF_K;            // [C][QP]
  float* v = q + Cfg::OFF_V;            // [C][TV]
  float* e = q + Cfg::OFF_E;            // [C]
  float* p = q + Cfg::OFF_P;            // [C][PP]: eta_j * (q_i . k_j) for j <= i, else 0
  float* s = q + Cfg::OFF_S;            // [DK][TV]
  const int NV = DV / TV;
  const int nchunks = (T + C - 1) / C;
  const int wg = PAR ? (int)blockIdx.x / nchunks : (int)blockIdx.x;
  const int c_own = PAR ? (int)blockIdx.x % nchunks : nchunks - 1;   // the last chunk this workgroup reaches
  const int bh = wg / NV;
  const int tv0 = (wg % NV) * TV;
  const int tid = threadIdx.x;
  const float* Qh = Q + (size_t)bh * T * DK;
  const float* Kh = K + (size_t)bh * T * DK;
  const float* Vh = V + (size_t)bh * T * DV;
  const float* Eh = eta + (size_t)bh * T;
  float* Oh = O + (size_t)bh * T * DV;
  // thread roles: score block (rows SB*bi.., cols SB*bj..); output / state column group cg (4 columns)
  const int bi = tid / 16, bj = tid % 16;
  const int cg = tid % 8, r8 = tid / 8;
  // original token of position t of the walk
  auto tok = [&](int t) -> size_t { return REV ? (size_t)(T - 1 - t) : (size_t)t; };
  constexpr int RS = DK / 32;           // state rows r8 + 32m of each thread
  static_assert(TV == 32, "8 column groups of 4 x 32 row groups cover the state tile");
  if constexpr (PAR) {
    // the state before chunk c_own: W0 plus every earlier token's update, in token order
    floatx4 acc[RS];
#pragma unroll
    for (int m = 0; m < RS; ++m)
      acc[m] = *(const floatx4*)(W0 + (size_t)bh * DK * DV + (size_t)(r8 + 32 * m) * DV + tv0 + 4 * cg);
    const int tend = c_own * C;   // < T
#pragma unroll 8
    for (int t = 0; t < tend; ++t) {
      const size_t o = tok(t);
      const floatx4 ev = (EM == 0 ? Eh[o] : 1.f) * *(const floatx4*)(Vh + o * DV + tv0 + 4 * cg);
#pragma unroll
      for (int m = 0; m < RS; ++m) acc[m] += Kh[o * DK + r8 + 32 * m] * ev;
    }
#pragma unroll
    for (int m = 0; m < RS; ++m) *(floatx4*)(s + (r8 + 32 * m) * TV + 4 * cg) = acc[m];
  } else {
    for (int i = tid; i < DK * TV / 4; i += 256) {
      const int a = i / (TV / 4), n4 = i % (TV / 4);
      *(floatx4*)(s + a * TV + 4 * n4) = *(const floatx4*)(W0 + (size_t)bh * DK * DV + (size_t)a * DV + tv0 + 4 * n4);
    }
  }
  for (int c = PAR ? c_own : 0; c <= c_own; ++c) {
    const int t0 = c * C;
    const bool out = !PAR || c == c_own;                        // this chunk's outputs (workgroup-uniform)
    const bool upd = !PAR || c < c_own || c_own == nchunks - 1;  // its state update is needed here
    __syncthreads();
    for (int i = tid; i < C * DK / 4; i += 256) {
      const int r = i / (DK / 4), a4 = i % (DK / 4);
      const bool ok = t0 + r < T;
      const floatx4 z = {0.f, 0.f, 0.f, 0.f};
      if (out) *(floatx4*)(q + r * QP + 4 * a4) = ok ? *(const floatx4*)(Qh + tok(t0 + r) * DK + 4 * a4) : z;
      *(floatx4*)(k + r * QP + 4 * a4) = ok ? *(const floatx4*)(Kh + tok(t0 + r) * DK + 4 * a4) : z;
    }
    for (int i = tid; i < C * TV / 4; i += 256) {
      const int r = i / (TV / 4), n4 = i % (TV / 4);
      const floatx4 z = {0.f, 0.f, 0.f, 0.f};
      *(floatx4*)(v + r * TV + 4 * n4) = (t0 + r < T) ? *(const floatx4*)(Vh + tok(t0 + r) * DV + tv0 + 4 * n4) : z;
    }
    for (int i = tid; i < C; i += 256) e[i] = (t0 + i < T) ? Eh[tok(t0 + i)] : 0.f;
    __syncthreads();
    if (out) {
      // scores with the causal mask (diagonal included) and eta of the key token: SB x SB block per thread
      if (bj <= bi) {
        float acc[SB][SB];
#pragma unroll
        for (int r = 0; r < SB; ++r)
#pragma unroll
          for (int cc = 0; cc < SB; ++cc) acc[r][cc] = 0.f;
#pragma unroll 2
        for (int a = 0; a < DK; a += 4) {
          floatx4 qa[SB], ka[SB];
#pragma unroll
          for (int r = 0; r < SB; ++r) qa[r] = *(const floatx4*)(q + (SB * bi + r) * QP + a);
#pragma unroll
          for (int cc = 0; cc < SB; ++cc) ka[cc] = *(const floatx4*)(k + (SB * bj + cc) * QP + a);
#pragma unroll
          for (int r = 0; r < SB; ++r)
#pragma unroll
            for (int cc = 0; cc < SB; ++cc)
#pragma unroll
              for (int x = 0; x < 4; ++x) acc[r][cc] = fmaf(qa[r][x], ka[cc][x], acc[r][cc]);
        }
#pragma unroll
        for (int r = 0; r < SB; ++r)
#pragma unroll
          for (int cc = 0; cc < SB; ++cc) {
            const int i = SB * bi + r, j = SB * bj + cc;
            p[i * PP + j] = (EXCL ? j < i : j <= i) ? (EM == 0 ? acc[r][cc] * e[j] : acc[r][cc]) : 0.f;
          }
      } else {
#pragma unroll
        for (int r = 0; r < SB; ++r)
#pragma unroll
          for (int cc = 0; cc < SB; ++cc) p[(SB * bi + r) * PP + SB * bj + cc] = 0.f;
      }
      __syncthreads();
      // outputs: rows r8 + 32m, columns 4cg..4cg+3
#pragma unroll 1
      for (int i = r8; i < C; i += 32) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int j = 0; j < C; ++j) acc += p[i * PP + j] * *(const floatx4*)(v + j * TV + 4 * cg);
        floatx4 acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int a = 0; a < DK; a += 4) {
          const floatx4 qa = *(const floatx4*)(q + i * QP + a);
#pragma unroll
          for (int x = 0; x < 4; ++x) acc2 += qa[x] * *(const floatx4*)(s + (a + x) * TV + 4 * cg);
        }
        if (t0 + i < T)
          *(floatx4*)(Oh + tok(t0 + i) * DV + tv0 + 4 * cg) = EM == 1 ? e[i] * (acc + acc2) : acc + acc2;
      }
      __syncthreads();
    }
    // state: rows r8 + 32m of s, columns 4cg..4cg+3, over the chunk's keys
    if (upd) {
      floatx4 acc[RS];
#pragma unroll
      for (int m = 0; m < RS; ++m) acc[m] = *(const floatx4*)(s + (r8 + 32 * m) * TV + 4 * cg);
#pragma unroll 4
      for (int j = 0; j < C; ++j) {
        const floatx4 ev = (EM == 0 ? e[j] : 1.f) * *(const floatx4*)(v + j * TV + 4 * cg);
#pragma unroll
        for (int m = 0; m < RS; ++m) acc[m] += k[j * QP + r8 + 32 * m] * ev;
      }
#pragma unroll
      for (int m = 0; m < RS; ++m) *(floatx4*)(s + (r8 + 32 * m) * TV + 4 * cg) = acc[m];
    }
  }
  __syncthreads();
  if (PAR && c_own != nchunks - 1) return;   // workgroup-uniform
  for (int i = tid; i < DK * TV / 4; i += 256) {
    const int a = i / (TV / 4), n4 = i % (TV / 4);
    *(floatx4*)(Wout + (size_t)bh * DK * DV + (size_t)a * DV + tv0 + 4 * n4) = *(const floatx4*)(s + a * TV + 4 * n4);
  }
}

// The float32 kernel's PAR form repeats the earlier chunks' state updates in every chunk's workgroup
// (quadratic in the chunk count): only for short sequences.
constexpr long long FP32_PAR_MAX_CHUNKS = 16;

template <int DK, int C>
static size_t fp32_lds_bytes() {
  return sizeof(float) * Fp32Cfg<DK, C>::FLOATS;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int DK, int C>
static hipError_t launch_fp32(const PerTokenArgs& a, hipStream_t stream, const Timing& tm) {
  // few (head, column tile) workgroups over a short sequence: one workgroup per chunk as well (PAR)
  const long long wgs = a.B * a.H * (a.DV / 32), nchunks = (a.T + C - 1) / C;
  const bool par = nchunks >= 2 && nchunks <= FP32_PAR_MAX_CHUNKS && wgs * nchunks <= 256;
  auto kern = par ? (a.exclusive ? per_token_fp32_kernel<DK, C, true, false, 0, true>
                                 : per_token_fp32_kernel<DK, C, false, false, 0, true>)
                  : (a.exclusive ? per_token_fp32_kernel<DK, C, true> : per_token_fp32_kernel<DK, C, false>);
  const size_t lds = fp32_lds_bytes<DK, C>();
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int grid = (int)(par ? wgs * nchunks : wgs);
  if ((e = mark(tm.start, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, stream, (const float*)a.Q, (const float*)a.K,
                     (const float*)a.V, a.eta, a.W0, (float*)a.O, a.W_out, (int)a.T, (int)a.DV);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return mark(tm.stop, stream);
}

bool per_token_supported(int64_t dk, int64_t dv, int64_t chunk, int dtype) {
  if (dk != dv || (dk != 64 && dk != 128)) return false;
  if (chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128) return false;
  if (dtype == 0 && chunk > 64) return false;
  return true;
}

// Segment plan of the bf16 path: about one workgroup per workgroup slot of
// the chip (256 compute units x workgroups per CU) over heads x segments,
// each segment whole tiles of both passes (multiples of 64 tokens).
SegPlan per_token_seg_plan(int64_t BH, int64_t T, int64_t dk, int64_t max_seg_tokens) {
  const int64_t slots = 256 * (dk == 128 ? SegCfg<128, seg_tile<128>()>::WG_PER_CU : SegCfg<64, seg_tile<64>()>::WG_PER_CU);
  const int64_t nchunks = (T + 63) / 64;
  int64_t p = BH >= slots ? 1 : slots / BH;
  p = std::max<int64_t>(1, std::min(p, nchunks));
  // a segment's bytes are addressed with 32-bit offsets below 2^31: at most max_seg_tokens tokens each
  const int64_t max_tiles = max_seg_tokens / 64;
  p = std::max<int64_t>(p, (nchunks + max_tiles - 1) / max_tiles);
  const int64_t tiles = nchunks > 0 ? (nchunks + p - 1) / p : 0;
  const int64_t nseg = tiles > 0 ? (nchunks + tiles - 1) / tiles : 1;
  return SegPlan{(int)nseg, (int)(tiles * 64)};
}

// float32 output rows of a segment stay below 2^31 bytes: 2^21 tokens at d = 128
constexpr int64_t F32_OUT_MAX_SEG_TOKENS = (int64_t)1 << 21;

size_t per_token_workspace(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int dtype, int o_f32) {
  if (dtype != 1) return 0;
  const SegPlan sp = per_token_seg_plan(B * H, T, dk, o_f32 ? F32_OUT_MAX_SEG_TOKENS : ((int64_t)1 << 22));
  return sp.nseg > 1 ? (size_t)sp.nseg * (size_t)(B * H) * (size_t)dk * (size_t)dv * sizeof(float) : 0;
}

// The three kernels of one bf16 pass over every head (forward order, or reversed with REV).
template <int D, bool REV, int EM, bool OF32 = false, bool DOT = false>
static hipError_t launch_seg_pass(const SegArgs& A, int BH, bool excl, hipStream_t stream, const Timing& tm) {
  // (start_transposed: the slots already hold the transposed start states; no increments, no scan)
  using CfgD = IncrCfg<D>;
  using CfgF = SegCfg<D, seg_tile<D>()>;
  // The scan kernel turns the increments into start states, so each output workgroup loads one
  // slot (measured: cheaper than summing the earlier slots in every workgroup's prologue, the
  // increments are still in the last-level cache when the scan reads them).
  hipError_t e;
  if (A.nseg > 1 && !A.start_transposed) {
    auto kd = pt_incr_kernel<D, REV, EM != 0>;
    if ((e = hipFuncSetAttribute((const void*)kd, hipFuncAttributeMaxDynamicSharedMemorySize, CfgD::LDS_BYTES)) !=
        hipSuccess)
      return e;
    hipLaunchKernelGGL(kd, dim3(BH * (A.nseg - 1)), dim3(CfgD::THREADS), CfgD::LDS_BYTES, stream, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(pt_seg_scan_kernel<D>, dim3(BH * (D * D / 4 / 256)), dim3(256), 0, stream, A.W0, A.part,
                       A.nseg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  auto kf = excl ? pt_seg_kernel<D, seg_tile<D>(), true, REV, EM, OF32, DOT>
                 : pt_seg_kernel<D, seg_tile<D>(), false, REV, EM, OF32, DOT>;
  if ((e = hipFuncSetAttribute((const void*)kf, hipFuncAttributeMaxDynamicSharedMemorySize, CfgF::LDS_BYTES)) !=
      hipSuccess)
    return e;
  if ((e = mark(tm.start, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(kf, dim3(BH * A.nseg), dim3(CfgF::THREADS), CfgF::LDS_BYTES, stream, A);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return mark(tm.stop, stream);
}

template <int D>
static hipError_t launch_seg(const PerTokenArgs& a, hipStream_t stream, const Timing& tm) {
  const int BH = (int)(a.B * a.H);
  const SegPlan sp = per_token_seg_plan(BH, a.T, D, a.o_f32 ? F32_OUT_MAX_SEG_TOKENS : ((int64_t)1 << 22));
  // (SegArgs.O is typed bf16; with float32 outputs the kernel writes floats through it)
  const SegArgs A{(const bf16*)a.Q, (const bf16*)a.K, (const bf16*)a.V, a.eta, a.W0, (floatx4*)a.ws,
                  (bf16*)a.O, a.W_out, (int)a.T, sp.nseg, sp.seg_len};
  if (a.o_f32) return launch_seg_pass<D, false, 0, true>(A, BH, a.exclusive != 0, stream, tm);
  return launch_seg_pass<D, false, 0>(A, BH, a.exclusive != 0, stream, tm);
}

hipError_t launch_per_token(const PerTokenArgs& a, hipStream_t stream, const Timing& tm) {
  if (a.dtype == 0) {
    const int c = a.chunk <= 16 ? 16 : a.chunk <= 32 ? 32 : 64;
    if (a.DK == 64) return c == 16 ? launch_fp32<64, 16>(a, stream, tm) : c == 32 ? launch_fp32<64, 32>(a, stream, tm) : launch_fp32<64, 64>(a, stream, tm);
    return c == 16 ? launch_fp32<128, 16>(a, stream, tm) : c == 32 ? launch_fp32<128, 32>(a, stream, tm) : launch_fp32<128, 64>(a, stream, tm);
  }
  return a.DK == 128 ? launch_seg<128>(a, stream, tm) : launch_seg<64>(a, stream, tm);
}


// ---------------------------------------------------------------------------
// Backward of the bf16 per-token form.  With G_t = dW_T + sum over the reads
// at or after step t (strictly after for the exclusive read) of q^T dO, the
// gradients are dq_t = dO_t S_t^T, dk_t = eta_t v_t G_t^T, dv_t = eta_t k_t G_t,
// deta_t = <k_t G_t, v_t> and dW0 = G_0 (the memory's gradient after the
// first token).  Each is the forward recurrence with other operands and the
// rates placed elsewhere:
//   dQ:  queries dO, keys V, values K, rates on the keys, from W0^T  (forward order)
//   u:   queries K, keys Q, values dO, unit rates, from dW_T
//        (reverse order: u_t = k_t G_t, written into dV; the final memory is dW0)
//   dK:  queries V, keys dO, values Q, rates on the outputs, from dW_T^T
//        (reverse order: dk_t = eta_t v_t G_t^T)
// then one elementwise pass turns u into dV = eta u and deta = <u, v>.
// The gradients are written as float32 (a bf16 result could not be more
// accurate than its own rounding, which for these heavy-tailed rows is about
// the size of the accuracy budget).
// Workspace: the segment slots (shared by the passes, which run in stream
// order), W0^T, dW_T^T and a discarded final memory.
// ---------------------------------------------------------------------------
// float32 rows of a segment must stay below 2^31 bytes: 2^21 tokens at d = 128
constexpr int64_t BWD_MAX_SEG_TOKENS = (int64_t)1 << 21;
struct BwdLayout {
  size_t slots, w0t, dwt, junk, dpart, total;
};
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static BwdLayout bwd_layout(int64_t B, int64_t H, int64_t T, int64_t D) {
  BwdLayout L;
  const size_t BH = (size_t)(B * H), st = BH * D * D * 4;
  size_t o = 0;
  const SegPlan sp = per_token_seg_plan(B * H, T, D, BWD_MAX_SEG_TOKENS);
  L.slots = o; o += align256(sp.nseg > 1 ? (size_t)sp.nseg * st : 0);
  L.w0t = o; o += align256(st);
  L.dwt = o; o += align256(st);
  L.junk = o; o += align256(st);
  L.dpart = o; o += align256((size_t)B * H * T * (D / 16) * 4);   // bf16 path: the u pass's partial dots
  L.total = o;
  return L;
}

size_t per_token_backward_workspace(int64_t B, int64_t H, int64_t T, int64_t dk) {
  return bwd_layout(B, H, T, dk).total;
}

// at[bh] = a[bh]^T and bt[bh] = b[bh]^T for D x D fp32 matrices: one 64 x 64
// tile of one matrix per workgroup (grid BH x 2 x (D/64)^2), read and written
// in whole rows through LDS.
template <int D>
__global__ __launch_bounds__(256) void pt_transpose2_kernel(const float* __restrict__ a, const float* __restrict__ b,
                                                            float* __restrict__ at, float* __restrict__ bt) {
  constexpr int NT = D / 64;
  __shared__ float tile[64][65];
  const int bh = blockIdx.x / (2 * NT * NT), which = (blockIdx.x / (NT * NT)) % 2, tt = blockIdx.x % (NT * NT);
  const int tr = tt / NT, tc = tt % NT;            // source tile row, column
  const float* src = (which ? b : a) + (size_t)bh * D * D;
  float* dst = (which ? bt : at) + (size_t)bh * D * D;
  const int x = threadIdx.x & 63, y0 = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int y = y0 + 4 * k;
    tile[y][x] = src[(size_t)(64 * tr + y) * D + 64 * tc + x];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int y = y0 + 4 * k;
    dst[(size_t)(64 * tc + y) * D + 64 * tr + x] = tile[x][y];
  }
}

// In place: u -> dV = eta u, and deta = <u, v> per token (u fp32, V bf16 or
// fp32).  A token's row is covered by D/8 consecutive lanes, 8 values each;
// the products are summed over those lanes.
__device__ __forceinline__ void v8_of(const bf16* p, floatx4& a, floatx4& b) {
  const u32x4 vv = *(const u32x4*)p;
  a = floatx4{bf16lo_f(vv[0]), bf16hi_f(vv[0]), bf16lo_f(vv[1]), bf16hi_f(vv[1])};
  b = floatx4{bf16lo_f(vv[2]), bf16hi_f(vv[2]), bf16lo_f(vv[3]), bf16hi_f(vv[3])};
}
__device__ __forceinline__ void v8_of(const float* p, floatx4& a, floatx4& b) {
  a = *(const floatx4*)p;
  b = *(const floatx4*)(p + 4);
}
template <int D, typename VT>
__global__ __launch_bounds__(256) void pt_bwd_rate_grad_kernel(float* __restrict__ u, const VT* __restrict__ V,
                                                               const float* __restrict__ eta, float* __restrict__ deta,
                                                               long long ntok) {
  constexpr int LPT = D / 8;          // lanes per token
  constexpr int TPB = 256 / LPT;      // tokens per block and step
  const int sub = threadIdx.x % LPT;
  for (long long t = (long long)blockIdx.x * TPB + threadIdx.x / LPT; t < ntok; t += (long long)gridDim.x * TPB) {
    const size_t o = (size_t)t * D + sub * 8;
    const floatx4 u0 = *(const floatx4*)(u + o), u1 = *(const floatx4*)(u + o + 4);
    floatx4 v0, v1;
    v8_of(V + o, v0, v1);
    const float e = eta[t];
    *(floatx4*)(u + o) = e * u0;
    *(floatx4*)(u + o + 4) = e * u1;
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) dot = fmaf(u0[j], v0[j], dot);
#pragma unroll
    for (int j = 0; j < 4; ++j) dot = fmaf(u1[j], v1[j], dot);
#pragma unroll
    for (int m = LPT / 2; m >= 1; m >>= 1) dot += __shfl_xor(dot, m);   // within the token's lanes
    if (sub == 0) deta[t] = dot;
  }
}

// deta_t = <u_t, v_t> from the u pass's per-wave partials (NW of them per token, summed in wave order).
template <int NW>
__global__ __launch_bounds__(256) void pt_bwd_dot_sum_kernel(const float* __restrict__ dpart, float* __restrict__ deta,
                                                             long long ntok) {
  for (long long t = (long long)blockIdx.x * 256 + threadIdx.x; t < ntok; t += (long long)gridDim.x * 256) {
    float x = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) x += dpart[t * NW + w];
    deta[t] = x;
  }
}

template <int D>
static hipError_t launch_bwd(const BackwardArgs& a, hipStream_t stream) {
  const int BH = (int)(a.B * a.H);
  const long long ntok = (long long)BH * a.T;
  const BwdLayout L = bwd_layout(a.B, a.H, a.T, D);
  char* ws = (char*)a.ws;
  float* w0t = (float*)(ws + L.w0t);
  float* dwt = (float*)(ws + L.dwt);
  float* junk = (float*)(ws + L.junk);
  floatx4* slots = (floatx4*)(ws + L.slots);
  const bf16 *Q = (const bf16*)a.Q, *K = (const bf16*)a.K, *V = (const bf16*)a.V, *dO = (const bf16*)a.dO;
  hipError_t e;
  hipLaunchKernelGGL(pt_transpose2_kernel<D>, dim3(BH * 2 * (D / 64) * (D / 64)), dim3(256), 0, stream, a.W0, a.dW,
                     w0t, dwt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const SegPlan sp = per_token_seg_plan(BH, a.T, D, BWD_MAX_SEG_TOKENS);
  const int T = (int)a.T;
  const bool excl = a.other_order != 0;
  const Timing none;
  // (SegArgs.O is typed bf16; the OF32 passes write floats through it)
  const SegArgs Aq{dO, V, K, a.eta, w0t, slots, (bf16*)a.dQ, junk, T, sp.nseg, sp.seg_len};
  if ((e = launch_seg_pass<D, false, 0, true>(Aq, BH, excl, stream, none)) != hipSuccess) return e;
  // u_t = k_t G_t: written as dV = eta u (rates on the outputs), with the partials of deta = <u, v>
  float* dpart = (float*)(ws + L.dpart);
  SegArgs Au{K, Q, dO, a.eta, a.dW, slots, (bf16*)a.dV, a.dW0, T, sp.nseg, sp.seg_len};
  Au.aux = V;
  Au.dpart = dpart;
  if ((e = launch_seg_pass<D, true, 1, true, true>(Au, BH, excl, stream, none)) != hipSuccess) return e;
  // G^T's recurrence has the transposed increments and start states: it reuses the u pass's slots
  const SegArgs Ak{V, dO, Q, a.eta, dwt, slots, (bf16*)a.dK, junk, T, sp.nseg, sp.seg_len, 1};
  if ((e = launch_seg_pass<D, true, 1, true>(Ak, BH, excl, stream, none)) != hipSuccess) return e;
  if (ntok > 0) {
    const unsigned grid = (unsigned)std::min<long long>((ntok + 255) / 256, 8192);
    hipLaunchKernelGGL((pt_bwd_dot_sum_kernel<D / 16>), dim3(grid), dim3(256), 0, stream, dpart, a.deta, ntok);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

// float32 inputs: the same three passes with the float32 kernel (tiles of `chunk` tokens, one
// workgroup per head and 32 columns, sequential over the head's tiles)
template <int DK, int C>
static hipError_t launch_bwd_fp32(const BackwardArgs& a, hipStream_t stream) {
  const int BH = (int)(a.B * a.H), T = (int)a.T, DV = (int)a.DV;
  const long long ntok = (long long)BH * a.T;
  const BwdLayout L = bwd_layout(a.B, a.H, a.T, DK);
  char* ws = (char*)a.ws;
  float* w0t = (float*)(ws + L.w0t);
  float* dwt = (float*)(ws + L.dwt);
  float* junk = (float*)(ws + L.junk);
  const float *Q = (const float*)a.Q, *K = (const float*)a.K, *V = (const float*)a.V, *dO = (const float*)a.dO;
  const bool excl = a.other_order != 0;
  hipError_t e;
  hipLaunchKernelGGL(pt_transpose2_kernel<DK>, dim3(BH * 2 * (DK / 64) * (DK / 64)), dim3(256), 0, stream, a.W0, a.dW,
                     w0t, dwt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t lds = fp32_lds_bytes<DK, C>();
  const long long wgs = (long long)BH * (DV / 32), nchunks = (a.T + C - 1) / C;
  const bool par = nchunks >= 2 && nchunks <= FP32_PAR_MAX_CHUNKS && wgs * nchunks <= 256;
  auto pass = [&](auto kern, const float* q, const float* k, const float* v, const float* w0, float* o,
                  float* wout) -> hipError_t {
    hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3((unsigned)(par ? wgs * nchunks : wgs)), dim3(256), lds, stream, q, k, v, a.eta, w0,
                       o, wout, T, DV);
    return hipGetLastError();
  };
  // the kernel of one pass: read order, walk direction, rate placement, and the PAR form for short sequences
  auto pick = [&](auto excl_t, auto rev_t, auto em_t) {
    constexpr bool X = decltype(excl_t)::value, R = decltype(rev_t)::value;
    constexpr int M = decltype(em_t)::value;
    return par ? per_token_fp32_kernel<DK, C, X, R, M, true> : per_token_fp32_kernel<DK, C, X, R, M, false>;
  };
  using F = std::false_type;
  using Tr = std::true_type;
  using E0 = std::integral_constant<int, 0>;
  using E1 = std::integral_constant<int, 1>;
  using E2 = std::integral_constant<int, 2>;
  if ((e = pass(excl ? pick(Tr{}, F{}, E0{}) : pick(F{}, F{}, E0{}), dO, V, K, w0t, (float*)a.dQ, junk)) != hipSuccess)
    return e;
  if ((e = pass(excl ? pick(Tr{}, Tr{}, E2{}) : pick(F{}, Tr{}, E2{}), K, Q, dO, a.dW, (float*)a.dV, a.dW0)) !=
      hipSuccess)
    return e;
  if ((e = pass(excl ? pick(Tr{}, Tr{}, E1{}) : pick(F{}, Tr{}, E1{}), V, dO, Q, dwt, (float*)a.dK, junk)) != hipSuccess)
    return e;
  if (ntok > 0) {
    constexpr int TPB = 256 / (DK / 8);
    const unsigned grid = (unsigned)std::min<long long>((ntok + TPB - 1) / TPB, 8192);
    hipLaunchKernelGGL((pt_bwd_rate_grad_kernel<DK, float>), dim3(grid), dim3(256), 0, stream, (float*)a.dV, V, a.eta,
                       a.deta, ntok);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

bool per_token_backward_supported(int64_t dk, int64_t dv, int64_t chunk, int dtype) {
  return per_token_supported(dk, dv, chunk, dtype);
}

hipError_t launch_per_token_backward(const BackwardArgs& a, hipStream_t stream) {
  if (a.dtype == 0) {
    const int c = a.chunk <= 16 ? 16 : a.chunk <= 32 ? 32 : 64;
    if (a.DK == 64)
      return c == 16 ? launch_bwd_fp32<64, 16>(a, stream) : c == 32 ? launch_bwd_fp32<64, 32>(a, stream)
                                                             : launch_bwd_fp32<64, 64>(a, stream);
    return c == 16 ? launch_bwd_fp32<128, 16>(a, stream) : c == 32 ? launch_bwd_fp32<128, 32>(a, stream)
                                                          : launch_bwd_fp32<128, 64>(a, stream);
  }
  return a.DK == 128 ? launch_bwd<128>(a, stream) : launch_bwd<64>(a, stream);
}

}  // namespace ttt
