// Device helpers shared by the gfx950 kernels: vector types, bf16
// conversion, MFMA wrappers, LDS transpose reads, direct-to-LDS loads and
// explicit wait counters.
//
// MFMA lane layouts (verified on gfx950):
//   v_mfma_f32_16x16x32_bf16: A[16][32]: lane l holds A[l%16][8*(l/16)+j], j<8
//                             B[32][16]: lane l holds B[8*(l/16)+j][l%16]
//                             D[16][16]: lane l holds D[4*(l/16)+r][l%16], r<4
//   v_mfma_f32_32x32x16_bf16: A: A[l%32][8*(l/32)+j]; B: B[8*(l/32)+j][l%32]
//                             D: reg i of lane l = D[8*(i/4)+4*(l/32)+i%4][l%32]
//   v_mfma_f32_16x16x4_f32:   A: A[l%16][l/16]; B: B[l/16][l%16]; D as 16x16.
// ds_read_b64_tr_b16 (per 16-lane group, each lane addressing 8 bytes):
//   lane i receives element (i%4) of the 8 bytes read by lanes 4*e + i/4,
//   for e = 0..3.  So if lane L of the group addresses row (r0 + L/4),
//   columns (c0 + 4*(L%4)) .. +3 of a row-major 16-bit matrix, lane i gets
//   column c0 + i of rows r0..r0+3: a transposed 4x16 block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) short4v lds_short4;

constexpr int WAVE = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ floatx4 mfma16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx16 mfma32(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x16_bf16: A[16][16]: lane l holds A[l%16][4*(l/16)+j], j<4;
// B[16][16]: B[4*(l/16)+j][l%16]; D as for the 16x16x32 form.
__device__ __forceinline__ floatx4 mfma16k16(const bf16x4& a, const bf16x4& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, a), __builtin_bit_cast(short4v, b), c,
                                                  0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16_f32(float a, float b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Transposed 4x16 read of 16-bit elements from LDS (see header comment).
__device__ __forceinline__ bf16x4 lds_read_tr16(const void* p) {
  short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(uintptr_t)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// 32-bit LDS address of a pointer into LDS (the low half of its generic address).
__device__ __forceinline__ unsigned lds_addr(const void* p) { return (unsigned)(uintptr_t)p; }

// Sixteen transposed reads issued from one inline-asm statement:
// o[4*k + t] = transposed read at LDS byte address a_k + t*STRIDE.
// When the compiler emits this instruction itself it first waits for every
// outstanding global->LDS copy (it cannot tell that they do not overlap),
// which empties a copy pipeline at each use.  Here the batch is issued and
// waited for (lgkmcnt(0)) inside the same statement, so no output register
// is visible to the compiler before its data has arrived.
template <int STRIDE>
__device__ __forceinline__ void lds_tr16_4x4(bf16x4 (&o)[16], unsigned a0, unsigned a1, unsigned a2, unsigned a3) {
  static_assert(STRIDE >= 0 && 3 * STRIDE < 65536, "ds offset out of range");
  uint2 r[16];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:%20\n\t"
      "ds_read_b64_tr_b16 %2, %16 offset:%21\n\t"
      "ds_read_b64_tr_b16 %3, %16 offset:%22\n\t"
      "ds_read_b64_tr_b16 %4, %17\n\t"
      "ds_read_b64_tr_b16 %5, %17 offset:%20\n\t"
      "ds_read_b64_tr_b16 %6, %17 offset:%21\n\t"
      "ds_read_b64_tr_b16 %7, %17 offset:%22\n\t"
      "ds_read_b64_tr_b16 %8, %18\n\t"
      "ds_read_b64_tr_b16 %9, %18 offset:%20\n\t"
      "ds_read_b64_tr_b16 %10, %18 offset:%21\n\t"
      "ds_read_b64_tr_b16 %11, %18 offset:%22\n\t"
      "ds_read_b64_tr_b16 %12, %19\n\t"
      "ds_read_b64_tr_b16 %13, %19 offset:%20\n\t"
      "ds_read_b64_tr_b16 %14, %19 offset:%21\n\t"
      "ds_read_b64_tr_b16 %15, %19 offset:%22\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
        "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]),
        "=&v"(r[15])
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "n"(STRIDE), "n"(2 * STRIDE), "n"(3 * STRIDE));
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = __builtin_bit_cast(bf16x4, r[i]);
}

// Four transposed reads from one base: o[t] = read at a + t*STRIDE.
template <int STRIDE>
__device__ __forceinline__ void lds_tr16_1x4(bf16x4 (&o)[4], unsigned a) {
  static_assert(STRIDE >= 0 && 3 * STRIDE < 65536, "ds offset out of range");
  uint2 r0, r1, r2, r3;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\tds_read_b64_tr_b16 %1, %4 offset:%5\n\t"
      "ds_read_b64_tr_b16 %2, %4 offset:%6\n\tds_read_b64_tr_b16 %3, %4 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a), "n"(STRIDE), "n"(2 * STRIDE), "n"(3 * STRIDE));
  o[0] = __builtin_bit_cast(bf16x4, r0); o[1] = __builtin_bit_cast(bf16x4, r1);
  o[2] = __builtin_bit_cast(bf16x4, r2); o[3] = __builtin_bit_cast(bf16x4, r3);
}

// Batches of transposed reads at arbitrary LDS byte addresses, issued and
// waited for inside one asm statement each (same reason as above):
// o[i] = transposed read at a[i], i < N.
__device__ __forceinline__ void lds_tr16_x8(bf16x4* o, const unsigned* a) {
  uint2 r0, r1, r2, r3, r4, r5, r6, r7;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\tds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\tds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\tds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]));
  o[0] = __builtin_bit_cast(bf16x4, r0); o[1] = __builtin_bit_cast(bf16x4, r1);
  o[2] = __builtin_bit_cast(bf16x4, r2); o[3] = __builtin_bit_cast(bf16x4, r3);
  o[4] = __builtin_bit_cast(bf16x4, r4); o[5] = __builtin_bit_cast(bf16x4, r5);
  o[6] = __builtin_bit_cast(bf16x4, r6); o[7] = __builtin_bit_cast(bf16x4, r7);
}
__device__ __forceinline__ void lds_tr16_x4(bf16x4* o, const unsigned* a) {
  uint2 r0, r1, r2, r3;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\tds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\tds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
  o[0] = __builtin_bit_cast(bf16x4, r0); o[1] = __builtin_bit_cast(bf16x4, r1);
  o[2] = __builtin_bit_cast(bf16x4, r2); o[3] = __builtin_bit_cast(bf16x4, r3);
}
__device__ __forceinline__ void lds_tr16_x2(bf16x4* o, const unsigned* a) {
  uint2 r0, r1;
  asm volatile("ds_read_b64_tr_b16 %0, %2\n\tds_read_b64_tr_b16 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(r0), "=&v"(r1)
               : "v"(a[0]), "v"(a[1]));
  o[0] = __builtin_bit_cast(bf16x4, r0); o[1] = __builtin_bit_cast(bf16x4, r1);
}
template <int N>
__device__ __forceinline__ void lds_tr16_batch(bf16x4* o, const unsigned* a) {
  static_assert(N % 2 == 0, "even batch sizes only");
  if constexpr (N >= 8) {
    lds_tr16_x8(o, a);
    lds_tr16_batch<N - 8>(o + 8, a + 8);
  } else if constexpr (N >= 4) {
    lds_tr16_x4(o, a);
    lds_tr16_batch<N - 4>(o + 4, a + 4);
  } else if constexpr (N == 2) {
    lds_tr16_x2(o, a);
  }
}

__device__ __forceinline__ bf16x8 join(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Asynchronous 16-byte global -> LDS copy.  `lds_wave_base` must be uniform
// across the wave; lane l's 16 bytes land at lds_wave_base + 16*l.
__device__ __forceinline__ void g2lds16(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void*)(uintptr_t)lds_wave_base, 16, 0, 0);
}
// 4-byte variant: lane l's 4 bytes land at lds_wave_base + 4*l.
__device__ __forceinline__ void g2lds4(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void*)(uintptr_t)lds_wave_base, 4, 0, 0);
}

// Buffer resources: raw (stride 0) view of `nbytes` bytes from `base`;
// accesses at or beyond nbytes read 0 and drop writes, which is how the
// kernels treat the ragged end of a sequence.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned uint2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long long nbytes) {
  const int n = nbytes <= 0 ? 0 : (nbytes > 0x7fffffffLL ? 0x7fffffff : (int)nbytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
// 16 bytes per lane from a buffer straight into LDS (lane l -> lds_wave_base + 16*l).
// STREAM: non-temporal load (data read once).
template <bool STREAM = false>
__device__ __forceinline__ void buf2lds16(__amdgpu_buffer_rsrc_t r, unsigned voff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(uintptr_t)lds_wave_base, 16, voff, 0, 0, STREAM ? 2 : 0);
}
template <bool STREAM = false>
__device__ __forceinline__ void buf2lds4(__amdgpu_buffer_rsrc_t r, unsigned voff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(uintptr_t)lds_wave_base, 4, voff, 0, 0, STREAM ? 2 : 0);
}
// The same direct-to-LDS loads issued from inline asm.  The compiler then
// does not see that LDS is written asynchronously and adds no waits of its
// own before LDS reads (its rule for compiler-issued copies is to wait for
// all of them before any LDS read it cannot prove disjoint, transposed reads
// included).  Every read of the destination must therefore be ordered by an
// explicit wait_vm_barrier / wait_vm.  M0 holds the wave's LDS destination;
// it is saved and restored around the load (the compiler treats M0 as
// reserved), and one wait state separates its write from the load.
// STREAM marks data read once: the load is non-temporal, so it does not
// displace cached lines (measured on gfx950: with many dirty lines in the
// caches, streaming loads without the hint run at about half the bandwidth).
#define TTT_DMA_ASM(op, pol)                                                                                     \
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t" op " %1, %2, 0 offen " pol "lds\n\ts_mov_b32 m0, %0" \
               : "=&s"(saved)                                                                                   \
               : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_wave_base)))
template <bool STREAM = false>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned voff, const void* lds_wave_base) {
  unsigned saved;
  if constexpr (STREAM)
    TTT_DMA_ASM("buffer_load_dwordx4", "nt ");
  else
    TTT_DMA_ASM("buffer_load_dwordx4", "");
}
template <bool STREAM = false>
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, unsigned voff, const void* lds_wave_base) {
  unsigned saved;
  if constexpr (STREAM)
    TTT_DMA_ASM("buffer_load_dword", "nt ");
  else
    TTT_DMA_ASM("buffer_load_dword", "");
}
#undef TTT_DMA_ASM
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, unsigned voff, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, 0);
}

// s_waitcnt vmcnt(N) lgkmcnt(0) followed by a workgroup barrier: this
// wave's LDS accesses are complete and at most N of its vector-memory
// operations are outstanding when it arrives.  The "memory" clobber keeps
// the compiler from moving LDS or global accesses across it.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// bf16 hi + lo split of two floats at once: hi = bf16(f) (round to nearest
// even), lo = bf16(f - hi); f = hi + lo to about 16 significant bits.
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Returns {hi, lo}, each a packed bf16 pair (a in the low half).
__device__ __forceinline__ uint2 split2(float a, float b) {
  const unsigned h = __builtin_bit_cast(unsigned, __builtin_convertvector(floatx2{a, b}, bf16x2));
  const float ah = __builtin_bit_cast(float, h << 16), bh = __builtin_bit_cast(float, h & 0xffff0000u);
  return uint2{h, __builtin_bit_cast(unsigned, __builtin_convertvector(floatx2{a - ah, b - bh}, bf16x2))};
}
// Four splits into bf16x8 hi and lo operands (element order a0..a7).
__device__ __forceinline__ void split8(const floatx4& a, const floatx4& b, bf16x8& hi, bf16x8& lo) {
  const uint2 s0 = split2(a[0], a[1]), s1 = split2(a[2], a[3]), s2 = split2(b[0], b[1]), s3 = split2(b[2], b[3]);
  hi = __builtin_bit_cast(bf16x8, u32x4{s0.x, s1.x, s2.x, s3.x});
  lo = __builtin_bit_cast(bf16x8, u32x4{s0.y, s1.y, s2.y, s3.y});
}
// bf16 -> float of the two halves of a packed pair
__device__ __forceinline__ float bf16lo_f(unsigned x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float bf16hi_f(unsigned x) { return __builtin_bit_cast(float, x & 0xffff0000u); }

__device__ __forceinline__ bf16x4 to_bf16x4(float a, float b, float c, float d) {
  bf16x4 r;
  r[0] = (bf16)a; r[1] = (bf16)b; r[2] = (bf16)c; r[3] = (bf16)d;
  return r;
}

// Sum of x over the 64 lanes of a wave, the same value in every lane, in a
// fixed order: within each row of 16 lanes by DPP moves (pair, quad, half-row
// mirror, row mirror), then the four row sums read from lanes 0, 16, 32, 48.
// No LDS traffic, unlike a shuffle butterfly.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f32<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp_f32<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp_f32<0x141>(x);   // row_half_mirror: the other quad of the half row
  x += dpp_f32<0x140>(x);   // row_mirror: the other half of the row
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
  return (r0 + r1) + (r2 + r3);
}

// Map a flat block index to a logical index such that consecutive logical
// indices share an XCD (blocks are dispatched round-robin over 8 XCDs).
// Requires nblocks % 8 == 0.
__device__ __forceinline__ int xcd_logical_block(int b, int nblocks) {
  const int per = nblocks >> 3;
  return (b & 7) * per + (b >> 3);
}

}  // namespace ttt
