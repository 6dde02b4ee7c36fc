// LDS tile staging and MFMA operand helpers shared by the attention kernels (gfx950,
// wave64): direct-to-LDS tile copies with XOR-swizzled 16-byte chunks, exact
// vector-memory waits, and bf16 packing of accumulators into MFMA operands.
#pragma once
#include "common.h"

namespace bsa {

// ---- LDS tile geometry ------------------------------------------------------
// A tile row holds RB = D * elem bytes = NCH 16-byte chunks. 256 bytes of LDS span
// all 64 banks, i.e. 16 chunks; rows shorter than that share a bank line.
template <int RB>
struct TileGeom {
  static constexpr int NCH = RB / 16;           // chunks per row
  static constexpr int RPL = 16 / NCH;          // rows per 256-byte bank line
  // K-style swizzle: 16 consecutive rows at the same chunk hit 16 distinct chunk slots
  static __device__ __forceinline__ int swz_k(int r) { return (r / RPL) % NCH; }
  // V-style swizzle: 4 consecutive rows x 4 consecutive chunks hit 16 distinct slots
  static __device__ __forceinline__ int swz_v(int r) { return 4 * ((r / RPL) % (NCH / 4)); }
};

// One direct-to-LDS 16-byte load per lane: lane L's 16 bytes at gbase + voff land at
// LDS address lds + 16 L. Issued from inline asm so that the compiler does not put a
// blanket wait for every outstanding load in front of each LDS read; the kernel
// waits for exactly the tiles it needs (wait_vm). The instruction has no register
// result; its address operands are read at issue. M0 (the LDS base of the DMA) is
// saved and restored around it.
__device__ __forceinline__ void dma16(const char* gbase, unsigned voff, unsigned lds) {
  unsigned sv;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(sv)
      : "v"(voff), "s"(gbase), "s"(lds)
      : "memory");
}
// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// A tile copy is 64 / RPI instructions of 1 KB, instruction t filling rows
// [t RPI, (t + 1) RPI). Wave w of a P-wave workgroup issues t = u P + w, u = 0 .. NH-1:
// the rows of one wave's instructions are P RPI apart, a multiple of both swizzle
// periods (16 and 4 rows), so all of them use the same per-lane offset and only the
// scalar base moves (one address register per tile instead of NH).
template <int RB, bool VSWZ, int P>
__device__ __forceinline__ void load_tile_part(const char* gtile, unsigned rs, unsigned lds, int lane, int w) {
  using G = TileGeom<RB>;
  constexpr int RPI = 1024 / RB;
  constexpr int NH = 64 / RPI / P;
  static_assert(NH * RPI * P == 64, "tile copy must split evenly");
  static_assert(NH == 1 || (P * RPI) % 16 == 0, "the instructions of a wave must share the swizzle phase");
  const int r0 = w * RPI + lane / G::NCH;
  const int c = (lane % G::NCH) ^ (VSWZ ? G::swz_v(r0) : G::swz_k(r0));
  const unsigned voff = (unsigned)r0 * rs + (unsigned)c * 16u;
#pragma unroll
  for (int u = 0; u < NH; ++u) dma16(gtile + (int64_t)(u * P * RPI) * rs, voff, lds + (u * P + w) * 1024);
}

// byte offset of (row r, byte column cb) in a K-swizzled / V-swizzled tile
template <int RB>
__device__ __forceinline__ int koff(int r, int cb) {
  using G = TileGeom<RB>;
  return r * RB + (((cb >> 4) ^ G::swz_k(r)) << 4) + (cb & 15);
}
template <int RB>
__device__ __forceinline__ int voff(int r, int cb) {
  using G = TileGeom<RB>;
  return r * RB + (((cb >> 4) ^ G::swz_v(r)) << 4) + (cb & 15);
}

// Operand reads of bf16 tiles as lane base ^ step. K-swizzled rows, 16-byte chunk 2s + hi:
// koff(r, 32 s + 16 hi) = koff_lane(r, hi) ^ (32 s) (the swizzle moves bits 4 .. log2(RB)-1
// of the offset only, and bit 4 separately from the others). V-swizzled rows, byte column
// 64 dt + c with c < 64: voff(r, 64 dt + c) = voff(r, c) ^ (64 dt) (the swizzle is a
// multiple of 4 chunks). Rows 4 apart (V) or 16 apart (K) share the swizzle, so other
// rows are these offsets plus a multiple of RB.
template <int RB>
__device__ __forceinline__ int koff_lane(int r, int hi) {
  using G = TileGeom<RB>;
  const int w = G::swz_k(r);
  return r * RB + 16 * (hi ^ (w & 1)) + 32 * (w >> 1);
}
// keeps a value in a register as computed, so that offsets derived from it are formed
// where they are used instead of being hoisted into registers of their own
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ float partner(float x) {
  // value of x in lane (l ^ 32)
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return lane_id() < 32 ? __uint_as_float(r[1]) : __uint_as_float(r[0]);
}

__device__ __forceinline__ bf16x8_t join_bf16x8(s16x4_t a, s16x4_t b) {
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// two floats -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even). MFMA
// operands are assembled from such packed 32-bit words and cast as whole vectors:
// building a bf16 vector element by element is mis-compiled by the current toolchain.
__device__ __forceinline__ unsigned pk_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// acc + (the two bf16 halves of w), in fp32 (v_dot2c_f32_bf16 against (1, 1))
__device__ __forceinline__ float add_bf16_pair(unsigned w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), bf16x2_t{(__bf16)1.0f, (__bf16)1.0f}, acc,
                                         false);
}

// Scheduling order for a run of NM MFMAs that each consume NR LDS reads: the reads of
// the first P MFMAs, then each MFMA followed by the reads of the MFMA P places later.
// Without it the compiler, short of registers, issues each operand read right before
// its MFMA and waits for it there; with it P operand sets are in flight.
template <int NM, int NR, int P>
__device__ __forceinline__ void pipeline_reads() {
  constexpr int D = P < NM ? P : NM;
  __builtin_amdgcn_sched_group_barrier(0x100, NR * D, 0);    // DS reads
#pragma unroll
  for (int x = 0; x < NM - D; ++x) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, D, 0);
}

__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace bsa
