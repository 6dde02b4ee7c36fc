// Device-side helpers shared by the kernels of the library (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define BSA_WAVE 64
#define BSA_N 64   // tokens per block
#define BSA_NXCD 8 // XCDs of an MI355X; workgroups are dealt to them round-robin

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

#define BSA_LDS __attribute__((address_space(3)))

// Checked build (-DBSA_CHECKED): indices that kernels read from list data (kv-list entries,
// list lengths) are tested before use; a failed test sets its bit in this translation
// unit's device word (read and cleared by bsa_check_flags) and the access is skipped.
// Elsewhere BSA_CHECK is the constant true and the tests compile away.
enum : unsigned {
  CHK_ATTN_ENTRY = 1u,     // attention: kv-list entry outside [0, nb)
  CHK_ATTN_LEN = 2u,       // attention / work order: list length outside [0, nb]
  CHK_ROW_BITS = 4u,       // pairing: list entry outside the bit row
  CHK_BWD_ENTRY = 8u,      // backward: list entry outside [0, nb)
};
#ifdef BSA_CHECKED
static __device__ unsigned bsa_check_word;
__device__ __forceinline__ bool bsa_check(bool ok, unsigned bit) {
  if (!ok) atomicOr(&bsa_check_word, bit);
  return ok;
}
#define BSA_CHECK(ok, bit) bsa_check((ok), (bit))
// host: this translation unit's word (and clear it), synchronous
#define BSA_CHECK_ACCESSOR(fn)                                              \
  unsigned fn(int clear) {                                                  \
    unsigned v = 0;                                                         \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(bsa_check_word), sizeof v) != hipSuccess) return ~0u; \
    if (clear) {                                                            \
      const unsigned z = 0;                                                 \
      if (hipMemcpyToSymbol(HIP_SYMBOL(bsa_check_word), &z, sizeof z) != hipSuccess) return ~0u; \
    }                                                                       \
    return v;                                                               \
  }
#else
#define BSA_CHECK(ok, bit) true
#define BSA_CHECK_ACCESSOR(fn) \
  unsigned fn(int) { return 0; }
#endif

__device__ __forceinline__ float bf16_bits_to_f32(u16 h) {
  return __uint_as_float(((unsigned)h) << 16);
}

// Round-to-nearest-even f32 -> bf16 bits (finite inputs).
__device__ __forceinline__ u16 f32_to_bf16_bits(float f) {
  unsigned u = __float_as_uint(f);
  unsigned r = u + 0x7FFFu + ((u >> 16) & 1u);
  return (u16)(r >> 16);
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Wave-wide reductions (all 64 lanes participate).
__device__ __forceinline__ double wave_max_f64(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ int wave_sum_i32(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
// Inclusive prefix sum over lanes 0..63 (lane 0 first).
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t x) {
  int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint64_t y = __shfl_up(x, o, 64);
    if (l >= o) x += y;
  }
  return x;
}
__device__ __forceinline__ int wave_incl_scan_i32(int x) {
  int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (l >= o) x += y;
  }
  return x;
}
