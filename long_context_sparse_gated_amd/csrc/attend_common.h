// Shared pieces of the attention kernels (H = 64, D = 512, bf16 fast paths):
// MFMA and lane-swap wrappers, the row-id encoding of the row list and the LDS
// chunk swizzle.
#pragma once

#include "csa_device.h"

namespace csa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

constexpr int kMaxRope = 128;    // rope channels supported by the fast path
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;    // log2 headroom before the running max is raised
// Tuning (compile time): the blocks per CU the register budget targets.
#ifndef CSA_ATTN_MIN_BLOCKS
#define CSA_ATTN_MIN_BLOCKS 2
#endif

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;

// Reductions across lane l and l ^ 16 / l ^ 32 with the gfx950 lane-swap
// instructions (no LDS round trip); the max / sum of the two swapped values
// pairs every lane with its partner whichever half moves.
__device__ __forceinline__ float xmax16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xmax32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xsum16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xsum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row id encoding in LDS: >= 0 window ring row, <= -2 pool row -(id+2), -1 none.
// Pool rows are those of the pool tensor (through the block table when the
// pools are paged).
__device__ __forceinline__ int row_id(int jr, int nwin, int64_t lo, int64_t win_cap, int b,
                                      int64_t pool_cap, const int32_t* idx_row, int csa,
                                      int64_t nvis, const Seqs& sq) {
  if (jr < nwin) return (int)((int64_t)b * win_cap + (lo + jr) % win_cap);
  const int e = jr - nwin;
  const int64_t w = csa ? (int64_t)idx_row[e] : (int64_t)e;
  if (w < 0 || w >= nvis) return -1;
  return (int)(-2 - sq.prow(b, w, pool_cap));
}

// Chunk swizzle of LDS row r (16-byte chunks, 64 per row; only the low four
// chunk bits move): the 16 rows of a QK^T read get 16 distinct chunk slots.
// Measured on gfx950 with the read patterns of this kernel: 16-byte reads
// run at the contiguous rate with this swizzle (about 300+ bytes/clk/CU,
// against about 120 with no swizzle); the transpose reads run at about 115
// bytes/clk/CU with any of the swizzles tried.
__device__ __forceinline__ int swz(int r) { return r & 15; }

// LDS accesses kept out of the compiler's sight.  While LDS-DMA loads are in
// flight the compiler makes every LDS access it cannot prove disjoint from
// an array some DMA writes (the small control arrays here never are DMA
// targets) wait for all of them, and __syncthreads() also waits for all
// outstanding global loads: either would drain the next chunk's row gather
// in the middle of a chunk.  Loads wait for their own data inside the asm
// block (outputs early-clobbered, so no output shares a register with an
// address still to be used).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const lds_void*)p;
}
__device__ __forceinline__ void lds_st128(void* p, uint4 v) {
  const u32x4 x = __builtin_bit_cast(u32x4, v);
  asm volatile("ds_write_b128 %0, %1" ::"v"(lds_addr(p)), "v"(x) : "memory");
}
__device__ __forceinline__ void lds_st32(void* p, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
// This wave's LDS writes complete, then the workgroup barrier; global loads
// (the row gathers) stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Four 16-byte loads at a + i*SA and four 4-byte loads at b + i*SB (byte
// strides, immediate offsets), complete on return.
template <int SA, int SB>
__device__ __forceinline__ void lds_ld_4x128_4x32(const void* a, const void* b, uint4 (&o)[4],
                                                  uint32_t (&w)[4]) {
  static_assert(3 * SA < 65536 && 3 * SB < 65536, "immediate LDS offsets are 16-bit");
  u32x4 x0, x1, x2, x3;
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:%10\n\t"
      "ds_read_b128 %2, %8 offset:%11\n\t"
      "ds_read_b128 %3, %8 offset:%12\n\t"
      "ds_read_b32 %4, %9\n\t"
      "ds_read_b32 %5, %9 offset:%13\n\t"
      "ds_read_b32 %6, %9 offset:%14\n\t"
      "ds_read_b32 %7, %9 offset:%15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3), "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]),
        "=&v"(w[3])
      : "v"(lds_addr(a)), "v"(lds_addr(b)), "i"(SA), "i"(2 * SA), "i"(3 * SA), "i"(SB),
        "i"(2 * SB), "i"(3 * SB)
      : "memory");
  o[0] = __builtin_bit_cast(uint4, x0);
  o[1] = __builtin_bit_cast(uint4, x1);
  o[2] = __builtin_bit_cast(uint4, x2);
  o[3] = __builtin_bit_cast(uint4, x3);
}

__device__ __forceinline__ void lds_st64(void* p, uint32_t a, uint32_t b) {
  asm volatile("ds_write_b64 %0, %1" ::"v"(lds_addr(p)), "v"((uint64_t)a | ((uint64_t)b << 32))
               : "memory");
}
__device__ __forceinline__ uint32_t lds_ld32(const void* p) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}
// Eight 16-byte loads at a + i*SA + j*SB (i < 2, j < 4) and two 4-byte loads at
// b and b + SC (byte offsets), complete on return.
template <int SA, int SB, int SC>
__device__ __forceinline__ void lds_ld_8x128_2x32(const void* a, const void* b, uint4 (&o)[2][4],
                                                  uint32_t (&w)[2]) {
  static_assert(SA + 3 * SB < 65536 && SC < 65536, "immediate LDS offsets are 16-bit");
  u32x4 x[8];
  asm volatile(
      "ds_read_b128 %0, %10\n\t"
      "ds_read_b128 %1, %10 offset:%13\n\t"
      "ds_read_b128 %2, %10 offset:%14\n\t"
      "ds_read_b128 %3, %10 offset:%15\n\t"
      "ds_read_b128 %4, %10 offset:%12\n\t"
      "ds_read_b128 %5, %10 offset:%16\n\t"
      "ds_read_b128 %6, %10 offset:%17\n\t"
      "ds_read_b128 %7, %10 offset:%18\n\t"
      "ds_read_b32 %8, %11\n\t"
      "ds_read_b32 %9, %11 offset:%19\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
        "=&v"(x[6]), "=&v"(x[7]), "=&v"(w[0]), "=&v"(w[1])
      : "v"(lds_addr(a)), "v"(lds_addr(b)), "i"(SA), "i"(SB), "i"(2 * SB), "i"(3 * SB),
        "i"(SA + SB), "i"(SA + 2 * SB), "i"(SA + 3 * SB), "i"(SC)
      : "memory");
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o[0][j] = __builtin_bit_cast(uint4, x[j]);
    o[1][j] = __builtin_bit_cast(uint4, x[4 + j]);
  }
}

}  // namespace csa
