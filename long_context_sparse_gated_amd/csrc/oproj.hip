// Grouped low-rank output projection of the attention block, and the bf16
// GEMM it runs on.
//
// The attention output of a token, [H, D] (after the -t rotation), is split
// into o_groups groups of H / o_groups consecutive heads; group g's
// (H / o_groups) * D values go through its own [o_lora_rank, (H / o_groups) * D]
// matrix (o_a_proj, a per-group batched product), the o_groups * o_lora_rank
// results are concatenated and projected to hidden_size by o_b_proj
// [DeepSeek-V4 model page, sec. 2.3 ("Grouped Output Projection": groups of
// heads -> o_lora_rank per group -> hidden_size, o_a_proj then o_b_proj);
// transformers PR 45616 notes (DeepseekV4GroupedLinear: an (out, in) weight,
// forward by per-group bmm)].  The intermediate is stored at bf16 like the
// module output it is.
//
// gemm_nt_bf16: C[b][m, n] = sum_k A[b][m, k] B[b][n, k], all row-major
// with k contiguous in A and B (a weight in (out, in) layout is B as it is),
// bf16 inputs, float32 accumulation, bf16 output rounded to nearest even.
// A block computes a 128 x 256 tile with four waves of 64 x 128 (2 x 4
// tiles of v_mfma_f32_32x32x16_bf16); K advances in 32-wide stages that
// reach LDS by LDS-DMA, three buffers deep (two stages in flight while one
// is multiplied).  In LDS a row is 64 bytes (four 16-byte chunks) and chunk
// c of row r sits at slot c ^ ((r >> 1) & 3), so that the eight rows of a
// 16-byte fragment read hit distinct bank groups.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

namespace {

typedef __bf16 bf16x8g __attribute__((ext_vector_type(8)));
typedef float f32x16g __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_vg;

constexpr int kGM = 128, kGN = 256, kGK = 32, kGStages = 3;
constexpr int kGRowB = kGK * 2;  // bytes per LDS row

__device__ __forceinline__ f32x16g mfma32g(uint4 a, uint4 b, f32x16g c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8g, a),
                                                 __builtin_bit_cast(bf16x8g, b), c, 0, 0, 0);
}

// Four 16-byte LDS reads, waited for in the same block (the compiler then
// sees no LDS load to order after the DMA in flight).
__device__ __forceinline__ void lds_rd4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                        uint4& o0, uint4& o1, uint4& o2, uint4& o3) {
  asm volatile(
      "ds_read_b128 %0, %4\n"
      "ds_read_b128 %1, %5\n"
      "ds_read_b128 %2, %6\n"
      "ds_read_b128 %3, %7\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o0), "=&v"(o1), "=&v"(o2), "=&v"(o3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}

}  // namespace

__global__ void __launch_bounds__(256, 2) gemm_nt_bf16(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, bf16_t* __restrict__ C, int M,
    int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int64_t sa, int64_t sb, int64_t sc) {
  __shared__ __attribute__((aligned(1024))) bf16_t As[kGStages][kGM * kGK];
  __shared__ __attribute__((aligned(1024))) bf16_t Bs[kGStages][kGN * kGK];
  const int64_t bz = blockIdx.z;
  A += bz * sa;
  B += bz * sb;
  C += bz * sc;
  const int m0 = blockIdx.y * kGM, n0 = blockIdx.x * kGN;
  const int lane = threadIdx.x & 63, l32 = lane & 31, h32 = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wv & 1, wn = wv >> 1;  // the wave's 64 x 128 part of the tile
  const int nk = K / kGK;
  // DMA of one stage: 16 rows of 64 bytes per instruction (lane = 4 row +
  // slot); A: 2 instructions per wave, B: 4; rows past M / N re-read the last
  const int lr = lane >> 2, slot = lane & 3;
  auto issue = [&](int kt, int buf) {
    const int k0 = kt * kGK;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 16 * (2 * wv + j) + lr;
      const int row = min(m0 + r, M - 1);
      const bf16_t* src = A + (int64_t)row * lda + k0 + 8 * (slot ^ ((r >> 1) & 3));
      __builtin_amdgcn_global_load_lds((const void*)src,
                                       (lds_vg*)(&As[buf][16 * (2 * wv + j) * kGK]), 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * (4 * wv + j) + lr;
      const int row = min(n0 + r, N - 1);
      const bf16_t* src = B + (int64_t)row * ldb + k0 + 8 * (slot ^ ((r >> 1) & 3));
      __builtin_amdgcn_global_load_lds((const void*)src,
                                       (lds_vg*)(&Bs[buf][16 * (4 * wv + j) * kGK]), 16, 0, 0);
    }
  };
  f32x16g acc[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mt][nt][v] = 0.f;
  // fragment of row r (tile-relative), 16-deep step s: chunk 2 s + h32
  auto faddr = [&](const bf16_t* base, int r, int s) {
    return (uint32_t)(size_t)(lds_vg*)base +
           (uint32_t)(r * kGRowB + 16 * ((2 * s + h32) ^ ((r >> 1) & 3)));
  };
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's DMA of stage kt is done once at most the next stage's six
    // instructions are outstanding (none after the last issue)
    if (kt + 1 < nk)
      asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    // after the barrier every wave is past stage kt - 1: its buffer is free
    if (kt + 2 < nk) issue(kt + 2, (kt + 2) % kGStages);
    const int buf = kt % kGStages;
    const bf16_t* as = As[buf];
    const bf16_t* bs = Bs[buf];
    uint4 af[2][2], bf[4][2];
    const int ra = 64 * wm + l32, rb = 128 * wn + l32;
    lds_rd4(faddr(as, ra, 0), faddr(as, ra, 1), faddr(as, ra + 32, 0), faddr(as, ra + 32, 1),
            af[0][0], af[0][1], af[1][0], af[1][1]);
    lds_rd4(faddr(bs, rb, 0), faddr(bs, rb, 1), faddr(bs, rb + 32, 0), faddr(bs, rb + 32, 1),
            bf[0][0], bf[0][1], bf[1][0], bf[1][1]);
    lds_rd4(faddr(bs, rb + 64, 0), faddr(bs, rb + 64, 1), faddr(bs, rb + 96, 0),
            faddr(bs, rb + 96, 1), bf[2][0], bf[2][1], bf[3][0], bf[3][1]);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma32g(af[mt][s], bf[nt][s], acc[mt][nt]);
  }
  // register v of tile (mt, nt): row 8 (v / 4) + 4 h32 + v % 4, column l32
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int col = n0 + 128 * wn + 32 * nt + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + 64 * wm + 32 * mt + 8 * (v / 4) + 4 * h32 + v % 4;
        if (row < M && col < N) C[(int64_t)row * ldc + col] = f32_to_bf16(acc[mt][nt][v]);
      }
    }
}

hipError_t launch_gemm_nt(const bf16_t* A, const bf16_t* B, bf16_t* C, int M, int N, int K,
                          int64_t lda, int64_t ldb, int64_t ldc, int64_t sa, int64_t sb,
                          int64_t sc, int batch, hipStream_t s) {
  dim3 grid((N + kGN - 1) / kGN, (M + kGM - 1) / kGM, batch);
  gemm_nt_bf16<<<grid, 256, 0, s>>>(A, B, C, M, N, K, lda, ldb, ldc, sa, sb, sc);
  return hipGetLastError();
}

hipError_t launch_output_projection(int T, int H, int D, int G, int R, int hidden,
                                    const bf16_t* x, const bf16_t* wa, const bf16_t* wb,
                                    bf16_t* y1, bf16_t* out, hipStream_t s) {
  const int Ig = (H / G) * D;  // inputs per group
  // y1[t, g, :] = wa[g] x[t, g, :]: batch over groups, rows of x strided by H D
  hipError_t e = launch_gemm_nt(x, wa, y1, T, R, Ig, (int64_t)H * D, Ig, (int64_t)G * R, Ig,
                                (int64_t)R * Ig, R, G, s);
  if (e != hipSuccess) return e;
  // out[t, :] = wb y1[t, :]
  return launch_gemm_nt(y1, wb, out, T, hidden, G * R, (int64_t)G * R, (int64_t)G * R, hidden, 0,
                        0, 0, 1, s);
}

}  // namespace csa
