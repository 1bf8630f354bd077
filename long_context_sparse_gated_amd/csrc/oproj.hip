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
// A block of four waves computes a 256 x 256 tile, each wave a 128 x 128
// part as 4 x 4 tiles of v_mfma_f32_32x32x16_bf16 (accumulators in AGPRs,
// one wave per SIMD): per 16-deep step 16 MFMAs from eight 16-byte fragment
// reads.  K advances 32 per stage; stages reach LDS by LDS-DMA into four
// buffers.  One barrier per stage, between its two steps: after it the next
// stage is complete in LDS and the buffer just read is free, so the wave
// issues the DMA four stages ahead into it and reads the next stage's
// fragments while the second step's MFMAs run.
// The DMA is issued from inline asm (it has no register results): the
// kernel counts its completions itself, and the compiler, which then sees
// only the LDS reads, orders those by the LDS counter alone instead of
// draining every DMA in flight before each read.  In LDS a row is 64 bytes
// (four 16-byte chunks) and chunk c of row r sits at slot c ^ ((r >> 2) & 3),
// so that the sixteen rows of a fragment read fill all 64 banks.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

namespace {

typedef __bf16 bf16x8g __attribute__((ext_vector_type(8)));
typedef float f32x16g __attribute__((ext_vector_type(16)));

constexpr int kGM = 256, kGN = 256, kGK = 32;
constexpr int kGRows = 256;  // rows per operand per stage

typedef __attribute__((address_space(3))) void lds_vg;

__device__ __forceinline__ f32x16g mfma32g(uint4 a, uint4 b, f32x16g c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8g, a),
                                                 __builtin_bit_cast(bf16x8g, b), c, 0, 0, 0);
}

}  // namespace

// kRouted: the columns of C go to the outputs of `map` (columns
// map.col0[s] .. map.col0[s + 1] - 1 to map.ptr[s], row stride map.ld[s]);
// one batch only.  Otherwise C with row stride ldc and batch stride sc.
template <bool kRouted>
__global__ void __launch_bounds__(256, 1) gemm_nt_bf16(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, bf16_t* __restrict__ C, int M,
    int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int64_t sa, int64_t sb, int64_t sc,
    GemmOut map) {
  // [stage buffer][operand][row * 4 + slot]
  __shared__ __attribute__((aligned(1024))) uint4 lds[4][2][kGRows * 4];
  // Tile order: consecutive blocks are dealt round-robin to the eight XCDs
  // (each with its own L2), so block L runs on XCD L % 8.  When the tile
  // count is a multiple of 8, XCD c takes tiles c T/8 .. (c+1) T/8 - 1 in
  // order, and tiles are numbered group by group of 8 row tiles (column
  // tile fastest within a group's 8 rows), so the blocks an XCD runs at once
  // cover a compact patch and share their A and B tiles in that L2.
  const int gx = gridDim.x, gy = gridDim.y;
  const int ntile = gx * gy * (int)gridDim.z;
  int t = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  if ((ntile & 7) == 0) t = (t & 7) * (ntile >> 3) + (t >> 3);
  const int tz = t / (gx * gy), tr = t - tz * gx * gy;
  const int g0 = (tr / (8 * gx)) * 8, gh = min(8, gy - g0);
  const int tq = tr - g0 * gx;
  const int ty = g0 + tq % gh, tx = tq / gh;
  const int64_t bz = tz;
  A += bz * sa;
  B += bz * sb;
  C += bz * sc;
  const int m0 = ty * kGM, n0 = tx * kGN;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h32 = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv & 1, wn = wv >> 1;  // the wave's 128 x 128 part of the tile
  const int nk = K / kGK;
  // DMA of one stage: 16 rows of 64 bytes per instruction (lane = 4 row +
  // slot), four instructions per operand per wave; rows past M / N re-read
  // the last row
  const int lr = lane >> 2, slot = lane & 3;
  const bf16_t* pa[4];
  const bf16_t* pb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 16 * (4 * wv + j) + lr;
    pa[j] = A + (int64_t)min(m0 + r, M - 1) * lda + 8 * (slot ^ ((r >> 2) & 3));
    pb[j] = B + (int64_t)min(n0 + r, N - 1) * ldb + 8 * (slot ^ ((r >> 2) & 3));
  }
  const uint32_t lds0 = (uint32_t)(size_t)(lds_vg*)&lds[0][0][0];
  // DMA instruction i (0..7) of stage slot `st` into buffer `buf`: operand
  // i & 1, rows 16 (4 wv + i / 2).  Every stage issues eight instructions,
  // so the count of instructions in flight is the same at every wait; a slot
  // past the last stage re-reads the last stage into a buffer that no wave
  // reads again.
  auto issue1 = [&](int st, int buf, int i) {
    const uint32_t d = lds0 + (uint32_t)buf * (2 * kGRows * 64) + (i & 1) * (kGRows * 64) +
                       (uint32_t)(4 * wv + (i >> 1)) * 1024;
    const bf16_t* src = ((i & 1) ? pb[i >> 1] : pa[i >> 1]) + min(st, nk - 1) * kGK;
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(src), "s"(d)
        : "memory", "m0");
  };
  f32x16g acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mt][nt][v] = 0.f;
  // fragment of tile row r0 + l32 (r0 a multiple of 32), step s: chunk
  // 2 s + h32 at slot (2 s + h32) ^ ((l32 >> 2) & 3)
  const int fsw = (l32 >> 2) & 3;
  const int ra = (128 * wm + l32) * 4, rb = (128 * wn + l32) * 4;
  typedef uint4 frags_t[2][4];
  frags_t fa0, fb0, fa1, fb1;
  auto read_stage = [&](int kt, frags_t& fa, frags_t& fb) {
    const uint4* la = lds[kt & 3][0];
    const uint4* lb = lds[kt & 3][1];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int sl = (2 * s + h32) ^ fsw;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        fa[s][t] = la[ra + 128 * t + sl];
        fb[s][t] = lb[rb + 128 * t + sl];
      }
    }
  };
  auto mfma_step = [&](const frags_t& fa, const frags_t& fb, int s) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma32g(fb[s][nt], fa[s][mt], acc[mt][nt]);
  };
  auto stage = [&](int kt, frags_t& fa, frags_t& fb, frags_t& na, frags_t& nb) {
    mfma_step(fa, fb, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nk) {
      // slots up to kt + 3 were issued: this wave's stage kt + 1 has landed
      // once at most the sixteen instructions of kt + 2 and kt + 3 fly;
      // after the barrier every wave's has, and every wave has read stage
      // kt, so its buffer takes slot kt + 4
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      __builtin_amdgcn_s_barrier();
    }
    // in the last stage no barrier runs and other waves may still read
    // stage kt: its eight instructions then go to buffer (kt + 1) & 3, whose
    // stage was consumed three stages ago
    const int dbuf = (kt + 1 < nk) ? (kt & 3) : ((kt + 1) & 3);
    __builtin_amdgcn_sched_barrier(0);
    // (after the last stage these reads fetch a quiet buffer and are unused)
    const uint4* la = lds[(kt + 1) & 3][0];
    const uint4* lb = lds[(kt + 1) & 3][1];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc[i >> 2][i & 3] = mfma32g(fb[1][i & 3], fa[1][i >> 2], acc[i >> 2][i & 3]);
      const int st = i >> 3, t = (i >> 1) & 3;
      const int sl = (2 * st + h32) ^ fsw;
      if (i & 1)
        nb[st][t] = lb[rb + 128 * t + sl];
      else
        na[st][t] = la[ra + 128 * t + sl];
      if (i & 1) issue1(kt + 4, dbuf, i >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) issue1(j, j, i);
  asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  read_stage(0, fa0, fb0);
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    stage(kt, fa0, fb0, fa1, fb1);
    stage(kt + 1, fa1, fb1, fa0, fb0);
  }
  if (kt < nk) stage(kt, fa0, fb0, fa1, fb1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // Epilogue through LDS, free once every wave is past its last reads.  The
  // MFMAs take the B fragment as their first operand, so tile (mt, nt) holds
  // C^T: register v of lane (l32, h32) is row 32 mt + l32 and column
  // 32 nt + 8 (v / 4) + 4 h32 + v % 4 of the wave's part, four adjacent
  // columns per group of four registers.  Each wave writes its 128 x 128
  // part as bf16 rows of 256 bytes into its own 32 KB, 8 bytes per write,
  // 16-byte chunk k of row r at slot k ^ (r & 15) (the 32 rows of one write
  // spread over the banks); lane l then reads back columns 8 (l mod 16) ..
  // +7 of rows l / 16 + 4 j and stores them, 256 contiguous bytes per 16
  // lanes.  (Stores of the groups of four straight from the registers, 32
  // rows of 16 bytes per instruction, made twice the memory requests and
  // took the latent product of the producer projections from 0.83 to
  // 1.54 ms, its rows being 64 KB apart.)
  __syncthreads();
  char* st = (char*)&lds[0][0][0] + (size_t)wv * 128 * 256;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    char* sr = st + (32 * mt + l32) * 256 + 8 * h32;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(uint2*)(sr + (((4 * nt + i) ^ (l32 & 15)) << 4)) =
            make_uint2(pack_bf16x2(acc[mt][nt][4 * i], acc[mt][nt][4 * i + 1]),
                       pack_bf16x2(acc[mt][nt][4 * i + 2], acc[mt][nt][4 * i + 3]));
  }
  // The lane's columns are the same in every row it stores, so their output
  // is found once, by selects over the map's (uniform) entries: indexing the
  // map by a lane's segment number made the compiler load the entry from
  // memory and wait for it before each store.
  const int rbase = m0 + 128 * wm, c8 = (lane & 15) * 8, col = n0 + 128 * wn + c8;
  bf16_t* cp;
  int64_t cld = ldc;
  int cend = N;  // first column past this output
  if (!kRouted) {
    cp = C + col;
  } else {
    bf16_t* sp = map.ptr[0];
    int64_t sld = map.ld[0];
    int sc0 = map.col0[0];
#pragma unroll
    for (int q = 1; q < kGemmOutMax; ++q) {
      const bool live = q < map.nseg;
      const bool in = live && map.col0[q] <= col;
      sp = in ? map.ptr[q] : sp;
      sld = in ? map.ld[q] : sld;
      sc0 = in ? map.col0[q] : sc0;
      if (live && map.col0[q] > col) cend = min(cend, map.col0[q]);
    }
    cp = sp + (col - sc0);
    cld = sld;
  }
  // eight pieces are read from LDS before any is stored, so that the reads
  // share one latency
#pragma unroll 1
  for (int j0 = 0; j0 < 32; j0 += 8) {
    uint4 vv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = (lane >> 4) + 4 * (j0 + u);
      vv[u] = *(const uint4*)(st + r * 256 + (((lane & 15) ^ (r & 15)) << 4));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = rbase + (lane >> 4) + 4 * (j0 + u);
      if (row >= M || col >= N) continue;
      bf16_t* dst = cp + (int64_t)row * cld;
      if (col + 7 < cend && ((uintptr_t)dst & 15u) == 0) {
        *(uint4*)dst = vv[u];
      } else {
        // edge of the matrix, of an output, or an unaligned row: one value
        // at a time, each routed on its own
        const uint32_t w4[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int ce = col + e;
          if (ce >= N) break;
          bf16_t* de = C + (int64_t)row * ldc + ce;
          if (kRouted) {
            int sg = 0;
            for (int q = 1; q < map.nseg; ++q)
              if (map.col0[q] <= ce) sg = q;
            de = map.ptr[sg] + (int64_t)row * map.ld[sg] + (ce - map.col0[sg]);
          }
          *de = (bf16_t)(w4[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
}

hipError_t launch_gemm_nt(const bf16_t* A, const bf16_t* B, bf16_t* C, int M, int N, int K,
                          int64_t lda, int64_t ldb, int64_t ldc, int64_t sa, int64_t sb,
                          int64_t sc, int batch, hipStream_t s) {
  dim3 grid((N + kGN - 1) / kGN, (M + kGM - 1) / kGM, batch);
  gemm_nt_bf16<false><<<grid, 256, 0, s>>>(A, B, C, M, N, K, lda, ldb, ldc, sa, sb, sc,
                                           GemmOut{});
  return hipGetLastError();
}

hipError_t launch_gemm_nt_routed(const bf16_t* A, const bf16_t* B, int M, int N, int K,
                                 int64_t lda, int64_t ldb, const GemmOut& map, hipStream_t s) {
  dim3 grid((N + kGN - 1) / kGN, (M + kGM - 1) / kGM, 1);
  gemm_nt_bf16<true><<<grid, 256, 0, s>>>(A, B, nullptr, M, N, K, lda, ldb, 0, 0, 0, 0, map);
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
