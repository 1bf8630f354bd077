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
// A block of four waves computes a 256 x 256 tile (or 128 x 512, the waves
// side by side, where a row of 512 columns must stay in one block), each
// wave a 128 x 128 part as 4 x 4 tiles of v_mfma_f32_32x32x16_bf16
// (accumulators in AGPRs, one wave per SIMD): per 16-deep step 16 MFMAs from
// eight 16-byte fragment reads.  K advances 32 per stage; stages reach LDS
// by LDS-DMA into four buffers.  One barrier per stage, between its two
// steps: after it the next
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

constexpr int kGK = 32;  // K per stage

typedef __attribute__((address_space(3))) void lds_vg;

__device__ __forceinline__ f32x16g mfma32g(uint4 a, uint4 b, f32x16g c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8g, a),
                                                 __builtin_bit_cast(bf16x8g, b), c, 0, 0, 0);
}

}  // namespace

// kRouted: the columns of C go to the outputs of `map` (columns
// map.col0[s] .. map.col0[s + 1] - 1 to map.ptr[s], row stride map.ld[s]);
// one batch only.  Otherwise C with row stride ldc and batch stride sc.
// kWide: 128 x 512 tiles, the four waves side by side along N, so that a
// block holds whole rows of 512 columns (a routed output whose rows are
// RMS-normalised per 512 columns gets that norm in the epilogue);
// otherwise 256 x 256 tiles, 2 x 2 waves.
template <bool kRouted, bool kWide>
__global__ void __launch_bounds__(256, 1) gemm_nt_bf16(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, bf16_t* __restrict__ C, int M,
    int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int64_t sa, int64_t sb, int64_t sc,
    GemmOut map) {
  constexpr int TM = kWide ? 128 : 256, TN = kWide ? 512 : 256;
  constexpr int RS = TM + TN;  // rows per stage: the A tile's, then the B tile's
  constexpr int NI = RS / 64;  // DMA instructions per wave per stage (16 rows each)
  // [stage buffer][row * 4 + slot]
  __shared__ __attribute__((aligned(1024))) uint4 lds[4][RS * 4];
  // Tile order: consecutive blocks are dealt round-robin to the eight XCDs
  // (each with its own L2), so block L runs on XCD L % 8.  When the tile
  // count is a multiple of 8, XCD c takes tiles c T/8 .. (c+1) T/8 - 1 in
  // order, and tiles are numbered group by group of GH row tiles (row tile
  // fastest within a group), so the blocks an XCD runs at once cover a
  // compact patch and share their A and B tiles in that L2.  GH = 16 for
  // the wide tiles keeps the patch as tall (2048 rows) as with 256-row
  // tiles: with 8, each XCD of the latent product of the producer
  // projections streamed all of B instead of half (0.98 against 0.84 ms).
  constexpr int GH = kWide ? 16 : 8;
  const int gx = gridDim.x, gy = gridDim.y;
  const int ntile = gx * gy * (int)gridDim.z;
  int t = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  if ((ntile & 7) == 0) t = (t & 7) * (ntile >> 3) + (t >> 3);
  const int tz = t / (gx * gy), tr = t - tz * gx * gy;
  const int g0 = (tr / (GH * gx)) * GH, gh = min(GH, gy - g0);
  const int tq = tr - g0 * gx;
  const int ty = g0 + tq % gh, tx = tq / gh;
  const int64_t bz = tz;
  A += bz * sa;
  B += bz * sb;
  C += bz * sc;
  const int m0 = ty * TM, n0 = tx * TN;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h32 = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the wave's 128 x 128 part of the tile
  const int wm = kWide ? 0 : (wv & 1), wn = kWide ? wv : (wv >> 1);
  const int nk = K / kGK;
  // DMA of one stage: 16 rows of 64 bytes per instruction (lane = 4 row +
  // slot); instruction i of wave wv moves row group g = NI wv + i of the
  // stage's RS rows (A's, then B's); rows past M / N re-read the last row
  const int lr = lane >> 2, slot = lane & 3;
  const bf16_t* src0[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = 16 * (NI * wv + i) + lr;
    const int sw = 8 * (slot ^ ((r >> 2) & 3));  // TM is a multiple of 16
    src0[i] = r < TM ? A + (int64_t)min(m0 + r, M - 1) * lda + sw
                     : B + (int64_t)min(n0 + r - TM, N - 1) * ldb + sw;
  }
  const uint32_t lds0 = (uint32_t)(size_t)(lds_vg*)&lds[0][0];
  // DMA instruction i of stage slot `st` into buffer `buf`.  Every stage
  // issues NI instructions per wave, so the count of instructions in flight
  // is the same at every wait; a slot past the last stage re-reads the last
  // stage into a buffer that no wave reads again.
  auto issue1 = [&](int st, int buf, int i) {
    const uint32_t d = lds0 + (uint32_t)buf * (RS * 64) + (uint32_t)(NI * wv + i) * 1024;
    const bf16_t* src = src0[i] + min(st, nk - 1) * kGK;
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
  const int ra = (128 * wm + l32) * 4, rb = (TM + 128 * wn + l32) * 4;
  typedef uint4 frags_t[2][4];
  frags_t fa0, fb0, fa1, fb1;
  auto read_stage = [&](int kt, frags_t& fa, frags_t& fb) {
    const uint4* l = lds[kt & 3];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int sl = (2 * s + h32) ^ fsw;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        fa[s][t] = l[ra + 128 * t + sl];
        fb[s][t] = l[rb + 128 * t + sl];
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
      // once at most the instructions of kt + 2 and kt + 3 fly; after the
      // barrier every wave's has, and every wave has read stage kt, so its
      // buffer takes slot kt + 4
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NI) : "memory");
      __builtin_amdgcn_s_barrier();
    }
    // in the last stage no barrier runs and other waves may still read
    // stage kt: its instructions then go to buffer (kt + 1) & 3, whose
    // stage was consumed three stages ago
    const int dbuf = (kt + 1 < nk) ? (kt & 3) : ((kt + 1) & 3);
    __builtin_amdgcn_sched_barrier(0);
    // (after the last stage these reads fetch a quiet buffer and are unused)
    const uint4* l = lds[(kt + 1) & 3];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc[i >> 2][i & 3] = mfma32g(fb[1][i & 3], fa[1][i >> 2], acc[i >> 2][i & 3]);
      const int st = i >> 3, t = (i >> 1) & 3;
      const int sl = (2 * st + h32) ^ fsw;
      if (i & 1)
        nb[st][t] = l[rb + 128 * t + sl];
      else
        na[st][t] = l[ra + 128 * t + sl];
      // DMA instructions 0..7 after the odd MFMAs, any further ones after
      // the first even ones
      if (i & 1)
        issue1(kt + 4, dbuf, i >> 1);
      else if (8 + (i >> 1) < NI)
        issue1(kt + 4, dbuf, 8 + (i >> 1));
      __builtin_amdgcn_sched_barrier(0);
    }
  };
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < NI; ++i) issue1(j, j, i);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * NI) : "memory");
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
  char* st = (char*)&lds[0][0] + (size_t)wv * 128 * 256;
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
  // The output holding column c0, by selects over the map's (uniform)
  // entries: indexing the map by a lane's segment number made the compiler
  // load the entry from memory and wait for it before each store.
  struct Out {
    bf16_t* p;
    int64_t ld;
    int end;  // first column past this output
    int seg;
  };
  auto route = [&](int c0) {
    Out o{nullptr, ldc, N, 0};
    if (!kRouted) {
      o.p = C + c0;
    } else {
      bf16_t* sp = map.ptr[0];
      int sc0 = map.col0[0];
      o.ld = map.ld[0];
#pragma unroll
      for (int q = 1; q < kGemmOutMax; ++q) {
        const bool live = q < map.nseg;
        const bool in = live && map.col0[q] <= c0;
        sp = in ? map.ptr[q] : sp;
        o.ld = in ? map.ld[q] : o.ld;
        sc0 = in ? map.col0[q] : sc0;
        o.seg = in ? q : o.seg;
        if (live && map.col0[q] > c0) o.end = min(o.end, map.col0[q]);
      }
      o.p = sp + (c0 - sc0);
    }
    return o;
  };
  if (kWide && kRouted && map.norm_seg1 > 0) {
    // RMS norm over each row's 512 columns [the per-head q_b_norm] on tiles
    // that are whole 512-column groups of the normalised output (the
    // condition is the block's, so its barrier is safe).  Float32 sums and
    // scale, within about 2^-16 of the exact value (relative): a result
    // differs from the float64 form's by one bf16 unit at most, and only
    // next to a rounding boundary.  The float64 form of the separate norm
    // pass cost 0.17 ms here against 0.05.
    const Out on = route(n0);
    const int gc = (int)(on.p - map.ptr[on.seg]);  // n0's column in that output
    if (on.seg + 1 == map.norm_seg1 && n0 + 512 <= on.end && gc % 512 == 0) {
      __syncthreads();  // every wave's part is in LDS
      // wave wv takes tile rows 32 wv .. +31; lane l holds columns
      // 128 (l / 16) + 8 (l mod 16) .. +7 (wave part l / 16, chunk l mod 16)
      const char* part = (const char*)&lds[0][0] + (size_t)(lane >> 4) * 128 * 256;
      bf16_t* op = on.p + 128 * (lane >> 4) + 8 * (lane & 15);
#pragma unroll 1
      for (int j0 = 0; j0 < 32; j0 += 8) {
        uint4 vv[8];
        float ss[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int r = 32 * wv + j0 + u;
          vv[u] = *(const uint4*)(part + r * 256 + (((lane & 15) ^ (r & 15)) << 4));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t w4[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
          ss[u] = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x0 = __uint_as_float(w4[e] << 16);
            const float x1 = __uint_as_float(w4[e] & 0xffff0000u);
            ss[u] = fmaf(x0, x0, fmaf(x1, x1, ss[u]));
          }
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1)
#pragma unroll
          for (int u = 0; u < 8; ++u) ss[u] += __shfl_xor(ss[u], d, 64);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int row = m0 + 32 * wv + j0 + u;
          if (row >= M) continue;
          const float rr = 1.f / sqrtf(ss[u] * (1.f / 512.f) + (float)map.norm_eps);
          const uint32_t w4[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
          uint32_t o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[e] = pack_bf16x2(__uint_as_float(w4[e] << 16) * rr,
                               __uint_as_float(w4[e] & 0xffff0000u) * rr);
          *(uint4*)(op + (int64_t)row * on.ld) = make_uint4(o[0], o[1], o[2], o[3]);
        }
      }
      return;
    }
  }
  // Lane l stores columns 8 (l mod 16) .. +7 of rows l / 16 + 4 j: the same
  // columns in every row, so their output is found once.
  const int rbase = m0 + 128 * wm, c8 = (lane & 15) * 8, col = n0 + 128 * wn + c8;
  const Out oc = route(col);
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
      bf16_t* dst = oc.p + (int64_t)row * oc.ld;
      if (col + 7 < oc.end && ((uintptr_t)dst & 15u) == 0) {
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
  dim3 grid((N + 255) / 256, (M + 255) / 256, batch);
  gemm_nt_bf16<false, false><<<grid, 256, 0, s>>>(A, B, C, M, N, K, lda, ldb, ldc, sa, sb, sc,
                                           GemmOut{});
  return hipGetLastError();
}

hipError_t launch_gemm_nt_routed(const bf16_t* A, const bf16_t* B, int M, int N, int K,
                                 int64_t lda, int64_t ldb, const GemmOut& map, hipStream_t s) {
  if (map.norm_seg1 > 0) {  // 128 x 512 tiles: whole 512-column groups per block
    dim3 grid((N + 511) / 512, (M + 127) / 128, 1);
    gemm_nt_bf16<true, true><<<grid, 256, 0, s>>>(A, B, nullptr, M, N, K, lda, ldb, 0, 0, 0, 0,
                                                  map);
  } else {
    dim3 grid((N + 255) / 256, (M + 255) / 256, 1);
    gemm_nt_bf16<true, false><<<grid, 256, 0, s>>>(A, B, nullptr, M, N, K, lda, ldb, 0, 0, 0, 0,
                                                   map);
  }
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
