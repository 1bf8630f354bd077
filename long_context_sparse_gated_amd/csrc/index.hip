// Lightning Indexer scores and per-query top-k block selection (CSA layers).
//
// score(t, w) = sum_h wt[t,h] * ReLU(rot_t(q[t,h]) . k[w]) over the visible
// entries w < (t+1)/m; the k best (score descending, entry id ascending) are
// emitted in ascending id order, padded with -1 [DeepSeek-V4 model page,
// sec. 2.3 (the indexer scores queries against the pool and gathers the top
// index_topk blocks per query) and "Attention mask layout" (the -1 sentinel);
// TransformerLens adapter, indexer submodules q_b_proj, scorer.weights_proj,
// rotary_emb].
//
// Kernels:
//  * index_prefill_mfma: H_I = 64, D_I = 128, bf16, rope widths other than
//    64.  A block takes 8 consecutive queries (2 per wave, rotated query
//    fragments held in VGPRs) and streams the visible keys through LDS in
//    tiles of 64 keys shared by the four waves: 64 x 16 x 32 bf16 MFMA tiles,
//    then ReLU, head weights and the head sum in registers (16 heads in-lane,
//    4 lane groups by shuffles).
//  * index_decode_x32 (few queries per sequence): queries rotated once
//    (rotate_queries_bf16), then each block streams a run of one query's keys
//    from HBM through LDS (LDS-DMA, two tiles in flight per wave) into MFMA
//    fragments; each key is read once.  It also counts the query's scores in
//    a histogram of the top 12 bits of their order keys.
//  * topk_block (decode rows of at most 32768 keys): one block per query
//    selects with the histogram's cut bin and a radix select inside it.
//  * topk_collect / topk_final (decode rows beyond that): the histogram names
//    the bin holding the k-th best score; per 1024-key slice the ids above
//    that bin and inside it are compacted in id order; a radix select inside
//    the bin settles the last places and both id lists are merged in id order.
//  * index_prefill_x32 (H_I = 64, D_I = 128, rope width 64, bf16): one query
//    per wave on 32 x 32 x 16 MFMA tiles, 128-key LDS tiles shared by the
//    block's four waves; see its comment below.
//  * index_generic: any head count / width, float or bf16, VALU float32.
//  * topk_radix (prefill path): per query, four 8-bit radix-select passes
//    find the k-th largest ordered key; one ordered pass emits ids by ballot
//    prefix counts.
#include <cstdlib>

#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Rotate the rope pairs among 8 consecutive bf16 channels d0..d0+7 (packed in
// a uint4) in float64 and round back; cs[j] = (cos, sin) of pair j.
__device__ __forceinline__ uint4 rope8_bf16(uint4 v, int d0, int width, int R,
                                            const double2* cs) {
  const int first = width - R;
  if (d0 + 8 <= first) return v;
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int d = d0 + 2 * p;
    if (d >= first) {
      double a = bf16_to_f32((bf16_t)(w[p] & 0xffffu));
      double b = bf16_to_f32((bf16_t)(w[p] >> 16));
      const double2 c = cs[(d - first) >> 1];
      rot64(a, b, c.x, c.y);
      w[p] = (uint32_t)f64_to_bf16(a) | ((uint32_t)f64_to_bf16(b) << 16);
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// The same rotation with a float32 fast path, for 8 channels that are all
// rope channels; c[p] holds the float32 images (ch, sh) of the float64 (cos,
// sin) of pair p.  With S = |a| + |b|, x1 = fma(a, ch, -(b sh)) differs from
// a cos - b sin by at most 2^-24 (|a| + 2|b| + |x1|) (1 + 2^-23) < 3.01 2^-24 S
// (the cos/sin roundings, the rounded product and the fma), and the same
// bound holds for y1 = fma(a, sh, b ch) against a sin + b cos.  The float64
// evaluation is that close to the exact value too, so both round to the same
// bf16 unless a rounding boundary (a bf16 midpoint) lies within e = 2^-22 S
// of x1, or e is not below a quarter of x1's bf16 spacing (|x1| <= 1024 e);
// a floor of 2^-120 on e covers float32 underflow.  A lane meeting either
// case for any value redoes its 8 channels in float64 (rope8_bf16), so the
// result is always that of the float64 path.
__device__ __forceinline__ bool near_bf16_mid(float v, float e) {
  const float mid = __uint_as_float((__float_as_uint(v) & 0xffff0000u) | 0x8000u);
  return fabsf(v - mid) <= e;  // exact difference: same binade
}

__device__ __forceinline__ uint4 rope4_fast(uint4 v, const float2 (&c)[4], int d0, int width,
                                            int R, const double2* cs) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  bool hard = false;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float a = __uint_as_float(w[p] << 16), b = __uint_as_float(w[p] & 0xffff0000u);
    const float x = fmaf(a, c[p].x, -(b * c[p].y));
    const float y = fmaf(a, c[p].y, b * c[p].x);
    const float S = fabsf(a) + fabsf(b);
    const float e = fmaxf(S * 0x1p-22f, 0x1p-120f), e10 = e * 1024.f;
    const bool h = (int)near_bf16_mid(x, e) | (int)near_bf16_mid(y, e) |
                   (int)(fminf(fabsf(x), fabsf(y)) <= e10);
    hard = hard | (h & (S != 0.f));
    w[p] = pack_bf16x2(x, y);
  }
  if (hard) return rope8_bf16(v, d0, width, R, cs);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------------------
// prefill: 8 queries per block, keys through LDS

constexpr int kIdxKT = 64;    // keys per LDS tile
constexpr int kIdxRow = 136;  // LDS row stride in bf16 (128 + 8 pad)

__global__ void __launch_bounds__(256) index_prefill_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ wts, const bf16_t* __restrict__ keys,
    float* __restrict__ scores, Seqs sq, int Ri, Rope base, int m, int64_t pool_cap) {
  constexpr int Hi = 64, Di = 128;
  __shared__ __attribute__((aligned(16))) bf16_t ktile[2][kIdxKT * kIdxRow];
  __shared__ double2 cs[kIdxQPB][64];
  __shared__ float wsh[kIdxQPB][Hi];
  const int b = blockIdx.y, i0 = blockIdx.x * kIdxQPB;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int64_t p0 = sq.pos0[b];
  const int nq = min(kIdxQPB, sq.len(b) - i0);
  if (nq <= 0) return;  // padding rows only (block-uniform, before any barrier)
  for (int e = tid; e < kIdxQPB * (Ri / 2); e += 256) {
    const int qq = e / (Ri / 2), j = e % (Ri / 2);
    double sn, c;
    sincos((double)(p0 + i0 + qq) * rope_freq(base, j, Ri), &sn, &c);
    cs[qq][j] = make_double2(c, sn);
  }
  for (int e = tid; e < kIdxQPB * Hi; e += 256) {
    const int qq = e / Hi, h = e % Hi;
    wsh[qq][h] = qq < nq ? bf16_to_f32(wts[sq.row(b, i0 + qq) * Hi + h]) : 0.f;
  }
  __syncthreads();

  // visible keys of the block's last query bound the loop
  int64_t nv_last = (p0 + i0 + nq) / m;
  if (nv_last > pool_cap) nv_last = pool_cap;
  const int nkeys = (int)nv_last;

  uint4 A[2][4][4];
  float wr[2][4][4];
  int nvis[2];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int ql = 2 * wv + qq;
    int64_t nv = (p0 + i0 + ql + 1) / m;
    nvis[qq] = ql < nq ? (int)(nv < pool_cap ? nv : pool_cap) : 0;
    const bf16_t* qrow = q + sq.row(b, i0 + (ql < nq ? ql : 0)) * Hi * Di;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int d0 = 32 * kk + 8 * g;
        uint4 v = *(const uint4*)(qrow + (16 * mt + r16) * Di + d0);
        if (ql >= nq) v = make_uint4(0, 0, 0, 0);
        A[qq][mt][kk] = rope8_bf16(v, d0, Di, Ri, cs[ql]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) wr[qq][mt][i] = wsh[ql][16 * mt + 4 * g + i];
    }
  }

  float* srow0 = scores + ((int64_t)b * sq.n + i0 + 2 * wv) * pool_cap;
  for (int kt = 0, it = 0; kt < nkeys; kt += kIdxKT, ++it) {
    bf16_t* tile = ktile[it & 1];
    // a 64-key tile never straddles a pool block (blocks hold a multiple of 128)
    const int64_t kt_row = sq.prow(b, kt, pool_cap);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = tid + 256 * r, key = c >> 4, part = c & 15;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kt + key < nkeys) v = *(const uint4*)(keys + (kt_row + key) * Di + part * 8);
      *(uint4*)(tile + key * kIdxRow + part * 8) = v;
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      uint4 B[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        B[kk] = *(const uint4*)(tile + (16 * nt + r16) * kIdxRow + 32 * kk + 8 * g);
      const int key = kt + 16 * nt + r16;
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        f32x4 acc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma16(A[qq][mt][kk], B[kk], acc[mt]);
        float v = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) v += wr[qq][mt][i] * fmaxf(acc[mt][i], 0.f);
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        if (g == 0 && key < nvis[qq]) srow0[(int64_t)qq * pool_cap + key] = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// prefill on 32 x 32 x 16 MFMA tiles: one query per wave, four per block
//
// For one query the scores of 32 keys come from a 64 x 32 product (heads x
// keys) over 128 channels: two 32 x 32 output tiles of eight 16-deep steps.
// A wave keeps its query's rotated fragments (64 VGPRs, heads as rows) and
// the weights of the heads its lanes receive; the four waves of a block share
// 128-key tiles that reach LDS through LDS-DMA, two buffers deep, and each
// tile is scored in four 32-key steps.  In a 32 x 32 result each lane holds
// 16 heads of one key, so ReLU, weights and the sum over them stay in-lane;
// one lane-half swap then adds the other 16 heads and packs two steps so that
// lane l holds key l of the pair.  The query itself arrives by whole-row DMA
// through the tile buffers (coalesced, unlike fragment-shaped global loads)
// and is rotated with the float32 fast path.  Blocks take the longest query
// groups first.  Rope width 64 only (a template parameter; other widths use
// index_prefill_mfma).

constexpr int kX32Q = 4;     // queries per block, one per wave
constexpr int kX32KT = 128;  // keys per LDS tile (32 KB): four 32-key steps

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// max(x, 0) for a finite float (-0 -> +0) by its bits: a single integer max.
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Eight 16-byte LDS reads at a[i] + OFF, waited for in the same block (the
// compiler then sees no LDS load to order after the DMA in flight).
template <int OFF>
__device__ __forceinline__ void lds_frag8(const uint32_t (&a)[8], uint4 (&o)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:%16\n"
      "ds_read_b128 %1, %9 offset:%16\n"
      "ds_read_b128 %2, %10 offset:%16\n"
      "ds_read_b128 %3, %11 offset:%16\n"
      "ds_read_b128 %4, %12 offset:%16\n"
      "ds_read_b128 %5, %13 offset:%16\n"
      "ds_read_b128 %6, %14 offset:%16\n"
      "ds_read_b128 %7, %15 offset:%16\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
        "=&v"(o[6]), "=&v"(o[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
        "n"(OFF)
      : "memory");
}

template <int RI>
__global__ void __launch_bounds__(256, 2) index_prefill_x32(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ wts, const bf16_t* __restrict__ keys,
    float* __restrict__ scores, float* __restrict__ discard, Seqs sq, int B, Rope base, int m,
    int64_t pool_cap) {
  constexpr int Hi = 64, Di = 128, kFirst = Di - RI, kK0 = kFirst / 16;
  static_assert(RI > 0 && RI <= Di && RI % 16 == 0, "rope channels: whole 16-channel steps");
  __shared__ __attribute__((aligned(1024))) bf16_t kt0[kX32KT * Di];
  __shared__ __attribute__((aligned(1024))) bf16_t kt1[kX32KT * Di];
  __shared__ double2 cs[kX32Q][RI / 2];
  __shared__ float2 csf[kX32Q][RI / 2];
  __shared__ float wsh[kX32Q][Hi];
  const int nblk = (sq.n + kX32Q - 1) / kX32Q;
  const int b = blockIdx.x % B, i0 = (nblk - 1 - (int)(blockIdx.x / B)) * kX32Q;
  const int tid = threadIdx.x, lane = tid & 63, h32 = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t p0 = sq.pos0[b];
  // padding queries (a suffix of the sequence's rows) are not scored; a block
  // whose first query is padding has no other
  const int nq = min(kX32Q, sq.len(b) - i0);
  if (nq <= 0) return;  // block-uniform
  int64_t nv_last = (p0 + i0 + nq) / m;  // the block's last query sees the most keys
  if (nv_last > pool_cap) nv_last = pool_cap;
  const int nkeys = (int)nv_last;
  if (nkeys == 0) return;  // block-uniform
  const int ntile = (nkeys + kX32KT - 1) / kX32KT;

  // DMA of this wave's 32 rows of a tile (8 instructions of 4 rows); chunk c
  // of row r sits at slot c ^ (r & 15); rows past the keys re-read the last.
  // A 128-key tile lies in one pool block (blocks hold a multiple of 128
  // entries): trow is the pool row of its first key.
  const int lrow = lane >> 4, slot = lane & 15;
  auto tile_row = [&](int tile) { return sq.prow(b, (int64_t)tile * kX32KT, pool_cap); };
  auto issue = [&](int tile, bf16_t* dst, int64_t trow) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 32 * wv + 4 * j + lrow;
      const int key = min(tile * kX32KT + r, nkeys - 1) - tile * kX32KT;
      const bf16_t* src = keys + (trow + key) * Di + 8 * (slot ^ ((4 * j + lrow) & 15));
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(dst + (32 * wv + 4 * j) * Di),
                                       16, 0, 0);
    }
  };
  const int ql = wv < nq ? wv : 0;
  int64_t nv = (p0 + i0 + wv + 1) / m;
  if (nv > pool_cap) nv = pool_cap;
  const int nvis = wv < nq ? (int)nv : 0;
  const bf16_t* qrow = q + sq.row(b, i0 + ql) * Hi * Di;
  const bf16_t wt_raw = wts[sq.row(b, i0 + min(tid / Hi, nq - 1)) * Hi + tid % Hi];
  int64_t trow = tile_row(0);
  // The query reaches registers through LDS: head rows 0-31 go to this
  // wave's 32 rows of kt0, rows 32-63 to its rows of kt1 (whole-row DMA in
  // the keys' layout), and are read back as A fragments like the keys.  The
  // wave's own DMA of key tile 0 then refills its rows of kt0; kt1 is free
  // until tile 1, which is issued after a barrier.
  auto issue_q = [&](int mt, bf16_t* dst) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 4 * j + lrow;
      const bf16_t* src = qrow + (32 * mt + r) * Di + 8 * (slot ^ (r & 15));
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(dst + (32 * wv + 4 * j) * Di),
                                       16, 0, 0);
    }
  };
  // lane address of step kk = 0 in a 32-row block of the keys' layout; step
  // kk adds nothing but an XOR of 32 kk (bits 5-7)
  auto frag_addr = [&](const bf16_t* rows, uint32_t (&a)[8]) {
    int ln;  // opaque copy: keeps the per-lane addresses out of loop-invariant registers
    asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
    const int l = ln & 31, h = ln >> 5;
    const uint32_t a0 = (uint32_t)(size_t)(lds_void*)rows +
                        (uint32_t)(l * Di * 2 + 16 * (h ^ (l & 1)) + 32 * ((l >> 1) & 7));
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) a[kk] = a0 ^ (32u * kk);
  };
  issue_q(0, kt0);
  issue_q(1, kt1);  // both overlap the tables
  for (int e = tid; e < kX32Q * (RI / 2); e += 256) {
    const int qq = e / (RI / 2), j = e % (RI / 2);
    double sn, c;
    sincos((double)(p0 + i0 + qq) * rope_freq(base, j, RI), &sn, &c);
    cs[qq][j] = make_double2(c, sn);
    csf[qq][j] = make_float2((float)c, (float)sn);
  }
  wsh[tid / Hi][tid % Hi] = tid / Hi < nq ? bf16_to_f32(wt_raw) : 0.f;
  __syncthreads();  // the tables are written
  uint4 A[2][8];  // this wave's query, head 32 mt + l32, channels 16 kk + 8 h32 .. + 7
  float wr[2][16];
  // (cos, sin) of the lane's rope pairs, read before the key DMA (LDS reads
  // after it would wait for it)
  float2 c[8 - kK0][4];
#pragma unroll
  for (int kk = kK0; kk < 8; ++kk)
#pragma unroll
    for (int p = 0; p < 4; ++p) c[kk - kK0][p] = csf[ql][8 * kk + 4 * h32 + p - kFirst / 2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) wr[mt][r] = wsh[ql][32 * mt + 8 * (r / 4) + 4 * h32 + r % 4];
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's query rows landed
  {
    uint32_t a[8];
    frag_addr(kt0 + 32 * wv * Di, a);
    lds_frag8<0>(a, A[0]);
    frag_addr(kt1 + 32 * wv * Di, a);
    lds_frag8<0>(a, A[1]);
  }
  issue(0, kt0, trow);  // this wave's rows only: its own staging reads are done
  trow = tile_row(ntile > 1 ? 1 : 0);  // the next tile's pool row, loaded ahead of its issue
  if (wv < nq) {  // waves past the last query score nothing that is kept
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int kk = kK0; kk < 8; ++kk)
        A[mt][kk] = rope4_fast(A[mt][kk], c[kk - kK0], 16 * kk + 8 * h32, Di, RI, cs[wv]);
  }

  // The B fragment of step kk for the 32 keys of step st: row 32 st + l32,
  // channels 16 kk + 8 h32, i.e. chunk 2 kk + h32 at slot (2 kk + h32) ^ (l32 & 15):
  // byte offset (row base) + 16 (h32 ^ (l32 & 1)) + 32 (kk ^ ((l32 >> 1) & 7)),
  // an XOR of 32 kk into the lane's kk = 0 offset.
  float* srow = scores + ((int64_t)b * sq.n + i0 + ql) * pool_cap;
  auto step = [&](uint4 (&Bf)[8]) {
    f32x16 acc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) acc[mt] = mfma32(A[mt][kk], Bf[kk], acc[mt]);
    float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r & 3] += wr[mt][r] * relu_bits(acc[mt][r]);
    return (p[0] + p[1]) + (p[2] + p[3]);
  };
  // lanes 0-31: keys 0-31 of the pair of steps, lanes 32-63: keys 32-63;
  // every path stores (the loop's wait counts the stores)
  auto store = [&](int key0, float v0, float v1) {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v1), false,
                                               false);
    const float sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const int key = key0 + lane;
    *(key < nvis ? srow + key : discard + lane) = sc;
  };
  auto compute = [&](int tile, const bf16_t* kt) {
    uint32_t a[8];
    frag_addr(kt, a);
    const int k0 = tile * kX32KT;
    uint4 Bf[8];
    lds_frag8<0>(a, Bf);
    const float v0 = step(Bf);
    lds_frag8<32 * Di * 2>(a, Bf);
    const float v1 = step(Bf);
    store(k0, v0, v1);
    float v2 = 0.f, v3 = 0.f;
    if (k0 + 64 < nkeys) {  // block-uniform: skip the steps past the keys
      lds_frag8<64 * Di * 2>(a, Bf);
      v2 = step(Bf);
      lds_frag8<96 * Di * 2>(a, Bf);
      v3 = step(Bf);
    }
    store(k0 + 64, v2, v3);
  };
  // Tile t is in kt0 for even t, kt1 for odd t.  At the top of each tile
  // this wave's DMA of it is done once at most two later VMEM operations (the
  // previous tile's two score stores) are outstanding; the barrier then
  // publishes every wave's rows and retires every read of the other array.
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  for (int tile = 0;;) {
    if (tile + 1 < ntile) {
      issue(tile + 1, kt1, trow);
      trow = tile_row(tile + 2 < ntile ? tile + 2 : tile + 1);
    }
    compute(tile, kt0);
    if (++tile >= ntile) break;
    asm volatile("s_waitcnt vmcnt(2)\n\ts_barrier" ::: "memory");
    if (tile + 1 < ntile) {
      issue(tile + 1, kt0, trow);
      trow = tile_row(tile + 2 < ntile ? tile + 2 : tile + 1);
    }
    compute(tile, kt1);
    if (++tile >= ntile) break;
    asm volatile("s_waitcnt vmcnt(2)\n\ts_barrier" ::: "memory");
  }
}

// ---------------------------------------------------------------------------
// decode: rotate queries once, then stream keys from HBM into MFMA fragments
//
// Selection of the k best among up to millions of visible keys runs in three
// steps spread over the whole chip: the scoring kernel also counts each
// token's scores in a histogram of the top kHBits bits of their order keys;
// topk_collect finds from the histogram the bin holding the k-th best score
// and compacts, per 1024-key slice, the ids of the keys above that bin and of
// those inside it; topk_final settles the bin by radix select over the few
// keys in it and merges both id lists in ascending order.

constexpr int kHShift = 32 - kHBits;

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) u = 0u;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One count into bins[bin] for every active lane with `add`.  When all the
// adding lanes of the wave name the same bin (ties: every key equal, as with
// all-zero scores) a single atomic adds their number; otherwise each lane
// adds its own.  One LDS address hit by a whole row of equal keys otherwise
// serialises tens of thousands of atomics.
__device__ __forceinline__ void bin_add(uint32_t* bins, bool add, uint32_t bin) {
  const unsigned long long am = __ballot(add);
  if (am == 0ull) return;
  const int first = __ffsll((long long)am) - 1;
  const uint32_t fb = (uint32_t)__shfl((int)bin, first, 64);
  if (__ballot(add && bin == fb) == am) {
    if ((int)(threadIdx.x & 63) == first) atomicAdd(&bins[fb], (uint32_t)__popcll(am));
  } else if (add) {
    atomicAdd(&bins[bin], 1u);
  }
}

__global__ void __launch_bounds__(1024) rotate_queries_bf16(const bf16_t* __restrict__ q,
                                                           bf16_t* __restrict__ qr,
                                                           uint32_t* __restrict__ hist, Seqs sq,
                                                           int Hi, int Di, int Ri, Rope base) {
  __shared__ double2 cs[128];
  const int i = blockIdx.x, b = blockIdx.y;
  if (i >= sq.len(b)) return;  // padding slot: no query
  const int64_t t = sq.pos0[b] + i;
  const int64_t tok = (int64_t)b * sq.n + i;  // the query's slot in the workspace
  const int64_t off = tok * Hi * Di, qoff = sq.row(b, i) * Hi * Di;
  const int chunks = Hi * Di / 8;
  // the thread's first chunk is loaded before the rope table is computed, so
  // that the two overlap (with 1024 threads and 64 x 128 channels, the only
  // chunk)
  const int e0 = threadIdx.x;
  uint4 v0 = make_uint4(0, 0, 0, 0);
  if (e0 < chunks) v0 = *(const uint4*)(q + qoff + (int64_t)e0 * 8);
  for (int j = threadIdx.x; j < kHBins; j += blockDim.x) hist[tok * kHBins + j] = 0u;
  for (int j = threadIdx.x; j < Ri / 2; j += blockDim.x) {
    double sn, c;
    sincos((double)t * rope_freq(base, j, Ri), &sn, &c);
    cs[j] = make_double2(c, sn);
  }
  __syncthreads();
  for (int e = e0; e < chunks; e += blockDim.x) {
    const int d0 = (e * 8) % Di;
    const uint4 v = e == e0 ? v0 : *(const uint4*)(q + qoff + (int64_t)e * 8);
    *(uint4*)(qr + off + (int64_t)e * 8) = rope8_bf16(v, d0, Di, Ri, cs);
  }
}

constexpr int kDecTile = 128;  // keys per LDS tile: 32 per wave, 32 KB

// Decode key scan on 32 x 32 x 16 MFMA tiles, with index_prefill_x32's
// operands (the rotated query as A, heads as rows; keys as B).  One block
// scores a run of keys of one token, 128-key tiles at a time; the keys reach
// LDS through LDS-DMA loads (no VGPRs held while in flight), two tiles in
// flight per wave, each wave fetching and scoring its own 32 rows of a tile
// in one step of 16 MFMAs.  ReLU, weights and the sum over a lane's 16 heads
// stay in-lane, and one lane-half swap adds the other 16.  Each score also
// goes into the block's LDS histogram as it is made, so no pass over the
// stored scores follows the loop.
__global__ void __launch_bounds__(256, 2) index_decode_x32(
    const bf16_t* __restrict__ qr, const bf16_t* __restrict__ wts, const bf16_t* __restrict__ keys,
    float* __restrict__ scores, float* __restrict__ discard, uint32_t* __restrict__ hist,
    Seqs sq, int m, int64_t pool_cap, int block_keys) {
  constexpr int Hi = 64, Di = 128;
  __shared__ __attribute__((aligned(1024))) bf16_t kt0[kDecTile * Di];
  __shared__ __attribute__((aligned(1024))) bf16_t kt1[kDecTile * Di];
  __shared__ uint32_t lh[kHBins];
  const int tok = blockIdx.y;  // the query's slot b n + i
  const int b = tok / sq.n, i = tok % sq.n;
  if (i >= sq.len(b)) return;  // padding slot (block-uniform, before any barrier)
  const int lane = threadIdx.x & 63, l32 = lane & 31, h32 = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t nv = (sq.pos0[b] + i + 1) / m;
  if (nv > pool_cap) nv = pool_cap;
  const int64_t kb = (int64_t)blockIdx.x * block_keys;
  if (kb >= nv) return;  // block-uniform, before any barrier
  const int64_t ke = kb + block_keys < nv ? kb + block_keys : nv;
  const int ntile = (int)((ke - kb + kDecTile - 1) / kDecTile);
  // DMA of this wave's 32 rows of tile `tile` (8 instructions of 4 rows);
  // rows past the run re-read its last row (already in cache, never scored).
  // A tile's keys lie in one pool block (runs and blocks are multiples of
  // 128 entries): trow is the pool row of the tile's first key, or of the
  // run's last key for a tile past the run (tile_row).
  const int lrow = lane >> 4, slot = lane & 15;
  auto tile_key = [&](int tile) {
    const int64_t t0 = kb + (int64_t)tile * kDecTile;
    return t0 < ke - 1 ? t0 : ke - 1;
  };
  auto tile_row = [&](int tile) { return sq.prow(b, tile_key(tile), pool_cap); };
  auto issue = [&](int tile, bf16_t* dst, int64_t trow) {
    const int64_t t0 = tile_key(tile);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 32 * wv + 4 * j + lrow;
      int64_t key = kb + (int64_t)tile * kDecTile + r;
      if (key > ke - 1) key = ke - 1;
      const bf16_t* src = keys + (trow + (key - t0)) * Di + 8 * (slot ^ (r & 15));
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(dst + (32 * wv + 4 * j) * Di),
                                       16, 0, 0);
    }
  };
  // query fragments and weights first: their loads then complete before the
  // tiles' DMA, so the first wait on them leaves the DMA in flight
  const bf16_t* qrow = qr + (int64_t)tok * Hi * Di;
  const int64_t wrow = sq.row(b, i) * Hi;
  uint4 A[2][8];  // head 32 mt + l32, channels 16 kk + 8 h32 .. + 7
  float wr[2][16];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      A[mt][kk] = *(const uint4*)(qrow + (32 * mt + l32) * Di + 16 * kk + 8 * h32);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      wr[mt][r] = bf16_to_f32(wts[wrow + 32 * mt + 8 * (r / 4) + 4 * h32 + r % 4]);
  }
  const int64_t row0 = tile_row(0), row1 = tile_row(1);
  asm volatile("" ::: "memory");  // keeps those loads ahead of the DMA
  issue(0, kt0, row0);
  issue(1, kt1, row1);
  int64_t trow = tile_row(2);  // loaded a tile ahead of its issue
  for (int j = threadIdx.x; j < kHBins; j += 256) lh[j] = 0u;
  // the histogram is clear before any wave adds to it (LDS stores only: the
  // DMA in flight need not land here)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // B fragment of step kk: row 32 wv + l32 of the tile, chunk 2 kk + h32 at
  // slot (2 kk + h32) ^ (l32 & 15): the lane's kk = 0 offset XOR 32 kk
  auto frags = [&](const bf16_t* buf, uint4 (&Bf)[8]) {
    int ln;  // opaque copy: keeps the per-lane addresses out of loop-invariant registers
    asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
    const int l = ln & 31, h = ln >> 5;
    const uint32_t a0 = (uint32_t)(size_t)(lds_void*)buf +
                        (uint32_t)((32 * wv + l) * Di * 2 + 16 * (h ^ (l & 1)) + 32 * ((l >> 1) & 7));
    uint32_t a[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) a[kk] = a0 ^ (32u * kk);
    lds_frag8<0>(a, Bf);
  };
  float* srow = scores + (int64_t)tok * pool_cap;
  auto compute = [&](int tile, const uint4 (&Bf)[8]) {
    f32x16 acc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) acc[mt] = mfma32(A[mt][kk], Bf[kk], acc[mt]);
    float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r & 3] += wr[mt][r] * relu_bits(acc[mt][r]);
    const float v = (p[0] + p[1]) + (p[2] + p[3]);
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                               false);
    const float sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // all 64 heads
    const int64_t key = kb + (int64_t)tile * kDecTile + 32 * wv + l32;
    const bool ok = key < ke;
    // both lane halves hold the score: all store it (one store per tile on
    // every path; keys past the run go to a discard slot)
    *(ok ? srow + key : discard) = sc;
    // histogram add by asm: a compiler-visible LDS atomic would first wait
    // for every DMA in flight (it cannot tell lh from the tiles); the next
    // fragment read's lgkmcnt wait orders it
    if (ok && h32 == 0) {
      const uint32_t ha = (uint32_t)(size_t)(lds_void*)&lh[order_key(sc) >> kHShift];
      asm volatile("ds_add_u32 %0, %1" ::"v"(ha), "v"(1u) : "memory");
    }
  };
  // Two tiles in flight per wave: the fragments of tile t are copied to
  // VGPRs (the asm read waits for them), then tile t+2 is fetched into the
  // same array while tile t is scored.  After vmcnt(8) only the newest
  // tile's 8 DMA rows may be in flight (score stores issued after an older
  // tile only make the wait longer).  Prefetches are unconditional.
  uint4 Bf[8];
  for (int tile = 0;;) {
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    frags(kt0, Bf);
    issue(tile + 2, kt0, trow);
    trow = tile_row(tile + 3);
    compute(tile, Bf);
    if (++tile >= ntile) break;
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    frags(kt1, Bf);
    issue(tile + 2, kt1, trow);
    trow = tile_row(tile + 3);
    compute(tile, Bf);
    if (++tile >= ntile) break;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS-DMA outlives the block
  __syncthreads();  // every wave's histogram adds are in
  uint32_t* h = hist + (int64_t)tok * kHBins;
  for (int j = threadIdx.x; j < kHBins; j += 256) {
    const uint32_t c = lh[j];
    if (c) atomicAdd(&h[j], c);
  }
}

// Block-wide (256 threads): the bin holding the k-th largest key of a
// histogram whose total exceeds k, and the number of keys in the bins above.
__device__ void hist_cut(const uint32_t* __restrict__ h, uint32_t k, uint32_t* wsum,
                         uint32_t* res) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  constexpr int per = kHBins / 256;
  if (tid == 0) {  // kept if no bin qualifies (a histogram of <= k keys)
    res[0] = 0u;
    res[1] = 0u;
  }
  uint32_t c[per], s = 0;
#pragma unroll
  for (int e = 0; e < per; ++e) {
    c[e] = h[kHBins - 1 - per * tid - e];  // thread 0 holds the top bins
    s += c[e];
  }
  uint32_t x = s;  // inclusive scan in thread order
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  uint32_t before = x - s;
  for (int w = 0; w < wv; ++w) before += wsum[w];
  if (before < k && before + s >= k) {
    uint32_t acc = before;
#pragma unroll
    for (int e = 0; e < per; ++e) {
      if (acc + c[e] >= k) {
        res[0] = (uint32_t)(kHBins - 1 - per * tid - e);
        res[1] = acc;
        break;
      }
      acc += c[e];
    }
  }
  __syncthreads();
}

// Per 1024-key slice (one wave): ids of keys above the cut bin and of keys
// inside it, each list compacted in id order at the slice's own offset.
__global__ void __launch_bounds__(256) topk_collect(const float* __restrict__ scores,
                                                    const uint32_t* __restrict__ hist,
                                                    int32_t* __restrict__ cand_hi,
                                                    int32_t* __restrict__ cand_tie,
                                                    uint32_t* __restrict__ counts, Seqs sq,
                                                    int m, int k, int64_t pool_cap, int nslice) {
  __shared__ uint32_t wsum[4], res[2];
  const int tok = blockIdx.y;  // the query's slot b n + i
  const int b = tok / sq.n, i = tok % sq.n;
  if (i >= sq.len(b)) return;  // padding slot (block-uniform)
  int64_t nv = (sq.pos0[b] + i + 1) / m;
  if (nv > pool_cap) nv = pool_cap;
  const int64_t c0b = (int64_t)blockIdx.x * 4 * kSlice;
  if (nv <= k || c0b >= nv) return;  // block-uniform
  hist_cut(hist + (int64_t)tok * kHBins, (uint32_t)k, wsum, res);
  const uint32_t T = res[0];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t c0 = c0b + (int64_t)wv * kSlice;
  if (c0 >= nv) return;
  const int64_t c1 = c0 + kSlice < nv ? c0 + kSlice : nv;
  const float* sc = scores + (int64_t)tok * pool_cap;
  int32_t* hi = cand_hi + (int64_t)tok * pool_cap + c0;
  int32_t* ti = cand_tie + (int64_t)tok * pool_cap + c0;
  const unsigned long long lt = (1ull << lane) - 1ull;
  constexpr int U = kSlice / 64;
  // all loads first, unconditional (ids past the slice re-read its last
  // score and are never counted): one latency per slice.  Guarded loads were
  // each waited for inside their own branch.
  float v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) v[u] = sc[min(c0 + 64 * u + lane, c1 - 1)];
  uint32_t bin[U];
#pragma unroll
  for (int u = 0; u < U; ++u) bin[u] = order_key(v[u]) >> kHShift;
  uint32_t nh = 0, nt = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t j = c0 + 64 * u + lane;
    const bool above = j < c1 && bin[u] > T, in = j < c1 && bin[u] == T;
    const unsigned long long ba = __ballot(above), bi = __ballot(in);
    if (above) hi[nh + __popcll(ba & lt)] = (int32_t)j;
    if (in) ti[nt + __popcll(bi & lt)] = (int32_t)j;
    nh += (uint32_t)__popcll(ba);
    nt += (uint32_t)__popcll(bi);
  }
  if (lane == 0) {
    const int64_t sl = c0 / kSlice;
    counts[((int64_t)tok * nslice + sl) * 2] = nh;
    counts[((int64_t)tok * nslice + sl) * 2 + 1] = nt;
  }
}

// Position of the first element >= x in an ascending LDS array.
__device__ __forceinline__ int lower_bound_lds(const int32_t* a, int n, int32_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int slice_of(const uint32_t* off, int ns, uint32_t i) {
  int lo = 0, hi = ns;  // last slice with off[s] <= i
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= i) lo = mid;
    else hi = mid;
  }
  return lo;
}

constexpr int kTieCap = 4096;  // keys of the cut bin held in LDS (more: read from L2)

// Per token: radix select inside the cut bin for the k - above keys still
// needed (ties to the lower id), then the ascending merge of both id lists.
__global__ void __launch_bounds__(256) topk_final(const float* __restrict__ scores,
                                                  const int32_t* __restrict__ cand_hi,
                                                  const int32_t* __restrict__ cand_tie,
                                                  const uint32_t* __restrict__ counts,
                                                  int32_t* __restrict__ out, Seqs sq,
                                                  int m, int k, int64_t pool_cap, int nslice) {
  __shared__ uint32_t off_hi[kMaxSlices + 1], off_tie[kMaxSlices + 1];
  __shared__ int32_t sel_hi[kMaxTopK], sel_tie[kMaxTopK];
  __shared__ int32_t tie_id[kTieCap];
  __shared__ uint32_t tie_key[kTieCap];
  __shared__ uint32_t bins[256], wsum[4], wcnt[4], sh_prefix, sh_rem;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int tok = blockIdx.x;  // the query's slot b n + i
  const int b = tok / sq.n, i = tok % sq.n;
  if (i >= sq.len(b)) return;  // padding slot (block-uniform)
  int64_t nv = (sq.pos0[b] + i + 1) / m;
  if (nv > pool_cap) nv = pool_cap;
  int32_t* o = out + sq.row(b, i) * k;
  if (nv <= k) {
    for (int j = tid; j < k; j += 256) o[j] = j < nv ? j : -1;
    return;
  }
  const int ns = (int)((nv + kSlice - 1) / kSlice);
  // exclusive prefix sums of the per-slice counts, 256 slices at a time
  uint32_t carry_h = 0, carry_t = 0;
  for (int s0 = 0; s0 < ns; s0 += 256) {
    const int s = s0 + tid;
    uint32_t ch = 0, ct = 0;
    if (s < ns) {
      ch = counts[((int64_t)tok * nslice + s) * 2];
      ct = counts[((int64_t)tok * nslice + s) * 2 + 1];
    }
    uint32_t xh = ch, xt = ct;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t yh = __shfl_up(xh, d, 64), yt = __shfl_up(xt, d, 64);
      if (lane >= d) { xh += yh; xt += yt; }
    }
    if (lane == 63) { wsum[wv] = xh; wcnt[wv] = xt; }
    __syncthreads();
    uint32_t bh = carry_h + xh - ch, bt = carry_t + xt - ct;
    for (int w = 0; w < wv; ++w) { bh += wsum[w]; bt += wcnt[w]; }
    if (s < ns) { off_hi[s] = bh; off_tie[s] = bt; }
    for (int w = 0; w < 4; ++w) { carry_h += wsum[w]; carry_t += wcnt[w]; }
    __syncthreads();
  }
  if (tid == 0) { off_hi[ns] = carry_h; off_tie[ns] = carry_t; }
  __syncthreads();
  // by construction 0 <= A < k <= A + C; the clamps below only keep every
  // index in bounds should the counts ever disagree
  const uint32_t A = carry_h < (uint32_t)k ? carry_h : (uint32_t)k;
  const uint32_t C = carry_t < (uint32_t)nv ? carry_t : (uint32_t)nv;
  const uint32_t need = (uint32_t)k - A < C ? (uint32_t)k - A : C;
  const bool in_lds = C <= (uint32_t)kTieCap;
  // position of list entry e of a slice list (offsets `off`) in its buffer,
  // and the id stored there, clamped into the token's rows
  auto list_pos = [&](const uint32_t* off, uint32_t e) -> int64_t {
    const int s = slice_of(off, ns, e);
    uint32_t d = e - off[s];
    if (d > (uint32_t)kSlice - 1u) d = (uint32_t)kSlice - 1u;
    int64_t p = (int64_t)s * kSlice + d;
    return p > pool_cap - 1 ? pool_cap - 1 : p;
  };
  auto clamp_id = [&](int32_t id) -> int32_t {
    return id < 0 ? 0 : (id >= nv ? (int32_t)(nv - 1) : id);
  };
  auto list_id = [&](const int32_t* base, const uint32_t* off, uint32_t e) -> int32_t {
    return clamp_id(base[list_pos(off, e)]);
  };
  const float* sc = scores + (int64_t)tok * pool_cap;
  const int32_t* hb = cand_hi + (int64_t)tok * pool_cap;
  const int32_t* tb = cand_tie + (int64_t)tok * pool_cap;
  // the cut bin's keys share their top kHBits bits: keep the low ones
  constexpr uint32_t kLow = (1u << kHShift) - 1u;
  // gather both id lists, 4 items per thread in flight: the positions first
  // (LDS searches), then every id load, then every score load, all
  // unconditional (positions and ids clamped into the buffers; items past a
  // list are not kept), so that each group shares one latency (loads guarded
  // by their own branches were each waited for inside it)
  for (uint32_t e0 = 0; e0 < (A > C ? A : C); e0 += 1024) {
    int64_t pa[4], pt[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t e = e0 + 256 * u + tid;
      pa[u] = list_pos(off_hi, e);
      pt[u] = list_pos(off_tie, e);
    }
    int32_t ida[4], idt[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ida[u] = clamp_id(hb[pa[u]]);
      idt[u] = clamp_id(tb[pt[u]]);
    }
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = sc[idt[u]];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t e = e0 + 256 * u + tid;
      if (e < A) sel_hi[e] = ida[u];
      if (in_lds && e < C) {
        tie_id[e] = idt[u];
        tie_key[e] = order_key(v[u]) & kLow;
      }
    }
  }
  __syncthreads();
  auto tie_at = [&](uint32_t e, int32_t& id) -> uint32_t {
    if (in_lds) {
      id = tie_id[e];
      return tie_key[e];
    }
    id = list_id(tb, off_tie, e);
    return order_key(sc[id]) & kLow;
  };
  // radix select over the low bits: 8 + 8 + 4
  uint32_t prefix = 0, mask = 0, rem = need;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? kHShift - 8 : (pass == 1 ? kHShift - 16 : 0);
    const uint32_t nb = pass == 2 ? (1u << (kHShift - 16)) : 256u;
    bins[tid] = 0u;
    __syncthreads();
    for (uint32_t e = tid; e < C; e += 256) {
      int32_t id;
      const uint32_t key = tie_at(e, id);
      bin_add(bins, (key & mask) == prefix, (key >> shift) & (nb - 1u));
    }
    __syncthreads();
    if (tid < 64) {
      const uint32_t c0 = bins[4 * lane], c1 = bins[4 * lane + 1], c2 = bins[4 * lane + 2],
                     c3 = bins[4 * lane + 3];
      const uint32_t sum = c0 + c1 + c2 + c3;
      uint32_t suf = sum;  // inclusive suffix sum over lanes
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t x = __shfl_down(suf, d, 64);
        if (lane + d < 64) suf += x;
      }
      const unsigned long long bal = __ballot(suf >= rem);
      const int Lb = 63 - __clzll(bal);
      if (lane == Lb) {
        uint32_t above = suf - sum;
        const uint32_t cnt[4] = {c0, c1, c2, c3};
        int d = 3;
        for (; d > 0; --d) {
          if (above + cnt[d] >= rem) break;
          above += cnt[d];
        }
        sh_prefix = prefix | ((uint32_t)(4 * Lb + d) << shift);
        sh_rem = rem - above;
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    rem = sh_rem;
    mask |= (nb - 1u) << shift;
  }
  // every cut-bin key above `prefix`, and the first `rem` equal to it, in id order
  uint32_t base_sel = 0, base_eq = 0;
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (uint32_t e0 = 0; e0 < C; e0 += 256) {
    const uint32_t e = e0 + tid;
    int32_t id = -1;
    uint32_t key = 0u;
    if (e < C) key = tie_at(e, id);
    const bool gt = e < C && key > prefix, eq = e < C && key == prefix;
    const unsigned long long be = __ballot(eq);
    if (lane == 0) wcnt[wv] = (uint32_t)__popcll(be);
    __syncthreads();
    uint32_t eq_off = base_eq, eq_tot = 0;
    for (int w = 0; w < 4; ++w) {
      if (w < wv) eq_off += wcnt[w];
      eq_tot += wcnt[w];
    }
    const bool sel = gt || (eq && eq_off + (uint32_t)__popcll(be & lt) < rem);
    const unsigned long long bs = __ballot(sel);
    if (lane == 0) wsum[wv] = (uint32_t)__popcll(bs);
    __syncthreads();
    uint32_t off = base_sel, tot = 0;
    for (int w = 0; w < 4; ++w) {
      if (w < wv) off += wsum[w];
      tot += wsum[w];
    }
    const uint32_t pos = off + (uint32_t)__popcll(bs & lt);
    if (sel && pos < need) sel_tie[pos] = id;
    base_sel += tot;
    base_eq += eq_tot;
    __syncthreads();
    if (base_sel >= need) break;  // block-uniform: every later key is unselected
  }
  // both lists ascend; an id's output slot is its rank in its own list plus
  // the number of smaller ids in the other one
  for (uint32_t a = tid; a < A; a += 256) {
    const int32_t x = sel_hi[a];
    o[a + lower_bound_lds(sel_tie, (int)need, x)] = x;
  }
  for (uint32_t j = tid; j < need; j += 256) {
    const int32_t y = sel_tie[j];
    o[j + lower_bound_lds(sel_hi, (int)A, y)] = y;
  }
}

// Exclusive prefix sum of one value per thread over a block of NW waves.
template <int NW>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  uint32_t before = x - v;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wv) before += wsum[w];
    total += wsum[w];
  }
  __syncthreads();
  return before;
}

// hist_cut for a 1024-thread block: res[0] = the bin holding the k-th best
// key of histogram h, res[1] = the number of keys in the bins above it.
__device__ void hist_cut1024(const uint32_t* __restrict__ h, uint32_t k, uint32_t* wsum,
                             uint32_t* res) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  constexpr int per = kHBins / 1024;
  if (tid == 0) {
    res[0] = 0u;
    res[1] = 0u;
  }
  uint32_t c[per], s = 0;
#pragma unroll
  for (int e = 0; e < per; ++e) {
    c[e] = h[kHBins - 1 - per * tid - e];  // thread 0 holds the top bins
    s += c[e];
  }
  uint32_t x = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  uint32_t before = x - s;
  for (int w = 0; w < wv; ++w) before += wsum[w];
  if (before < k && before + s >= k) {
    uint32_t acc = before;
#pragma unroll
    for (int e = 0; e < per; ++e) {
      if (acc + c[e] >= k) {
        res[0] = (uint32_t)(kHBins - 1 - per * tid - e);
        res[1] = acc;
        break;
      }
      acc += c[e];
    }
  }
  __syncthreads();
}

// Decode selection in one launch for rows of at most kBlkTopK keys: one
// block per query, thread t reading the scores of ids 128 t .. 128 t + 127.
// The histogram the scan built names the cut bin T; a score is a candidate
// when its order key is at least the first key of bin T, i.e. when the
// score itself is at least the smallest float of that bin (one compare per
// score).  The candidates' ids go to LDS in id order (a block scan of the
// per-thread counts gives each thread its first slot; writes of non-
// candidates land on a per-lane spare slot, so the unrolled loop has no
// branches).  A radix select on the low 20 bits settles bin T among the
// candidates (scores re-read from L2 by id), and an ordered pass over the
// candidates emits the k ids ascending, ties to the lower id.
constexpr int kBlkTopKT = 1024;  // threads: four waves per SIMD hide VALU latency
constexpr int kBlkTopKU = 32;    // scores per thread
constexpr int kBlkTopK = kBlkTopKT * kBlkTopKU;

__global__ void __launch_bounds__(kBlkTopKT) topk_block(const float* __restrict__ scores,
                                                  const uint32_t* __restrict__ hist,
                                                  int32_t* __restrict__ out, Seqs sq,
                                                  int m, int k, int64_t pool_cap) {
  __shared__ int32_t cand[kBlkTopK + 64];  // candidate ids in id order (+ a spare per lane)
  __shared__ uint32_t wsum[kBlkTopKT / 64], wcnt[kBlkTopKT / 64], res[2], bins[256], sh_prefix,
      sh_rem;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int tok = blockIdx.x;  // the query's slot b n + i
  const int b = tok / sq.n, i = tok % sq.n;
  if (i >= sq.len(b)) return;  // padding slot (block-uniform)
  int64_t nv = (sq.pos0[b] + i + 1) / m;
  if (nv > pool_cap) nv = pool_cap;
  int32_t* o = out + sq.row(b, i) * k;
  if (nv <= k) {
    for (int j = tid; j < k; j += kBlkTopKT) o[j] = j < nv ? j : -1;
    return;
  }
  constexpr int U = kBlkTopKU;
  const int j0 = tid * U;
  const int nval = (int)(nv - j0 < 0 ? 0 : (nv - j0 > U ? U : nv - j0));
  const float* row = scores + (int64_t)tok * pool_cap;
  const float* sc = row + j0;
  // the loads go out before the histogram is read; ids past the row get a
  // NaN, which no comparison selects
  float x[U];
  if (nval == U && (pool_cap & 3) == 0) {
#pragma unroll
    for (int u = 0; u < U; u += 4) {
      const float4 v = *(const float4*)(sc + u);
      x[u] = v.x;
      x[u + 1] = v.y;
      x[u + 2] = v.z;
      x[u + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = u < nval ? sc[u] : __uint_as_float(0x7fc00000u);
  }
  hist_cut1024(hist + (int64_t)tok * kHBins, (uint32_t)k, wsum, res);
  const uint32_t T = res[0];
  const uint32_t A = res[1];  // keys in the bins above T: all selected
  // smallest float whose order key lies in bin T (order keys are monotonic
  // in the score; -0 and +0 share one)
  const uint32_t tkey = T << kHShift;
  const float thr = __uint_as_float((tkey & 0x80000000u) ? (tkey & 0x7fffffffu) : ~tkey);
  // candidate flags as four bit words (kept as masks, 128 of them would not
  // fit the scalar registers)
  uint32_t cw[U / 32];
#pragma unroll
  for (int w = 0; w < U / 32; ++w) {
    uint32_t bits = 0;
#pragma unroll
    for (int u = 0; u < 32; ++u) bits |= (x[32 * w + u] >= thr ? 1u : 0u) << u;
    cw[w] = bits;
  }
  uint32_t nc = 0;
#pragma unroll
  for (int w = 0; w < U / 32; ++w) nc += (uint32_t)__popc(cw[w]);
  uint32_t N;
  uint32_t pos = block_scan<kBlkTopKT / 64>(nc, wsum, N);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t c = (cw[u >> 5] >> (u & 31)) & 1u;
    cand[c ? pos : (uint32_t)(kBlkTopK + lane)] = j0 + u;
    pos += c;
  }
  __syncthreads();
  if (N > (uint32_t)nv) N = (uint32_t)nv;  // only should the histogram disagree
  constexpr uint32_t kLow = (1u << kHShift) - 1u;
  auto key_of = [&](uint32_t e) -> uint32_t { return order_key(row[cand[e]]); };
  // radix select over the low bits of the candidates in bin T: 8 + 8 + 4
  const uint32_t need = (uint32_t)k - A;
  uint32_t prefix = 0, mask = 0, rem = need;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? kHShift - 8 : (pass == 1 ? kHShift - 16 : 0);
    const uint32_t nb = pass == 2 ? (1u << (kHShift - 16)) : 256u;
    if (tid < 256) bins[tid] = 0u;
    __syncthreads();
    for (uint32_t e = tid; e < N; e += kBlkTopKT) {
      const uint32_t key = key_of(e);
      bin_add(bins, (key >> kHShift) == T && ((key & kLow) & mask) == prefix,
              ((key & kLow) >> shift) & (nb - 1u));
    }
    __syncthreads();
    if (tid < 64) {
      const uint32_t c0 = bins[4 * lane], c1 = bins[4 * lane + 1], c2 = bins[4 * lane + 2],
                     c3 = bins[4 * lane + 3];
      const uint32_t sum = c0 + c1 + c2 + c3;
      uint32_t suf = sum;  // inclusive suffix sum over lanes
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_down(suf, d, 64);
        if (lane + d < 64) suf += y;
      }
      const unsigned long long bal = __ballot(suf >= rem);
      const int Lb = 63 - __clzll(bal);
      if (lane == Lb) {
        uint32_t above = suf - sum;
        const uint32_t cnt[4] = {c0, c1, c2, c3};
        int d = 3;
        for (; d > 0; --d) {
          if (above + cnt[d] >= rem) break;
          above += cnt[d];
        }
        sh_prefix = prefix | ((uint32_t)(4 * Lb + d) << shift);
        sh_rem = rem - above;
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    rem = sh_rem;
    mask |= (nb - 1u) << shift;
  }
  // the k-th best key is tk: every candidate above it, and the first `rem`
  // equal to it in id order, go out in id order
  const uint32_t tk = tkey | prefix;
  const unsigned long long lt = (1ull << lane) - 1ull;
  uint32_t base_sel = 0, base_eq = 0;
  for (uint32_t e0 = 0; e0 < N; e0 += kBlkTopKT) {
    const uint32_t e = e0 + tid;
    const uint32_t key = e < N ? key_of(e) : 0u;
    const bool gt = e < N && key > tk, eq = e < N && key == tk;
    const unsigned long long be = __ballot(eq);
    if (lane == 0) wcnt[wv] = (uint32_t)__popcll(be);
    __syncthreads();
    uint32_t eq_off = base_eq, eq_tot = 0;
    for (int w = 0; w < kBlkTopKT / 64; ++w) {
      if (w < wv) eq_off += wcnt[w];
      eq_tot += wcnt[w];
    }
    const bool sel = gt || (eq && eq_off + (uint32_t)__popcll(be & lt) < rem);
    const unsigned long long bs = __ballot(sel);
    if (lane == 0) wsum[wv] = (uint32_t)__popcll(bs);
    __syncthreads();
    uint32_t off = base_sel, tot = 0;
    for (int w = 0; w < kBlkTopKT / 64; ++w) {
      if (w < wv) off += wsum[w];
      tot += wsum[w];
    }
    const uint32_t p = off + (uint32_t)__popcll(bs & lt);
    if (sel && p < (uint32_t)k) o[p] = cand[e];
    base_sel += tot;
    base_eq += eq_tot;
    __syncthreads();
    if (base_sel >= (uint32_t)k) break;  // block-uniform
  }
}

// ---------------------------------------------------------------------------
// generic: any shape, VALU float32

template <typename T>
__global__ void __launch_bounds__(256) index_generic(const T* __restrict__ q,
                                                     const T* __restrict__ wts,
                                                     const T* __restrict__ keys,
                                                     float* __restrict__ scores, Seqs sq,
                                                     int Hi, int Di, int Ri, Rope base, int m,
                                                     int64_t pool_cap) {
  extern __shared__ float qs[];  // [Hi * Di] rotated query, then [Hi] weights
  const int i = blockIdx.x, b = blockIdx.y;
  if (i >= sq.len(b)) return;  // padding slot (block-uniform)
  const int64_t t = sq.pos0[b] + i;
  const int64_t tok = (int64_t)b * sq.n + i;  // the query's slot (scores row)
  const int64_t qr_ = sq.row(b, i);           // its row in q and the weights
  const T* qrow = q + qr_ * Hi * Di;
  const int first = Di - Ri;
  for (int e = threadIdx.x; e < Hi * Di; e += blockDim.x) {
    const int d = e % Di;
    if (d < first) {
      qs[e] = store_t<T>::ld(qrow + e);
    } else if (((d - first) & 1) == 0) {
      const int j = (d - first) >> 1;
      double sn, c;
      sincos((double)t * rope_freq(base, j, Ri), &sn, &c);
      double a = store_t<T>::ld(qrow + e), bb = store_t<T>::ld(qrow + e + 1);
      rot64(a, bb, c, sn);
      // the rotated query is stored at the storage dtype
      T ra, rb;
      store_t<T>::st64(&ra, a);
      store_t<T>::st64(&rb, bb);
      qs[e] = store_t<T>::cvt(ra);
      qs[e + 1] = store_t<T>::cvt(rb);
    }
  }
  float* wsh = qs + Hi * Di;
  for (int h = threadIdx.x; h < Hi; h += blockDim.x) wsh[h] = store_t<T>::ld(wts + qr_ * Hi + h);
  __syncthreads();
  int64_t nv = (t + 1) / m;
  if (nv > pool_cap) nv = pool_cap;
  for (int64_t w = threadIdx.x; w < nv; w += blockDim.x) {
    const T* krow = keys + sq.prow(b, w, pool_cap) * Di;
    float s = 0.f;
    for (int h = 0; h < Hi; ++h) {
      float dot = 0.f;
      for (int d = 0; d < Di; ++d) dot = fmaf(qs[h * Di + d], store_t<T>::ld(krow + d), dot);
      s = fmaf(wsh[h], fmaxf(dot, 0.f), s);
    }
    scores[tok * pool_cap + w] = s;
  }
}

// ---------------------------------------------------------------------------
// top-k by radix select

template <int BS>
__global__ void __launch_bounds__(BS) topk_radix(const float* __restrict__ scores,
                                                 int64_t stride, int32_t* __restrict__ out,
                                                 Seqs sq, int m, int k, int64_t pool_cap) {
  constexpr int NW = BS / 64;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_prefix, sh_rem;
  __shared__ uint32_t wcnt[2][NW];
  const int i = blockIdx.x, b = blockIdx.y;
  if (i >= sq.len(b)) return;  // padding slot (block-uniform)
  const int64_t tok = (int64_t)b * sq.n + i;  // the query's slot (scores row)
  int64_t nv = (sq.pos0[b] + i + 1) / m;
  if (nv > pool_cap) nv = pool_cap;
  const int n = (int)nv;
  const float* sc = scores + tok * stride;
  int32_t* o = out + sq.row(b, i) * k;
  if (n <= k) {
    for (int j = threadIdx.x; j < k; j += BS) o[j] = j < n ? j : -1;
    return;
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t prefix = 0, mask = 0, rem = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int j = threadIdx.x; j < 256; j += BS) hist[j] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < n; j += BS) {
      const uint32_t key = order_key(sc[j]);
      bin_add(hist, (key & mask) == prefix, (key >> shift) & 255u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                     c3 = hist[4 * lane + 3];
      const uint32_t s = c0 + c1 + c2 + c3;
      uint32_t suf = s;  // inclusive suffix sum over lanes
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_down(suf, off, 64);
        if (lane + off < 64) suf += v;
      }
      const unsigned long long bal = __ballot(suf >= rem);
      const int L = 63 - __clzll(bal);
      if (lane == L) {
        uint32_t above = suf - s;
        const uint32_t cnt[4] = {c0, c1, c2, c3};
        int d = 3;
        for (; d > 0; --d) {
          if (above + cnt[d] >= rem) break;
          above += cnt[d];
        }
        sh_prefix = prefix | ((uint32_t)(4 * L + d) << shift);
        sh_rem = rem - above;
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    rem = sh_rem;
    mask |= 255u << shift;
  }
  // prefix is the k-th largest key; take every larger key and the first
  // `rem` keys equal to it, in id order.
  uint32_t base_sel = 0, base_eq = 0;
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int j0 = 0; j0 < n; j0 += BS) {
    const int j = j0 + threadIdx.x;
    const uint32_t key = j < n ? order_key(sc[j]) : 0u;
    const bool gt = j < n && key > prefix;
    const bool eq = j < n && key == prefix;
    const unsigned long long be = __ballot(eq);
    if (lane == 0) wcnt[0][wv] = (uint32_t)__popcll(be);
    __syncthreads();
    uint32_t eq_off = base_eq, eq_tot = 0;
    for (int w = 0; w < NW; ++w) {
      if (w < wv) eq_off += wcnt[0][w];
      eq_tot += wcnt[0][w];
    }
    const bool sel = gt || (eq && eq_off + (uint32_t)__popcll(be & lt) < rem);
    const unsigned long long bs = __ballot(sel);
    if (lane == 0) wcnt[1][wv] = (uint32_t)__popcll(bs);
    __syncthreads();
    uint32_t off = base_sel, tot = 0;
    for (int w = 0; w < NW; ++w) {
      if (w < wv) off += wcnt[1][w];
      tot += wcnt[1][w];
    }
    const uint32_t pos = off + (uint32_t)__popcll(bs & lt);
    if (sel && pos < (uint32_t)k) o[pos] = j;
    base_sel += tot;
    base_eq += eq_tot;
    __syncthreads();
  }
}

// Per query one wave (four per block) for rows of at most 2048 scores: the
// row stays in registers (32 scores per lane, id 64 u + lane) through the
// same four 8-bit radix passes as topk_radix and the emit in id order by
// ballots; no block barriers.  Each pass counts into four copies of a
// 256-bin histogram private to the wave (copy = lane mod 4): the row's
// scores share few leading bits, and adds of equal bins from one instruction
// serialize.
constexpr int kTkPer = 32;

__global__ void __launch_bounds__(256) topk_wave(const float* __restrict__ scores, int64_t stride,
                                                 int32_t* __restrict__ out,
                                                 Seqs sq, int m, int k, int64_t pool_cap) {
  __shared__ uint32_t hist_all[4][4][256];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = blockIdx.x * 4 + wv, b = blockIdx.y;
  // wave-uniform (padding rows are left as they are); the waves never meet
  // at a barrier
  if (i >= sq.len(b)) return;
  uint32_t (*hist)[256] = hist_all[wv];
  const int64_t tok = (int64_t)b * sq.n + i;  // the query's slot (scores row)
  int64_t nv = (sq.pos0[b] + i + 1) / m;
  if (nv > pool_cap) nv = pool_cap;
  const int n = (int)nv;
  const float* sc = scores + tok * stride;
  int32_t* o = out + sq.row(b, i) * k;
  if (n <= k) {
    for (int j = lane; j < k; j += 64) o[j] = j < n ? j : -1;
    return;
  }
  // every load is unconditional (ids past the row re-read its last score,
  // never counted) so that all 32 are in flight at once; a load guarded by
  // its own branch was waited for inside that branch, one latency each
  float v[kTkPer];
#pragma unroll
  for (int u = 0; u < kTkPer; ++u) v[u] = sc[min(64 * u + lane, n - 1)];
  uint32_t key[kTkPer];
#pragma unroll
  for (int u = 0; u < kTkPer; ++u)  // masked, not branched: keeps the loads together
    key[u] = order_key(v[u]) & (0u - (uint32_t)(64 * u + lane < n));
  uint32_t* myh = hist[lane & 3];
  uint32_t prefix = 0, mask = 0, rem = (uint32_t)k;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) hist[c][64 * e + lane] = 0u;
#pragma unroll
    for (int u = 0; u < kTkPer; ++u)
      if (64 * u + lane < n && (key[u] & mask) == prefix)
        atomicAdd(&myh[(key[u] >> shift) & 255u], 1u);
    uint32_t cnt[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      cnt[e] = hist[0][4 * lane + e] + hist[1][4 * lane + e] + hist[2][4 * lane + e] +
               hist[3][4 * lane + e];
    const uint32_t sum = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    uint32_t suf = sum;  // inclusive suffix sum over lanes (lane 63: the largest keys)
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t v = __shfl_down(suf, off, 64);
      if (lane + off < 64) suf += v;
    }
    const unsigned long long bal = __ballot(suf >= rem);
    const int L = 63 - __clzll(bal);
    uint32_t above = suf - sum;
    int d = 3;
    for (; d > 0; --d) {
      if (above + cnt[d] >= rem) break;
      above += cnt[d];
    }
    const uint32_t np = prefix | ((uint32_t)(4 * L + d) << shift), nr = rem - above;
    prefix = (uint32_t)__builtin_amdgcn_readlane((int)np, L);
    rem = (uint32_t)__builtin_amdgcn_readlane((int)nr, L);
    mask |= 255u << shift;
  }
  // prefix is the k-th largest key: every larger key and the first `rem`
  // keys equal to it, in id order
  const unsigned long long lt = (1ull << lane) - 1ull;
  uint32_t base_sel = 0, base_eq = 0;
#pragma unroll
  for (int u = 0; u < kTkPer; ++u) {
    const int j = 64 * u + lane;
    const bool gt = j < n && key[u] > prefix, eq = j < n && key[u] == prefix;
    const unsigned long long be = __ballot(eq);
    const bool sel = gt || (eq && base_eq + (uint32_t)__popcll(be & lt) < rem);
    const unsigned long long bs = __ballot(sel);
    if (sel) o[base_sel + (uint32_t)__popcll(bs & lt)] = j;
    base_sel += (uint32_t)__popcll(bs);
    base_eq += (uint32_t)__popcll(be);
  }
}

// ---------------------------------------------------------------------------

hipError_t launch_index_topk(const Layer& L, const Batch& bt, const void* q, const void* w,
                             const void* keys, int64_t pool_cap, int32_t* idx, float* scores_out,
                             void* ws, hipStream_t s) {
  char* wsp = (char*)ws;
  const Seqs sq = seqs_of(bt);
  const size_t bn = (size_t)bt.B * bt.n;
  float* scores = (float*)wsp;
  wsp += align256(bn * pool_cap * sizeof(float));
  if (scores_out) scores = scores_out;
  if (index_decode_path(L, bt.n, pool_cap)) {
    const int nslice = (int)((pool_cap + kSlice - 1) / kSlice);
    bf16_t* qr = (bf16_t*)wsp;
    wsp += align256(bn * L.Hi * L.Di * 2);
    uint32_t* hist = (uint32_t*)wsp;
    wsp += align256(bn * kHBins * sizeof(uint32_t));
    int32_t* cand_hi = (int32_t*)wsp;
    wsp += align256(bn * pool_cap * sizeof(int32_t));
    int32_t* cand_tie = (int32_t*)wsp;
    wsp += align256(bn * pool_cap * sizeof(int32_t));
    uint32_t* counts = (uint32_t*)wsp;
    // 1024 threads: one 16-byte chunk of the query each (64 x 128 channels),
    // many waves per SIMD to cover the float64 rotation's latency
    rotate_queries_bf16<<<dim3(bt.n, bt.B), 1024, 0, s>>>((const bf16_t*)q, qr, hist, sq, L.Hi,
                                                         L.Di, L.Ri, L.base);
    int64_t nv = (bt.pos0_max + bt.n) / L.m;
    if (nv > pool_cap) nv = pool_cap;
    const unsigned tokens = (unsigned)bn;
    if (nv > 0) {
      // ~512 blocks over the call (two per CU), runs of whole tiles
      const int64_t per_tok = (512 + tokens - 1) / tokens;
      int64_t bk = (nv + per_tok - 1) / per_tok;
      bk = (bk + kDecTile - 1) / kDecTile * kDecTile;
      dim3 g1((unsigned)((nv + bk - 1) / bk), tokens);
      index_decode_x32<<<g1, 256, 0, s>>>(qr, (const bf16_t*)w, (const bf16_t*)keys, scores,
                                          (float*)(counts + bn * nslice * 2), hist, sq, L.m,
                                          pool_cap, (int)bk);
    }
    if (nv <= kBlkTopK) {
      topk_block<<<tokens, kBlkTopKT, 0, s>>>(scores, hist, idx, sq, L.m, L.k, pool_cap);
      return hipGetLastError();
    }
    if (nv > L.k) {
      dim3 g2((unsigned)((nv + 4 * kSlice - 1) / (4 * kSlice)), tokens);
      topk_collect<<<g2, 256, 0, s>>>(scores, hist, cand_hi, cand_tie, counts, sq, L.m, L.k,
                                      pool_cap, nslice);
    }
    topk_final<<<tokens, 256, 0, s>>>(scores, cand_hi, cand_tie, counts, idx, sq, L.m, L.k,
                                      pool_cap, nslice);
    return hipGetLastError();
  }
  if (index_fast_shape(L) && L.Ri == 64) {
    const unsigned nblk = (unsigned)((bt.n + kX32Q - 1) / kX32Q);
    index_prefill_x32<64><<<nblk * bt.B, 256, 0, s>>>((const bf16_t*)q, (const bf16_t*)w,
                                                      (const bf16_t*)keys, scores, (float*)wsp,
                                                      sq, bt.B, L.base, L.m, pool_cap);
  } else if (index_fast_shape(L)) {
    dim3 grid((bt.n + kIdxQPB - 1) / kIdxQPB, bt.B);
    index_prefill_mfma<<<grid, 256, 0, s>>>((const bf16_t*)q, (const bf16_t*)w,
                                            (const bf16_t*)keys, scores, sq, L.Ri, L.base, L.m,
                                            pool_cap);
  } else {
    const size_t shm = ((size_t)L.Hi * L.Di + L.Hi) * sizeof(float);
    dim3 grid(bt.n, bt.B);
    if (L.dtype == 1)
      index_generic<bf16_t><<<grid, 256, shm, s>>>((const bf16_t*)q, (const bf16_t*)w,
                                                   (const bf16_t*)keys, scores, sq, L.Hi, L.Di,
                                                   L.Ri, L.base, L.m, pool_cap);
    else
      index_generic<float><<<grid, 256, shm, s>>>((const float*)q, (const float*)w,
                                                  (const float*)keys, scores, sq, L.Hi, L.Di,
                                                  L.Ri, L.base, L.m, pool_cap);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((bt.pos0_max + bt.n) / L.m <= 64 * kTkPer) {  // every row fits in one wave's registers
    dim3 gw((bt.n + 3) / 4, bt.B);
    topk_wave<<<gw, 256, 0, s>>>(scores, pool_cap, idx, sq, L.m, L.k, pool_cap);
    return hipGetLastError();
  }
  dim3 grid(bt.n, bt.B);
  if ((bt.pos0_max + bt.n) / L.m > 16384)
    topk_radix<1024><<<grid, 1024, 0, s>>>(scores, pool_cap, idx, sq, L.m, L.k, pool_cap);
  else
    topk_radix<256><<<grid, 256, 0, s>>>(scores, pool_cap, idx, sq, L.m, L.k, pool_cap);
  return hipGetLastError();
}

}  // namespace csa
