// Attention over the sliding window plus compressed rows, K = V, with sink,
// on 32 x 32 x 16 bf16 MFMA tiles, two blocks per CU (H = 64, D = 512)
// [DeepSeek-V4 model page, sec. 2.3: shared K=V MQA over the sliding window
// and the compressed rows, sink (eq. 27), output rotation (eq. 26)].
//
// One block of four waves per (token, row split); two blocks share a CU, so
// one block's barriers, softmax and gather issue overlap the other's MFMAs.
// Rows come in chunks of 32, gathered by LDS-DMA (one 1 KB row per wave
// instruction) into two 32 KB buffers; the next chunk's gather is issued
// during this chunk's QK^T.
//  * S^T = K Q^T: wave w scores the chunk's 32 rows for heads 32 ht .. +31
//    (ht = w & 1) over channels 256 kh .. +255 (kh = w >> 1): 16 steps of
//    32 x 32 x 16 (on gfx950 about twice the rate of 16 x 16 x 32).  The two
//    waves of a head tile add their partial scores through LDS, each keeping
//    half of the rows (8-row groups kh and kh + 2), then exchange their
//    maxima; both take the same lazy-rescale decision (the running maximum
//    is raised only by more than 2^8).  The kh = 1 wave reads its K rows
//    with 8-row groups swapped (row ^ 8), so in both waves the kept rows sit
//    in accumulator groups 0 and 2 and the given ones in 1 and 3;
//  * P (32 rows x 64 heads, bf16) goes to LDS; O^T += V^T P^T: wave w
//    accumulates channels 128 w .. 128 w + 127 of all 64 heads (8 tiles of
//    32 x 32), V^T from the row-major K = V tile through the LDS transpose
//    read;
//  * the sink is folded once at the end; the bf16 output (or the float32
//    partial of a row split) is staged through LDS and written in whole rows.
#include "csa_device.h"
#include "csa_internal.h"
#include "attend_common.h"

namespace csa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two 16-byte stores of MFMA results at a and a + S (byte offset).  The
// hardware does not hold a VALU or LDS read of an MFMA result until the MFMA
// has written it, and the compiler's wait states do not cover inline asm:
// the nops (20 cycles) come first.
template <int S>
__device__ __forceinline__ void lds_st2x128_mfma(void* a, f32x4 v0, f32x4 v1) {
  asm volatile(
      "s_nop 7\n\ts_nop 7\n\ts_nop 3\n\tds_write_b128 %0, %1\n\tds_write_b128 %0, %2 offset:%3"
      ::"v"(lds_addr(a)), "v"(__builtin_bit_cast(u32x4, v0)), "v"(__builtin_bit_cast(u32x4, v1)),
      "i"(S)
      : "memory");
}
// One 16-byte load, complete on return.
__device__ __forceinline__ u32x4 lds_ld128(const void* a) {
  u32x4 x;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(x) : "v"(lds_addr(a)) : "memory");
  return x;
}
// Two 16-byte loads at a and a + S (byte offset), complete on return.
template <int S>
__device__ __forceinline__ void lds_ld_2x128(const void* a, f32x4& o0, f32x4& o1) {
  u32x4 x0, x1;
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:%3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(x0), "=&v"(x1)
               : "v"(lds_addr(a)), "i"(S)
               : "memory");
  o0 = __builtin_bit_cast(f32x4, x0);
  o1 = __builtin_bit_cast(f32x4, x1);
}
// Four 16-byte loads at a + i*SA + j*SB (i, j < 2) and two 4-byte loads at b
// and b + SC (byte offsets), complete on return.
template <int SA, int SB, int SC>
__device__ __forceinline__ void lds_ld_2x2x128_2x32(const void* a, const void* b,
                                                    uint4 (&o)[2][2], uint32_t (&w)[2]) {
  static_assert(SA + SB < 65536 && SC < 65536, "immediate LDS offsets are 16-bit");
  u32x4 x[4];
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %6 offset:%9\n\t"
      "ds_read_b128 %2, %6 offset:%8\n\t"
      "ds_read_b128 %3, %6 offset:%10\n\t"
      "ds_read_b32 %4, %7\n\t"
      "ds_read_b32 %5, %7 offset:%11\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(w[0]), "=&v"(w[1])
      : "v"(lds_addr(a)), "v"(lds_addr(b)), "i"(SA), "i"(SB), "i"(SA + SB), "i"(SC)
      : "memory");
  o[0][0] = __builtin_bit_cast(uint4, x[0]);
  o[0][1] = __builtin_bit_cast(uint4, x[1]);
  o[1][0] = __builtin_bit_cast(uint4, x[2]);
  o[1][1] = __builtin_bit_cast(uint4, x[3]);
}

constexpr int kHCh = 32;          // rows per chunk
constexpr int kHPRow = kHCh + 8;  // LDS row of P per head: 32 row slots + pad (bf16)
#ifndef CSA_H32_QD
#define CSA_H32_QD 2
#endif
constexpr int kHQD = CSA_H32_QD;  // K fragment reads ahead of their MFMAs

// Query fragments of head row qrow for the 32 x 32 x 16 B operand over the
// channel half kh: fragment s holds channels 256 kh + 16 s + 8 hi .. +7.
// Fragments inside the last R channels come from qrot (this head's R rotated
// channels, bf16, in LDS); the others straight from the query row.
template <int R>
__device__ __forceinline__ void load_qfrag32h(const bf16_t* __restrict__ qrow, const bf16_t* qrot,
                                              int hi, int kh, uint4 (&Qf)[16]) {
  constexpr int first = kAD - R;  // multiple of 16: a fragment is all in or all out
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int d0 = 256 * kh + 16 * s + 8 * hi;
    Qf[s] = d0 >= first ? *(const uint4*)(qrot + (d0 - first)) : *(const uint4*)(qrow + d0);
  }
}

// LDS byte offset of 16-byte chunk `ch` (0..63) of row r under the row swizzle.
__device__ __forceinline__ int swz_chunk(int r, int ch) {
  return r * 1024 + (((ch & ~15) | ((ch & 15) ^ swz(r))) << 4);
}

template <int R>
__global__ void __launch_bounds__(256, 2) attend_h32(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ win, int64_t win_cap,
    const bf16_t* __restrict__ pool, int64_t pool_cap, const int32_t* __restrict__ idx, int k,
    const float* __restrict__ sinks, bf16_t* __restrict__ out, float* __restrict__ part,
    const int64_t* __restrict__ pos0, int n_new, int W, int m, Rope base, float scale,
    int nsplit, int csa) {
  static_assert(R % 16 == 0 && R <= kMaxRope, "rope channels: multiple of 16, <= 128");
  // two separate arrays (not one indexed by parity) so the compiler can tell
  // the DMA target from the tile being read
  __shared__ __attribute__((aligned(1024))) bf16_t kb0[kHCh * kAD];
  __shared__ __attribute__((aligned(1024))) bf16_t kb1[kHCh * kAD];
  // row ids (>= 0 window ring row, <= -2 pool row), masked rows and rows past
  // the list replaced by the query's own window row (finite, never weighted)
  __shared__ __attribute__((aligned(16))) int32_t rid[kMaxRows];
  // partial-score exchange (4 waves x 2 KB), reused for P once every wave
  // has read its partner's scores
  __shared__ __attribute__((aligned(16))) char xp[4 * 2048];
  __shared__ uint32_t vmask[kMaxRows / 32 + 1];
  __shared__ double2 cs[kMaxRope / 2];
  __shared__ float cmx[4][32];   // each wave's chunk maximum per head of its tile
  __shared__ __attribute__((aligned(16))) uint32_t flg[4];  // wave's rows exceed its maximum
  __shared__ float alph[kAH];    // this chunk's rescale of O per head
  __shared__ float lfin[4][32];  // each wave's running sum per head of its tile
  __shared__ float mfin[kAH];    // final running maximum per head
  static_assert(kAH * kHPRow * 2 <= (int)sizeof(xp), "P fits the exchange buffer");
  bf16_t* const ps = (bf16_t*)xp;  // P per head, row slots

  const int i = n_new - 1 - (int)blockIdx.x;  // longest rows first
  const int b = blockIdx.y, split = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, lo = lane & 31, hi = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: role selects stay uniform
  const int ht = wv & 1, kh = wv >> 1;  // QK^T head tile and channel half of this wave
  const int64_t t = pos0[b] + i;
  const int64_t tok = (int64_t)b * n_new + i;
  const int64_t wlo = t - W + 1 > 0 ? t - W + 1 : 0;
  const int nwin = (int)(t - wlo + 1);
  int64_t nvis = m > 0 ? (t + 1) / m : 0;
  if (nvis > pool_cap) nvis = pool_cap;
  const int npool = csa ? (int)(nvis < k ? nvis : k) : (int)nvis;
  const int nrows = nwin + npool;
  const int nch = (nrows + kHCh - 1) / kHCh;
  const int cps = (nch + nsplit - 1) / nsplit;
  const int c0 = min(nch, split * cps), c1 = min(nch, c0 + cps);
  const int r0 = c0 * kHCh, r1 = min(nrows, c1 * kHCh);
  const int32_t* idx_row = csa ? idx + tok * k : nullptr;
  const int self_id = (int)((int64_t)b * win_cap + t % win_cap);

  for (int j = tid; j < R / 2; j += 256) {
    double sn, c;
    sincos((double)t * rope_freq(base, j, R), &sn, &c);
    cs[j] = make_double2(c, sn);
  }
  // row ids of the split's chunks; bit r of vmask[c - c0]: row r of chunk c
  // takes part
  for (int j0 = 64 * wv; j0 < r1 - r0; j0 += 256) {
    const int j = j0 + lane;
    const int id = j < r1 - r0 ? row_id(r0 + j, nwin, wlo, win_cap, b, pool_cap, idx_row, csa, nvis)
                               : -1;
    rid[j] = id == -1 ? self_id : id;
    const unsigned long long bal = __ballot(id != -1);
    if (lane == 0) {
      vmask[j0 >> 5] = (uint32_t)bal;
      vmask[(j0 >> 5) + 1] = (uint32_t)(bal >> 32);
    }
  }
  __syncthreads();

  // gather of chunk c into dst: this wave moves rows 8 wv .. 8 wv + 7 (one
  // 1 KB row per DMA instruction); lane e < 8 reads row e's id and the ids
  // are made scalar, the lane id is copied opaquely so nothing here is
  // spilled (a scratch reload would wait on every DMA in flight)
  struct Gather {
    int id[8];
    int ln;
    bf16_t* dst;
  };
  auto gather_prep = [&](Gather& G, int c, bf16_t* dst) {
    asm volatile("v_mov_b32 %0, %1" : "=v"(G.ln) : "v"(lane));
    G.dst = dst;
    // past the last chunk (a dummy gather, see chunk()) read chunk c0's rows
    const int base_r = (c < c1 ? c - c0 : 0) * kHCh + 8 * wv;
    const int mine = rid[base_r + (lane & 7)];
#pragma unroll
    for (int e = 0; e < 8; ++e) G.id[e] = __builtin_amdgcn_readlane(mine, e);
  };
  auto gather_row = [&](const Gather& G, int e) {
    const int rr = 8 * wv + e;
    const int id = G.id[e];
    const bf16_t* src = id >= 0 ? win + (int64_t)id * kAD : pool + (int64_t)(-2 - id) * kAD;
    __builtin_amdgcn_global_load_lds((const void*)((const char*)src + 16 * (G.ln ^ swz(rr))),
                                     (lds_void*)(G.dst + rr * kAD), 16, 0, 0);
  };
  // the last R channels of every head rotated at the query's position in
  // float64 and rounded to bf16 once, staged in kb1 (idle until the second
  // chunk's gather): head h at kb1[h * R ..]
  constexpr int first = kAD - R;
  {
    // 16-byte pieces (4 pairs); the loads of a thread's pieces are issued
    // together
    constexpr int kPieces = kAH * R / 8, kPer = (kPieces + 255) / 256;
    const bf16_t* qt = q + tok * kAH * kAD;
    uint4 v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + 256 * u;
      v[u] = e < kPieces ? *(const uint4*)(qt + (e / (R / 8)) * kAD + first + 8 * (e % (R / 8)))
                         : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + 256 * u;
      if (e < kPieces) {
        const int h = e / (R / 8), pc = e % (R / 8);
        uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          double a = bf16_to_f32((bf16_t)(w4[p] & 0xffffu));
          double bb = bf16_to_f32((bf16_t)(w4[p] >> 16));
          const double2 c = cs[4 * pc + p];
          rot64(a, bb, c.x, c.y);
          w4[p] = (uint32_t)f64_to_bf16(a) | ((uint32_t)f64_to_bf16(bb) << 16);
        }
        *(uint4*)(kb1 + h * R + 8 * pc) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      }
    }
  }
  __syncthreads();
  // rotated queries of head 32 ht + lo, channels 256 kh + 16 s + 8 hi .. +7,
  // read before the first gather is issued (no DMA in flight yet)
  uint4 Qf[16];
  load_qfrag32h<R>(q + (tok * kAH + 32 * ht + lo) * kAD, kb1 + (32 * ht + lo) * R, hi, kh, Qf);
  __syncthreads();  // kb1 is a gather target from the first chunk on

  if (c0 < c1) {
    Gather G;
    gather_prep(G, c0, kb0);
#pragma unroll
    for (int e = 0; e < 8; ++e) gather_row(G, e);
  }

  // O^T tiles of the wave's channel slice (channel tile ct, head tile hh):
  // lane (lo, hi) holds channels 128 wv + 32 ct + 8 (v / 4) + 4 hi + v % 4
  // of head 32 hh + lo
  f32x16 O[4][2];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int v = 0; v < 16; ++v) O[ct][hh][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // head 32 ht + lo: shared maximum, this wave's rows' sum
  const float sl2 = scale * kLog2e;
  const int ka = kh, kb = kh + 2;  // the 8-row groups of the tile this wave keeps

  // per-lane LDS byte offsets; the swizzle XOR only touches the low four
  // chunk bits, so each read is a base plus a lane mask XORed with a
  // compile-time step.  K fragment of step s = 8 u + s8 (A operand): row
  // kr = lo ^ 8 kh, 16-byte chunk 32 kh + 16 u + 2 s8 + hi, i.e.
  // kq_b + ((s8 << 5) ^ kq_x) + 256 u.  V^T fragment of channel tile ct, row
  // step ks, half h2 (transpose read): the address lane a = 4 j + q of
  // 16-lane group (sub, hi) names row 16 ks + 8 hi + 4 h2 + j and channels
  // 32 ct + 16 sub + 4 q .. +3 of the wave's slice, i.e.
  // tv_b + 4096 h2 + 16384 ks + ((ct << 6) ^ tv_x ^ (h2 << 6)); lane a
  // receives channel 16 sub + a of the tile for rows j = 0..3.
  int kq_b, kq_x, tv_b, tv_x;
  {
    const int kr = lo ^ (8 * kh), kz = swz(kr);
    kq_b = kr * 1024 + 512 * kh + 16 * (hi ^ (kz & 1));
    kq_x = (kz >> 1) << 5;
    const int sub = (lane >> 4) & 1, i16 = lane & 15, j = i16 >> 2, q4 = i16 & 3;
    const int x = 2 * sub + (q4 >> 1);  // chunk bits 0..1 before the swizzle
    // row 8 hi + j (h2 = 0): swizzle 8 hi + j, so bits 2..3 flip by 2 hi
    tv_b = (8 * hi + j) * 1024 + 256 * wv + 16 * (x ^ j) + (q4 & 1) * 8;
    tv_x = (2 * hi) << 6;
  }

  auto chunk = [&](int c, const bf16_t* cur, int cn, bf16_t* nxt) {
    // opaque copies of the offset bases and of the lane id: the per-lane
    // LDS addresses are loop invariant, and hoisted out of the loop they
    // would each hold a VGPR for its whole length (about 40 of them)
    int kqb, kqx, tvb, tvx, ln;
    asm volatile(
        "v_mov_b32 %0, %5\n\tv_mov_b32 %1, %6\n\tv_mov_b32 %2, %7\n\tv_mov_b32 %3, %8\n\t"
        "v_mov_b32 %4, %9"
        : "=v"(kqb), "=v"(kqx), "=v"(tvb), "=v"(tvx), "=v"(ln)
        : "v"(kq_b), "v"(kq_x), "v"(tv_b), "v"(tv_x), "v"(lane));
    const int lo = ln & 31, hi = ln >> 5;
    const char* kbp = (const char*)cur;
    // read before this chunk's gather is issued (no DMA in flight yet)
    // bits b and 16 + b: kept rows 8 ka + 4 hi + b and 8 kb + 4 hi + b
    const uint32_t vmk = vmask[c - c0] >> (4 * hi + 8 * ka);
    // The next chunk's rows are gathered during QK^T.  After the last chunk
    // the gather still runs (into the idle buffer): a gather under a branch
    // would make the compiler wait for every LDS read in flight where the
    // branches join.
    Gather G;
    gather_prep(G, cn, nxt);
    // ---- partial S^T = K Q^T: rows 0 .. 31 x heads 32 ht .. +31 over the
    // channel half kh
    f32x16 S;
#pragma unroll
    for (int v = 0; v < 16; ++v) S[v] = 0.f;
    auto kfrag = [&](int s) {
      return *(const uint4*)(kbp + kqb + (((s & 7) << 5) ^ kqx) + (s >> 3) * 256);
    };
    uint4 kf[kHQD];
#pragma unroll
    for (int j = 0; j < kHQD; ++j) kf[j] = kfrag(j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      S = mfma32(kf[s % kHQD], Qf[s], S);
      if (s + kHQD < 16) kf[s % kHQD] = kfrag(s + kHQD);
      if (s & 1) gather_row(G, s >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- the partner wave (other channel half) gets the row groups this
    // wave gives away; lane (lo, hi) of S holds rows 8 (g ^ kh) + 4 hi + b
    // (v = 4 g + b) of head 32 ht + lo: groups 0 and 2 kept (rows of 8-row
    // groups kh and kh + 2), 1 and 3 given
    lds_st2x128_mfma<1024>(xp + wv * 2048 + ln * 16, f32x4{S[4], S[5], S[6], S[7]},
                           f32x4{S[12], S[13], S[14], S[15]});
    lds_barrier();
    f32x4 pa, pb;
    lds_ld_2x128<1024>(xp + (wv ^ 2) * 2048 + ln * 16, pa, pb);
    // ---- softmax (log2 domain) over the kept rows 8 ka + 4 hi + b and
    // 8 kb + 4 hi + b of head 32 ht + lo
    float sv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int bq = j & 3;
      const float full = S[j < 4 ? bq : 8 + bq] + (j < 4 ? pa[bq] : pb[bq]);
      sv[j] = (vmk >> (j < 4 ? bq : 16 + bq)) & 1u ? full * sl2 : -INFINITY;
      mx = fmaxf(mx, sv[j]);
    }
    mx = xmax32(mx);
    // P with the running maximum of the earlier chunks.  A kept row above it
    // by more than 2^8 (always in a split's first chunk) sends every wave
    // through the second pass below, which takes the decision of the lazy
    // rescale on the pair's combined maximum and rewrites P: the result is
    // the same as exchanging the maxima up front, without that barrier in
    // the common case.
    const bool need = __any(mx > m_run + kLazy);
    if (hi == 0) lds_st32(&cmx[wv][lo], __float_as_uint(mx));
    if (ln == 0) lds_st32(&flg[wv], need ? 1u : 0u);
    bf16_t* prow = ps + (32 * ht + lo) * kHPRow + 4 * hi;
    auto write_p = [&]() {
      float psum = 0.f;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float p[4];
#pragma unroll
        for (int bq = 0; bq < 4; ++bq) {
          // exp2(-inf) = 0 for masked rows; m_run is finite once a row was seen
          p[bq] = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[4 * g + bq] - m_run);
          psum += p[bq];
        }
        lds_st64(prow + 8 * (g == 0 ? ka : kb), pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
      }
      return psum;
    };
    const float l_prev = l_run;
    l_run += write_p();
    if (kh == 0 && hi == 0) lds_st32(&alph[32 * ht + lo], __float_as_uint(1.f));
    lds_barrier();
    {
      const u32x4 f4 = lds_ld128(flg);
      if ((f4[0] | f4[1] | f4[2] | f4[3]) != 0) {  // the same in every wave
        const float cmax = fmaxf(mx, __uint_as_float(lds_ld32(&cmx[wv ^ 2][lo])));
        if (__any(cmax > m_run + kLazy)) {  // the same in both waves of the head tile
          const float m_new = fmaxf(m_run, cmax);
          const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          l_run = l_prev * alpha + write_p();
          if (kh == 0 && hi == 0) lds_st32(&alph[32 * ht + lo], __float_as_uint(alpha));
        }
        lds_barrier();
      }
    }
    // ---- O^T += V^T P^T over the wave's channel slice, all 64 heads; P^T
    // fragment (head tile hh, row step ks): rows 16 ks + 8 hi .. +7 of head
    // 32 hh + lo
    uint4 Pf[2][2];
    uint32_t au[2];
    lds_ld_2x2x128_2x32<32 * kHPRow * 2, 32, 32 * 4>(ps + lo * kHPRow + 8 * hi, &alph[lo], Pf, au);
    {
      const float a0 = __uint_as_float(au[0]), a1 = __uint_as_float(au[1]);
      if (__any(a0 != 1.f || a1 != 1.f)) {  // a head whose maximum stayed has alpha exactly 1
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          O[ct][0] *= a0;
          O[ct][1] *= a1;
        }
      }
    }
    auto vfrag = [&](int ct, int ks) {
      const char* pa2 = kbp + tvb + ks * 16384;
      const v4s x0 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(pa2 + ((ct << 6) ^ tvx)));
      const v4s x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4s*)(pa2 + 4096 + ((ct << 6) ^ tvx ^ 64)));
      return make_uint4((uint32_t)(uint16_t)x0[0] | ((uint32_t)(uint16_t)x0[1] << 16),
                        (uint32_t)(uint16_t)x0[2] | ((uint32_t)(uint16_t)x0[3] << 16),
                        (uint32_t)(uint16_t)x1[0] | ((uint32_t)(uint16_t)x1[1] << 16),
                        (uint32_t)(uint16_t)x1[2] | ((uint32_t)(uint16_t)x1[3] << 16));
    };
    uint4 vf[2];
    vf[0] = vfrag(0, 0);
    vf[1] = vfrag(1, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < 8; ++st) {  // step st: row step st / 4, channel tile st % 4
      const int ks = st >> 2, ct = st & 3;
      const uint4 a = vf[st & 1];
      if (st + 2 < 8) vf[st & 1] = vfrag((st + 2) & 3, (st + 2) >> 2);
      O[ct][0] = mfma32(a, Pf[0][ks], O[ct][0]);
      O[ct][1] = mfma32(a, Pf[1][ks], O[ct][1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int c = c0; c < c1; c += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this chunk's rows are in LDS
    lds_barrier();
    chunk(c, kb0, c + 1, kb1);
    if (c + 1 < c1) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
      chunk(c + 1, kb1, c + 2, kb0);
    }
  }

  // ---- finalisation: per head the shared maximum and the two waves' sums
  l_run = xsum32(l_run);
  if (hi == 0) {
    lfin[wv][lo] = l_run;
    if (kh == 0) mfin[32 * ht + lo] = m_run;
  }
  __syncthreads();  // every wave is done with the chunk buffers (the dummy gather drained)
  if (nsplit == 1) {
    // the whole [64 heads][512] bf16 output, 16-byte chunk c of head row h at
    // slot c ^ (h & 15): heads 0..31 in kb0, 32..63 in kb1
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int head = 32 * hh + lo;
      const float mh = mfin[head], lh = lfin[hh][lo] + lfin[hh + 2][lo];
      const float sink = sinks ? sinks[head] * kLog2e : -INFINITY;
      const float M = fmaxf(mh, sink);
      const float f = __builtin_amdgcn_exp2f(mh - M);
      const float lt = lh * f + (sinks ? __builtin_amdgcn_exp2f(sink - M) : 0.f);
      const float inv = f / lt;
      char* ob = (hh == 0 ? (char*)kb0 : (char*)kb1) + lo * 1024;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int d = 128 * wv + 32 * ct + 8 * a + 4 * hi;
          float o[4];
#pragma unroll
          for (int bq = 0; bq < 4; ++bq) o[bq] = O[ct][hh][4 * a + bq] * inv;
#pragma unroll
          for (int bq = 0; bq < 4; bq += 2) {
            if (d + bq >= first) {  // pair (d + bq, d + bq + 1) rotated at -t
              const double2 cz = cs[(d + bq - first) >> 1];
              const float cf = (float)cz.x, sf = (float)cz.y;
              const float x0 = o[bq] * cf + o[bq + 1] * sf, x1 = o[bq + 1] * cf - o[bq] * sf;
              o[bq] = x0;
              o[bq + 1] = x1;
            }
          }
          *(uint2*)(ob + (((d >> 3) ^ (lo & 15)) << 4) + ((d & 7) << 1)) =
              make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        }
    }
    __syncthreads();
    bf16_t* orow = out + tok * kAH * kAD;
#pragma unroll 4
    for (int hq = 0; hq < 16; ++hq) {
      const int head = 16 * wv + hq;
      const char* ob = (head < 32 ? (const char*)kb0 : (const char*)kb1) + (head & 31) * 1024;
      const uint4 v = *(const uint4*)(ob + ((lane ^ (head & 15)) << 4));
      *(uint4*)(orow + head * kAD + 8 * lane) = v;
    }
  } else {
    float* pbase = part + (tok * nsplit + split) * kAH * kPart;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          *(f32x4*)(pbase + (32 * hh + lo) * kPart + 128 * wv + 32 * ct + 8 * a + 4 * hi) =
              f32x4{O[ct][hh][4 * a], O[ct][hh][4 * a + 1], O[ct][hh][4 * a + 2],
                    O[ct][hh][4 * a + 3]};
    if (tid < kAH) {
      float* pr = pbase + tid * kPart;
      const int h2 = tid >> 5, l2 = tid & 31;
      pr[kAD] = mfin[tid];
      pr[kAD + 1] = lfin[h2][l2] + lfin[h2 + 2][l2];
    }
  }
}

}  // namespace

hipError_t launch_attend_h32(const Layer& L, const Batch& bt, const void* q, const void* win,
                             int64_t win_cap, const void* pool, int64_t pool_cap,
                             const int32_t* idx, const float* sinks, void* out, void* ws, bool csa,
                             int ns, hipStream_t s) {
  dim3 grid(bt.n, bt.B, ns);
#define CSA_H32_LAUNCH(RR)                                                                   \
  attend_h32<RR><<<grid, 256, 0, s>>>((const bf16_t*)q, (const bf16_t*)win, win_cap,          \
                                      (const bf16_t*)pool, pool_cap, idx, L.k, sinks,         \
                                      (bf16_t*)out, (float*)ws, bt.pos0, bt.n, L.W, L.m,      \
                                      L.base, L.scale, ns, csa ? 1 : 0)
  switch (L.R) {
    case 16: CSA_H32_LAUNCH(16); break;
    case 32: CSA_H32_LAUNCH(32); break;
    case 64: CSA_H32_LAUNCH(64); break;
    default: CSA_H32_LAUNCH(128); break;
  }
#undef CSA_H32_LAUNCH
  return hipGetLastError();
}

}  // namespace csa
