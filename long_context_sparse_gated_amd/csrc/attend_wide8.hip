// Attention over the sliding window plus compressed rows, K = V, with sink,
// on 32 x 32 x 16 bf16 MFMA tiles with two waves per SIMD (H = 64, D = 512)
// [DeepSeek-V4 model page, sec. 2.3: shared K=V MQA over the sliding window
// and the compressed rows, sink (eq. 27), output rotation (eq. 26)].
//
// One block of eight waves per (token, row split), one block per CU, so each
// SIMD runs two waves and one wave's LDS waits, softmax and gather issue
// overlap the other's MFMAs.  Rows come in chunks of 64, gathered by LDS-DMA
// (one 1 KB row per wave instruction) into two 64 KB buffers; the next
// chunk's gather is issued during this chunk's QK^T.
//  * S^T = K Q^T: wave w scores rows 32 rt .. +31 (rt = w & 1) for heads
//    32 ht .. +31 (ht = (w >> 1) & 1) over channels 256 kh .. +255
//    (kh = w >> 2): 16 steps, two accumulators.  The two waves that differ
//    only in kh add their partial scores through LDS, each keeping half of
//    the tile's rows (row groups kh and kh + 2 of the four 8-row groups);
//  * the four waves of a head tile exchange their maxima per head; all take
//    the same lazy-rescale decision (the running maximum is raised only by
//    more than 2^8);
//  * P (64 rows x 64 heads, bf16) goes to LDS; O^T += V^T P^T: wave w
//    accumulates channels 64 w .. 64 w + 63 of all 64 heads (4 tiles, 64
//    float32 per lane, kept in AGPRs), V^T from the row-major K = V tile
//    through the LDS transpose read;
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
// Four 4-byte loads at a, a + O1, a + O2, a + O3 (byte offsets), complete on return.
template <int O1, int O2, int O3>
__device__ __forceinline__ void lds_ld_4x32(const void* a, uint32_t (&w)[4]) {
  static_assert(O1 < 65536 && O2 < 65536 && O3 < 65536, "immediate LDS offsets are 16-bit");
  asm volatile(
      "ds_read_b32 %0, %4\n\tds_read_b32 %1, %4 offset:%5\n\t"
      "ds_read_b32 %2, %4 offset:%6\n\tds_read_b32 %3, %4 offset:%7\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3])
      : "v"(lds_addr(a)), "i"(O1), "i"(O2), "i"(O3)
      : "memory");
}

constexpr int kOCh = 64;          // rows per chunk
constexpr int kOPRow = kOCh + 8;  // LDS row of P per head: 64 row slots + pad (bf16)
#ifndef CSA_W8_QD
#define CSA_W8_QD 4
#endif
constexpr int kOQD = CSA_W8_QD;  // K fragment reads ahead of their MFMAs

// Query fragments of head row qrow for the 32 x 32 x 16 B operand over the
// channel half kh: fragment s holds channels 256 kh + 16 s + 8 hi .. +7; the
// last R channels rotated at the query's position in float64 and rounded to
// bf16 once.
template <int R>
__device__ __forceinline__ void load_qfrag32h(const bf16_t* __restrict__ qrow, const double2* cs,
                                              int hi, int kh, uint4 (&Qf)[16]) {
  constexpr int first = kAD - R;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int d0 = 256 * kh + 16 * s + 8 * hi;
    uint4 v = *(const uint4*)(qrow + d0);
    if (d0 + 8 > first) {  // uniform per wave half
      uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int d = d0 + 2 * p;
        if (d >= first) {
          double a = bf16_to_f32((bf16_t)(w4[p] & 0xffffu));
          double bb = bf16_to_f32((bf16_t)(w4[p] >> 16));
          const double2 c = cs[(d - first) >> 1];
          rot64(a, bb, c.x, c.y);
          w4[p] = (uint32_t)f64_to_bf16(a) | ((uint32_t)f64_to_bf16(bb) << 16);
        }
      }
      v = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
    Qf[s] = v;
  }
}

// LDS byte offset of 16-byte chunk `ch` (0..63) of row r under the row swizzle.
__device__ __forceinline__ int swz_chunk(int r, int ch) {
  return r * 1024 + (((ch & ~15) | ((ch & 15) ^ swz(r))) << 4);
}

template <int R>
__global__ void __launch_bounds__(512, 1) attend_w8(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ win, int64_t win_cap,
    const bf16_t* __restrict__ pool, int64_t pool_cap, const int32_t* __restrict__ idx, int k,
    const float* __restrict__ sinks, bf16_t* __restrict__ out, float* __restrict__ part,
    const int64_t* __restrict__ pos0, int n_new, int W, int m, Rope base, float scale,
    int nsplit, int csa) {
  static_assert(R % 16 == 0 && R <= kMaxRope, "rope channels: multiple of 16, <= 128");
  __shared__ __attribute__((aligned(1024))) bf16_t kb0[kOCh * kAD];
  __shared__ __attribute__((aligned(1024))) bf16_t kb1[kOCh * kAD];
  __shared__ __attribute__((aligned(16))) uint64_t raddr[kMaxRows];  // byte address of each row
  // partial-score exchange (8 waves x 2 KB), reused for P once every wave
  // has read its partner's scores
  __shared__ __attribute__((aligned(16))) char xp[8 * 2048];
  __shared__ uint32_t vmask[kMaxRows / 32 + 2];
  __shared__ double2 cs[kMaxRope / 2];
  __shared__ float cmx[8][32];   // each wave's chunk maximum per head of its tile
  __shared__ float alph[kAH];    // this chunk's rescale of O per head
  __shared__ float lfin[8][32];  // each wave's running sum per head of its tile
  __shared__ float mfin[kAH];    // final running maximum per head
  static_assert(kAH * kOPRow * 2 <= (int)sizeof(xp), "P fits the exchange buffer");
  bf16_t* const ps = (bf16_t*)xp;  // P per head, row slots

  const int i = n_new - 1 - (int)blockIdx.x;  // longest rows first
  const int b = blockIdx.y, split = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, lo = lane & 31, hi = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: role selects stay uniform
  const int rt = wv & 1, ht = (wv >> 1) & 1, kh = wv >> 2;  // QK^T row tile, head tile, half
  const int64_t t = pos0[b] + i;
  const int64_t tok = (int64_t)b * n_new + i;
  const int64_t wlo = t - W + 1 > 0 ? t - W + 1 : 0;
  const int nwin = (int)(t - wlo + 1);
  int64_t nvis = m > 0 ? (t + 1) / m : 0;
  if (nvis > pool_cap) nvis = pool_cap;
  const int npool = csa ? (int)(nvis < k ? nvis : k) : (int)nvis;
  const int nrows = nwin + npool;
  const int nch = (nrows + kOCh - 1) / kOCh;
  const int cps = (nch + nsplit - 1) / nsplit;
  const int c0 = min(nch, split * cps), c1 = min(nch, c0 + cps);
  const int r0 = c0 * kOCh, r1 = min(nrows, c1 * kOCh);
  const int32_t* idx_row = csa ? idx + tok * k : nullptr;

  for (int j = tid; j < R / 2; j += 512) {
    double sn, c;
    sincos((double)t * rope_freq(base, j, R), &sn, &c);
    cs[j] = make_double2(c, sn);
  }
  // the global address of every row (a masked row reads the query's own
  // window row, finite and never weighted), computed once so that a gather
  // issue is a handful of instructions; bits of vmask[2 (c - c0)],
  // [2 (c - c0) + 1]: rows of chunk c that take part
  {
    const bf16_t* self_row = win + ((int64_t)b * win_cap + t % win_cap) * kAD;
    for (int j0 = 64 * wv; j0 < r1 - r0; j0 += 512) {
      const int j = j0 + lane;
      const int id = j < r1 - r0 ? row_id(r0 + j, nwin, wlo, win_cap, b, pool_cap, idx_row, csa, nvis)
                                 : -1;
      const bf16_t* rp = id >= 0 ? win + (int64_t)id * kAD
                                 : (id == -1 ? self_row : pool + (int64_t)(-2 - id) * kAD);
      raddr[j] = (uint64_t)(size_t)rp;
      const unsigned long long bal = __ballot(id != -1);
      if (lane == 0) {
        vmask[j0 >> 5] = (uint32_t)bal;
        vmask[(j0 >> 5) + 1] = (uint32_t)(bal >> 32);
      }
    }
  }
  __syncthreads();

  // gather of chunk c into dst: this wave moves rows 8 wv .. 8 wv + 7 (one
  // 1 KB row per DMA instruction); lane e < 8 reads row e's address and the
  // addresses are made scalar, the lane id is copied opaquely and the wave
  // index made scalar so nothing here is spilled (a scratch reload would
  // wait on every DMA in flight)
  struct Gather {
    uint64_t a[8];
    int ln, wvs;
    bf16_t* dst;
  };
  auto gather_prep = [&](Gather& G, int c, bf16_t* dst) {
    asm volatile("v_mov_b32 %0, %1" : "=v"(G.ln) : "v"(lane));
    G.wvs = __builtin_amdgcn_readfirstlane(wv);
    G.dst = dst;
    // past the last chunk (a dummy gather, see chunk()) read chunk c0's rows
    const int base_r = (c < c1 ? c - c0 : 0) * kOCh + 8 * G.wvs;
    const uint64_t mine = raddr[base_r + (lane & 7)];
    // readlane returns int: widen through uint32_t so that a low word with
    // bit 31 set does not sign-extend into the high word
    const int lo32 = (int)(uint32_t)mine, hi32 = (int)(uint32_t)(mine >> 32);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      G.a[e] = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(hi32, e) << 32) |
               (uint32_t)__builtin_amdgcn_readlane(lo32, e);
  };
  auto gather_row = [&](const Gather& G, int e) {
    const int rr = 8 * G.wvs + e;
    const char* src = (const char*)(size_t)G.a[e] + 16 * (G.ln ^ swz(rr));
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(G.dst + rr * kAD), 16, 0, 0);
  };
  if (c0 < c1) {
    Gather G;
    gather_prep(G, c0, kb0);
#pragma unroll
    for (int e = 0; e < 8; ++e) gather_row(G, e);
  }

  // rotated queries of head 32 ht + lo, channels 256 kh + 16 s + 8 hi .. +7
  uint4 Qf[16];
  load_qfrag32h<R>(q + (tok * kAH + 32 * ht + lo) * kAD, cs, hi, kh, Qf);

  // O^T tiles (channel tile ct of the wave's 64, head tile hh): lane holds
  // channels 64 wv + 32 ct + 8 (v / 4) + 4 hi + v % 4 of head 32 hh + lo
  f32x16 O[2][2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int v = 0; v < 16; ++v) O[ct][hh][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // head 32 ht + lo: shared maximum, this wave's rows' sum
  const float sl2 = scale * kLog2e;
  const int ka = kh, kb = kh + 2;  // the 8-row groups of the tile this wave keeps

  // per-lane LDS byte offsets.  K fragment of step s (A operand): row
  // 32 rt + lo, 16-byte chunk 32 kh + 2 s + hi: kq_v[s & 7] + (s >> 3) * 256.
  // V^T fragment of channel tile ct, row step ks, half h2 (transpose read):
  // the address lane a = 4 j + q of a 16-lane group names row
  // 16 ks + 8 hi + 4 h2 + j and channels 4 q .. 4 q + 3 of the group's 16;
  // lane a receives channel a of the 16 for rows j = 0..3:
  // tv_v[2 ct + h2] + ks * 16 KB.
  int kq_v[8], tv_v[4];
  {
    const int row = 32 * rt + lo;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) kq_v[s8] = swz_chunk(row, 32 * kh + 2 * s8 + hi);
    const int g16 = lane >> 4, sub = g16 & 1, i16 = lane & 15, j = i16 >> 2, q4 = i16 & 3;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int r = 8 * hi + 4 * h2 + j;
        tv_v[2 * ct + h2] = swz_chunk(r, 8 * wv + 4 * ct + 2 * sub + (q4 >> 1)) + (q4 & 1) * 8;
      }
  }

  auto chunk = [&](int c, const bf16_t* cur, int cn, bf16_t* nxt) {
    const char* kbp = (const char*)cur;
    // read before this chunk's gather is issued (no DMA in flight yet)
    const uint32_t vmw = vmask[2 * (c - c0) + rt];
    // The next chunk's rows are gathered during QK^T.  After the last chunk
    // the gather still runs (rows past r1 read the query's own window row
    // into the idle buffer): a gather under a branch would make the compiler
    // wait for every LDS read in flight where the branches join.
    Gather G;
    gather_prep(G, cn, nxt);
    // ---- partial S^T = K Q^T: rows 32 rt .. +31 x heads 32 ht .. +31 over
    // the channel half kh
    f32x16 S, S1;
#pragma unroll
    for (int v = 0; v < 16; ++v) S[v] = S1[v] = 0.f;
    auto kfrag = [&](int s) { return *(const uint4*)(kbp + kq_v[s & 7] + (s >> 3) * 256); };
    uint4 kf[kOQD];
#pragma unroll
    for (int j = 0; j < kOQD; ++j) kf[j] = kfrag(j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      if (s & 1) S1 = mfma32(kf[s % kOQD], Qf[s], S1);
      else S = mfma32(kf[s % kOQD], Qf[s], S);
      if (s + kOQD < 16) kf[s % kOQD] = kfrag(s + kOQD);
      if (s & 1) gather_row(G, s >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    S += S1;
    // ---- the partner wave (other channel half) gets the row groups this
    // wave gives away (1 - kh, 3 - kh) and sends those it keeps (kh, kh + 2);
    // lane (lo, hi) of S holds rows 8 a + 4 hi + b (v = 4 a + b) of head
    // 32 ht + lo.  Selects on kh keep every vector index compile time.
    float keep[8], give[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int g = j < 4 ? 0 : 2, bq = j & 3;  // group pair (g, g + 1)
      keep[j] = kh ? S[4 * (g + 1) + bq] : S[4 * g + bq];
      give[j] = kh ? S[4 * g + bq] : S[4 * (g + 1) + bq];
    }
    lds_st2x128_mfma<1024>(xp + wv * 2048 + lane * 16, f32x4{give[0], give[1], give[2], give[3]},
                           f32x4{give[4], give[5], give[6], give[7]});
    lds_barrier();
    f32x4 pa, pb;
    lds_ld_2x128<1024>(xp + (wv ^ 4) * 2048 + lane * 16, pa, pb);
    // ---- softmax (log2 domain) over the kept rows 8 ka + 4 hi + b and
    // 8 kb + 4 hi + b of head 32 ht + lo
    float sv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int a = j < 4 ? ka : kb, bq = j & 3;
      const float full = keep[j] + (j < 4 ? pa[bq] : pb[bq]);
      const int r = 8 * a + 4 * hi + bq;
      sv[j] = (vmw >> r) & 1u ? full * sl2 : -INFINITY;
      mx = fmaxf(mx, sv[j]);
    }
    mx = xmax32(mx);
    if (hi == 0) lds_st32(&cmx[wv][lo], __float_as_uint(mx));
    lds_barrier();
    float cmax;
    {
      // waves 2 ht, 2 ht + 1, 2 ht + 4, 2 ht + 5 (rows of 32 floats)
      uint32_t w4[4];
      lds_ld_4x32<128, 512, 640>(&cmx[2 * ht][lo], w4);
      cmax = fmaxf(fmaxf(__uint_as_float(w4[0]), __uint_as_float(w4[1])),
                   fmaxf(__uint_as_float(w4[2]), __uint_as_float(w4[3])));
    }
    float alpha = 1.f;
    if (__any(cmax > m_run + kLazy)) {  // the same decision in all four waves of the head tile
      const float m_new = fmaxf(m_run, cmax);
      alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
    }
    float psum = 0.f;
    bf16_t* prow = ps + (32 * ht + lo) * kOPRow + 32 * rt + 4 * hi;
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
    l_run += psum;
    if (rt == 0 && kh == 0 && hi == 0) lds_st32(&alph[32 * ht + lo], __float_as_uint(alpha));
    lds_barrier();
    // ---- O^T += V^T P^T over the wave's channel slice, all 64 heads
    uint4 Pf[2][4];
    uint32_t au[2];
    lds_ld_8x128_2x32<32 * kOPRow * 2, 32, 32 * 4>(ps + lo * kOPRow + 8 * hi, &alph[lo], Pf, au);
    {
      const float a0 = __uint_as_float(au[0]), a1 = __uint_as_float(au[1]);
      if (__any(a0 != 1.f || a1 != 1.f)) {  // a head whose maximum stayed has alpha exactly 1
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          O[ct][0] *= a0;
          O[ct][1] *= a1;
        }
      }
    }
    auto vfrag = [&](int ct, int ks) {
      const char* pa2 = kbp + ks * 16384;
      const v4s x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(pa2 + tv_v[2 * ct]));
      const v4s x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(pa2 + tv_v[2 * ct + 1]));
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
    for (int st = 0; st < 8; ++st) {  // step st: row step st / 2, channel tile st % 2
      const int ks = st >> 1, ct = st & 1;
      const uint4 a = vf[st & 1];
      if (st + 2 < 8) vf[st & 1] = vfrag((st + 2) & 1, (st + 2) >> 1);
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

  // ---- finalisation: per head the shared maximum and the four waves' sums
  l_run = xsum32(l_run);
  if (hi == 0) {
    lfin[wv][lo] = l_run;
    if (rt == 0 && kh == 0) mfin[32 * ht + lo] = m_run;
  }
  __syncthreads();  // every wave is done with the chunk buffers (the dummy gather drained)
  constexpr int first = kAD - R;
  float mh[2], lh[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    mh[hh] = mfin[32 * hh + lo];
    lh[hh] = (lfin[2 * hh][lo] + lfin[2 * hh + 1][lo]) + (lfin[2 * hh + 4][lo] + lfin[2 * hh + 5][lo]);
  }
  if (nsplit == 1) {
    // 64 bf16 rows staged in kb0; 16-byte chunk c of head row h at slot c ^ (h & 15)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int head = 32 * hh + lo;
      const float sink = sinks ? sinks[head] * kLog2e : -INFINITY;
      const float M = fmaxf(mh[hh], sink);
      const float f = __builtin_amdgcn_exp2f(mh[hh] - M);
      const float lt = lh[hh] * f + (sinks ? __builtin_amdgcn_exp2f(sink - M) : 0.f);
      const float inv = f / lt;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int d = 64 * wv + 32 * ct + 8 * a + 4 * hi;
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
          char* rowb = (char*)kb0 + head * 1024;
          *(uint2*)(rowb + (((d >> 3) ^ (head & 15)) << 4) + ((d & 7) << 1)) =
              make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        }
    }
    __syncthreads();
    bf16_t* orow = out + tok * kAH * kAD;
#pragma unroll 4
    for (int hq = 0; hq < 8; ++hq) {
      const int head = 8 * wv + hq;
      const uint4 v = *(const uint4*)((const char*)kb0 + head * 1024 + ((lane ^ (head & 15)) << 4));
      *(uint4*)(orow + head * kAD + 8 * lane) = v;
    }
  } else {
    // float32 partial rows (2 KB per head) staged in kb0 (heads 0..31) and
    // kb1 (32..63); 16-byte chunk c of head row h at slot c ^ (h & 15)
    float* pbase = part + (tok * nsplit + split) * kAH * kPart;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      char* bufh = hh == 0 ? (char*)kb0 : (char*)kb1;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int ch = 16 * wv + 8 * ct + 2 * a + hi;  // 16-byte chunk of the 512-float row
          f32x4 v4;
#pragma unroll
          for (int bq = 0; bq < 4; ++bq) v4[bq] = O[ct][hh][4 * a + bq];
          *(f32x4*)(bufh + lo * 2048 + ((ch ^ (lo & 15)) << 4)) = v4;
        }
    }
    __syncthreads();
#pragma unroll 4
    for (int hq = 0; hq < 8; ++hq) {
      const int head = 8 * wv + hq;
      const char* bufh = head < 32 ? (const char*)kb0 : (const char*)kb1;
      const int hr = head & 31;
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int ch = lane + 64 * it;
        *(f32x4*)(pbase + head * kPart + 4 * ch) =
            *(const f32x4*)(bufh + hr * 2048 + ((ch ^ (hr & 15)) << 4));
      }
    }
    if (tid < kAH) {
      float* pr = pbase + tid * kPart;
      const int h2 = tid >> 5, l2 = tid & 31;
      pr[kAD] = mfin[tid];
      pr[kAD + 1] = (lfin[2 * h2][l2] + lfin[2 * h2 + 1][l2]) + (lfin[2 * h2 + 4][l2] + lfin[2 * h2 + 5][l2]);
    }
  }
}

}  // namespace

hipError_t launch_attend_w8(const Layer& L, const Batch& bt, const void* q, const void* win,
                            int64_t win_cap, const void* pool, int64_t pool_cap,
                            const int32_t* idx, const float* sinks, void* out, void* ws, bool csa,
                            int ns, hipStream_t s) {
  dim3 grid(bt.n, bt.B, ns);
#define CSA_W8_LAUNCH(RR)                                                                    \
  attend_w8<RR><<<grid, 512, 0, s>>>((const bf16_t*)q, (const bf16_t*)win, win_cap,           \
                                     (const bf16_t*)pool, pool_cap, idx, L.k, sinks,          \
                                     (bf16_t*)out, (float*)ws, bt.pos0, bt.n, L.W, L.m,       \
                                     L.base, L.scale, ns, csa ? 1 : 0)
  switch (L.R) {
    case 16: CSA_W8_LAUNCH(16); break;
    case 32: CSA_W8_LAUNCH(32); break;
    case 64: CSA_W8_LAUNCH(64); break;
    default: CSA_W8_LAUNCH(128); break;
  }
#undef CSA_W8_LAUNCH
  return hipGetLastError();
}

}  // namespace csa
