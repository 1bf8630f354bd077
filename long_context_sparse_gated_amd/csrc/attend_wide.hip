// Attention over the sliding window plus compressed rows, K = V, with sink,
// on 32 x 32 x 16 bf16 MFMA tiles (H = 64, D = 512) [DeepSeek-V4 model page,
// sec. 2.3: shared K=V MQA over the sliding window and the compressed rows,
// sink (eq. 27), output rotation (eq. 26)].
//
// On gfx950 the 32 x 32 x 16 bf16 MFMA sustains about twice the rate of the
// 16 x 16 x 32 one (measured: 2.45 against 1.41 PFLOP/s), so this kernel
// computes on 32 x 32 tiles.  One block of four waves per (token, row split),
// one block per CU; rows come in chunks of 64:
//  * S^T = K Q^T: wave w scores rows 32 (w & 1) .. +31 of the chunk for heads
//    32 (w >> 1) .. +31 (K rows as the A operand from LDS, the rotated
//    queries as the B operand in VGPRs, 32 steps over the 512 channels);
//  * the two waves sharing a head tile exchange their maxima per head through
//    LDS; both take the same lazy-rescale decision (the running maximum is
//    raised only by more than 2^8);
//  * P (64 rows x 64 heads, bf16) goes to LDS; O^T += V^T P^T: wave w
//    accumulates channels 128 w .. 128 w + 127 of all 64 heads (8 tiles, 128
//    float32 per lane), V^T from the row-major K = V tile through the LDS
//    transpose read;
//  * rows are gathered by LDS-DMA (one 1 KB row per wave instruction) into
//    two 64 KB buffers; the next chunk's gather is issued during this chunk's
//    QK^T and stays in flight across the chunk: barriers inside a chunk only
//    wait for LDS writes (lds_barrier), and the small control arrays are
//    accessed through lds_* so that the compiler does not wait for the DMA;
//  * the sink is folded once at the end; the bf16 output (or the float32
//    partial of a row split) is staged through LDS and written in whole rows.
#include "csa_device.h"
#include "csa_internal.h"
#include "attend_common.h"

namespace csa {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}


// x *= s for an accumulator tile kept in AGPRs, element by element in place
// (a plain C++ multiply makes the compiler copy every tile out of the AGPRs
// and back at each chunk, rescale or not).  The trailing nops keep the next
// MFMA from reading an AGPR the moment it is written.
__device__ __forceinline__ void scale_acc(f32x16& o, float s) {
  float x[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) x[v] = o[v];
  float t0, t1, t2, t3;
#define CSA_SC4(A, B, C, D)                                                         \
  "v_accvgpr_read_b32 %16, " A "\n\tv_accvgpr_read_b32 %17, " B "\n\t"             \
  "v_accvgpr_read_b32 %18, " C "\n\tv_accvgpr_read_b32 %19, " D "\n\t"             \
  "v_mul_f32 %16, %16, %20\n\tv_mul_f32 %17, %17, %20\n\t"                         \
  "v_mul_f32 %18, %18, %20\n\tv_mul_f32 %19, %19, %20\n\t"                         \
  "v_accvgpr_write_b32 " A ", %16\n\tv_accvgpr_write_b32 " B ", %17\n\t"           \
  "v_accvgpr_write_b32 " C ", %18\n\tv_accvgpr_write_b32 " D ", %19\n\t"
  asm volatile(CSA_SC4("%0", "%1", "%2", "%3") CSA_SC4("%4", "%5", "%6", "%7")
                   CSA_SC4("%8", "%9", "%10", "%11") CSA_SC4("%12", "%13", "%14", "%15")
               "s_nop 7\n\ts_nop 7\n\ts_nop 3"
               : "+a"(x[0]), "+a"(x[1]), "+a"(x[2]), "+a"(x[3]), "+a"(x[4]), "+a"(x[5]),
                 "+a"(x[6]), "+a"(x[7]), "+a"(x[8]), "+a"(x[9]), "+a"(x[10]), "+a"(x[11]),
                 "+a"(x[12]), "+a"(x[13]), "+a"(x[14]), "+a"(x[15]), "=&v"(t0), "=&v"(t1),
                 "=&v"(t2), "=&v"(t3)
               : "v"(s));
#undef CSA_SC4
#pragma unroll
  for (int v = 0; v < 16; ++v) o[v] = x[v];
}

constexpr int kWCh = 64;          // rows per chunk
constexpr int kWPRow = kWCh + 8;  // LDS row of P per head: 64 row slots + pad (bf16)
#ifndef CSA_WIDE_QD
#define CSA_WIDE_QD 8
#endif
constexpr int kWQD = CSA_WIDE_QD;  // K fragment reads ahead of their MFMAs

// Query fragments of head row qrow for the 32 x 32 x 16 B operand: fragment s
// holds channels 16 s + 8 hi .. +7; the last R channels rotated at the
// query's position in float64 and rounded to bf16 once.
template <int R>
__device__ __forceinline__ void load_qfrag32(const bf16_t* __restrict__ qrow, const double2* cs,
                                             int hi, uint4 (&Qf)[32]) {
  constexpr int first = kAD - R;
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    const int d0 = 16 * s + 8 * hi;
    uint4 v = *(const uint4*)(qrow + d0);
    if (16 * s + 16 > first && d0 + 8 > first) {  // first test is compile time
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

template <int R>
__global__ void __launch_bounds__(256, 1) attend_x32(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ win, int64_t win_cap,
    const bf16_t* __restrict__ pool, int64_t pool_cap, const int32_t* __restrict__ idx, int k,
    const float* __restrict__ sinks, bf16_t* __restrict__ out, float* __restrict__ part,
    const int64_t* __restrict__ pos0, int n_new, int W, int m, Rope base, float scale,
    int nsplit, int csa) {
  static_assert(R % 16 == 0 && R <= kMaxRope, "rope channels: multiple of 16, <= 128");
  __shared__ __attribute__((aligned(1024))) bf16_t kb0[kWCh * kAD];
  __shared__ __attribute__((aligned(1024))) bf16_t kb1[kWCh * kAD];
  __shared__ __attribute__((aligned(16))) uint64_t raddr[kMaxRows];  // byte address of each row
  __shared__ uint32_t vmask[kMaxRows / 32 + 2];
  __shared__ double2 cs[kMaxRope / 2];
  __shared__ __attribute__((aligned(16))) bf16_t ps[kAH * kWPRow];  // P per head, row slots
  __shared__ float cmx[4][32];   // each wave's chunk maximum per head of its tile
  __shared__ float alph[kAH];    // this chunk's rescale of O per head
  __shared__ float lfin[4][32];  // each wave's running sum per head of its tile
  __shared__ float mfin[kAH];    // final running maximum per head

  const int i = n_new - 1 - (int)blockIdx.x;  // longest rows first
  const int b = blockIdx.y, split = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, lo = lane & 31, hi = lane >> 5;
  const int rt = wv & 1, ht = wv >> 1;  // QK^T row tile and head tile of this wave
  const int64_t t = pos0[b] + i;
  const int64_t tok = (int64_t)b * n_new + i;
  const int64_t wlo = t - W + 1 > 0 ? t - W + 1 : 0;
  const int nwin = (int)(t - wlo + 1);
  int64_t nvis = m > 0 ? (t + 1) / m : 0;
  if (nvis > pool_cap) nvis = pool_cap;
  const int npool = csa ? (int)(nvis < k ? nvis : k) : (int)nvis;
  const int nrows = nwin + npool;
  const int nch = (nrows + kWCh - 1) / kWCh;
  const int cps = (nch + nsplit - 1) / nsplit;
  const int c0 = min(nch, split * cps), c1 = min(nch, c0 + cps);
  const int r0 = c0 * kWCh, r1 = min(nrows, c1 * kWCh);
  const int32_t* idx_row = csa ? idx + tok * k : nullptr;

  for (int j = tid; j < R / 2; j += 256) {
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
    for (int j0 = 64 * wv; j0 < r1 - r0; j0 += 256) {
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

  // gather of chunk c into dst: this wave moves rows 16 wv .. 16 wv + 15 (one
  // 1 KB row per DMA instruction); the row addresses are read in one go and
  // made scalar, the lane id is copied opaquely and the wave index made
  // scalar so nothing here is spilled (a scratch reload would wait on every
  // DMA in flight)
  struct Gather {
    uint64_t a[16];
    int ln, wvs;
    bf16_t* dst;
  };
  auto gather_prep = [&](Gather& G, int c, bf16_t* dst) {
    asm volatile("v_mov_b32 %0, %1" : "=v"(G.ln) : "v"(lane));
    G.wvs = __builtin_amdgcn_readfirstlane(wv);
    G.dst = dst;
    // past the last chunk (a dummy gather, see chunk()) read chunk c0's rows;
    // lane e < 16 reads row e's address, one LDS read per wave
    const int base_r = (c < c1 ? c - c0 : 0) * kWCh + 16 * G.wvs;
    const uint64_t mine = raddr[base_r + (lane & 15)];
    const int lo32 = (int)(uint32_t)mine, hi32 = (int)(uint32_t)(mine >> 32);
#pragma unroll
    for (int e = 0; e < 16; ++e)
      G.a[e] = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(hi32, e) << 32) |
               (uint32_t)__builtin_amdgcn_readlane(lo32, e);
  };
  auto gather_row = [&](const Gather& G, int e) {
    const int rr = 16 * G.wvs + e;
    const char* src = (const char*)(size_t)G.a[e] + 16 * (G.ln ^ e);  // swz(rr) == e
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(G.dst + rr * kAD), 16, 0, 0);
  };
  if (c0 < c1) {
    Gather G;
    gather_prep(G, c0, kb0);
#pragma unroll
    for (int e = 0; e < 16; ++e) gather_row(G, e);
  }

  // rotated queries of head 32 ht + lo, channels 16 s + 8 hi .. +7
  uint4 Qf[32];
  load_qfrag32<R>(q + (tok * kAH + 32 * ht + lo) * kAD, cs, hi, Qf);

  // O^T tiles (channel tile ct of the wave's 128, head tile hh): lane holds
  // channels 128 wv + 32 ct + 8 (v / 4) + 4 hi + v % 4 of head 32 hh + lo
  f32x16 O[4][2];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int v = 0; v < 16; ++v) O[ct][hh][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // head 32 ht + lo: shared maximum, this wave's rows' sum
  const float sl2 = scale * kLog2e;

  // per-lane LDS byte offsets.  K fragment of step s (A operand): row
  // 32 rt + lo, 16-byte chunk 2 s + hi at slot chunk ^ (row & 15):
  // kq_v[s & 7] + (s >> 3) * 256.  V^T fragment of channel tile ct, row step
  // ks, half h2 (transpose read): the address lane a = 4 j + q of a 16-lane
  // group names row 16 ks + 8 hi + 4 h2 + j and channels 4 q .. 4 q + 3 of
  // the group's 16; lane a receives channel a of the 16 for rows j = 0..3:
  // tv_v[2 ct + h2] + ks * 16 KB.
  int kq_v[8], tv_v[8];
  {
    const int row = 32 * rt + lo;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) kq_v[s8] = row * 1024 + (((2 * s8 + hi) ^ swz(row)) << 4);
    const int g16 = lane >> 4, sub = g16 & 1, i16 = lane & 15, j = i16 >> 2, q4 = i16 & 3;
    const int hh16 = g16 >> 1;  // == hi
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int r = 8 * hh16 + 4 * h2 + j;
        tv_v[2 * ct + h2] =
            r * 1024 + (((4 * ct + 2 * sub + (q4 >> 1)) ^ swz(r)) << 4) + (q4 & 1) * 8 + 256 * wv;
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
    // ---- S^T = K Q^T: rows 32 rt .. +31 x heads 32 ht .. +31
    f32x16 S, S1;
#pragma unroll
    for (int v = 0; v < 16; ++v) S[v] = S1[v] = 0.f;
    auto kfrag = [&](int s) {
      return *(const uint4*)(kbp + kq_v[s & 7] + (s >> 3) * 256);
    };
    uint4 kf[kWQD];
#pragma unroll
    for (int j = 0; j < kWQD; ++j) kf[j] = kfrag(j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      if (s & 1) S1 = mfma32(kf[s % kWQD], Qf[s], S1);
      else S = mfma32(kf[s % kWQD], Qf[s], S);
      if (s + kWQD < 32) kf[s % kWQD] = kfrag(s + kWQD);
      if (s & 1) gather_row(G, s >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- softmax (log2 domain); lane (lo, hi): rows 32 rt + 8 a + 4 hi + b
    // (v = 4 a + b) of head 32 ht + lo
    S += S1;
    float sv[16];
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 8 * (v >> 2) + 4 * hi + (v & 3);
      sv[v] = (vmw >> r) & 1u ? S[v] * sl2 : -INFINITY;
      mx = fmaxf(mx, sv[v]);
    }
    mx = xmax32(mx);
    if (hi == 0) lds_st32(&cmx[wv][lo], __float_as_uint(mx));
    lds_barrier();
    const float cmax = fmaxf(mx, __uint_as_float(lds_ld32(&cmx[wv ^ 1][lo])));
    float alpha = 1.f;
    if (__any(cmax > m_run + kLazy)) {  // the same decision in both waves of the head tile
      const float m_new = fmaxf(m_run, cmax);
      alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
    }
    float psum = 0.f;
    bf16_t* prow = ps + (32 * ht + lo) * kWPRow + 32 * rt + 4 * hi;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      float p[4];
#pragma unroll
      for (int bq = 0; bq < 4; ++bq) {
        // exp2(-inf) = 0 for masked rows; m_run is finite once a row was seen
        p[bq] = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[4 * a + bq] - m_run);
        psum += p[bq];
      }
      lds_st64(prow + 8 * a, pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
    }
    l_run += psum;
    if (rt == 0 && hi == 0) lds_st32(&alph[32 * ht + lo], __float_as_uint(alpha));
    lds_barrier();
    // ---- O^T += V^T P^T over the wave's channel slice, all 64 heads
    uint4 Pf[2][4];
    uint32_t au[2];
    lds_ld_8x128_2x32<32 * kWPRow * 2, 32, 32 * 4>(ps + lo * kWPRow + 8 * hi, &alph[lo], Pf, au);
    {
      const float a0 = __uint_as_float(au[0]), a1 = __uint_as_float(au[1]);
      if (__any(a0 != 1.f || a1 != 1.f)) {  // a head whose maximum stayed has alpha exactly 1
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          scale_acc(O[ct][0], a0);
          scale_acc(O[ct][1], a1);
        }
      }
    }
    auto vfrag = [&](int ct, int ks) {
      const char* pa = kbp + ks * 16384;
      const v4s x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(pa + tv_v[2 * ct]));
      const v4s x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(pa + tv_v[2 * ct + 1]));
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
    for (int st = 0; st < 16; ++st) {  // step st: row step st / 4, channel tile st % 4
      const int ks = st >> 2, ct = st & 3;
      const uint4 a = vf[st & 1];
      if (st + 2 < 16) vf[st & 1] = vfrag((st + 2) & 3, (st + 2) >> 2);
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
    if (rt == 0) mfin[32 * ht + lo] = m_run;
  }
  __syncthreads();  // every wave is done with the chunk buffers
  constexpr int first = kAD - R;
  float mh[2], lh[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    mh[hh] = mfin[32 * hh + lo];
    lh[hh] = lfin[2 * hh][lo] + lfin[2 * hh + 1][lo];
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
          char* rowb = (char*)kb0 + head * 1024;
          *(uint2*)(rowb + (((d >> 3) ^ (head & 15)) << 4) + ((d & 7) << 1)) =
              make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        }
    }
    __syncthreads();
    bf16_t* orow = out + tok * kAH * kAD;
#pragma unroll 4
    for (int hh = 0; hh < 16; ++hh) {
      const int head = 16 * wv + hh;
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
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int ch = 32 * wv + 8 * ct + 2 * a + hi;  // 16-byte chunk of the 512-float row
          f32x4 v4;
#pragma unroll
          for (int bq = 0; bq < 4; ++bq) v4[bq] = O[ct][hh][4 * a + bq];
          *(f32x4*)(bufh + lo * 2048 + ((ch ^ (lo & 15)) << 4)) = v4;
        }
    }
    __syncthreads();
#pragma unroll 4
    for (int hq = 0; hq < 16; ++hq) {
      const int head = 16 * wv + hq;
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
      pr[kAD] = mfin[tid];
      pr[kAD + 1] = lfin[2 * (tid >> 5)][tid & 31] + lfin[2 * (tid >> 5) + 1][tid & 31];
    }
  }
}

hipError_t launch_attend_x32(const Layer& L, const Batch& bt, const void* q, const void* win,
                             int64_t win_cap, const void* pool, int64_t pool_cap,
                             const int32_t* idx, const float* sinks, void* out, void* ws, bool csa,
                             int ns, hipStream_t s) {
  dim3 grid(bt.n, bt.B, ns);
#define CSA_X32_LAUNCH(RR)                                                                   \
  attend_x32<RR><<<grid, 256, 0, s>>>((const bf16_t*)q, (const bf16_t*)win, win_cap,          \
                                      (const bf16_t*)pool, pool_cap, idx, L.k, sinks,         \
                                      (bf16_t*)out, (float*)ws, bt.pos0, bt.n, L.W, L.m,      \
                                      L.base, L.scale, ns, csa ? 1 : 0)
  switch (L.R) {
    case 16: CSA_X32_LAUNCH(16); break;
    case 32: CSA_X32_LAUNCH(32); break;
    case 64: CSA_X32_LAUNCH(64); break;
    default: CSA_X32_LAUNCH(128); break;
  }
#undef CSA_X32_LAUNCH
  return hipGetLastError();
}

}  // namespace csa
