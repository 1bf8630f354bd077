// Attention over the sliding window plus compressed rows, K = V, with sink.
//
// For query t and head h the row list is the window positions
// max(0, t-W+1) .. t (ring slot = position mod cap) followed by the pooled
// rows: the top-k entries of t (CSA) or every visible entry w < (t+1)/m
// (HCA; none for sliding-only layers).  logits = scale * rot_t(q) . row; one
// softmax over all rows plus the unscaled sink logit of h; the output is the
// probability-weighted sum of the same rows, its rope slice rotated at -t
// [DeepSeek-V4 model page, sec. 2.3: shared K=V MQA, sliding branch
// concatenated with the compressor rows before the main attention, sink
// (eq. 27), output rotation (eq. 26); transformers PR 45616: sink from the
// GPT-OSS eager attention].
//
// attend_mfma (H = 64, D = 512, bf16) -- one block of four waves per
// (token, split).  The two products are divided differently among the waves:
//  * S^T = K Q^T by head groups: wave w scores heads 16w .. 16w+15; their
//    rotated queries live in VGPRs as the B operand (16 x 16 x 32 bf16
//    MFMA), so the softmax state of a lane column is one head, and P goes to
//    LDS (32 rows x 64 heads, bf16, 4 KB per chunk);
//  * O^T += V^T P^T by channel slices: wave w accumulates all 64 heads over
//    channels 128w .. 128w+127, so each V^T fragment read from LDS feeds four
//    MFMAs (one per head group) and the slow transpose reads drop fourfold;
//  * the K = V rows are gathered 32 at a time straight from HBM/L2 into LDS
//    by the LDS-DMA loads (one 1 KB row per wave instruction), double
//    buffered so the next chunk's gather overlaps this chunk's MFMAs.  Each
//    row is stored once, row-major; the V^T operand comes from the same bytes
//    through the LDS transpose read (ds_read_b64_tr_b16);
//  * 16-byte chunks of row r sit at a per-row XOR swizzle (swz below) so the
//    16-byte K reads run at the contiguous rate;
//  * the running max is only raised when a chunk exceeds it by more than 2^8
//    (P stays <= 256, exact to bf16 precision); a raise is published per head
//    so the channel-slice waves rescale their O columns;
//  * P is rounded to bf16 for the PV product; accumulation is float32;
//  * the sink enters once, at the end: (m, l) -> (max(m, s), l e^(m-M) +
//    e^(s-M)); with several splits the merge kernel does this instead;
//  * the bf16 output is staged through LDS and written as whole 1 KB rows.
// attend_generic: any H, D; float32 VALU; used for float32 layers and small
// shapes.
#include <cstdlib>

#include "csa_device.h"
#include "csa_internal.h"
#include "attend_common.h"

namespace csa {

constexpr int kPRow = kCH + 8;  // LDS row of P^T per head: 32 row slots + pad (bf16)
// Software-pipeline depth of the K fragment reads (steps ahead).
constexpr int kQD = 2;

typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma32x(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
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

template <int R>
__global__ void __launch_bounds__(256, CSA_ATTN_MIN_BLOCKS) attend_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ win, int64_t win_cap,
    const bf16_t* __restrict__ pool, int64_t pool_cap, const int32_t* __restrict__ idx, int k,
    const float* __restrict__ sinks, bf16_t* __restrict__ out, float* __restrict__ part, Seqs sq,
    int W, int m, Rope base, float scale, int nsplit, int csa) {
  static_assert(R % 16 == 0 && R <= kMaxRope, "rope channels: multiple of 16, <= 128");
  // two separate arrays (not one indexed by parity) so the compiler can tell
  // the DMA target from the tile being read and need not wait for the DMA
  __shared__ __attribute__((aligned(1024))) bf16_t kbuf0[kCH * kAD];
  __shared__ __attribute__((aligned(1024))) bf16_t kbuf1[kCH * kAD];
  __shared__ __attribute__((aligned(16))) int32_t rid[kMaxRows];
  __shared__ uint32_t vmask[kMaxRows / 32 + 1];
  __shared__ double2 cs[kMaxRope / 2];
  __shared__ __attribute__((aligned(16))) float2 csf[kMaxRope / 2];  // cs rounded to float
  __shared__ __attribute__((aligned(16))) bf16_t ps[kAH * kPRow];  // P^T, row slots per head
  __shared__ float alph[kAH];   // this chunk's rescale of O per head
  __shared__ float mlf[2][kAH];  // final running max and sum per head
  __shared__ float sinkl[kAH];   // sink logits (natural units)

  constexpr int NTH = 256;
  constexpr int RPW = kCH / 4;  // rows each wave gathers per chunk
  const int i = sq.n - 1 - (int)blockIdx.x;  // longest rows first
  const int b = blockIdx.y, split = blockIdx.z;
  if (i >= sq.len(b)) return;  // a padding row: left as it is
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int64_t t = sq.pos0[b] + i;
  const int64_t tok = sq.row(b, i);             // row of q, the ids and the output
  const int64_t slot = (int64_t)b * sq.n + i;   // slot of the split partials
  const int64_t lo = t - W + 1 > 0 ? t - W + 1 : 0;
  const int nwin = (int)(t - lo + 1);
  int64_t nvis = m > 0 ? (t + 1) / m : 0;
  if (nvis > pool_cap) nvis = pool_cap;
  const int npool = csa ? (int)(nvis < k ? nvis : k) : (int)nvis;
  const int nrows = nwin + npool;
  const int nch = (nrows + kCH - 1) / kCH;
  const int cps = (nch + nsplit - 1) / nsplit;
  const int c0 = split * cps, c1 = min(nch, c0 + cps);
  const int r0 = c0 * kCH, r1 = min(nrows, c1 * kCH);
  const int32_t* idx_row = csa ? idx + tok * k : nullptr;
  const int self_id = (int)((int64_t)b * win_cap + t % win_cap);  // always a valid row

  // the wave's query fragments (head 16*wv + r16, channels 32*kk + 8*g +
  // 0..7) start loading now; they are rotated once the rope table is in LDS
  constexpr int first = kAD - R;
  uint4 Qf[16];
  {
    const bf16_t* qrow = q + (tok * kAH + 16 * wv + r16) * kAD + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) Qf[kk] = *(const uint4*)(qrow + 32 * kk);
  }
  // the sink logit and every selected index of the thread's rows are loaded
  // next, so that all the prologue's loads share one memory latency (every
  // lane loads a sink, so that no branch holds a wait for it)
  const float sink_raw = sinks ? sinks[tid & (kAH - 1)] : 0.f;
  constexpr int U = kMaxRows / NTH;
  int32_t sel[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int e = r0 + tid + NTH * u - nwin;
    sel[u] = (csa && tid + NTH * u < r1 - r0 && e >= 0) ? idx_row[e] : 0;
  }
  // row ids: window row j is ring slot (lo + j) mod cap, and j < nwin <= cap
  // (the ring holds the window or the whole sequence) leaves one wrap at
  // most.  Bit r of vmask[c - c0]: row r of chunk c takes part in the
  // softmax; wave wv holds rows 256 u + 64 wv + lane, so one ballot per u
  // gives two whole words.
  {
    const int lo_mod = (int)(lo % win_cap), cap = (int)win_cap, wb = (int)((int64_t)b * win_cap);
    // pool rows of all the thread's entries first (with a block table these
    // are loads: all in flight at once; entries that are not visible pool
    // rows look up entry 0 and are not used)
    int64_t prw[U];
    bool vis[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jr = r0 + tid + NTH * u;
      const int64_t w = csa ? (int64_t)sel[u] : (int64_t)(jr - nwin);
      vis[u] = w >= 0 && w < nvis;
      prw[u] = sq.prow(b, vis[u] ? w : 0, pool_cap);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = tid + NTH * u;
      int id = -1;
      if (j < r1 - r0) {
        const int jr = r0 + j;
        if (jr < nwin) {
          const int v = lo_mod + jr;
          id = wb + (v >= cap ? v - cap : v);
        } else {
          id = vis[u] ? (int)(-2 - prw[u]) : -1;
        }
        rid[j] = id;
      }
      const unsigned long long bal = __ballot(id != -1);
      if (lane == 0) {
        const int j0 = NTH * u + 64 * wv;
        vmask[j0 >> 5] = (uint32_t)bal;
        vmask[(j0 >> 5) + 1] = (uint32_t)(bal >> 32);
      }
    }
  }
  if (tid < kAH) sinkl[tid] = sink_raw;  // scaled to log2 units at the end
  __syncthreads();

  // gather of chunk c into dst: this wave moves rows RPW*wv .. +RPW-1.
  // gather_prep loads the wave's row ids in one go (16-byte aligned; entries
  // past r1 are replaced below) so the DMA issues do not each wait on an LDS
  // read; gather_row(e) issues row e.  The per-row source offsets come from
  // an opaque copy of the lane id and the wave index is made scalar: hoisted
  // out of the loop these values would be spilled, and a scratch reload
  // waits on vmcnt, i.e. on every DMA issued before it.
  struct Gather {
    int ids[RPW];
    int ln, wvs, c;
    bf16_t* dst;
  };
  auto gather_prep = [&](Gather& G, int c, bf16_t* dst) {
    asm volatile("v_mov_b32 %0, %1" : "=v"(G.ln) : "v"(lane));
    G.wvs = __builtin_amdgcn_readfirstlane(wv);
    G.c = c;
    G.dst = dst;
    const int base_r = (c - c0) * kCH + RPW * G.wvs;
#pragma unroll
    for (int e = 0; e < RPW; e += 4) {
      const int4 v = *(const int4*)&rid[base_r + e];
      G.ids[e] = v.x;
      G.ids[e + 1] = v.y;
      G.ids[e + 2] = v.z;
      G.ids[e + 3] = v.w;
    }
  };
  auto gather_row = [&](const Gather& G, int e) {
    const int rr = RPW * G.wvs + e;
    const int jr = G.c * kCH + rr;
    int id = jr < r1 ? G.ids[e] : -1;
    if (id == -1) id = self_id;  // masked below; any finite row will do
    const bf16_t* src = id >= 0 ? win + (int64_t)id * kAD : pool + (int64_t)(-2 - id) * kAD;
    src += 8 * (G.ln ^ swz(rr));
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(G.dst + rr * kAD), 16, 0, 0);
  };
  auto issue = [&](int c, bf16_t* dst) {
    Gather G;
    gather_prep(G, c, dst);
#pragma unroll
    for (int e = 0; e < RPW; ++e) gather_row(G, e);
  };
  if (c0 < c1) issue(c0, kbuf0);

  // the rope table (float64 for the query, float32 for the output), computed
  // while the first chunk is in flight
  for (int j = tid; j < R / 2; j += NTH) {
    double sn, c;
    sincos((double)t * rope_freq(base, j, R), &sn, &c);
    cs[j] = make_double2(c, sn);
    csf[j] = make_float2((float)c, (float)sn);
  }
  __syncthreads();

  // the rope channels of the query fragments rotated at t in float64 and
  // rounded to bf16 once
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) {
    const int d0 = 32 * kk + 8 * g;
    if (32 * kk + 32 > first && d0 + 8 > first) {  // first test is compile time
      uint32_t w4[4] = {Qf[kk].x, Qf[kk].y, Qf[kk].z, Qf[kk].w};
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
      Qf[kk] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
  }

  // O^T tiles of the wave's channel slice (channel tile ct, head tile hh):
  // lane (l32, h32) holds channels 128*wv + 32*ct + 8*(v/4) + 4*h32 + v%4 of
  // head 32*hh + l32
  const int l32 = lane & 31, h32 = lane >> 5;
  f32x16 O[4][2];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int v = 0; v < 16; ++v) O[ct][hh][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // head 16*wv + r16
  const float sl2 = scale * kLog2e;

  // LDS byte offsets (constant per lane).  The swizzle only touches the low
  // four chunk bits, so every read is a per-lane base plus a compile-time
  // multiple of 256 bytes (16 chunks):
  //  * QK^T: row r16 (+16 for the second row tile), chunk 4kk + g; with
  //    kk = 4u + v the chunk is 16u + ((4v + g) ^ swz(r16)): bases kb_v[v];
  //  * transpose read: source lane s = r16 of group g supplies row 4g + s/4
  //    (+16 for the upper 4 rows) and channels 4 (s mod 4) .. +3 of the
  //    16-channel tile mt = 8u + v, i.e. chunk 16u + ((2v + (s mod 4)/2) ^
  //    swz(row)) plus 8 bytes for odd s: bases tr_v[v] (row + 16 adds 16 KB).
  //    The wave's slice is tiles mt = 8 wv + dt: base tr_v[dt] + 256 wv.
  int kb_v[4], tr_v[8];
#pragma unroll
  for (int v = 0; v < 4; ++v) kb_v[v] = r16 * 1024 + (((4 * v + g) ^ swz(r16)) << 4);
  // 32 x 32 x 16 V^T fragment of channel tile ct, row step ks, half h2: the
  // address lane a = 4 j + q of 16-lane group (sub, h32) names row
  // 16 ks + 8 h32 + 4 h2 + j and channels 32 ct + 16 sub + 4 q .. +3 of the
  // wave's slice; lane a receives channel 16 sub + a of the tile for rows
  // j = 0..3: tr_v[2 ct + h2] + ks * 16 KB
  {
    const int sub = g & 1, j4 = r16 >> 2, q4 = r16 & 3;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int r = 8 * h32 + 4 * h2 + j4;
        tr_v[2 * ct + h2] =
            r * 1024 + (((4 * ct + 2 * sub + (q4 >> 1)) ^ swz(r)) << 4) + (q4 & 1) * 8 + 256 * wv;
      }
  }

  auto chunk = [&](int c, const bf16_t* cur, int cn, bf16_t* nxt) {
    const char* kb = (const char*)cur;
    // read before this chunk's gather is issued (no DMA in flight yet)
    const uint32_t vm = vmask[c - c0] >> (4 * g);
    // the next chunk's gather (if any) is issued row by row between the
    // QK^T MFMAs below
    Gather G;
    const bool gat = cn < c1;
    if (gat) gather_prep(G, cn, nxt);
    // ---- S^T = K Q^T: 32 rows x the wave's 16 heads
    f32x4 S0 = (f32x4){0.f, 0.f, 0.f, 0.f}, S1 = S0;
    // swz(16*mt + r16) == swz(r16): the second row tile is 16 KB further
    auto kfrag = [&](int kk, int mt) {
      return *(const uint4*)(kb + kb_v[kk & 3] + (kk >> 2) * 256 + mt * 16384);
    };
    // K fragments are read kQD steps ahead of their MFMAs (an LDS read takes
    // longer than the two MFMAs of one step); the scheduling barriers keep
    // the compiler from sinking the reads next to their use
    uint4 kf[kQD][2];
#pragma unroll
    for (int j = 0; j < kQD; ++j) {
      kf[j][0] = kfrag(j, 0);
      kf[j][1] = kfrag(j, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      S0 = mfma16(kf[kk % kQD][0], Qf[kk], S0);
      S1 = mfma16(kf[kk % kQD][1], Qf[kk], S1);
      if (kk + kQD < 16) {
        kf[kk % kQD][0] = kfrag(kk + kQD, 0);
        kf[kk % kQD][1] = kfrag(kk + kQD, 1);
      }
      if (gat && (kk & 1) && (kk >> 1) < RPW) gather_row(G, kk >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- online softmax (log2 domain); lane column = head 16*wv + r16
    float sv[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      sv[ii] = (vm >> ii) & 1u ? S0[ii] * sl2 : -INFINITY;
      sv[4 + ii] = (vm >> (16 + ii)) & 1u ? S1[ii] * sl2 : -INFINITY;
      cmax = fmaxf(cmax, fmaxf(sv[ii], sv[4 + ii]));
    }
    cmax = xmax32(xmax16(cmax));
    const bool raise = __any(cmax > m_run + kLazy);
    float alpha = 1.f;
    if (raise) {
      const float m_new = fmaxf(m_run, cmax);
      alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
    }
    float psum = 0.f;
    uint32_t pk[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      // exp2(-inf) = 0 for masked rows; m_run is finite once a row was seen
      const float pa = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[j] - m_run);
      const float pb = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[j + 1] - m_run);
      psum += pa + pb;
      pk[j >> 1] = pack_bf16x2(pa, pb);
    }
    l_run += psum;
    // P^T slots of lane group g hold rows 4g..4g+3 and 16+4g..16+4g+3; the
    // next chunk's gather is in flight, so these LDS accesses and the
    // barrier go through lds_* (they must not wait for it)
    // rows in natural order: slots 4g..4g+3 and 16+4g..16+4g+3
    lds_st64(&ps[(16 * wv + r16) * kPRow + 4 * g], pk[0], pk[1]);
    lds_st64(&ps[(16 * wv + r16) * kPRow + 16 + 4 * g], pk[2], pk[3]);
    if (g == 0) lds_st32(&alph[16 * wv + r16], __float_as_uint(alpha));
    lds_barrier();

    // ---- O^T += V^T P^T over the wave's channel slice, all 64 heads
    // P^T fragment (head tile hh, row step ks): rows 16 ks + 8 h32 .. +7 of
    // head 32 hh + l32
    uint4 Pf[2][2];
    uint32_t a2u[2];
    lds_ld_2x2x128_2x32<32 * kPRow * 2, 32, 32 * 4>(&ps[l32 * kPRow + 8 * h32], &alph[l32], Pf,
                                                    a2u);
    {
      const float a0 = __uint_as_float(a2u[0]), a1 = __uint_as_float(a2u[1]);
      // a head whose maximum was not raised has alpha exactly 1
      if (__any(a0 != 1.f || a1 != 1.f)) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          O[ct][0] *= a0;
          O[ct][1] *= a1;
        }
      }
    }
    auto vfrag = [&](int ct, int ks) {
      const char* pa = kb + ks * 16384;
      const v4s x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(pa + tr_v[2 * ct]));
      const v4s x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(pa + tr_v[2 * ct + 1]));
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
      O[ct][0] = mfma32x(a, Pf[0][ks], O[ct][0]);
      O[ct][1] = mfma32x(a, Pf[1][ks], O[ct][1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int c = c0; c < c1; c += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this chunk's rows are in LDS
    lds_barrier();
    chunk(c, kbuf0, c + 1, kbuf1);
    if (c + 1 < c1) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
      chunk(c + 1, kbuf1, c + 2, kbuf0);
    }
  }

  l_run = xsum32(xsum16(l_run));
  if (g == 0) {
    mlf[0][16 * wv + r16] = m_run;
    mlf[1][16 * wv + r16] = l_run;
  }
  __syncthreads();  // every wave is done with kbuf; m, l of every head published

  if (nsplit == 1) {
    // the whole [64 heads][512] bf16 output, chunks swizzled by head: heads
    // 0..31 in kbuf0, 32..63 in kbuf1
    float iv[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int head = 32 * hh + l32;
      const float mh = mlf[0][head], lh = mlf[1][head];
      const float sink = sinks ? sinkl[head] * kLog2e : -INFINITY;
      const float M = fmaxf(mh, sink);
      const float f = __builtin_amdgcn_exp2f(mh - M);
      const float lt = lh * f + (sinks ? __builtin_amdgcn_exp2f(sink - M) : 0.f);
      iv[hh] = f / lt;
    }
    // the lane's channels d .. d + 3, d = 128 wv + 32 ct + 8 a + 4 h32.  The
    // rope slice (at most 128 channels, starting at a multiple of 16) lies in
    // wave 3's channels, and the 16 channels from 384 + 32 ct + 16 (a / 2)
    // on are all rope channels or none: for each (ct, a) the test is known
    // at compile time up to the wave index, which is uniform.  Every wave
    // reads the table entries wave 3 would use (unconditional reads issue
    // together instead of each waiting in a branch).
    static_assert(kAD - kMaxRope >= 384, "rope channels within wave 3's slice");
    const int wvs = __builtin_amdgcn_readfirstlane(wv);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = 128 * wvs + 32 * ct + 8 * a + 4 * h32;
        const bool rope_w3 = 384 + 32 * ct + 16 * (a >> 1) >= first;
        const bool rope = rope_w3 && wvs == 3;
        float4 cz = make_float4(1.f, 0.f, 1.f, 0.f);
        if (rope_w3)  // pairs (d, d+1), (d+2, d+3) of wave 3
          cz = *(const float4*)&csf[(384 + 32 * ct + 8 * a + 4 * h32 - first) >> 1];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int head = 32 * hh + l32;
          float o[4];
#pragma unroll
          for (int bq = 0; bq < 4; ++bq) o[bq] = O[ct][hh][4 * a + bq] * iv[hh];
          if (rope) {  // pairs rotated at -t
            const float x0 = o[0] * cz.x + o[1] * cz.y, x1 = o[1] * cz.x - o[0] * cz.y;
            const float x2 = o[2] * cz.z + o[3] * cz.w, x3 = o[3] * cz.z - o[2] * cz.w;
            o[0] = x0;
            o[1] = x1;
            o[2] = x2;
            o[3] = x3;
          }
          char* ob = (hh == 0 ? (char*)kbuf0 : (char*)kbuf1) + (head & 31) * 1024;
          *(uint2*)(ob + (((d >> 3) ^ (head & 15)) << 4) + ((d & 7) << 1)) =
              make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        }
      }
    __syncthreads();
    bf16_t* orow = out + tok * kAH * kAD;
#pragma unroll 4
    for (int hh = 0; hh < 16; ++hh) {
      const int head = 16 * wv + hh;
      const char* ob = (head < 32 ? (const char*)kbuf0 : (const char*)kbuf1) + (head & 31) * 1024;
      const uint4 v = *(const uint4*)(ob + ((lane ^ (head & 15)) << 4));
      *(uint4*)(orow + head * kAD + 8 * lane) = v;
    }
  } else {
    float* pbase = part + (slot * nsplit + split) * kAH * kPart;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          *(f32x4*)(pbase + (32 * hh + l32) * kPart + 128 * wv + 32 * ct + 8 * a + 4 * h32) =
              f32x4{O[ct][hh][4 * a], O[ct][hh][4 * a + 1], O[ct][hh][4 * a + 2],
                    O[ct][hh][4 * a + 3]};
    if (g == 0) {
      float* prow = pbase + (16 * wv + r16) * kPart;
      prow[kAD] = m_run;
      prow[kAD + 1] = l_run;
    }
  }
}

// Merge of split partials (m in log2 units, l, unnormalised O) with the sink,
// then the -t rotation of the rope slice and the store.  One block of four
// waves per (token, head), wave q merging channels 128 q .. 128 q + 127
// (two per lane): lane s first reads split s's (m, l), then every lane sums
// its two channels over all splits, sixteen splits' loads in flight at a
// time.  (One wave per (token, head) over all 512 channels kept a quarter
// of the CUs busy for the four tokens of a long-context decode step, with
// 16 KB in flight per wave.)
constexpr int kMergeQ = 4;  // waves (channel quarters) per merge block

__global__ void __launch_bounds__(64 * kMergeQ) attend_merge(
    const float* __restrict__ part, const float* __restrict__ sinks, bf16_t* __restrict__ out,
    Seqs sq, int R, Rope base, int nsplit) {
  __shared__ double2 cs[kAD / 2];
  __shared__ float fs[kMergeQ][kMaxSplits];
  const int64_t tok = blockIdx.x;  // the token's slot b n + i (partials)
  const int lane = threadIdx.x & 63, qd = threadIdx.x >> 6;
  const int h = blockIdx.y;
  const int b = (int)(tok / sq.n), i = (int)(tok % sq.n);
  if (i >= sq.len(b)) return;  // padding slot (block-uniform)
  const int64_t t = sq.pos0[b] + i;
  const float* ph = part + (tok * nsplit * kAH + h) * kPart;  // split s at + s * kAH * kPart
  // every lane's (m, l) of its splits and the sink are loaded first (one
  // latency), the rope table is computed meanwhile
  constexpr int KS = kMaxSplits / 64;  // splits per lane at most
  float msv[KS], lsv[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const int s = min(lane + 64 * k, nsplit - 1);  // clamped: masked below
    msv[k] = ph[(int64_t)s * kAH * kPart + kAD];
    lsv[k] = ph[(int64_t)s * kAH * kPart + kAD + 1];
  }
  const float sink_raw = sinks ? sinks[h] : 0.f;
  for (int j = threadIdx.x; j < R / 2; j += 64 * kMergeQ) {
    double sn, c;
    sincos((double)t * rope_freq(base, j, R), &sn, &c);
    cs[j] = make_double2(c, sn);
  }
  const float sink = sinks ? sink_raw * kLog2e : -INFINITY;
  float M = sink;
#pragma unroll
  for (int k = 0; k < KS; ++k)
    if (lane + 64 * k < nsplit) M = fmaxf(M, msv[k]);
  M = wave_max(M);
  float lt = 0.f;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const int s = lane + 64 * k;
    if (s < nsplit) {
      const float f = msv[k] == -INFINITY ? 0.f : exp2f(msv[k] - M);
      fs[qd][s] = f;
      lt += f * lsv[k];
    }
  }
  lt = wave_sum(lt);
  if (sinks) lt += exp2f(sink - M);
  __syncthreads();
  const int d0 = 128 * qd + 2 * lane;
  float o0 = 0.f, o1 = 0.f;
  // a split without rows holds O = 0 and f = 0, so every split is summed;
  // splits past the last re-read it with weight 0, which adds exact zeros
  constexpr int SB = 16;
  for (int s0 = 0; s0 < nsplit; s0 += SB) {
    float2 v[SB];
#pragma unroll
    for (int k = 0; k < SB; ++k)
      v[k] = *(const float2*)(ph + (int64_t)min(s0 + k, nsplit - 1) * kAH * kPart + d0);
#pragma unroll
    for (int k = 0; k < SB; ++k) {
      const float f = s0 + k < nsplit ? fs[qd][s0 + k] : 0.f;
      o0 += f * v[k].x;
      o1 += f * v[k].y;
    }
  }
  const float inv = 1.f / lt;
  o0 *= inv;
  o1 *= inv;
  const int first = kAD - R;
  if (d0 >= first) {
    const double2 c = cs[(d0 - first) >> 1];
    const float cf = (float)c.x, sf = (float)c.y;
    const float a = o0 * cf + o1 * sf, bb = o1 * cf - o0 * sf;
    o0 = a;
    o1 = bb;
  }
  *(uint32_t*)(out + (sq.row(b, i) * kAH + h) * kAD + d0) = pack_bf16x2(o0, o1);
}

// ---------------------------------------------------------------------------
// generic path

constexpr int kGCh = 32;

template <typename T>
__global__ void __launch_bounds__(256) attend_generic(
    const T* __restrict__ q, const T* __restrict__ win, int64_t win_cap, const T* __restrict__ pool,
    int64_t pool_cap, const int32_t* __restrict__ idx, int k, const float* __restrict__ sinks,
    T* __restrict__ out, Seqs sq, int H, int D, int R, int W, int m, Rope base, float scale,
    int csa) {
  extern __shared__ float sm[];
  float* qs = sm;                      // [H*D]
  float* acc = qs + H * D;             // [H*D]
  float* rows = acc + H * D;           // [kGCh*D]
  float* lg = rows + kGCh * D;         // [H*kGCh]
  float* mrun = lg + H * kGCh;         // [H]
  float* lrun = mrun + H;              // [H]
  float* alph = lrun + H;              // [H]
  int* ok = (int*)(alph + H);          // [kGCh]
  const int i = blockIdx.x, b = blockIdx.y;
  if (i >= sq.len(b)) return;  // padding slot (block-uniform)
  const int64_t t = sq.pos0[b] + i;
  const int64_t tok = sq.row(b, i);
  const int64_t lo = t - W + 1 > 0 ? t - W + 1 : 0;
  const int nwin = (int)(t - lo + 1);
  int64_t nvis = m > 0 ? (t + 1) / m : 0;
  if (nvis > pool_cap) nvis = pool_cap;
  const int npool = csa ? (int)(nvis < k ? nvis : k) : (int)nvis;
  const int nrows = nwin + npool;
  const int first = D - R;
  const T* qrow = q + tok * H * D;
  for (int e = threadIdx.x; e < H * D; e += blockDim.x) {
    const int d = e % D;
    acc[e] = 0.f;
    if (d < first) {
      qs[e] = store_t<T>::ld(qrow + e);
    } else if (((d - first) & 1) == 0) {
      double sn, c;
      sincos((double)t * rope_freq(base, (d - first) >> 1, R), &sn, &c);
      double a = store_t<T>::ld(qrow + e), bb = store_t<T>::ld(qrow + e + 1);
      rot64(a, bb, c, sn);
      T ra, rb;
      store_t<T>::st64(&ra, a);
      store_t<T>::st64(&rb, bb);
      qs[e] = store_t<T>::cvt(ra);
      qs[e + 1] = store_t<T>::cvt(rb);
    }
  }
  for (int h = threadIdx.x; h < H; h += blockDim.x) {
    mrun[h] = -INFINITY;
    lrun[h] = 0.f;
  }
  const int32_t* idx_row = csa ? idx + tok * k : nullptr;
  for (int c0 = 0; c0 < nrows; c0 += kGCh) {
    __syncthreads();
    for (int e = threadIdx.x; e < kGCh * D; e += blockDim.x) {
      const int r = e / D, d = e % D;
      const int id = c0 + r < nrows ? row_id(c0 + r, nwin, lo, win_cap, b, pool_cap, idx_row,
                                              csa, nvis, sq)
                                    : -1;
      float v = 0.f;
      if (id >= 0) v = store_t<T>::ld(win + (int64_t)id * D + d);
      else if (id <= -2) v = store_t<T>::ld(pool + (int64_t)(-2 - id) * D + d);
      rows[e] = v;
      if (d == 0) ok[r] = id != -1;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < H * kGCh; e += blockDim.x) {
      const int h = e / kGCh, r = e % kGCh;
      float s = 0.f;
      for (int d = 0; d < D; ++d) s = fmaf(qs[h * D + d], rows[r * D + d], s);
      lg[e] = ok[r] ? s * scale : -INFINITY;
    }
    __syncthreads();
    for (int h = threadIdx.x; h < H; h += blockDim.x) {
      float mx = -INFINITY;
      for (int r = 0; r < kGCh; ++r) mx = fmaxf(mx, lg[h * kGCh + r]);
      const float mn = fmaxf(mrun[h], mx);
      const float a = mn == -INFINITY ? 1.f : expf(mrun[h] - mn);
      float ps = 0.f;
      for (int r = 0; r < kGCh; ++r) {
        const float p = mn == -INFINITY ? 0.f : expf(lg[h * kGCh + r] - mn);
        lg[h * kGCh + r] = p;
        ps += p;
      }
      lrun[h] = lrun[h] * a + ps;
      mrun[h] = mn;
      alph[h] = a;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < H * D; e += blockDim.x) {
      const int h = e / D, d = e % D;
      float s = acc[e] * alph[h];
      for (int r = 0; r < kGCh; ++r) s = fmaf(lg[h * kGCh + r], rows[r * D + d], s);
      acc[e] = s;
    }
  }
  __syncthreads();
  T* orow = out + tok * H * D;
  for (int e = threadIdx.x; e < H * D; e += blockDim.x) {
    const int h = e / D, d = e % D;
    const float sink = sinks ? sinks[h] : -INFINITY;
    const float M = fmaxf(mrun[h], sink);
    const float f = expf(mrun[h] - M);
    const float lt = lrun[h] * f + (sinks ? expf(sink - M) : 0.f);
    const double inv = (double)f / (double)lt;
    if (d < first) {
      store_t<T>::st64(orow + e, (double)acc[e] * inv);
    } else if (((d - first) & 1) == 0) {
      double sn, c;
      sincos(-(double)t * rope_freq(base, (d - first) >> 1, R), &sn, &c);
      double a = (double)acc[e] * inv, bb = (double)acc[e + 1] * inv;
      rot64(a, bb, c, sn);
      store_t<T>::st64(orow + e, a);
      store_t<T>::st64(orow + e + 1, bb);
    }
  }
}

size_t attend_generic_shm(const Layer& L) {
  return ((size_t)2 * L.H * L.D + (size_t)kGCh * L.D + (size_t)L.H * kGCh + 3 * L.H + kGCh) *
         sizeof(float);
}

// ---------------------------------------------------------------------------

hipError_t launch_attend(const Layer& L, const Batch& bt, const void* q, const void* win,
                         int64_t win_cap, const void* pool, int64_t pool_cap, const int32_t* idx,
                         const float* sinks, void* out, void* ws, bool csa, hipStream_t s) {
  const int m = L.m;
  const Seqs sq = seqs_of(bt);
  if (attend_fast_shape(L)) {
    const int ns = attend_splits(L, bt.B, bt.n, pool_cap, csa);
    if (attend_dec(L, bt.B, bt.n, pool_cap, csa)) {
      hipError_t e = launch_attend_decode(L, bt, q, win, win_cap, pool, pool_cap, idx, sinks, out,
                                          ws, csa, ns, s);
      if (e != hipSuccess || ns == 1) return e;
      attend_merge<<<dim3(bt.B * bt.n, kAH), 64 * kMergeQ, 0, s>>>(
          (const float*)ws, sinks, (bf16_t*)out, sq, L.R, L.base, ns);
      return hipGetLastError();
    }
    dim3 grid(bt.n, bt.B, ns);
#define CSA_ATTN_LAUNCH(RR)                                                                 \
  attend_mfma<RR><<<grid, 256, 0, s>>>(                                                     \
      (const bf16_t*)q, (const bf16_t*)win, win_cap, (const bf16_t*)pool, pool_cap, idx, L.k, \
      sinks, (bf16_t*)out, (float*)ws, sq, L.W, m, L.base, L.scale, ns,                     \
      csa ? 1 : 0)
    switch (L.R) {
      case 16: CSA_ATTN_LAUNCH(16); break;
      case 32: CSA_ATTN_LAUNCH(32); break;
      case 64: CSA_ATTN_LAUNCH(64); break;
      default: CSA_ATTN_LAUNCH(128); break;
    }
#undef CSA_ATTN_LAUNCH
    if (ns > 1) {
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      attend_merge<<<dim3(bt.B * bt.n, kAH), 64 * kMergeQ, 0, s>>>(
          (const float*)ws, sinks, (bf16_t*)out, sq, L.R, L.base, ns);
    }
    return hipGetLastError();
  }
  const size_t shm = attend_generic_shm(L);
  dim3 grid(bt.n, bt.B);
  if (L.dtype == 1)
    attend_generic<bf16_t><<<grid, 256, shm, s>>>(
        (const bf16_t*)q, (const bf16_t*)win, win_cap, (const bf16_t*)pool, pool_cap, idx, L.k,
        sinks, (bf16_t*)out, sq, L.H, L.D, L.R, L.W, m, L.base, L.scale, csa ? 1 : 0);
  else
    attend_generic<float><<<grid, 256, shm, s>>>(
        (const float*)q, (const float*)win, win_cap, (const float*)pool, pool_cap, idx, L.k,
        sinks, (float*)out, sq, L.H, L.D, L.R, L.W, m, L.base, L.scale, csa ? 1 : 0);
  return hipGetLastError();
}

}  // namespace csa
