// Attention for calls of few tokens (decode steps, short chunks): H = 64,
// D = 512, bf16, same row list, softmax, sink and output rotation as
// attend_mfma [DeepSeek-V4 model page, sec. 2.3: shared K=V MQA over the
// sliding window and the compressed rows, sink (eq. 27), output rotation
// (eq. 26)].
//
// With few tokens the whole chip has to work on few row lists, and the cost
// is memory traffic and latency, not MFMA time.  attend_decode divides the
// work by (token, group of 16 heads, slice of rows):
//  * a block holds only its 16 heads' rotated queries (16 KB, not the
//    token's 64 KB), and its float32 partial (with several row slices) is a
//    quarter of a 64-head one, so split partials stay small;
//  * the four head groups of a token gather the same rows; their blocks get
//    ids of equal residue mod 8, which the dispatcher places on one XCD
//    (workgroups go to the XCDs round-robin), so the second to fourth
//    gathers of a row hit that XCD's L2;
//  * rows come in chunks of 64 through LDS (LDS-DMA, double buffered); wave
//    w scores rows 16w .. 16w+15 of a chunk for the 16 heads (S^T = K Q^T,
//    queries as the B operand), the chunk maximum per head is shared through
//    LDS, and P^T (64 rows x 16 heads, bf16) goes to LDS; wave w then
//    accumulates O^T for channels 128w .. 128w+127 of the 16 heads over all
//    64 rows (V^T through the LDS transpose read);
//  * the running maximum is raised lazily (by more than 2^8 only); every
//    wave takes the same decision from the same shared maxima, so no rescale
//    factors are exchanged;
//  * a single row slice ends like attend_mfma (sink folded once, rotation at
//    -t, bf16 rows staged through LDS); several slices write float32
//    partials (O, m, l) in the layout attend_merge reads.
#include "csa_device.h"
#include "csa_internal.h"
#include "attend_common.h"

namespace csa {

constexpr int kDPRow = 2 * 32 + 8;    // LDS row of P^T per head: 2 x 32 row slots + pad

template <int R>
__global__ void __launch_bounds__(256, 1) attend_decode(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ win, int64_t win_cap,
    const bf16_t* __restrict__ pool, int64_t pool_cap, const int32_t* __restrict__ idx, int k,
    const float* __restrict__ sinks, bf16_t* __restrict__ out, float* __restrict__ part,
    Seqs sq, int tokens, int W, int m, Rope base, float scale, int nsplit, int csa) {
  static_assert(R % 16 == 0 && R <= kMaxRope, "rope channels: multiple of 16, <= 128");
  __shared__ __attribute__((aligned(1024))) bf16_t kb0[kDCh * kAD];
  __shared__ __attribute__((aligned(1024))) bf16_t kb1[kDCh * kAD];
  __shared__ __attribute__((aligned(16))) int32_t rid[kDMaxRows];
  __shared__ uint32_t vmask[kDMaxRows / 32 + 2];
  __shared__ double2 cs[kMaxRope / 2];
  __shared__ __attribute__((aligned(16))) bf16_t ps[16 * kDPRow];
  __shared__ float cmx[4][16];   // each wave's chunk maximum per head
  __shared__ float lsum[4][16];  // each wave's running sum per head

  // block -> (token, head group, row slice); a token's blocks share id mod 8
  const int G = 4 * nsplit;
  const int id = blockIdx.x;
  const int tq = (id / (8 * G)) * 8 + (id & 7);
  if (tq >= tokens) return;  // padding blocks (block-uniform, before any barrier)
  const int jg = (id >> 3) % G;
  const int hg = jg & 3, sp = jg >> 2;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int b = tq / sq.n, i = tq % sq.n;
  if (i >= sq.len(b)) return;  // padding slot (block-uniform, before any barrier)
  const int64_t t = sq.pos0[b] + i;
  const int64_t tok = sq.row(b, i);  // row of q, the ids and the output
  const int64_t slot = tq;           // slot of the split partials
  const int64_t lo = t - W + 1 > 0 ? t - W + 1 : 0;
  const int nwin = (int)(t - lo + 1);
  int64_t nvis = m > 0 ? (t + 1) / m : 0;
  if (nvis > pool_cap) nvis = pool_cap;
  const int npool = csa ? (int)(nvis < k ? nvis : k) : (int)nvis;
  const int nrows = nwin + npool;
  const int nch = (nrows + kDCh - 1) / kDCh;
  const int cps = (nch + nsplit - 1) / nsplit;
  const int c0 = min(nch, sp * cps), c1 = min(nch, c0 + cps);
  const int r0 = c0 * kDCh, r1 = min(nrows, c1 * kDCh);
  const int32_t* idx_row = csa ? idx + tok * k : nullptr;
  const int self_id = (int)((int64_t)b * win_cap + t % win_cap);  // always a valid row

  for (int j = tid; j < r1 - r0; j += 256)
    rid[j] = row_id(r0 + j, nwin, lo, win_cap, b, pool_cap, idx_row, csa, nvis, sq);
  for (int j = tid; j < R / 2; j += 256) {
    double sn, c;
    sincos((double)t * rope_freq(base, j, R), &sn, &c);
    cs[j] = make_double2(c, sn);
  }
  __syncthreads();
  // bits of vmask[2 (c - c0)], [2 (c - c0) + 1]: rows of chunk c that take part
  for (int j0 = 64 * wv; j0 < r1 - r0; j0 += 256) {
    const bool ok = j0 + lane < r1 - r0 && rid[j0 + lane] != -1;
    const unsigned long long bal = __ballot(ok);
    if (lane == 0) {
      vmask[j0 >> 5] = (uint32_t)bal;
      vmask[(j0 >> 5) + 1] = (uint32_t)(bal >> 32);
    }
  }
  __syncthreads();

  // gather of chunk c into dst: this wave moves rows 16 wv .. 16 wv + 15 (one
  // 1 KB row per DMA instruction).  The row ids are read in one go; the lane
  // id is copied opaquely and the wave index made scalar so that nothing
  // here is spilled (a scratch reload would wait on every DMA in flight).
  struct Gather {
    int ids[16];
    int ln, wvs, c;
    bf16_t* dst;
  };
  auto gather_prep = [&](Gather& Gt, int c, bf16_t* dst) {
    asm volatile("v_mov_b32 %0, %1" : "=v"(Gt.ln) : "v"(lane));
    Gt.wvs = __builtin_amdgcn_readfirstlane(wv);
    Gt.c = c;
    Gt.dst = dst;
    const int base_r = (c - c0) * kDCh + 16 * Gt.wvs;
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      const int4 v = *(const int4*)&rid[base_r + e];
      Gt.ids[e] = v.x;
      Gt.ids[e + 1] = v.y;
      Gt.ids[e + 2] = v.z;
      Gt.ids[e + 3] = v.w;
    }
  };
  auto gather_row = [&](const Gather& Gt, int e) {
    const int rr = 16 * Gt.wvs + e;
    const int jr = Gt.c * kDCh + rr;
    int rw = jr < r1 ? Gt.ids[e] : -1;
    if (rw == -1) rw = self_id;  // masked in the softmax; any finite row will do
    const bf16_t* src = rw >= 0 ? win + (int64_t)rw * kAD : pool + (int64_t)(-2 - rw) * kAD;
    src += 8 * (Gt.ln ^ swz(rr));
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(Gt.dst + rr * kAD), 16, 0, 0);
  };
  if (c0 < c1) {
    Gather Gt;
    gather_prep(Gt, c0, kb0);
#pragma unroll
    for (int e = 0; e < 16; ++e) gather_row(Gt, e);
  }

  // the 16 heads' rotated queries: head 16 hg + r16, channels 32 kk + 8 g ..
  uint4 Qf[16];
  load_qfrag<R>(q + (tok * kAH + 16 * hg + r16) * kAD, cs, g, Qf);

  // O^T of the wave's channel slice: channel 128 wv + 16 dt + 4 g + e, head r16
  f32x4 O[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) O[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;  // head r16: shared maximum, this wave's rows' sum
  const float sl2 = scale * kLog2e;

  // per-lane LDS byte offsets (see attend_mfma): K fragment of row
  // 16 wv + r16, chunk 4 kk + g at kb_v[kk & 3] + (kk >> 2) 256 + 16 wv KB;
  // transpose read for channel tile dt of the wave's slice and row step ks at
  // tr_v[dt] + 32 ks KB (+16 KB for the upper 16 rows of the step)
  int kb_v[4], tr_v[8];
#pragma unroll
  for (int v = 0; v < 4; ++v)
    kb_v[v] = 16 * wv * 1024 + r16 * 1024 + (((4 * v + g) ^ swz(r16)) << 4);
  {
    const int trA = 4 * g + (r16 >> 2);
    const int trc = (r16 & 3) >> 1, trh = (r16 & 1) * 8;
#pragma unroll
    for (int v = 0; v < 8; ++v)
      tr_v[v] = trA * 1024 + (((2 * v + trc) ^ swz(trA)) << 4) + trh + 256 * wv;
  }

  auto chunk = [&](int c, const bf16_t* cur, int cn, bf16_t* nxt) {
    const char* kbp = (const char*)cur;
    Gather Gt;
    const bool gat = cn < c1;
    if (gat) gather_prep(Gt, cn, nxt);
    // ---- S^T = K Q^T: the wave's 16 rows x 16 heads
    f32x4 S = (f32x4){0.f, 0.f, 0.f, 0.f};
    auto kfrag = [&](int kk) {
      return *(const uint4*)(kbp + kb_v[kk & 3] + (kk >> 2) * 256);
    };
    uint4 kf[2];
    kf[0] = kfrag(0);
    kf[1] = kfrag(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      S = mfma16(kf[kk & 1], Qf[kk], S);
      if (kk + 2 < 16) kf[kk & 1] = kfrag(kk + 2);
      if (gat) gather_row(Gt, kk);
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- softmax (log2 domain); lane (g, r16): rows 16 wv + 4 g + ii, head r16
    const int cl = c - c0;
    const uint32_t vm = vmask[2 * cl + (wv >> 1)] >> (16 * (wv & 1) + 4 * g);
    float sv[4];
    float mx = -INFINITY;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      sv[ii] = (vm >> ii) & 1u ? S[ii] * sl2 : -INFINITY;
      mx = fmaxf(mx, sv[ii]);
    }
    mx = xmax32(xmax16(mx));
    if (g == 0) cmx[wv][r16] = mx;
    __syncthreads();
    const float cmax = fmaxf(fmaxf(cmx[0][r16], cmx[1][r16]), fmaxf(cmx[2][r16], cmx[3][r16]));
    if (__any(cmax > m_run + kLazy)) {  // the same decision in every wave
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) O[dt] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      // exp2(-inf) = 0 for masked rows; m_run is finite once a row was seen
      p[ii] = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[ii] - m_run);
      l_run += p[ii];
    }
    // P^T slots of row step ks = wv / 2: lane group g' holds rows 4 g' ..
    // 4 g' + 3 of wave 2 ks (slots 8 g' .. +3) and of wave 2 ks + 1 (+4 ..)
    *(uint2*)&ps[r16 * kDPRow + (wv >> 1) * 32 + 8 * g + 4 * (wv & 1)] =
        make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
    __syncthreads();
    // ---- O^T += V^T P^T over the wave's channel slice, all 64 rows
    uint4 Pf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) Pf[ks] = *(const uint4*)&ps[r16 * kDPRow + ks * 32 + 8 * g];
    auto vfrag = [&](int dt, int ks) {
      const char* pa = kbp + tr_v[dt] + ks * 32768;
      const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)pa);
      const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(pa + 16384));
      return make_uint4((uint32_t)(uint16_t)lo4[0] | ((uint32_t)(uint16_t)lo4[1] << 16),
                        (uint32_t)(uint16_t)lo4[2] | ((uint32_t)(uint16_t)lo4[3] << 16),
                        (uint32_t)(uint16_t)hi4[0] | ((uint32_t)(uint16_t)hi4[1] << 16),
                        (uint32_t)(uint16_t)hi4[2] | ((uint32_t)(uint16_t)hi4[3] << 16));
    };
    uint4 vf[2];
    vf[0] = vfrag(0, 0);
    vf[1] = vfrag(0, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < 16; ++st) {  // step st: channel tile st / 2, row step st % 2
      const uint4 a = vf[st & 1];
      if (st + 2 < 16) vf[st & 1] = vfrag((st + 2) >> 1, st & 1);
      O[st >> 1] = mfma16(a, Pf[st & 1], O[st >> 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int c = c0; c < c1; c += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    chunk(c, kb0, c + 1, kb1);
    if (c + 1 < c1) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      chunk(c + 1, kb1, c + 2, kb0);
    }
  }

  l_run = xsum32(xsum16(l_run));
  if (g == 0) lsum[wv][r16] = l_run;
  __syncthreads();  // every wave is done with the chunk buffers; sums published
  const float lb = (lsum[0][r16] + lsum[1][r16]) + (lsum[2][r16] + lsum[3][r16]);
  const int head = 16 * hg + r16;
  constexpr int first = kAD - R;
  if (nsplit == 1) {
    // 16 bf16 rows staged in kb0, 16-byte chunk c of head row h at slot c ^ h
    const float sink = sinks ? sinks[head] * kLog2e : -INFINITY;
    const float M = fmaxf(m_run, sink);
    const float f = __builtin_amdgcn_exp2f(m_run - M);
    const float lt = lb * f + (sinks ? __builtin_amdgcn_exp2f(sink - M) : 0.f);
    const float inv = f / lt;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d = 128 * wv + 16 * dt + 4 * g;
      float o0 = O[dt][0] * inv, o1 = O[dt][1] * inv, o2 = O[dt][2] * inv, o3 = O[dt][3] * inv;
      if (d >= first) {  // pair (d, d+1) rotated at -t
        const double2 ca = cs[(d - first) >> 1];
        const float cf = (float)ca.x, sf = (float)ca.y;
        const float a0 = o0 * cf + o1 * sf, a1 = o1 * cf - o0 * sf;
        o0 = a0;
        o1 = a1;
      }
      if (d + 2 >= first) {  // pair (d+2, d+3)
        const double2 cb = cs[(d + 2 - first) >> 1];
        const float cf = (float)cb.x, sf = (float)cb.y;
        const float b0 = o2 * cf + o3 * sf, b1 = o3 * cf - o2 * sf;
        o2 = b0;
        o3 = b1;
      }
      char* rowb = (char*)kb0 + r16 * 1024;
      *(uint2*)(rowb + (((d >> 3) ^ r16) << 4) + ((d & 7) << 1)) =
          make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
    }
    __syncthreads();
    bf16_t* orow = out + (tok * kAH + 16 * hg) * kAD;
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const int h = 4 * wv + hh;
      const uint4 v = *(const uint4*)((const char*)kb0 + h * 1024 + ((lane ^ h) << 4));
      *(uint4*)(orow + h * kAD + 8 * lane) = v;
    }
  } else {
    // float32 partial rows staged in kb0 (2 KB per head, 16-byte chunk c of
    // head row h at slot c ^ h), then written whole
    float* pbase = part + ((slot * nsplit + sp) * kAH + 16 * hg) * kPart;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int ch = 32 * wv + 4 * dt + g;  // 16-byte chunk of the 512-float row
      *(f32x4*)((char*)kb0 + r16 * 2048 + ((ch ^ r16) << 4)) = O[dt];
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const int h = 4 * wv + hh;
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int ch = lane + 64 * it;
        *(f32x4*)(pbase + h * kPart + 4 * ch) =
            *(const f32x4*)((const char*)kb0 + h * 2048 + ((ch ^ h) << 4));
      }
    }
    if (wv == 0 && g == 0) {
      float* prow = pbase + r16 * kPart;
      prow[kAD] = m_run;
      prow[kAD + 1] = lb;
    }
  }
}

hipError_t launch_attend_decode(const Layer& L, const Batch& bt, const void* q, const void* win,
                                int64_t win_cap, const void* pool, int64_t pool_cap,
                                const int32_t* idx, const float* sinks, void* out, void* ws,
                                bool csa, int ns, hipStream_t s) {
  const int tokens = bt.B * bt.n;
  const int grid = (tokens + 7) / 8 * 8 * 4 * ns;
#define CSA_DEC_LAUNCH(RR)                                                                       \
  attend_decode<RR><<<grid, 256, 0, s>>>((const bf16_t*)q, (const bf16_t*)win, win_cap,          \
                                         (const bf16_t*)pool, pool_cap, idx, L.k, sinks,          \
                                         (bf16_t*)out, (float*)ws, seqs_of(bt), tokens, L.W,     \
                                         L.m, L.base, L.scale, ns, csa ? 1 : 0)
  switch (L.R) {
    case 16: CSA_DEC_LAUNCH(16); break;
    case 32: CSA_DEC_LAUNCH(32); break;
    case 64: CSA_DEC_LAUNCH(64); break;
    default: CSA_DEC_LAUNCH(128); break;
  }
#undef CSA_DEC_LAUNCH
  return hipGetLastError();
}

}  // namespace csa
