// Attention for calls of few tokens (decode steps, short chunks): H = 64,
// D = 512, bf16, same row list, softmax, sink and output rotation as
// attend_mfma [DeepSeek-V4 model page, sec. 2.3: shared K=V MQA over the
// sliding window and the compressed rows, sink (eq. 27), output rotation
// (eq. 26)].
//
// With few tokens the whole chip has to work on few row lists, and the cost
// is moving rows, not MFMA time.  attend_decode divides the work by (token,
// group of 16 heads, slice of rows):
//  * a block holds only its 16 heads' rotated queries, and its float32
//    partial (with several row slices) is a quarter of a 64-head one;
//  * the four head groups of a token gather the same rows; their blocks get
//    ids of equal residue mod 8, which the dispatcher places on one XCD
//    (workgroups go to the XCDs round-robin), so the second to fourth
//    gathers of a row hit that XCD's L2;
//  * inside a block each wave owns whole 16-row groups of the row list
//    (groups w, w + 4, w + 8, ...): it gathers them into its own two LDS
//    buffers by LDS-DMA (one group in flight while the other is scored),
//    scores them (S^T = K Q^T, 16 x 16 x 32 MFMA, queries as the B operand),
//    keeps its own running maximum and sum per head, and accumulates
//    O^T += V^T P^T over all 512 channels (16 x 16 x 16 MFMA: the P^T
//    operand is exactly the lanes' own softmax values, V^T comes from the
//    same LDS rows through the transpose read).  No wave waits for another
//    inside the loop: the rate of a CU's row gathers (not the MFMA work)
//    bounds the kernel, and a gather issue that stalls holds up only the
//    wave issuing it.
//  * the four waves' (m, l, O) are merged once at the end through LDS; one
//    row slice ends with the sink folded once, rotation at -t and bf16 rows;
//    several slices write float32 partials (O, m, l) in attend_merge's
//    layout.
//  * the running maximum is raised lazily (by more than 2^8 only).
#include "csa_device.h"
#include "csa_internal.h"
#include "attend_common.h"

namespace csa {

constexpr int kGR = 16;  // rows per wave group

// LDS reads of the DMA-filled group buffers, out of the compiler's sight: a
// compiler-visible LDS load there would first wait for every LDS-DMA in
// flight (the compiler cannot tell the buffer read from the one being
// filled).  Each block waits for its own data before returning.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// four 16-byte reads at a[j] + OFF
template <int OFF>
__device__ __forceinline__ void lds_rd4x128(const uint32_t (&a)[4], uint4 (&o)[4]) {
  u32x4 x0, x1, x2, x3;
  asm volatile(
      "ds_read_b128 %0, %4 offset:%8\n\t"
      "ds_read_b128 %1, %5 offset:%8\n\t"
      "ds_read_b128 %2, %6 offset:%8\n\t"
      "ds_read_b128 %3, %7 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "n"(OFF)
      : "memory");
  o[0] = __builtin_bit_cast(uint4, x0);
  o[1] = __builtin_bit_cast(uint4, x1);
  o[2] = __builtin_bit_cast(uint4, x2);
  o[3] = __builtin_bit_cast(uint4, x3);
}
// eight transposed 8-byte reads (ds_read_b64_tr_b16) at a[j] + OFF
template <int OFF>
__device__ __forceinline__ void lds_rdtr8(const uint32_t (&a)[8], uint2 (&o)[8]) {
  u32x2 x[8];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%16\n\t"
      "ds_read_b64_tr_b16 %1, %9 offset:%16\n\t"
      "ds_read_b64_tr_b16 %2, %10 offset:%16\n\t"
      "ds_read_b64_tr_b16 %3, %11 offset:%16\n\t"
      "ds_read_b64_tr_b16 %4, %12 offset:%16\n\t"
      "ds_read_b64_tr_b16 %5, %13 offset:%16\n\t"
      "ds_read_b64_tr_b16 %6, %14 offset:%16\n\t"
      "ds_read_b64_tr_b16 %7, %15 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
        "=&v"(x[6]), "=&v"(x[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
        "n"(OFF)
      : "memory");
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = make_uint2(x[j][0], x[j][1]);
}

typedef short bf16x4_s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16k16(uint2 a, uint2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_s, a),
                                                  __builtin_bit_cast(bf16x4_s, b), c, 0, 0, 0);
}

template <int R>
__global__ void __launch_bounds__(256, 1) attend_decode(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ win, int64_t win_cap,
    const bf16_t* __restrict__ pool, int64_t pool_cap, const int32_t* __restrict__ idx, int k,
    const float* __restrict__ sinks, bf16_t* __restrict__ out, float* __restrict__ part,
    Seqs sq, int tokens, int W, int m, Rope base, float scale, int nsplit, int csa) {
  static_assert(R % 16 == 0 && R <= kMaxRope, "rope channels: multiple of 16, <= 128");
  // per wave two 16-row group buffers (8 named arrays so the compiler can
  // tell the DMA target from the buffer being read); after the loop the
  // same 128 KB hold the waves' O for the merge
  __shared__ __attribute__((aligned(1024))) bf16_t gb[8][kGR * kAD];
  __shared__ __attribute__((aligned(16))) int32_t rid[kDMaxRows];
  __shared__ double2 cs[kMaxRope / 2];
  __shared__ __attribute__((aligned(16))) float2 csf[kMaxRope / 2];  // cs rounded to float
  __shared__ float wm[4][16], wl[4][16];  // each wave's running maximum and sum per head
  __shared__ float sinkl[16];             // the group's sink logits (natural units)

  // block -> (token, head group, row slice); a token's blocks share id mod 8
  const int G = 4 * nsplit;
  const int id = blockIdx.x;
  const int tq = (id / (8 * G)) * 8 + (id & 7);
  if (tq >= tokens) return;  // padding blocks (block-uniform, before any barrier)
  const int jg = (id >> 3) % G;
  const int hg = jg & 3, sp = jg >> 2;

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int nr = r1 - r0;                   // rows of this block
  const int ngr = (nr + kGR - 1) / kGR;     // 16-row groups (whole kDCh chunks: <= kDMaxRows)
  const int32_t* idx_row = csa ? idx + tok * k : nullptr;
  const int self_id = (int)((int64_t)b * win_cap + t % win_cap);  // always a valid row

  // the 16 heads' query fragments (head 16 hg + r16, channels 32 kk + 8 g ..)
  // start loading now; they are rotated once the rope table is in LDS
  constexpr int first = kAD - R;
  uint4 Qf[16];
  {
    const bf16_t* qrow = q + (tok * kAH + 16 * hg + r16) * kAD + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) Qf[kk] = *(const uint4*)(qrow + 32 * kk);
  }
  // the sink logit is loaded by every lane (no branch holds a wait for it)
  const float sink_raw = sinks ? sinks[16 * hg + (tid & 15)] : 0.f;
  // row ids: every selected index of the thread's rows is loaded first (one
  // memory latency, not one per row); window row j is ring slot
  // (lo + j) mod cap, and j < nwin <= cap (the ring holds the window or the
  // whole sequence) leaves one wrap at most
  {
    constexpr int U = kDMaxRows / 256;
    int32_t sel[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = r0 + tid + 256 * u - nwin;
      sel[u] = (csa && tid + 256 * u < nr && e >= 0) ? idx_row[e] : 0;
    }
    // the rope table while the loads are in flight
    for (int j = tid; j < R / 2; j += 256) {
      double sn, c;
      sincos((double)t * rope_freq(base, j, R), &sn, &c);
      cs[j] = make_double2(c, sn);
      csf[j] = make_float2((float)c, (float)sn);
    }
    const int lo_mod = (int)(lo % win_cap), cap = (int)win_cap, wb = (int)((int64_t)b * win_cap);
    // pool rows of all the thread's entries first (with a block table these
    // are loads: all in flight at once; entries that are not visible pool
    // rows look up entry 0 and are not used)
    int64_t prw[U];
    bool vis[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jr = r0 + tid + 256 * u;
      const int64_t w = csa ? (int64_t)sel[u] : (int64_t)(jr - nwin);
      vis[u] = w >= 0 && w < nvis;
      prw[u] = sq.prow(b, vis[u] ? w : 0, pool_cap);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = tid + 256 * u;
      if (j < ngr * kGR) {
        const int jr = r0 + j;
        int id = -1;
        if (j >= nr) {
        } else if (jr < nwin) {
          const int v = lo_mod + jr;
          id = wb + (v >= cap ? v - cap : v);
        } else if (vis[u]) {
          id = (int)(-2 - prw[u]);
        }
        rid[j] = id;
      }
    }
  }
  if (tid < 16) sinkl[tid] = sink_raw;  // scaled to log2 units at the end
  __syncthreads();

  // DMA of group gi into buffer dst: 16 rows of 1 KB, one per instruction;
  // 16-byte chunk c of row e lands at slot c ^ swz(e).  Masked rows load the
  // token's own window row (finite; its weight is zero).  The lane id is
  // copied opaquely so that the per-lane offset is not hoisted and spilled
  // (a scratch reload would wait on every DMA in flight).
  auto issue = [&](int gi, bf16_t* dst) {
    int ln;
    asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
    const int4* rp = (const int4*)&rid[gi * kGR];
    int ids[kGR];
#pragma unroll
    for (int e = 0; e < kGR; e += 4) {
      const int4 v = rp[e >> 2];
      ids[e] = v.x;
      ids[e + 1] = v.y;
      ids[e + 2] = v.z;
      ids[e + 3] = v.w;
    }
#pragma unroll
    for (int e = 0; e < kGR; ++e) {
      const int rw = ids[e] == -1 ? self_id : ids[e];
      const bf16_t* src = rw >= 0 ? win + (int64_t)rw * kAD : pool + (int64_t)(-2 - rw) * kAD;
      __builtin_amdgcn_global_load_lds((const void*)(src + 8 * (ln ^ swz(e))),
                                       (lds_void*)(dst + e * kAD), 16, 0, 0);
    }
  };

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

  // O^T of all 512 channels for the wave's rows: channel 16 d + 4 g + e, head r16
  f32x4 O[32];
#pragma unroll
  for (int d = 0; d < 32; ++d) O[d] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;  // head r16 (l: this lane's rows)
  const float sl2 = scale * kLog2e;

  // per-lane LDS byte offsets inside a group buffer.  K fragment kk (row
  // r16, chunk 4 kk + g) sits at kofs[kk & 3] + 256 (kk >> 2).  The V^T
  // fragment of channel tile d (rows 4 g + r16 / 4, channels 16 d + 4 (r16 & 3)
  // .. + 3, 8 bytes) sits at tofs[d & 7] + 256 (d >> 3): chunk 2 d + (r16 & 3) / 2
  // at slot chunk ^ swz(row), and the swizzle only moves the low four bits.
  uint32_t kofs[4], tofs[8];
  const int trow = 4 * g + (r16 >> 2), tsel = (r16 & 3) >> 1;
#pragma unroll
  for (int v = 0; v < 4; ++v) kofs[v] = r16 * 1024 + (((4 * v + g) ^ swz(r16)) << 4);
#pragma unroll
  for (int d = 0; d < 8; ++d)
    tofs[d] = trow * 1024 + (((2 * d + tsel) ^ swz(trow)) << 4) + (r16 & 1) * 8;

  auto group = [&](int gi, const bf16_t* buf) {
    const uint32_t kb = lds_addr(buf);
    uint32_t ka[4], ta[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) ka[v] = kb + kofs[v];
#pragma unroll
    for (int d = 0; d < 8; ++d) ta[d] = kb + tofs[d];
    // ---- S^T = K Q^T: the group's 16 rows x 16 heads, two accumulation chains
    f32x4 Sa = (f32x4){0.f, 0.f, 0.f, 0.f}, Sb = Sa;
    uint4 kf[4];
    lds_rd4x128<0>(ka, kf);
    Sa = mfma16(kf[0], Qf[0], Sa);
    Sb = mfma16(kf[1], Qf[1], Sb);
    Sa = mfma16(kf[2], Qf[2], Sa);
    Sb = mfma16(kf[3], Qf[3], Sb);
    lds_rd4x128<256>(ka, kf);
    Sa = mfma16(kf[0], Qf[4], Sa);
    Sb = mfma16(kf[1], Qf[5], Sb);
    Sa = mfma16(kf[2], Qf[6], Sa);
    Sb = mfma16(kf[3], Qf[7], Sb);
    lds_rd4x128<512>(ka, kf);
    Sa = mfma16(kf[0], Qf[8], Sa);
    Sb = mfma16(kf[1], Qf[9], Sb);
    Sa = mfma16(kf[2], Qf[10], Sa);
    Sb = mfma16(kf[3], Qf[11], Sb);
    lds_rd4x128<768>(ka, kf);
    Sa = mfma16(kf[0], Qf[12], Sa);
    Sb = mfma16(kf[1], Qf[13], Sb);
    Sa = mfma16(kf[2], Qf[14], Sa);
    Sb = mfma16(kf[3], Qf[15], Sb);
    // ---- softmax (log2 domain): lane (g, r16) holds rows 4 g .. 4 g + 3, head r16
    const int4 vr = *(const int4*)&rid[gi * kGR + 4 * g];
    const int vids[4] = {vr.x, vr.y, vr.z, vr.w};
    float sv[4];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sv[e] = vids[e] != -1 ? (Sa[e] + Sb[e]) * sl2 : -INFINITY;
      mx = fmaxf(mx, sv[e]);
    }
    mx = xmax32(xmax16(mx));  // over the group's 16 rows
    if (mx > m_run + kLazy) {  // per head (lane-wise): rescale this lane's O
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < 32; ++d) O[d] *= alpha;
      m_run = m_new;
    }
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[e] - m_run);
      l_run += p[e];
    }
    // P^T operand of the 16 x 16 x 16 MFMA: rows 4 g .. 4 g + 3 of head r16
    const uint2 pf = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
    // ---- O^T += V^T P^T over the 32 channel tiles (8 transposed reads at a time)
    uint2 vf[8];
    lds_rdtr8<0>(ta, vf);
#pragma unroll
    for (int d = 0; d < 8; ++d) O[d] = mfma16k16(vf[d], pf, O[d]);
    lds_rdtr8<256>(ta, vf);
#pragma unroll
    for (int d = 0; d < 8; ++d) O[8 + d] = mfma16k16(vf[d], pf, O[8 + d]);
    lds_rdtr8<512>(ta, vf);
#pragma unroll
    for (int d = 0; d < 8; ++d) O[16 + d] = mfma16k16(vf[d], pf, O[16 + d]);
    lds_rdtr8<768>(ta, vf);
#pragma unroll
    for (int d = 0; d < 8; ++d) O[24 + d] = mfma16k16(vf[d], pf, O[24 + d]);
  };

  // groups wv, wv + 4, ...; buffer gb[2 wv + (j & 1)] for the wave's j-th
  // group.  Before scoring group j the wave's DMA of it has landed (at most
  // the 16 instructions of group j + 1 still in flight); after scoring, the
  // buffer is refilled with group j + 2.
  const int nmine = ngr > wv ? (ngr - wv + 3) / 4 : 0;  // wave-uniform
  bf16_t* B0 = gb[2 * wv];
  bf16_t* B1 = gb[2 * wv + 1];
  if (nmine > 0) issue(wv, B0);
  if (nmine > 1) issue(wv + 4, B1);
  for (int j = 0; j < nmine; j += 2) {
    if (j + 1 < nmine) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    group(wv + 4 * j, B0);
    if (j + 2 < nmine) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this buffer's reads are done
      issue(wv + 4 * (j + 2), B0);
    }
    if (j + 1 < nmine) {
      if (j + 2 < nmine) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      group(wv + 4 * (j + 1), B1);
      if (j + 3 < nmine) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue(wv + 4 * (j + 3), B1);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS-DMA outlives the loop

  // ---- merge of the four waves: M = max_w m_w, L = sum_w l_w 2^(m_w - M),
  // O = sum_w O_w 2^(m_w - M), through LDS (the group buffers, 128 KB:
  // wave w's O at [w][head][512] floats, 16-byte chunk c of head row h at
  // slot c ^ h)
  l_run = xsum32(xsum16(l_run));  // over the lanes holding head r16's rows
  if (g == 0) {
    wm[wv][r16] = m_run;
    wl[wv][r16] = l_run;
  }
  __syncthreads();  // every wave is done with the group buffers; maxima published
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][r16]);
  const float fw = M == -INFINITY || m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
  float* ob = (float*)&gb[0][0];
  {
    float* mine = ob + wv * (16 * kAD) + r16 * kAD;
#pragma unroll
    for (int d = 0; d < 32; ++d)
      *(f32x4*)(mine + (((4 * d + g) ^ r16) << 2)) = O[d] * fw;
  }
  __syncthreads();
  // wave wv writes channels 128 wv .. 128 wv + 127 of the 16 heads: lane l
  // takes head h = l / 4 and channels 128 wv + 32 (l & 3) .. + 31
  const int h = lane >> 2;
  float Mh = -INFINITY, Lh = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) Mh = fmaxf(Mh, wm[w][h]);
#pragma unroll
  for (int w = 0; w < 4; ++w)
    if (wm[w][h] != -INFINITY) Lh += wl[w][h] * __builtin_amdgcn_exp2f(wm[w][h] - Mh);
  const int ch0 = 128 * wv + 32 * (lane & 3);
  float o[32];
#pragma unroll
  for (int c = 0; c < 32; c += 4) {
    f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w)
      acc += *(const f32x4*)(ob + w * (16 * kAD) + h * kAD + ((((ch0 + c) >> 2) ^ h) << 2));
    o[c] = acc[0];
    o[c + 1] = acc[1];
    o[c + 2] = acc[2];
    o[c + 3] = acc[3];
  }
  const int head = 16 * hg + h;
  if (nsplit == 1) {
    const float sink = sinks ? sinkl[h] * kLog2e : -INFINITY;
    const float Mt = fmaxf(Mh, sink);
    const float f = Mh == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(Mh - Mt);
    const float lt = Lh * f + (sinks ? __builtin_amdgcn_exp2f(sink - Mt) : 0.f);
    const float inv = f / lt;
#pragma unroll
    for (int c = 0; c < 32; ++c) o[c] *= inv;
    if (ch0 + 32 > first) {
      // pairs (d, d+1) at and above `first` rotated at -t; the table reads
      // are unconditional (clamped index) so that they issue together
#pragma unroll
      for (int c = 0; c < 32; c += 2) {
        const int d = ch0 + c;
        const float2 cz = csf[d >= first ? (d - first) >> 1 : 0];
        const float a0 = o[c] * cz.x + o[c + 1] * cz.y, a1 = o[c + 1] * cz.x - o[c] * cz.y;
        if (d >= first) {
          o[c] = a0;
          o[c + 1] = a1;
        }
      }
    }
    bf16_t* orow = out + (tok * kAH + head) * kAD + ch0;
#pragma unroll
    for (int c = 0; c < 32; c += 8)
      *(uint4*)(orow + c) = make_uint4(pack_bf16x2(o[c], o[c + 1]), pack_bf16x2(o[c + 2], o[c + 3]),
                                       pack_bf16x2(o[c + 4], o[c + 5]),
                                       pack_bf16x2(o[c + 6], o[c + 7]));
  } else {
    // float32 partial row of head `head`: O (relative to M), then m = M, l = L
    float* prow = part + ((slot * nsplit + sp) * kAH + head) * kPart;
#pragma unroll
    for (int c = 0; c < 32; c += 4)
      *(f32x4*)(prow + ch0 + c) = (f32x4){o[c], o[c + 1], o[c + 2], o[c + 3]};
    if (wv == 0 && (lane & 3) == 0) {
      prow[kAD] = Mh;
      prow[kAD + 1] = Lh;
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
