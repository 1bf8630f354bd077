// KV compressor: learned gated pooling with streaming state.
//
// Entry w of a stream pools the tokens [(w - overlap) m, (w + 1) m) that are
// >= 0: per channel, a softmax of the gate logits over those tokens weights
// their kv values; then an optional RMSNorm over the entry; then RoPE at
// position w m [DeepSeek-V4 model page, sec. 2.3 (CSA overlapping windows at
// m = 4, HCA non-overlapping at m' = 128) and "Cache layers" (buffer, pool,
// counter and overlap state); TransformerLens adapter, compressor submodules
// kv_proj, gate_proj, kv_norm, rotary_emb].
//
// A call carries n new tokens per sequence at positions p0 .. p0+n-1.  The
// tokens an entry needs from before p0 live in the caller's state ring of
// (1 + overlap) m raw rows (slot = position mod ring length).  The math is
// float64 (exp, sums, norm, rotation) and each pooled value is rounded once
// to the storage dtype.  The work is a few hundred bytes per entry channel
// and is bound by reading kv and gate once from HBM.
#include <type_traits>

#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

constexpr int kMaxWidth = 2048;

// Eight consecutive channels (16 bytes of bf16, 32 of float32) as floats.
template <typename T> struct row8;
template <> struct row8<bf16_t> {
  typedef uint4 raw;
  static __device__ __forceinline__ raw ld(const bf16_t* p) { return *(const uint4*)p; }
  static __device__ __forceinline__ float get(const raw& r, int e) {
    const uint32_t u = e < 2 ? r.x : (e < 4 ? r.y : (e < 6 ? r.z : r.w));
    return __uint_as_float((e & 1) ? (u & 0xffff0000u) : (u << 16));
  }
};
template <> struct row8<float> {
  struct raw {
    float4 a, b;
  };
  static __device__ __forceinline__ raw ld(const float* p) {
    return raw{*(const float4*)p, *(const float4*)(p + 4)};
  }
  static __device__ __forceinline__ float get(const raw& r, int e) {
    const float4 v = e < 4 ? r.a : r.b;
    const int k = e & 3;
    return k == 0 ? v.x : (k == 1 ? v.y : (k == 2 ? v.z : v.w));
  }
};

// LDS of the one-token pooling's token-group partials: per (group, channel)
// the group's maximum (float) and its two sums (double); groups x width is
// at most 2048.
constexpr int kPoolWideBytes = kMaxWidth * (4 + 8 + 8);

// Entry w of sequence b by one block of 256 threads (the one-token decode
// call; pooled and red in LDS).  Widths of 8 c channels with c dividing 256
// go "wide": thread t takes the 8 channels of chunk t mod c and every
// (256/c)-th token of the window from token t / c on, with 16-byte loads,
// eight tokens in flight; the groups' maxima and sums meet in LDS (`wide`),
// summed in group order.  Other widths take one channel per thread over the
// whole window, eight tokens at a time.
template <typename T>
__device__ __forceinline__ void pool_entry(
    const T* __restrict__ kv, const T* __restrict__ gate, const float* __restrict__ norm_w,
    float eps, const T* __restrict__ st_kv, const T* __restrict__ st_gate, T* __restrict__ pool,
    int b, int64_t p0, int64_t w, int64_t row0, int64_t dst_row, int width, int R, Rope base,
    int m, int overlap, double* pooled, double* red, void* wide) {
  const int Ls = (1 + overlap) * m;
  const int64_t lo = max((w - overlap) * (int64_t)m, (int64_t)0), hi = (w + 1) * (int64_t)m;
  const T* kv_b = kv + row0 * width;  // the call's token rows of sequence b
  const T* g_b = gate + row0 * width;
  const T* skv_b = st_kv + (int64_t)b * Ls * width;
  const T* sg_b = st_gate + (int64_t)b * Ls * width;
  double ss = 0.0;
  // the window's tokens go eight at a time: their loads are unconditional
  // (tokens past the window re-read its last one and are masked out) so that
  // the eight share one latency; a load per loop step was waited for at
  // once, one latency per token (128 for an HCA entry)
  constexpr int TB = 8;
  auto grow = [&](int64_t s) {
    return s >= p0 ? g_b + (s - p0) * width : sg_b + (int64_t)(s % Ls) * width;
  };
  auto vrow = [&](int64_t s) {
    return s >= p0 ? kv_b + (s - p0) * width : skv_b + (int64_t)(s % Ls) * width;
  };
  const int NC = width >> 3;
  const bool wide_ok = (width & 7) == 0 && NC >= 1 && NC <= 256 && (256 % NC) == 0 &&
                       blockDim.x == 256;
  if (wide_ok) {
    typedef typename row8<T>::raw raw;
    float* mx = (float*)wide;
    double* dn = (double*)(mx + kMaxWidth);
    double* nm = dn + kMaxWidth;
    const int t = threadIdx.x, QG = 256 / NC, c8 = 8 * (t % NC), q = t / NC;
    const int64_t span = hi - lo - q;
    const int64_t nt = span > 0 ? (span + QG - 1) / QG : 0;  // this thread's tokens
    auto tok = [&](int64_t u) { return lo + q + (int64_t)QG * (u < nt ? u : nt - 1); };
    float gm[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) gm[e] = -INFINITY;
    for (int64_t u0 = 0; u0 < nt; u0 += TB) {
      raw gr[TB];
#pragma unroll
      for (int k = 0; k < TB; ++k) gr[k] = row8<T>::ld(grow(tok(u0 + k)) + c8);
#pragma unroll
      for (int k = 0; k < TB; ++k)
        if (u0 + k < nt)
#pragma unroll
          for (int e = 0; e < 8; ++e) gm[e] = fmaxf(gm[e], row8<T>::get(gr[k], e));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) mx[q * width + c8 + e] = gm[e];
    __syncthreads();
    double M[8], L[8], N[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = -INFINITY;
      for (int k = 0; k < QG; ++k) v = fmaxf(v, mx[k * width + c8 + e]);
      M[e] = v;
      L[e] = 0.0;
      N[e] = 0.0;
    }
    for (int64_t u0 = 0; u0 < nt; u0 += TB) {
      raw gr[TB], vr[TB];
#pragma unroll
      for (int k = 0; k < TB; ++k) {
        const int64_t sk = tok(u0 + k);
        gr[k] = row8<T>::ld(grow(sk) + c8);
        vr[k] = row8<T>::ld(vrow(sk) + c8);
      }
#pragma unroll
      for (int k = 0; k < TB; ++k)
        if (u0 + k < nt)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const double ex = exp((double)row8<T>::get(gr[k], e) - M[e]);
            L[e] += ex;
            N[e] += ex * (double)row8<T>::get(vr[k], e);
          }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      dn[q * width + c8 + e] = L[e];
      nm[q * width + c8 + e] = N[e];
    }
    __syncthreads();
    for (int c = t; c < width; c += 256) {
      double Lt = 0.0, Nt = 0.0;
      for (int k = 0; k < QG; ++k) {
        Lt += dn[k * width + c];
        Nt += nm[k * width + c];
      }
      const double x = Nt / Lt;
      pooled[c] = x;
      ss += x * x;
    }
  } else
  for (int c = threadIdx.x; c < width; c += blockDim.x) {
    double gmax = -INFINITY;
    for (int64_t s0 = lo; s0 < hi; s0 += TB) {
      float gv[TB];
#pragma unroll
      for (int u = 0; u < TB; ++u) gv[u] = store_t<T>::ld(grow(min(s0 + u, hi - 1)) + c);
#pragma unroll
      for (int u = 0; u < TB; ++u)
        if (s0 + u < hi) gmax = fmax(gmax, (double)gv[u]);
    }
    double num = 0.0, den = 0.0;
    for (int64_t s0 = lo; s0 < hi; s0 += TB) {
      float gv[TB], vv[TB];
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        const int64_t sc = min(s0 + u, hi - 1);
        gv[u] = store_t<T>::ld(grow(sc) + c);
        vv[u] = store_t<T>::ld(vrow(sc) + c);
      }
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        if (s0 + u < hi) {
          const double e = exp((double)gv[u] - gmax);
          den += e;
          num += e * (double)vv[u];
        }
      }
    }
    const double x = num / den;
    pooled[c] = x;
    ss += x * x;
  }
  if (norm_w != nullptr) {
    ss = wave_sum64(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    double tot = 0.0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) tot += red[i];
    const double inv = 1.0 / sqrt(tot / (double)width + (double)eps);
    for (int c = threadIdx.x; c < width; c += blockDim.x)
      pooled[c] = pooled[c] * inv * (double)norm_w[c];
  }
  __syncthreads();
  T* dst = pool + dst_row * width;
  for (int c = threadIdx.x; c < width - R; c += blockDim.x) store_t<T>::st64(dst + c, pooled[c]);
  for (int j = threadIdx.x; j < R / 2; j += blockDim.x) {
    const int c = width - R + 2 * j;
    double sn, cs;
    sincos((double)(w * m) * rope_freq(base, j, R), &sn, &cs);
    double a = pooled[c], bb = pooled[c + 1];
    rot64(a, bb, cs, sn);
    store_t<T>::st64(dst + c, a);
    store_t<T>::st64(dst + c + 1, bb);
  }
}

// Window ring append of a prefill call: a block takes kWaTok consecutive
// tokens of one sequence; the channels before the rope slice are copied with
// 16-byte moves where rows allow it, then each (token, pair) of the slice is
// rotated by one thread at the token's position (pair j = (c, c+1),
// c = D - R + 2j, times exp(i t base^(-2j/R)) [transformers PR 45616, RoPE
// apply notes; DeepSeek-V4 model page, sec. 2.3]), in float64 and rounded
// once, with the pair frequencies computed once per block (freq: R / 2
// doubles of LDS).  Any block size; block-uniform control flow.
constexpr int kWaTok = 8;

template <typename T>
__device__ __forceinline__ void window_block(const T* __restrict__ kv, T* __restrict__ ring,
                                             const Seqs& sq, int D, int R, const Rope& base,
                                             int64_t cap, double* freq, int i0, int b) {
  // padding tokens of a variable-length call are not appended
  const int nt = min(kWaTok, sq.len(b) - i0);
  if (nt <= 0) return;  // block-uniform
  const int64_t p0 = sq.pos0[b];
  const int64_t r0 = sq.row(b, i0);  // the block's tokens sit in rows r0 .. r0 + nt - 1
  for (int j = threadIdx.x; j < R / 2; j += blockDim.x) freq[j] = rope_freq(base, j, R);
  const int plain = D - R;  // channels copied unchanged
  constexpr int V = 16 / (int)sizeof(T);
  if ((D % V) == 0 && (plain % V) == 0) {
    const int per = plain / V;
    for (int e = threadIdx.x; e < nt * per; e += blockDim.x) {
      const int k = e / per, c = (e % per) * V;
      const int64_t t = p0 + i0 + k;
      *(uint4*)(ring + ((int64_t)b * cap + t % cap) * D + c) =
          *(const uint4*)(kv + (r0 + k) * D + c);
    }
  } else {
    for (int e = threadIdx.x; e < nt * plain; e += blockDim.x) {
      const int k = e / plain, c = e % plain;
      const int64_t t = p0 + i0 + k;
      ring[((int64_t)b * cap + t % cap) * D + c] = kv[(r0 + k) * D + c];
    }
  }
  __syncthreads();
  const int np = R / 2;
  for (int e = threadIdx.x; e < nt * np; e += blockDim.x) {
    const int k = e / np, j = e % np, c = D - R + 2 * j;
    const int64_t t = p0 + i0 + k;
    const T* src = kv + (r0 + k) * D;
    T* dst = ring + ((int64_t)b * cap + t % cap) * D;
    double sn, cs;
    sincos((double)t * freq[j], &sn, &cs);
    double a = store_t<T>::ld(src + c), bb = store_t<T>::ld(src + c + 1);
    rot64(a, bb, cs, sn);
    store_t<T>::st64(dst + c, a);
    store_t<T>::st64(dst + c + 1, bb);
  }
}

template <typename T>
__global__ void __launch_bounds__(256) window_append_kernel(const T* __restrict__ kv,
                                                            T* __restrict__ ring,
                                                            Seqs sq, int D, int R, Rope base,
                                                            int64_t cap) {
  extern __shared__ double freq[];  // R / 2 pair frequencies
  window_block<T>(kv, ring, sq, D, R, base, cap, freq, blockIdx.x * kWaTok, blockIdx.y);
}

// The window append beside a prefill compressor launch: its rows and ring.
template <typename T> struct WinArgsT {
  const T* kv;
  T* ring;
  int64_t cap;
  int D, R;
};

// Prefill pooling, one block of NT threads per entry (NT = 256 for windows of
// at most kTokReg tokens, else 512).  With P = width / 2 channel pairs, at
// most NT, thread (g, p) takes the pair (2p, 2p + 1) and the window's tokens
// lo + g, lo + g + G, ... (G = NT / P token groups): first
// the per-channel window maximum (the groups' maxima merged through LDS), then
// exp(gate - max) and the weighted sums over the same tokens (merged through
// LDS).  These are the float64 terms of a serial pass, summed in another
// order.  Wider rows take several pairs per thread.  Then the
// optional RMSNorm over the entry and the rotation at position w m.
constexpr int kCmpT = 512;

template <typename T>
__device__ __forceinline__ void ld2(const T* p, double& a, double& b);
template <>
__device__ __forceinline__ void ld2<bf16_t>(const bf16_t* p, double& a, double& b) {
  const uint32_t u = *(const uint32_t*)p;
  a = bf16_to_f32((bf16_t)(u & 0xffffu));
  b = bf16_to_f32((bf16_t)(u >> 16));
}
template <>
__device__ __forceinline__ void ld2<float>(const float* p, double& a, double& b) {
  const float2 f = *(const float2*)p;
  a = f.x;
  b = f.y;
}

// A channel pair as stored: two bf16 in one word, or two floats.
template <typename T> struct pair_t;
template <> struct pair_t<bf16_t> {
  typedef uint32_t raw;
  static __device__ __forceinline__ raw ld(const bf16_t* p) { return *(const uint32_t*)p; }
  static __device__ __forceinline__ void cvt(raw u, double& a, double& b) {
    a = bf16_to_f32((bf16_t)(u & 0xffffu));
    b = bf16_to_f32((bf16_t)(u >> 16));
  }
};
template <> struct pair_t<float> {
  typedef float2 raw;
  static __device__ __forceinline__ raw ld(const float* p) { return *(const float2*)p; }
  static __device__ __forceinline__ void cvt(raw u, double& a, double& b) {
    a = u.x;
    b = u.y;
  }
};
// Tokens a thread of the register path holds (window of at most G * kTokReg).
constexpr int kTokReg = 8;

// One stream of a prefill compressor launch: its token rows, state slots,
// pool, width and rope channels.  A launch takes up to two streams (main and
// indexer, blockIdx.z), so the indexer's entries fill the chip beside the
// main ones instead of waiting for a launch of their own.
template <typename T> struct CmpStream {
  const T* kv;
  const T* gate;
  const float* norm_w;
  T* st_kv;
  T* st_gate;
  T* pool;
  int width, R;
};

// Keep the raw rows of the last (1 + overlap) m = Ls positions of sequence b
// for later calls: slot j of the block (j < Ls) copies one row of kv and
// gate into the stream's state ring.  It overwrites slots the entries of the
// same call read when the call starts past position 0, so it then runs after
// them (its own launch); a call that starts at 0 reads no state and runs it
// in the entries' launch.
template <typename T>
__device__ __forceinline__ void state_rows(const CmpStream<T>& cs, const Seqs& sq, int Ls, int j,
                                           int b) {
  const int width = cs.width;
  const int64_t p0 = sq.pos0[b];
  // the last Ls valid positions (padding rows are never kept)
  const int64_t s = p0 + sq.len(b) - Ls + j;
  if (j >= Ls || s < p0) return;
  const T* src_kv = cs.kv + (sq.row(b, 0) + (s - p0)) * width;
  const T* src_g = cs.gate + (sq.row(b, 0) + (s - p0)) * width;
  T* dk = cs.st_kv + ((int64_t)b * Ls + (s % Ls)) * width;
  T* dg = cs.st_gate + ((int64_t)b * Ls + (s % Ls)) * width;
  for (int c = threadIdx.x; c < width; c += blockDim.x) {
    dk[c] = src_kv[c];
    dg[c] = src_g[c];
  }
}

template <typename T, int NT>
__global__ void __launch_bounds__(NT) compress_entry_kernel(CmpStream<T> s0, CmpStream<T> s1,
                                                            WinArgsT<T> wa, int wz, int sz0,
                                                            float eps,
                                                            Seqs sq, Rope base, int m,
                                                            int overlap, int64_t pool_cap) {
  __shared__ double pooled[kMaxWidth];
  __shared__ double pa[NT][2], pb[NT][2];
  __shared__ double red[NT / 64];
  constexpr int kTab = 128;              // rope pairs kept in the table
  __shared__ double2 csr[kTab];          // (cos, sin) of the rope pairs at w m
  if (sz0 >= 0 && (int)blockIdx.z >= sz0) {  // the state updates' blocks (block-uniform)
    state_rows<T>((int)blockIdx.z == sz0 ? s0 : s1, sq, (1 + overlap) * m, blockIdx.x, blockIdx.y);
    return;
  }
  if ((int)blockIdx.z == wz) {  // the window append's blocks (block-uniform)
    window_block<T>(wa.kv, wa.ring, sq, wa.D, wa.R, base, wa.cap, pooled, blockIdx.x * kWaTok,
                    blockIdx.y);
    return;
  }
  const CmpStream<T> cs = blockIdx.z ? s1 : s0;  // uniform
  const T* __restrict__ kv = cs.kv;
  const T* __restrict__ gate = cs.gate;
  const float* __restrict__ norm_w = cs.norm_w;
  const T* __restrict__ st_kv = cs.st_kv;
  const T* __restrict__ st_gate = cs.st_gate;
  T* __restrict__ pool = cs.pool;
  const int width = cs.width, R = cs.R;
  const int b = blockIdx.y;
  const int64_t p0 = sq.pos0[b];
  const int64_t w = p0 / m + blockIdx.x;
  // entries that close within the sequence's valid tokens
  const int nl = sq.len(b);
  if (w >= (p0 + nl) / m || w >= pool_cap) return;  // block-uniform
  const int Ls = (1 + overlap) * m, tid = threadIdx.x;
  const int64_t lo = max((w - overlap) * (int64_t)m, (int64_t)0), hi = (w + 1) * (int64_t)m;
  const T* kv_b = kv + sq.row(b, 0) * width;  // the call's token rows of sequence b
  const T* g_b = gate + sq.row(b, 0) * width;
  const T* skv_b = st_kv + (int64_t)b * Ls * width;
  const T* sg_b = st_gate + (int64_t)b * Ls * width;
  auto row = [&](const T* cur, const T* st, int64_t s) {
    return s >= p0 ? cur + (s - p0) * width : st + (int64_t)(s % Ls) * width;
  };
  const int P = width / 2;
  // the rope table of the entry, while the loads below are in flight
  auto rope_table = [&]() __attribute__((always_inline)) {
    for (int j = tid; j < R / 2 && j < kTab; j += NT) {
      double sn, cs;
      sincos((double)(w * m) * rope_freq(base, j, R), &sn, &cs);
      csr[j] = make_double2(cs, sn);
    }
  };
  if (P <= NT && hi - lo <= (int64_t)(NT / P) * kTokReg) {
    // register path (windows of at most G * kTokReg tokens, e.g. the CSA
    // window of 8): every thread loads its tokens' gate and kv pairs once,
    // then the maximum and the sums come from registers
    typedef typename pair_t<T>::raw raw;
    const int G = NT / P, p = tid % P, g = tid / P;
    const bool act = g < G;
    raw gq[kTokReg], vq[kTokReg];
#pragma unroll
    for (int u = 0; u < kTokReg; ++u) {
      const int64_t s = lo + g + (int64_t)u * G;
      if (act && s < hi) {
        gq[u] = pair_t<T>::ld(row(g_b, sg_b, s) + 2 * p);
        vq[u] = pair_t<T>::ld(row(kv_b, skv_b, s) + 2 * p);
      }
    }
    rope_table();
    double mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
    for (int u = 0; u < kTokReg; ++u) {
      if (act && lo + g + (int64_t)u * G < hi) {
        double a, c;
        pair_t<T>::cvt(gq[u], a, c);
        mx0 = fmax(mx0, a);
        mx1 = fmax(mx1, c);
      }
    }
    pa[tid][0] = mx0;
    pa[tid][1] = mx1;
    __syncthreads();
    double M0 = -INFINITY, M1 = -INFINITY;
    for (int k = 0; k < G; ++k) {
      M0 = fmax(M0, pa[p + k * P][0]);
      M1 = fmax(M1, pa[p + k * P][1]);
    }
    double l0 = 0.0, l1 = 0.0, n0 = 0.0, n1 = 0.0;
#pragma unroll
    for (int u = 0; u < kTokReg; ++u) {
      if (act && lo + g + (int64_t)u * G < hi) {
        double ga, gc, va, vc;
        pair_t<T>::cvt(gq[u], ga, gc);
        pair_t<T>::cvt(vq[u], va, vc);
        const double e0 = exp(ga - M0), e1 = exp(gc - M1);
        l0 += e0;
        l1 += e1;
        n0 += e0 * va;
        n1 += e1 * vc;
      }
    }
    __syncthreads();  // the maxima are read
    pa[tid][0] = l0;
    pa[tid][1] = l1;
    pb[tid][0] = n0;
    pb[tid][1] = n1;
    __syncthreads();
    if (tid < P) {
      double L0 = 0.0, L1 = 0.0, N0 = 0.0, N1 = 0.0;
      for (int k = 0; k < G; ++k) {
        L0 += pa[p + k * P][0];
        L1 += pa[p + k * P][1];
        N0 += pb[p + k * P][0];
        N1 += pb[p + k * P][1];
      }
      pooled[2 * p] = N0 / L0;
      pooled[2 * p + 1] = N1 / L1;
    }
  } else if (P <= NT) {
    rope_table();
    const int G = NT / P, p = tid % P, g = tid / P;
    const bool act = g < G;
    // the thread's tokens lo + g, lo + g + G, ... go eight at a time with
    // unconditional loads (past the window: its last token again, masked
    // out), so that eight share one latency instead of one each
    typedef typename pair_t<T>::raw raw;
    const int64_t span = hi - lo - g;
    const int64_t nt = act && span > 0 ? (span + G - 1) / G : 0;
    auto tk = [&](int64_t u) { return lo + g + (int64_t)G * (u < nt ? u : nt - 1); };
    double mx0 = -INFINITY, mx1 = -INFINITY;
    for (int64_t u0 = 0; u0 < nt; u0 += kTokReg) {
      raw gq[kTokReg];
#pragma unroll
      for (int u = 0; u < kTokReg; ++u) gq[u] = pair_t<T>::ld(row(g_b, sg_b, tk(u0 + u)) + 2 * p);
#pragma unroll
      for (int u = 0; u < kTokReg; ++u) {
        if (u0 + u < nt) {
          double a, c;
          pair_t<T>::cvt(gq[u], a, c);
          mx0 = fmax(mx0, a);
          mx1 = fmax(mx1, c);
        }
      }
    }
    pa[tid][0] = mx0;
    pa[tid][1] = mx1;
    __syncthreads();
    double M0 = -INFINITY, M1 = -INFINITY;
    for (int k = 0; k < G; ++k) {
      M0 = fmax(M0, pa[p + k * P][0]);
      M1 = fmax(M1, pa[p + k * P][1]);
    }
    double l0 = 0.0, l1 = 0.0, n0 = 0.0, n1 = 0.0;
    for (int64_t u0 = 0; u0 < nt; u0 += kTokReg) {
      raw gq[kTokReg], vq[kTokReg];
#pragma unroll
      for (int u = 0; u < kTokReg; ++u) {
        const int64_t sk = tk(u0 + u);
        gq[u] = pair_t<T>::ld(row(g_b, sg_b, sk) + 2 * p);
        vq[u] = pair_t<T>::ld(row(kv_b, skv_b, sk) + 2 * p);
      }
#pragma unroll
      for (int u = 0; u < kTokReg; ++u) {
        if (u0 + u < nt) {
          double ga, gc, va, vc;
          pair_t<T>::cvt(gq[u], ga, gc);
          pair_t<T>::cvt(vq[u], va, vc);
          const double e0 = exp(ga - M0), e1 = exp(gc - M1);
          l0 += e0;
          l1 += e1;
          n0 += e0 * va;
          n1 += e1 * vc;
        }
      }
    }
    __syncthreads();  // the maxima are read
    pa[tid][0] = l0;
    pa[tid][1] = l1;
    pb[tid][0] = n0;
    pb[tid][1] = n1;
    __syncthreads();
    if (tid < P) {
      double L0 = 0.0, L1 = 0.0, N0 = 0.0, N1 = 0.0;
      for (int k = 0; k < G; ++k) {
        L0 += pa[p + k * P][0];
        L1 += pa[p + k * P][1];
        N0 += pb[p + k * P][0];
        N1 += pb[p + k * P][1];
      }
      pooled[2 * p] = N0 / L0;
      pooled[2 * p + 1] = N1 / L1;
    }
  } else {
    rope_table();
    for (int p = tid; p < P; p += NT) {
      double mx0 = -INFINITY, mx1 = -INFINITY;
      for (int64_t s = lo; s < hi; ++s) {
        double a, c;
        ld2<T>(row(g_b, sg_b, s) + 2 * p, a, c);
        mx0 = fmax(mx0, a);
        mx1 = fmax(mx1, c);
      }
      double l0 = 0.0, l1 = 0.0, n0 = 0.0, n1 = 0.0;
      for (int64_t s = lo; s < hi; ++s) {
        double ga, gc, va, vc;
        ld2<T>(row(g_b, sg_b, s) + 2 * p, ga, gc);
        ld2<T>(row(kv_b, skv_b, s) + 2 * p, va, vc);
        const double e0 = exp(ga - mx0), e1 = exp(gc - mx1);
        l0 += e0;
        l1 += e1;
        n0 += e0 * va;
        n1 += e1 * vc;
      }
      pooled[2 * p] = n0 / l0;
      pooled[2 * p + 1] = n1 / l1;
    }
  }
  __syncthreads();
  if (norm_w != nullptr) {
    double ss = 0.0;
    for (int c = tid; c < width; c += NT) ss += pooled[c] * pooled[c];
    ss = wave_sum64(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    double tot = 0.0;
    for (int k = 0; k < NT / 64; ++k) tot += red[k];
    const double inv = 1.0 / sqrt(tot / (double)width + (double)eps);
    for (int c = tid; c < width; c += NT) pooled[c] = pooled[c] * inv * (double)norm_w[c];
    __syncthreads();
  }
  T* dst = pool + sq.prow(b, w, pool_cap) * width;
  for (int c = tid; c < width - R; c += NT) store_t<T>::st64(dst + c, pooled[c]);
  for (int j = tid; j < R / 2; j += NT) {
    const int c = width - R + 2 * j;
    double cs, sn;
    if (j < kTab) {
      const double2 cz = csr[j];
      cs = cz.x;
      sn = cz.y;
    } else {
      sincos((double)(w * m) * rope_freq(base, j, R), &sn, &cs);
    }
    double a = pooled[c], bb = pooled[c + 1];
    rot64(a, bb, cs, sn);
    store_t<T>::st64(dst + c, a);
    store_t<T>::st64(dst + c + 1, bb);
  }
}

// One new token per sequence (decode): the entry that closes at it, if any,
// then the token's raw row into its state slot, in one launch.  The entry's
// earlier tokens sit in the other Ls - 1 slots, so the slot written here
// (p0 mod Ls, holding position p0 - Ls) is never one the entry reads.
template <typename T>
__device__ __forceinline__ void compress_one_seq(
    const T* __restrict__ kv, const T* __restrict__ gate, const float* __restrict__ norm_w,
    float eps, T* __restrict__ st_kv, T* __restrict__ st_gate, T* __restrict__ pool,
    const Seqs& sq, int b, int width, int R, const Rope& base, int m, int overlap,
    int64_t pool_cap, double* pooled, double* red, void* wide) {
  const int64_t p0 = sq.pos0[b];
  const int Ls = (1 + overlap) * m;
  const int64_t w = p0 / m;
  const int64_t r = sq.row(b, 0);
  if ((p0 + 1) % m == 0 && w < pool_cap)  // uniform per block
    pool_entry<T>(kv, gate, norm_w, eps, st_kv, st_gate, pool, b, p0, w, r,
                  sq.prow(b, w, pool_cap), width, R, base, m, overlap, pooled, red, wide);
  const T* src_kv = kv + r * width;
  const T* src_g = gate + r * width;
  T* dk = st_kv + ((int64_t)b * Ls + p0 % Ls) * width;
  T* dg = st_gate + ((int64_t)b * Ls + p0 % Ls) * width;
  for (int c = threadIdx.x; c < width; c += blockDim.x) {
    dk[c] = src_kv[c];
    dg[c] = src_g[c];
  }
}

template <typename T>
__global__ void __launch_bounds__(256) compress_one_kernel(
    const T* __restrict__ kv, const T* __restrict__ gate, const float* __restrict__ norm_w,
    float eps, T* __restrict__ st_kv, T* __restrict__ st_gate, T* __restrict__ pool, Seqs sq,
    int width, int R, Rope base, int m, int overlap, int64_t pool_cap) {
  __shared__ double pooled[kMaxWidth];
  __shared__ double red[256 / 64];
  __shared__ __attribute__((aligned(16))) unsigned char wide[kPoolWideBytes];
  const int b = blockIdx.x;
  if (sq.len(b) == 0) return;  // a padding token: nothing to record
  compress_one_seq<T>(kv, gate, norm_w, eps, st_kv, st_gate, pool, sq, b, width, R, base, m,
                      overlap, pool_cap, pooled, red, wide);
}

// The token's K=V row appended to sequence b's window ring (slot = position
// mod cap): channels before the rope slice copied, the slice rotated at the
// token's position in float64 and rounded once (as window_append_kernel).
template <typename T>
__device__ __forceinline__ void window_one_seq(const T* __restrict__ kv, T* __restrict__ ring,
                                               const Seqs& sq, int b, int D, int R,
                                               const Rope& base, int64_t cap, double* freq) {
  const int64_t t = sq.pos0[b];
  const T* src = kv + sq.row(b, 0) * D;
  T* dst = ring + ((int64_t)b * cap + t % cap) * D;
  for (int j = threadIdx.x; j < R / 2; j += blockDim.x) freq[j] = rope_freq(base, j, R);
  for (int c = threadIdx.x; c < D - R; c += blockDim.x) dst[c] = src[c];
  __syncthreads();
  for (int j = threadIdx.x; j < R / 2; j += blockDim.x) {
    const int c = D - R + 2 * j;
    double sn, cs;
    sincos((double)t * freq[j], &sn, &cs);
    double a = store_t<T>::ld(src + c), bb = store_t<T>::ld(src + c + 1);
    rot64(a, bb, cs, sn);
    store_t<T>::st64(dst + c, a);
    store_t<T>::st64(dst + c + 1, bb);
  }
}

// A decode step's cache updates in one launch: block (b, role) takes
// sequence b's new token into the window ring (role 0), the main
// compressor (role 1) or the indexer's compressor (role 2).
template <typename T>
__global__ void __launch_bounds__(256) cache_update_one_kernel(
    const T* __restrict__ kv, T* __restrict__ ring, int64_t cap, const T* __restrict__ ckv,
    const T* __restrict__ cgate, const float* __restrict__ norm_w, T* __restrict__ st_kv,
    T* __restrict__ st_gate, T* __restrict__ pool, const T* __restrict__ ikv,
    const T* __restrict__ igate, const float* __restrict__ inorm_w, T* __restrict__ ist_kv,
    T* __restrict__ ist_gate, T* __restrict__ ipool, float eps, Seqs sq, int D, int R, int Di,
    int Ri, Rope base, int m, int overlap, int64_t pool_cap) {
  __shared__ double pooled[kMaxWidth];
  __shared__ double red[256 / 64];
  __shared__ __attribute__((aligned(16))) unsigned char wide[kPoolWideBytes];
  const int b = blockIdx.x;
  if (sq.len(b) == 0) return;  // a padding token: nothing to record
  if (blockIdx.y == 0)
    window_one_seq<T>(kv, ring, sq, b, D, R, base, cap, pooled);
  else if (blockIdx.y == 1)
    compress_one_seq<T>(ckv, cgate, norm_w, eps, st_kv, st_gate, pool, sq, b, D, R, base, m,
                        overlap, pool_cap, pooled, red, wide);
  else
    compress_one_seq<T>(ikv, igate, inorm_w, eps, ist_kv, ist_gate, ipool, sq, b, Di, Ri, base,
                        m, overlap, pool_cap, pooled, red, wide);
}

// The state update as a launch of its own, after the entries' launch.
template <typename T>
__global__ void __launch_bounds__(256) state_update_kernel(CmpStream<T> s0, CmpStream<T> s1,
                                                           Seqs sq, int Ls) {
  state_rows<T>(blockIdx.z ? s1 : s0, sq, Ls, blockIdx.x, blockIdx.y);
}

hipError_t launch_window_append(const Layer& L, const Batch& bt, const void* kv, void* ring,
                                int64_t cap, hipStream_t s) {
  dim3 grid((bt.n + kWaTok - 1) / kWaTok, bt.B);
  const size_t shm = (size_t)(L.R / 2) * sizeof(double);
  if (L.dtype == 1)
    window_append_kernel<bf16_t><<<grid, 256, shm, s>>>((const bf16_t*)kv, (bf16_t*)ring,
                                                        seqs_of(bt), L.D, L.R, L.base, cap);
  else
    window_append_kernel<float><<<grid, 256, shm, s>>>((const float*)kv, (float*)ring,
                                                       seqs_of(bt), L.D, L.R, L.base, cap);
  return hipGetLastError();
}

hipError_t launch_compress(const Layer& L, const Batch& bt, int width, int rope_dim,
                           const void* kv, const void* gate, const float* norm_w, float eps,
                           void* st_kv, void* st_gate, void* pool, int64_t pool_cap,
                           hipStream_t s, const CmpArgs* second, const WinArgs* win) {
  const int m = L.m, Ls = (1 + L.overlap) * m;
  const Seqs sq = seqs_of(bt);
  if (bt.n == 1) {
    hipError_t e = hipSuccess;
    if (win) e = launch_window_append(L, bt, win->kv, win->ring, win->cap, s);
    if (e != hipSuccess) return e;
    if (L.dtype == 1)
      compress_one_kernel<bf16_t><<<bt.B, 256, 0, s>>>(
          (const bf16_t*)kv, (const bf16_t*)gate, norm_w, eps, (bf16_t*)st_kv, (bf16_t*)st_gate,
          (bf16_t*)pool, sq, width, rope_dim, L.base, m, L.overlap, pool_cap);
    else
      compress_one_kernel<float><<<bt.B, 256, 0, s>>>(
          (const float*)kv, (const float*)gate, norm_w, eps, (float*)st_kv, (float*)st_gate,
          (float*)pool, sq, width, rope_dim, L.base, m, L.overlap, pool_cap);
    e = hipGetLastError();
    if (e != hipSuccess || !second) return e;
    return launch_compress(L, bt, second->width, second->rope_dim, second->kv, second->gate,
                           second->norm_w, eps, second->st_kv, second->st_gate, second->pool,
                           pool_cap, s, nullptr, nullptr);
  }
  // windows that fit one thread's registers (the CSA window of 8) take
  // 256-thread blocks, one channel pair per thread: twice the blocks
  // resident per CU as with 512 threads, and no merge of token groups
  const bool narrow = (1 + L.overlap) * m <= kTokReg && width <= 512 &&
                      (!second || second->width <= 512);
  // the window append joins the launch there; with HCA's few long entries
  // its 8-token blocks would outnumber them 16 to 1 (one launch: 135-162
  // us, two: 113-157), so it keeps its own launch
  if (win && !narrow) {
    const hipError_t e = launch_window_append(L, bt, win->kv, win->ring, win->cap, s);
    if (e != hipSuccess) return e;
    win = nullptr;
  }
  // grid.z: the streams' entries (z = 0, 1), then the window append's
  // blocks of kWaTok tokens (z = ns) if it comes along
  const int ns = second ? 2 : 1;
  const int max_entries = bt.n / m + 1;
  const int wblocks = win ? (bt.n + kWaTok - 1) / kWaTok : 0;
  // a call from position 0 reads no state: the state updates join the
  // launch (grid.z after the entries and the window append)
  const bool fold_state = bt.pos0_max == 0;
  const int nz = ns + (win ? 1 : 0);
  dim3 g1(max(max(max_entries, wblocks), fold_state ? Ls : 0), bt.B, nz + (fold_state ? ns : 0));
  dim3 g2(Ls, bt.B, ns);
  auto stream_of = [&](auto* tag, int w, int r, const void* k, const void* g, const float* nw,
                       void* sk, void* sg, void* pl) {
    typedef std::remove_pointer_t<decltype(tag)> T;
    return CmpStream<T>{(const T*)k, (const T*)g, nw, (T*)sk, (T*)sg, (T*)pl, w, r};
  };
  auto launch = [&](auto* tag) {
    typedef std::remove_pointer_t<decltype(tag)> T;
    const CmpStream<T> a0 = stream_of(tag, width, rope_dim, kv, gate, norm_w, st_kv, st_gate, pool);
    const CmpStream<T> a1 =
        second ? stream_of(tag, second->width, second->rope_dim, second->kv, second->gate,
                           second->norm_w, second->st_kv, second->st_gate, second->pool)
               : a0;
    const WinArgsT<T> wa =
        win ? WinArgsT<T>{(const T*)win->kv, (T*)win->ring, win->cap, L.D, L.R}
            : WinArgsT<T>{nullptr, nullptr, 1, L.D, L.R};
    const int wz = win ? ns : -1, sz0 = fold_state ? nz : -1;
    if (narrow)
      compress_entry_kernel<T, 256><<<g1, 256, 0, s>>>(a0, a1, wa, wz, sz0, eps, sq, L.base, m,
                                                       L.overlap, pool_cap);
    else
      compress_entry_kernel<T, kCmpT><<<g1, kCmpT, 0, s>>>(a0, a1, wa, wz, sz0, eps, sq, L.base,
                                                           m, L.overlap, pool_cap);
    if (!fold_state) state_update_kernel<T><<<g2, 256, 0, s>>>(a0, a1, sq, Ls);
  };
  if (L.dtype == 1)
    launch((bf16_t*)nullptr);
  else
    launch((float*)nullptr);
  return hipGetLastError();
}

hipError_t launch_cache_update_one(const Layer& L, const Batch& bt, const void* kv, void* ring,
                                   int64_t cap, const void* ckv, const void* cgate,
                                   const float* norm_w, void* st_kv, void* st_gate, void* pool,
                                   const void* ikv, const void* igate, const float* inorm_w,
                                   void* ist_kv, void* ist_gate, void* ipool, int64_t pool_cap,
                                   float eps, int roles, hipStream_t s) {
  const dim3 grid(bt.B, roles);
  const Seqs sq = seqs_of(bt);
#define CSA_CU_LAUNCH(T)                                                                       \
  cache_update_one_kernel<T><<<grid, 256, 0, s>>>(                                            \
      (const T*)kv, (T*)ring, cap, (const T*)ckv, (const T*)cgate, norm_w, (T*)st_kv,          \
      (T*)st_gate, (T*)pool, (const T*)ikv, (const T*)igate, inorm_w, (T*)ist_kv, (T*)ist_gate, \
      (T*)ipool, eps, sq, L.D, L.R, L.Di, L.Ri, L.base, L.m, L.overlap, pool_cap)
  if (L.dtype == 1)
    CSA_CU_LAUNCH(bf16_t);
  else
    CSA_CU_LAUNCH(float);
#undef CSA_CU_LAUNCH
  return hipGetLastError();
}

}  // namespace csa
