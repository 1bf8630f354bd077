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
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

constexpr int kMaxWidth = 2048;

// Entry w of sequence b, one block serially over the window (the one-token
// decode call; pooled and red in LDS).
template <typename T>
__device__ __forceinline__ void pool_entry(
    const T* __restrict__ kv, const T* __restrict__ gate, const float* __restrict__ norm_w,
    float eps, const T* __restrict__ st_kv, const T* __restrict__ st_gate, T* __restrict__ pool,
    int b, int64_t p0, int64_t w, int n_new, int width, int R, Rope base, int m, int overlap,
    int64_t pool_cap, double* pooled, double* red) {
  const int Ls = (1 + overlap) * m;
  const int64_t lo = max((w - overlap) * (int64_t)m, (int64_t)0), hi = (w + 1) * (int64_t)m;
  const T* kv_b = kv + (int64_t)b * n_new * width;
  const T* g_b = gate + (int64_t)b * n_new * width;
  const T* skv_b = st_kv + (int64_t)b * Ls * width;
  const T* sg_b = st_gate + (int64_t)b * Ls * width;
  double ss = 0.0;
  for (int c = threadIdx.x; c < width; c += blockDim.x) {
    double gmax = -INFINITY;
    for (int64_t s = lo; s < hi; ++s) {
      const T* g = s >= p0 ? g_b + (s - p0) * width : sg_b + (int64_t)(s % Ls) * width;
      gmax = fmax(gmax, (double)store_t<T>::ld(g + c));
    }
    double num = 0.0, den = 0.0;
    for (int64_t s = lo; s < hi; ++s) {
      const T* g = s >= p0 ? g_b + (s - p0) * width : sg_b + (int64_t)(s % Ls) * width;
      const T* v = s >= p0 ? kv_b + (s - p0) * width : skv_b + (int64_t)(s % Ls) * width;
      const double e = exp((double)store_t<T>::ld(g + c) - gmax);
      den += e;
      num += e * (double)store_t<T>::ld(v + c);
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
  T* dst = pool + ((int64_t)b * pool_cap + w) * width;
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

// Prefill pooling, one 512-thread block per entry.  With P = width / 2
// channel pairs below 512, thread (g, p) takes the pair (2p, 2p + 1) and the
// window's tokens lo + g, lo + g + G, ... (G = 512 / P token groups): first
// the per-channel window maximum (the groups' maxima merged through LDS), then
// exp(gate - max) and the weighted sums over the same tokens (merged through
// LDS).  These are the float64 terms of a serial pass, summed in another
// order.  Wider rows take G = 1 and several pairs per thread.  Then the
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

template <typename T>
__global__ void __launch_bounds__(kCmpT) compress_entry_kernel(
    const T* __restrict__ kv, const T* __restrict__ gate, const float* __restrict__ norm_w,
    float eps, const T* __restrict__ st_kv, const T* __restrict__ st_gate, T* __restrict__ pool,
    const int64_t* __restrict__ pos0, const int32_t* __restrict__ nvalid, int n_new, int width,
    int R, Rope base, int m, int overlap, int64_t pool_cap) {
  __shared__ double pooled[kMaxWidth];
  __shared__ double pa[kCmpT][2], pb[kCmpT][2];
  __shared__ double red[kCmpT / 64];
  const int b = blockIdx.y;
  const int64_t p0 = pos0[b];
  const int64_t w = p0 / m + blockIdx.x;
  // entries that close within the sequence's valid tokens
  const int nl = valid_tokens(nvalid, b, n_new);
  if (w >= (p0 + nl) / m || w >= pool_cap) return;  // block-uniform
  const int Ls = (1 + overlap) * m, tid = threadIdx.x;
  const int64_t lo = max((w - overlap) * (int64_t)m, (int64_t)0), hi = (w + 1) * (int64_t)m;
  const T* kv_b = kv + (int64_t)b * n_new * width;
  const T* g_b = gate + (int64_t)b * n_new * width;
  const T* skv_b = st_kv + (int64_t)b * Ls * width;
  const T* sg_b = st_gate + (int64_t)b * Ls * width;
  auto row = [&](const T* cur, const T* st, int64_t s) {
    return s >= p0 ? cur + (s - p0) * width : st + (int64_t)(s % Ls) * width;
  };
  const int P = width / 2;
  if (P < kCmpT) {
    const int G = kCmpT / P, p = tid % P, g = tid / P;
    const bool act = g < G;
    double mx0 = -INFINITY, mx1 = -INFINITY;
    if (act)
      for (int64_t s = lo + g; s < hi; s += G) {
        double a, c;
        ld2<T>(row(g_b, sg_b, s) + 2 * p, a, c);
        mx0 = fmax(mx0, a);
        mx1 = fmax(mx1, c);
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
    if (act)
      for (int64_t s = lo + g; s < hi; s += G) {
        double ga, gc, va, vc;
        ld2<T>(row(g_b, sg_b, s) + 2 * p, ga, gc);
        ld2<T>(row(kv_b, skv_b, s) + 2 * p, va, vc);
        const double e0 = exp(ga - M0), e1 = exp(gc - M1);
        l0 += e0;
        l1 += e1;
        n0 += e0 * va;
        n1 += e1 * vc;
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
    for (int p = tid; p < P; p += kCmpT) {
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
    for (int c = tid; c < width; c += kCmpT) ss += pooled[c] * pooled[c];
    ss = wave_sum64(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    double tot = 0.0;
    for (int k = 0; k < kCmpT / 64; ++k) tot += red[k];
    const double inv = 1.0 / sqrt(tot / (double)width + (double)eps);
    for (int c = tid; c < width; c += kCmpT) pooled[c] = pooled[c] * inv * (double)norm_w[c];
    __syncthreads();
  }
  T* dst = pool + ((int64_t)b * pool_cap + w) * width;
  for (int c = tid; c < width - R; c += kCmpT) store_t<T>::st64(dst + c, pooled[c]);
  for (int j = tid; j < R / 2; j += kCmpT) {
    const int c = width - R + 2 * j;
    double sn, cs;
    sincos((double)(w * m) * rope_freq(base, j, R), &sn, &cs);
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
__global__ void __launch_bounds__(256) compress_one_kernel(
    const T* __restrict__ kv, const T* __restrict__ gate, const float* __restrict__ norm_w,
    float eps, T* __restrict__ st_kv, T* __restrict__ st_gate, T* __restrict__ pool,
    const int64_t* __restrict__ pos0, const int32_t* __restrict__ nvalid, int width, int R,
    Rope base, int m, int overlap, int64_t pool_cap) {
  __shared__ double pooled[kMaxWidth];
  __shared__ double red[256 / 64];
  const int b = blockIdx.x;
  if (valid_tokens(nvalid, b, 1) == 0) return;  // a padding token: nothing to record
  const int64_t p0 = pos0[b];
  const int Ls = (1 + overlap) * m;
  const int64_t w = p0 / m;
  if ((p0 + 1) % m == 0 && w < pool_cap)  // uniform per block
    pool_entry<T>(kv, gate, norm_w, eps, st_kv, st_gate, pool, b, p0, w, 1, width, R, base, m,
                  overlap, pool_cap, pooled, red);
  const T* src_kv = kv + (int64_t)b * width;
  const T* src_g = gate + (int64_t)b * width;
  T* dk = st_kv + ((int64_t)b * Ls + p0 % Ls) * width;
  T* dg = st_gate + ((int64_t)b * Ls + p0 % Ls) * width;
  for (int c = threadIdx.x; c < width; c += blockDim.x) {
    dk[c] = src_kv[c];
    dg[c] = src_g[c];
  }
}

// Keep the raw rows of the last (1 + overlap) m positions for later calls.
// Runs after compress_entry_kernel on the same stream (it overwrites slots that
// kernel reads).
template <typename T>
__global__ void __launch_bounds__(256) state_update_kernel(const T* __restrict__ kv,
                                                           const T* __restrict__ gate,
                                                           T* __restrict__ st_kv,
                                                           T* __restrict__ st_gate,
                                                           const int64_t* __restrict__ pos0,
                                                           const int32_t* __restrict__ nvalid,
                                                           int n_new, int width, int Ls) {
  const int b = blockIdx.y;
  const int64_t p0 = pos0[b];
  // the last Ls valid positions (padding rows are never kept)
  const int64_t s = p0 + valid_tokens(nvalid, b, n_new) - Ls + blockIdx.x;
  if (s < p0) return;
  const T* src_kv = kv + ((int64_t)b * n_new + (s - p0)) * width;
  const T* src_g = gate + ((int64_t)b * n_new + (s - p0)) * width;
  T* dk = st_kv + ((int64_t)b * Ls + (s % Ls)) * width;
  T* dg = st_gate + ((int64_t)b * Ls + (s % Ls)) * width;
  for (int c = threadIdx.x; c < width; c += blockDim.x) {
    dk[c] = src_kv[c];
    dg[c] = src_g[c];
  }
}

hipError_t launch_compress(const Layer& L, const Batch& bt, int width, int rope_dim,
                           const void* kv, const void* gate, const float* norm_w, float eps,
                           void* st_kv, void* st_gate, void* pool, int64_t pool_cap,
                           hipStream_t s) {
  const int m = L.m, Ls = (1 + L.overlap) * m;
  const int max_entries = bt.n / m + 1;
  dim3 g1(max_entries, bt.B), g2(Ls, bt.B);
  if (bt.n == 1) {
    if (L.dtype == 1)
      compress_one_kernel<bf16_t><<<bt.B, 256, 0, s>>>(
          (const bf16_t*)kv, (const bf16_t*)gate, norm_w, eps, (bf16_t*)st_kv, (bf16_t*)st_gate,
          (bf16_t*)pool, bt.pos0, bt.nvalid, width, rope_dim, L.base, m, L.overlap, pool_cap);
    else
      compress_one_kernel<float><<<bt.B, 256, 0, s>>>(
          (const float*)kv, (const float*)gate, norm_w, eps, (float*)st_kv, (float*)st_gate,
          (float*)pool, bt.pos0, bt.nvalid, width, rope_dim, L.base, m, L.overlap, pool_cap);
    return hipGetLastError();
  }
  if (L.dtype == 1) {
    compress_entry_kernel<bf16_t><<<g1, kCmpT, 0, s>>>(
        (const bf16_t*)kv, (const bf16_t*)gate, norm_w, eps, (const bf16_t*)st_kv,
        (const bf16_t*)st_gate, (bf16_t*)pool, bt.pos0, bt.nvalid, bt.n, width, rope_dim, L.base,
        m, L.overlap, pool_cap);
    state_update_kernel<bf16_t><<<g2, 256, 0, s>>>((const bf16_t*)kv, (const bf16_t*)gate,
                                                   (bf16_t*)st_kv, (bf16_t*)st_gate, bt.pos0,
                                                   bt.nvalid, bt.n, width, Ls);
  } else {
    compress_entry_kernel<float><<<g1, kCmpT, 0, s>>>((const float*)kv, (const float*)gate, norm_w, eps,
                                              (const float*)st_kv, (const float*)st_gate,
                                              (float*)pool, bt.pos0, bt.nvalid, bt.n, width,
                                              rope_dim, L.base, m, L.overlap, pool_cap);
    state_update_kernel<float><<<g2, 256, 0, s>>>((const float*)kv, (const float*)gate,
                                                  (float*)st_kv, (float*)st_gate, bt.pos0,
                                                  bt.nvalid, bt.n, width, Ls);
  }
  return hipGetLastError();
}

}  // namespace csa
