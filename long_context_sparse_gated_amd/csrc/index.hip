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
//  * index_prefill_mfma: H_I = 64, D_I = 128, bf16.  A block takes 8
//    consecutive queries (2 per wave, rotated query fragments held in VGPRs)
//    and streams the visible keys through LDS in tiles of 64 keys shared by
//    the four waves: 64 x 16 x 32 bf16 MFMA tiles, then ReLU, head weights and
//    the head sum in registers (16 heads in-lane, 4 lane groups by shuffles).
//    Per tile a wave reads 16 KB of keys from LDS for 128 MFMAs.
//  * index_decode_mfma: one query per block row and 256 keys per block, keys
//    streamed from HBM straight into MFMA B fragments (the decode bottleneck:
//    each key is read once).
//  * index_generic: any head count / width, float or bf16, VALU float32.
//  * topk_radix: per query, four 8-bit radix-select passes find the k-th
//    largest ordered key; one ordered pass emits ids by ballot prefix counts.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

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

// ---------------------------------------------------------------------------
// prefill: 8 queries per block, keys through LDS

constexpr int kIdxQPB = 8;    // queries per block
constexpr int kIdxKT = 64;    // keys per LDS tile
constexpr int kIdxRow = 136;  // LDS row stride in bf16 (128 + 8 pad)

__global__ void __launch_bounds__(256) index_prefill_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ wts, const bf16_t* __restrict__ keys,
    float* __restrict__ scores, const int64_t* __restrict__ pos0, int n_new, int Ri, double base,
    int m, int64_t pool_cap) {
  constexpr int Hi = 64, Di = 128;
  __shared__ __attribute__((aligned(16))) bf16_t ktile[2][kIdxKT * kIdxRow];
  __shared__ double2 cs[kIdxQPB][64];
  __shared__ float wsh[kIdxQPB][Hi];
  const int b = blockIdx.y, i0 = blockIdx.x * kIdxQPB;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int64_t p0 = pos0[b];
  const int nq = min(kIdxQPB, n_new - i0);
  for (int e = tid; e < kIdxQPB * (Ri / 2); e += 256) {
    const int qq = e / (Ri / 2), j = e % (Ri / 2);
    double sn, c;
    sincos((double)(p0 + i0 + qq) * rope_freq(base, j, Ri), &sn, &c);
    cs[qq][j] = make_double2(c, sn);
  }
  for (int e = tid; e < kIdxQPB * Hi; e += 256) {
    const int qq = e / Hi, h = e % Hi;
    wsh[qq][h] = qq < nq ? bf16_to_f32(wts[((int64_t)b * n_new + i0 + qq) * Hi + h]) : 0.f;
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
    const bf16_t* qrow = q + ((int64_t)b * n_new + i0 + (ql < nq ? ql : 0)) * Hi * Di;
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

  float* srow0 = scores + ((int64_t)b * n_new + i0 + 2 * wv) * pool_cap;
  for (int kt = 0, it = 0; kt < nkeys; kt += kIdxKT, ++it) {
    bf16_t* tile = ktile[it & 1];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = tid + 256 * r, key = c >> 4, part = c & 15;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kt + key < nkeys)
        v = *(const uint4*)(keys + ((int64_t)b * pool_cap + kt + key) * Di + part * 8);
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
// decode: rotate queries once, then stream keys from HBM into MFMA fragments

__global__ void __launch_bounds__(256) rotate_queries_bf16(const bf16_t* __restrict__ q,
                                                           bf16_t* __restrict__ qr,
                                                           const int64_t* __restrict__ pos0,
                                                           int n_new, int Hi, int Di, int Ri,
                                                           double base) {
  __shared__ double2 cs[128];
  const int i = blockIdx.x, b = blockIdx.y;
  const int64_t t = pos0[b] + i;
  for (int j = threadIdx.x; j < Ri / 2; j += blockDim.x) {
    double sn, c;
    sincos((double)t * rope_freq(base, j, Ri), &sn, &c);
    cs[j] = make_double2(c, sn);
  }
  __syncthreads();
  const int64_t off = ((int64_t)b * n_new + i) * Hi * Di;
  const int chunks = Hi * Di / 8;
  for (int e = threadIdx.x; e < chunks; e += blockDim.x) {
    const int d0 = (e * 8) % Di;
    uint4 v = *(const uint4*)(q + off + (int64_t)e * 8);
    *(uint4*)(qr + off + (int64_t)e * 8) = rope8_bf16(v, d0, Di, Ri, cs);
  }
}

constexpr int kDecKeys = 256;  // keys per block (64 per wave)

__global__ void __launch_bounds__(256) index_decode_mfma(const bf16_t* __restrict__ qr,
                                                         const bf16_t* __restrict__ wts,
                                                         const bf16_t* __restrict__ keys,
                                                         float* __restrict__ scores,
                                                         const int64_t* __restrict__ pos0,
                                                         int n_new, int m, int64_t pool_cap) {
  constexpr int Hi = 64, Di = 128;
  const int tok = blockIdx.y;  // b * n_new + i
  const int b = tok / n_new, i = tok % n_new;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;
  int64_t nv = (pos0[b] + i + 1) / m;
  if (nv > pool_cap) nv = pool_cap;
  const int64_t k0 = (int64_t)blockIdx.x * kDecKeys + 64 * wv;
  if (k0 >= nv) return;
  const bf16_t* qrow = qr + (int64_t)tok * Hi * Di;
  uint4 A[4][4];
  float wr[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      A[mt][kk] = *(const uint4*)(qrow + (16 * mt + r16) * Di + 32 * kk + 8 * g);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
      wr[mt][ii] = bf16_to_f32(wts[(int64_t)tok * Hi + 16 * mt + 4 * g + ii]);
  }
  uint4 B[4][4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t key = k0 + 16 * nt + r16;
    const bf16_t* krow = keys + ((int64_t)b * pool_cap + (key < nv ? key : 0)) * Di;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) B[nt][kk] = *(const uint4*)(krow + 32 * kk + 8 * g);
  }
  float* srow = scores + (int64_t)tok * pool_cap;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    f32x4 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma16(A[mt][kk], B[nt][kk], acc[mt]);
    float v = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) v += wr[mt][ii] * fmaxf(acc[mt][ii], 0.f);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    const int64_t key = k0 + 16 * nt + r16;
    if (g == 0 && key < nv) srow[key] = v;
  }
}

// ---------------------------------------------------------------------------
// generic: any shape, VALU float32

template <typename T>
__global__ void __launch_bounds__(256) index_generic(const T* __restrict__ q,
                                                     const T* __restrict__ wts,
                                                     const T* __restrict__ keys,
                                                     float* __restrict__ scores,
                                                     const int64_t* __restrict__ pos0, int n_new,
                                                     int Hi, int Di, int Ri, double base, int m,
                                                     int64_t pool_cap) {
  extern __shared__ float qs[];  // [Hi * Di] rotated query, then [Hi] weights
  const int i = blockIdx.x, b = blockIdx.y;
  const int64_t t = pos0[b] + i;
  const int64_t tok = (int64_t)b * n_new + i;
  const T* qrow = q + tok * Hi * Di;
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
  for (int h = threadIdx.x; h < Hi; h += blockDim.x) wsh[h] = store_t<T>::ld(wts + tok * Hi + h);
  __syncthreads();
  int64_t nv = (t + 1) / m;
  if (nv > pool_cap) nv = pool_cap;
  for (int64_t w = threadIdx.x; w < nv; w += blockDim.x) {
    const T* krow = keys + ((int64_t)b * pool_cap + w) * Di;
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

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) u = 0u;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int BS>
__global__ void __launch_bounds__(BS) topk_radix(const float* __restrict__ scores,
                                                 int64_t stride, int32_t* __restrict__ out,
                                                 const int64_t* __restrict__ pos0, int n_new,
                                                 int m, int k, int64_t pool_cap) {
  constexpr int NW = BS / 64;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_prefix, sh_rem;
  __shared__ uint32_t wcnt[2][NW];
  const int i = blockIdx.x, b = blockIdx.y;
  const int64_t tok = (int64_t)b * n_new + i;
  int64_t nv = (pos0[b] + i + 1) / m;
  if (nv > pool_cap) nv = pool_cap;
  const int n = (int)nv;
  const float* sc = scores + tok * stride;
  int32_t* o = out + tok * k;
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
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
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

// ---------------------------------------------------------------------------

static bool index_fast_shape(const Layer& L) {
  return L.dtype == 1 && L.Hi == 64 && L.Di == 128 && L.Ri <= 128;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t index_workspace_bytes(const Layer& L, int B, int n, int64_t pool_cap) {
  size_t s = align256((size_t)B * n * pool_cap * sizeof(float));
  if (index_fast_shape(L) && n < kIdxQPB) s += align256((size_t)B * n * L.Hi * L.Di * 2);
  return s;
}

hipError_t launch_index_topk(const Layer& L, const Batch& bt, const void* q, const void* w,
                             const void* keys, int64_t pool_cap, int32_t* idx, float* scores_out,
                             void* ws, hipStream_t s) {
  char* wsp = (char*)ws;
  float* scores = (float*)wsp;
  wsp += align256((size_t)bt.B * bt.n * pool_cap * sizeof(float));
  if (scores_out) scores = scores_out;
  if (index_fast_shape(L)) {
    if (bt.n >= kIdxQPB) {
      dim3 grid((bt.n + kIdxQPB - 1) / kIdxQPB, bt.B);
      index_prefill_mfma<<<grid, 256, 0, s>>>((const bf16_t*)q, (const bf16_t*)w,
                                              (const bf16_t*)keys, scores, bt.pos0, bt.n, L.Ri,
                                              L.base, L.m, pool_cap);
    } else {
      bf16_t* qr = (bf16_t*)wsp;
      rotate_queries_bf16<<<dim3(bt.n, bt.B), 256, 0, s>>>((const bf16_t*)q, qr, bt.pos0, bt.n,
                                                           L.Hi, L.Di, L.Ri, L.base);
      int64_t nv = (bt.pos0_max + bt.n) / L.m;
      if (nv > pool_cap) nv = pool_cap;
      dim3 grid((unsigned)((nv + kDecKeys - 1) / kDecKeys), bt.B * bt.n);
      if (grid.x > 0)
        index_decode_mfma<<<grid, 256, 0, s>>>(qr, (const bf16_t*)w, (const bf16_t*)keys, scores,
                                               bt.pos0, bt.n, L.m, pool_cap);
    }
  } else {
    const size_t shm = ((size_t)L.Hi * L.Di + L.Hi) * sizeof(float);
    dim3 grid(bt.n, bt.B);
    if (L.dtype == 1)
      index_generic<bf16_t><<<grid, 256, shm, s>>>((const bf16_t*)q, (const bf16_t*)w,
                                                   (const bf16_t*)keys, scores, bt.pos0, bt.n,
                                                   L.Hi, L.Di, L.Ri, L.base, L.m, pool_cap);
    else
      index_generic<float><<<grid, 256, shm, s>>>((const float*)q, (const float*)w,
                                                  (const float*)keys, scores, bt.pos0, bt.n, L.Hi,
                                                  L.Di, L.Ri, L.base, L.m, pool_cap);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid(bt.n, bt.B);
  if ((bt.pos0_max + bt.n) / L.m > 16384)
    topk_radix<1024><<<grid, 1024, 0, s>>>(scores, pool_cap, idx, bt.pos0, bt.n, L.m, L.k,
                                           pool_cap);
  else
    topk_radix<256><<<grid, 256, 0, s>>>(scores, pool_cap, idx, bt.pos0, bt.n, L.m, L.k,
                                         pool_cap);
  return hipGetLastError();
}

}  // namespace csa
