// Partial interleaved-pair RoPE of stored rows, and the window ring append.
//
// The rope slice is the last R channels of a row; pair j = (c, c+1),
// c = D - R + 2j, is a complex number multiplied by exp(i * p * base^(-2j/R))
// [transformers PR 45616, RoPE apply notes; DeepSeek-V4 model page, sec. 2.3].
// Angles, cos/sin and the product are float64; each stored value is rounded
// once to the storage dtype.  Memory-bound: one read and one write per row.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

// One block per (token, sequence); threads stride over the row's channels.
template <typename T>
__global__ void __launch_bounds__(256) window_append_kernel(const T* __restrict__ kv,
                                                            T* __restrict__ ring,
                                                            const int64_t* __restrict__ pos0,
                                                            int n_new, int D, int R, Rope base,
                                                            int64_t cap) {
  const int i = blockIdx.x, b = blockIdx.y;
  const int64_t t = pos0[b] + i;
  const T* src = kv + ((int64_t)b * n_new + i) * D;
  T* dst = ring + ((int64_t)b * cap + (t % cap)) * D;
  for (int c = threadIdx.x; c < D - R; c += blockDim.x) dst[c] = src[c];
  for (int j = threadIdx.x; j < R / 2; j += blockDim.x) {
    const int c = D - R + 2 * j;
    double sn, cs;
    sincos((double)t * rope_freq(base, j, R), &sn, &cs);
    double a = store_t<T>::ld(src + c), bb = store_t<T>::ld(src + c + 1);
    rot64(a, bb, cs, sn);
    store_t<T>::st64(dst + c, a);
    store_t<T>::st64(dst + c + 1, bb);
  }
}

// In place; one block per (token, sequence), threads over (row, pair).
template <typename T>
__global__ void __launch_bounds__(256) rope_kernel(T* __restrict__ x,
                                                   const int64_t* __restrict__ pos0, int n_new,
                                                   int rows, int width, int R, Rope base,
                                                   int sign) {
  const int i = blockIdx.x, b = blockIdx.y;
  const int64_t t = pos0[b] + i;
  const double p = (double)(sign * t);
  T* base_ptr = x + ((int64_t)b * n_new + i) * (int64_t)rows * width;
  const int np = R / 2;
  for (int e = threadIdx.x; e < rows * np; e += blockDim.x) {
    const int r = e / np, j = e % np;
    const int c = width - R + 2 * j;
    double sn, cs;
    sincos(p * rope_freq(base, j, R), &sn, &cs);
    T* row = base_ptr + (int64_t)r * width;
    double a = store_t<T>::ld(row + c), bb = store_t<T>::ld(row + c + 1);
    rot64(a, bb, cs, sn);
    store_t<T>::st64(row + c, a);
    store_t<T>::st64(row + c + 1, bb);
  }
}

hipError_t launch_window_append(const Layer& L, const Batch& bt, const void* kv, void* ring,
                                int64_t cap, hipStream_t s) {
  dim3 grid(bt.n, bt.B);
  if (L.dtype == 1)
    window_append_kernel<bf16_t><<<grid, 256, 0, s>>>((const bf16_t*)kv, (bf16_t*)ring, bt.pos0,
                                                      bt.n, L.D, L.R, L.base, cap);
  else
    window_append_kernel<float><<<grid, 256, 0, s>>>((const float*)kv, (float*)ring, bt.pos0,
                                                     bt.n, L.D, L.R, L.base, cap);
  return hipGetLastError();
}

hipError_t launch_rope(const Layer& L, const Batch& bt, void* x, int rows, int width, int rope_dim,
                       int sign, hipStream_t s) {
  dim3 grid(bt.n, bt.B);
  if (L.dtype == 1)
    rope_kernel<bf16_t><<<grid, 256, 0, s>>>((bf16_t*)x, bt.pos0, bt.n, rows, width, rope_dim,
                                             L.base, sign);
  else
    rope_kernel<float><<<grid, 256, 0, s>>>((float*)x, bt.pos0, bt.n, rows, width, rope_dim,
                                            L.base, sign);
  return hipGetLastError();
}

}  // namespace csa
