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

// A block takes kWaTok consecutive tokens of one sequence: the channels
// before the rope slice are copied with 16-byte moves where rows allow it,
// then each (token, pair) of the slice is rotated by one thread, with the
// pair frequencies computed once per block.
constexpr int kWaTok = 8;

template <typename T>
__global__ void __launch_bounds__(256) window_append_kernel(const T* __restrict__ kv,
                                                            T* __restrict__ ring,
                                                            Seqs sq, int D, int R, Rope base,
                                                            int64_t cap) {
  extern __shared__ double freq[];  // R / 2 pair frequencies
  const int i0 = blockIdx.x * kWaTok, b = blockIdx.y;
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

// In place; one block per (token, sequence), threads over (row, pair).
template <typename T>
__global__ void __launch_bounds__(256) rope_kernel(T* __restrict__ x, Seqs sq, int rows,
                                                   int width, int R, Rope base, int sign) {
  const int i = blockIdx.x, b = blockIdx.y;
  if (i >= sq.len(b)) return;  // padding rows are left as they are
  const int64_t t = sq.pos0[b] + i;
  const double p = (double)(sign * t);
  T* base_ptr = x + sq.row(b, i) * (int64_t)rows * width;
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

hipError_t launch_rope(const Layer& L, const Batch& bt, void* x, int rows, int width, int rope_dim,
                       int sign, hipStream_t s) {
  dim3 grid(bt.n, bt.B);
  if (L.dtype == 1)
    rope_kernel<bf16_t><<<grid, 256, 0, s>>>((bf16_t*)x, seqs_of(bt), rows, width, rope_dim,
                                             L.base, sign);
  else
    rope_kernel<float><<<grid, 256, 0, s>>>((float*)x, seqs_of(bt), rows, width, rope_dim,
                                            L.base, sign);
  return hipGetLastError();
}

}  // namespace csa
