// Partial interleaved-pair RoPE of stored rows (the window ring append, which
// rotates the same way, sits with the compressors, whose prefill launch also
// takes it).
//
// The rope slice is the last R channels of a row; pair j = (c, c+1),
// c = D - R + 2j, is a complex number multiplied by exp(i * p * base^(-2j/R))
// [transformers PR 45616, RoPE apply notes; DeepSeek-V4 model page, sec. 2.3].
// Angles, cos/sin and the product are float64; each stored value is rounded
// once to the storage dtype.  Memory-bound: one read and one write per row.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

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
