// Producer side of the attention block: the projections that make the
// layer's inputs from the block's normalised hidden states x [T, hidden]
// [TransformerLens deepseek_v4 adapter: the self_attn module list (q_a_proj,
// q_a_norm, q_b_proj, q_b_norm, kv_proj, kv_norm, compressor) and the
// compressor / indexer submodules (kv_proj, gate_proj, q_b_proj,
// scorer.weights_proj); DeepSeek-V4 model page, sec. 2.3: kv_proj makes the
// one K=V head].
//
// Two products on gemm_nt_bf16 with routed epilogues, so that every stream
// lands in its own tensor as the product is stored:
//  1. x times the stacked weight of everything read from x: the query
//     latent (q_a_proj) to the workspace, kv_proj to kv, the compressor's
//     kv_proj / gate_proj to ckv / cgate, the indexer's kv_proj / gate_proj to
//     ikv / igate, weights_proj to wi;
//  2. after q_a_norm (in place on the latent), the latent times the stacked
//     q_b_proj and indexer q_b_proj weights, to q and qi.
// kv_norm runs in place on kv, and q_b_norm (a weightless RMS normalisation
// of each head) in place on q.  Every norm reads the stored bf16 projection
// and works in float64, rounded once to bf16.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

// One wave per row of n values (row stride ld), in place:
// x <- x / sqrt(mean(x^2) + eps) * w (w = 1 when null), in float64 over the
// stored values (the division as a product with the float64 reciprocal).
// Rows of n = 8 c (c <= 4 chunks of 8 per lane, n <= 2048) are read once,
// 16 bytes per lane, and kept in registers; other widths take a two-pass loop.
template <int C>
__global__ void __launch_bounds__(256) rmsnorm_rows_bf16(bf16_t* __restrict__ x, int64_t nrows,
                                                         int n, int64_t ld,
                                                         const float* __restrict__ w,
                                                         double eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= nrows) return;
  bf16_t* p = x + row * ld;
  double ss = 0.0;
  if constexpr (C > 0) {
    // the row's chunks and their weights are all loaded before any is used
    // (a weight load inside the scaling loop was waited for at each use)
    uint4 v[C];
    float4 wa[C], wb[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int i = 8 * (lane + 64 * c);
      v[c] = i < n ? *(const uint4*)(p + i) : make_uint4(0, 0, 0, 0);
      if (w) {
        const int iw = i < n ? i : 0;
        wa[c] = *(const float4*)(w + iw);
        wb[c] = *(const float4*)(w + iw + 4);
      }
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const uint32_t u[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double a = (double)__uint_as_float(u[e] << 16);
        const double b = (double)__uint_as_float(u[e] & 0xffff0000u);
        ss += a * a + b * b;
      }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) ss += __shfl_xor(ss, d, 64);
    const double r = 1.0 / sqrt(ss / (double)n + eps);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int i = 8 * (lane + 64 * c);
      if (i >= n) break;
      const uint32_t u[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        double a = (double)__uint_as_float(u[e] << 16) * r;
        double b = (double)__uint_as_float(u[e] & 0xffff0000u) * r;
        if (w) {
          const float4 wq = e < 2 ? wa[c] : wb[c];
          a *= (double)((e & 1) ? wq.z : wq.x);
          b *= (double)((e & 1) ? wq.w : wq.y);
        }
        o[e] = (uint32_t)f64_to_bf16(a) | ((uint32_t)f64_to_bf16(b) << 16);
      }
      *(uint4*)(p + i) = make_uint4(o[0], o[1], o[2], o[3]);
    }
    return;
  }
  for (int i = lane; i < n; i += 64) {
    const double v = (double)bf16_to_f32(p[i]);
    ss += v * v;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) ss += __shfl_xor(ss, d, 64);
  const double r = 1.0 / sqrt(ss / (double)n + eps);
  for (int i = lane; i < n; i += 64) {
    const double v = (double)bf16_to_f32(p[i]) * r;
    p[i] = f64_to_bf16(w ? v * (double)w[i] : v);
  }
}

static hipError_t launch_rmsnorm(bf16_t* x, int64_t nrows, int n, int64_t ld, const float* w,
                                 double eps, hipStream_t s) {
  if (nrows <= 0 || n <= 0) return hipSuccess;
  const unsigned g = (unsigned)((nrows + 3) / 4);
  // the register path needs whole 16-byte chunks on 16-byte aligned rows
  const bool vec = n % 8 == 0 && ld % 8 == 0 && ((uintptr_t)x & 15u) == 0 &&
                   ((uintptr_t)w & 15u) == 0;  // (null passes)
  const int c = vec ? (n + 511) / 512 : 0;
  if (c == 1)
    rmsnorm_rows_bf16<1><<<g, 256, 0, s>>>(x, nrows, n, ld, w, eps);
  else if (c == 2)
    rmsnorm_rows_bf16<2><<<g, 256, 0, s>>>(x, nrows, n, ld, w, eps);
  else if (c == 3 || c == 4)
    rmsnorm_rows_bf16<4><<<g, 256, 0, s>>>(x, nrows, n, ld, w, eps);
  else
    rmsnorm_rows_bf16<0><<<g, 256, 0, s>>>(x, nrows, n, ld, w, eps);
  return hipGetLastError();
}

hipError_t launch_project(int T, int hidden, int q_lora, int H, int D, int comp, int Di, int Hi,
                          float eps, int q_head_norm, const bf16_t* x, const bf16_t* w_x,
                          const float* g_qa, const float* g_kv, const bf16_t* w_q, bf16_t* q,
                          bf16_t* kv, bf16_t* ckv, bf16_t* cgate, bf16_t* ikv, bf16_t* igate,
                          bf16_t* qi, bf16_t* wi, bf16_t* latent, hipStream_t s) {
  GemmOut m1{};
  int col = 0;
  auto add = [](GemmOut& m, int& c, bf16_t* p, int width) {
    if (width <= 0) return;
    m.ptr[m.nseg] = p;
    m.ld[m.nseg] = width;
    m.col0[m.nseg] = c;
    ++m.nseg;
    c += width;
  };
  add(m1, col, latent, q_lora);
  add(m1, col, kv, D);
  add(m1, col, ckv, comp);
  add(m1, col, cgate, comp);
  add(m1, col, ikv, Di);
  add(m1, col, igate, Di);
  add(m1, col, wi, Hi);
  hipError_t e = launch_gemm_nt_routed(x, w_x, T, col, hidden, hidden, hidden, m1, s);
  if (e != hipSuccess) return e;
  if ((e = launch_rmsnorm(latent, T, q_lora, q_lora, g_qa, (double)eps, s)) != hipSuccess) return e;
  if ((e = launch_rmsnorm(kv, T, D, D, g_kv, (double)eps, s)) != hipSuccess) return e;
  GemmOut m2{};
  col = 0;
  add(m2, col, q, H * D);
  add(m2, col, qi, Hi * Di);
  // heads of 512 channels: q_b_norm in the product's epilogue (128 x 512
  // tiles, one head per tile column, stored 16 bytes at a time), otherwise a
  // pass of its own
  const bool fused = q_head_norm && D == 512 && ((uintptr_t)q & 15u) == 0;
  if (fused) {
    m2.norm_seg1 = 1;
    m2.norm_eps = (double)eps;
  }
  e = launch_gemm_nt_routed(latent, w_q, T, col, q_lora, q_lora, q_lora, m2, s);
  if (e != hipSuccess) return e;
  if (q_head_norm && !fused) e = launch_rmsnorm(q, (int64_t)T * H, D, D, nullptr, (double)eps, s);
  return e;
}

}  // namespace csa
