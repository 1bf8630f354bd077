// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

typedef uint16_t bf16_t;  // bfloat16 carried as its raw bits

constexpr int kMaxTopK = 4096;  // largest index_topk the library accepts

// Rope frequencies of a layer: pair j of R rope channels turns at
// base^(-2j/R) per position, remapped by YaRN when factor > 1 (rope_freq in
// csa_device.h).
struct Rope {
  double base;
  double factor;  // YaRN scale s; <= 1: none
  // YaRN ramp terms (host-computed): ln(orig / (2 pi beta_fast)),
  // ln(orig / (2 pi beta_slow)) and 2 ln(base), orig being the original
  // context; the correction index of n turns is R ln(orig / (2 pi n)) / (2 ln base)
  double ln_fast, ln_slow, ln_base2;
};

struct Layer {
  int dtype;       // 0 float32, 1 bf16
  int H, D, R;     // heads, head_dim, rope channels
  Rope base;       // rope frequencies (both the main and the indexer rope)
  int W;           // sliding window
  int m, overlap;  // compress ratio (0 = none), overlap flag
  int Hi, Di, Ri;  // indexer heads, dim, rope channels
  int k;           // top-k
  float scale;     // logit scale (resolved, never 0)
};

struct Batch {
  int B, n;             // sequences, new tokens per sequence
  const int64_t* pos0;  // device [B]
  int64_t pos0_max;     // host bound
  const int32_t* nvalid;  // device [B] valid tokens per sequence, or null (all n)
};

// Valid tokens of sequence b in a call of n per sequence.
__device__ __forceinline__ int valid_tokens(const int32_t* nvalid, int b, int n) {
  if (!nvalid) return n;
  const int v = nvalid[b];
  return v < 0 ? 0 : (v > n ? n : v);
}

// oproj.hip
// Column routing of a GEMM's output: columns col0[s] .. col0[s + 1] - 1
// (the last segment runs to N) go to ptr[s] with row stride ld[s].
constexpr int kGemmOutMax = 8;
struct GemmOut {
  bf16_t* ptr[kGemmOutMax];
  int64_t ld[kGemmOutMax];
  int col0[kGemmOutMax];
  int nseg;
};

hipError_t launch_gemm_nt_routed(const bf16_t* A, const bf16_t* B, int M, int N, int K,
                                 int64_t lda, int64_t ldb, const GemmOut& map, hipStream_t s);
hipError_t launch_project(int T, int hidden, int q_lora, int H, int D, int comp, int Di, int Hi,
                          float eps, int q_head_norm, const bf16_t* x, const bf16_t* w_x,
                          const float* g_qa, const float* g_kv, const bf16_t* w_q, bf16_t* q,
                          bf16_t* kv, bf16_t* ckv, bf16_t* cgate, bf16_t* ikv, bf16_t* igate,
                          bf16_t* qi, bf16_t* wi, bf16_t* latent, hipStream_t s);

hipError_t launch_output_projection(int T, int H, int D, int G, int R, int hidden,
                                    const bf16_t* x, const bf16_t* wa, const bf16_t* wb,
                                    bf16_t* y1, bf16_t* out, hipStream_t s);

// rope.hip
hipError_t launch_window_append(const Layer& L, const Batch& b, const void* kv, void* ring,
                                int64_t cap, hipStream_t s);
hipError_t launch_rope(const Layer& L, const Batch& b, void* x, int rows, int width, int rope_dim,
                       int sign, hipStream_t s);
// compress.hip
hipError_t launch_compress(const Layer& L, const Batch& b, int width, int rope_dim, const void* kv,
                           const void* gate, const float* norm_w, float eps, void* st_kv,
                           void* st_gate, void* pool, int64_t pool_cap, hipStream_t s);
// index.hip
size_t index_workspace_bytes(const Layer& L, int B, int n, int64_t pool_cap);
hipError_t launch_index_topk(const Layer& L, const Batch& b, const void* q, const void* w,
                             const void* keys, int64_t pool_cap, int32_t* idx, float* scores_out,
                             void* ws, hipStream_t s);
// attend.hip
bool attend_fast_shape(const Layer& L);
int attend_splits(const Layer& L, int B, int n, int64_t pool_cap, bool csa);
size_t attend_workspace_bytes(const Layer& L, int B, int n, int64_t pool_cap, bool csa);
// attend_wide.hip
hipError_t launch_attend_x32(const Layer& L, const Batch& b, const void* q, const void* win,
                             int64_t win_cap, const void* pool, int64_t pool_cap,
                             const int32_t* idx, const float* sinks, void* out, void* ws, bool csa,
                             int nsplit, hipStream_t s);
hipError_t launch_attend_w8(const Layer& L, const Batch& b, const void* q, const void* win,
                             int64_t win_cap, const void* pool, int64_t pool_cap,
                             const int32_t* idx, const float* sinks, void* out, void* ws, bool csa,
                             int nsplit, hipStream_t s);
hipError_t launch_attend_h32(const Layer& L, const Batch& b, const void* q, const void* win,
                             int64_t win_cap, const void* pool, int64_t pool_cap,
                             const int32_t* idx, const float* sinks, void* out, void* ws, bool csa,
                             int nsplit, hipStream_t s);
// attend_decode.hip
int attend_decode_splits(const Layer& L, int B, int n, int64_t pool_cap, bool csa);
hipError_t launch_attend_decode(const Layer& L, const Batch& b, const void* q, const void* win,
                                int64_t win_cap, const void* pool, int64_t pool_cap,
                                const int32_t* idx, const float* sinks, void* out, void* ws,
                                bool csa, int nsplit, hipStream_t s);
hipError_t launch_attend(const Layer& L, const Batch& b, const void* q, const void* win,
                         int64_t win_cap, const void* pool, int64_t pool_cap, const int32_t* idx,
                         const float* sinks, void* out, void* ws, bool csa, hipStream_t s);

}  // namespace csa
