// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

typedef uint16_t bf16_t;  // bfloat16 carried as its raw bits

constexpr int kMaxTopK = 4096;  // largest index_topk the library accepts

// Tile sizes shared by the kernels and the host planning (plan.hip).
constexpr int kAH = 64, kAD = 512;  // heads and head_dim of the attention fast path
constexpr int kCH = 32;             // rows per chunk of attend_mfma
constexpr int kMaxRows = 1024;      // rows of one attend_mfma block
constexpr int kPart = kAD + 4;      // split partial row: O[512], m, l, 2 pad (16-byte rows)
constexpr int kMaxSplits = 256;     // row splits the merge takes
constexpr int kDCh = 64;            // rows per chunk of attend_decode
constexpr int kDMaxRows = 2048;     // rows of one attend_decode block (ids kept in LDS)
constexpr int kIdxQPB = 8;          // queries per block of index_prefill_mfma; fewer new
                                    // tokens per sequence take the decode indexer
constexpr int kHBits = 12, kHBins = 1 << kHBits;  // decode score histogram
constexpr int kSlice = 1024;        // keys per topk_collect wave
constexpr int kMaxSlices = 2048;    // topk_final keeps slice offsets in LDS

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
  int B, n;             // sequences, rows per sequence (packed: a bound on any length)
  const int64_t* pos0;  // device [B]
  int64_t pos0_max;     // host bound
  const int32_t* nvalid;  // device [B] valid tokens per sequence, or null (all n)
  const int32_t* cu;      // device [B + 1] packed row offsets, or null (padded rows)
  const int32_t* table;   // device [B, tstride] pool block table, or null (contiguous pools)
  int bshift;             // log2 of the entries per pool block (paged pools)
  int tstride;            // row stride of the block table
};

// The token rows and pooled entries of one call, as the kernels see them.
//  * Token i of sequence b (i < len(b)) sits at position pos0[b] + i and in
//    row row(b, i) of every per-token tensor: b n + i for padded calls,
//    cu[b] + i for packed ones.  len(b) is n, n_valid[b] (padded calls) or
//    cu[b + 1] - cu[b] (packed calls), clamped to 0 .. n.
//  * Entry w of sequence b sits in row prow(b, w, cap) of a pool tensor:
//    b cap + w for contiguous pools, or through the block table,
//    table[b][w / E] E + w mod E for paged ones (E = 2^bshift entries per
//    block).
struct Seqs {
  const int64_t* pos0;
  const int32_t* nvalid;
  const int32_t* cu;
  const int32_t* table;
  int n, bshift, tstride;
  __device__ __forceinline__ int len(int b) const {
    int v = n;
    if (cu) v = cu[b + 1] - cu[b];
    else if (nvalid) v = nvalid[b];
    return v < 0 ? 0 : (v > n ? n : v);
  }
  __device__ __forceinline__ int64_t row(int b, int i) const {
    return cu ? (int64_t)cu[b] + i : (int64_t)b * n + i;
  }
  // The block table is read through the constant address space: a lookup
  // whose index is the same for the whole wave (a tile's first entry) then
  // becomes a scalar load, waited for on the scalar counter instead of
  // draining the LDS-DMA in flight (per-lane lookups stay vector loads).
  // The table is not written while a kernel runs.
  __device__ __forceinline__ int64_t prow(int b, int64_t w, int64_t cap) const {
    if (!table) return (int64_t)b * cap + w;
    typedef const __attribute__((address_space(4))) int32_t ctab;
    const int64_t blk = ((ctab*)table)[(int64_t)b * tstride + (w >> bshift)];
    return (blk << bshift) + (w & (((int64_t)1 << bshift) - 1));
  }
};

inline Seqs seqs_of(const Batch& b) {
  return Seqs{b.pos0, b.nvalid, b.cu, b.table, b.n, b.bshift, b.tstride};
}

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
  // 1 + the output whose rows are RMS-normalised per 512 columns (no
  // weight) in the GEMM's epilogue, 0 for none; its eps
  int norm_seg1;
  double norm_eps;
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
// A second stream of the same layer (the indexer's), pooled in the same
// launches as the first.
struct CmpArgs {
  int width, rope_dim;
  const void* kv;
  const void* gate;
  const float* norm_w;
  void* st_kv;
  void* st_gate;
  void* pool;
};
// The window append of the same call (kv rows into the ring), in the same
// launch as the compressors' entries.
struct WinArgs {
  const void* kv;
  void* ring;
  int64_t cap;
};
hipError_t launch_compress(const Layer& L, const Batch& b, int width, int rope_dim, const void* kv,
                           const void* gate, const float* norm_w, float eps, void* st_kv,
                           void* st_gate, void* pool, int64_t pool_cap, hipStream_t s,
                           const CmpArgs* second = nullptr, const WinArgs* win = nullptr);
// One launch for a decode step's cache updates: roles 1 (window), 2 (+ main
// compressor) or 3 (+ indexer compressor) per sequence.
hipError_t launch_cache_update_one(const Layer& L, const Batch& b, const void* kv, void* ring,
                                   int64_t cap, const void* ckv, const void* cgate,
                                   const float* norm_w, void* st_kv, void* st_gate, void* pool,
                                   const void* ikv, const void* igate, const float* inorm_w,
                                   void* ist_kv, void* ist_gate, void* ipool, int64_t pool_cap,
                                   float eps, int roles, hipStream_t s);
// plan.hip
size_t align256(size_t x);
bool index_fast_shape(const Layer& L);
bool index_decode_path(const Layer& L, int n, int64_t pool_cap);
size_t index_workspace_bytes(const Layer& L, int B, int n, int64_t pool_cap);
bool attend_dec(const Layer& L, int B, int n, int64_t pool_cap, bool csa);
// index.hip
hipError_t launch_index_topk(const Layer& L, const Batch& b, const void* q, const void* w,
                             const void* keys, int64_t pool_cap, int32_t* idx, float* scores_out,
                             void* ws, hipStream_t s);
bool attend_fast_shape(const Layer& L);
int attend_splits(const Layer& L, int B, int n, int64_t pool_cap, bool csa);
size_t attend_workspace_bytes(const Layer& L, int B, int n, int64_t pool_cap, bool csa);
int attend_decode_splits(const Layer& L, int B, int n, int64_t pool_cap, bool csa);
// attend_decode.hip
hipError_t launch_attend_decode(const Layer& L, const Batch& b, const void* q, const void* win,
                                int64_t win_cap, const void* pool, int64_t pool_cap,
                                const int32_t* idx, const float* sinks, void* out, void* ws,
                                bool csa, int nsplit, hipStream_t s);
hipError_t launch_attend(const Layer& L, const Batch& b, const void* q, const void* win,
                         int64_t win_cap, const void* pool, int64_t pool_cap, const int32_t* idx,
                         const float* sinks, void* out, void* ws, bool csa, hipStream_t s);

}  // namespace csa
