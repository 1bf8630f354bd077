// C ABI of libcsa: argument validation, workspace sizing and kernel dispatch.
// Every check runs on the host before any launch; a rejected call touches no
// buffer.  See include/csa.h for the contract of each entry point.
#include <math.h>

#include <mutex>

#include "csa.h"
#include "csa_internal.h"

namespace {

using csa::Batch;
using csa::Layer;

constexpr int kMaxWidth = 2048;   // compressor row width (LDS row buffer)
constexpr int64_t kMaxRowId = 2147483000LL;

csa_status to_layer(const csa_layer* in, Layer* L) {
  if (!in) return CSA_ERR_NULL;
  if (in->dtype != CSA_F32 && in->dtype != CSA_BF16) return CSA_ERR_DTYPE;
  if (in->num_heads < 1 || in->head_dim < 2 || (in->head_dim & 1) || in->qk_rope_head_dim < 0 ||
      (in->qk_rope_head_dim & 1) || in->qk_rope_head_dim > in->head_dim ||
      in->sliding_window < 1 || in->compress_ratio < 0 || in->overlap < 0 || in->overlap > 1 ||
      !(in->rope_theta > 0.0) || !isfinite(in->rope_theta) || in->softmax_scale < 0.f ||
      !isfinite(in->softmax_scale))
    return CSA_ERR_SHAPE;
  if (!(in->rope_factor >= 0.0) || !isfinite(in->rope_factor) ||
      (in->rope_factor > 0.0 && in->rope_factor < 1.0))
    return CSA_ERR_SHAPE;
  if (in->rope_factor > 1.0 &&
      (!(in->rope_original_context > 0.0) || !isfinite(in->rope_original_context) ||
       !(in->rope_beta_slow > 0.0) || !(in->rope_beta_fast > in->rope_beta_slow) ||
       !isfinite(in->rope_beta_fast) || in->rope_theta == 1.0))
    return CSA_ERR_SHAPE;
  L->dtype = in->dtype;
  L->H = in->num_heads;
  L->D = in->head_dim;
  L->R = in->qk_rope_head_dim;
  L->base.base = in->rope_theta;
  L->base.factor = in->rope_factor > 1.0 ? in->rope_factor : 0.0;
  L->base.ln_fast = L->base.ln_slow = L->base.ln_base2 = 0.0;
  if (L->base.factor > 1.0) {
    const double two_pi = 2.0 * 3.141592653589793;
    L->base.ln_fast = log(in->rope_original_context / (two_pi * in->rope_beta_fast));
    L->base.ln_slow = log(in->rope_original_context / (two_pi * in->rope_beta_slow));
    L->base.ln_base2 = 2.0 * log(in->rope_theta);
  }
  L->W = in->sliding_window;
  L->m = in->compress_ratio;
  L->overlap = in->overlap;
  L->Hi = in->index_n_heads;
  L->Di = in->index_head_dim;
  L->Ri = in->index_rope_dim;
  L->k = in->index_topk;
  L->scale = in->softmax_scale > 0.f ? in->softmax_scale : (float)(1.0 / sqrt((double)L->D));
  return CSA_OK;
}

csa_status to_batch(const csa_batch* in, Batch* b, int64_t* pool_rows = nullptr) {
  if (!in) return CSA_ERR_NULL;
  if (!in->pos0) return CSA_ERR_NULL;
  if (in->batch < 1 || in->n_new < 1 || in->pos0_max < 0 ||
      in->pos0_max > (int64_t)1 << 48)
    return CSA_ERR_SHAPE;
  if (in->n_valid && in->cu_seqlens) return CSA_ERR_SHAPE;  // one layout per call
  b->B = in->batch;
  b->n = in->n_new;
  b->pos0 = in->pos0;
  b->pos0_max = in->pos0_max;
  b->nvalid = in->n_valid;
  b->cu = in->cu_seqlens;
  b->table = in->block_table;
  b->bshift = 0;
  b->tstride = 0;
  int64_t rows = 0;
  if (in->block_table) {
    const int32_t e = in->block_entries;
    // a power of two holding whole 128-entry tiles of the key scans
    if (e < 128 || e > (1 << 24) || (e & (e - 1)) != 0 || in->block_table_stride < 1 ||
        in->pool_blocks < 1 || in->pool_blocks > ((int64_t)1 << 40))
      return CSA_ERR_SHAPE;
    while ((1 << b->bshift) < e) ++b->bshift;
    b->tstride = in->block_table_stride;
    rows = in->pool_blocks * (int64_t)e;
  }
  if (pool_rows) *pool_rows = rows;
  return CSA_OK;
}

// A pool argument of pool_cap entries per sequence: the contiguous tensor
// [B, pool_cap, width], or (paged) pool_rows rows addressed through the
// block table, which must cover pool_cap entries.  Row ids of the attention
// kernels are int32.
csa_status pool_ok(const Batch& b, int64_t pool_cap, int64_t pool_rows) {
  if (b.table) {
    if (pool_cap > ((int64_t)b.tstride << b.bshift)) return CSA_ERR_SHAPE;
    if (pool_rows > kMaxRowId) return CSA_ERR_UNSUPPORTED;
  } else if ((int64_t)b.B * pool_cap > kMaxRowId) {
    return CSA_ERR_UNSUPPORTED;
  }
  return CSA_OK;
}

csa_status indexer_ok(const Layer& L) {
  if (L.m < 1 || L.Hi < 1 || L.Di < 2 || (L.Di & 1) || L.Ri < 0 || (L.Ri & 1) || L.Ri > L.Di ||
      L.k < 1 || L.k > csa::kMaxTopK)
    return CSA_ERR_SHAPE;
  return CSA_OK;
}

int64_t entries_needed(const Layer& L, const Batch& b) {
  return L.m > 0 ? (b.pos0_max + b.n) / L.m : 0;
}

csa_status window_ok(const Layer& L, const Batch& b, int64_t cap) {
  if (cap < 1) return CSA_ERR_SHAPE;
  const int64_t need_a = (int64_t)L.W + b.n - 1, need_b = b.pos0_max + b.n;
  if (cap < (need_a < need_b ? need_a : need_b)) return CSA_ERR_SHAPE;
  if ((int64_t)b.B * cap > kMaxRowId) return CSA_ERR_UNSUPPORTED;
  return CSA_OK;
}

csa_status hip_status(hipError_t e) { return e == hipSuccess ? CSA_OK : CSA_ERR_HIP; }

size_t generic_attend_limit_ok(const Layer& L) {
  // float32 LDS copies of q, the accumulator and a 32-row chunk
  const size_t shm = ((size_t)2 * L.H * L.D + (size_t)32 * L.D + (size_t)L.H * 32 + 3 * L.H + 32) *
                     sizeof(float);
  return shm <= 64 * 1024;
}

bool generic_index_ok(const Layer& L) {
  return ((size_t)L.Hi * L.Di + L.Hi) * sizeof(float) <= 64 * 1024;
}

csa_status attend_common(const csa_layer* layer, const csa_batch* batch, const void* q,
                         const void* win, int64_t win_cap, const void* pool, int64_t pool_cap,
                         const int32_t* topk_idx, const float* sinks, void* out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream, bool csa_layer_kind) {
  Layer L;
  Batch b;
  int64_t prow = 0;
  csa_status st = to_layer(layer, &L);
  if (st != CSA_OK) return st;
  if ((st = to_batch(batch, &b, &prow)) != CSA_OK) return st;
  if (!q || !win || !out) return CSA_ERR_NULL;
  if (csa_layer_kind) {
    if (L.m < 1 || L.k < 1 || L.k > csa::kMaxTopK) return CSA_ERR_SHAPE;
    if (!topk_idx || !pool) return CSA_ERR_NULL;
  }
  if (L.m > 0) {
    if (!pool) return CSA_ERR_NULL;
    if (pool_cap < entries_needed(L, b)) return CSA_ERR_SHAPE;
    if ((st = pool_ok(b, pool_cap, prow)) != CSA_OK) return st;
  }
  if ((st = window_ok(L, b, win_cap)) != CSA_OK) return st;
  if (!csa::attend_fast_shape(L) && !generic_attend_limit_ok(L)) return CSA_ERR_UNSUPPORTED;
  if (csa::attend_splits(L, b.B, b.n, L.m > 0 ? pool_cap : 0, csa_layer_kind) < 1)
    return CSA_ERR_UNSUPPORTED;  // more rows per token than the split grid covers
  const size_t need = csa::attend_workspace_bytes(L, b.B, b.n, L.m > 0 ? pool_cap : 0,
                                                  csa_layer_kind);
  if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255)))
    return CSA_ERR_WORKSPACE;
  return hip_status(csa::launch_attend(L, b, q, win, win_cap, pool, L.m > 0 ? pool_cap : 0,
                                       topk_idx, sinks, out, workspace, csa_layer_kind, stream));
}

// Static scratch of csa_index_topk_noalloc: one array per device (each
// device that loads the library holds its own copy until the process ends).
// Host code never passes `scratch` itself to a kernel (in host code the name
// is a host-side stand-in); it uses the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current and kept in scratch_dev.
constexpr size_t kScratchBytes = CSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 256;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices];

csa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return CSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return CSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CSA_ERR_HIP;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return CSA_OK;
}

// Argument checks of csa_index_topk (no launch); *need receives the
// workspace bytes of the call.
csa_status index_topk_check(const csa_layer* layer, const csa_batch* batch, const void* q_idx,
                            const void* weights, const void* k_pool, int64_t pool_cap,
                            const int32_t* topk_idx, Layer* L, Batch* b, size_t* need) {
  int64_t prow = 0;
  csa_status st = to_layer(layer, L);
  if (st != CSA_OK) return st;
  if ((st = to_batch(batch, b, &prow)) != CSA_OK) return st;
  if (!q_idx || !weights || !k_pool || !topk_idx) return CSA_ERR_NULL;
  if ((st = indexer_ok(*L)) != CSA_OK) return st;
  if (pool_cap < entries_needed(*L, *b) || pool_cap < 1) return CSA_ERR_SHAPE;
  if ((st = pool_ok(*b, pool_cap, prow)) != CSA_OK) return st;
  if (!(L->dtype == CSA_BF16 && L->Hi == 64 && L->Di == 128) && !generic_index_ok(*L))
    return CSA_ERR_UNSUPPORTED;
  *need = csa::index_workspace_bytes(*L, b->B, b->n, pool_cap);
  return CSA_OK;
}

}  // namespace

extern "C" {

csa_status csa_window_append(const csa_layer* layer, const csa_batch* batch, const void* kv,
                             void* ring, int64_t cap, hipStream_t stream) {
  Layer L;
  Batch b;
  csa_status st = to_layer(layer, &L);
  if (st != CSA_OK) return st;
  if ((st = to_batch(batch, &b)) != CSA_OK) return st;
  if (!kv || !ring) return CSA_ERR_NULL;
  if ((st = window_ok(L, b, cap)) != CSA_OK) return st;
  return hip_status(csa::launch_window_append(L, b, kv, ring, cap, stream));
}

csa_status csa_rope(const csa_layer* layer, const csa_batch* batch, void* x,
                    int32_t rows_per_token, int32_t width, int32_t rope_dim, int32_t sign,
                    hipStream_t stream) {
  Layer L;
  Batch b;
  csa_status st = to_layer(layer, &L);
  if (st != CSA_OK) return st;
  if ((st = to_batch(batch, &b)) != CSA_OK) return st;
  if (!x) return CSA_ERR_NULL;
  if (rows_per_token < 1 || width < 2 || (width & 1) || rope_dim < 0 || (rope_dim & 1) ||
      rope_dim > width || (sign != 1 && sign != -1))
    return CSA_ERR_SHAPE;
  return hip_status(csa::launch_rope(L, b, x, rows_per_token, width, rope_dim, sign, stream));
}

csa_status csa_compress(const csa_layer* layer, const csa_batch* batch, int32_t width,
                        int32_t rope_dim, const void* kv, const void* gate,
                        const float* norm_weight, float norm_eps, void* state_kv,
                        void* state_gate, void* pool, int64_t pool_cap, hipStream_t stream) {
  Layer L;
  Batch b;
  int64_t prow = 0;
  csa_status st = to_layer(layer, &L);
  if (st != CSA_OK) return st;
  if ((st = to_batch(batch, &b, &prow)) != CSA_OK) return st;
  if (!kv || !gate || !state_kv || !state_gate || !pool) return CSA_ERR_NULL;
  if (L.m < 1) return CSA_ERR_SHAPE;
  if (width < 2 || (width & 1) || width > kMaxWidth || rope_dim < 0 || (rope_dim & 1) ||
      rope_dim > width || !(norm_eps >= 0.f))
    return CSA_ERR_SHAPE;
  if (pool_cap < entries_needed(L, b)) return CSA_ERR_SHAPE;
  if ((st = pool_ok(b, pool_cap, prow)) != CSA_OK) return st;
  return hip_status(csa::launch_compress(L, b, width, rope_dim, kv, gate, norm_weight, norm_eps,
                                         state_kv, state_gate, pool, pool_cap, stream));
}

csa_status csa_cache_update(const csa_layer* layer, const csa_batch* batch, const void* kv,
                            void* ring, int64_t win_cap, const void* ckv, const void* cgate,
                            const float* norm_weight, void* state_kv, void* state_gate,
                            void* pool, const void* ikv, const void* igate,
                            const float* inorm_weight, void* istate_kv, void* istate_gate,
                            void* ipool, int64_t pool_cap, float norm_eps, hipStream_t stream) {
  Layer L;
  Batch b;
  int64_t prow = 0;
  csa_status st = to_layer(layer, &L);
  if (st != CSA_OK) return st;
  if ((st = to_batch(batch, &b, &prow)) != CSA_OK) return st;
  if (!kv || !ring) return CSA_ERR_NULL;
  if ((st = window_ok(L, b, win_cap)) != CSA_OK) return st;
  const bool main = L.m > 0, index = main && L.k > 0;
  if (main) {
    if (!ckv || !cgate || !state_kv || !state_gate || !pool) return CSA_ERR_NULL;
    if (index && (!ikv || !igate || !istate_kv || !istate_gate || !ipool)) return CSA_ERR_NULL;
    if (L.D > kMaxWidth || !(norm_eps >= 0.f)) return CSA_ERR_SHAPE;
    if (index && (L.Di < 2 || (L.Di & 1) || L.Di > kMaxWidth || L.Ri < 0 || (L.Ri & 1) ||
                  L.Ri > L.Di))
      return CSA_ERR_SHAPE;
    if (pool_cap < entries_needed(L, b)) return CSA_ERR_SHAPE;
    if ((st = pool_ok(b, pool_cap, prow)) != CSA_OK) return st;
  }
  if (b.n == 1)
    return hip_status(csa::launch_cache_update_one(
        L, b, kv, ring, win_cap, ckv, cgate, norm_weight, state_kv, state_gate, pool, ikv, igate,
        inorm_weight, istate_kv, istate_gate, ipool, pool_cap, norm_eps,
        index ? 3 : (main ? 2 : 1), stream));
  if (!main) return hip_status(csa::launch_window_append(L, b, kv, ring, win_cap, stream));
  // the window append and both compressors' entries in one launch (and the
  // compressors' state updates in another)
  const csa::CmpArgs ix{L.Di, L.Ri, ikv, igate, inorm_weight, istate_kv, istate_gate, ipool};
  const csa::WinArgs wa{kv, ring, win_cap};
  return hip_status(csa::launch_compress(L, b, L.D, L.R, ckv, cgate, norm_weight, norm_eps,
                                         state_kv, state_gate, pool, pool_cap, stream,
                                         index ? &ix : nullptr, &wa));
}

csa_status csa_index_topk(const csa_layer* layer, const csa_batch* batch, const void* q_idx,
                          const void* weights, const void* k_pool, int64_t pool_cap,
                          int32_t* topk_idx, float* scores_out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  Layer L;
  Batch b;
  size_t need = 0;
  const csa_status st = index_topk_check(layer, batch, q_idx, weights, k_pool, pool_cap, topk_idx,
                                         &L, &b, &need);
  if (st != CSA_OK) return st;
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255))
    return CSA_ERR_WORKSPACE;
  return hip_status(csa::launch_index_topk(L, b, q_idx, weights, k_pool, pool_cap, topk_idx,
                                           scores_out, workspace, stream));
}

csa_status csa_index_topk_noalloc(const csa_layer* layer, const csa_batch* batch,
                                  const void* q_idx, const void* weights, const void* k_pool,
                                  int64_t pool_cap, int32_t* topk_idx, float* scores_out,
                                  hipStream_t stream) {
  Layer L;
  Batch b;
  size_t need = 0;
  csa_status st = index_topk_check(layer, batch, q_idx, weights, k_pool, pool_cap, topk_idx, &L,
                                   &b, &need);
  if (st != CSA_OK) return st;
  if (need > kScratchBytes) return CSA_ERR_SCRATCH;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != CSA_OK) return st;
  return hip_status(csa::launch_index_topk(L, b, q_idx, weights, k_pool, pool_cap, topk_idx,
                                           scores_out, ws, stream));
}

csa_status csa_attend(const csa_layer* layer, const csa_batch* batch, const void* q,
                      const void* win, int64_t win_cap, const void* pool, int64_t pool_cap,
                      const int32_t* topk_idx, const float* sinks, void* out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  return attend_common(layer, batch, q, win, win_cap, pool, pool_cap, topk_idx, sinks, out,
                       workspace, workspace_bytes, stream, true);
}

csa_status hca_attend(const csa_layer* layer, const csa_batch* batch, const void* q,
                      const void* win, int64_t win_cap, const void* pool, int64_t pool_cap,
                      const float* sinks, void* out, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  return attend_common(layer, batch, q, win, win_cap, pool, pool_cap, nullptr, sinks, out,
                       workspace, workspace_bytes, stream, false);
}

size_t csa_workspace_bytes(const csa_layer* layer, int32_t batch, int32_t n_new,
                           int64_t pool_cap, int32_t op) {
  Layer L;
  if (to_layer(layer, &L) != CSA_OK || batch < 1 || n_new < 1 || pool_cap < 0) return (size_t)-1;
  switch (op) {
    case CSA_OP_INDEX_TOPK:
      if (indexer_ok(L) != CSA_OK) return (size_t)-1;
      return csa::index_workspace_bytes(L, batch, n_new, pool_cap);
    case CSA_OP_ATTEND:
      if (L.m < 1 || L.k < 1 || L.k > csa::kMaxTopK) return (size_t)-1;
      return csa::attend_workspace_bytes(L, batch, n_new, pool_cap, true);
    case CSA_OP_HCA_ATTEND:
      return csa::attend_workspace_bytes(L, batch, n_new, L.m > 0 ? pool_cap : 0, false);
    default:
      return (size_t)-1;
  }
}

static csa_status oproj_ok(const csa_oproj* p) {
  if (!p) return CSA_ERR_NULL;
  if (p->tokens < 1 || p->num_heads < 1 || p->head_dim < 1 || p->o_groups < 1 ||
      p->o_lora_rank < 1 || p->hidden_size < 1 || p->num_heads % p->o_groups != 0)
    return CSA_ERR_SHAPE;
  const int64_t ig = (int64_t)(p->num_heads / p->o_groups) * p->head_dim;
  const int64_t gr = (int64_t)p->o_groups * p->o_lora_rank;
  // row strides stay below 2^22 elements: a block's 256 rows are addressed
  // with 32-bit byte offsets
  if (ig % 32 != 0 || gr % 32 != 0 || gr > (1 << 22) ||
      (int64_t)p->num_heads * p->head_dim > (1 << 22) || p->tokens > (1 << 23))
    return CSA_ERR_UNSUPPORTED;
  return CSA_OK;
}

size_t csa_output_projection_workspace_bytes(const csa_oproj* p) {
  if (oproj_ok(p) != CSA_OK) return (size_t)-1;
  return (size_t)p->tokens * p->o_groups * p->o_lora_rank * sizeof(csa::bf16_t);
}

csa_status csa_output_projection(const csa_oproj* p, const void* attn_out, const void* w_a,
                                 const void* w_b, void* out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  const csa_status st = oproj_ok(p);
  if (st != CSA_OK) return st;
  if (!attn_out || !w_a || !w_b || !out) return CSA_ERR_NULL;
  // the products stage 16-byte chunks of their operands
  if (((uintptr_t)attn_out | (uintptr_t)w_a | (uintptr_t)w_b) & 15u) return CSA_ERR_UNSUPPORTED;
  const size_t need = csa_output_projection_workspace_bytes(p);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) return CSA_ERR_WORKSPACE;
  hipError_t e = csa::launch_output_projection(
      p->tokens, p->num_heads, p->head_dim, p->o_groups, p->o_lora_rank, p->hidden_size,
      (const csa::bf16_t*)attn_out, (const csa::bf16_t*)w_a, (const csa::bf16_t*)w_b,
      (csa::bf16_t*)workspace, (csa::bf16_t*)out, stream);
  return e == hipSuccess ? CSA_OK : CSA_ERR_HIP;
}

static csa_status proj_ok(const csa_proj* p) {
  if (!p) return CSA_ERR_NULL;
  if (p->tokens < 1 || p->hidden < 1 || p->q_lora_rank < 1 || p->num_heads < 1 ||
      p->head_dim < 1 || p->comp_dim < 0 || p->index_dim < 0 || p->index_heads < 0 ||
      (p->index_dim == 0) != (p->index_heads == 0) || !(p->eps >= 0.0f) ||
      (p->q_head_norm != 0 && p->q_head_norm != 1))
    return CSA_ERR_SHAPE;
  const int64_t nx = (int64_t)p->q_lora_rank + p->head_dim + 2 * (int64_t)p->comp_dim +
                     2 * (int64_t)p->index_dim + p->index_heads;
  const int64_t nq = (int64_t)p->num_heads * p->head_dim +
                     (int64_t)p->index_heads * p->index_dim;
  // the products address a block's 256 rows with 32-bit byte offsets
  if (p->hidden % 32 != 0 || p->q_lora_rank % 32 != 0 || p->hidden > (1 << 22) ||
      p->q_lora_rank > (1 << 22) || nx > (1 << 30) || nq > (1 << 30) || p->tokens > (1 << 23))
    return CSA_ERR_UNSUPPORTED;
  return CSA_OK;
}

size_t csa_project_workspace_bytes(const csa_proj* p) {
  if (proj_ok(p) != CSA_OK) return (size_t)-1;
  return (size_t)p->tokens * p->q_lora_rank * sizeof(csa::bf16_t);
}

csa_status csa_project(const csa_proj* p, const void* x, const void* w_x, const float* g_qa,
                       const float* g_kv, const void* w_q, void* q, void* kv, void* ckv,
                       void* cgate, void* ikv, void* igate, void* qi, void* wi, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  const csa_status st = proj_ok(p);
  if (st != CSA_OK) return st;
  if (!x || !w_x || !g_qa || !g_kv || !w_q || !q || !kv) return CSA_ERR_NULL;
  if (p->comp_dim > 0 && (!ckv || !cgate)) return CSA_ERR_NULL;
  if (p->index_dim > 0 && (!ikv || !igate || !qi || !wi)) return CSA_ERR_NULL;
  if (((uintptr_t)x | (uintptr_t)w_x | (uintptr_t)w_q) & 15u) return CSA_ERR_UNSUPPORTED;
  const size_t need = csa_project_workspace_bytes(p);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) return CSA_ERR_WORKSPACE;
  using csa::bf16_t;
  hipError_t e = csa::launch_project(
      p->tokens, p->hidden, p->q_lora_rank, p->num_heads, p->head_dim, p->comp_dim, p->index_dim,
      p->index_heads, p->eps, p->q_head_norm, (const bf16_t*)x, (const bf16_t*)w_x, g_qa, g_kv,
      (const bf16_t*)w_q, (bf16_t*)q, (bf16_t*)kv, (bf16_t*)ckv, (bf16_t*)cgate, (bf16_t*)ikv,
      (bf16_t*)igate, (bf16_t*)qi, (bf16_t*)wi, (bf16_t*)workspace, stream);
  return e == hipSuccess ? CSA_OK : CSA_ERR_HIP;
}

const char* csa_status_str(csa_status s) {
  switch (s) {
    case CSA_OK: return "CSA_OK";
    case CSA_ERR_NULL: return "CSA_ERR_NULL: a required pointer is NULL";
    case CSA_ERR_SHAPE: return "CSA_ERR_SHAPE: sizes inconsistent or out of range";
    case CSA_ERR_DTYPE: return "CSA_ERR_DTYPE: unknown storage dtype";
    case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED: configuration not implemented";
    case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE: workspace missing, short or misaligned";
    case CSA_ERR_HIP: return "CSA_ERR_HIP: HIP launch failed";
    case CSA_ERR_SCRATCH:
      return "CSA_ERR_SCRATCH: the call needs more than the library's static scratch buffer";
  }
  return "unknown csa_status";
}

int32_t csa_version(void) { return 400; }  // 0.4.0: paged pools, packed variable-length rows

}  // extern "C"
