/*
 * csa.h -- C ABI of the compressed attention core of a DeepSeek-V4 layer
 * (CSA: compressed sparse attention; HCA: heavily compressed attention;
 * sliding-only layers), for AMD Instinct MI355X (gfx950).
 *
 * The layer follows the Transformers documentation page for DeepSeek-V4,
 * section "Hybrid attention (sec. 2.3)": every attention block has one
 * shared K=V head (multi-query attention, the same tensor is key and value),
 * partial interleaved-pair RoPE on the last qk_rope_head_dim channels, the
 * same rotation at -t applied to the output's rope slice, a learnable sink
 * logit per head, and a sliding window branch whose rows are concatenated
 * with the compressor's rows before one softmax.  CSA layers pool the K=V
 * stream at ratio m (overlapping windows) and a Lightning Indexer picks the
 * top-k pooled entries per query; HCA layers pool at ratio m' (no overlap)
 * and attend to every closed entry.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is DEVICE memory owned by the caller.  The library
 *    allocates nothing and keeps no mutable global state (the one exception
 *    is csa_index_topk_noalloc's static scratch array); calls on different
 *    streams may run concurrently when their buffers do not overlap.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  Argument errors are returned before any launch and leave all
 *    buffers untouched.  A failed launch returns CSA_ERR_HIP; a device fault
 *    surfaces at the caller's next synchronisation.
 *  - Tensors are dense, row-major, with the shapes written next to each
 *    argument.  "dtype" means the layer's storage dtype (csa_layer.dtype):
 *    IEEE float32 or bfloat16.  Sinks, norm weights and scores are float32;
 *    positions are int64; top-k indices are int32.
 *  - A call covers `batch` sequences with `n_new` new tokens each.  Token i of
 *    sequence b sits at absolute position t = pos0[b] + i.  n_new == 1 is a
 *    decode step; the library picks its kernels from the sizes, both sides
 *    compute the same function.
 *  - Pooled entry w of a layer with ratio m closes at token (w+1)m-1 and is
 *    visible to query t iff w < (t+1)/m (integer division).  Window rows of
 *    query t are the positions t-W+1 .. t that are >= 0.
 *  - Every rounding to a bf16 or float32 store is round-to-nearest-even.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA_OK = 0,
  CSA_ERR_NULL = 1,        /* a required pointer is NULL                       */
  CSA_ERR_SHAPE = 2,       /* sizes inconsistent or out of range               */
  CSA_ERR_DTYPE = 3,       /* unknown storage dtype                            */
  CSA_ERR_UNSUPPORTED = 4, /* valid request this library does not implement    */
  CSA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required          */
  CSA_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed       */
  CSA_ERR_SCRATCH = 7      /* the call needs more than the static scratch of
                              csa_index_topk_noalloc                           */
} csa_status;

typedef enum { CSA_F32 = 0, CSA_BF16 = 1 } csa_dtype;

/* One attention layer.  Field names follow the model configuration fields the
 * DeepSeek-V4 pages name (head_dim, qk_rope_head_dim via partial_rotary_factor,
 * sliding_window, compress ratios, index_topk, index_head_dim). */
typedef struct {
  int32_t dtype;            /* csa_dtype of every stored tensor                */
  int32_t num_heads;        /* H query heads; one shared K=V head              */
  int32_t head_dim;         /* D, even                                         */
  int32_t qk_rope_head_dim; /* R: last R channels rotate in pairs; even, <= D  */
  double rope_theta;        /* RoPE base of this layer (compressed layers use
                               the slower compressed base)                     */
  int32_t sliding_window;   /* W >= 1                                          */
  int32_t compress_ratio;   /* m: 4 for CSA, 128 for HCA, 0 = sliding-only     */
  int32_t overlap;          /* 1: windows of 2m tokens at stride m (CSA);
                               0: windows of m tokens (HCA)                    */
  int32_t index_n_heads;    /* H_I (CSA only)                                  */
  int32_t index_head_dim;   /* D_I (CSA only), even                            */
  int32_t index_rope_dim;   /* R_I: rope channels of the indexer (<= D_I)      */
  int32_t index_topk;       /* k entries selected per query, 1..4096           */
  float softmax_scale;      /* logit scale; 0 selects 1/sqrt(head_dim).  The
                               sink logit is not scaled.                       */
  /* YaRN rope scaling (every rope of the layer: queries, window rows, pooled
   * entries, indexer queries and keys, the output's -t rotation).  With
   * rope_factor = s > 1 the frequency of pair j of R rope channels,
   * theta_j = rope_theta^(-2j/R), becomes theta_j (1 - r_j) + (theta_j / s) r_j,
   * the ramp r_j rising linearly in j from 0 at lo to 1 at hi, where lo / hi
   * are the pair indices, rounded down / up and clamped to [0, R - 1], at
   * which a pair turns rope_beta_fast / rope_beta_slow times over
   * rope_original_context positions:
   * R ln(rope_original_context / (2 pi n)) / (2 ln rope_theta).  Only the
   * frequencies change; any logit temperature goes through softmax_scale.
   * rope_factor 0 (or 1) leaves the rope unscaled and the other three fields
   * unread.  Source: optimum-intel issue 1748, "What V4-Flash adds vs V3"
   * (YaRN factor 16, 65k -> 1M context). */
  double rope_factor;           /* s: 0, or >= 1                              */
  double rope_original_context; /* > 0 when rope_factor > 1                   */
  double rope_beta_fast;        /* > rope_beta_slow > 0 when rope_factor > 1  */
  double rope_beta_slow;
} csa_layer;

/* Geometry of one call. */
typedef struct {
  int32_t batch;            /* B >= 1 sequences                                */
  int32_t n_new;            /* tokens per sequence in this call, >= 1          */
  const int64_t* pos0;      /* device [B]: position of each first new token    */
  int64_t pos0_max;         /* host: an upper bound of every pos0[b] (>= 0),
                               used to validate capacities; 0 also lets a
                               prefill's compressor state update run in the
                               entries' launch (no entry reads the state)      */
  const int32_t* n_valid;   /* device [B] or NULL: variable-length calls.
                               Sequence b has n_valid[b] valid tokens (clamped
                               to 0 .. n_new), the first ones of its n_new
                               rows; the rest are padding.  csa_window_append
                               and csa_compress advance the window ring, the
                               pool and the compressor state by the valid
                               tokens only (a later call continues at
                               pos0[b] + n_valid[b]); the index and attention
                               calls leave their outputs for padding rows
                               unspecified (they read only in-bounds rows).
                               NULL: every sequence has n_new tokens.        */
  /* Packed variable-length rows (NULL: rows of sequence b are b n_new .. b n_new
   * + n_new - 1, padded).  With cu_seqlens, a device [B + 1] array of
   * non-decreasing row offsets, sequence b has the cu_seqlens[b + 1] -
   * cu_seqlens[b] tokens (at most n_new; n_new is then the longest sequence's
   * length) in rows cu_seqlens[b] .. cu_seqlens[b + 1] - 1 of every per-token
   * tensor (kv, gate, q, q_idx, weights, topk_idx, out, csa_rope's x): the
   * tensors hold no padding rows.  Mutually exclusive with n_valid.  The
   * scores_out rows of csa_index_topk stay indexed by b n_new + i.          */
  const int32_t* cu_seqlens;
  /* Paged pools (NULL: every pool argument is the contiguous [B, pool_cap,
   * width] tensor).  With block_table, a device [B, block_table_stride] int32
   * array, entry w of sequence b lives in row
   *   block_table[b][w / block_entries] * block_entries + w % block_entries
   * of the pool tensor, which holds pool_blocks blocks of block_entries rows
   * ([pool_blocks * block_entries, width]); pool_cap stays the entries per
   * sequence and must not exceed block_table_stride * block_entries.  The main
   * pool and the indexer pool of a layer share the entry ids and so one table
   * (two tensors of different widths); each layer has its own table, since
   * the layers' pools differ in ratio and size.  The table entries a call
   * touches (blocks holding entries below (pos0[b] + n_new) / m) must lie in
   * 0 .. pool_blocks - 1 and must not be shared between sequences that a call
   * writes (not checked).  Window rings and compressor states do not grow with
   * the context and stay per-sequence arrays.
   * Source: model page, "Cache layers" (one cache type per layer, each with
   * its own pool); optimum-intel issue 1748 ("What native registration would
   * touch": the KV cache is not uniform across layers). */
  const int32_t* block_table;
  int32_t block_entries;       /* a power of two, 128 .. 2^24 (paged)          */
  int32_t block_table_stride;  /* blocks per sequence row of block_table       */
  int64_t pool_blocks;         /* blocks in each pool tensor (paged)          */
} csa_batch;

/* Write the window rows of the new tokens into a ring buffer.
 * Layout and meaning: kv [B, n_new, D] (dtype) holds the un-rotated K=V rows
 * of the new tokens; each is rotated at its position t (rope on the last R
 * channels, base rope_theta) and stored at ring[b, t mod cap, :], ring being
 * [B, cap, D] (dtype).  For a query of this call to find all its window rows,
 * cap must be >= min(W + n_new - 1, pos0_max + n_new); a linear buffer of a
 * prefill from position 0 is the case cap >= n_new + pos0_max.
 * Source: model page, sec. 2.3 (sliding window branch, K=V stored once). */
csa_status csa_window_append(const csa_layer* layer, const csa_batch* batch,
                             const void* kv, void* ring, int64_t cap,
                             hipStream_t stream);

/* Rotate rows in place: x [B, n_new, rows_per_token, width] (dtype; packed:
 * [rows, rows_per_token, width]); row r of token i of sequence b is rotated
 * at position sign * (pos0[b] + i) on its last rope_dim channels, interleaved
 * pairs (c, c+1) as complex numbers, frequency base^(-2j/rope_dim) for pair j
 * (YaRN-scaled as the layer's rope_factor asks).  sign is +1 or -1.  Rows of
 * padding tokens (n_valid) are left as they are.
 * Source: transformers PR 45616 notes on RoPE apply (interleaved-pair
 * rotation via complex multiplication) and the model page, sec. 2.3. */
csa_status csa_rope(const csa_layer* layer, const csa_batch* batch, void* x,
                    int32_t rows_per_token, int32_t width, int32_t rope_dim,
                    int32_t sign, hipStream_t stream);

/* KV compressor: learned gated pooling of one stream (the main K=V stream,
 * width = head_dim and rope_dim = qk_rope_head_dim, or the indexer's key
 * stream, width = index_head_dim and rope_dim = index_rope_dim).
 *  kv, gate    [B, n_new, width] dtype: raw rows and per-channel gate logits
 *              of the new tokens.
 *  norm_weight [width] float32 or NULL: optional RMSNorm after pooling
 *              (x / sqrt(mean(x^2) + norm_eps) * weight).
 *  state_kv, state_gate [B, (1+overlap)*m, width] dtype: the caller-owned
 *              compressor state, raw tokens of position p at slot
 *              p mod ((1+overlap)*m); zero-fill before a sequence starts,
 *              then pass unchanged between calls.  Updated by this call.
 *  pool        [B, pool_cap, width] dtype: entry w at row w.  Every entry
 *              closing in this call, w in [pos0/m, (pos0+n_new)/m), is
 *              written: per channel, softmax over the entry's tokens of the
 *              gate logits weights the kv values; then RMSNorm if given; then
 *              rotation at position w*m.  Entry w pools tokens
 *              [(w-overlap)*m, (w+1)*m) that are >= 0.  Rows of entries that
 *              do not close are left untouched; a call in which no entry
 *              closes writes only the state and returns CSA_OK.
 *  Requires m >= 1, pool_cap >= (pos0_max + n_new)/m.
 * Source: model page, sec. 2.3 (CSA overlapping windows, HCA non-overlapping)
 * and "Cache layers" (buffer, pool, counter, overlap state);
 * TransformerLens adapter, compressor submodules kv_proj, gate_proj,
 * kv_norm, rotary_emb; transformers PR 45616 (stateless compressor, state
 * in the cache, always returns a possibly empty tensor). */
csa_status csa_compress(const csa_layer* layer, const csa_batch* batch,
                        int32_t width, int32_t rope_dim, const void* kv,
                        const void* gate, const float* norm_weight,
                        float norm_eps, void* state_kv, void* state_gate,
                        void* pool, int64_t pool_cap, hipStream_t stream);

/* All of a layer call's cache updates in one call: csa_window_append of kv
 * into ring, then (compress_ratio > 0) csa_compress of the main stream
 * (width head_dim, rope_dim qk_rope_head_dim, ckv / cgate / norm_weight,
 * state_kv / state_gate / pool) and (index_topk > 0) of the indexer's key
 * stream (width index_head_dim, rope_dim index_rope_dim, ikv / igate /
 * inorm_weight, istate_kv / istate_gate / ipool); both pools share pool_cap
 * and the batch's block table.  Arguments, layouts and results are those of
 * the separate calls, bit for bit; pointers of a stream the layer does not
 * have are ignored (may be NULL).  With n_new == 1 (a decode step) the three
 * updates run as one launch, one block per (sequence, stream): a decode
 * step is a chain of small launches, each costing a few microseconds of
 * launch latency.  With n_new > 1 the separate kernels run in order.
 * Source: model page, "Cache layers" (the window, the compressor buffer /
 * pool / counter / overlap state, the indexer's own buffer and pool, one
 * cache update per call) and sec. 2.3. */
csa_status csa_cache_update(const csa_layer* layer, const csa_batch* batch,
                            const void* kv, void* ring, int64_t win_cap,
                            const void* ckv, const void* cgate, const float* norm_weight,
                            void* state_kv, void* state_gate, void* pool,
                            const void* ikv, const void* igate, const float* inorm_weight,
                            void* istate_kv, void* istate_gate, void* ipool,
                            int64_t pool_cap, float norm_eps, hipStream_t stream);

/* Lightning Indexer and per-query top-k (CSA layers).
 *  q_idx    [B, n_new, H_I, D_I] dtype: indexer queries, un-rotated (rotated
 *           here at t on their last R_I channels, stored at dtype).
 *  weights  [B, n_new, H_I] dtype: per-head weights of the scorer.
 *  k_pool   [B, pool_cap, D_I] dtype: pooled indexer keys (csa_compress
 *           output of the indexer stream, rotated).
 *  score(t, w) = sum_h weights[t,h] * ReLU(rot(q_idx[t,h]) . k_pool[w]) for
 *           every visible w < (t+1)/m, accumulated in float32.
 *  topk_idx [B, n_new, index_topk] int32 out: the index_topk visible entries
 *           of highest score, ties to the lower entry id, -0 == +0; emitted in
 *           ascending entry order and padded with -1 when fewer are visible.
 *  scores_out [B, n_new, pool_cap] float32 or NULL: the scores of the visible
 *           entries (other columns untouched), for inspection.
 *  workspace of at least csa_workspace_bytes(layer, B, n_new, pool_cap,
 *           CSA_OP_INDEX_TOPK) bytes.  Scores must be finite.
 * Source: model page, sec. 2.3 (Lightning Indexer scores queries against the
 * pool and gathers the top index_topk blocks per query) and "Attention mask
 * layout" (the -1 sentinel); TransformerLens adapter (indexer q_b_proj,
 * scorer.weights_proj, rotary_emb). */
csa_status csa_index_topk(const csa_layer* layer, const csa_batch* batch,
                          const void* q_idx, const void* weights,
                          const void* k_pool, int64_t pool_cap,
                          int32_t* topk_idx, float* scores_out,
                          void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* csa_index_topk without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments (minus workspace), same
 * results, same kernels.  The workspace is a static device array of the
 * library, CSA_NOALLOC_SCRATCH_BYTES bytes, one copy per device, held until
 * the process ends; its device address is looked up once per device (the
 * current device at the call; `stream` must belong to it).  A call whose
 * workspace (csa_workspace_bytes(..., CSA_OP_INDEX_TOPK)) exceeds that size
 * returns CSA_ERR_SCRATCH before any launch, e.g. decode of 64 sequences
 * over 32768-entry pools needs about 26 MiB.  Every call on a device shares
 * that device's array and leaves its contents behind: calls that overlap in
 * time on one device (different streams, or host threads racing) corrupt
 * each other's selection; calls queued on one stream are ordered and safe.
 * The call allocates nothing (no hipMalloc / hipFree). */
#define CSA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
csa_status csa_index_topk_noalloc(const csa_layer* layer, const csa_batch* batch,
                                  const void* q_idx, const void* weights,
                                  const void* k_pool, int64_t pool_cap,
                                  int32_t* topk_idx, float* scores_out,
                                  hipStream_t stream);

/* CSA attention: per query t and head h, one softmax over the window rows of
 * t (from the ring written by csa_window_append) and the pooled rows listed in
 * topk_idx[t] (entries < 0 are skipped), plus the sink logit sinks[h]; the
 * value of every row is the row itself (K = V).
 *  q      [B, n_new, H, D] dtype, un-rotated (rotated at t, stored at dtype).
 *  win    [B, win_cap, D] dtype ring (row of position p at slot p mod cap).
 *  pool   [B, pool_cap, D] dtype rotated pooled rows.
 *  topk_idx [B, n_new, index_topk] int32.
 *  sinks  [H] float32 or NULL (no sink).
 *  out    [B, n_new, H, D] dtype: sum_j p_j row_j, its rope slice rotated at
 *         -t (eq. 26 on the model page).
 *  workspace of csa_workspace_bytes(..., CSA_OP_ATTEND) bytes (decode splits).
 * Source: model page, sec. 2.3 (shared K=V MQA, sliding branch concatenated
 * with the compressor output before the main attention, sink eq. 27, output
 * rotation eq. 26) and "Attention mask layout"; transformers PR 45616 (sink
 * ported from the GPT-OSS eager attention). */
csa_status csa_attend(const csa_layer* layer, const csa_batch* batch,
                      const void* q, const void* win, int64_t win_cap,
                      const void* pool, int64_t pool_cap,
                      const int32_t* topk_idx, const float* sinks, void* out,
                      void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* HCA / sliding-only attention: as csa_attend, but the pooled rows of query t
 * are every visible entry w < (t+1)/m; compress_ratio == 0 attends to the
 * window alone.  workspace: csa_workspace_bytes(..., CSA_OP_HCA_ATTEND).
 * With H = 64, D = 512 in bf16, a query attends to at most 262144 rows
 * (window + pool_cap); beyond that the call returns CSA_ERR_UNSUPPORTED.
 * Source: model page, sec. 2.3 (HCA has no indexer, every pool entry takes
 * part; sliding_attention layers have no long-range branch). */
csa_status hca_attend(const csa_layer* layer, const csa_batch* batch,
                      const void* q, const void* win, int64_t win_cap,
                      const void* pool, int64_t pool_cap, const float* sinks,
                      void* out, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

enum { CSA_OP_INDEX_TOPK = 1, CSA_OP_ATTEND = 2, CSA_OP_HCA_ATTEND = 3 };

/* Workspace bytes an entry point needs for these sizes (0 if none); the
 * pointer passed must be 256-byte aligned.  Returns (size_t)-1 for an
 * invalid layer or op. */
size_t csa_workspace_bytes(const csa_layer* layer, int32_t batch, int32_t n_new,
                           int64_t pool_cap, int32_t op);

/* Grouped low-rank output projection, the step after the attention.
 * Source: model page, sec. 2.3 ("Grouped Output Projection": o_groups groups
 * of heads -> o_lora_rank per group -> hidden_size, o_a_proj then o_b_proj);
 * transformers PR 45616 notes (DeepseekV4GroupedLinear keeps an (out, in)
 * weight and runs a per-group bmm).  The pages give no sizes.
 *  attn_out [tokens, num_heads, head_dim] bf16: the attention output (after
 *           the -t rotation), heads of group g = g H/G .. (g+1) H/G - 1.
 *  w_a      [o_groups * o_lora_rank, (num_heads / o_groups) * head_dim] bf16:
 *           o_a_proj's weight; rows g R .. g R + R - 1 belong to group g.
 *  w_b      [hidden_size, o_groups * o_lora_rank] bf16: o_b_proj's weight.
 *  out      [tokens, hidden_size] bf16 out:
 *           y[t, g, r] = sum_i attn_out[t, group g, i] w_a[g R + r, i] (bf16),
 *           out[t, h] = sum_j y[t, j] w_b[h, j]; float32 accumulation, each
 *           stored value rounded once; no bias.
 *  workspace >= csa_output_projection_workspace_bytes(p) bytes (holds y).
 * Requires o_groups to divide num_heads (else CSA_ERR_SHAPE),
 * (num_heads / o_groups) * head_dim and o_groups * o_lora_rank to be
 * multiples of 32, num_heads * head_dim and o_groups * o_lora_rank to be at
 * most 2^22, tokens <= 2^23, and attn_out, w_a and w_b to be 16-byte
 * aligned (else CSA_ERR_UNSUPPORTED).  The caller owns every buffer; the two
 * products are queued on `stream` in order and the call returns without
 * waiting.  attn_out, w_a, w_b, out and workspace must not overlap. */
typedef struct {
  int32_t tokens;       /* T >= 1 rows                                       */
  int32_t num_heads;    /* H                                                 */
  int32_t head_dim;     /* D                                                 */
  int32_t o_groups;     /* G, divides H                                      */
  int32_t o_lora_rank;  /* R >= 1                                            */
  int32_t hidden_size;  /* >= 1                                              */
} csa_oproj;

csa_status csa_output_projection(const csa_oproj* p, const void* attn_out,
                                 const void* w_a, const void* w_b, void* out,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Workspace bytes of csa_output_projection (256-byte aligned pointer), or
 * (size_t)-1 for invalid sizes. */
size_t csa_output_projection_workspace_bytes(const csa_oproj* p);

/* Producer projections: the layer's inputs from the block's normalised
 * hidden states.
 * Source: TransformerLens deepseek_v4 adapter, the self_attn module list
 * (q_a_proj, q_a_norm, q_b_proj, q_b_norm, kv_proj, kv_norm, compressor) and
 * its compressor / indexer submodules (kv_proj, gate_proj, q_b_proj,
 * scorer.weights_proj); model page, sec. 2.3 (kv_proj makes the single K=V
 * head).  The pages give no sizes.
 *  x      [tokens, hidden] bf16.
 *  w_x    [q_lora + D + 2 comp + 2 D_I + H_I, hidden] bf16, (out, in) rows
 *         stacked in this order: q_a_proj, kv_proj, compressor kv_proj,
 *         compressor gate_proj, indexer kv_proj, indexer gate_proj,
 *         weights_proj (a stream of width 0 is absent).
 *  g_qa   [q_lora] float: q_a_norm weight;  g_kv [D] float: kv_norm weight.
 *  w_q    [H D + H_I D_I, q_lora] bf16: q_b_proj rows, then the indexer's
 *         q_b_proj rows.
 *  Outputs (bf16, row-major, the layout csa_window_append / csa_compress /
 *  csa_index_topk / csa_attend take): q [tokens, H, D], kv [tokens, D],
 *  ckv and cgate [tokens, comp], ikv and igate [tokens, D_I],
 *  qi [tokens, H_I, D_I], wi [tokens, H_I]; pointers of absent streams may
 *  be NULL.
 *  latent = q_a_norm(x w_qa^T), kv = kv_norm(x w_kv^T), q = latent w_qb^T
 *  (then, with q_head_norm, each head divided by its RMS over D), the other
 *  streams plain products; every product and norm output is stored at bf16
 *  (float32 accumulation; the norms over the stored values, RMSNorm(y) =
 *  y / sqrt(mean(y^2) + eps) * g, in float64, except q_head_norm on heads
 *  of D = 512 with q 16-byte aligned: float32, inside the product's
 *  epilogue, one bf16 unit at most from the float64 result).
 *  workspace >= csa_project_workspace_bytes(p) bytes (holds the latent).
 * Requires hidden and q_lora to be multiples of 32, every width to be >= 0
 * (q_lora, H, D >= 1), comp, D_I and H_I either all set or zero as the layer
 * has them, and x, w_x, w_q 16-byte aligned (else CSA_ERR_SHAPE or
 * CSA_ERR_UNSUPPORTED).  Buffers must not overlap; the call queues its
 * launches on `stream` and returns. */
typedef struct {
  int32_t tokens;       /* T >= 1                                   */
  int32_t hidden;       /* multiple of 32                           */
  int32_t q_lora_rank;  /* multiple of 32                           */
  int32_t num_heads;    /* H >= 1                                   */
  int32_t head_dim;     /* D >= 1                                   */
  int32_t comp_dim;     /* compressor width (D) or 0                */
  int32_t index_dim;    /* D_I or 0                                 */
  int32_t index_heads;  /* H_I or 0                                 */
  float eps;            /* RMSNorm epsilon                          */
  int32_t q_head_norm;  /* 1: q_b_norm on each head, 0: none        */
} csa_proj;

csa_status csa_project(const csa_proj* p, const void* x, const void* w_x,
                       const float* g_qa, const float* g_kv, const void* w_q,
                       void* q, void* kv, void* ckv, void* cgate, void* ikv,
                       void* igate, void* qi, void* wi, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of csa_project (256-byte aligned pointer), or (size_t)-1
 * for invalid sizes. */
size_t csa_project_workspace_bytes(const csa_proj* p);

/* Static description of a status code. */
const char* csa_status_str(csa_status status);

/* Library version, major*10000 + minor*100 + patch. */
int32_t csa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H_ */
