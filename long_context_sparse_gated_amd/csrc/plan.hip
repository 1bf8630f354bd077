// Host-side planning of libcsa: which kernels a call takes, how its rows are
// split over blocks, and the workspace each entry point needs.  Host code
// only (no kernels), so the argument checks of the C ABI and this planning can
// be built and run without a device.
#include "csa_internal.h"

namespace csa {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------
// indexer and top-k

bool index_fast_shape(const Layer& L) {
  return L.dtype == 1 && L.Hi == 64 && L.Di == 128 && L.Ri <= 128;
}

// Few new tokens per sequence over a pool the selection buffers can index.
bool index_decode_path(const Layer& L, int n, int64_t pool_cap) {
  return index_fast_shape(L) && n < kIdxQPB && (pool_cap + kSlice - 1) / kSlice <= kMaxSlices;
}

size_t index_workspace_bytes(const Layer& L, int B, int n, int64_t pool_cap) {
  const size_t bn = (size_t)B * n;
  size_t s = align256(bn * pool_cap * sizeof(float));
  if (index_decode_path(L, n, pool_cap)) {
    const size_t nslice = (size_t)((pool_cap + kSlice - 1) / kSlice);
    s += align256(bn * L.Hi * L.Di * 2);                     // rotated queries
    s += align256(bn * kHBins * sizeof(uint32_t));           // score histograms
    s += 2 * align256(bn * pool_cap * sizeof(int32_t));      // candidate ids
    s += align256(bn * nslice * 2 * sizeof(uint32_t) + 64);  // per-slice counts, discard
  } else if (index_fast_shape(L)) {
    s += 256;  // discard slots of index_prefill_x32
  }
  return s;
}

// ---------------------------------------------------------------------------
// attention

bool attend_fast_shape(const Layer& L) {
  return L.dtype == 1 && L.H == kAH && L.D == kAD && L.W >= 1 &&
         (L.R == 16 || L.R == 32 || L.R == 64 || L.R == 128);
}

static int64_t attend_rows(const Layer& L, int64_t pool_cap, bool csa) {
  int64_t npool = 0;
  if (L.m > 0) npool = csa ? (pool_cap < L.k ? pool_cap : (int64_t)L.k) : pool_cap;
  return (int64_t)L.W + npool;
}

// Calls of fewer than 256 tokens run attend_decode (rows and head groups
// spread over the chip), except a few tokens with long row lists: there
// attend_mfma's 64-head blocks, each splitting a list over many blocks, keep
// more rows in flight per block (4 tokens x 8320 HCA rows: 28 + 12.5 us of
// attention and merge against 56 + 7 us on attend_decode).
bool attend_dec(const Layer& L, int B, int n, int64_t pool_cap, bool csa) {
  const int64_t tokens = (int64_t)B * n;
  return tokens < 256 && (tokens >= 16 || attend_rows(L, pool_cap, csa) <= 256);
}

// Row slices per token of attend_decode: about 256 blocks over the call,
// whole chunks each, at most kDMaxRows rows per block; -1 if more slices
// than the merge takes.
int attend_decode_splits(const Layer& L, int B, int n, int64_t pool_cap, bool csa) {
  const int64_t nch = (attend_rows(L, pool_cap, csa) + kDCh - 1) / kDCh;
  const int64_t tokens = (int64_t)B * n;
  int64_t s = 64 / tokens;
  // a slice keeps >= 4 chunks: shorter ones cost more in partials and the
  // merge launch than they gain in parallel gathers (4 tokens x 128 window
  // rows: 13.6 us in one slice against 13.8 + 5.0 us in two and a merge)
  if (s > nch / 4) s = nch / 4;
  const int64_t need = (nch * kDCh + kDMaxRows - 1) / kDMaxRows;
  if (s < need) s = need;
  if (s < 1) s = 1;
  return s > kMaxSplits ? -1 : (int)s;
}

int attend_splits(const Layer& L, int B, int n, int64_t pool_cap, bool csa) {
  if (!attend_fast_shape(L)) return 1;
  if (attend_dec(L, B, n, pool_cap, csa)) return attend_decode_splits(L, B, n, pool_cap, csa);
  const int64_t nch = (attend_rows(L, pool_cap, csa) + kCH - 1) / kCH;
  const int64_t tokens = (int64_t)B * n;
  // no block above kMaxRows rows; calls of fewer than 256 tokens also split
  // while the grid is short of ~2 blocks per CU and every split keeps >= 4
  // chunks (128 rows: its float32 partial, 64 x 516 words, costs about as
  // much traffic as the rows)
  const int64_t need = (nch * kCH + kMaxRows - 1) / kMaxRows;
  int64_t s = tokens >= 256 ? 1 : (512 + tokens - 1) / tokens;
  const int64_t cap = nch / (128 / kCH) > 1 ? nch / (128 / kCH) : 1;
  if (s > cap) s = cap;
  if (s < need) s = need;
  if (s < 1) s = 1;
  return s > kMaxSplits ? -1 : (int)s;  // -1: too many rows
}

size_t attend_workspace_bytes(const Layer& L, int B, int n, int64_t pool_cap, bool csa) {
  const int s = attend_splits(L, B, n, pool_cap, csa);
  if (s <= 1) return 0;
  return (size_t)B * n * s * kAH * kPart * sizeof(float);
}

}  // namespace csa
