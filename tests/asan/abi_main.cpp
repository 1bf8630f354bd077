// Host-side sanitizer run of the C ABI's argument checks and planning: calls
// that must be rejected, calls that pass validation (their launches are stubs
// that record them), workspace sizing and status strings.  Exit status 0 when
// every expectation holds; AddressSanitizer aborts on any memory error.
#include <stdio.h>
#include <stdint.h>

#include <vector>

#include "csa.h"

extern int g_launches;

static int failures = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,    \
              __LINE__, #cond);                                       \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static csa_layer csa_spec() {
  csa_layer L{};
  L.dtype = CSA_BF16;
  L.num_heads = 64;
  L.head_dim = 512;
  L.qk_rope_head_dim = 64;
  L.rope_theta = 160000.0;
  L.sliding_window = 128;
  L.compress_ratio = 4;
  L.overlap = 1;
  L.index_n_heads = 64;
  L.index_head_dim = 128;
  L.index_rope_dim = 64;
  L.index_topk = 512;
  L.rope_factor = 16.0;
  L.rope_original_context = 65536.0;
  L.rope_beta_fast = 32.0;
  L.rope_beta_slow = 1.0;
  return L;
}

int main() {
  // host buffers stand in for device pointers: the stubs never read them
  std::vector<int64_t> pos0(64, 0);
  std::vector<int32_t> nvalid(64, 1), cu(65, 0), table(64 * 256, 0);
  std::vector<uint8_t> buf(1 << 20);
  void* P = buf.data();
  csa_layer L = csa_spec();
  csa_batch B{};
  B.batch = 1;
  B.n_new = 8192;
  B.pos0 = pos0.data();
  B.pos0_max = 0;

  // status strings cover every code
  for (int s = 0; s <= CSA_ERR_SCRATCH; ++s) EXPECT(csa_status_str((csa_status)s)[0] == 'C');
  EXPECT(csa_version() >= 400);

  // workspace sizes
  const size_t wi = csa_workspace_bytes(&L, 1, 8192, 2048, CSA_OP_INDEX_TOPK);
  EXPECT(wi >= (size_t)8192 * 2048 * 4);
  EXPECT(csa_workspace_bytes(&L, 1, 8192, 2048, CSA_OP_ATTEND) == 0);
  EXPECT(csa_workspace_bytes(&L, 4, 1, 262144, CSA_OP_ATTEND) > 0);
  EXPECT(csa_workspace_bytes(&L, 1, 1, 1, 99) == (size_t)-1);
  EXPECT(csa_workspace_bytes(nullptr, 1, 1, 1, 1) == (size_t)-1);

  // rejections, each before any launch
  const int before = g_launches;
  EXPECT(csa_attend(nullptr, &B, P, P, 8192, P, 2048, (int32_t*)P, nullptr, P, nullptr, 0,
                    nullptr) == CSA_ERR_NULL);
  EXPECT(csa_attend(&L, &B, P, P, 8191, P, 2048, (int32_t*)P, nullptr, P, nullptr, 0, nullptr) ==
         CSA_ERR_SHAPE);
  EXPECT(csa_attend(&L, &B, P, P, 8192, P, 2047, (int32_t*)P, nullptr, P, nullptr, 0, nullptr) ==
         CSA_ERR_SHAPE);
  csa_layer bad = L;
  bad.qk_rope_head_dim = 63;
  EXPECT(csa_attend(&bad, &B, P, P, 8192, P, 2048, (int32_t*)P, nullptr, P, nullptr, 0, nullptr) ==
         CSA_ERR_SHAPE);
  bad = L;
  bad.rope_factor = 0.5;
  EXPECT(csa_window_append(&bad, &B, P, P, 8192, nullptr) == CSA_ERR_SHAPE);
  EXPECT(csa_index_topk(&L, &B, P, P, P, 2048, (int32_t*)P, nullptr, nullptr, 0, nullptr) ==
         CSA_ERR_WORKSPACE);
  EXPECT(csa_index_topk(&L, &B, P, P, P, 2048, (int32_t*)P, nullptr, (char*)P + 16, 1 << 30,
                        nullptr) == CSA_ERR_WORKSPACE);
  EXPECT(csa_index_topk_noalloc(&L, &B, P, P, P, 2048, (int32_t*)P, nullptr, nullptr) ==
         CSA_ERR_SCRATCH);
  EXPECT(csa_rope(&L, &B, P, 1, 512, 65, 1, nullptr) == CSA_ERR_SHAPE);
  EXPECT(csa_compress(&L, &B, 4096, 64, P, P, nullptr, 1e-6f, P, P, P, 2048, nullptr) ==
         CSA_ERR_SHAPE);
  csa_batch both = B;
  both.n_valid = nvalid.data();
  both.cu_seqlens = cu.data();
  EXPECT(csa_window_append(&L, &both, P, P, 8192, nullptr) == CSA_ERR_SHAPE);
  csa_batch paged = B;
  paged.block_table = table.data();
  paged.block_entries = 192;  // not a power of two
  paged.block_table_stride = 16;
  paged.pool_blocks = 16;
  EXPECT(csa_attend(&L, &paged, P, P, 8192, P, 2048, (int32_t*)P, nullptr, P, nullptr, 0,
                    nullptr) == CSA_ERR_SHAPE);
  paged.block_entries = 128;
  paged.block_table_stride = 15;  // 1920 entries < pool_cap
  EXPECT(csa_compress(&L, &paged, 512, 64, P, P, nullptr, 1e-6f, P, P, P, 2048, nullptr) ==
         CSA_ERR_SHAPE);
  csa_oproj op{8192, 64, 512, 7, 1024, 4096};  // 7 groups do not divide 64 heads
  EXPECT(csa_output_projection_workspace_bytes(&op) == (size_t)-1);
  EXPECT(csa_output_projection(&op, P, P, P, P, P, 1 << 20, nullptr) == CSA_ERR_SHAPE);
  csa_proj pj{8192, 4004, 1024, 64, 512, 512, 128, 64, 1e-6f, 1};  // hidden not a multiple of 32
  EXPECT(csa_project_workspace_bytes(&pj) == (size_t)-1);
  EXPECT(g_launches == before);

  // calls that pass validation reach the (stub) launches
  std::vector<uint8_t> ws(wi + 256);
  void* wsa = (void*)(((uintptr_t)ws.data() + 255) & ~(uintptr_t)255);
  EXPECT(csa_window_append(&L, &B, P, P, 8192, nullptr) == CSA_OK);
  EXPECT(csa_compress(&L, &B, 512, 64, P, P, nullptr, 1e-6f, P, P, P, 2048, nullptr) == CSA_OK);
  EXPECT(csa_index_topk(&L, &B, P, P, P, 2048, (int32_t*)P, nullptr, wsa, wi, nullptr) == CSA_OK);
  EXPECT(csa_attend(&L, &B, P, P, 8192, P, 2048, (int32_t*)P, nullptr, P, nullptr, 0, nullptr) ==
         CSA_OK);
  csa_batch packed = B;
  packed.batch = 4;
  packed.n_new = 2048;
  packed.cu_seqlens = cu.data();
  packed.block_table = table.data();
  packed.block_entries = 256;
  packed.block_table_stride = 2;
  packed.pool_blocks = 8;
  EXPECT(csa_rope(&L, &packed, P, 64, 512, 64, -1, nullptr) == CSA_OK);
  EXPECT(csa_compress(&L, &packed, 128, 64, P, P, nullptr, 1e-6f, P, P, P, 512, nullptr) ==
         CSA_OK);
  const size_t wa = csa_workspace_bytes(&L, 4, 1, 262144, CSA_OP_ATTEND);
  std::vector<uint8_t> ws2(wa + 256);
  void* wsb = (void*)(((uintptr_t)ws2.data() + 255) & ~(uintptr_t)255);
  csa_batch dec = B;
  dec.batch = 4;
  dec.n_new = 1;
  dec.pos0_max = 1048576;
  EXPECT(csa_attend(&L, &dec, P, P, 128, P, 262144, (int32_t*)P, nullptr, P, wsb, wa, nullptr) ==
         CSA_OK);
  csa_oproj op2{8192, 64, 512, 8, 1024, 4096};
  const size_t wo = csa_output_projection_workspace_bytes(&op2);
  EXPECT(wo == (size_t)8192 * 8 * 1024 * 2);
  EXPECT(g_launches == before + 7);

  if (failures) {
    fprintf(stderr, "%d expectations failed\n", failures);
    return 1;
  }
  printf("abi checks ok (%d stub launches)\n", g_launches);
  return 0;
}
