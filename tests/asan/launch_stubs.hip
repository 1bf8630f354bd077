// Launch stubs for the host-side sanitizer build of the C ABI: every kernel
// launcher of libcsa is replaced by a function that records the call and
// launches nothing, so the argument checks and the planning code (api.hip,
// plan.hip) run under AddressSanitizer without touching a device.
#include "csa_internal.h"

int g_launches = 0;

namespace csa {

#define CSA_STUB(...) \
  hipError_t __VA_ARGS__ { ++g_launches; return hipSuccess; }

CSA_STUB(launch_gemm_nt_routed(const bf16_t*, const bf16_t*, int, int, int, int64_t, int64_t,
                               const GemmOut&, hipStream_t))
CSA_STUB(launch_project(int, int, int, int, int, int, int, int, float, int, const bf16_t*,
                        const bf16_t*, const float*, const float*, const bf16_t*, bf16_t*,
                        bf16_t*, bf16_t*, bf16_t*, bf16_t*, bf16_t*, bf16_t*, bf16_t*, bf16_t*,
                        hipStream_t))
CSA_STUB(launch_output_projection(int, int, int, int, int, int, const bf16_t*, const bf16_t*,
                                  const bf16_t*, bf16_t*, bf16_t*, hipStream_t))
CSA_STUB(launch_window_append(const Layer&, const Batch&, const void*, void*, int64_t,
                              hipStream_t))
CSA_STUB(launch_rope(const Layer&, const Batch&, void*, int, int, int, int, hipStream_t))
CSA_STUB(launch_compress(const Layer&, const Batch&, int, int, const void*, const void*,
                         const float*, float, void*, void*, void*, int64_t, hipStream_t,
                         const CmpArgs*, const WinArgs*))
CSA_STUB(launch_cache_update_one(const Layer&, const Batch&, const void*, void*, int64_t,
                                 const void*, const void*, const float*, void*, void*, void*,
                                 const void*, const void*, const float*, void*, void*, void*,
                                 int64_t, float, int, hipStream_t))
CSA_STUB(launch_index_topk(const Layer&, const Batch&, const void*, const void*, const void*,
                           int64_t, int32_t*, float*, void*, hipStream_t))
CSA_STUB(launch_attend_decode(const Layer&, const Batch&, const void*, const void*, int64_t,
                              const void*, int64_t, const int32_t*, const float*, void*, void*,
                              bool, int, hipStream_t))
CSA_STUB(launch_attend(const Layer&, const Batch&, const void*, const void*, int64_t,
                       const void*, int64_t, const int32_t*, const float*, void*, void*, bool,
                       hipStream_t))

}  // namespace csa
