// Launcher of the narrow kernel (units of at most 16 query rows; the kernel
// template is in mla_narrow_kernel.h): bf16, fp16 and FP8-with-scale caches.
#include "mla_narrow_kernel.h"

namespace mla {

hipError_t launch_narrow(const SplitKVParams& p, int d_qk, bool sparse, bool fp8, bool f16,
                         hipStream_t stream) {
  return f16 ? launch_narrow_t<true>(p, d_qk, sparse, false, stream)
             : launch_narrow_t<false>(p, d_qk, sparse, fp8, stream);
}

}  // namespace mla
