// Split-KV launcher for bf16 inputs (and the FP8 cache).  The kernel template
// is in mla_splitkv_kernel.h; the fp16 instantiations live in
// mla_splitkv_f16.hip so the two translation units compile in parallel.
#include "mla_splitkv_kernel.h"

namespace mla {

hipError_t launch_splitkv(const SplitKVParams& p, int d_qk, bool sparse, bool fp8, bool f16,
                          hipStream_t stream) {
  if (f16) return launch_splitkv_f16(p, d_qk, sparse, stream);
  return launch_splitkv_t<false>(p, d_qk, sparse, fp8, stream);
}

}  // namespace mla
