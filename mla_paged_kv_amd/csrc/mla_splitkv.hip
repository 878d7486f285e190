// Pair-kernel launcher for bf16 caches and the FP8-with-scale cache (the
// kernel template is in mla_splitkv_kernel.h; the fp16 instantiations are in
// mla_splitkv_f16.hip so the two translation units compile in parallel).
#include "mla_splitkv_kernel.h"

namespace mla {

hipError_t launch_pairs(const SplitKVParams& p, int d_qk, bool sparse, bool fp8, bool f16,
                        hipStream_t stream) {
  if (f16) return launch_pairs_f16(p, d_qk, sparse, stream);
  return launch_pairs_t<false>(p, d_qk, sparse, fp8, stream);
}

}  // namespace mla
