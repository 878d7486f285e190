// Pair-kernel launcher for fp16 caches (the kernel template is in
// mla_splitkv_kernel.h).
#include "mla_splitkv_kernel.h"

namespace mla {

hipError_t launch_pairs_f16(const SplitKVParams& p, int d_qk, bool sparse, hipStream_t stream) {
  return launch_pairs_t<true>(p, d_qk, sparse, false, stream);
}

}  // namespace mla
