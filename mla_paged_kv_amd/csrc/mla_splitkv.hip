// FP8-with-scale cache launcher (the kernel template is in
// mla_splitkv_kernel.h).
#include "mla_splitkv_kernel.h"

namespace mla {

hipError_t launch_splitkv_fp8(const SplitKVParams& p, bool sparse, hipStream_t stream) {
  return launch_splitkv_fp8_t(p, sparse, stream);
}

}  // namespace mla
