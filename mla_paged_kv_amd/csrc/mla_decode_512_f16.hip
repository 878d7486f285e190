// fp16 instantiations of the decode kernel for 512-wide cache rows.
#include "mla_decode_kernel.h"

namespace mla {
template hipError_t launch_decode_d<512, true>(const SplitKVParams&, bool, hipStream_t);
}  // namespace mla
