// Kernel launchers for the host-only sanitizer build: the driver only makes
// calls that argument validation rejects, so reaching any of these is a bug
// (a call that should have been rejected went on to launch).
#include <cstdio>
#include <cstdlib>

#include "mla_kernels.h"

namespace {
[[noreturn]] void reached(const char* what) {
  std::fprintf(stderr, "sanitizer build: %s reached after validation\n", what);
  std::abort();
}
}  // namespace

namespace mla {
template <int D_QK, bool F16>
hipError_t launch_decode_d(const SplitKVParams&, bool, hipStream_t) {
  reached("launch_decode_d");
}
template hipError_t launch_decode_d<576, false>(const SplitKVParams&, bool, hipStream_t);
template hipError_t launch_decode_d<576, true>(const SplitKVParams&, bool, hipStream_t);
template hipError_t launch_decode_d<512, false>(const SplitKVParams&, bool, hipStream_t);
template hipError_t launch_decode_d<512, true>(const SplitKVParams&, bool, hipStream_t);
hipError_t launch_pairs(const SplitKVParams&, int, bool, bool, bool, hipStream_t) {
  reached("launch_pairs");
}
hipError_t launch_narrow(const SplitKVParams&, int, bool, bool, bool, hipStream_t) {
  reached("launch_narrow");
}
hipError_t launch_combine(const CombineParams&, hipStream_t) { reached("launch_combine"); }
}  // namespace mla

extern "C" const char* hipGetErrorString(hipError_t) { reached("hipGetErrorString"); }
