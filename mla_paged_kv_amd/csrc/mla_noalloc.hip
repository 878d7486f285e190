// mla_decode_paged_noalloc: dense paged decode whose split partials live in a
// library-owned static device array instead of a caller workspace, for
// callers that cannot allocate device memory.
//
// The array `scratch` is a file-scope __device__ variable: every GPU that runs
// this library holds its own copy, at its own address, until the process
// ends.  In host code its name only stands in for the device symbol, so host
// code never passes it to a kernel; the device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and kept in
// g_scratch_ptr, and only that pointer is handed to the kernels.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "mla.h"
#include "mla_internal.h"

namespace mla {
namespace {

static __device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (nullptr on error, with
// the message set).
void* device_scratch() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error(MLA_E_HIP, "decode_paged_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_error(MLA_E_HIP, "decode_paged_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      set_error(MLA_E_HIP, "decode_paged_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace mla

extern "C" int mla_decode_paged_noalloc(
    const void* q, const void* kvcache, const int32_t* block_table, const int32_t* cache_seqlens,
    int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t dv,
    int32_t num_blocks, int32_t page_block_size, int32_t bt_stride, int32_t causal,
    float softmax_scale, const int32_t* meta_dev, const mla_sched_info* info, void* out,
    float* lse, void* stream) {
  using namespace mla;
  // every argument check of mla_decode_paged first (nothing is enqueued)
  int rc = decode_paged_impl(q, kvcache, block_table, cache_seqlens, batch, s_q, h_q, h_kv, d_qk,
                             dv, num_blocks, page_block_size, bt_stride, causal, softmax_scale,
                             meta_dev, info, nullptr, 0, out, lse, stream, kStageValidateOnly,
                             false, false);
  if (rc < 0 || batch == 0) return rc;
  const size_t need = mla_workspace_bytes(info, dv);
  if (need > size_t(MLA_NOALLOC_SCRATCH_BYTES))
    return set_error(MLA_E_NOSPC,
                     "decode_paged_noalloc: the schedule needs %zu bytes of split partials, more "
                     "than the %zu-byte static scratch; build the metadata with fewer parts",
                     need, size_t(MLA_NOALLOC_SCRATCH_BYTES));
  void* ws = device_scratch();
  if (ws == nullptr) return MLA_E_HIP;
  const int rc2 = decode_paged_impl(q, kvcache, block_table, cache_seqlens, batch, s_q, h_q, h_kv,
                                    d_qk, dv, num_blocks, page_block_size, bt_stride, causal,
                                    softmax_scale, meta_dev, info, ws, MLA_NOALLOC_SCRATCH_BYTES,
                                    out, lse, stream, kStageSplit | kStageCombine, false, false);
  return rc2;
}
