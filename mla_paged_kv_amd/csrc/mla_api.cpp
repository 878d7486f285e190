// C-ABI entry points of libmla.so: argument checks, workspace carving and
// kernel launches for dense paged and top-k sparse MLA decode.  Every check
// runs before anything is enqueued, so a rejected call touches no memory.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "mla.h"
#include "mla_internal.h"
#include "mla_kernels.h"

namespace mla {

namespace {

thread_local char g_last_error[512] = "";

constexpr int32_t kPage = 64;
constexpr int32_t kDV = 512;

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Checks shared by the dense and sparse entry points.
int check_common(const void* q, const void* kvcache, int32_t batch, int32_t s_q, int32_t h_q,
                 int32_t h_kv, int32_t d_qk, int32_t dv, int32_t num_blocks,
                 int32_t page_block_size, const int32_t* meta_dev, const mla_sched_info* info,
                 void* workspace, size_t workspace_bytes, void* out, float* lse, bool fp8,
                 bool check_workspace) {
  if (batch < 0 || s_q < 1 || h_q < 1 || h_kv < 1 || d_qk < 1 || dv < 1 || num_blocks < 0 ||
      page_block_size < 1)
    return set_error(MLA_E_INVAL, "decode: negative or zero shape");
  if (h_kv != 1) return set_error(MLA_E_NOTSUP, "decode: h_kv=%d (only 1 is built)", h_kv);
  if (page_block_size != kPage)
    return set_error(MLA_E_NOTSUP, "decode: page_block_size=%d (only 64)", page_block_size);
  if (d_qk != 576 && d_qk != 512) return set_error(MLA_E_NOTSUP, "decode: d_qk=%d", d_qk);
  if (fp8 && d_qk != 576)
    return set_error(MLA_E_NOTSUP, "decode: the FP8 cache format needs d_qk=576, got %d", d_qk);
  if (dv > d_qk) return set_error(MLA_E_INVAL, "decode: dv=%d > d_qk=%d", dv, d_qk);
  if (dv != kDV) return set_error(MLA_E_NOTSUP, "decode: dv=%d (only 512)", dv);
  if (info == nullptr) return set_error(MLA_E_INVAL, "decode: null info");
  if (int64_t(num_blocks) * kPage > INT32_MAX)
    return set_error(MLA_E_INVAL, "decode: num_blocks=%d too large", num_blocks);
  if (info->num_parts < 0 || info->row_blocks < 1 || info->rows < 1 || info->total_slots < 0 ||
      info->num_split_units < 0 || info->total_ints < kHeaderInts)
    return set_error(MLA_E_INVAL, "decode: malformed metadata header");
  {
    const int32_t rbk = rows_per_group(info->rows);
    if (info->row_blocks != (info->rows + rbk - 1) / rbk)
      return set_error(MLA_E_INVAL, "decode: metadata row_blocks inconsistent");
  }
  if (batch == 0) return MLA_OK;
  if (!q || !kvcache || !meta_dev || !out || !lse)
    return set_error(MLA_E_INVAL, "decode: null q/kvcache/meta/out/lse");
  if (!aligned(q, 16) || !aligned(kvcache, 16) || !aligned(out, 16) || !aligned(lse, 4))
    return set_error(MLA_E_INVAL, "decode: q/kvcache/out need 16-byte, lse 4-byte alignment");
  if (num_blocks < 1) return set_error(MLA_E_INVAL, "decode: empty kvcache");
  const size_t need = mla_workspace_bytes(info, dv);
  if (need > 0 && check_workspace) {
    if (!workspace) return set_error(MLA_E_INVAL, "decode: metadata has splits, workspace is null");
    if (!aligned(workspace, 256)) return set_error(MLA_E_INVAL, "decode: workspace not 256-aligned");
    if (workspace_bytes < need)
      return set_error(MLA_E_NOSPC, "decode: workspace %zu bytes < %zu needed", workspace_bytes, need);
  }
  (void)s_q;
  (void)h_q;
  return MLA_OK;
}

}  // namespace

hipError_t launch_decode(const SplitKVParams& p, int d_qk, bool sparse, bool f16, hipStream_t st) {
  if (d_qk == 576) return f16 ? launch_decode_d<576, true>(p, sparse, st) : launch_decode_d<576, false>(p, sparse, st);
  return f16 ? launch_decode_d<512, true>(p, sparse, st) : launch_decode_d<512, false>(p, sparse, st);
}

namespace {

// Workspace: fp32 partial outputs [slots, rows, dv], then (256-byte aligned)
// partial base-2 LSEs [slots, rows], then partial row maxima [slots, rows].
void carve_workspace(const mla_sched_info* info, void* workspace, int32_t dv, float** ws_o,
                     float** ws_lse, float** ws_max) {
  const size_t o_bytes = size_t(info->total_slots) * info->rows * dv * sizeof(float);
  const size_t l_bytes = size_t(info->total_slots) * info->rows * sizeof(float);
  char* w = static_cast<char*>(workspace);
  *ws_o = static_cast<float*>(workspace);
  *ws_lse = w ? reinterpret_cast<float*>(w + align256(o_bytes)) : nullptr;
  *ws_max = w ? reinterpret_cast<float*>(w + align256(o_bytes) + align256(l_bytes)) : nullptr;
}

int launch_combine_stage(const int32_t* meta_dev, const mla_sched_info* info, int32_t s_q,
                         int32_t h_q, int32_t heads, bool sparse, void* workspace, int32_t dv,
                         void* out, float* lse, float* max_logits, bool lse_base2, bool f16,
                         hipStream_t st) {
  if (info->num_split_units <= 0) return MLA_OK;
  CombineParams cp;
  float* ws_o;
  float* ws_lse;
  float* ws_max;
  carve_workspace(info, workspace, dv, &ws_o, &ws_lse, &ws_max);
  cp.meta = meta_dev;
  cp.ws_o = ws_o;
  cp.ws_lse = ws_lse;
  cp.ws_max = ws_max;
  cp.out = static_cast<uint16_t*>(out);
  cp.lse = lse;
  cp.max_logits = max_logits;
  cp.lse_base2 = lse_base2 ? 1 : 0;
  cp.out_f16 = f16 ? 1 : 0;
  cp.off_split_list = info->off_split_list;
  cp.num_split_units = info->num_split_units;
  cp.max_splits = info->max_splits;
  if (info->off_split_list < 0) {
    // device-built metadata: the host knows bounds only; pick the combine
    // layout from the mean number of parts per unit
    const int32_t units = info->num_units > 0 ? info->num_units : 1;
    cp.max_splits = (info->num_parts + units - 1) / units + 1;
  }
  cp.rows = info->rows;
  cp.s_q = s_q;
  cp.h_q = h_q;
  cp.heads = heads;
  cp.sparse = sparse ? 1 : 0;
  const hipError_t e = launch_combine(cp, st);
  if (e != hipSuccess) return set_error(MLA_E_HIP, "combine launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

int launch(SplitKVParams& kp, const mla_sched_info* info, int32_t d_qk, bool sparse, bool fp8,
           bool f16, void* workspace, int32_t dv, void* stream, int stages) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  carve_workspace(info, workspace, dv, &kp.ws_o, &kp.ws_lse, &kp.ws_max);
  kp.num_parts = info->num_parts;
  kp.row_blocks = info->row_blocks;
  kp.rows = info->rows;
  if (stages & kStageSplit) {
    // units of more than 64 rows: the decode kernel (each wavefront owns 32
    // rows and all 512 output columns, 128 rows per workgroup); otherwise, and
    // for the FP8 cache, the pair kernel.  The decode kernel reads the block
    // table (dense) or the index lists (sparse) through one buffer resource
    // with 32-bit byte offsets below 2^31; a larger table goes to the pair
    // kernel, which addresses it with 64-bit pointers.
    // Units of at most 16 rows (e.g. 16 active heads, one query token) go to
    // the narrow kernel, one 16-row MFMA block per workgroup (bf16, fp16 and
    // FP8 caches), when their sparse pool is addressable with 32-bit byte
    // offsets.
    const int64_t table_ints = int64_t(info->num_units) * (sparse ? kp.topk : kp.bt_stride);
    const bool table_fits = table_ints <= int64_t(INT32_MAX / 4);
    const uint64_t row_bytes = fp8 ? uint64_t(kFp8RowBytes) : uint64_t(d_qk) * 2;
    const bool pool32 = !sparse || (uint64_t(kp.num_rows) + 2) * row_bytes <= 0xFFFFFFFFull;
    hipError_t e;
    if (kp.rows <= 16 && pool32)
      e = launch_narrow(kp, d_qk, sparse, fp8, f16, st);
    else if (fp8 || kp.rows <= 64 || !table_fits)
      e = launch_pairs(kp, d_qk, sparse, fp8, f16, st);
    else
      e = launch_decode(kp, d_qk, sparse, f16, st);
    if (e != hipSuccess) return set_error(MLA_E_HIP, "splitkv launch: %s", hipGetErrorString(e));
  }
  if (stages & kStageCombine)
    return launch_combine_stage(kp.meta, info, kp.s_q, kp.h_q, kp.heads, sparse, workspace, dv,
                                kp.out, kp.lse, kp.max_logits, kp.lse_base2 != 0, f16, st);
  return MLA_OK;
}

}  // namespace

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_last_error[0] = '\0'; }

}  // namespace mla

extern "C" {

int32_t mla_version(void) { return 0x00010000; }

const char* mla_strerror(int code) {
  switch (code) {
    case MLA_OK: return "MLA_OK";
    case MLA_W_ACTIVE_FALLBACK: return "MLA_W_ACTIVE_FALLBACK";
    case MLA_E_INVAL: return "MLA_E_INVAL";
    case MLA_E_NOTSUP: return "MLA_E_NOTSUP";
    case MLA_E_NOSPC: return "MLA_E_NOSPC";
    case MLA_E_HIP: return "MLA_E_HIP";
    default: return "MLA_E_UNKNOWN";
  }
}

const char* mla_last_error(void) { return mla::g_last_error; }

size_t mla_workspace_bytes(const mla_sched_info* info, int32_t d_v) {
  if (info == nullptr || info->total_slots <= 0 || info->rows <= 0 || d_v <= 0) return 0;
  const size_t o = size_t(info->total_slots) * info->rows * d_v * sizeof(float);
  const size_t l = size_t(info->total_slots) * info->rows * sizeof(float);
  return mla::align256(o) + 2 * mla::align256(l);
}

}  // extern "C"

namespace mla {

int decode_paged_impl(const void* q, const void* kvcache, const int32_t* block_table,
                      const int32_t* cache_seqlens, int32_t batch, int32_t s_q, int32_t h_q,
                      int32_t h_kv, int32_t d_qk, int32_t dv, int32_t num_blocks,
                      int32_t page_block_size, int32_t bt_stride, int32_t causal,
                      float softmax_scale, const int32_t* meta_dev, const mla_sched_info* info,
                      void* workspace, size_t workspace_bytes, void* out, float* lse,
                      void* stream, int stages, bool fp8, bool f16) {
  clear_error();
  int rc = check_common(q, kvcache, batch, s_q, h_q, h_kv, d_qk, dv, num_blocks, page_block_size,
                        meta_dev, info, workspace, workspace_bytes, out, lse, fp8,
                        !(stages & kStageValidateOnly));
  if (rc != MLA_OK || batch == 0) return rc;
  if (!block_table || !cache_seqlens) return set_error(MLA_E_INVAL, "decode_paged: null block_table/seqlens");
  if (bt_stride < 1) return set_error(MLA_E_INVAL, "decode_paged: bt_stride=%d", bt_stride);
  if (causal != 0 && causal != 1) return set_error(MLA_E_INVAL, "decode_paged: causal=%d", causal);
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return set_error(MLA_E_INVAL, "decode_paged: softmax_scale must be positive and finite");
  if (info->num_units != batch)
    return set_error(MLA_E_INVAL, "decode_paged: metadata built for %d units, batch=%d (dense mode?)",
                     info->num_units, batch);
  if (info->rows % s_q != 0)
    return set_error(MLA_E_INVAL, "decode_paged: metadata rows %d not a multiple of s_q=%d", info->rows, s_q);
  const int32_t heads = info->rows / s_q;
  if (heads < 1 || heads > h_q)
    return set_error(MLA_E_INVAL, "decode_paged: metadata heads %d outside [1, h_q=%d]", heads, h_q);

  SplitKVParams kp{};
  kp.q = static_cast<const uint16_t*>(q);
  kp.kv = static_cast<const uint16_t*>(kvcache);
  kp.block_table = block_table;
  kp.seqlens = cache_seqlens;
  kp.indices = nullptr;
  kp.meta = meta_dev;
  kp.out = static_cast<uint16_t*>(out);
  kp.lse = lse;
  kp.s_q = s_q;
  kp.h_q = h_q;
  kp.heads = heads;
  kp.bt_stride = bt_stride;
  kp.num_rows = num_blocks * kPage;
  kp.topk = 0;
  kp.causal = causal;
  kp.scale_log2 = softmax_scale * 1.4426950408889634f;
  if (stages & kStageValidateOnly) return MLA_OK;
  return launch(kp, info, d_qk, false, fp8, f16, workspace, dv, stream, stages);
}

int decode_sparse_impl(const void* q, const void* kvcache, const int32_t* indices,
                       int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk,
                       int32_t dv, int32_t num_blocks, int32_t page_block_size, int32_t topk,
                       float softmax_scale, const int32_t* meta_dev,
                       const mla_sched_info* info, void* workspace, size_t workspace_bytes,
                       void* out, float* lse, void* stream, int stages, bool fp8, bool f16) {
  clear_error();
  int rc = check_common(q, kvcache, batch, s_q, h_q, h_kv, d_qk, dv, num_blocks, page_block_size,
                        meta_dev, info, workspace, workspace_bytes, out, lse, fp8, true);
  if (rc != MLA_OK || batch == 0) return rc;
  if (!indices) return set_error(MLA_E_INVAL, "decode_sparse: null indices");
  if (topk < 1) return set_error(MLA_E_INVAL, "decode_sparse: topk=%d", topk);
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return set_error(MLA_E_INVAL, "decode_sparse: softmax_scale must be positive and finite");
  if (int64_t(info->num_units) != int64_t(batch) * s_q)
    return set_error(MLA_E_INVAL, "decode_sparse: metadata built for %d units, batch*s_q=%lld (sparse mode?)",
                     info->num_units, (long long)batch * s_q);
  const int32_t heads = info->rows;
  if (heads < 1 || heads > h_q)
    return set_error(MLA_E_INVAL, "decode_sparse: metadata heads %d outside [1, h_q=%d]", heads, h_q);

  SplitKVParams kp{};
  kp.q = static_cast<const uint16_t*>(q);
  kp.kv = static_cast<const uint16_t*>(kvcache);
  kp.block_table = nullptr;
  kp.seqlens = nullptr;
  kp.indices = indices;
  kp.meta = meta_dev;
  kp.out = static_cast<uint16_t*>(out);
  kp.lse = lse;
  kp.s_q = s_q;
  kp.h_q = h_q;
  kp.heads = heads;
  kp.bt_stride = 0;
  kp.num_rows = num_blocks * kPage;
  kp.topk = topk;
  kp.causal = 0;
  kp.scale_log2 = softmax_scale * 1.4426950408889634f;
  return launch(kp, info, d_qk, true, fp8, f16, workspace, dv, stream, stages);
}

int sparse_prefill_impl(const void* q, const void* kv, const int32_t* indices, int32_t s_q,
                        int32_t s_kv, int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t dv,
                        int32_t topk, float sm_scale, const int32_t* meta_dev,
                        const mla_sched_info* info, void* workspace, size_t workspace_bytes,
                        void* out, float* max_logits, float* lse, void* stream, bool f16) {
  clear_error();
  if (s_kv < 1) return set_error(MLA_E_INVAL, "sparse_prefill: s_kv=%d", s_kv);
  // the shared checks see the KV rows as ceil(s_kv / 64) pages of 64
  const int64_t pages = (int64_t(s_kv) + kPage - 1) / kPage;
  int rc = check_common(q, kv, s_q, 1, h_q, h_kv, d_qk, dv, int32_t(pages), kPage, meta_dev, info,
                        workspace, workspace_bytes, out, lse, false, true);
  if (rc != MLA_OK || s_q == 0) return rc;
  if (!indices) return set_error(MLA_E_INVAL, "sparse_prefill: null indices");
  if (topk < 1) return set_error(MLA_E_INVAL, "sparse_prefill: topk=%d", topk);
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.f))
    return set_error(MLA_E_INVAL, "sparse_prefill: sm_scale must be positive and finite");
  if (max_logits && !aligned(max_logits, 4))
    return set_error(MLA_E_INVAL, "sparse_prefill: max_logits needs 4-byte alignment");
  if (info->num_units != s_q)
    return set_error(MLA_E_INVAL,
                     "sparse_prefill: metadata built for %d units, s_q=%d (build it in sparse mode "
                     "with batch = s_q and one query token each)",
                     info->num_units, s_q);
  const int32_t heads = info->rows;
  if (heads < 1 || heads > h_q)
    return set_error(MLA_E_INVAL, "sparse_prefill: metadata heads %d outside [1, h_q=%d]", heads, h_q);

  SplitKVParams kp{};
  kp.q = static_cast<const uint16_t*>(q);
  kp.kv = static_cast<const uint16_t*>(kv);
  kp.indices = indices;
  kp.meta = meta_dev;
  kp.out = static_cast<uint16_t*>(out);
  kp.lse = lse;
  kp.max_logits = max_logits;
  kp.lse_base2 = 1;
  kp.s_q = 1;  // every query token is a unit of its own
  kp.h_q = h_q;
  kp.heads = heads;
  kp.num_rows = s_kv;  // an index is valid iff 0 <= idx < s_kv
  kp.topk = topk;
  kp.scale_log2 = sm_scale * 1.4426950408889634f;
  return launch(kp, info, d_qk, true, false, f16, workspace, dv, stream, kStageSplit | kStageCombine);
}

}  // namespace mla

extern "C" {

int mla_sparse_prefill(const void* q, const void* kv, const int32_t* indices, int32_t s_q,
                       int32_t s_kv, int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t dv,
                       int32_t topk, float sm_scale, const int32_t* meta_dev,
                       const mla_sched_info* info, void* workspace, size_t workspace_bytes,
                       void* out, float* max_logits, float* lse, void* stream) {
  return mla::sparse_prefill_impl(q, kv, indices, s_q, s_kv, h_q, h_kv, d_qk, dv, topk, sm_scale,
                                  meta_dev, info, workspace, workspace_bytes, out, max_logits, lse,
                                  stream, false);
}

int mla_sparse_prefill_f16(const void* q, const void* kv, const int32_t* indices, int32_t s_q,
                           int32_t s_kv, int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t dv,
                           int32_t topk, float sm_scale, const int32_t* meta_dev,
                           const mla_sched_info* info, void* workspace, size_t workspace_bytes,
                           void* out, float* max_logits, float* lse, void* stream) {
  return mla::sparse_prefill_impl(q, kv, indices, s_q, s_kv, h_q, h_kv, d_qk, dv, topk, sm_scale,
                                  meta_dev, info, workspace, workspace_bytes, out, max_logits, lse,
                                  stream, true);
}

#define MLA_PAGED_ARGS                                                                          \
  const void *q, const void *kvcache, const int32_t *block_table, const int32_t *cache_seqlens, \
      int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t dv,          \
      int32_t num_blocks, int32_t page_block_size, int32_t bt_stride, int32_t causal,           \
      float softmax_scale, const int32_t *meta_dev, const mla_sched_info *info,                 \
      void *workspace, size_t workspace_bytes, void *out, float *lse, void *stream
#define MLA_PAGED_PASS                                                                          \
  q, kvcache, block_table, cache_seqlens, batch, s_q, h_q, h_kv, d_qk, dv, num_blocks,          \
      page_block_size, bt_stride, causal, softmax_scale, meta_dev, info, workspace,             \
      workspace_bytes, out, lse, stream
#define MLA_SPARSE_ARGS                                                                         \
  const void *q, const void *kvcache, const int32_t *indices, int32_t batch, int32_t s_q,      \
      int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t dv, int32_t num_blocks,                  \
      int32_t page_block_size, int32_t topk, float softmax_scale, const int32_t *meta_dev,      \
      const mla_sched_info *info, void *workspace, size_t workspace_bytes, void *out,           \
      float *lse, void *stream
#define MLA_SPARSE_PASS                                                                         \
  q, kvcache, indices, batch, s_q, h_q, h_kv, d_qk, dv, num_blocks, page_block_size, topk,     \
      softmax_scale, meta_dev, info, workspace, workspace_bytes, out, lse, stream

int mla_decode_paged(MLA_PAGED_ARGS) {
  return mla::decode_paged_impl(MLA_PAGED_PASS, mla::kStageSplit | mla::kStageCombine, false, false);
}

int mla_splitkv_paged(MLA_PAGED_ARGS) {
  return mla::decode_paged_impl(MLA_PAGED_PASS, mla::kStageSplit, false, false);
}

int mla_decode_sparse(MLA_SPARSE_ARGS) {
  return mla::decode_sparse_impl(MLA_SPARSE_PASS, mla::kStageSplit | mla::kStageCombine, false, false);
}

int mla_splitkv_sparse(MLA_SPARSE_ARGS) {
  return mla::decode_sparse_impl(MLA_SPARSE_PASS, mla::kStageSplit, false, false);
}

int mla_decode_paged_fp8(MLA_PAGED_ARGS) {
  return mla::decode_paged_impl(MLA_PAGED_PASS, mla::kStageSplit | mla::kStageCombine, true, false);
}

int mla_splitkv_paged_fp8(MLA_PAGED_ARGS) {
  return mla::decode_paged_impl(MLA_PAGED_PASS, mla::kStageSplit, true, false);
}

int mla_decode_sparse_fp8(MLA_SPARSE_ARGS) {
  return mla::decode_sparse_impl(MLA_SPARSE_PASS, mla::kStageSplit | mla::kStageCombine, true, false);
}

int mla_splitkv_sparse_fp8(MLA_SPARSE_ARGS) {
  return mla::decode_sparse_impl(MLA_SPARSE_PASS, mla::kStageSplit, true, false);
}

int mla_decode_paged_f16(MLA_PAGED_ARGS) {
  return mla::decode_paged_impl(MLA_PAGED_PASS, mla::kStageSplit | mla::kStageCombine, false, true);
}

int mla_splitkv_paged_f16(MLA_PAGED_ARGS) {
  return mla::decode_paged_impl(MLA_PAGED_PASS, mla::kStageSplit, false, true);
}

int mla_decode_sparse_f16(MLA_SPARSE_ARGS) {
  return mla::decode_sparse_impl(MLA_SPARSE_PASS, mla::kStageSplit | mla::kStageCombine, false, true);
}

int mla_splitkv_sparse_f16(MLA_SPARSE_ARGS) {
  return mla::decode_sparse_impl(MLA_SPARSE_PASS, mla::kStageSplit, false, true);
}

static int combine_impl(const int32_t* meta_dev, const mla_sched_info* info, int32_t batch,
                        int32_t s_q, int32_t h_q, int32_t dv, int32_t sparse,
                        const void* workspace, size_t workspace_bytes, void* out, float* lse,
                        void* stream, int f16) {
  using namespace mla;
  clear_error();
  if (info == nullptr) return set_error(MLA_E_INVAL, "combine: null info");
  if (batch < 0 || s_q < 1 || h_q < 1) return set_error(MLA_E_INVAL, "combine: bad shape");
  if (dv != kDV) return set_error(MLA_E_NOTSUP, "combine: dv=%d (only 512)", dv);
  if (sparse != 0 && sparse != 1) return set_error(MLA_E_INVAL, "combine: sparse=%d", sparse);
  if (info->rows < 1 || info->total_slots < 0 || info->num_split_units < 0 ||
      info->total_ints < kHeaderInts)
    return set_error(MLA_E_INVAL, "combine: malformed metadata header");
  int32_t heads;
  if (sparse) {
    if (int64_t(info->num_units) != int64_t(batch) * s_q)
      return set_error(MLA_E_INVAL, "combine: metadata units %d != batch*s_q", info->num_units);
    heads = info->rows;
  } else {
    if (info->num_units != batch || info->rows % s_q != 0)
      return set_error(MLA_E_INVAL, "combine: metadata does not match batch/s_q");
    heads = info->rows / s_q;
  }
  if (heads > h_q) return set_error(MLA_E_INVAL, "combine: metadata heads %d > h_q=%d", heads, h_q);
  if (info->num_split_units == 0 || batch == 0) return MLA_OK;
  if (!meta_dev || !out || !lse || !workspace)
    return set_error(MLA_E_INVAL, "combine: null meta/out/lse/workspace");
  if (!aligned(out, 16) || !aligned(lse, 4) || !aligned(workspace, 256))
    return set_error(MLA_E_INVAL, "combine: misaligned out/lse/workspace");
  if (workspace_bytes < mla_workspace_bytes(info, dv))
    return set_error(MLA_E_NOSPC, "combine: workspace too small");
  return launch_combine_stage(meta_dev, info, s_q, h_q, heads, sparse != 0,
                              const_cast<void*>(workspace), dv, out, lse, nullptr, false, f16 != 0,
                              static_cast<hipStream_t>(stream));
}

int mla_combine(const int32_t* meta_dev, const mla_sched_info* info, int32_t batch, int32_t s_q,
                int32_t h_q, int32_t dv, int32_t sparse, const void* workspace,
                size_t workspace_bytes, void* out, float* lse, void* stream) {
  return combine_impl(meta_dev, info, batch, s_q, h_q, dv, sparse, workspace, workspace_bytes, out,
                      lse, stream, 0);
}

int mla_combine_f16(const int32_t* meta_dev, const mla_sched_info* info, int32_t batch,
                    int32_t s_q, int32_t h_q, int32_t dv, int32_t sparse, const void* workspace,
                    size_t workspace_bytes, void* out, float* lse, void* stream) {
  return combine_impl(meta_dev, info, batch, s_q, h_q, dv, sparse, workspace, workspace_bytes, out,
                      lse, stream, 1);
}

}  // extern "C"
