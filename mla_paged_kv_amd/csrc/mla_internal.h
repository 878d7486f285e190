// Internal declarations shared by the host files of libmla.so.
#pragma once

#include <cstddef>
#include <cstdint>

#include "mla.h"

namespace mla {

constexpr int32_t kHeaderInts = 16;

// Records a formatted message for mla_last_error() and returns `code`.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Query rows per workgroup for units of `rows` query rows: 128 when rows > 64
// (the decode kernel), else 64 (the pair kernel).  A part spans
// ceil(rows / rows_per_group(rows)) workgroups.
inline int32_t rows_per_group(int32_t rows) { return rows > 64 ? 128 : 64; }

// Stages of a decode call (bit mask).  kStageValidateOnly runs every argument
// check except the workspace's and enqueues nothing.
enum { kStageSplit = 1, kStageCombine = 2, kStageValidateOnly = 4 };

// Dense paged decode behind the mla_decode_paged* entry points: argument
// checks, then the stages asked for on `stream`.
int decode_paged_impl(const void* q, const void* kvcache, const int32_t* block_table,
                      const int32_t* cache_seqlens, int32_t batch, int32_t s_q, int32_t h_q,
                      int32_t h_kv, int32_t d_qk, int32_t dv, int32_t num_blocks,
                      int32_t page_block_size, int32_t bt_stride, int32_t causal,
                      float softmax_scale, const int32_t* meta_dev, const mla_sched_info* info,
                      void* workspace, size_t workspace_bytes, void* out, float* lse,
                      void* stream, int stages, bool fp8, bool f16);

int32_t default_num_parts(int32_t rows, int32_t num_cus);
size_t metadata_capacity(int32_t num_units, int32_t target_parts);

// Work units, query rows per unit and part count of a scheduler call, after
// the argument checks shared by the host and device schedulers.  Returns
// MLA_OK, MLA_W_ACTIVE_FALLBACK (all heads are scheduled) or an error code
// (with the message set).
struct SchedShape {
  int32_t units, rows, parts;
};
int resolve_sched_shape(int32_t batch, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t topk,
                        int32_t active_h_q, int32_t num_cus, int32_t num_parts, SchedShape* out);

// Limits of the device scheduler (its whole state lives in one workgroup's LDS).
constexpr int32_t kSchedDevMaxUnits = 4096;
constexpr int32_t kSchedDevMaxParts = 1024;

}  // namespace mla
