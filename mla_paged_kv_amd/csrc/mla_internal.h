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
