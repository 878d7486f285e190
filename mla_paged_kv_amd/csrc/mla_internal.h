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

int32_t default_num_parts(int32_t rows, int32_t num_cus);
size_t metadata_capacity(int32_t num_units, int32_t target_parts);

}  // namespace mla
