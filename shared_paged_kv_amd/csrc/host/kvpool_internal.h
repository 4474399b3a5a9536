// Internal helpers shared by the host control plane and the HIP entry points.
#pragma once
#include <cstdint>

#include "kvpool.h"

namespace kvp {

// Most query rows one VALU work item carries (rows = consumers x q heads per kv head).
constexpr int32_t kMaxRowsValu = 16;

// Row classes, one kernel instantiation each: 16, 8, 4, 2, 1 rows.
inline int row_class(int rows) { return rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : rows <= 8 ? 8 : 16; }
inline int row_class_index(int rows) { return rows <= 1 ? 4 : rows <= 2 ? 3 : rows <= 4 ? 2 : rows <= 8 ? 1 : 0; }

int fail(int code, const char* msg);
int check_shape(const kvp_shape* s);
int64_t block_head_bytes(const kvp_shape* s, int32_t ntok);

}  // namespace kvp
