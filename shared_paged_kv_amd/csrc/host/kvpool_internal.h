// Internal helpers shared by the host control plane and the HIP entry points.
#pragma once
#include <cstdint>

#include "kvpool.h"

namespace kvp {

// Most query rows one narrow work item carries (rows = consumers x q heads per
// kv head): its 4 waves split the item's tiles and each carries every row.
constexpr int32_t kMaxRowsValu = 16;
// Most query rows one wide (matrix-core) item carries: its 4 waves share every
// tile through LDS and each owns 16 rows.
constexpr int32_t kMaxRowsWide = 64;

// Row classes: wide (> 16), 16, 8, 4, 2, 1 rows.
constexpr int kRowClasses = 6;
inline int row_class(int rows) {
  return rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : rows <= 8 ? 8 : rows <= 16 ? 16 : 64;
}
inline int row_class_index(int rows) {
  return rows <= 1 ? 5 : rows <= 2 ? 4 : rows <= 4 ? 3 : rows <= 8 ? 2 : rows <= 16 ? 1 : 0;
}

int fail(int code, const char* msg);
int check_shape(const kvp_shape* s);
int64_t block_head_bytes(const kvp_shape* s, int32_t ntok);

}  // namespace kvp
