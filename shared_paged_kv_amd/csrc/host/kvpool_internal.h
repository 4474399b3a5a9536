// Internal helpers shared by the host control plane and the HIP entry points.
#pragma once
#include <cstdint>
#include <vector>

#include "kvpool.h"

namespace kvp {

// Most query rows one narrow work item carries (rows = consumers x q heads per
// kv head): its 4 waves split the item's tiles and each carries every row.
constexpr int32_t kMaxRowsValu = 16;
// Most query rows one wide (matrix-core) item carries: its 4 waves share every
// tile through LDS and each owns 16 or 32 rows; at most 64 consumers (two mask
// words per block).
constexpr int32_t kMaxRowsWide = 128;
constexpr int32_t kMaxConsWide = 64;
// Most blocks one wide item reads (its block table is staged in LDS).
constexpr int32_t kMaxBlocksWide = 256;

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

// Rebuilds t's work plan (items, consumers, masks, combine lists) from its
// block tables; t's plan vectors must be empty.
void build_plan(const kvp_shape* sh, kvp_tables* t);

// Checks every index the device kernels take from t's tables and work plan
// against the extent of the array it indexes (physical ids against n_phys,
// consumer and mask ranges, partial rows against n_part_rows, the combine
// lists, valid-token counts against the block size).  KVP_OK, or KVP_EINVAL
// naming the first violation.  Run on every plan before it is handed out.
int check_plan_bounds(const kvp_shape* sh, const kvp_tables* t);

}  // namespace kvp

// Block tables of a round (opaque in the C ABI).
struct kvp_tables {
  int32_t n_agents = 0, max_blocks = 0, n_phys = 0, n_dedup = 0, n_delta = 0;
  std::vector<int32_t> n_blocks, block_table, delta_table, ntok, dst_pos0, shift;
  std::vector<int32_t> src_pos0, refcount, phys_ntok, phys_agent, phys_block;
  // plan
  std::vector<kvp_item> items;
  std::vector<int32_t> plan_blocks, cons, qcons, comb_ptr, comb_rows;
  std::vector<int32_t> plan_ntok, cons_row;  // derived: see kvp_tables_view
  std::vector<float> rope_cs;                // derived: see kvp_tables_view
  std::vector<uint32_t> mask;
  int32_t n_part_rows = 0;
  int32_t n_qcons_shifted = 0;
  int32_t class_items[kvp::kRowClasses] = {0, 0, 0, 0, 0, 0};
  int32_t unit_span = 1;
  int64_t unique_kv_bytes = 0;
};
