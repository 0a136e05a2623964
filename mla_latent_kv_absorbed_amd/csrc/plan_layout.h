// Byte layout of the decode plan blob.  The host planner writes it; the
// decode and merge kernels read the identical bytes from device memory.
#pragma once

#include <stdint.h>

namespace mla {

constexpr uint32_t kPlanMagic = 0x504C414Du;  // "MALP"
constexpr uint32_t kPlanVersion = 3;

constexpr int kLatent = 512;    // kv_lora_rank: width of c_kv and of the output
constexpr int kRope = 64;       // qk_rope_head_dim
constexpr int kRow = 576;       // elements per cached token
constexpr int kRowsPerWave = 32;
constexpr int kWavesPerWG = 4;
constexpr int kRowsPerWG = kRowsPerWave * kWavesPerWG;  // 128 query rows per workgroup
constexpr int kTile = 32;       // tokens per KV tile
constexpr int kMaxQLen = 8;

struct PlanHeader {
  uint32_t magic;
  uint32_t version;
  int32_t batch;
  int32_t q_len;
  int32_t num_heads;
  int32_t rows;          // M = q_len * num_heads
  int32_t row_groups;    // G = ceil(M / kRowsPerWG)
  int32_t num_wgs;       // grid of the decode kernel
  int32_t num_units;
  int32_t num_parts;     // partial (O, LSE) slots in the workspace
  int32_t num_split_reqs;
  int32_t kv_dtype;
  int32_t dcp_size;
  int32_t dcp_rank;
  int32_t off_wg;        // int32 wg_begin[num_wgs + 1]
  int32_t off_units;     // Unit units[num_units]
  int32_t off_reqs;      // ReqParts reqs[batch]
  int32_t off_split;     // SplitReq split_reqs[num_split_reqs]
  int32_t max_local;     // largest local length (table columns read)
  int32_t page_size;
  int64_t plan_bytes;
  int64_t workspace_bytes;
  int64_t ws_lse_offset;  // byte offset of the partial LSE array in the workspace
  int64_t ws_sc_offset;   // byte offset of the partial rows' power-of-two factors
};
static_assert(sizeof(PlanHeader) == 112, "plan header layout");

// One work unit: row group g of request b over local token range [j0, j1).
// part < 0: the unit covers the request's whole range, write the output;
// else: write partial slot `part` of the workspace.
struct Unit {
  int32_t b;
  int32_t g;
  int32_t j0;
  int32_t j1;
  int32_t part;
  int32_t pad[3];
};
static_assert(sizeof(Unit) == 32, "unit layout");

struct ReqParts {
  int32_t first_part;
  int32_t num_parts;  // 1: written directly by the decode kernel
};

// A request whose partials the merge combines, with its slots, so that a
// merge wave finds everything it needs in one 16-byte load.
struct SplitReq {
  int32_t b;
  int32_t first_part;
  int32_t num_parts;
  int32_t pad;
};
static_assert(sizeof(SplitReq) == 16, "split request layout");

inline int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

}  // namespace mla
