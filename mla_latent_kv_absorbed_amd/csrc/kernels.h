// Interface between the host code (mla_api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct SplitReq;  // plan_layout.h

// Element type of the KV pool (the values of mla_kv_dtype).
enum KvKind : int { kKvBf16 = 0, kKvFp8 = 1, kKvFp4 = 2, kKvMx = 3 };

// Arguments of the decode kernel (device pointers unless noted).
struct DecodeArgs {
  const uint8_t* plan;       // device copy of the plan blob
  const uint16_t* q_nope;    // bf16 bits [B, M, 512]
  const uint16_t* q_rope;    // bf16 bits [B, M, 64]
  const uint8_t* pool;       // [num_slots, 576] bf16 or e4m3fn elements; FP4 / MXFP8 rows
  const float* kv_scale;     // [num_slots] (FP8)
  int64_t num_slots;
  const int32_t* table;      // [B, stride]
  int64_t table_stride;
  const int32_t* seq_lens;   // [B] global lengths
  float c2;                  // softmax_scale * log2(e)
  float* out;                // [B, M, 512]
  float* lse;                // [B, M]
  uint16_t* ws_o;            // [parts, M, 512] fp16 bits of O_part / ws_sc (split partials)
  float* ws_lse;             // [parts, M]
  float* ws_sc;              // [parts, M] power-of-two factor of each partial row
};

hipError_t launch_decode(int kv, bool paged, int grid, const DecodeArgs& args,
                         hipStream_t stream);
// split_dev: the plan's split-request records in device memory; max_parts:
// the largest part count among them.
hipError_t launch_merge_split(const SplitReq* split_dev, int num_split_reqs, int rows,
                              int max_parts, const uint16_t* ws_o, const float* ws_lse,
                              const float* ws_sc, float* out, float* lse, hipStream_t stream);
// Device address of the current device's no-alloc scratch array (capacity
// kNoAllocScratchBytes), looked up once per device with hipGetSymbolAddress.
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_lse_combine(const float* part_o, const float* part_lse, int nparts,
                              int64_t rows, float* out, float* lse, hipStream_t stream);

}  // namespace mla
