// Interface between the host code (mla_api.cpp) and the kernels of the steps
// around decode: MLA prepare (before) and the merge fused with the w_vc
// up-projection (after).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Arguments of the MLA prepare kernels (device pointers).
struct PrepareArgs {
  int T;                        // new tokens
  int H;                        // heads
  int max_pos;                  // rows of cos_sin
  int kv;                       // pool format (mla_kv_dtype: 0 BF16, 1 FP8, 2 FP4, 3 MXFP8)
  int64_t num_slots;
  const uint16_t* q_nope;       // bf16 bits [T, H, 128]
  const uint16_t* q_rope_in;    // bf16 bits [T, H, 64]
  const uint16_t* w_kc_t;       // bf16 bits [H, 512, 128]
  const uint16_t* c_kv_new;     // bf16 bits [T, 512]
  const uint16_t* k_rope_new;   // bf16 bits [T, 64]
  const int32_t* positions;     // [T]
  const float* cos_sin;         // [max_pos, 64]
  const int32_t* slots;         // [T]
  uint16_t* q_nope_absorbed;    // bf16 bits [T, H, 512]
  uint16_t* q_rope_out;         // bf16 bits [T, H, 64]
  void* pool;                   // [num_slots, 576] bf16 bits or e4m3fn codes; FP4 / MXFP8 rows
  float* kv_scale;              // [num_slots] (FP8)
};

hipError_t launch_prepare(const PrepareArgs& args, hipStream_t stream);

// LSE merge of [P, T, H, 512] fp32 parts fused with the w_vc up-projection:
// out bf16 [T, H, 128], lse fp32 [T, H] (may be null).
hipError_t launch_combine_project(const float* part_o, const float* part_lse, int nparts, int T,
                                  int H, const uint16_t* w_vc_t, uint16_t* out, float* lse,
                                  hipStream_t stream);

}  // namespace mla
