// The step after absorbed decode: the LSE merge of per-shard (or per-piece)
// partial results fused with the w_vc up-projection (page "Kimi K3 decode:
// DP16 vs DP2 x DCP8": kv_b_proj is absorbed into w_kc / w_vc, so w_vc is
// applied after attention; section "MLA": the shards' (O, LSE) are merged by
// dcp_lse_combine).  The merged 512-wide latent O of a row goes from
// registers to LDS as bf16 and straight into the projection, so it is never
// stored:
//
//   O[t, h]      = sum_j w_j O_j[t, h] / sum_j w_j,  w_j = exp(LSE_j - max_j LSE_j)
//   out[t, h, :] = O[t, h, :] . w_vc[h]     (512 -> 128, bf16 MFMAs, fp32 sums)
//
// One 256-thread block per (head, 32 tokens), at most 128 VGPRs per lane so
// that four waves per SIMD keep enough part loads in flight (64-token blocks
// need twice the LDS and measured slower).  Merge: wave w merges rows w,
// w + 4, ..., lane l holding features 4 l .. + 4 and 256 + 4 l .. + 4, with
// the loads of 8 parts in flight together.
// Projection: wave w computes columns 32 w .. + 32 of the block's 32 x 128
// result; v_mfma_f32_32x32x16_bf16 with A = the merged rows (LDS) and B =
// rows of w_vc_t (k contiguous).  The result leaves through LDS as whole
// 256-byte rows.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels_step.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kAStride = 520;   // LDS row stride of the merged rows, in bf16 (512 + 8)
constexpr int kOStride = 136;   // LDS row stride of the result tile, in bf16 (128 + 8)
constexpr int kPartsPerStep = 8;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__global__ __launch_bounds__(256, 4) void combine_project_kernel(const float* part_o,
                                                              const float* part_lse, int nparts,
                                                              int T, int H,
                                                              const uint16_t* w_vc_t,
                                                              uint16_t* out, float* lse_out) {
  __shared__ __attribute__((aligned(16))) uint16_t at[32 * kAStride];
  const int h = blockIdx.x % H;
  const int t0 = (blockIdx.x / H) * 32;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int j = lane & 31, kh = lane >> 5;
  const int64_t rows = (int64_t)T * H;

  // ---- merge 8 rows per wave into LDS (bf16)
  for (int rr = w; rr < 32; rr += 4) {
    const int t = t0 + rr;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    float inv = 0.f;
    if (t < T) {
      const int64_t row = (int64_t)t * H + h;
      float m = -INFINITY;
      for (int p = lane; p < nparts; p += 64) m = fmaxf(m, part_lse[p * rows + row]);
      m = wave_max(m);
      float wsum = 0.f;
      if (m != -INFINITY) {
        for (int p0 = 0; p0 < nparts; p0 += kPartsPerStep) {
          f32x4 v0[kPartsPerStep], v1[kPartsPerStep];
          float wj[kPartsPerStep];
#pragma unroll
          for (int k = 0; k < kPartsPerStep; ++k) {
            const int p = p0 + k;
            if (p < nparts) {
              const f32x4* src = reinterpret_cast<const f32x4*>(part_o + (p * rows + row) * 512);
              v0[k] = src[lane];
              v1[k] = src[64 + lane];
              const float lj = part_lse[p * rows + row];
              wj[k] = lj == -INFINITY ? 0.f : __expf(lj - m);
            } else {
              v0[k] = v1[k] = f32x4{0.f, 0.f, 0.f, 0.f};
              wj[k] = 0.f;
            }
          }
#pragma unroll
          for (int k = 0; k < kPartsPerStep; ++k) {
            const bool use = wj[k] > 0.f;  // an empty part's O is never read as a weight
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              acc0[c] += use ? wj[k] * v0[k][c] : 0.f;
              acc1[c] += use ? wj[k] * v1[k][c] : 0.f;
            }
            wsum += wj[k];
          }
        }
        inv = 1.0f / wsum;
      }
      if (lane == 0 && lse_out) lse_out[row] = m == -INFINITY ? -INFINITY : m + __logf(wsum);
    }
    *reinterpret_cast<bf16x4*>(at + rr * kAStride + 4 * lane) = __builtin_convertvector(acc0 * inv, bf16x4);
    *reinterpret_cast<bf16x4*>(at + rr * kAStride + 256 + 4 * lane) =
        __builtin_convertvector(acc1 * inv, bf16x4);
  }
  __syncthreads();

  // ---- projection: D[token][column] over k = 0 .. 511, with the B operand
  // of k-step ks = w_vc_t[h][32 w + j][16 ks + 8 kh .. + 8] loaded 8 k-steps
  // at a time (the weights are loaded after the merge, so that the merge runs
  // with the registers free for its loads).
  const bf16x8* wrow =
      reinterpret_cast<const bf16x8*>(w_vc_t + ((int64_t)h * 128 + 32 * w + j) * 512 + 8 * kh);
  f32x16 acc = {};
#pragma unroll
  for (int k8 = 0; k8 < 4; ++k8) {
    bf16x8 bop[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) bop[ks] = wrow[2 * (8 * k8 + ks)];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 aop =
          *reinterpret_cast<const bf16x8*>(at + j * kAStride + 16 * (8 * k8 + ks) + 8 * kh);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop[ks], acc, 0, 0, 0);
    }
  }
  __syncthreads();  // every wave is done reading the merged rows
  uint16_t* os = at;  // [32][kOStride] result tile, reusing the LDS
#pragma unroll
  for (int r = 0; r < 16; ++r)
    os[(8 * (r >> 2) + 4 * kh + (r & 3)) * kOStride + 32 * w + j] =
        __builtin_bit_cast(uint16_t, (__bf16)acc[r]);
  __syncthreads();
  // Thread i writes token row i / 8, columns 16 (i % 8) .. + 16.
  const int lr = tid >> 3, lc = 16 * (tid & 7);
  const int t = t0 + lr;
  if (t < T) {
    const uint4* src = reinterpret_cast<const uint4*>(os + lr * kOStride + lc);
    uint4* dst = reinterpret_cast<uint4*>(out + ((int64_t)t * H + h) * 128 + lc);
    dst[0] = src[0];
    dst[1] = src[1];
  }
}

}  // namespace

hipError_t launch_combine_project(const float* part_o, const float* part_lse, int nparts, int T,
                                  int H, const uint16_t* w_vc_t, uint16_t* out, float* lse,
                                  hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int64_t grid = (int64_t)H * ((T + 31) / 32);
  if (grid > (int64_t)INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_project_kernel, dim3((unsigned)grid), dim3(256), 0, stream, part_o,
                     part_lse, nparts, T, H, w_vc_t, out, lse);
  return hipGetLastError();
}

}  // namespace mla
