// Streaming kernels that measure the HBM ceiling of the GPU they run on
// (libmla_probe.so; bench.py --hbm-peak times them).  Not part of the decode
// path: they only give the decode kernels' byte rates a measured reference.
//
// read: every lane loads 16-byte pieces of the buffer, eight in flight, and
// folds them into a running xor; one dword per workgroup is written, so the
// traffic is the buffer read once (plus one dword per lane written, at a
// lane-dependent address: a vector store).  copy: the same pieces stored to a second
// buffer.  Both take 16-byte aligned buffers whose size is a multiple of 16;
// the grid is 8 workgroups of 256 threads per compute unit.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kUnroll = 8;

__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, int64_t n,
                                                   uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) acc ^= v[k];
  }
  for (; i < n; i += stride) acc ^= src[i];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) __builtin_nontemporal_store(v[k], dst + i + k * stride);
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

int grid_for(int num_cus) { return 8 * (num_cus > 0 ? num_cus : 256); }

}  // namespace

extern "C" {

// Reads `bytes` of src; sink needs 2048 * num_cus dwords.  0 on success.
int mla_probe_read(const void* src, int64_t bytes, void* sink, int num_cus, void* stream) {
  if (!src || !sink || bytes <= 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15))
    return -1;
  hipLaunchKernelGGL(read_kernel, dim3(grid_for(num_cus)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), bytes / 16,
                     static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Copies `bytes` from src to dst (no overlap).  0 on success.
int mla_probe_copy(const void* src, void* dst, int64_t bytes, int num_cus, void* stream) {
  if (!src || !dst || bytes <= 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15) ||
      (reinterpret_cast<uintptr_t>(dst) & 15))
    return -1;
  hipLaunchKernelGGL(copy_kernel, dim3(grid_for(num_cus)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
