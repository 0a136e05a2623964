// MLA prepare: the step before absorbed decode, on the T new query tokens of
// a decode step (page "Kimi K3 decode: DP16 vs DP2 x DCP8": kv_b_proj is
// absorbed into w_kc / w_vc, w_kc is 96 x 128 x 512 in bf16, and the step is
// the mla_prepare of section "MLA").
//
// Absorption       q_nope_absorbed[t, h, :] = q_nope[t, h, :] . w_kc[h]
//                   (128 -> 512 per head) on bf16 MFMAs, fp32 accumulation,
//                   rounded to bf16.  HBM-bound: every head's 128 KB of
//                   weights is read once.
// RoPE and append  RoPE of every head's q_rope and of the new tokens'
//                   k_rope (interleaved pairs, caller-given cos / sin), then
//                   the append of the rows [c_kv | roped k_rope] to the pool
//                   at the given slots: BF16 bits, e4m3fn codes with the
//                   per-token scale amax / 448, or FP4 rows (e2m1 codes with
//                   a power-of-two scale per 16 elements; page "resident
//                   VRAM accounting", sections "KV ledger" and "cell_size"),
//                   or MXFP8 rows (e4m3fn codes with a power-of-two scale
//                   per 32 elements; same page, "cell_size").
//
// Every float32 step that decides a stored bit (the roped values, the scale,
// the quotients) is a correctly rounded IEEE operation with no contraction,
// so that the stored bytes are reproducible on the host.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels_step.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) {
  return __builtin_bit_cast(float, u & 0xffff0000u);
}
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return bf16_bits(a) | (bf16_bits(b) << 16);
}

// One interleaved RoPE pair (x0, x1) -> (x0 c - x1 s, x0 s + x1 c), every
// product and sum rounded on its own (no fused multiply-add).
__device__ __forceinline__ uint32_t rope_pair(uint32_t xx, float c, float s) {
#pragma clang fp contract(off)
  const float x0 = bf16_lo(xx), x1 = bf16_hi(xx);
  const float y0 = x0 * c - x1 * s;
  const float y1 = x0 * s + x1 * c;
  return pack_bf16(y0, y1);
}

// Block (head h, column quarter qb, token group): wave w computes columns
// n0 = 128 qb + 32 w .. + 32, 32 tokens per MFMA block.
// v_mfma_f32_32x32x16_bf16: lane l holds A[row l % 32][k 8 (l / 32) .. + 8]
// (a token's q_nope) and B[k 8 (l / 32) .. + 8][column l % 32] (a row of
// w_kc_t, k contiguous, kept in registers); accumulator r holds D[row
// 8 (r / 4) + 4 (l / 32) + r % 4][column l % 32].
// The 32 q_nope rows of a block (256 B each) are loaded once per block by
// all 256 threads with row-contiguous 16-byte loads (issued one block ahead)
// and shared through LDS; the block's 32 x 128 result goes back through LDS
// and out as whole 256-byte row segments.
constexpr int kQStride = 136;   // LDS row stride of a q block, in bf16 (128 + 8 pad)
constexpr int kOStride = 136;   // LDS row stride of a result tile, in bf16 (128 + 8 pad)

__device__ __forceinline__ void q_absorb_block(const uint16_t* q_nope, const uint16_t* w_kc_t,
                                               uint16_t* out, int T, int H, int blk, int tb,
                                               int te, uint16_t* qs, uint16_t* os) {
  const int h = blk >> 2, qb = blk & 3;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int j = lane & 31, kh = lane >> 5;
  const int n0 = 128 * qb + 32 * w;
  bf16x8 bop[8];
  {
    const bf16x8* wrow =
        reinterpret_cast<const bf16x8*>(w_kc_t + ((int64_t)h * 512 + n0 + j) * 128 + 8 * kh);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) bop[ks] = wrow[2 * ks];
  }
  // Cooperative q load: thread i takes row i / 8, bytes 32 (i % 8) .. + 32.
  const int lr = tid >> 3, lc = 16 * (tid & 7);  // row, first bf16 column
  auto gload = [&](int t0, uint4& x0, uint4& x1) {
    const int t = t0 + lr;
    if (t < te) {
      const uint4* src = reinterpret_cast<const uint4*>(q_nope + ((int64_t)t * H + h) * 128 + lc);
      x0 = src[0];
      x1 = src[1];
    } else {
      x0 = x1 = uint4{0u, 0u, 0u, 0u};
    }
  };
  uint4 x0, x1;
  gload(tb, x0, x1);
  for (int t0 = tb; t0 < te; t0 += 32) {
    __syncthreads();  // the previous block's LDS reads are done
    *reinterpret_cast<uint4*>(qs + lr * kQStride + lc) = x0;
    *reinterpret_cast<uint4*>(qs + lr * kQStride + lc + 8) = x1;
    __syncthreads();
    if (t0 + 32 < te) gload(t0 + 32, x0, x1);
    bf16x8 aop[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      aop[ks] = *reinterpret_cast<const bf16x8*>(qs + j * kQStride + 16 * ks + 8 * kh);
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[ks], bop[ks], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      os[(8 * (r >> 2) + 4 * kh + (r & 3)) * kOStride + 32 * w + j] = (uint16_t)bf16_bits(acc[r]);
    __syncthreads();
    // Thread i writes row i / 8, columns 16 (i % 8) .. + 16 of the tile.
    const int t = t0 + lr;
    if (t < te) {
      const uint4* src = reinterpret_cast<const uint4*>(os + lr * kOStride + lc);
      uint4* dst = reinterpret_cast<uint4*>(out + ((int64_t)t * H + h) * 512 + 128 * qb + lc);
      dst[0] = src[0];
      dst[1] = src[1];
    }
  }
}

__device__ __forceinline__ float block_max_256(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// e4m3fn code of a float32 already inside [-448, 448], nearest-even.
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// FP4 row of one token: thread i holds elements 2 i, 2 i + 1 of c_kv (c0,
// c1) and threads 0..31 also elements 512 + 2 i, + 1 of the roped k_rope (r0,
// r1).  Block k (16 elements) lies in threads 8 k .. 8 k + 7 (c_kv blocks 0..31;
// k_rope blocks 32..35 in threads 8 (k - 32) ..), so its largest magnitude
// is a reduction over 8 neighbouring lanes.  Its exponent e is the smallest
// with amax <= 6 * 2^e: with amax = f 2^E (0.5 <= f < 1), e = E - 3 if f <=
// 0.75, else E - 2; clamped to [-64, 64] (amax below 2^-100 takes -64, which
// is what the rule gives there).  Codes: e2m1 nearest to x 2^-e, ties to the
// even code, found by exact comparisons with the midpoints of the grid.
__device__ __forceinline__ int fp4_block_exponent(float amax) {
  if (!(amax >= 0x1p-100f)) return -64;
  const float f = __builtin_amdgcn_frexp_mantf(amax);
  const int E = __builtin_amdgcn_frexp_expf(amax);
  const int e = f <= 0.75f ? E - 3 : E - 2;
  return e > 64 ? 64 : (e < -64 ? -64 : e);
}

__device__ __forceinline__ uint32_t e2m1_code(float x, int e) {
  const float y = __builtin_amdgcn_ldexpf(x, -e);   // exact (power-of-two scaling)
  const float a = fabsf(y);
  const uint32_t m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                     (a >= 3.5f) + (a > 5.0f);
  return m | ((__builtin_bit_cast(uint32_t, y) >> 28) & 0x8u);
}

__device__ __forceinline__ float max8(float v) {
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Four bytes of lanes i .. i + 3 (gathered by lane i) and of lanes i, i + 8,
// i + 16, i + 24.
__device__ __forceinline__ uint32_t gather4(uint32_t b, int stride) {
  return b | (__shfl_down(b, stride) << 8) | (__shfl_down(b, 2 * stride) << 16) |
         (__shfl_down(b, 3 * stride) << 24);
}

__device__ __forceinline__ void append_fp4(uint8_t* row, int tid, float c0, float c1, float r0,
                                           float r1) {
  const int ec = fp4_block_exponent(max8(fmaxf(fabsf(c0), fabsf(c1))));
  const uint32_t bc = e2m1_code(c0, ec) | (e2m1_code(c1, ec) << 4);
  // The k_rope reduction runs in all of wave 0 (lanes 32..63 hold zeros).
  const int er = fp4_block_exponent(max8(fmaxf(fabsf(r0), fabsf(r1))));
  const uint32_t br = e2m1_code(r0, er) | (e2m1_code(r1, er) << 4);
  uint32_t* row32 = reinterpret_cast<uint32_t*>(row);
  const uint32_t codes = gather4(bc, 1);
  const uint32_t scales = gather4((uint32_t)(ec + 127), 8);
  const uint32_t rcodes = gather4(br, 1);
  const uint32_t rscales = gather4((uint32_t)(er + 127), 8);
  if ((tid & 3) == 0) row32[tid >> 2] = codes;                    // bytes 0..255
  if ((tid & 31) == 0) row32[72 + (tid >> 5)] = scales;          // bytes 288..319
  if (tid < 32) {
    if ((tid & 3) == 0) row32[64 + (tid >> 2)] = rcodes;          // bytes 256..287
    if (tid == 0) row32[80] = rscales;                            // bytes 320..323
  } else if (tid < 35) {
    row32[81 + (tid - 32)] = 0u;                                  // padding 324..335
  }
}

// MXFP8 row of one token: thread i holds elements 2 i, 2 i + 1 of c_kv and
// threads 0..31 also elements 512 + 2 i, + 1 of the roped k_rope.  Block k
// (32 elements) lies in threads 16 k .. 16 k + 15 (c_kv blocks 0..15;
// k_rope blocks 16, 17 in threads 0..15 and 16..31).  Its exponent e is the
// smallest with amax <= 448 * 2^e: with amax = f 2^E (0.5 <= f < 1) and 448 =
// 0.875 * 2^9, e = E - 9 if f <= 0.875, else E - 8; clamped to [-64, 64]
// (amax below 2^-100 takes -64).  Codes: e4m3fn nearest to x 2^-e (exact),
// ties to even, clamped to +-448.
__device__ __forceinline__ int mx_block_exponent(float amax) {
  if (!(amax >= 0x1p-100f)) return -64;
  const float f = __builtin_amdgcn_frexp_mantf(amax);
  const int E = __builtin_amdgcn_frexp_expf(amax);
  const int e = f <= 0.875f ? E - 9 : E - 8;
  return e > 64 ? 64 : (e < -64 ? -64 : e);
}

__device__ __forceinline__ float max16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ uint32_t mx_pair(float a, float b, int e) {
  const float ya = fminf(fmaxf(__builtin_amdgcn_ldexpf(a, -e), -448.0f), 448.0f);
  const float yb = fminf(fmaxf(__builtin_amdgcn_ldexpf(b, -e), -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ya, yb, 0, false) & 0xffffu;
}

__device__ __forceinline__ void append_mx(uint8_t* row, int tid, float c0, float c1, float r0,
                                          float r1) {
  const int ec = mx_block_exponent(max16(fmaxf(fabsf(c0), fabsf(c1))));
  const int er = mx_block_exponent(max16(fmaxf(fabsf(r0), fabsf(r1))));  // wave 0 lanes 0..31
  uint16_t* row16 = reinterpret_cast<uint16_t*>(row);
  uint32_t* row32 = reinterpret_cast<uint32_t*>(row);
  row16[tid] = (uint16_t)mx_pair(c0, c1, ec);                      // bytes 0..511
  const uint32_t scales = gather4((uint32_t)(ec + 127), 16);
  const uint32_t rscales = (uint32_t)(er + 127) | ((uint32_t)__shfl_down(er + 127, 16) << 8);
  if ((tid & 63) == 0) row32[144 + (tid >> 6)] = scales;           // bytes 576..591
  if (tid < 32) {
    row16[256 + tid] = (uint16_t)mx_pair(r0, r1, er);               // bytes 512..575
    if (tid == 0) row16[296] = (uint16_t)rscales;                   // bytes 592, 593
  } else if (tid == 32) {
    row16[297] = 0;                                                  // padding 594..595
  } else if (tid < 36) {
    row32[149 + (tid - 33)] = 0u;                                    // padding 596..607
  }
}

// One block per new token.  Threads 0..255 rotate the token's q_rope pairs
// (H x 32 of them), then thread i takes c_kv elements 2 i, 2 i + 1 and
// threads 0..31 the k_rope pair i of the row to append.
__device__ __forceinline__ void rope_append_block(const PrepareArgs& a, int t, float* red) {
  const int tid = threadIdx.x;
  const int64_t slot = a.slots[t];
  int pos = a.positions[t];
  pos = pos < 0 ? 0 : (pos >= a.max_pos ? a.max_pos - 1 : pos);
  const float* cs = a.cos_sin + (int64_t)pos * 64;
  // Pair p of the token uses frequency p % 32; a thread's pairs are tid +
  // 256 k, so all of them use frequency tid % 32.
  const float c = cs[tid & 31], s = cs[32 + (tid & 31)];

  const uint32_t* qin = reinterpret_cast<const uint32_t*>(a.q_rope_in + (int64_t)t * a.H * 64);
  uint32_t* qout = reinterpret_cast<uint32_t*>(a.q_rope_out + (int64_t)t * a.H * 64);
  const int npairs = a.H * 32;
#pragma unroll 4
  for (int p = tid; p < npairs; p += 256) qout[p] = rope_pair(qin[p], c, s);

  if (slot < 0 || slot >= a.num_slots) return;  // uniform in the block
  const uint32_t ckv = reinterpret_cast<const uint32_t*>(a.c_kv_new + (int64_t)t * 512)[tid];
  uint32_t kr = 0;
  if (tid < 32) {
    const uint32_t kin = reinterpret_cast<const uint32_t*>(a.k_rope_new + (int64_t)t * 64)[tid];
    kr = rope_pair(kin, c, s);
  }
  if (a.kv == 2 || a.kv == 3) {
    const float r0 = tid < 32 ? bf16_lo(kr) : 0.f, r1 = tid < 32 ? bf16_hi(kr) : 0.f;
    if (a.kv == 2) {
      append_fp4(static_cast<uint8_t*>(a.pool) + slot * 336, tid, bf16_lo(ckv), bf16_hi(ckv),
                 r0, r1);
    } else {
      append_mx(static_cast<uint8_t*>(a.pool) + slot * 608, tid, bf16_lo(ckv), bf16_hi(ckv),
                r0, r1);
    }
    return;
  }
  if (a.kv == 0) {
    uint32_t* row = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.pool) + slot * 576);
    row[tid] = ckv;
    if (tid < 32) row[256 + tid] = kr;
    return;
  }
  const float c0 = bf16_lo(ckv), c1 = bf16_hi(ckv);
  const float r0 = bf16_lo(kr), r1 = bf16_hi(kr);
  float m = fmaxf(fabsf(c0), fabsf(c1));
  if (tid < 32) m = fmaxf(m, fmaxf(fabsf(r0), fabsf(r1)));
  const float amax = block_max_256(m, red);
  const float scale = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  auto quot = [&](float x) { return fminf(fmaxf(__fdiv_rn(x, scale), -448.0f), 448.0f); };
  uint16_t* row = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(a.pool) + slot * 576);
  row[tid] = (uint16_t)e4m3_pair(quot(c0), quot(c1));
  if (tid < 32) row[256 + tid] = (uint16_t)e4m3_pair(quot(r0), quot(r1));
  if (tid == 0) a.kv_scale[slot] = scale;
}

// One launch for the whole step.  Blocks 0 .. 4 H G - 1 run the absorption:
// block b takes (head, column quarter) b % 4 H and tokens [128 g, 128 g +
// 128) with g = b / 4 H, so that the G token groups of one weight slice run
// on one XCD (4 H is a multiple of 8 when H is even) and read it from L2.
// The next T blocks run the RoPE and append of one token each; the two parts
// are independent and run side by side.
constexpr int kAbsorbTokens = 128;

__global__ __launch_bounds__(256) void prepare_kernel(PrepareArgs a) {
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint16_t qs[32 * kQStride];
  __shared__ __attribute__((aligned(16))) uint16_t os[32 * kOStride];
  const int blk = blockIdx.x;
  const int nhq = 4 * a.H;
  const int nabs = nhq * ((a.T + kAbsorbTokens - 1) / kAbsorbTokens);
  if (blk < nabs) {
    const int g = blk / nhq;
    const int tb = g * kAbsorbTokens;
    const int te = tb + kAbsorbTokens < a.T ? tb + kAbsorbTokens : a.T;
    q_absorb_block(a.q_nope, a.w_kc_t, a.q_nope_absorbed, a.T, a.H, blk - g * nhq, tb, te,
                   qs, os);
  } else {
    rope_append_block(a, blk - nabs, red);
  }
}

}  // namespace

hipError_t launch_prepare(const PrepareArgs& args, hipStream_t stream) {
  if (args.T <= 0) return hipSuccess;
  const int64_t grid =
      4 * (int64_t)args.H * ((args.T + kAbsorbTokens - 1) / kAbsorbTokens) + args.T;
  if (grid > (int64_t)INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prepare_kernel, dim3((unsigned)grid), dim3(256), 0, stream, args);
  return hipGetLastError();
}

}  // namespace mla
