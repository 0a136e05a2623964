// Absorbed MLA decode and LSE merge kernels for gfx950 (MI355X).
//
// Decode (page "Kimi K3 decode: DP16 vs DP2 x DCP8", section "MLA": all
// query heads of a request score against one shared latent KV head).
// One workgroup = 4 waves = 128 query rows of one request (a row group);
// wave w owns rows [32w, 32w + 32).  The workgroup streams the request's KV
// in tiles of 32 tokens through double-buffered LDS:
//
//   S^T[32 tok x 32 rows] = K[32 x 576] . Q^T       36 x mfma 32x32x16 bf16
//   online softmax in the log2 domain, lazily rescaled
//   O^T[512 x 32 rows]   += V^T[512 x 32] . P^T     32 x mfma 32x32x16 bf16
//
// Computing S transposed puts each row's 16 scores of a tile in one lane
// (and its other 16 in lane ^ 32), which is exactly the B operand layout the
// P.V product needs, so P never leaves registers, the row max needs one
// cross-lane exchange, and V^T comes from token-major LDS through the
// transposing ds_read_b64_tr_b16.  Q (144 VGPRs) stays in registers for the
// whole unit and O (256 values) accumulates in the MFMA accumulators.
//
// KV tiles arrive by direct global->LDS DMA (global_load_lds_dwordx4) two
// (BF16) or three (FP8) tiles ahead.  FP8 tiles stay e4m3fn codes in LDS:
// every MFMA operand is read as codes and widened to BF16 in registers
// (exact: every e4m3fn value is a BF16 value), which halves the LDS bytes per
// MFMA.  The per-token fp32 scale multiplies the score column and the
// probability, never the stored element, so K and V stay exact.
//
// BF16 tile layout: 16-byte chunk cc of token t at cc * 512 + 16 * (t ^ 4 *
// (cc & 3)); FP8: chunk c at c * 512 + 16 * (t ^ 16 (c & 1)).  Under these
// swizzles the K reads (one chunk of 32 tokens) and the transposing V reads
// are bank-conflict free, and every DMA lane keeps one token per tile.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "plan_layout.h"
#include "pv_asm.inc"
#include "qk_asm.inc"
#include "fp8_asm.inc"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))
// __shared__ objects are generic pointers in HIP C++; make the LDS address space explicit.
#define LDS_U8(p) ((LDS_AS uint8_t*)(p))
#define LDS_F32(p) ((LDS_AS float*)(p))

constexpr int kBlock = kTile * 16;          // one 16-byte chunk of all 32 tokens
constexpr int kChunksBf16 = kRow * 2 / 16;  // 72
constexpr int kChunksFp8 = kRow / 16;       // 36
constexpr int kTileBf16 = kChunksBf16 * kBlock;  // 36864 bytes
constexpr int kTileFp8 = kChunksFp8 * kBlock;    // 18432 bytes
constexpr int kKSteps = kRow / 16;          // 36 k-steps of the QK product
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyRescale = 8.0f;        // log2 units: p <= 2^8 before a rescale


__device__ __forceinline__ int swz_tok(int cc, int t) { return t ^ ((cc & 3) << 2); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt in [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ float wave_xor32_max(float v) {
  return fmaxf(v, __shfl_xor(v, 32));
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* p) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)p[i];
  return r;
}

// LDS map of the decode kernel (bytes).  BF16: three tiles of BF16 rows (the
// DMA runs two tiles ahead).  FP8: four tiles of e4m3fn rows (the DMA runs
// three tiles ahead) and the per-token scales of four tiles.  An FP8 tile
// keeps the 16-byte chunk c of token t at c * 512 + 16 * (t ^ 16 (c & 1)).
constexpr int kBf16Tiles = 3;
constexpr int kLdsBf16Total = kBf16Tiles * kTileBf16;
constexpr int kFp8Tiles = 4;
constexpr int kLdsScale = kFp8Tiles * kTileFp8;  // float[4][kTile], by tile & 3
constexpr int kLdsFp8Total = kLdsScale + 4 * kTile * 4;

// Workgroup barrier that drains this wave's LDS operations only.  Global->LDS
// DMA still in flight is deliberately not waited for (the callers wait for the
// tile they need with an explicit vmcnt), and the "memory" clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Issue the DMA of one KV tile: every lane of wave w moves chunks of one token
// whose pool row starts at `row` (already offset by the lane's first chunk).
// BF16: instruction k moves chunk 2 (w + 4 k) + hk of 32 tokens x 2 = 1 KB into
// tile bytes [1024 (w + 4 k), +1024).  FP8: the same over the 36 chunks of an
// FP8 row, into the staging buffer, plus the 32 per-token scales (wave 3).
template <bool kFp8>
__device__ __forceinline__ void issue_tile_dma(const uint8_t* row, const float* scale_src,
                                               LDS_AS uint8_t* dst, LDS_AS float* sc_dst, int w,
                                               int lane) {
  if constexpr (!kFp8) {
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      __builtin_amdgcn_global_load_lds((GLB_AS void*)(row + 128 * k),
                                       (LDS_AS void*)(dst + 1024 * (w + 4 * k)), 16, 0, 0);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      if (w + 4 * k < 18) {
        __builtin_amdgcn_global_load_lds((GLB_AS void*)(row + 128 * k),
                                         (LDS_AS void*)(dst + 1024 * (w + 4 * k)), 16, 0, 0);
      }
    }
    if (w == 3 && lane < 32) {
      __builtin_amdgcn_global_load_lds((GLB_AS void*)scale_src, (LDS_AS void*)sc_dst, 4, 0, 0);
    }
  }
}

// Wait until the DMA of an older tile has landed while `newer` later tiles'
// DMA (and, for general tables, `slots` vector slot loads) may stay in flight.
// vmcnt counts in issue order, so allowing exactly the instructions issued
// after the awaited tile is enough.  VMEM instructions per tile and wave:
// BF16 9; FP8 5, 5, 4, 4 rows + the scales on wave 3.
template <bool kFp8>
__device__ __forceinline__ void wait_dma(int w, int newer, int slots) {
  const int per = kFp8 ? (w == 2 ? 4 : 5) : 9;
  const int n = newer * per + slots;
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    case 15: wait_vmcnt<15>(); break;
    case 16: wait_vmcnt<16>(); break;
    case 17: wait_vmcnt<17>(); break;
    case 18: wait_vmcnt<18>(); break;
    case 19: wait_vmcnt<19>(); break;
    case 20: wait_vmcnt<20>(); break;
    case 21: wait_vmcnt<21>(); break;
    case 22: wait_vmcnt<22>(); break;
    case 23: wait_vmcnt<23>(); break;
    default: wait_vmcnt<0>(); break;  // never under-waits
  }
}

// The 16 per-token scales of the tokens whose scores this lane holds.
__device__ __forceinline__ void load_tile_scales(const LDS_AS float* sct, int hk, float* ksc) {
#pragma unroll
  for (int a4 = 0; a4 < 4; ++a4) {
    const f32x4 v = *(const LDS_AS f32x4*)(sct + 8 * a4 + 4 * hk);
#pragma unroll
    for (int c = 0; c < 4; ++c) ksc[4 * a4 + c] = v[c];
  }
}

// A copy of v the compiler cannot see through: values derived from it are
// recomputed where they are used instead of being kept live (or spilled).
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ int64_t clamp_slot(int64_t s, int64_t n) {
  return s < 0 ? 0 : (s >= n ? n - 1 : s);
}

// K operand of k-step ks from an FP8 tile: 8 codes of chunk ks (16 features),
// half hk, of this lane's token, widened to 8 BF16 (exact).
__device__ __forceinline__ bf16x8 k_operand_fp8(const LDS_AS uint8_t* p) {
  const u32x2 raw = *(const LDS_AS u32x2*)p;
  u32x4 o;
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, false));
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, true));
  o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, false));
  o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, true));
  return __builtin_bit_cast(bf16x8, o);
}

// S^T[32 tokens x 32 rows] = K . Q^T over the 576 features of one tile.
//
// The accumulators are pinned to VGPRs: the O accumulators take all 256
// AGPRs and Q takes 144 VGPRs, so this is the only assignment that fits the
// 512 registers of one wave per SIMD, and the compiler does not choose it by
// itself.  Even and odd k-steps go to two independent chains (s0, s1) so that
// consecutive MFMAs do not wait on each other.  K operands: BF16 tiles hold
// chunk cc = 2 ks + hk of token t at cc * 512 + 16 (t ^ 4 (cc & 3)); FP8 tiles
// hold chunk ks at ks * 512 + 16 (t ^ 16 (ks & 1)), half hk at +8.  `ke` /
// `ko` are the lane's offsets for even / odd k-steps.  Because the MFMAs are
// issued from inline asm, the hazards the compiler would otherwise cover are
// covered here: wait states before each group (operands may just have been
// written by VALU instructions) and after the last MFMA (its result is read
// by VALU instructions next).
template <bool kFp8>
__device__ __forceinline__ f32x16 qk_tile(const LDS_AS uint8_t* tile, int ke, int ko,
                                          const bf16x8* qf) {
  f32x16 s0, s1;
#pragma unroll
  for (int g = 0; g < kKSteps / 4; ++g) {
    const int ks = 4 * g;
    bf16x8 k0, k1, k2, k3;
    if constexpr (kFp8) {
      k0 = k_operand_fp8(tile + ke + 512 * (ks + 0));
      k1 = k_operand_fp8(tile + ko + 512 * (ks + 1));
      k2 = k_operand_fp8(tile + ke + 512 * (ks + 2));
      k3 = k_operand_fp8(tile + ko + 512 * (ks + 3));
    } else {
      k0 = *(const LDS_AS bf16x8*)(tile + ke + 1024 * (ks + 0));
      k1 = *(const LDS_AS bf16x8*)(tile + ko + 1024 * (ks + 1));
      k2 = *(const LDS_AS bf16x8*)(tile + ke + 1024 * (ks + 2));
      k3 = *(const LDS_AS bf16x8*)(tile + ko + 1024 * (ks + 3));
    }
    if (g == 0) {
      asm volatile(MLA_QK_GROUP_FIRST_ASM
                   : [s0] "=&v"(s0), [s1] "=&v"(s1)
                   : [k0] "v"(k0), [k1] "v"(k1), [k2] "v"(k2), [k3] "v"(k3),
                     [q0] "v"(qf[ks]), [q1] "v"(qf[ks + 1]), [q2] "v"(qf[ks + 2]),
                     [q3] "v"(qf[ks + 3]));
    } else {
      asm volatile(MLA_QK_GROUP_ASM
                   : [s0] "+v"(s0), [s1] "+v"(s1)
                   : [k0] "v"(k0), [k1] "v"(k1), [k2] "v"(k2), [k3] "v"(k3),
                     [q0] "v"(qf[ks]), [q1] "v"(qf[ks + 1]), [q2] "v"(qf[ks + 2]),
                     [q3] "v"(qf[ks + 3]));
    }
  }
  // Results consumed by VALU next: wait out the MFMA write latency.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s0), "+v"(s1));
  return s0 + s1;
}

// Wait out the MFMA write latency before the O accumulators are read by
// VALU instructions (rescale by the lazy max, or the epilogue).
__device__ __forceinline__ void acc_settle(f32x16 (&acc)[16]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]), "+a"(acc[4]),
                 "+a"(acc[5]), "+a"(acc[6]), "+a"(acc[7]), "+a"(acc[8]), "+a"(acc[9]),
                 "+a"(acc[10]), "+a"(acc[11]), "+a"(acc[12]), "+a"(acc[13]), "+a"(acc[14]),
                 "+a"(acc[15]));
}

#define CONST_AS __attribute__((address_space(4)))

// kPaged: req_to_token is paged with page_size a multiple of the 32-token
// tile, i.e. every aligned 32-position run maps to 32 consecutive slots.  The
// kernel then reads one table entry per tile, with a scalar load (counted by
// lgkmcnt), so no vector load is ever consumed while a tile's DMA is in
// flight.  Otherwise every lane loads its own token's slot (general tables;
// this serializes the DMA behind each slot load and is slower).
template <bool kFp8, bool kPaged>
__global__ __launch_bounds__(256, 1) void decode_kernel(const DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kFp8 ? kLdsFp8Total : kLdsBf16Total];
  LDS_AS uint8_t* lds = LDS_U8(smem);

  // The plan is read through the constant address space: scalar loads, and
  // every value derived from it is known to be wave-uniform.
  const CONST_AS uint8_t* plan = (const CONST_AS uint8_t*)a.plan;
  const CONST_AS PlanHeader* ph = (const CONST_AS PlanHeader*)plan;
  const CONST_AS int32_t* wg_begin = (const CONST_AS int32_t*)(plan + ph->off_wg);
  const CONST_AS Unit* units = (const CONST_AS Unit*)(plan + ph->off_units);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int n_lane = lane & 31;   // row within the wave / token within a tile
  const int hk = lane >> 5;       // k-half of MFMA operands
  const int M = ph->rows;
  const int H = ph->num_heads;
  const int qlen = ph->q_len;
  const int W = ph->dcp_size;
  const int R = ph->dcp_rank;
  constexpr int kAhead = kFp8 ? 3 : 2;  // how many tiles the DMA runs ahead
  const float tau_raw = kLazyRescale / a.c2;
  constexpr int kRowBytes = kFp8 ? kRow : 2 * kRow;

  // Lane-constant parts of the LDS operand addresses (see qk_tile for the
  // K operand).  BF16 V^T (ds_read_b64_tr_b16): in 16-lane group g16, lane
  // 4 krow + cpart addresses token 16 e + 8 x + 4 hk + krow, features
  // 32 db + 16 (g16 & 1) + 4 cpart.  FP8 V^T (ds_read_b64_tr_b8): lane
  // 2 k + c addresses row k = token 16 e + 8 (k / 4) + 4 kg + k % 4 (kg =
  // g16 / 2), byte half c of features 32 db + 16 (g16 & 1) .. +16.
  const int g16 = lane >> 4;
  int ke, ko, va_off, vb_off;
  if constexpr (!kFp8) {
    ke = 512 * hk + 16 * (n_lane ^ (4 * hk));
    ko = 512 * hk + 16 * (n_lane ^ (8 + 4 * hk));
    const int krow = (lane & 15) >> 2;
    const int cpart = lane & 3;
    const int c3 = 2 * (g16 & 1) + (cpart >> 1);  // (chunk index) & 3
    va_off = 512 * c3 + 16 * ((4 * hk + krow) ^ (4 * c3)) + 8 * (cpart & 1);
    vb_off = 512 * c3 + 16 * ((8 + 4 * hk + krow) ^ (4 * c3)) + 8 * (cpart & 1);
  } else {
    ke = 16 * n_lane + 8 * hk;
    ko = 16 * (n_lane ^ 16) + 8 * hk;
    const int fh = g16 & 1, kg = g16 >> 1, k8 = (lane & 15) >> 1, c = lane & 1;
    const int tok = 8 * (k8 >> 2) + 4 * kg + (k8 & 3);
    va_off = 512 * fh + 16 * (tok ^ (16 * fh)) + 8 * c;
    vb_off = 512 * fh + 16 * ((16 + tok) ^ (16 * fh)) + 8 * c;
  }
  // DMA: the token this lane moves (chunk parity decides the swizzle), and
  // its first chunk's byte offset in a row.
  const int dma_tok = kFp8 ? (n_lane ^ (16 * hk)) : (n_lane ^ (((2 * w + hk) & 3) << 2));
  const int dma_chunk_off = 16 * (2 * w + hk);

  const int u_begin = wg_begin[blockIdx.x];
  const int u_end = wg_begin[blockIdx.x + 1];

  for (int u = u_begin; u < u_end; ++u) {
    const int b = units[u].b;
    const int g = units[u].g;
    const int j0 = units[u].j0;
    const int j1 = units[u].j1;
    const int part = units[u].part;
    const int row = g * kRowsPerWG + w * kRowsPerWave + n_lane;  // this lane's query row
    const bool row_ok = row < M;

    // ---- Q^T operand: lane holds Q[row][16 ks + 8 hk .. +8] for every ks.
    bf16x8 qf[kKSteps];
    {
      const int64_t rbase = (int64_t)b * M + (row_ok ? row : 0);
      const u32x4* qn = reinterpret_cast<const u32x4*>(a.q_nope + rbase * kLatent);
      const u32x4* qr = reinterpret_cast<const u32x4*>(a.q_rope + rbase * kRope);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        u32x4 v = (ks < 32) ? qn[2 * ks + hk] : qr[2 * (ks - 32) + hk];
        if (!row_ok) v = u32x4{0u, 0u, 0u, 0u};
        qf[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }

    // Last visible local index of this row: p = j W + R <= L - q + i.
    int jmax = -1;
    {
      const int L = ((const CONST_AS int32_t*)a.seq_lens)[b];
      const int i_draft = row_ok ? row / H : 0;
      const int last_p = L - qlen + i_draft;
      if (last_p >= R) jmax = (last_p - R) / W;
      jmax = min(jmax, j1 - 1);
    }

    f32x16 acc_o[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) acc_o[d] = f32x16{};
    float m_ref = -INFINITY;  // running max of this lane's row, raw units (q.k [x scale])
    float l_part = 0.f;       // this lane's share of the row sum

    const int ntiles = (j1 - j0 + kTile - 1) / kTile;
    const int32_t* trow = a.table + (int64_t)b * a.table_stride;
    const CONST_AS int32_t* trow_s = (const CONST_AS int32_t*)trow;
    const int jlast = j1 - 1;
    // Raw table value that locates this lane's token in tile t (clamped into
    // the unit): the tile's first slot (paged) or the token's own slot.
    auto slot_raw = [&](int t) -> int32_t {
      t = t < ntiles ? t : ntiles - 1;
      const int jt = j0 + t * kTile;
      if constexpr (kPaged) return trow_s[jt];
      else return trow[min(jt + dma_tok, jlast)];
    };
    auto lane_slot = [&](int32_t raw, int t) -> int64_t {
      int64_t s = raw;
      if constexpr (kPaged) s += min(dma_tok, jlast - (j0 + t * kTile));
      return clamp_slot(s, a.num_slots);
    };

    if (ntiles > 0) {
      // BF16: the DMA runs kAhead = 2 tiles ahead into three tile buffers.
      // FP8: the DMA runs kAhead = 3 tiles ahead into four tile buffers.
      LDS_AS float* sc_lds = (LDS_AS float*)(lds + (kFp8 ? kLdsScale : 0));
      auto tile_at = [&](int t) -> LDS_AS uint8_t* {
        return kFp8 ? lds + (t & 3) * kTileFp8 : lds + (t % 3) * kTileBf16;
      };
      // Prologue: DMA of tiles 0 .. kAhead-1.
#pragma unroll
      for (int t = 0; t < kAhead; ++t) {
        if (t < ntiles) {
          const int64_t sl = lane_slot(slot_raw(t), t);
          issue_tile_dma<kFp8>(a.pool + sl * kRowBytes + dma_chunk_off, a.kv_scale + sl,
                               tile_at(t), sc_lds + kTile * (t & 3), w, lane);
        }
      }
      int32_t raw_pending = slot_raw(kAhead);  // locates tile it + kAhead

      for (int it = 0; it < ntiles; ++it) {
        // ---- prefetch: table entry of tile it+kAhead+1, DMA of tile it+kAhead.
        // A vector slot load (general tables) must be issued before the DMA:
        // the vmcnt arithmetic of wait_dma counts it there.
        const int32_t raw_later = slot_raw(it + kAhead + 1);
        asm volatile("" ::: "memory");
        if (it + kAhead < ntiles) {
          const int tn = it + kAhead;
          // DMA lane constants recomputed here rather than kept live.
          const int tid_o = opaque(tid), hk_o = (tid_o >> 5) & 1, w_o = tid_o >> 6;
          const int tok_o = kFp8 ? ((tid_o & 31) ^ (16 * hk_o))
                                 : ((tid_o & 31) ^ (((2 * w_o + hk_o) & 3) << 2));
          int64_t sl = raw_pending;
          if constexpr (kPaged) sl += min(tok_o, jlast - (j0 + tn * kTile));
          sl = clamp_slot(sl, a.num_slots);
          issue_tile_dma<kFp8>(a.pool + sl * kRowBytes + 16 * (2 * w_o + hk_o), a.kv_scale + sl,
                               tile_at(tn), sc_lds + kTile * (tn & 3), w, lane);
        }
        // Tile it must have landed; later tiles may stay in flight.
        wait_dma<kFp8>(w, min(ntiles - 1, it + kAhead) - it, kPaged ? 0 : kAhead);
        barrier_lds();

        const LDS_AS uint8_t* tile = tile_at(it);
        const int jt = j0 + it * kTile;

        // ---- S^T = K . Q^T
        f32x16 s = qk_tile<kFp8>(tile, ke, ko, qf);

        // ---- scores in raw units x = q.k (times the token scale for FP8),
        // mask, tile max.  acc index i holds token 8 (i / 4) + 4 hk + (i % 4).
        const LDS_AS float* sct = sc_lds + kTile * (it & 3);
        float ksc[16];
        if constexpr (kFp8) {
          load_tile_scales(sct, hk, ksc);
#pragma unroll
          for (int i = 0; i < 16; ++i) s[i] *= ksc[i];
        }
        const int lim = jmax - jt;  // tokens m <= lim are visible to this row
        if (__any(lim < kTile - 1)) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int m = 8 * (i >> 2) + 4 * hk + (i & 3);
            s[i] = (m <= lim) ? s[i] : -INFINITY;
          }
        }
        float mt = s[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mt = fmaxf(mt, s[i]);
        mt = wave_xor32_max(mt);

        // ---- lazy rescale: only when the max grows by more than 2^8 in the
        // exponent (tau_raw = 8 / c2 in raw units).
        const bool need = mt > m_ref + tau_raw;
        if (__any(need)) {
          const float m_new = need ? mt : m_ref;
          const float alpha = need ? __builtin_amdgcn_exp2f((m_ref - m_new) * a.c2) : 1.0f;
          m_ref = m_new;
          l_part *= alpha;
#pragma unroll
          for (int d = 0; d < 16; ++d) {
            // One block at a time through VGPRs and straight back to AGPRs;
            // left to itself the allocator gives all of O a VGPR home here.
            f32x16 t = acc_o[d];
            asm volatile("" : "+v"(t));
            t = t * alpha;
            asm volatile("" : "+a"(t));
            acc_o[d] = t;
          }
        }
        // p = 2^((x - m) c2); a row with nothing visible yet keeps p = 0.
        const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * a.c2;

        // ---- P (fp32 -> bf16), FP8 value scale folded in.
        if constexpr (kFp8) load_tile_scales(sct, hk, ksc);
        bf16x8 pb0, pb1;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], a.c2, -mc));
          l_part += e;
          const float pv = kFp8 ? e * ksc[i] : e;
          if (i < 8) pb0[i] = (__bf16)pv; else pb1[i - 8] = (__bf16)pv;
        }

        // ---- O^T += V^T . P^T.  For MFMA e, k-slot 8 hk + jj is token
        // 16 e + 8 (jj / 4) + 4 hk + jj % 4 (the layout of P above); the V^T
        // operands are read with transposing LDS loads inside one asm
        // statement (lane addresses va / vb: token half 0 / 1 for FP8, the two
        // 4-token runs for BF16).
        {
          const LDS_AS uint8_t* va = tile + va_off;
          const LDS_AS uint8_t* vb = tile + vb_off;
#define MLA_PV_OPERANDS                                                                   \
  : [a0] "+a"(acc_o[0]), [a1] "+a"(acc_o[1]), [a2] "+a"(acc_o[2]), [a3] "+a"(acc_o[3]),   \
    [a4] "+a"(acc_o[4]), [a5] "+a"(acc_o[5]), [a6] "+a"(acc_o[6]), [a7] "+a"(acc_o[7]),   \
    [a8] "+a"(acc_o[8]), [a9] "+a"(acc_o[9]), [a10] "+a"(acc_o[10]),                     \
    [a11] "+a"(acc_o[11]), [a12] "+a"(acc_o[12]), [a13] "+a"(acc_o[13]),                 \
    [a14] "+a"(acc_o[14]), [a15] "+a"(acc_o[15])                                          \
  : [va] "v"(va), [vb] "v"(vb), [p0] "v"(pb0), [p1] "v"(pb1)                             \
  : "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249",      \
    "v250", "v251", "v252", "v253", "v254", "v255", "memory"
          if constexpr (kFp8) {
            asm volatile(MLA_PV8_TILE_ASM MLA_PV_OPERANDS);
          } else {
            asm volatile(MLA_PV_TILE_ASM MLA_PV_OPERANDS);
          }
#undef MLA_PV_OPERANDS
        }

        raw_pending = raw_later;
        barrier_lds();
      }
    }

    // ---- epilogue: O = acc / l, LSE = ln 2 * (m + log2 l).
    acc_settle(acc_o);
    const float l_row = l_part + __shfl_xor(l_part, 32);
    const bool empty = !(l_row > 0.f);
    const float inv = empty ? 0.f : 1.0f / l_row;
    const float lse_v =
        empty ? -INFINITY : (m_ref * a.c2 + __builtin_amdgcn_logf(l_row)) * kLn2;
    if (row_ok) {
      float* obase;
      float* lbase;
      if (part < 0) {
        obase = a.out + ((int64_t)b * M + row) * kLatent;
        lbase = a.lse + (int64_t)b * M + row;
      } else {
        obase = a.ws_o + ((int64_t)part * M + row) * kLatent;
        lbase = a.ws_lse + (int64_t)part * M + row;
      }
#pragma unroll
      for (int db = 0; db < 16; ++db) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          f32x4 v;
#pragma unroll
          for (int c = 0; c < 4; ++c) v[c] = acc_o[db][4 * a4 + c] * inv;
          *reinterpret_cast<f32x4*>(obase + 32 * db + 8 * a4 + 4 * hk) = v;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (hk == 0) *lbase = lse_v;
    }
  }
}

// ---------------------------------------------------------------- LSE merge

// One wave per output row: lane handles 8 of the 512 features.
__device__ __forceinline__ void merge_row(const float* part_o, const float* part_lse,
                                          int64_t part_stride_rows, int nparts, float* out,
                                          float* lse_out, int lane) {
  float mstar = -INFINITY;
  for (int j = 0; j < nparts; ++j) mstar = fmaxf(mstar, part_lse[(int64_t)j * part_stride_rows]);
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mstar != -INFINITY) {
    for (int j = 0; j < nparts; ++j) {
      const float lj = part_lse[(int64_t)j * part_stride_rows];
      if (lj == -INFINITY) continue;
      const float wj = __expf(lj - mstar);
      wsum += wj;
      const f32x4* src = reinterpret_cast<const f32x4*>(part_o + (int64_t)j * part_stride_rows * kLatent);
      const f32x4 v0 = src[lane];
      const f32x4 v1 = src[64 + lane];
      acc0 += wj * v0;
      acc1 += wj * v1;
    }
  }
  const bool empty = !(wsum > 0.f);
  const float inv = empty ? 0.f : 1.0f / wsum;
  f32x4* dst = reinterpret_cast<f32x4*>(out);
  dst[lane] = acc0 * inv;
  dst[64 + lane] = acc1 * inv;
  if (lane == 0) *lse_out = empty ? -INFINITY : mstar + __logf(wsum);
}

// Merge of the planner's split requests: one wave per (split request, row).
__global__ __launch_bounds__(256) void merge_split_kernel(const uint8_t* plan, const float* ws_o,
                                                          const float* ws_lse, float* out,
                                                          float* lse) {
  const PlanHeader& ph = *reinterpret_cast<const PlanHeader*>(plan);
  const ReqParts* reqs = reinterpret_cast<const ReqParts*>(plan + ph.off_reqs);
  const int32_t* split = reinterpret_cast<const int32_t*>(plan + ph.off_split);
  const int M = ph.rows;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (gw >= (int64_t)ph.num_split_reqs * M) return;
  const int sr = (int)(gw / M);
  const int row = (int)(gw % M);
  const int b = split[sr];
  const ReqParts rp = reqs[b];
  merge_row(ws_o + ((int64_t)rp.first_part * M + row) * kLatent,
            ws_lse + (int64_t)rp.first_part * M + row, M, rp.num_parts,
            out + ((int64_t)b * M + row) * kLatent, lse + (int64_t)b * M + row, lane);
}

// Generic merge of num_parts stacked [rows, 512] partials.
__global__ __launch_bounds__(256) void lse_combine_kernel(const float* part_o,
                                                          const float* part_lse, int nparts,
                                                          int64_t rows, float* out, float* lse) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  merge_row(part_o + row * kLatent, part_lse + row, rows, nparts, out + row * kLatent,
            lse + row, lane);
}

// ---------------------------------------------------------------- launchers

hipError_t launch_decode(bool fp8, bool paged, int grid, const DecodeArgs& args,
                         hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (fp8 && paged) {
    hipLaunchKernelGGL((decode_kernel<true, true>), dim3(grid), dim3(256), 0, stream, args);
  } else if (fp8) {
    hipLaunchKernelGGL((decode_kernel<true, false>), dim3(grid), dim3(256), 0, stream, args);
  } else if (paged) {
    hipLaunchKernelGGL((decode_kernel<false, true>), dim3(grid), dim3(256), 0, stream, args);
  } else {
    hipLaunchKernelGGL((decode_kernel<false, false>), dim3(grid), dim3(256), 0, stream, args);
  }
  return hipGetLastError();
}

hipError_t launch_merge_split(const uint8_t* plan_dev, int num_split_reqs, int rows,
                              const float* ws_o, const float* ws_lse, float* out, float* lse,
                              hipStream_t stream) {
  const int64_t waves = (int64_t)num_split_reqs * rows;
  if (waves <= 0) return hipSuccess;
  const int64_t grid = (waves + 3) / 4;
  hipLaunchKernelGGL(merge_split_kernel, dim3((unsigned)grid), dim3(256), 0, stream, plan_dev,
                     ws_o, ws_lse, out, lse);
  return hipGetLastError();
}

hipError_t launch_lse_combine(const float* part_o, const float* part_lse, int nparts,
                              int64_t rows, float* out, float* lse, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int64_t grid = (rows + 3) / 4;
  hipLaunchKernelGGL(lse_combine_kernel, dim3((unsigned)grid), dim3(256), 0, stream, part_o,
                     part_lse, nparts, rows, out, lse);
  return hipGetLastError();
}

}  // namespace mla
