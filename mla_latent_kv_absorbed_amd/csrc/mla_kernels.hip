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
// KV tiles arrive by direct global->LDS DMA (global_load_lds_dwordx4), one
// tile ahead.  FP8 rows land in a staging buffer and are widened to BF16
// (exact: every e4m3fn value is a BF16 value) by the workgroup before use;
// the per-token fp32 scale multiplies the score column and the probability,
// never the stored element, so K and V stay exact.
//
// LDS tile layout: 16-byte chunk cc of token t at cc * 512 + 16 * (t ^ 4 *
// (cc & 3)).  Reading chunk cc of tokens 0..31 (QK operand) and 4-token x
// 32-byte blocks of 4 chunks (transposed V operand) are both bank-conflict
// free under this swizzle, and every DMA lane keeps one token per tile.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "plan_layout.h"
#include "pv_asm.inc"

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

// LDS map of the decode kernel (bytes).
constexpr int kLdsTile0 = 0;
constexpr int kLdsTile1 = kTileBf16;
constexpr int kLdsStage0 = 2 * kTileBf16;
constexpr int kLdsStage1 = kLdsStage0 + kTileFp8;
constexpr int kLdsScale = kLdsStage1 + kTileFp8;  // float[4][kTile], indexed by tile & 3
constexpr int kLdsBf16Total = 2 * kTileBf16;
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

// VMEM instructions one wave issues per tile: BF16 9; FP8 5, 5, 4, 4 + 1 scale.
// The wait allows one slot load and the next tile's DMA to stay in flight:
// vmcnt counts in issue order, so the awaited (older) tile has then landed.
template <bool kFp8>
__device__ __forceinline__ void wait_prev_tile_dma(int w) {
  if constexpr (!kFp8) {
    wait_vmcnt<10>();
  } else {
    if (w == 2) wait_vmcnt<5>(); else wait_vmcnt<6>();
  }
}

// Same, when no vector slot load sits between the two tiles' DMA (paged
// tables read their entry with a scalar load).
template <bool kFp8>
__device__ __forceinline__ void wait_prev_tile_dma_noslot(int w) {
  if constexpr (!kFp8) {
    wait_vmcnt<9>();
  } else {
    if (w == 2) wait_vmcnt<4>(); else wait_vmcnt<5>();
  }
}

// Widen a staged FP8 tile into the BF16 tile layout (exact conversion).
__device__ __forceinline__ void widen_fp8_tile(const LDS_AS uint8_t* stage, LDS_AS uint8_t* tile,
                                               int tid) {
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    const int u = tid + 256 * k;
    const int half = u & 1;
    const int t = (u >> 1) & 31;
    const int c8 = u >> 6;
    const u32x2 raw = *(const LDS_AS u32x2*)(stage + (c8 * kTile + t) * 16 + 8 * half);
    // Two e4m3fn codes -> two packed BF16 per instruction (scale 1: exact).
    // (Extracting the elements of v_cvt_pk_f32_fp8 and repacking them was
    // miscompiled: both halves received the first element.)
    u32x4 o;
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, false));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, true));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, false));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, true));
    const int cc = 2 * c8 + half;
    *(LDS_AS u32x4*)(tile + cc * kBlock + swz_tok(cc, t) * 16) = o;
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

__device__ __forceinline__ int64_t clamp_slot(int64_t s, int64_t n) {
  return s < 0 ? 0 : (s >= n ? n - 1 : s);
}

// S^T[32 tokens x 32 rows] = K . Q^T over the 576 features of one tile.
//
// The accumulator is pinned to VGPRs: the O accumulators take all 256 AGPRs
// and Q takes 144 VGPRs, so this is the only assignment that fits the 512
// registers of one wave per SIMD, and the compiler does not choose it by
// itself.  Because the MFMAs are issued from inline asm, the hazards the
// compiler would otherwise cover are covered here: a few wait states before
// each block (operands may have just been written by a VALU move), and
// enough after the last MFMA for its result to be read by VALU instructions.
// Dependent MFMAs on the same accumulator issue back to back.
#define MLA_MFMA4(first)                                                           \
  "v_mfma_f32_32x32x16_bf16 %0, %1, %5, " first "\n\t"                             \
  "v_mfma_f32_32x32x16_bf16 %0, %2, %6, %0\n\t"                                    \
  "v_mfma_f32_32x32x16_bf16 %0, %3, %7, %0\n\t"                                    \
  "v_mfma_f32_32x32x16_bf16 %0, %4, %8, %0\n\t"

__device__ __forceinline__ f32x16 qk_tile(const LDS_AS uint8_t* tile, int kbase_e, int kbase_o,
                                          const bf16x8* qf) {
  f32x16 s;
#pragma unroll
  for (int g = 0; g < kKSteps / 4; ++g) {
    const int ks = 4 * g;
    const bf16x8 k0 = *(const LDS_AS bf16x8*)(tile + kbase_e + 1024 * (ks + 0));
    const bf16x8 k1 = *(const LDS_AS bf16x8*)(tile + kbase_o + 1024 * (ks + 1));
    const bf16x8 k2 = *(const LDS_AS bf16x8*)(tile + kbase_e + 1024 * (ks + 2));
    const bf16x8 k3 = *(const LDS_AS bf16x8*)(tile + kbase_o + 1024 * (ks + 3));
    if (g == 0) {
      asm volatile("s_nop 2\n\t" MLA_MFMA4("0")
                   : "=&v"(s)
                   : "v"(k0), "v"(k1), "v"(k2), "v"(k3), "v"(qf[ks]), "v"(qf[ks + 1]),
                     "v"(qf[ks + 2]), "v"(qf[ks + 3]));
    } else {
      asm volatile("s_nop 2\n\t" MLA_MFMA4("%0")
                   : "+v"(s)
                   : "v"(k0), "v"(k1), "v"(k2), "v"(k3), "v"(qf[ks]), "v"(qf[ks + 1]),
                     "v"(qf[ks + 2]), "v"(qf[ks + 3]));
    }
  }
  // Result consumed by VALU next: wait out the MFMA write latency.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s));
  return s;
}
#undef MLA_MFMA4

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
  const int w = tid >> 6;
  const int n_lane = lane & 31;   // row within the wave / token within a tile
  const int hk = lane >> 5;       // k-half of MFMA operands
  const int M = ph->rows;
  const int H = ph->num_heads;
  const int qlen = ph->q_len;
  const int W = ph->dcp_size;
  const int R = ph->dcp_rank;
  constexpr int kAhead = kFp8 ? 2 : 1;  // how many tiles the DMA runs ahead
  constexpr int kRowBytes = kFp8 ? kRow : 2 * kRow;

  // Lane-constant parts of the LDS operand addresses.  QK operand (chunk
  // cc = 2 ks + hk of token n_lane): the swizzle only depends on ks & 1.
  const int kbase_e = 512 * hk + 16 * (n_lane ^ (4 * hk));
  const int kbase_o = 512 * hk + 16 * (n_lane ^ (8 + 4 * hk));
  // Transposed V operand: in 16-lane group g16 lane 4 krow + cpart addresses
  // token 16 e + 8 x + 4 hk + krow, features 32 db + 16 (g16 & 1) + 4 cpart.
  const int g16 = lane >> 4;
  const int krow = (lane & 15) >> 2;
  const int cpart = lane & 3;
  const int c3 = 2 * (g16 & 1) + (cpart >> 1);  // (chunk index) & 3
  const int vbase0 = 512 * c3 + 16 * ((4 * hk + krow) ^ (4 * c3)) + 8 * (cpart & 1);
  const int vbase1 = 512 * c3 + 16 * ((8 + 4 * hk + krow) ^ (4 * c3)) + 8 * (cpart & 1);
  // DMA: the token this lane moves, and its first chunk's byte offset in a row.
  const int dma_tok = kFp8 ? n_lane : (n_lane ^ (((2 * w + hk) & 3) << 2));
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
    float m_ref = -INFINITY;  // running max (log2 domain) of this lane's row
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
      // BF16: the DMA of tile it+1 overlaps the compute of tile it.
      // FP8: the DMA runs two tiles ahead into a staging buffer, and tile
      // it+1 is widened to BF16 after the P.V product of tile it.
      LDS_AS uint8_t* dma_buf0 = lds + (kFp8 ? kLdsStage0 : kLdsTile0);
      LDS_AS uint8_t* dma_buf1 = lds + (kFp8 ? kLdsStage1 : kLdsTile1);
      LDS_AS float* sc_lds = (LDS_AS float*)(lds + kLdsScale);
      {
        const int64_t s0 = lane_slot(slot_raw(0), 0);
        issue_tile_dma<kFp8>(a.pool + s0 * kRowBytes + dma_chunk_off, a.kv_scale + s0,
                             dma_buf0, sc_lds, w, lane);
      }
      if constexpr (kFp8) {
        if (ntiles > 1) {
          const int64_t s1 = lane_slot(slot_raw(1), 1);
          issue_tile_dma<kFp8>(a.pool + s1 * kRowBytes + dma_chunk_off, a.kv_scale + s1,
                               dma_buf1, sc_lds + kTile, w, lane);
        }
      }
      int32_t raw_pending = slot_raw(kAhead);  // locates tile it + kAhead
      if constexpr (kFp8) {
        if (ntiles > 1) {
          if constexpr (kPaged) wait_prev_tile_dma_noslot<kFp8>(w);
          else wait_prev_tile_dma<kFp8>(w);
        } else {
          wait_vmcnt<0>();
        }
        barrier_lds();
        widen_fp8_tile(lds + kLdsStage0, lds + kLdsTile0, tid);
        barrier_lds();
      }

      for (int it = 0; it < ntiles; ++it) {
        // ---- prefetch: table entry of tile it+kAhead+1, DMA of tile it+kAhead.
        // A vector slot load (general tables) must be issued before the DMA:
        // the vmcnt arithmetic of wait_prev_tile_dma counts it there.
        const int32_t raw_later = slot_raw(it + kAhead + 1);
        asm volatile("" ::: "memory");
        if (it + kAhead < ntiles) {
          const int tn = it + kAhead;
          const int64_t sl = lane_slot(raw_pending, tn);
          issue_tile_dma<kFp8>(a.pool + sl * kRowBytes + dma_chunk_off, a.kv_scale + sl,
                               (tn & 1) ? dma_buf1 : dma_buf0, sc_lds + kTile * (tn & 3), w,
                               lane);
          if constexpr (kPaged) wait_prev_tile_dma_noslot<kFp8>(w);
          else wait_prev_tile_dma<kFp8>(w);
        } else {
          wait_vmcnt<0>();
        }
        barrier_lds();

        const LDS_AS uint8_t* tile = lds + ((it & 1) ? kLdsTile1 : kLdsTile0);
        const int jt = j0 + it * kTile;

        // ---- S^T = K . Q^T
        f32x16 s = qk_tile(tile, kbase_e, kbase_o, qf);

        // ---- scores -> log2 domain, mask, tile max.
        // acc index i holds token 8 (i / 4) + 4 hk + (i % 4) of the tile; for
        // FP8 its scale is read from LDS here and again for P (cheaper than
        // holding 16 more registers across the rescale).
        const LDS_AS float* sct = sc_lds + kTile * (it & 3);
        float ksc[16];
        if constexpr (kFp8) load_tile_scales(sct, hk, ksc);
        const int lim = jmax - jt;  // tokens m <= lim are visible to this row
        float mt = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = 8 * (i >> 2) + 4 * hk + (i & 3);
          float v = s[i] * (kFp8 ? a.c2 * ksc[i] : a.c2);
          v = (m <= lim) ? v : -INFINITY;
          s[i] = v;
          mt = fmaxf(mt, v);
        }
        mt = wave_xor32_max(mt);

        // ---- lazy rescale: only when the max grows by more than 2^8.
        const bool need = mt > m_ref + kLazyRescale;
        if (__any(need)) {
          const float m_new = need ? mt : m_ref;
          const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
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
        const float msafe = (m_ref == -INFINITY) ? 0.f : m_ref;

        // ---- P (fp32 -> bf16), FP8 value scale folded in.
        if constexpr (kFp8) load_tile_scales(sct, hk, ksc);
        bf16x8 pb0, pb1;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = __builtin_amdgcn_exp2f(s[i] - msafe);
          l_part += e;
          const float pv = kFp8 ? e * ksc[i] : e;
          if (i < 8) pb0[i] = (__bf16)pv; else pb1[i - 8] = (__bf16)pv;
        }

        // ---- O^T += V^T . P^T.  For MFMA e, k-slot 8 hk + jj is token
        // 16 e + 8 (jj / 4) + 4 hk + jj % 4: two transposing reads of 4 tokens
        // each (lane addresses va / vb), all inside one asm statement.
        {
          const LDS_AS uint8_t* va = tile + vbase0;
          const LDS_AS uint8_t* vb = tile + vbase1;
          asm volatile(MLA_PV_TILE_ASM
                       : [a0] "+a"(acc_o[0]), [a1] "+a"(acc_o[1]), [a2] "+a"(acc_o[2]),
                         [a3] "+a"(acc_o[3]), [a4] "+a"(acc_o[4]), [a5] "+a"(acc_o[5]),
                         [a6] "+a"(acc_o[6]), [a7] "+a"(acc_o[7]), [a8] "+a"(acc_o[8]),
                         [a9] "+a"(acc_o[9]), [a10] "+a"(acc_o[10]), [a11] "+a"(acc_o[11]),
                         [a12] "+a"(acc_o[12]), [a13] "+a"(acc_o[13]), [a14] "+a"(acc_o[14]),
                         [a15] "+a"(acc_o[15])
                       : [va] "v"(va), [vb] "v"(vb), [p0] "v"(pb0), [p1] "v"(pb1)
                       : "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247",
                         "v248", "v249", "v250", "v251", "v252", "v253", "v254", "v255",
                         "memory");
        }

        raw_pending = raw_later;
        if constexpr (kFp8) {
          if (it + 1 < ntiles)
            widen_fp8_tile(lds + (((it + 1) & 1) ? kLdsStage1 : kLdsStage0),
                           lds + (((it + 1) & 1) ? kLdsTile1 : kLdsTile0), tid);
        }
        barrier_lds();
      }
    }

    // ---- epilogue: O = acc / l, LSE = ln 2 * (m + log2 l).
    acc_settle(acc_o);
    const float l_row = l_part + __shfl_xor(l_part, 32);
    const bool empty = !(l_row > 0.f);
    const float inv = empty ? 0.f : 1.0f / l_row;
    const float lse_v = empty ? -INFINITY : (m_ref + __builtin_amdgcn_logf(l_row)) * kLn2;
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
