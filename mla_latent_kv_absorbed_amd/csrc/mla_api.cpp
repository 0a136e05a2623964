// Host side of the C ABI in include/mla.h: argument checks, the decode
// planner and kernel launches.
//
// Planner.  The page "Kimi K3 decode: DP16 vs DP2 x DCP8" (section "MLA")
// shows a fixed split rule, min(148 // B // (2 q), 32), that leaves one wave
// of 148 CTAs plus a 12-CTA second wave at 16 requests and so doubles the
// layer time.  Here the decode kernel is persistent instead: one workgroup
// per compute unit, each given an equal share of the total work, so no batch
// size leaves a partial wave.  The work of request b is n_b tokens (its local
// length) for each of its G = ceil(q_len H / 128) row groups, plus a fixed
// per-unit overhead (loading Q, writing O).  The concatenated work of all
// requests is cut into S equal pieces (S = compute units / G); piece s runs on
// G workgroups, one per row group, that stream the same tokens.  Workgroups
// are dispatched round-robin over the 8 XCDs (id modulo 8), each with its own
// L2: the G siblings get ids of one XCD, and each XCD takes a contiguous run
// of pieces, so that the pieces of a request mostly share one L2.  A request cut by
// piece boundaries produces one partial (O, LSE) per piece, merged by LSE
// afterwards (same page: partial results are merged by log-sum-exp).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "mla.h"
#include "kernels.h"
#include "kernels_step.h"
#include "plan_layout.h"


namespace {

using namespace mla;

// launch_decode takes the plan's mla_kv_dtype as a KvKind.
static_assert(kKvBf16 == MLA_KV_BF16 && kKvFp8 == MLA_KV_FP8_E4M3 && kKvFp4 == MLA_KV_FP4_E2M1 &&
                  kKvMx == MLA_KV_MXFP8_E4M3,
              "KvKind and mla_kv_dtype differ");

// Fixed cost of one work unit, in token-equivalents (Q load + O write).
constexpr int64_t kUnitOverheadTokens = 128;
// Smallest piece worth a workgroup of its own, in token-equivalents.
constexpr int64_t kMinPieceTokens = 512;
// Used by mla_plan_max_bytes when num_cus is left to the device query.
constexpr int kMaxCusBound = 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mla_status check_desc(const mla_decode_desc* d) {
  if (!d) return MLA_ERR_INVALID_ARG;
  if (d->kv_lora_rank != kLatent || d->rope_dim != kRope) return MLA_ERR_UNSUPPORTED;
  if (d->batch < 1 || d->q_len < 1 || d->q_len > kMaxQLen || d->num_heads < 1)
    return MLA_ERR_INVALID_ARG;
  if ((int64_t)d->q_len * d->num_heads > (1 << 20)) return MLA_ERR_INVALID_ARG;
  if (d->page_size < 1) return MLA_ERR_INVALID_ARG;
  if (d->kv_dtype != MLA_KV_BF16 && d->kv_dtype != MLA_KV_FP8_E4M3 &&
      d->kv_dtype != MLA_KV_FP4_E2M1 && d->kv_dtype != MLA_KV_MXFP8_E4M3)
    return MLA_ERR_INVALID_ARG;
  if (d->dcp_size < 1 || d->dcp_rank < 0 || d->dcp_rank >= d->dcp_size)
    return MLA_ERR_INVALID_ARG;
  if (d->num_cus < 0 || d->force_splits < 0) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

int row_groups(const mla_decode_desc* d) {
  const int M = d->q_len * d->num_heads;
  return (M + kRowsPerWG - 1) / kRowsPerWG;
}

int64_t local_len(int64_t L, int W, int r) {
  const int64_t n = (L - r + W - 1) / W;
  return n > 0 ? n : 0;
}

// Round a token cut down to the 32-token tile grid.
int64_t tile_floor(int64_t t) { return t / kTile * kTile; }

struct Seg {
  int b;
  int64_t j0, j1;
};

struct Layout {
  int64_t off_wg, off_units, off_reqs, off_split, total;
};

Layout layout_for(int64_t num_wgs, int64_t num_units, int64_t batch, int64_t num_split) {
  Layout l;
  l.off_wg = align_up(sizeof(PlanHeader), 16);
  l.off_units = align_up(l.off_wg + 4 * (num_wgs + 1), 16);
  l.off_reqs = align_up(l.off_units + (int64_t)sizeof(Unit) * num_units, 16);
  l.off_split = align_up(l.off_reqs + (int64_t)sizeof(ReqParts) * batch, 16);
  l.total = align_up(l.off_split + (int64_t)sizeof(SplitReq) * num_split, 16);
  return l;
}

// Upper bounds used to size the plan buffer.
void plan_bounds(const mla_decode_desc* d, int cus, int64_t* max_wgs, int64_t* max_units) {
  const int64_t G = row_groups(d);
  const int64_t B = d->batch;
  if (d->force_splits > 0) {
    *max_units = B * d->force_splits * G;
    *max_wgs = *max_units;
  } else {
    const int64_t S = std::max<int64_t>(1, cus / G);
    *max_wgs = 8 * G * ((S + 7) / 8);
    *max_units = (B + S) * G;
  }
}

}  // namespace

extern "C" {

mla_status mla_prepare(int32_t num_tokens, int32_t num_heads, int32_t kv_dtype,
                       const void* q_nope, const void* q_rope_in, const void* w_kc_t,
                       const void* c_kv_new, const void* k_rope_new, const int32_t* positions,
                       const float* cos_sin, int32_t max_pos, const int32_t* slots,
                       void* q_nope_absorbed, void* q_rope_out, void* kv_pool, float* kv_scale,
                       int64_t num_slots, void* stream) {
  if (num_tokens < 0 || num_heads < 1 || max_pos < 1 || num_slots < 1) return MLA_ERR_INVALID_ARG;
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3 && kv_dtype != MLA_KV_FP4_E2M1 &&
      kv_dtype != MLA_KV_MXFP8_E4M3)
    return MLA_ERR_INVALID_ARG;
  const bool fp8 = kv_dtype == MLA_KV_FP8_E4M3;
  for (const void* p : {q_nope, q_rope_in, w_kc_t, c_kv_new, k_rope_new, (const void*)positions,
                        (const void*)cos_sin, (const void*)slots, (const void*)q_nope_absorbed,
                        (const void*)q_rope_out, (const void*)kv_pool})
    if (!p || !aligned16(p)) return MLA_ERR_INVALID_ARG;
  if (fp8 && (!kv_scale || (reinterpret_cast<uintptr_t>(kv_scale) & 3u))) return MLA_ERR_INVALID_ARG;
  if (q_rope_out == q_rope_in) return MLA_ERR_INVALID_ARG;
  if ((int64_t)num_tokens * num_heads > INT32_MAX / 64) return MLA_ERR_INVALID_ARG;
  PrepareArgs a{};
  a.T = num_tokens;
  a.H = num_heads;
  a.max_pos = max_pos;
  a.kv = kv_dtype;
  a.num_slots = num_slots;
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_rope_in = static_cast<const uint16_t*>(q_rope_in);
  a.w_kc_t = static_cast<const uint16_t*>(w_kc_t);
  a.c_kv_new = static_cast<const uint16_t*>(c_kv_new);
  a.k_rope_new = static_cast<const uint16_t*>(k_rope_new);
  a.positions = positions;
  a.cos_sin = cos_sin;
  a.slots = slots;
  a.q_nope_absorbed = static_cast<uint16_t*>(q_nope_absorbed);
  a.q_rope_out = static_cast<uint16_t*>(q_rope_out);
  a.pool = kv_pool;
  a.kv_scale = fp8 ? kv_scale : nullptr;
  if (launch_prepare(a, static_cast<hipStream_t>(stream)) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

mla_status mla_lse_combine_project(const float* part_o, const float* part_lse, int32_t num_parts,
                                   int32_t num_tokens, int32_t num_heads, const void* w_vc_t,
                                   void* out_v, float* lse, void* stream) {
  if (num_parts < 1 || num_tokens < 0 || num_heads < 1) return MLA_ERR_INVALID_ARG;
  for (const void* p : {(const void*)part_o, (const void*)part_lse, w_vc_t, (const void*)out_v})
    if (!p || !aligned16(p)) return MLA_ERR_INVALID_ARG;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return MLA_ERR_INVALID_ARG;
  if (launch_combine_project(part_o, part_lse, num_parts, num_tokens, num_heads,
                             static_cast<const uint16_t*>(w_vc_t), static_cast<uint16_t*>(out_v),
                             lse, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace or plan buffer too small";
    case MLA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

size_t mla_plan_max_bytes(const mla_decode_desc* d) {
  if (check_desc(d) != MLA_OK) return 0;
  int64_t wgs, units;
  plan_bounds(d, d->num_cus > 0 ? d->num_cus : kMaxCusBound, &wgs, &units);
  return (size_t)layout_for(wgs, units, d->batch, d->batch).total;
}

mla_status mla_decode_plan(const mla_decode_desc* d, const int32_t* seq_lens_host,
                           void* plan_host, size_t plan_host_bytes, size_t* plan_bytes,
                           size_t* workspace_bytes) {
  const mla_status st = check_desc(d);
  if (st != MLA_OK) return st;
  if (!seq_lens_host || !plan_host || !plan_bytes || !workspace_bytes) return MLA_ERR_INVALID_ARG;
  if (!aligned16(plan_host)) return MLA_ERR_INVALID_ARG;

  int cus = d->num_cus;
  if (cus == 0) {
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return MLA_ERR_HIP;
    cus = prop.multiProcessorCount;
    if (cus < 1) return MLA_ERR_HIP;
  }
  if (plan_host_bytes < mla_plan_max_bytes(d)) {
    // The bound for a queried CU count may exceed the one computed without it.
    mla_decode_desc dd = *d;
    dd.num_cus = cus;
    if (plan_host_bytes < mla_plan_max_bytes(&dd)) return MLA_ERR_WORKSPACE_TOO_SMALL;
  }

  const int B = d->batch;
  const int M = d->q_len * d->num_heads;
  const int G = row_groups(d);
  const int W = d->dcp_size, R = d->dcp_rank;

  std::vector<int64_t> n(B);
  int64_t max_local = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t L = seq_lens_host[b];
    if (L < d->q_len || L > (int64_t)INT32_MAX) return MLA_ERR_INVALID_ARG;
    n[b] = local_len(L, W, R);
    max_local = std::max(max_local, n[b]);
  }

  // ---- cut the work into pieces: (piece index, segment) lists.
  std::vector<std::vector<Seg>> pieces;
  bool forced = d->force_splits > 0;
  if (forced) {
    const int k = d->force_splits;
    for (int b = 0; b < B; ++b) {
      int64_t prev = 0;
      bool any = false;
      for (int i = 1; i <= k; ++i) {
        const int64_t cut = (i == k) ? n[b] : tile_floor(n[b] * i / k);
        if (cut > prev || (i == k && !any)) {
          pieces.push_back({Seg{b, prev, cut}});
          any = true;
        }
        prev = std::max(prev, cut);
      }
    }
  } else {
    const int64_t S_max = std::max(1, cus / G);
    int64_t total = 0;
    std::vector<int64_t> start(B);
    for (int b = 0; b < B; ++b) {
      start[b] = total;
      total += n[b] + kUnitOverheadTokens;
    }
    const int64_t S = std::max<int64_t>(
        1, std::min<int64_t>(S_max, (total + kMinPieceTokens - 1) / kMinPieceTokens));
    pieces.assign(S, {});
    const double piece = (double)total / (double)S;
    for (int b = 0; b < B; ++b) {
      const double c0 = (double)start[b];
      const double c1 = c0 + (double)(n[b] + kUnitOverheadTokens);
      auto tokpos = [&](double c) -> int64_t {
        if (c <= c0) return 0;
        if (c >= c1) return n[b];
        int64_t t = tile_floor((int64_t)std::llround(c - c0 - (double)kUnitOverheadTokens));
        return std::min<int64_t>(std::max<int64_t>(t, 0), n[b]);
      };
      int64_t s_first = std::min<int64_t>(S - 1, (int64_t)(c0 / piece));
      int64_t s_last = std::min<int64_t>(S - 1, (int64_t)((c1 - 1e-9) / piece));
      bool any = false;
      for (int64_t s = s_first; s <= s_last; ++s) {
        const double cs = std::max(c0, (double)s * piece);
        const double ce = (s == s_last) ? c1 : std::min(c1, (double)(s + 1) * piece);
        const int64_t t0 = tokpos(cs), t1 = tokpos(ce);
        if (t1 > t0) {
          pieces[s].push_back(Seg{b, t0, t1});
          any = true;
        }
      }
      if (!any) pieces[s_first].push_back(Seg{b, 0, n[b]});  // empty request: (0, -inf)
    }
  }

  // ---- partial slots: requests that appear in more than one piece.
  std::vector<int> nparts(B, 0);
  for (auto& p : pieces)
    for (auto& sg : p) nparts[sg.b]++;
  std::vector<ReqParts> reqs(B);
  std::vector<int32_t> split;
  int total_parts = 0;
  for (int b = 0; b < B; ++b) {
    reqs[b].num_parts = nparts[b];
    if (nparts[b] > 1) {
      reqs[b].first_part = total_parts;
      total_parts += nparts[b];
      split.push_back(b);
    } else {
      reqs[b].first_part = -1;
    }
  }

  // ---- workgroups and units.
  const int64_t S = (int64_t)pieces.size();
  int64_t num_wgs;
  std::vector<int64_t> wg_of;  // (piece, g) -> workgroup id
  wg_of.resize(S * G);
  if (forced) {
    num_wgs = S * G;
    for (int64_t s = 0; s < S; ++s)
      for (int g = 0; g < G; ++g) wg_of[s * G + g] = s * G + g;
  } else if (8 * G * ((S + 7) / 8) <= cus) {
    // XCD k (workgroup ids congruent to k modulo 8) takes a contiguous run
    // of pieces, so that the pieces of one request share its L2 (and load
    // its Q rows once), and the G siblings of a piece take ids of the same
    // XCD (they stream the same KV tiles).  The first S % 8 XCDs take one
    // piece more; the ids this leaves unused are the highest ones, and all
    // ids stay below the number of compute units.
    const int64_t q = S / 8, r = S % 8;
    num_wgs = 0;
    for (int64_t s = 0; s < S; ++s) {
      const int64_t k = s < r * (q + 1) ? s / (q + 1) : r + (s - r * (q + 1)) / q;
      const int64_t slot = s < r * (q + 1) ? s % (q + 1) : (s - r * (q + 1)) % q;
      for (int g = 0; g < G; ++g) {
        const int64_t x = k + 8 * (G * slot + g);
        wg_of[s * G + g] = x;
        num_wgs = std::max(num_wgs, x + 1);
      }
    }
  } else {
    num_wgs = S * G;
    for (int64_t s = 0; s < S; ++s)
      for (int g = 0; g < G; ++g) wg_of[s * G + g] = s * G + g;
  }
  std::vector<std::vector<Unit>> per_wg(num_wgs);
  std::vector<int> next_part(B, 0);
  int64_t num_units = 0;
  for (int64_t s = 0; s < S; ++s) {
    for (const Seg& sg : pieces[s]) {
      const int part = reqs[sg.b].num_parts > 1 ? reqs[sg.b].first_part + next_part[sg.b]++ : -1;
      for (int g = 0; g < G; ++g) {
        Unit u{};
        u.b = sg.b;
        u.g = g;
        u.j0 = (int32_t)sg.j0;
        u.j1 = (int32_t)sg.j1;
        u.part = part;
        per_wg[wg_of[s * G + g]].push_back(u);
        ++num_units;
      }
    }
  }

  const Layout lay = layout_for(num_wgs, num_units, B, (int64_t)split.size());
  if ((size_t)lay.total > plan_host_bytes) return MLA_ERR_WORKSPACE_TOO_SMALL;

  uint8_t* base = static_cast<uint8_t*>(plan_host);
  std::memset(base, 0, (size_t)lay.total);
  PlanHeader* h = reinterpret_cast<PlanHeader*>(base);
  h->magic = kPlanMagic;
  h->version = kPlanVersion;
  h->batch = B;
  h->q_len = d->q_len;
  h->num_heads = d->num_heads;
  h->rows = M;
  h->row_groups = G;
  h->num_wgs = (int32_t)num_wgs;
  h->num_units = (int32_t)num_units;
  h->num_parts = total_parts;
  h->num_split_reqs = (int32_t)split.size();
  h->kv_dtype = d->kv_dtype;
  h->dcp_size = W;
  h->dcp_rank = R;
  h->off_wg = (int32_t)lay.off_wg;
  h->off_units = (int32_t)lay.off_units;
  h->off_reqs = (int32_t)lay.off_reqs;
  h->off_split = (int32_t)lay.off_split;
  h->max_local = (int32_t)max_local;
  h->page_size = d->page_size;
  h->plan_bytes = lay.total;
  // Split partials: O in fp16, each row scaled by a power of two (its factor
  // in the ws_sc array), then the partial LSE and the factors in fp32.
  const int64_t ws_o_bytes = (int64_t)total_parts * M * kLatent * 2;
  const int64_t ws_row_bytes = (int64_t)total_parts * M * 4;
  h->ws_lse_offset = align_up(ws_o_bytes, 256);
  h->ws_sc_offset = align_up(h->ws_lse_offset + ws_row_bytes, 256);
  h->workspace_bytes = total_parts > 0 ? align_up(h->ws_sc_offset + ws_row_bytes, 256) : 0;

  int32_t* wgb = reinterpret_cast<int32_t*>(base + lay.off_wg);
  Unit* units = reinterpret_cast<Unit*>(base + lay.off_units);
  int64_t k = 0;
  for (int64_t x = 0; x < num_wgs; ++x) {
    wgb[x] = (int32_t)k;
    for (const Unit& u : per_wg[x]) units[k++] = u;
  }
  wgb[num_wgs] = (int32_t)k;
  std::memcpy(base + lay.off_reqs, reqs.data(), sizeof(ReqParts) * B);
  SplitReq* sreq = reinterpret_cast<SplitReq*>(base + lay.off_split);
  for (size_t i = 0; i < split.size(); ++i)
    sreq[i] = SplitReq{split[i], reqs[split[i]].first_part, reqs[split[i]].num_parts, 0};

  *plan_bytes = (size_t)lay.total;
  *workspace_bytes = (size_t)h->workspace_bytes;
  return MLA_OK;
}

mla_status mla_check_table(const mla_decode_desc* d, const int32_t* seq_lens_host,
                           const int32_t* table, int64_t stride, int64_t num_slots,
                           int64_t* bad_request, int64_t* bad_index) {
  auto fail = [&](int64_t b, int64_t j) {
    if (bad_request) *bad_request = b;
    if (bad_index) *bad_index = j;
    return MLA_ERR_INVALID_ARG;
  };
  if (check_desc(d) != MLA_OK || !seq_lens_host || !table || num_slots < 1 || stride < 1)
    return fail(-1, -1);
  const bool runs = d->page_size % kTile == 0;
  for (int b = 0; b < d->batch; ++b) {
    const int64_t L = seq_lens_host[b];
    if (L < d->q_len) return fail(-1, -1);
    const int64_t n = local_len(L, d->dcp_size, d->dcp_rank);
    if (n > stride) return fail(-1, -1);
    const int32_t* row = table + (int64_t)b * stride;
    for (int64_t j = 0; j < n; ++j) {
      const int64_t s = row[j];
      if (s < 0 || s >= num_slots) return fail(b, j);
      if (runs && s != (int64_t)row[j - j % kTile] + j % kTile) return fail(b, j);
    }
  }
  return MLA_OK;
}

}  // extern "C"

namespace {

// Checks the arguments of a decode call and fills the kernel arguments.
mla_status decode_args(const void* plan_host, const void* plan_device, const void* q_nope,
                       const void* q_rope, const void* kv_pool, const float* kv_scale,
                       int64_t num_slots, const int32_t* req_to_token,
                       int64_t req_to_token_stride, const int32_t* seq_lens, float softmax_scale,
                       void* workspace, size_t workspace_bytes, float* out, float* lse,
                       DecodeArgs* a, const PlanHeader** header) {
  if (!plan_host || !plan_device || !q_nope || !q_rope || !kv_pool || !req_to_token ||
      !seq_lens || !out || !lse)
    return MLA_ERR_INVALID_ARG;
  if (!aligned16(plan_host)) return MLA_ERR_INVALID_ARG;
  const PlanHeader* h = static_cast<const PlanHeader*>(plan_host);
  if (h->magic != kPlanMagic || h->version != kPlanVersion) return MLA_ERR_INVALID_ARG;
  const bool fp8 = h->kv_dtype == MLA_KV_FP8_E4M3;
  if (fp8 && !kv_scale) return MLA_ERR_INVALID_ARG;
  for (const void* p : {plan_device, q_nope, q_rope, kv_pool, (const void*)req_to_token,
                        (const void*)seq_lens, (const void*)out, (const void*)lse})
    if (!aligned16(p)) return MLA_ERR_INVALID_ARG;
  if (fp8 && (reinterpret_cast<uintptr_t>(kv_scale) & 3u)) return MLA_ERR_INVALID_ARG;
  if (num_slots < 1 || num_slots > INT32_MAX ||
      req_to_token_stride < std::max<int64_t>(1, h->max_local))
    return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_INVALID_ARG;
  if ((int64_t)workspace_bytes < h->workspace_bytes) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (h->workspace_bytes > 0 && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)))
    return MLA_ERR_INVALID_ARG;

  *a = DecodeArgs{};
  a->plan = static_cast<const uint8_t*>(plan_device);
  a->q_nope = static_cast<const uint16_t*>(q_nope);
  a->q_rope = static_cast<const uint16_t*>(q_rope);
  a->pool = static_cast<const uint8_t*>(kv_pool);
  a->kv_scale = kv_scale;
  a->num_slots = num_slots;
  a->table = req_to_token;
  a->table_stride = req_to_token_stride;
  a->seq_lens = seq_lens;
  a->c2 = softmax_scale * 1.4426950408889634f;
  a->out = out;
  a->lse = lse;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a->ws_o = reinterpret_cast<uint16_t*>(ws);
  a->ws_lse = ws ? reinterpret_cast<float*>(ws + h->ws_lse_offset) : nullptr;
  a->ws_sc = ws ? reinterpret_cast<float*>(ws + h->ws_sc_offset) : nullptr;
  *header = h;
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_decode_attend(const void* plan_host, const void* plan_device, const void* q_nope,
                             const void* q_rope, const void* kv_pool, const float* kv_scale,
                             int64_t num_slots, const int32_t* req_to_token,
                             int64_t req_to_token_stride, const int32_t* seq_lens,
                             float softmax_scale, void* workspace, size_t workspace_bytes,
                             float* out, float* lse, void* stream) {
  DecodeArgs a;
  const PlanHeader* h = nullptr;
  const mla_status st = decode_args(plan_host, plan_device, q_nope, q_rope, kv_pool, kv_scale,
                                    num_slots, req_to_token, req_to_token_stride, seq_lens,
                                    softmax_scale, workspace, workspace_bytes, out, lse, &a, &h);
  if (st != MLA_OK) return st;
  const bool paged = (h->page_size % kTile) == 0;
  if (launch_decode(h->kv_dtype, paged, h->num_wgs, a, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

mla_status mla_decode_merge(const void* plan_host, const void* plan_device, const void* workspace,
                            size_t workspace_bytes, float* out, float* lse, void* stream) {
  if (!plan_host || !plan_device || !out || !lse) return MLA_ERR_INVALID_ARG;
  if (!aligned16(plan_host) || !aligned16(plan_device) || !aligned16(out) || !aligned16(lse))
    return MLA_ERR_INVALID_ARG;
  const PlanHeader* h = static_cast<const PlanHeader*>(plan_host);
  if (h->magic != kPlanMagic || h->version != kPlanVersion) return MLA_ERR_INVALID_ARG;
  if ((int64_t)workspace_bytes < h->workspace_bytes) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (h->num_split_reqs == 0) return MLA_OK;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return MLA_ERR_INVALID_ARG;
  const uint8_t* ws = static_cast<const uint8_t*>(workspace);
  const uint16_t* ws_o = reinterpret_cast<const uint16_t*>(ws);
  const float* ws_lse = reinterpret_cast<const float*>(ws + h->ws_lse_offset);
  const float* ws_sc = reinterpret_cast<const float*>(ws + h->ws_sc_offset);
  const uint8_t* blob = static_cast<const uint8_t*>(plan_host);
  const SplitReq* split = reinterpret_cast<const SplitReq*>(blob + h->off_split);
  int max_parts = 0;
  for (int i = 0; i < h->num_split_reqs; ++i)
    max_parts = split[i].num_parts > max_parts ? split[i].num_parts : max_parts;
  const SplitReq* split_dev =
      reinterpret_cast<const SplitReq*>(static_cast<const uint8_t*>(plan_device) + h->off_split);
  if (launch_merge_split(split_dev, h->num_split_reqs, h->rows, max_parts, ws_o, ws_lse, ws_sc,
                         out, lse,
                         static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

mla_status mla_decode(const void* plan_host, const void* plan_device, const void* q_nope,
                      const void* q_rope, const void* kv_pool, const float* kv_scale,
                      int64_t num_slots, const int32_t* req_to_token,
                      int64_t req_to_token_stride, const int32_t* seq_lens, float softmax_scale,
                      void* workspace, size_t workspace_bytes, float* out, float* lse,
                      void* stream) {
  const mla_status st = mla_decode_attend(plan_host, plan_device, q_nope, q_rope, kv_pool,
                                          kv_scale, num_slots, req_to_token,
                                          req_to_token_stride, seq_lens, softmax_scale,
                                          workspace, workspace_bytes, out, lse, stream);
  if (st != MLA_OK) return st;
  return mla_decode_merge(plan_host, plan_device, workspace, workspace_bytes, out, lse, stream);
}

mla_status mla_decode_noalloc(const void* plan_host, const void* plan_device, const void* q_nope,
                              const void* q_rope, const void* kv_pool, const float* kv_scale,
                              int64_t num_slots, const int32_t* req_to_token,
                              int64_t req_to_token_stride, const int32_t* seq_lens,
                              float softmax_scale, float* out, float* lse, void* stream) {
  if (!plan_host || !aligned16(plan_host)) return MLA_ERR_INVALID_ARG;
  const PlanHeader* h = static_cast<const PlanHeader*>(plan_host);
  if (h->magic != kPlanMagic || h->version != kPlanVersion) return MLA_ERR_INVALID_ARG;
  if (h->workspace_bytes > (int64_t)kNoAllocScratchBytes) return MLA_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (h->workspace_bytes > 0 && noalloc_scratch(&ws) != hipSuccess) return MLA_ERR_HIP;
  return mla_decode(plan_host, plan_device, q_nope, q_rope, kv_pool, kv_scale, num_slots,
                    req_to_token, req_to_token_stride, seq_lens, softmax_scale, ws,
                    ws ? kNoAllocScratchBytes : 0, out, lse, stream);
}

mla_status mla_lse_combine(const float* part_o, const float* part_lse, int32_t num_parts,
                           int64_t rows, float* out, float* lse, void* stream) {
  if (num_parts < 1 || rows < 0) return MLA_ERR_INVALID_ARG;
  if (rows == 0) return MLA_OK;
  if (!part_o || !part_lse || !out || !lse) return MLA_ERR_INVALID_ARG;
  if (!aligned16(part_o) || !aligned16(out) || (reinterpret_cast<uintptr_t>(part_lse) & 3u) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return MLA_ERR_INVALID_ARG;
  if (rows > (int64_t)INT32_MAX) return MLA_ERR_INVALID_ARG;
  if (launch_lse_combine(part_o, part_lse, num_parts, rows, out, lse,
                         static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

}  // extern "C"
