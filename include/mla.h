/*
 * mla.h -- C ABI of the MI355X (gfx950) absorbed MLA decode library.
 *
 * The operation (page "Kimi K3 decode: DP16 vs DP2 x DCP8", section "MLA";
 * page "resident VRAM accounting", sections "KV ledger" and "cell_size"):
 * every request b has q_len x num_heads query rows.  Row (i, h) is the
 * 576-wide vector [q_nope_absorbed (512) | q_rope (64)]; the no-RoPE half has
 * already been multiplied by w_kc, into which kv_b_proj was absorbed.  All
 * rows of a request score against ONE shared latent KV head: a paged pool of
 * 576-element rows [c_kv (512) | k_rope (64)], one row per token, no head
 * dimension.  The attended value is c_kv itself (the first 512 elements), so
 * the output stays in the 512-wide latent space, and the per-row
 * log-sum-exp (LSE) is returned with it so that partial results over
 * disjoint token sets can be merged exactly:
 *
 *   s_p  = softmax_scale * (q . k_p)            over visible positions p
 *   LSE  = ln sum_p exp(s_p)                     (natural log, scale included)
 *   O    = sum_p exp(s_p - LSE) * k_p[0:512]
 *
 * Visible positions of draft row i of request b: 0 <= p <= L_b - q_len + i,
 * where L_b = seq_lens[b] counts the q_len draft tokens (their latent rows
 * are already in the pool).  Under decode context parallelism (DCP, same
 * page, section "problem: how to split"), shard r of W holds only positions
 * p % W == r, and its table is indexed by the local index j = (p - r) / W.
 *
 * Memory: every buffer belongs to the caller.  The library allocates no
 * device memory and keeps no mutable global state; every call is
 * asynchronous on the caller's HIP stream and thread-safe.  Argument errors
 * are detected on the host and returned synchronously; nothing is enqueued
 * when a call fails.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,         /* a null pointer, bad size, bad alignment, ... */
  MLA_ERR_UNSUPPORTED = -2,         /* a valid but unimplemented shape (dims != 512/64) */
  MLA_ERR_WORKSPACE_TOO_SMALL = -3, /* workspace or plan buffer smaller than required */
  MLA_ERR_HIP = -4                  /* a HIP runtime call or kernel launch failed */
} mla_status;

typedef enum {
  MLA_KV_BF16 = 0,     /* pool element = bfloat16 */
  MLA_KV_FP8_E4M3 = 1  /* pool element = OCP e4m3fn byte; fp32 scale per slot */
} mla_kv_dtype;

/* Problem description shared by the planner and the decode call. */
typedef struct {
  int32_t batch;        /* B >= 1 requests */
  int32_t q_len;        /* 1..8 query (draft) positions per request */
  int32_t num_heads;    /* H >= 1 query heads; rows per request M = q_len * H */
  int32_t kv_lora_rank; /* must be 512 */
  int32_t rope_dim;     /* must be 64 */
  int32_t page_size;    /* tokens per pool page (>= 1).  When it is a multiple of 32
                           the kernel reads one table entry per 32 local indices
                           and assumes that the 32 slots behind it are consecutive
                           (slot of j = table[j - j % 32] + j % 32), which holds for
                           any paged layout whose pages are page_size consecutive
                           slots starting at a multiple of page_size in the local
                           index.  Otherwise every entry is read. */
  int32_t kv_dtype;     /* mla_kv_dtype */
  int32_t dcp_size;     /* W >= 1 shards; 1 = unsharded */
  int32_t dcp_rank;     /* 0 <= r < W: this pool holds positions p % W == r */
  int32_t num_cus;      /* compute units to plan for; 0 = query the current device */
  int32_t force_splits; /* 0 = planner decides; k > 0 = split every request into k
                           equal token ranges, one work unit each (for tests) */
} mla_decode_desc;

/*
 * Upper bound, in bytes, of the plan that mla_decode_plan writes for `desc`.
 * Returns 0 if desc is invalid.
 */
size_t mla_plan_max_bytes(const mla_decode_desc* desc);

/*
 * Host-side planner (wave-quantisation aware; replaces the fixed-split rule
 * the DP16-vs-DP2 page analyses in its section "MLA").  Reads the GLOBAL
 * lengths seq_lens_host[B] (host memory, each >= q_len) and writes a
 * self-contained plan blob into plan_host (host memory, plan_host_bytes >=
 * mla_plan_max_bytes(desc)).  The work is cut into one persistent workgroup
 * per compute unit, with equal token work per workgroup, and partial results
 * where a request is cut.  On success *plan_bytes is the number of plan bytes
 * written and *workspace_bytes the device scratch that mla_decode needs for
 * partial (O, LSE) results (0 if no request is split).
 *
 * The caller copies the first *plan_bytes bytes of plan_host, unchanged, to
 * a device buffer (16-byte aligned) and passes both copies to mla_decode.
 * With num_cus == 0 the current HIP device is queried (a HIP error gives
 * MLA_ERR_HIP); any other value plans without touching a GPU.
 */
mla_status mla_decode_plan(const mla_decode_desc* desc, const int32_t* seq_lens_host,
                           void* plan_host, size_t plan_host_bytes, size_t* plan_bytes,
                           size_t* workspace_bytes);

/*
 * Absorbed MLA decode (DP16-vs-DP2 page, section "MLA": the kernel that
 * scores heads x q_len rows against the latent KV, called attn_mqa there).
 *
 *   plan_host / plan_device: the plan from mla_decode_plan, in host memory and
 *       its byte-identical device copy.
 *   q_nope_absorbed: bf16 [B, q_len, H, 512], contiguous, device.
 *   q_rope:          bf16 [B, q_len, H, 64], contiguous, device.
 *   kv_pool:         [num_slots, 576] contiguous, device; bf16 or e4m3fn bytes
 *                    per desc.kv_dtype; row = [c_kv (512) | k_rope (64)];
 *                    1 <= num_slots <= 2^31 - 1.
 *   kv_scale:        fp32 [num_slots] for FP8 (value = e4m3fn(code) * scale),
 *                    NULL for BF16.
 *   req_to_token:    int32 [B, req_to_token_stride], device; column j holds the
 *                    pool slot of local index j (= position p when W == 1).
 *                    Slots outside [0, num_slots) are clamped (no fault, but the
 *                    result is then undefined).
 *   seq_lens:        int32 [B] device copy of the global lengths used to plan.
 *   softmax_scale:   the scale applied to q . k before the exponent (finite, > 0).
 *   workspace:       device scratch of >= *workspace_bytes from the plan (may
 *                    be NULL when that is 0), 256-byte aligned.
 *   out:             fp32 [B, q_len, H, 512] device output O.
 *   lse:             fp32 [B, q_len, H] device output LSE (natural log).
 *   stream:          HIP stream (hipStream_t), 0 = default stream.
 *
 * When the plan cuts a request into several token ranges, their partial
 * (O, LSE) go to the workspace and a merge kernel is enqueued on the same
 * stream, so the caller always sees the final result.  All device pointers
 * must be 16-byte aligned.
 */
mla_status mla_decode(const void* plan_host, const void* plan_device,
                      const void* q_nope_absorbed, const void* q_rope, const void* kv_pool,
                      const float* kv_scale, int64_t num_slots, const int32_t* req_to_token,
                      int64_t req_to_token_stride, const int32_t* seq_lens,
                      float softmax_scale, void* workspace, size_t workspace_bytes,
                      float* out, float* lse, void* stream);

/*
 * The two halves of mla_decode, for callers that time them apart or run
 * other work between them (same arguments, checks and errors as mla_decode).
 *
 * mla_decode_attend enqueues only the attention kernel: requests the plan
 * keeps whole get their final (O, LSE) in out / lse; each piece of a cut
 * request writes its partial (O, LSE) to the workspace (split KV, merged by
 * LSE as on the DP16-vs-DP2 page, section "MLA").
 *
 * mla_decode_merge enqueues the LSE merge of the cut requests' partials
 * from the workspace into out / lse (nothing when the plan cuts no request).
 * It must follow mla_decode_attend with the same plan and workspace on the
 * same stream (or after it completes); the workspace is read, not written.
 */
mla_status mla_decode_attend(const void* plan_host, const void* plan_device,
                             const void* q_nope_absorbed, const void* q_rope,
                             const void* kv_pool, const float* kv_scale, int64_t num_slots,
                             const int32_t* req_to_token, int64_t req_to_token_stride,
                             const int32_t* seq_lens, float softmax_scale, void* workspace,
                             size_t workspace_bytes, float* out, float* lse, void* stream);
mla_status mla_decode_merge(const void* plan_host, const void* plan_device,
                            const void* workspace, size_t workspace_bytes, float* out,
                            float* lse, void* stream);

/*
 * Merge num_parts partial results by log-sum-exp (DP16-vs-DP2 page, section
 * "MLA": per-shard (O, LSE) are exchanged and merged, dcp_lse_combine).
 *
 *   part_o:   fp32 [num_parts, rows, 512] device; part_lse: fp32 [num_parts, rows].
 *   out:      fp32 [rows, 512] device;      lse: fp32 [rows].
 * For each row: M* = max_j LSE_j; if M* = -inf the row is (0, -inf); else
 * w_j = exp(LSE_j - M*), LSE = M* + ln sum_j w_j, O = sum_j w_j O_j / sum_j w_j.
 * Parts with LSE = -inf contribute nothing (their O is never read as a
 * weight > 0).  num_parts >= 1, rows >= 0; 16-byte aligned pointers.
 */
mla_status mla_lse_combine(const float* part_o, const float* part_lse, int32_t num_parts,
                           int64_t rows, float* out, float* lse, void* stream);

/* Static description of a status code. */
const char* mla_status_string(mla_status status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
