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
 * device memory and keeps no mutable global state, with one exception that
 * only mla_decode_noalloc uses: a fixed scratch array per GPU, held from its
 * first use until the process ends.  Every call is asynchronous on the
 * caller's HIP stream and thread-safe (mla_decode_noalloc: see its own note
 * on overlapping calls).  Argument errors are detected on the host and
 * returned synchronously; nothing is enqueued when a call fails.
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

/*
 * KV pool formats.  FP4 (page "resident VRAM accounting", sections "KV ledger"
 * and "cell_size": two codes per byte plus one scale per 16 elements, a
 * little over a quarter of BF16 per token) is read as: OCP e2m1 codes and
 * one power-of-two scale byte per 16 elements.  A token's row is 336 bytes:
 *   bytes   0..287  the 576 codes, element 2 i in the low nibble of byte i;
 *   bytes 288..323  block scales, byte 288 + k for elements 16 k .. 16 k + 15,
 *                   code c meaning 2^(c - 127), valid for 63 <= c <= 191;
 *   bytes 324..335  padding (ignored; rows stay 16-byte aligned).
 * Element value = e2m1(code) * 2^(c - 127).  A referenced row with a scale
 * code outside 63..191 gives an undefined result (no fault).
 *
 * MXFP8 (same page, "cell_size": one byte per element plus one scale per 32
 * elements) is read as OCP e4m3fn codes with one power-of-two scale byte per
 * 32 elements, 608 bytes a row:
 *   bytes   0..575  the 576 codes, element i in byte i;
 *   bytes 576..593  block scales, byte 576 + k for elements 32 k .. 32 k + 31,
 *                   code c meaning 2^(c - 127), valid for 63 <= c <= 191;
 *   bytes 594..607  padding (ignored).
 * Element value = e4m3fn(code) * 2^(c - 127).
 */
typedef enum {
  MLA_KV_BF16 = 0,       /* pool element = bfloat16 */
  MLA_KV_FP8_E4M3 = 1,   /* pool element = OCP e4m3fn byte; fp32 scale per slot */
  MLA_KV_FP4_E2M1 = 2,   /* 336-byte rows of e2m1 codes and block scales (above) */
  MLA_KV_MXFP8_E4M3 = 3  /* 608-byte rows of e4m3fn codes and block scales (above) */
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
 * Opt-in host check of the table contract that mla_decode relies on (page
 * "resident VRAM accounting", section "req_to_token": an int32 table maps
 * each request's token index to a pool slot; pages are page_size
 * consecutive slots).  mla_decode never reads the table on the host; a
 * caller that wants the contract verified copies the table to host memory
 * and calls this before decoding.
 *
 *   desc:              the description the plan is made from (batch,
 *                      q_len, page_size, dcp_size, dcp_rank are used).
 *   seq_lens_host:     int32 [B] global lengths, host memory.
 *   req_to_token_host: int32 [B, stride] host copy of the table.
 *   stride:            its row stride in entries (>= every local length).
 *   num_slots:         the pool's slot count.
 *
 * For every request b and local index j < n_b (n_b = the number of
 * positions p < L_b with p % W == r) it checks 0 <= table[b, j] < num_slots
 * and, when page_size is a multiple of 32, table[b, j] = table[b, j - j % 32]
 * + j % 32 (the 32 slots behind each entry the kernel reads are
 * consecutive).  Entries past n_b are not read by mla_decode and not checked.
 * Returns MLA_OK; MLA_ERR_INVALID_ARG for bad arguments or a broken contract,
 * with *bad_request / *bad_index (if not NULL) set to the first failing
 * entry (-1 / -1 for an argument error); nothing else is written.
 */
mla_status mla_check_table(const mla_decode_desc* desc, const int32_t* seq_lens_host,
                           const int32_t* req_to_token_host, int64_t stride, int64_t num_slots,
                           int64_t* bad_request, int64_t* bad_index);

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
 *                    FP4: [num_slots, 336], MXFP8: [num_slots, 608] bytes in
 *                    the row formats above.
 *                    1 <= num_slots <= 2^31 - 1.
 *   kv_scale:        fp32 [num_slots] for FP8 (value = e4m3fn(code) * scale),
 *                    ignored (may be NULL) for the other formats.
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
 * mla_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same call without the workspace arguments.  The split partials go to a
 * scratch array of MLA_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on, from the first such call on that GPU until the process
 * ends; nothing is allocated per call (no hipMalloc, hipFree or allocating
 * library routine).
 *
 * Arguments, layouts and errors as for mla_decode; in addition a plan whose
 * *workspace_bytes exceeds MLA_NOALLOC_SCRATCH_BYTES is rejected with
 * MLA_ERR_WORKSPACE_TOO_SMALL (nothing is enqueued; mla_decode with a
 * caller workspace handles it).  The scratch array is shared by every call
 * on a GPU and keeps the last call's contents (the kernels write every
 * partial before reading it, so nothing needs clearing); calls that overlap
 * on one GPU (on different streams, or from different host threads without
 * ordering) race on it and must not be issued.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
mla_status mla_decode_noalloc(const void* plan_host, const void* plan_device,
                              const void* q_nope_absorbed, const void* q_rope,
                              const void* kv_pool, const float* kv_scale, int64_t num_slots,
                              const int32_t* req_to_token, int64_t req_to_token_stride,
                              const int32_t* seq_lens, float softmax_scale, float* out,
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

/*
 * MLA prepare: the step before mla_decode, on the T = B * q_len new tokens of
 * a decode step (page "Kimi K3 decode: DP16 vs DP2 x DCP8": kv_b_proj is
 * absorbed into w_kc / w_vc, whose w_kc is 96 x 128 x 512 bf16; the step is
 * the mla_prepare of section "MLA").  It computes:
 *
 *   q_nope_absorbed[t, h, n] = sum_k q_nope[t, h, k] * w_kc[h, k, n]
 *       (fp32 accumulation, rounded to bf16: the decode kernel's query input);
 *   q_rope_out[t, h, :] = RoPE(q_rope_in[t, h, :], positions[t]);
 *   pool row slots[t] = [c_kv_new[t] | RoPE(k_rope_new[t], positions[t])],
 *       as bf16, or for FP8 pools as e4m3fn codes of x / scale with
 *       scale = amax / 448 over the row's 576 values (1 if all are zero),
 *       stored in kv_scale[slots[t]], or for FP4 pools as an FP4 row (format
 *       at mla_kv_dtype): per 16-element block with largest magnitude a,
 *       the exponent e is the smallest integer with a <= 6 * 2^e, clamped to
 *       [-64, 64] (a = 0 gives -64), and each code is the e2m1 value nearest
 *       to x * 2^-e (ties to the code with an even mantissa bit, clamped to
 *       +-6); the padding bytes are written as zeros; or for MXFP8 pools the
 *       same per 32-element block with 448 in place of 6 and e4m3fn codes.
 *
 * RoPE rotates the interleaved pairs (x[2i], x[2i+1]) of a 64-wide vector:
 * (x0 c - x1 s, x0 s + x1 c) with c = cos_sin[pos, i], s = cos_sin[pos, 32 + i];
 * products and sums are correctly rounded float32 operations, and the result
 * is rounded to bf16 (to nearest even) before it is stored or quantised.  The
 * FP8 scale and the quotients x / scale are correctly rounded float32
 * divisions, the quotients clamped to [-448, 448] and rounded to the nearest
 * e4m3fn value (ties to even).
 *
 *   num_tokens:      T >= 0 (0: nothing is enqueued).
 *   num_heads:       H >= 1.
 *   kv_dtype:        mla_kv_dtype of the pool.
 *   q_nope:          bf16 [T, H, 128] device, the no-RoPE query parts.
 *   q_rope_in:       bf16 [T, H, 64] device, the RoPE query parts before rotation.
 *   w_kc_t:          bf16 [H, 512, 128] device: every head's w_kc transposed,
 *                    element (h, n, k) = w_kc[h, k, n] (laid out once when the
 *                    weights are loaded, so that both MFMA operands read rows
 *                    with k contiguous).
 *   c_kv_new:        bf16 [T, 512] device, the new tokens' latent.
 *   k_rope_new:      bf16 [T, 64] device, their RoPE key parts before rotation.
 *   positions:       int32 [T] device, each token's position (row of cos_sin);
 *                    values outside [0, max_pos) are clamped into it.
 *   cos_sin:         fp32 [max_pos, 64] device: cos of the 32 frequencies, then
 *                    their sin, for every position (the caller's choice of base
 *                    and scaling).
 *   slots:           int32 [T] device, the pool slot of each new token's row;
 *                    a slot outside [0, num_slots) is not stored (for example
 *                    a token that another DCP shard holds).  Slots must be
 *                    distinct.
 *   q_nope_absorbed: bf16 [T, H, 512] device output.
 *   q_rope_out:      bf16 [T, H, 64] device output (must not alias q_rope_in).
 *   kv_pool:         [num_slots, 576] device pool (as for mla_decode; FP4:
 *                    [num_slots, 336], MXFP8: [num_slots, 608] bytes), written
 *                    at the stored slots only.
 *   kv_scale:        fp32 [num_slots] device for FP8 pools (written at the
 *                    stored slots), NULL for the other formats.
 *   stream:          HIP stream, 0 = default stream.
 *
 * All pointers 16-byte aligned (kv_scale 4-byte).  Errors are detected on the
 * host and returned before anything is enqueued.
 */
mla_status mla_prepare(int32_t num_tokens, int32_t num_heads, int32_t kv_dtype,
                       const void* q_nope, const void* q_rope_in, const void* w_kc_t,
                       const void* c_kv_new, const void* k_rope_new, const int32_t* positions,
                       const float* cos_sin, int32_t max_pos, const int32_t* slots,
                       void* q_nope_absorbed, void* q_rope_out, void* kv_pool, float* kv_scale,
                       int64_t num_slots, void* stream);

/*
 * LSE merge fused with the w_vc up-projection: the step after mla_decode
 * (DP16-vs-DP2 page: kv_b_proj is absorbed into w_kc / w_vc, so w_vc is
 * applied after attention in the latent space; section "MLA": the per-shard
 * (O, LSE) are merged by LSE, dcp_lse_combine).  For every token t and head
 * h, the num_parts partial results are merged as in mla_lse_combine and the
 * merged latent O (rounded to bf16, never stored) is projected:
 *
 *   out[t, h, n] = sum_k O[t, h, k] * w_vc[h, k, n]   (k < 512, n < 128),
 *
 * with fp32 accumulation, rounded to bf16.  A row whose parts all have
 * LSE = -inf gives out = 0 and LSE = -inf.  With num_parts = 1 this is the
 * plain projection of one decode output.
 *
 *   part_o:    fp32 [num_parts, T, H, 512] device (e.g. the stacked outputs of
 *              the DCP shards' mla_decode calls).
 *   part_lse:  fp32 [num_parts, T, H] device.
 *   w_vc_t:    bf16 [H, 128, 512] device: every head's w_vc transposed, element
 *              (h, n, k) = w_vc[h, k, n] (laid out once when the weights are
 *              loaded, so that the MFMA operand reads rows with k contiguous).
 *   out_v:     bf16 [T, H, 128] device output (the value heads o_proj reads).
 *   lse:       fp32 [T, H] device output of the merged LSE, or NULL.
 *   num_parts >= 1, num_tokens >= 0 (0: nothing is enqueued), num_heads >= 1;
 *   16-byte aligned pointers (lse 4-byte).
 */
mla_status mla_lse_combine_project(const float* part_o, const float* part_lse, int32_t num_parts,
                                   int32_t num_tokens, int32_t num_heads, const void* w_vc_t,
                                   void* out_v, float* lse, void* stream);

/* Static description of a status code. */
const char* mla_status_string(mla_status status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
