/*
 * hstu.h -- C ABI of the MI355X (gfx950) fused HSTU attention forward.
 *
 * Operation (RecOps Running Case Documentation, HSTU_V1 forward operator
 * page: the feature table's attention row, the operator introduction and the
 * inputs/outputs table). For every query head h and every query token i of
 * sequence b, with kv head hk = floor(h * num_heads_kv / num_heads_q):
 *
 *   O[i, h, :] = out_scale * sum_{j visible to i}
 *                  silu(alpha * (Q[i,h,:] . K[j,hk,:] + rab[b,h,i,j])) * V[j,hk,:]
 *
 * with silu(x) = x / (1 + exp(-x)). There is no softmax and no running max.
 * The page leaves three placements open; this library reads them as:
 * rab is added before alpha scales, the page's silu_scale is out_scale and
 * multiplies after SiLU, and P = silu(...) is rounded to the input dtype
 * before the product with V (fp32 accumulation throughout).
 *
 * Masks (the page's mask_type codes): HSTU_MASK_CAUSAL (0) is the built-in
 * lower-triangular mask with context and targets; HSTU_MASK_NONE (2) is the
 * bidirectional case; HSTU_MASK_CUSTOM (3) takes the user's mask tensor
 * (the table's mask input, [B, N, S, S] in the dtype of q): every key of
 * the sequence is a candidate, the mask value m for (i, j) multiplies P,
 * and m == 0 removes the key entirely (it contributes exactly zero whatever
 * its score, as with the built-in masks). Code 1 (upper triangular, which
 * the page itself does not support) returns HSTU_ERR_UNSUPPORTED.
 * For HSTU_MASK_CAUSAL, per sequence of length L with nc = num_context[b],
 * nt = num_targets[b] (0 when the array is NULL) and g = target_group_size:
 * clamp nt to [0, L], H = L - nt, clamp nc to [0, H]. Key j < H is visible to
 * query i iff j <= i, or both i and j are context tokens (< nc). Key j >= H
 * (a target) is visible iff j <= i when g == 0; when g >= 1 only if i is a
 * target of the same group of g consecutive targets and j <= i.
 * Local mask (feature table, local-mask row, which names the feature
 * without defining it; read here as a sliding window): with local_window
 * W >= 1, key j is visible to query i only if the causal mask above allows
 * it and i - j < W. The window bounds every pair alike (context, history and
 * targets); W = 0 means no window. It is taken with HSTU_MASK_CAUSAL only.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE memory owned by the caller. The library
 *    never allocates, frees, retains or reads them on the host, and never
 *    synchronises: work is enqueued on `stream` and the call returns.
 *  - Tensors are contiguous, row-major, 16-byte aligned.
 *  - Integer side inputs are int32 device arrays.
 *  - `workspace` is caller-allocated device memory of at least the size the
 *    matching *_workspace_size call returns; its contents need no
 *    initialisation and are scratch after the call. Calls that share one
 *    workspace must be ordered on one stream.
 *  - Validity of device arrays (offsets non-decreasing from 0, every length
 *    <= max_seq_len, queries never more than their keys, last_page_len in
 *    [1, page_size], page ids in range) is the caller's duty, as the page
 *    says for seq_offsets. With HSTU_VALIDATE=1 in the environment (a debug
 *    mode, read at every call) each call first checks all of these but the
 *    page ids on the device, waits for the stream, and returns
 *    HSTU_ERR_INVALID_ARG without launching the forward kernels when one
 *    fails. That mode synchronises, so it cannot be used under graph
 *    capture; by default nothing is checked and nothing waits.
 *  - Return codes only; nothing is thrown across the ABI.
 *  - batch is at most 2048 (the page's B range).
 *  - If batch, num_heads_q or head_dim is 0 the input is empty: the call
 *    returns HSTU_OK and launches nothing (the page's note on empty inputs).
 */
#ifndef HSTU_H_
#define HSTU_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HSTU_OK = 0,
  HSTU_ERR_INVALID_ARG = 1, /* bad size, null required pointer, misaligned pointer, bad combination */
  HSTU_ERR_UNSUPPORTED = 2, /* valid per the page but not built here (mask code 1, the user mask in f32 or
                               paged, head_dim, page_size) */
  HSTU_ERR_WORKSPACE = 3,   /* workspace missing or smaller than *_workspace_size */
  HSTU_ERR_HIP = 4          /* a HIP launch failed; the HIP error is left for hipGetLastError */
} hstu_status_t;

/* HSTU_FP8_E4M3 is the FP8 cast (the feature table's FP8 quantization row,
 * "cast": element-level quantization with no scale): q, k and v are OCP
 * E4M3 (FN) bytes (1 byte per element: sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, largest finite value 448, no infinities); both products
 * run on E4M3 operands with fp32 accumulation; P = silu(alpha * S) is cast
 * to E4M3 (nearest, ties to even, saturating at +-448) before the product
 * with V; out is bf16. Supported for jagged calls with head_dim 128,
 * without rab, the user mask or seq_offsets_k. */
typedef enum { HSTU_F32 = 0, HSTU_F16 = 1, HSTU_BF16 = 2, HSTU_FP8_E4M3 = 3 } hstu_dtype_t;

typedef enum { HSTU_MASK_CAUSAL = 0, HSTU_MASK_NONE = 2, HSTU_MASK_CUSTOM = 3 } hstu_mask_t;

/* Supported sizes: batch in [0, 2048] (the page's B range; larger batches
 * return HSTU_ERR_INVALID_ARG and a workspace size of 0); head_dim in
 * {32, 64, 128, 256} for f16/bf16, {32, 64, 128} for f32 and 128 for
 * FP8 (the page allows multiples of 16 up to 512); num_heads_q % num_heads_kv == 0 (the
 * page's GQA rule); page_size in {32, 64, 128, 256}; max_seq_len in
 * [1, 20480]; rab and user-mask head counts 1 or num_heads_q; the user mask
 * (HSTU_MASK_CUSTOM) in f16/bf16 jagged calls. */

/*
 * Workspace bytes hstu_fwd needs for these sizes (the work list of the tile
 * scheduler and its queue counters; with is_delta_qk != 0, the page's flag
 * for different Q and K lengths, i.e. calls that pass seq_offsets_k, also the
 * fp32 partial sums of items split over the key range). Returns 0 for
 * invalid sizes.
 */
size_t hstu_fwd_workspace_size(int32_t batch, int32_t max_seq_len, int32_t num_heads_q, int32_t num_heads_kv,
                               int32_t head_dim, hstu_dtype_t dtype, int32_t is_delta_qk);

/*
 * Jagged forward (the page's "jagged" layout: q/k/v [T, N, D] addressed by
 * seq_offsets, and seq_offsets_k with is_delta_qk when Q and K lengths
 * differ).
 *  q             [Tq, num_heads_q,  head_dim]  dtype  (Tq = seq_offsets[batch])
 *  k, v          [Tk, num_heads_kv, head_dim]  dtype  (Tk = seq_offsets_k[batch])
 *  rab           [batch, rab_num_heads, max_seq_len, max_seq_len] dtype, or
 *                NULL. rab_num_heads is num_heads_q or 1 (the page's rab
 *                broadcast [b, 1, s, s]: one rab for every head). Indexed by
 *                absolute positions (i, j) within the sequence. Entries the
 *                mask removes may be loaded (whole tile rows are read) but
 *                never affect the output, even when they hold NaN or inf.
 *                Rows past the sequence are never read. When max_seq_len is
 *                a multiple of 8, columns past the sequence may be read too
 *                (in 16-byte chunks, never past the row's end), with the
 *                same guarantee; otherwise they are never read.
 *  mask          [batch, mask_num_heads, max_seq_len, max_seq_len] dtype with
 *                HSTU_MASK_CUSTOM, else NULL. mask_num_heads is num_heads_q or
 *                1; indexed and read as rab (masked entries and columns
 *                past the sequence never affect the output). f16/bf16 only.
 *  out           [Tq, num_heads_q, head_dim]   dtype, bf16 for HSTU_FP8_E4M3
 *                (written for every query)
 *  seq_offsets   [batch + 1] int32, non-decreasing, seq_offsets[0] == 0.
 *  seq_offsets_k [batch + 1] int32, or NULL (keys = queries). When given, the
 *                Lq = seq_offsets[b+1] - seq_offsets[b] queries of sequence b
 *                are its last Lq positions among Lk = seq_offsets_k[b+1] -
 *                seq_offsets_k[b] keys (query t at absolute position
 *                Lk - Lq + t); Lq <= Lk is the caller's duty (queries past Lk
 *                are left unwritten). Masks and rab use absolute positions.
 *  num_context, num_targets [batch] int32, or NULL (= all zero). Must be
 *                NULL unless mask_type is HSTU_MASK_CAUSAL.
 *  target_group_size >= 0 (0 = no target mask).
 *  local_window  >= 0: the local mask's window W (0 = none); nonzero only
 *                with HSTU_MASK_CAUSAL.
 *  alpha         scale applied to (Q.K^T + rab) before SiLU.
 *  out_scale     scale applied after SiLU (the page's silu_scale; its default
 *                is 1/max_seq_len, applied by the Python binding).
 * Errors: HSTU_ERR_INVALID_ARG for negative sizes, num_heads_q not a
 * multiple of num_heads_kv, null q/k/v/out/seq_offsets, pointers not 16-byte
 * aligned, num_context/num_targets or local_window > 0 with a mask other
 * than causal, a mask without HSTU_MASK_CUSTOM or HSTU_MASK_CUSTOM without a
 * mask, rab or mask head counts other than 1 and num_heads_q,
 * target_group_size < 0, local_window < 0 or an unknown mask code; HSTU_ERR_UNSUPPORTED for mask code 1, head_dim, dtype,
 * HSTU_MASK_CUSTOM in f32, or HSTU_FP8_E4M3 with rab, the user mask or
 * seq_offsets_k; HSTU_ERR_WORKSPACE if workspace_bytes is too small;
 * HSTU_ERR_HIP if a launch fails.
 */
hstu_status_t hstu_fwd(const void* q, const void* k, const void* v, const void* rab, const void* mask, void* out,
                       const int32_t* seq_offsets, const int32_t* seq_offsets_k, const int32_t* num_context,
                       const int32_t* num_targets, int32_t batch, int32_t max_seq_len, int32_t num_heads_q,
                       int32_t num_heads_kv, int32_t head_dim, int32_t rab_num_heads, int32_t mask_num_heads,
                       hstu_mask_t mask_type, int32_t target_group_size, int32_t local_window, float alpha,
                       float out_scale, hstu_dtype_t dtype, void* workspace, size_t workspace_bytes,
                       void* stream /* hipStream_t */);

/*
 * hstu_fwd in two steps, for callers that time or reuse them separately
 * (the work list depends only on the sequence layout and mask inputs, so
 * stacked layers over the same batch can plan once and run many times).
 *
 * hstu_fwd_plan: the tile scheduler alone. It reads seq_offsets,
 * seq_offsets_k, num_context and num_targets on the device and writes into
 * `workspace` a work list of (sequence, query tile) items, longest first (by
 * the number of key tiles not fully masked), plus the queue counters the run
 * consumes. Arguments and errors as hstu_fwd (q, k, v, rab, mask and out are
 * not needed).
 *
 * hstu_fwd_run: the fused forward kernel alone, consuming the plan held in
 * `workspace`. The caller guarantees that the plan was made with the same
 * seq_offsets / seq_offsets_k contents, num_context, num_targets, batch,
 * max_seq_len, head counts, head_dim, mask_type, target_group_size,
 * local_window and dtype, and that no other call uses the workspace between
 * the plan and the run. A run leaves the plan intact, so further runs may
 * follow.
 * hstu_fwd == plan + run.
 */
hstu_status_t hstu_fwd_plan(const int32_t* seq_offsets, const int32_t* seq_offsets_k, const int32_t* num_context,
                            const int32_t* num_targets, int32_t batch, int32_t max_seq_len, int32_t num_heads_q,
                            int32_t num_heads_kv, int32_t head_dim, hstu_mask_t mask_type, int32_t target_group_size,
                            int32_t local_window, hstu_dtype_t dtype, void* workspace, size_t workspace_bytes,
                            void* stream /* hipStream_t */);

hstu_status_t hstu_fwd_run(const void* q, const void* k, const void* v, const void* rab, const void* mask, void* out,
                           const int32_t* seq_offsets, const int32_t* seq_offsets_k, const int32_t* num_context,
                           const int32_t* num_targets, int32_t batch, int32_t max_seq_len, int32_t num_heads_q,
                           int32_t num_heads_kv, int32_t head_dim, int32_t rab_num_heads, int32_t mask_num_heads,
                           hstu_mask_t mask_type, int32_t target_group_size, int32_t local_window, float alpha,
                           float out_scale, hstu_dtype_t dtype, void* workspace, size_t workspace_bytes,
                           void* stream /* hipStream_t */);

/*
 * Workspace bytes hstu_fwd_paged needs. max_seq_len bounds history + new
 * tokens of every request. Returns 0 for invalid sizes.
 */
size_t hstu_fwd_paged_workspace_size(int32_t batch, int32_t page_size, int32_t max_seq_len, int32_t num_heads_q,
                                     int32_t num_heads_kv, int32_t head_dim, hstu_dtype_t dtype);

/*
 * Paged-KV forward (the page's Page feature row and its kv_cache,
 * page_offsets, page_ids and last_page_len inputs). The cache holds each
 * request's history; the new tokens bring their own K/V.
 *  q              [Tq, num_heads_q, head_dim]   new tokens' queries (Tq = seq_offsets_q[batch])
 *  k_new, v_new   [Tq, num_heads_kv, head_dim]  new tokens' keys/values
 *  out            [Tq, num_heads_q, head_dim]
 *  seq_offsets_q  [batch + 1] int32: new tokens per request.
 *  kv_cache       [num_pages, 2, page_size, num_heads_kv, head_dim]: [p,0] = K, [p,1] = V.
 *  page_offsets   [batch + 1] int32; page_ids [page_offsets[batch]] int32;
 *  last_page_len  [batch] int32 in [1, page_size]. Request b's history has
 *                 (n_pages - 1) * page_size + last_page_len[b] tokens (0 if
 *                 it owns no page).
 * Query t of request b sits at absolute position history_len + t of a
 * sequence of history_len + Tq_b tokens; the mask (num_context, num_targets,
 * target_group_size) is applied on those absolute positions. No rab and no
 * user mask. Errors as hstu_fwd, plus HSTU_ERR_UNSUPPORTED for page_size
 * outside {32, 64, 128, 256}, for HSTU_MASK_CUSTOM and for HSTU_FP8_E4M3.
 */
hstu_status_t hstu_fwd_paged(const void* q, const void* k_new, const void* v_new, void* out,
                             const int32_t* seq_offsets_q, const void* kv_cache, const int32_t* page_offsets,
                             const int32_t* page_ids, const int32_t* last_page_len, const int32_t* num_context,
                             const int32_t* num_targets, int32_t batch, int32_t page_size, int32_t max_seq_len,
                             int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, hstu_mask_t mask_type,
                             int32_t target_group_size, int32_t local_window, float alpha, float out_scale,
                             hstu_dtype_t dtype, void* workspace, size_t workspace_bytes,
                             void* stream /* hipStream_t */);

/* hstu_fwd_paged in two steps, with the same contract as hstu_fwd_plan /
 * hstu_fwd_run. The plan reads seq_offsets_q, page_offsets, last_page_len,
 * num_context and num_targets; q, k_new, v_new, out, kv_cache and page_ids
 * are needed by the run only. */
hstu_status_t hstu_fwd_paged_plan(const int32_t* seq_offsets_q, const int32_t* page_offsets,
                                  const int32_t* last_page_len, const int32_t* num_context, const int32_t* num_targets,
                                  int32_t batch, int32_t page_size, int32_t max_seq_len, int32_t num_heads_q,
                                  int32_t num_heads_kv, int32_t head_dim, hstu_mask_t mask_type,
                                  int32_t target_group_size, int32_t local_window, hstu_dtype_t dtype, void* workspace,
                                  size_t workspace_bytes, void* stream /* hipStream_t */);

hstu_status_t hstu_fwd_paged_run(const void* q, const void* k_new, const void* v_new, void* out,
                                 const int32_t* seq_offsets_q, const void* kv_cache, const int32_t* page_offsets,
                                 const int32_t* page_ids, const int32_t* last_page_len, const int32_t* num_context,
                                 const int32_t* num_targets, int32_t batch, int32_t page_size, int32_t max_seq_len,
                                 int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, hstu_mask_t mask_type,
                                 int32_t target_group_size, int32_t local_window, float alpha, float out_scale,
                                 hstu_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                 void* stream /* hipStream_t */);

/*
 * hstu_fwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc. Arguments, results and errors are those
 * of hstu_fwd. The tile scheduler's work list, queue counters and partial
 * sums live in a static 16 MiB array of the library's own device memory
 * (one per GPU, held until the process ends; its address is taken once per
 * device). The call allocates nothing and frees nothing. The stream must
 * belong to the current device. Calls with separate key offsets get as
 * many partial-sum slots as fit, so their key chunks may be longer than
 * hstu_fwd's (same results up to fp32 summation order). Sizes whose work
 * list does not fit (in practice batch * ceil(max_seq_len / rows per item)
 * beyond about 2 million entries) return HSTU_ERR_WORKSPACE. Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other threads) race and must be ordered by the caller.
 */
hstu_status_t hstu_fwd_noalloc(const void* q, const void* k, const void* v, const void* rab, const void* mask,
                               void* out, const int32_t* seq_offsets, const int32_t* seq_offsets_k,
                               const int32_t* num_context, const int32_t* num_targets, int32_t batch,
                               int32_t max_seq_len, int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                               int32_t rab_num_heads, int32_t mask_num_heads, hstu_mask_t mask_type,
                               int32_t target_group_size, int32_t local_window, float alpha, float out_scale,
                               hstu_dtype_t dtype, void* stream /* hipStream_t */);

/* Static description of a status code. Never NULL. */
const char* hstu_status_string(hstu_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_H_ */
