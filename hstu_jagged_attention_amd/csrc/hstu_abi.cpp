// C ABI of the fused HSTU forward: argument checks, workspace sizing and
// dispatch to the gfx950 kernels. Argument rules follow the inputs/outputs
// table of the HSTU_V1 forward operator page (RecOps Running Case
// Documentation): shape ranges, the GQA divisibility rule, the mask_type
// codes, page_size, and the rule that an empty dimension means the
// operator does not run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdlib>

#include "hstu.h"
#include "hstu_internal.h"

namespace {

constexpr int32_t kMaxSeqLen = 20480;
// The page's batch bound (B in [1, 2048]). The scheduler also relies on it:
// a work-list entry packs the sequence index into 16 bits.
constexpr int32_t kMaxBatch = 2048;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool dtype_ok(hstu_dtype_t dt) { return dt == HSTU_F32 || dt == HSTU_F16 || dt == HSTU_BF16 || dt == HSTU_FP8_E4M3; }

bool head_dim_ok(int32_t d, hstu_dtype_t dt) {
  if (dt == HSTU_F32) return d == 32 || d == 64 || d == 128;
  if (dt == HSTU_FP8_E4M3) return d == 128;
  return d == 32 || d == 64 || d == 128 || d == 256;
}

bool page_size_ok(int32_t ps) { return ps == 32 || ps == 64 || ps == 128 || ps == 256; }

hstu::DType to_internal(hstu_dtype_t dt) {
  switch (dt) {
    case HSTU_F32: return hstu::DType::F32;
    case HSTU_F16: return hstu::DType::F16;
    case HSTU_FP8_E4M3: return hstu::DType::FP8;
    default: return hstu::DType::BF16;
  }
}

// Checks shared by both entry points. Returns HSTU_OK or the error.
hstu_status_t check_common(int32_t batch, int32_t max_seq_len, int32_t hq, int32_t hk, int32_t d, hstu_mask_t mask,
                           int32_t group_size, int32_t local_window, hstu_dtype_t dtype, const int32_t* num_context,
                           const int32_t* num_targets) {
  if (batch < 0 || hq < 0 || d < 0 || hk < 0 || max_seq_len < 0 || group_size < 0 || local_window < 0)
    return HSTU_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return HSTU_ERR_UNSUPPORTED;
  if (mask != HSTU_MASK_CAUSAL && mask != HSTU_MASK_NONE && mask != HSTU_MASK_CUSTOM) {
    return mask == 1 ? HSTU_ERR_UNSUPPORTED : HSTU_ERR_INVALID_ARG;
  }
  if (batch == 0 || hq == 0 || d == 0) return HSTU_OK;  // empty input: nothing runs
  if (batch > kMaxBatch) return HSTU_ERR_INVALID_ARG;
  if (hk <= 0 || hq % hk != 0) return HSTU_ERR_INVALID_ARG;
  if (max_seq_len < 1 || max_seq_len > kMaxSeqLen) return HSTU_ERR_INVALID_ARG;
  if (!head_dim_ok(d, dtype)) return HSTU_ERR_UNSUPPORTED;
  if (mask != HSTU_MASK_CAUSAL && (num_context || num_targets || local_window > 0)) return HSTU_ERR_INVALID_ARG;
  if ((num_context && !aligned4(num_context)) || (num_targets && !aligned4(num_targets))) return HSTU_ERR_INVALID_ARG;
  return HSTU_OK;
}

}  // namespace

extern "C" {

size_t hstu_fwd_workspace_size(int32_t batch, int32_t max_seq_len, int32_t num_heads_q, int32_t num_heads_kv,
                               int32_t head_dim, hstu_dtype_t dtype, int32_t is_delta_qk) {
  if (batch < 0 || max_seq_len < 0 || num_heads_q < 0 || num_heads_kv < 0 || head_dim < 0) return 0;
  if (batch == 0 || num_heads_q == 0 || head_dim == 0) return 256;
  if (batch > kMaxBatch || num_heads_kv == 0 || num_heads_q % num_heads_kv != 0 || !dtype_ok(dtype)) return 0;
  return hstu::fwd_workspace_bytes(batch, max_seq_len, num_heads_q, num_heads_kv, head_dim, to_internal(dtype),
                                   is_delta_qk != 0);
}

size_t hstu_fwd_paged_workspace_size(int32_t batch, int32_t page_size, int32_t max_seq_len, int32_t num_heads_q,
                                     int32_t num_heads_kv, int32_t head_dim, hstu_dtype_t dtype) {
  if (page_size < 0 || batch < 0 || max_seq_len < 0 || num_heads_q < 0 || num_heads_kv < 0 || head_dim < 0) return 0;
  if (batch == 0 || num_heads_q == 0 || head_dim == 0) return 256;
  if (batch > kMaxBatch || num_heads_kv == 0 || num_heads_q % num_heads_kv != 0 || !dtype_ok(dtype)) return 0;
  // New tokens per request are bounded by max_seq_len (history + new).
  return hstu::fwd_workspace_bytes(batch, max_seq_len, num_heads_q, num_heads_kv, head_dim, to_internal(dtype), true);
}

}  // extern "C"

namespace {

enum Phase { kPlan = 1, kRun = 2, kBoth = 3 };

// HSTU_VALIDATE=1 in the environment (read at every call) turns on the
// debug check of the device-side inputs: a validation kernel writes its
// result into the workspace header, the call waits for the stream
// and reads it, and returns HSTU_ERR_INVALID_ARG without launching the
// forward kernels when the inputs break the rules. Off by default: the
// library then never synchronises and never reads device memory.
bool validate_mode() {
  const char* v = std::getenv("HSTU_VALIDATE");
  return v && v[0] == '1' && v[1] == '\0';
}

hstu_status_t validate(const hstu::FwdArgs& a) {
  // An unused word of the workspace header (its first 64-byte line holds
  // only the plan's item count, in word 0).
  int32_t* flag = reinterpret_cast<int32_t*>(static_cast<char*>(a.workspace) + 32);
  if (hstu::launch_validate(a, flag) != hipSuccess) return HSTU_ERR_HIP;
  int32_t host = 1;
  if (hipMemcpyAsync(&host, flag, sizeof(host), hipMemcpyDeviceToHost, a.stream) != hipSuccess) return HSTU_ERR_HIP;
  if (hipStreamSynchronize(a.stream) != hipSuccess) return HSTU_ERR_HIP;
  return host == 0 ? HSTU_OK : HSTU_ERR_INVALID_ARG;
}

hstu_status_t enqueue(const hstu::FwdArgs& a, int phase) {
  if (validate_mode()) {
    const hstu_status_t st = validate(a);
    if (st != HSTU_OK) return st;
  }
  if ((phase & kPlan) && hstu::launch_plan(a) != hipSuccess) return HSTU_ERR_HIP;
  if ((phase & kRun) && hstu::launch_run(a) != hipSuccess) return HSTU_ERR_HIP;
  return HSTU_OK;
}

// Jagged entry points share this body. Pointers a run does not need (q, k,
// v, out) may be NULL in the plan-only phase.
// scratch: the workspace is the library's static device scratch (the
// allocation-free entry point); its layout is then sized to fit it.
hstu_status_t jagged(int phase, const void* q, const void* k, const void* v, const void* rab, const void* mask,
                     void* out, const int32_t* seq_offsets, const int32_t* seq_offsets_k, const int32_t* num_context,
                     const int32_t* num_targets, int32_t batch, int32_t max_seq_len, int32_t num_heads_q,
                     int32_t num_heads_kv, int32_t head_dim, int32_t rab_num_heads, int32_t mask_num_heads,
                     hstu_mask_t mask_type, int32_t target_group_size, int32_t local_window, float alpha,
                     float out_scale, hstu_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream,
                     bool scratch = false) {
  hstu_status_t st = check_common(batch, max_seq_len, num_heads_q, num_heads_kv, head_dim, mask_type,
                                  target_group_size, local_window, dtype, num_context, num_targets);
  if (st != HSTU_OK) return st;
  if (batch == 0 || num_heads_q == 0 || head_dim == 0) return HSTU_OK;
  if (mask_type == HSTU_MASK_CUSTOM && dtype == HSTU_F32) return HSTU_ERR_UNSUPPORTED;
  // The FP8 cast is built for jagged calls with equal Q and K lengths,
  // without rab or the user mask.
  if (dtype == HSTU_FP8_E4M3 && (mask_type == HSTU_MASK_CUSTOM || seq_offsets_k || rab)) return HSTU_ERR_UNSUPPORTED;
  if (!seq_offsets || !aligned4(seq_offsets) || (seq_offsets_k && !aligned4(seq_offsets_k)))
    return HSTU_ERR_INVALID_ARG;
  if (phase & kRun) {
    if (!q || !k || !v || !out) return HSTU_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || (rab && !aligned16(rab)))
      return HSTU_ERR_INVALID_ARG;
    // The user mask comes with mask_type 3 and only then.
    if ((mask_type == HSTU_MASK_CUSTOM) != (mask != nullptr) || (mask && !aligned16(mask)))
      return HSTU_ERR_INVALID_ARG;
    if (rab && rab_num_heads != 1 && rab_num_heads != num_heads_q) return HSTU_ERR_INVALID_ARG;
    if (mask && mask_num_heads != 1 && mask_num_heads != num_heads_q) return HSTU_ERR_INVALID_ARG;
  }
  const size_t need =
      scratch ? hstu::fwd_workspace_bytes(batch, max_seq_len, num_heads_q, num_heads_kv, head_dim,
                                          to_internal(dtype), seq_offsets_k != nullptr, workspace_bytes)
              : hstu_fwd_workspace_size(batch, max_seq_len, num_heads_q, num_heads_kv, head_dim, dtype,
                                        seq_offsets_k ? 1 : 0);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return HSTU_ERR_WORKSPACE;

  hstu::FwdArgs a{};
  a.dtype = to_internal(dtype);
  a.causal = mask_type == HSTU_MASK_CAUSAL;
  a.user_mask = mask_type == HSTU_MASK_CUSTOM;
  a.paged = false;
  a.q = q;
  a.k = k;
  a.v = v;
  a.rab = rab;
  a.mask = mask;
  a.out = out;
  a.seq_offsets = seq_offsets;
  a.seq_offsets_k = seq_offsets_k;
  a.rab_heads = rab_num_heads;
  a.mask_heads = mask_num_heads;
  a.num_context = num_context;
  a.num_targets = num_targets;
  a.batch = batch;
  a.max_seq_len = max_seq_len;
  a.num_heads_q = num_heads_q;
  a.num_heads_kv = num_heads_kv;
  a.head_dim = head_dim;
  a.target_group_size = target_group_size;
  a.local_window = local_window;
  a.alpha = alpha;
  a.out_scale = out_scale;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  a.workspace_cap = scratch ? workspace_bytes : 0;
  a.stream = reinterpret_cast<hipStream_t>(stream);
  return enqueue(a, phase);
}

hstu_status_t paged(int phase, const void* q, const void* k_new, const void* v_new, void* out,
                    const int32_t* seq_offsets_q, const void* kv_cache, const int32_t* page_offsets,
                    const int32_t* page_ids, const int32_t* last_page_len, const int32_t* num_context,
                    const int32_t* num_targets, int32_t batch, int32_t page_size, int32_t max_seq_len,
                    int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, hstu_mask_t mask_type,
                    int32_t target_group_size, int32_t local_window, float alpha, float out_scale, hstu_dtype_t dtype,
                    void* workspace, size_t workspace_bytes, void* stream) {
  hstu_status_t st = check_common(batch, max_seq_len, num_heads_q, num_heads_kv, head_dim, mask_type,
                                  target_group_size, local_window, dtype, num_context, num_targets);
  if (st != HSTU_OK) return st;
  if (mask_type == HSTU_MASK_CUSTOM) return HSTU_ERR_UNSUPPORTED;  // the user mask is built for jagged calls
  if (dtype == HSTU_FP8_E4M3 && batch > 0 && num_heads_q > 0 && head_dim > 0)
    return HSTU_ERR_UNSUPPORTED;  // the FP8 cast is built for jagged calls
  if (page_size < 0) return HSTU_ERR_INVALID_ARG;
  if (batch == 0 || num_heads_q == 0 || head_dim == 0) return HSTU_OK;
  if (!page_size_ok(page_size)) return HSTU_ERR_UNSUPPORTED;
  if (!seq_offsets_q || !page_offsets || !last_page_len) return HSTU_ERR_INVALID_ARG;
  if (!aligned4(seq_offsets_q) || !aligned4(page_offsets) || !aligned4(last_page_len)) return HSTU_ERR_INVALID_ARG;
  if (phase & kRun) {
    if (!q || !k_new || !v_new || !out || !kv_cache || !page_ids) return HSTU_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out) || !aligned16(kv_cache) ||
        !aligned4(page_ids))
      return HSTU_ERR_INVALID_ARG;
  }
  const size_t need =
      hstu_fwd_paged_workspace_size(batch, page_size, max_seq_len, num_heads_q, num_heads_kv, head_dim, dtype);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return HSTU_ERR_WORKSPACE;

  hstu::FwdArgs a{};
  a.dtype = to_internal(dtype);
  a.causal = mask_type == HSTU_MASK_CAUSAL;
  a.paged = true;
  a.q = q;
  a.k = k_new;
  a.v = v_new;
  a.rab = nullptr;
  a.out = out;
  a.seq_offsets = seq_offsets_q;
  a.num_context = num_context;
  a.num_targets = num_targets;
  a.kv_cache = kv_cache;
  a.page_offsets = page_offsets;
  a.page_ids = page_ids;
  a.last_page_len = last_page_len;
  a.page_size = page_size;
  a.batch = batch;
  a.max_seq_len = max_seq_len;
  a.num_heads_q = num_heads_q;
  a.num_heads_kv = num_heads_kv;
  a.head_dim = head_dim;
  a.target_group_size = target_group_size;
  a.local_window = local_window;
  a.alpha = alpha;
  a.out_scale = out_scale;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  a.stream = reinterpret_cast<hipStream_t>(stream);
  return enqueue(a, phase);
}

}  // namespace

extern "C" {

hstu_status_t hstu_fwd(const void* q, const void* k, const void* v, const void* rab, const void* mask, void* out,
                       const int32_t* seq_offsets, const int32_t* seq_offsets_k, const int32_t* num_context,
                       const int32_t* num_targets, int32_t batch, int32_t max_seq_len, int32_t num_heads_q,
                       int32_t num_heads_kv, int32_t head_dim, int32_t rab_num_heads, int32_t mask_num_heads,
                       hstu_mask_t mask_type, int32_t target_group_size, int32_t local_window, float alpha,
                       float out_scale, hstu_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return jagged(kBoth, q, k, v, rab, mask, out, seq_offsets, seq_offsets_k, num_context, num_targets, batch,
                max_seq_len, num_heads_q, num_heads_kv, head_dim, rab_num_heads, mask_num_heads, mask_type,
                target_group_size, local_window, alpha, out_scale, dtype, workspace, workspace_bytes, stream);
}

hstu_status_t hstu_fwd_noalloc(const void* q, const void* k, const void* v, const void* rab, const void* mask,
                               void* out, const int32_t* seq_offsets, const int32_t* seq_offsets_k,
                               const int32_t* num_context, const int32_t* num_targets, int32_t batch,
                               int32_t max_seq_len, int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                               int32_t rab_num_heads, int32_t mask_num_heads, hstu_mask_t mask_type,
                               int32_t target_group_size, int32_t local_window, float alpha, float out_scale,
                               hstu_dtype_t dtype, void* stream) {
  // Empty inputs and argument errors are reported before the scratch is touched.
  hstu_status_t st = check_common(batch, max_seq_len, num_heads_q, num_heads_kv, head_dim, mask_type,
                                  target_group_size, local_window, dtype, num_context, num_targets);
  if (st != HSTU_OK || batch == 0 || num_heads_q == 0 || head_dim == 0) return st;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (hstu::scratch_workspace(&ws, &ws_bytes) != hipSuccess) return HSTU_ERR_HIP;
  return jagged(kBoth, q, k, v, rab, mask, out, seq_offsets, seq_offsets_k, num_context, num_targets, batch,
                max_seq_len, num_heads_q, num_heads_kv, head_dim, rab_num_heads, mask_num_heads, mask_type,
                target_group_size, local_window, alpha, out_scale, dtype, ws, ws_bytes, stream, true);
}

hstu_status_t hstu_fwd_plan(const int32_t* seq_offsets, const int32_t* seq_offsets_k, const int32_t* num_context,
                            const int32_t* num_targets, int32_t batch, int32_t max_seq_len, int32_t num_heads_q,
                            int32_t num_heads_kv, int32_t head_dim, hstu_mask_t mask_type, int32_t target_group_size,
                            int32_t local_window, hstu_dtype_t dtype, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return jagged(kPlan, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, seq_offsets, seq_offsets_k, num_context,
                num_targets, batch, max_seq_len, num_heads_q, num_heads_kv, head_dim, 0, 0, mask_type,
                target_group_size, local_window, 1.0f, 1.0f, dtype, workspace, workspace_bytes, stream);
}

hstu_status_t hstu_fwd_run(const void* q, const void* k, const void* v, const void* rab, const void* mask, void* out,
                           const int32_t* seq_offsets, const int32_t* seq_offsets_k, const int32_t* num_context,
                           const int32_t* num_targets, int32_t batch, int32_t max_seq_len, int32_t num_heads_q,
                           int32_t num_heads_kv, int32_t head_dim, int32_t rab_num_heads, int32_t mask_num_heads,
                           hstu_mask_t mask_type, int32_t target_group_size, int32_t local_window, float alpha,
                           float out_scale, hstu_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return jagged(kRun, q, k, v, rab, mask, out, seq_offsets, seq_offsets_k, num_context, num_targets, batch,
                max_seq_len, num_heads_q, num_heads_kv, head_dim, rab_num_heads, mask_num_heads, mask_type,
                target_group_size, local_window, alpha, out_scale, dtype, workspace, workspace_bytes, stream);
}

hstu_status_t hstu_fwd_paged(const void* q, const void* k_new, const void* v_new, void* out,
                             const int32_t* seq_offsets_q, const void* kv_cache, const int32_t* page_offsets,
                             const int32_t* page_ids, const int32_t* last_page_len, const int32_t* num_context,
                             const int32_t* num_targets, int32_t batch, int32_t page_size, int32_t max_seq_len,
                             int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, hstu_mask_t mask_type,
                             int32_t target_group_size, int32_t local_window, float alpha, float out_scale,
                             hstu_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return paged(kBoth, q, k_new, v_new, out, seq_offsets_q, kv_cache, page_offsets, page_ids, last_page_len,
               num_context, num_targets, batch, page_size, max_seq_len, num_heads_q, num_heads_kv, head_dim,
               mask_type, target_group_size, local_window, alpha, out_scale, dtype, workspace, workspace_bytes, stream);
}

hstu_status_t hstu_fwd_paged_plan(const int32_t* seq_offsets_q, const int32_t* page_offsets,
                                  const int32_t* last_page_len, const int32_t* num_context, const int32_t* num_targets,
                                  int32_t batch, int32_t page_size, int32_t max_seq_len, int32_t num_heads_q,
                                  int32_t num_heads_kv, int32_t head_dim, hstu_mask_t mask_type,
                                  int32_t target_group_size, int32_t local_window, hstu_dtype_t dtype, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return paged(kPlan, nullptr, nullptr, nullptr, nullptr, seq_offsets_q, nullptr, page_offsets, nullptr, last_page_len,
               num_context, num_targets, batch, page_size, max_seq_len, num_heads_q, num_heads_kv, head_dim, mask_type,
               target_group_size, local_window, 1.0f, 1.0f, dtype, workspace, workspace_bytes, stream);
}

hstu_status_t hstu_fwd_paged_run(const void* q, const void* k_new, const void* v_new, void* out,
                                 const int32_t* seq_offsets_q, const void* kv_cache, const int32_t* page_offsets,
                                 const int32_t* page_ids, const int32_t* last_page_len, const int32_t* num_context,
                                 const int32_t* num_targets, int32_t batch, int32_t page_size, int32_t max_seq_len,
                                 int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, hstu_mask_t mask_type,
                                 int32_t target_group_size, int32_t local_window, float alpha, float out_scale,
                                 hstu_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return paged(kRun, q, k_new, v_new, out, seq_offsets_q, kv_cache, page_offsets, page_ids, last_page_len,
               num_context, num_targets, batch, page_size, max_seq_len, num_heads_q, num_heads_kv, head_dim,
               mask_type, target_group_size, local_window, alpha, out_scale, dtype, workspace, workspace_bytes, stream);
}

const char* hstu_status_string(hstu_status_t status) {
  switch (status) {
    case HSTU_OK:
      return "HSTU_OK";
    case HSTU_ERR_INVALID_ARG:
      return "HSTU_ERR_INVALID_ARG: invalid argument";
    case HSTU_ERR_UNSUPPORTED:
      return "HSTU_ERR_UNSUPPORTED: valid but not supported by this library";
    case HSTU_ERR_WORKSPACE:
      return "HSTU_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case HSTU_ERR_HIP:
      return "HSTU_ERR_HIP: a HIP launch failed";
  }
  return "HSTU: unknown status";
}

}  // extern "C"
