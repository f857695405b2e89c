// Internal launch interface between the C ABI (hstu_abi.cpp) and the gfx950
// kernels (hstu_kernels.hip). Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hstu {

// FP8: q, k, v in OCP E4M3 (FN), out in bf16.
enum class DType : int { F32 = 0, F16 = 1, BF16 = 2, FP8 = 3 };

// Everything one forward launch needs. Pointers are device memory.
struct FwdArgs {
  DType dtype;
  bool causal;
  bool paged;
  bool user_mask;  // mask_type 3: the mask tensor decides (causal is false)
  const void* q;
  const void* k;  // jagged: k; paged: k_new
  const void* v;  // jagged: v; paged: v_new
  const void* rab;
  const void* mask;            // user mask [B, mask_heads, S, S] (user_mask only)
  void* out;
  const int32_t* seq_offsets;  // jagged: [B+1]; paged: new tokens per request [B+1]
  const int32_t* seq_offsets_k;  // jagged keys [B+1], or NULL (the same as seq_offsets)
  const int32_t* num_context;
  const int32_t* num_targets;
  const void* kv_cache;
  const int32_t* page_offsets;
  const int32_t* page_ids;
  const int32_t* last_page_len;
  int32_t page_size;
  int32_t batch;
  int32_t max_seq_len;
  int32_t num_heads_q;
  int32_t num_heads_kv;
  int32_t head_dim;
  int32_t rab_heads;   // 1 (one rab for every head) or num_heads_q
  int32_t mask_heads;  // 1 or num_heads_q
  int32_t target_group_size;
  int32_t local_window;  // local mask window W (causal only), 0: none
  float alpha;
  float out_scale;
  void* workspace;
  size_t workspace_bytes;
  size_t workspace_cap;  // 0, or the fixed size of the static scratch (see fwd_workspace_bytes)
  hipStream_t stream;
};

// Bytes of workspace a launch needs: work list, queue counters and, when
// the launch may split long items over the key range (split_keys: paged
// calls and jagged calls with their own key offsets), the split list and
// the fp32 partial sums.
// cap > 0 sizes the layout for a workspace of at most cap bytes (fewer
// partial-sum slots for split items); the result may still exceed cap.
size_t fwd_workspace_bytes(int32_t batch, int32_t max_q_len, int32_t num_heads_q, int32_t num_heads_kv,
                           int32_t head_dim, DType dtype, bool split_keys, size_t cap = 0);

// The static device scratch of the allocation-free entry point on the
// current device: *ptr receives its device address (taken once per device
// with hipGetSymbolAddress), *bytes its size. Allocates nothing.
hipError_t scratch_workspace(void** ptr, size_t* bytes);

// Enqueues the validation kernel on args.stream: it writes 1 to *flag
// (device memory) if the device-side offsets, lengths or page counters
// break the rules the page leaves to the caller, else 0.
hipError_t launch_validate(const FwdArgs& args, int32_t* flag);

// Enqueues the planner on args.stream: it writes the work list into the
// workspace and zeroes the work-queue counters.
hipError_t launch_plan(const FwdArgs& args);

// Enqueues the forward kernel (and, for plans with split items, the split
// reduction kernel) on args.stream; it consumes the work list the planner
// left in the workspace (same sizes and mask inputs) and leaves the queue
// counters at zero when it ends, so one plan serves many runs.
hipError_t launch_run(const FwdArgs& args);

}  // namespace hstu
