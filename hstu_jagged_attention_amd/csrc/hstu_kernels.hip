// gfx950 (MI355X, CDNA4) kernels of the fused HSTU attention forward.
//
// Operation (RecOps Running Case Documentation, HSTU_V1 forward operator:
// feature table, operator introduction, inputs/outputs table): per query
// head, O = out_scale * (M .* silu(alpha * (Q K^T + rab))) V over jagged
// sequences, MHA or GQA, with the bidirectional mask, the causal mask built
// from num_context / num_targets / target_group_size, or the user's mask
// tensor (mask_type 3, whose values multiply P), optionally narrowed by a
// local window (the feature table's local-mask row: key j is visible to
// query i only when i - j < W as well); rab may be shared by all
// heads ([B, 1, S, S]); queries may be the last positions of longer key
// sequences (seq_offsets_k); and a paged variant reads history K/V from
// kv_cache pages. No softmax: partial sums over key tiles add exactly, so no
// running max or rescale is kept.
//
// Kernels per call, all on the caller's stream:
//  1. plan_kernel: one workgroup turns seq_offsets (and the mask inputs)
//     into the work list: one item per (sequence, query tile), costed by the
//     number of key tiles that are not fully masked, counting-sorted longest
//     first. It also zeroes the work-queue counter. Small batches skip it
//     (direct mode: workgroup w runs item w of the full grid).
//  2. fwd_kernel: persistent workgroups of 4 waves (8 in the key-split
//     variant) pop items from the queue in list order. A workgroup owns one
//     item and a group of query heads that share one kv head (1 head x 128
//     rows for MHA, up to 4 heads x 32 rows for GQA), so each K/V tile is
//     staged through LDS once for all of them. K/V tiles go global -> LDS by
//     DMA (no register staging), double buffered, into rows padded so every
//     fragment read is conflict-free. rab and the user mask go through a
//     ring of three LDS tiles by DMA, two tiles ahead, where LDS allows and
//     max_seq_len is a multiple of 8 (else into registers, one tile ahead).
//     Per key tile: S^T = K Q^T on MFMA (the
//     accumulator then holds one query per lane and 16 keys per lane), the
//     SiLU epilogue in registers, then O^T += V^T P^T on MFMA with P used
//     straight from the S^T registers as the B operand; the V^T A operand
//     comes from transposing LDS reads of the row-major V tile, taken in the
//     key order the S^T accumulator holds.
//  3. reduce_kernel (calls with split items only: paged, and jagged with
//     separate key offsets): items longer than the planner's chunk size run
//     as several key-range chunks that store fp32 partial O; this kernel
//     sums them in chunk order.
//  fwd_kernel_f32 is the fp32 path (v_mfma_f32_32x32x2f32, K/V staged
//  through registers).
//
// MFMA lane layouts (checked on the device): v_mfma_f32_32x32x16_{bf16,f16}
// takes A[m = lane%32][k = 8*(lane/32) + 0..7] and B[k = 8*(lane/32) + 0..7]
// [n = lane%32] and returns C[m = 8*(r/4) + 4*(lane/32) + r%4][n = lane%32]
// in register r; v_mfma_f32_32x32x2f32 takes one k per half-wave.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include <cmath>
#include <type_traits>

#include "hstu_internal.h"

namespace hstu {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kMaxBins = 1024;  // > max key tiles of one row (20480 / 32)
constexpr int kPlanThreads = 1024;
static_assert(kMaxBins == kPlanThreads, "the planner keeps one cost bin per thread");
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef _Float16 f16x8_t __attribute__((__vector_size__(16)));
typedef float f32x16_t __attribute__((__vector_size__(64)));
typedef float f32x4_t __attribute__((__vector_size__(16)));
typedef uint32_t u32x4_t __attribute__((__vector_size__(16)));
typedef uint32_t u32x2_t __attribute__((__vector_size__(8)));

// Kernel parameters (passed by value).
struct KParams {
  const void* q;
  const void* k;
  const void* v;
  const void* rab;
  const void* mask;   // user mask (mask_type 3), laid out as rab
  void* out;
  const int32_t* seq_offsets;
  const int32_t* seq_offsets_k;  // jagged keys, or NULL: the queries' offsets
  const int32_t* num_context;
  const int32_t* num_targets;
  const void* kv_cache;
  const int32_t* page_offsets;
  const int32_t* page_ids;
  const int32_t* last_page_len;
  int32_t* items;     // work list, two ints per entry (see the planner)
  int32_t* n_items;   // number of valid list entries
  float* partials;    // split items: fp32 partial O, one slot per (chunk, head group)
  int32_t* split_items;  // split items: four ints each (see the planner)
  int32_t* n_split;      // number of split items
  int32_t split_slots;   // partial-sum slots available (0: never split)
  int32_t target_chunks; // chunks the planner aims for (per resident workgroup: 1/2 paged, 1 jagged)
  int32_t* counter;   // work-queue head
  int32_t* exited;    // workgroups that left the queue (the last one resets both counters)
  int32_t batch;
  int32_t max_seq_len;
  int32_t Hq;
  int32_t Hk;
  int32_t group;      // Hq / Hk
  int32_t hpw_log2;   // log2(query heads per workgroup)
  int32_t n_hg;       // Hq >> hpw_log2
  int32_t bm;         // query rows per item = 32 * (4 >> hpw_log2)
  int32_t n_qt_max;   // q tiles per sequence, upper bound
  int32_t direct_items; // > 0: no work list; workgroup w runs item w of the
                        // full (q tile descending, sequence, head group) grid
  int32_t ps_log2;    // log2(page_size)
  int32_t g;          // target_group_size
  int32_t win;        // local window W (causal mask only), 0: none
  int32_t rab_vec;    // rab rows allow 4-element vector loads
  int32_t rab_heads;  // 1: one rab (and mask_heads 1: one mask) for every query head
  int32_t mask_heads;
  float alpha;
  float c_exp;        // -alpha * log2(e)
  float c_q;          // scale applied to Q as it is loaded (16-bit kernels): c_exp / y_mul
  float y_mul;        // 1, or the power of two that restores c_exp (fp16 with |c_exp| > 1)
  float out_mul;      // final scale of O (see the kernels)
};

// ------------------------------------------------------------------------
// Sequence geometry and the mask
// ------------------------------------------------------------------------
struct Seq {
  int q_tok0;  // row of query 0 in q / out
  int k_tok0;  // row of key position Lh in k / v (paged), of position 0 (jagged)
  int Lq;      // queries of this sequence
  int Lh;      // absolute position of query 0 (paged: history length;
               // jagged: keys minus queries, 0 when they are equal)
  int L;       // key positions 0 .. L-1
  int H;       // first target position (L - clamped num_targets)
  int nc;      // clamped num_context
  int page0;   // first page_ids entry (paged)
};

template <bool PAGED>
__device__ inline Seq load_seq(const KParams& p, int b, bool causal) {
  Seq s;
  const int o0 = p.seq_offsets[b], o1 = p.seq_offsets[b + 1];
  s.q_tok0 = o0;
  s.k_tok0 = o0;
  s.Lq = o1 - o0;
  s.page0 = 0;
  s.Lh = 0;
  if (PAGED) {
    const int pg0 = p.page_offsets[b], pg1 = p.page_offsets[b + 1];
    s.page0 = pg0;
    s.Lh = pg1 > pg0 ? ((pg1 - pg0 - 1) << p.ps_log2) + p.last_page_len[b] : 0;
  } else if (p.seq_offsets_k) {
    // The queries are the last Lq of the Lk key positions. More queries
    // than keys is invalid input; the rows past Lk are then left unwritten.
    const int k0 = p.seq_offsets_k[b], Lk = p.seq_offsets_k[b + 1] - k0;
    s.k_tok0 = k0;
    s.Lq = min(s.Lq, max(Lk, 0));
    s.Lh = max(Lk, 0) - s.Lq;
  }
  s.L = s.Lh + s.Lq;
  int nt = (causal && p.num_targets) ? p.num_targets[b] : 0;
  nt = min(max(nt, 0), s.L);
  s.H = s.L - nt;
  int nc = (causal && p.num_context) ? p.num_context[b] : 0;
  s.nc = min(max(nc, 0), s.H);
  return s;
}

// Key tiles that are not fully masked for the query rows [i_lo, i_hi]
// (absolute positions): tiles [t0, ta) then [tb0, tb1).
// Rows below H see keys up to max(i, nc - 1); target rows see all of
// [0, H) and, causally, their own group of g targets (all targets if g = 0).
// A local window W hides the keys below i - W + 1 from row i, so no row of
// the range sees a key below i_lo - W + 1.
struct Tiles {
  int t0, ta, tb0, tb1;
};

__device__ inline Tiles tile_range(const Seq& s, int i_lo, int i_hi, int g, int win, bool causal, int bn) {
  Tiles t;
  t.t0 = 0;
  if (!causal) {
    t.ta = (s.L + bn - 1) / bn;
    t.tb0 = t.tb1 = t.ta;
    return t;
  }
  int a_end, b_lo = 0, b_end = 0;
  if (i_hi < s.H) {
    a_end = max(i_hi + 1, i_lo < s.nc ? s.nc : 0);
  } else if (g <= 0) {
    a_end = i_hi + 1;
  } else {
    a_end = s.H;
    const int d = max(i_lo, s.H) - s.H;
    b_lo = s.H + (g == 1 ? d : (d / g) * g);  // group start of row i_lo (no division for groups of one)
    b_end = i_hi + 1;
  }
  const int w_lo = win > 0 ? max(i_lo - win + 1, 0) : 0;  // first key inside some row's window
  t.ta = (a_end + bn - 1) / bn;
  t.t0 = min(w_lo / bn, t.ta);
  t.tb0 = max(max(b_lo, w_lo) / bn, t.ta);
  t.tb1 = max((b_end + bn - 1) / bn, t.tb0);
  return t;
}

// Number of tiles in the range, and its n-th tile.
__device__ inline int tile_count(const Tiles& t) { return (t.ta - t.t0) + (t.tb1 - t.tb0); }
__device__ inline int nth_tile(const Tiles& t, int n) {
  const int na = t.ta - t.t0;
  return n < na ? t.t0 + n : t.tb0 + (n - na);
}

// ------------------------------------------------------------------------
// Planner: (sequence, q tile) items, costed by visible key tiles, optionally
// split into chunks of consecutive key tiles, counting-sorted longest first.
//
// Work list entry = two ints: (b << 16) | q_tile, and
// (chunk << 24) | (n_chunks << 16) | slot, where `slot` is the first of the
// n_chunks partial-sum slots of a split item (0xffff when not split).
// Split items are also listed once each in the reduction list:
// (b << 16) | q_tile, (n_chunks << 16) | slot, the row of the sequence's
// first query, and its query count (at most half as many entries as slots,
// so the list fits the two ints per slot the workspace reserves).
// Chunk size: the total work over target_chunks (one chunk per two resident
// workgroups on paged calls, one per workgroup on jagged ones; at least
// kMinChunkTiles), doubled until the split items fit the partial-sum slots.
// ------------------------------------------------------------------------
// Wave-wide inclusive prefix sum (64 lanes) by DPP lane shifts: within each
// row of 16 lanes by shifts of 1, 2, 4 and 8, then across rows by the
// row-broadcasts of lanes 15 and 31. (Cross-lane shuffles through LDS cost
// several times more; the planner runs dozens of these.)
__device__ inline int wave_inclusive_sum(int x) {
#if defined(__HIP_DEVICE_COMPILE__)
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
#endif
  return x;
}

// Wave-wide exclusive prefix sum of v (64 lanes); *total gets the wave sum.
__device__ inline int wave_exclusive_sum(int v, int* total) {
  const int x = wave_inclusive_sum(v);
  *total = __builtin_amdgcn_readlane(x, 63);
  return x - v;
}

// Wave-wide maximum of non-negative v.
__device__ inline int wave_max(int v) {
#if defined(__HIP_DEVICE_COMPILE__)
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false));
  return __builtin_amdgcn_readlane(v, 63);
#else
  return v;
#endif
}

// Adds v of every lane to *counter with one atomic per wave; returns the
// value of *counter before this lane's share (lanes in order).
__device__ inline int wave_fetch_add(int* counter, int v) {
  int total;
  const int ex = wave_exclusive_sum(v, &total);
  int base = 0;
  if ((threadIdx.x & 63) == 63 && total != 0) base = atomicAdd(counter, total);
  base = __builtin_amdgcn_readlane(base, 63);
  return base + ex;
}

constexpr int kMinChunkTiles = 4;
constexpr int kCostCache = 4096;  // items whose cost the planner keeps in LDS
constexpr int kSeqCache = 2048;   // sequences whose lengths the planner keeps in LDS


// BN: the key-tile size costs are counted in (32 or 64).
template <bool PAGED, int BN>
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(KParams p, int causal) {
  __shared__ int hist[kMaxBins];  // items per cost, then chunks per cost
  __shared__ short cost_cache[kCostCache];
  // Per-sequence lengths (Lq, Lh, H, nc), loaded once: the item loops below
  // touch every (sequence, q tile) pair, most of which may lie past the end
  // of their sequence (the q-tile bound comes from max_seq_len).
  __shared__ int seq_lq[kSeqCache], seq_lh[kSeqCache], seq_h[kSeqCache], seq_nc[kSeqCache], seq_q0[kSeqCache];
  __shared__ int count, total_cost, chunk_tiles, slot_alloc, n_split, qt_bound;
  const int tid = threadIdx.x;
  hist[tid] = 0;
  if (tid == 0) {
    count = 0;
    total_cost = 0;
    slot_alloc = 0;
    n_split = 0;
    qt_bound = p.batch > kSeqCache ? p.n_qt_max : 0;
  }
  __syncthreads();
  // Sequence lengths, and the largest q-tile count among them (the item
  // loops below then skip the q tiles no sequence has).
  for (int b0 = 0; b0 < p.batch && b0 < kSeqCache; b0 += kPlanThreads) {  // uniform trip count
    const int b = b0 + tid;
    int nq = 0;
    if (b < p.batch && b < kSeqCache) {
      const Seq s = load_seq<PAGED>(p, b, causal != 0);
      seq_lq[b] = s.Lq;
      seq_q0[b] = s.q_tok0;
      seq_lh[b] = s.Lh;
      seq_h[b] = s.H;
      seq_nc[b] = s.nc;
      nq = (s.Lq + p.bm - 1) / p.bm;
    }
    nq = wave_max(nq);
    if ((tid & 63) == 0) atomicMax(&qt_bound, nq);
  }
  __syncthreads();
  const int n_qt = min(qt_bound, p.n_qt_max);  // q tiles per sequence in the loops below
  const int n_items = p.batch * n_qt;
  auto seq_of = [&](int b) -> Seq {
    if (b >= kSeqCache) return load_seq<PAGED>(p, b, causal != 0);
    Seq s;
    s.k_tok0 = s.page0 = 0;  // not used for costing
    s.q_tok0 = seq_q0[b];
    s.Lq = seq_lq[b];
    s.Lh = seq_lh[b];
    s.L = s.Lh + s.Lq;
    s.H = seq_h[b];
    s.nc = seq_nc[b];
    return s;
  };
  // idx / n_qt through a float reciprocal (idx < 2^24, so the estimate is
  // off by at most one and one correction step makes it exact).
  const float inv_nqt = 1.0f / (float)max(n_qt, 1);
  auto split_idx = [&](int idx, int& b, int& qt) {
    b = (int)((float)idx * inv_nqt);
    if (b * n_qt > idx) --b;
    else if ((b + 1) * n_qt <= idx) ++b;
    qt = idx - b * n_qt;
  };
  auto compute_cost = [&](int idx) -> int {  // -1: no such item
    int b, qt;
    split_idx(idx, b, qt);
    const Seq s = seq_of(b);
    const int q_lo = qt * p.bm;
    if (q_lo >= s.Lq) return -1;
    const int i_lo = s.Lh + q_lo, i_hi = s.Lh + min(q_lo + p.bm, s.Lq) - 1;
    return min(tile_count(tile_range(s, i_lo, i_hi, p.g, p.win, causal != 0, BN)), kMaxBins - 1);
  };
  auto cost_of = [&](int idx) -> int { return idx < kCostCache ? (int)cost_cache[idx] : compute_cost(idx); };
  // The planner runs on one CU, so its passes over the items are
  // instruction-bound: the totals are summed per thread and added once.
  int my_cost = 0, my_count = 0;
  for (int base = 0; base < n_items; base += kPlanThreads) {
    const int idx = base + tid;
    const int c = idx < n_items ? compute_cost(idx) : -1;
    if (idx < kCostCache && idx < n_items) cost_cache[idx] = (short)c;
    if (c >= 0) {
      atomicAdd(&hist[c], 1);
      my_cost += c;
      ++my_count;
    }
  }
  wave_fetch_add(&total_cost, my_cost);
  wave_fetch_add(&count, my_count);
  __syncthreads();
  // Chunk size from the cost histogram (no further pass over the items):
  // candidates t0, 2 t0, 4 t0, ... in turn, one histogram bin per thread;
  // the first whose split items fit the slots wins (usually the first).
  constexpr int kCand = 10;  // t0 << 9 >= kMaxBins: the last candidate never splits
  __shared__ int need[kCand];
  if (tid < kCand) need[tid] = 0;
  if (tid == 0) chunk_tiles = INT_MAX;
  __syncthreads();
  const long long units = (long long)total_cost * p.n_hg;
  const int t0 = (int)min((long long)kMaxBins,
                          max((long long)kMinChunkTiles, (units + p.target_chunks - 1) / p.target_chunks));
  if (p.split_slots > 0) {  // uniform: every thread takes part in the wave sums and barriers
    const int h = hist[tid];
    // Chunks of a cost-tid item at chunk size t0 << ci: ceil(tid / t0)
    // halved ci times (rounding up), which is ceil(tid / (t0 << ci)).
    const int q0 = (tid + t0 - 1) / t0;
    for (int ci = 0; ci < kCand; ++ci) {
      const int t = t0 << ci;
      const int nk = (q0 + (1 << ci) - 1) >> ci;
      wave_fetch_add(&need[ci], (h > 0 && tid > t) ? min(h * min(nk, 255), 1 << 24) : 0);
      __syncthreads();
      if (need[ci] <= p.split_slots) {  // the same value in every thread
        if (tid == 0) chunk_tiles = t;
        break;
      }
    }
  }
  __syncthreads();
  const int T = chunk_tiles;
  auto n_chunks = [&](int c) { return c > T ? min((c + T - 1) / T, 255) : 1; };
  // Cost of chunk k of nk of an item of cost c: c / nk or c / nk + 1, the
  // latter for c % nk of the chunks.
  auto chunk_cost = [&](int c, int k, int nk) { return nk == 1 ? c : (k + 1) * c / nk - k * c / nk; };
  if (T != INT_MAX) {  // uniform; without splits the histogram and count above already hold
    // Chunks per cost, from the items per cost (thread tid holds cost
    // tid): every item of cost c splits alike, so each bin adds its items'
    // chunks to at most two bins (one atomic each instead of one per chunk,
    // which serialised on the few popular chunk costs).
    const int h = hist[tid];
    __syncthreads();
    if (tid == 0) count = 0;
    hist[tid] = 0;
    __syncthreads();
    const int nk = h > 0 ? n_chunks(tid) : 0;
    if (nk > 0) {
      const int q = tid / nk, r = tid - q * nk;
      if (nk - r > 0) atomicAdd(&hist[q], h * (nk - r));
      if (r > 0) atomicAdd(&hist[q + 1], h * r);
    }
    wave_fetch_add(&count, h * nk);
    __syncthreads();
  }
  // Exclusive scan over bins in descending cost: start[c] = sum of hist[c']
  // for c' > c. Thread tid holds bin kMaxBins - 1 - tid: a wave-wide scan of
  // 64 bins, then the sums of the waves before.
  __shared__ int wave_tot[kPlanThreads / 64];
  {
    const int own = hist[kMaxBins - 1 - tid];
    const int inc = wave_inclusive_sum(own);
    if ((tid & 63) == 63) wave_tot[tid >> 6] = inc;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < (tid >> 6); ++w) before += wave_tot[w];
    hist[kMaxBins - 1 - tid] = before + inc - own;
    __syncthreads();
  }
  for (int base = 0; base < n_items; base += kPlanThreads) {
    const int idx = base + tid;
    const int c = idx < n_items ? cost_of(idx) : -1;
    const int nk = c < 0 ? 0 : n_chunks(c);
    const int split_nk = nk > 1 ? nk : 0;
    int slot_at = 0, split_at = 0;
    if (T != INT_MAX) {  // uniform: only calls that split need slots
      slot_at = wave_fetch_add(&slot_alloc, split_nk);
      split_at = wave_fetch_add(&n_split, split_nk ? 1 : 0);
    }
    if (c < 0) continue;
    int b, qt;
    split_idx(idx, b, qt);
    int slot = 0xffff;
    if (nk > 1) {
      slot = slot_at;
      // The reduction reads the entry whole: no sequence loads there.
      const Seq s = seq_of(b);
      p.split_items[4 * split_at] = (b << 16) | qt;
      p.split_items[4 * split_at + 1] = (nk << 16) | slot;
      p.split_items[4 * split_at + 2] = s.q_tok0;
      p.split_items[4 * split_at + 3] = s.Lq;
    }
    if (nk == 1) {  // unsplit: one position in its cost's bin, no divisions
      const int pos = atomicAdd(&hist[c], 1);
      p.items[2 * pos] = (b << 16) | qt;
      p.items[2 * pos + 1] = (1 << 16) | slot;
      continue;
    }
    // The item's chunks of cost q take consecutive positions in that bin,
    // and those of cost q + 1 in the next: two atomics per item.
    const int q = c / nk, r = c - q * nk;
    const int pos_lo = nk - r > 0 ? atomicAdd(&hist[q], nk - r) : 0;
    const int pos_hi = r > 0 ? atomicAdd(&hist[q + 1], r) : 0;
    for (int k = 0, n_lo = 0, n_hi = 0; k < nk; ++k) {
      const int pos = chunk_cost(c, k, nk) == q ? pos_lo + n_lo++ : pos_hi + n_hi++;
      p.items[2 * pos] = (b << 16) | qt;
      p.items[2 * pos + 1] = (k << 24) | (nk << 16) | slot;
    }
  }
  __syncthreads();
  if (tid == 0) {
    *p.n_items = count;
    *p.n_split = n_split;
    *p.counter = 0;
    *p.exited = 0;
  }
}

// ------------------------------------------------------------------------
// Helpers
// ------------------------------------------------------------------------
template <typename T>
struct Frag;
template <>
struct Frag<__bf16> {
  using v8 = bf16x8_t;
  __device__ static inline f32x16_t mfma(v8 a, v8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Frag<_Float16> {
  using v8 = f16x8_t;
  __device__ static inline f32x16_t mfma(v8 a, v8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// Key position j -> pointer to its K (which = 0) or V (which = 1) row of kv head hk.
template <typename T, int D, bool PAGED>
__device__ inline const T* kv_row(const KParams& p, const Seq& s, int hk, int j, int which) {
  if (PAGED) {
    if (j < s.Lh) {
      const int page = p.page_ids[s.page0 + (j >> p.ps_log2)];
      const int slot = j & ((1 << p.ps_log2) - 1);
      const size_t row = ((((size_t)page * 2 + which) << p.ps_log2) + slot) * p.Hk + hk;
      return (const T*)p.kv_cache + row * D;
    }
    j -= s.Lh;
  }
  return (const T*)(which ? p.v : p.k) + ((size_t)(s.k_tok0 + j) * p.Hk + hk) * D;
}

// Bits [0, n) set, n clamped to [0, 32].
__device__ inline uint32_t low_bits(int n) {
  n = min(max(n, 0), 32);
  return n >= 32 ? 0xffffffffu : ((1u << n) - 1u);
}

__device__ inline int next_item(int* sh, int* counter) {
  __syncthreads();
  if (threadIdx.x == 0) *sh = atomicAdd(counter, 1);
  __syncthreads();
  return *sh;
}

// Called by every workgroup after its last (failed) queue pop. Every
// workgroup has popped for the last time before the final one arrives, so
// that one can rewind the queue for the next run of the same plan.
__device__ inline void leave_queue(const KParams& p) {
  if (threadIdx.x == 0) {
    // The workgroup's last pop returned before this point (its value ended
    // the loop), so it is ordered before this count without a fence.
    const int done = atomicAdd(p.exited, 1);
    if (done == (int)gridDim.x - 1) {
      atomicExch(p.counter, 0);
      atomicExch(p.exited, 0);
    }
  }
}

// ------------------------------------------------------------------------
// bf16 / fp16 forward
//
// LDS holds two buffers of one K tile and one V tile, both row-major
// [BN keys][D features] with padded rows: a K row is followed by 16 bytes
// and a V row stride is 64 bytes past a multiple of 256, so every MFMA
// operand read below hits distinct banks with plain addresses (one base
// register per lane and compile-time offsets). Tiles arrive by
// global->LDS DMA (16 bytes per lane), so no registers stage them; the
// padding slots receive a dummy load. One barrier per tile: tile n+1 is
// requested right after the barrier that publishes tile n, into the buffer
// tile n-1 used. (The output staging at the end of an item reuses these
// buffers with unpadded rows and an XOR swizzle of 16-byte chunks, swz.)
//
// Q is pre-scaled by c = -alpha*log2(e) while it is loaded (rounded to the
// input dtype), so the MFMA yields y = c*(Q.K) directly; with rab,
// y += c*rab. Then
//   silu(alpha*s) = -(y / (1 + 2^y)) / log2(e),
// and the constant -1/log2(e) joins out_scale in the final store, leaving
// exp2, add, rcp, mul and a packed convert per element. In fp16, c*Q could
// overflow when |c| > 1; Q is then scaled by c / 2^k (|c / 2^k| <= 1, so
// |c Q / 2^k| <= |Q| stays finite) and S by the exact power of two 2^k
// (y_mul) before the epilogue, in a block that is skipped when y_mul == 1.
// ------------------------------------------------------------------------
// Chunk-slot swizzle of key row j. For D = 128 (16 chunks of 16 bytes, one
// row = all 64 banks) it is 4 (j % 4) + (j / 4) % 4: the 16 rows a 16-lane
// K-fragment read touches get 16 different slots, and the 4 rows x 4
// chunks a 32-lane half of a transposing V read touches get 16 different
// slots too. Other head dims keep the low bits that fit their row width.
template <int D>
__device__ inline int swz(int j) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  if constexpr (CPR >= 16) {
    return ((j & 3) << 2) | ((j >> 2) & 3);
  } else if constexpr (CPR == 8) {
    return (j >> 1) & 7;  // two rows share the 64 banks
  } else {
    return (j >> 2) & 3;  // four rows share the 64 banks
  }
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));

// 16 bytes per lane from global memory straight into LDS: lane l of the
// wave writes lds_base + 16 l (lds_base must be wave-uniform; it goes in M0).
// Written as inline assembly on purpose: the compiler then does not track
// these LDS writes, so it does not make reads of the other buffer wait for
// the prefetch in flight (its alias analysis cannot always separate them).
// The kernel orders them itself: a vmcnt(0) wait and a barrier before any
// wave reads a filled buffer, and a barrier between the last read of a
// buffer and the next DMA into it. The DMA reads M0 one cycle after it
// issues, so a wait state separates it from the M0 write the compiler
// places right before the statement (the compiler adds the same s_nop to
// its own LDS DMA; it cannot see into this one).
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(__attribute__((address_space(3))) const char*)p;
}
// The source address is a per-lane 64-bit VGPR pair (the form the compiler
// itself uses after a VALU address add). No SGPR operand: a VMEM read of an
// SGPR written by a VALU instruction (v_readfirstlane) needs five wait
// states, which the compiler cannot insert for an asm statement.
__device__ inline void dma16(const void* src, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_addr(lds_base)));
#endif
}

// Transposing LDS read (16-lane groups): lane t of a group receives element
// t%4 of the 8-byte reads of lanes t/4, t/4+4, t/4+8 and t/4+12.
__device__ inline v4i16_t lds_read_tr16(const void* addr) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)addr);
#else
  return v4i16_t{};
#endif
}

__device__ inline void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)
// s_getreg operand for the whole HW_ID register (id 4, bits 0..31): bits
// 3:0 are the wave's slot on its SIMD, bits 5:4 the SIMD.
constexpr int kHwRegHwId = (31 << 11) | 4;

// KSP = 1: a workgroup of 4 waves walks all key tiles of its item.
// KSP = 2: 8 waves in two groups of 4; group g takes key tiles g, g+2, ...
// of the item (each group with its own LDS buffers) and the two partial
// O tiles are summed through LDS at the end. This halves an item's latency,
// for work lists too short to fill the chip.
// MSK: the user mask (mask_type 3, no built-in mask): its value m for
// (i, j) multiplies P, and m == 0 removes the key like the built-in masks do.
// SQL: which of rab (bit 0) and the user mask (bit 1) are staged through a
// ring of three LDS tiles by DMA, two tiles ahead (the others are loaded
// into registers one tile ahead). Needs KSP == 1 and rows of max_seq_len
// elements that are 16-byte multiples.
template <typename T, int D, int BN, bool CAUSAL, bool RAB, bool PAGED, int WPE, int KSP, bool MSK = false, int SQL = 0>
__global__ __launch_bounds__(kThreads * KSP) __attribute__((amdgpu_waves_per_eu(WPE))) void fwd_kernel(KParams p) {
  using F = Frag<T>;
  using V8 = typename F::v8;
  constexpr int KS = D / 16;    // k steps of S^T = K Q^T
  constexpr int NJB = BN / 32;  // 32-key blocks per tile
  constexpr int NDB = D / 32;   // 32-wide blocks of O^T
  constexpr int ROW_B = D * 2;  // bytes per key row in global memory
  // LDS rows are padded so that every fragment read is bank-conflict free
  // with plain (unswizzled) addresses, i.e. one base register per lane and
  // compile-time offsets: a K row is followed by 16 bytes (16 consecutive
  // rows then start in 16 different 4-bank groups); a V row stride is 64
  // bytes past a multiple of 256 (the 4 rows x 64 bytes a half-wave
  // transposing read touches then cover all 64 banks once).
  constexpr int KS_B = ROW_B + 16;
  constexpr int VS_B = ROW_B + (ROW_B % 256 == 64 ? 0 : 64);
  constexpr int K_SLOTS = KS_B / 16, V_SLOTS = VS_B / 16;  // 16-byte slots per LDS row
  constexpr int K_TILE_B = (BN * KS_B + 1023) / 1024 * 1024;  // whole 1 KB DMA blocks
  constexpr int V_TILE_B = (BN * VS_B + 1023) / 1024 * 1024;
  constexpr int K_BLK = K_TILE_B / 1024, V_BLK = V_TILE_B / 1024;
  constexpr int K_BLK_W = (K_BLK + kWaves - 1) / kWaves, V_BLK_W = (V_BLK + kWaves - 1) / kWaves;
  static_assert(KSP == 1 || (KSP == 2 && BN == 64), "the key split exchanges O through one 64-key K/V buffer per wave");
  // Side-tensor ring (see SQL): one tile of one tensor holds the BN keys of
  // the 128 (query row, head) pairs of the item, row r of the tile (pair
  // r = 32 w + l of wave w, lane l) in BN * 2 bytes whose 16-byte chunks
  // are permuted by the swizzle below, so that the 8-byte reads of the 32
  // rows of a wave spread over all banks.
  constexpr bool R_LDS = RAB && (SQL & 1), M_LDS = MSK && (SQL & 2);
  constexpr int N_RING = (R_LDS ? 1 : 0) + (M_LDS ? 1 : 0);
  constexpr int RING = 3;
  constexpr int SQ_ROW_B = BN * 2;
  constexpr int SQ_TILE_B = kWaves * kRowsPerWave * SQ_ROW_B;
  constexpr int SQ_CH = SQ_ROW_B / 16;         // 16-byte chunks per row
  constexpr int SQ_G = 256 / SQ_ROW_B;         // rows per sweep of the 64 banks
  constexpr int SQ_BLK_W = SQ_TILE_B / 1024 / kWaves;  // DMA blocks per wave per tile
  static_assert(N_RING == 0 || (KSP == 1 && SQ_TILE_B % (1024 * kWaves) == 0 && SQ_G >= 1), "side-tensor ring");
  using Buf0 = std::integral_constant<int, 0>;
  using Buf1 = std::integral_constant<int, 1>;

  // Separate objects per buffer: the compiler's alias analysis can then see
  // that the DMA filling one buffer does not write the one being read, and
  // does not wait for the prefetch before reading the current tile.
  // One slice per key group; group g uses slice g of every array.
  __shared__ __attribute__((aligned(1024))) char smem_k0[KSP][K_TILE_B];
  __shared__ __attribute__((aligned(1024))) char smem_v0[KSP][V_TILE_B];
  __shared__ __attribute__((aligned(1024))) char smem_k1[KSP][K_TILE_B];
  __shared__ __attribute__((aligned(1024))) char smem_v1[KSP][V_TILE_B];
  __shared__ __attribute__((aligned(1024))) char smem_sq[N_RING ? N_RING * RING : 1][N_RING ? SQ_TILE_B : 16];
  __shared__ int sh_item[2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave = wave_id & (kWaves - 1);  // role inside the key group
  const int l32 = lane & 31, half = lane >> 5;
  // Logical wave lw (query row block and head of this wave): the rank of
  // the key (SIMD + 2 x wave-slot parity) mod 4 of this wave among the four
  // of its key group (ties by wave index), from the hardware id register.
  // Two workgroups share a CU, in wave slots 0 and 1, one wave per SIMD
  // each: their logical waves 0 and 1 then sit on different SIMD pairs, so
  // items with fewer rows than a workgroup holds (few-token paged and
  // delta-QK calls) do not stack both workgroups' active waves on the same
  // SIMDs. The ranks form a permutation whatever the placement, and results
  // do not depend on it.
  __shared__ int sh_key[kWaves];
  if (lane == 0 && wave_id < kWaves) {
    const uint32_t hw = __builtin_amdgcn_s_getreg(kHwRegHwId);
    sh_key[wave_id] = (int)((((hw >> 4) & 3u) + 2u * (hw & 1u)) & 3u);
  }
  __syncthreads();
  int lw = 0;
  {
    const int mine = sh_key[wave];
#pragma unroll
    for (int j = 0; j < kWaves; ++j) {
      const int k = sh_key[j];
      lw += (k < mine || (k == mine && j < wave)) ? 1 : 0;
    }
  }
  lw = __builtin_amdgcn_readfirstlane(lw);
  const bool direct = p.direct_items > 0;
  const int n_work = direct ? p.direct_items : *p.n_items * p.n_hg;
  const int hpw = 1 << p.hpw_log2;
  const uint32_t row_stride_b = (uint32_t)p.Hk * ROW_B;  // bytes between key rows of one kv head

  // DMA geometry of this lane, the same for every tile: lane `lane` of the
  // wave's block u fills 16-byte LDS slot (blk * 64 + lane) of a tile, with
  // blk = wave + kWaves u, i.e. row slot / SLOTS and chunk slot % SLOTS.
  // Padding slots, and slots past the last row, load chunk 0 of a valid row
  // (the bytes are never read).
  auto slot_row = [&](int slots, int blk) { return min((blk * 64 + lane) / slots, BN - 1); };
  auto slot_col_b = [&](int slots, int blk) {
    const int c = (blk * 64 + lane) % slots;
    return (uint32_t)(c < ROW_B / 16 && (blk * 64 + lane) / slots < BN ? c * 16 : 0);
  };
  uint32_t dma_k_off[K_BLK_W], dma_v_off[V_BLK_W];
#pragma unroll
  for (int u = 0; u < K_BLK_W; ++u) {
    const int blk = wave + kWaves * u;
    dma_k_off[u] = (uint32_t)slot_row(K_SLOTS, blk) * row_stride_b + slot_col_b(K_SLOTS, blk);
  }
#pragma unroll
  for (int u = 0; u < V_BLK_W; ++u) {
    const int blk = wave + kWaves * u;
    dma_v_off[u] = (uint32_t)slot_row(V_SLOTS, blk) * row_stride_b + slot_col_b(V_SLOTS, blk);
  }

  // Each key group runs its own copy of the loop with its group index as a
  // constant, so every LDS buffer address is known at compile time (which
  // lets the compiler see that a DMA into one buffer never aliases reads of
  // another). Both copies execute the same sequence of barriers.
  const bool dyn = (int)gridDim.x < n_work;
  auto run = [&](auto grpc) {
    constexpr int GRP = decltype(grpc)::value;
    auto kv_smem = [&](auto bufc, int which) -> char* {
      constexpr int B = decltype(bufc)::value;
      if constexpr (B == 0) return which ? smem_v0[GRP] : smem_k0[GRP]; else return which ? smem_v1[GRP] : smem_k1[GRP];
    };
  // Work item w of workgroup g: first w = g, then, when there are more
  // items than workgroups, gridDim.x + (pops of the shared counter). The
  // pop for the next item is issued when an item starts, so its latency
  // hides behind the item's first tile load.
  int w = blockIdx.x, parity = 0;
  while (w < n_work) {
    int w_next = n_work;
    if (dyn && tid == 0) w_next = (int)gridDim.x + atomicAdd(p.counter, 1);
    const int item = w / p.n_hg;
    const int hg = w - item * p.n_hg;
    int b, qt, meta = (1 << 16);  // direct items: one chunk
    if (direct) {
      // Highest q tiles first: under the causal mask they see the most key
      // tiles, and workgroups start in index order.
      qt = p.n_qt_max - 1 - item / p.batch;
      b = item - (p.n_qt_max - 1 - qt) * p.batch;
    } else {
      const int packed = p.items[2 * item];
      meta = p.items[2 * item + 1];
      b = packed >> 16;
      qt = packed & 0xffff;
    }
    const int chunk = (int)((uint32_t)meta >> 24), n_chunks = (meta >> 16) & 0xff, slot0 = meta & 0xffff;
    const Seq s = load_seq<PAGED>(p, b, CAUSAL);
    // A direct item past the end of its sequence has no rows; in direct mode
    // every workgroup has exactly one item, so it simply has no work.
    if (direct && qt * p.bm >= s.Lq) break;
    const int h = hg * hpw + (lw & (hpw - 1));
    const int rb = lw >> p.hpw_log2;
    const int hk = (hg * hpw) / p.group;
    const int q_lo = qt * p.bm;
    const int q_hi = min(q_lo + p.bm, s.Lq);
    const int i_lo = s.Lh + q_lo, i_hi = s.Lh + q_hi - 1;
    const int q_loc = q_lo + rb * kRowsPerWave + l32;
    const bool row_ok = q_loc < s.Lq;
    const bool wave_active = q_lo + rb * kRowsPerWave < s.Lq;
    const int i = s.Lh + q_loc;

    // Paged calls: a key tile lies in one cache page when it ends inside the
    // history and pages hold at least BN rows; its page id is then
    // page_ids[page0 + j0 / page_size].
    auto in_page = [&](int j0) { return PAGED && j0 + BN <= s.Lh && (1 << p.ps_log2) >= BN; };
    // Uniform base addresses of a whole tile whose BN rows are consecutive
    // rows of one tensor (stride row_stride_b); false for tiles that end past
    // the sequence, straddle the history / new-token boundary, or span pages.
    // page: the tile's page id when in_page(j0).
    auto tile_bases = [&](int j0, int page, const char*& kb, const char*& vb) -> bool {
      if (!PAGED) {
        if (j0 + BN > s.L) return false;
        const size_t e = ((size_t)(s.k_tok0 + j0) * p.Hk + hk) * D;
        kb = (const char*)((const T*)p.k + e);
        vb = (const char*)((const T*)p.v + e);
        return true;
      } else {
        if (j0 + BN <= s.Lh) {
          if ((1 << p.ps_log2) < BN) return false;
          const size_t slot0 = (size_t)(j0 & ((1 << p.ps_log2) - 1));
          const size_t ek = (((((size_t)page * 2) << p.ps_log2) + slot0) * p.Hk + hk) * D;
          const size_t ev = (((((size_t)page * 2 + 1) << p.ps_log2) + slot0) * p.Hk + hk) * D;
          kb = (const char*)((const T*)p.kv_cache + ek);
          vb = (const char*)((const T*)p.kv_cache + ev);
          return true;
        }
        if (j0 >= s.Lh && j0 + BN <= s.L) {
          const size_t e = ((size_t)(s.k_tok0 + j0 - s.Lh) * p.Hk + hk) * D;
          kb = (const char*)((const T*)p.k + e);
          vb = (const char*)((const T*)p.v + e);
          return true;
        }
        return false;
      }
    };
    // DMA of key tile kt into buffer BUF (page: its page id when in a page).
    // Rows past the sequence repeat its last row (finite values, masked to
    // zero by the epilogue).
    auto dma_tile = [&](int kt, auto bufc, int page) {
      constexpr int BUF = decltype(bufc)::value;
      const int j0 = kt * BN;
      const char *kb, *vb;
      if (tile_bases(j0, page, kb, vb)) {
#pragma unroll
        for (int u = 0; u < K_BLK_W; ++u) {
          const int blk = wave + kWaves * u;
          if (K_BLK % kWaves == 0 || blk < K_BLK) dma16(kb + dma_k_off[u], kv_smem(bufc, 0) + blk * 1024);
        }
#pragma unroll
        for (int u = 0; u < V_BLK_W; ++u) {
          const int blk = wave + kWaves * u;
          if (V_BLK % kWaves == 0 || blk < V_BLK) dma16(vb + dma_v_off[u], kv_smem(bufc, 1) + blk * 1024);
        }
      } else {
#pragma unroll
        for (int u = 0; u < K_BLK_W; ++u) {
          const int blk = wave + kWaves * u;
          if (K_BLK % kWaves == 0 || blk < K_BLK) {
            const int j = min(j0 + slot_row(K_SLOTS, blk), s.L - 1);
            dma16((const char*)kv_row<T, D, PAGED>(p, s, hk, j, 0) + slot_col_b(K_SLOTS, blk), kv_smem(bufc, 0) + blk * 1024);
          }
        }
#pragma unroll
        for (int u = 0; u < V_BLK_W; ++u) {
          const int blk = wave + kWaves * u;
          if (V_BLK % kWaves == 0 || blk < V_BLK) {
            const int j = min(j0 + slot_row(V_SLOTS, blk), s.L - 1);
            dma16((const char*)kv_row<T, D, PAGED>(p, s, hk, j, 1) + slot_col_b(V_SLOTS, blk), kv_smem(bufc, 1) + blk * 1024);
          }
        }
      }
    };

    const Tiles tr = tile_range(s, i_lo, i_hi, p.g, p.win, CAUSAL, BN);
    const int n_tiles = tile_count(tr);
    auto tile_at = [&](int n) { return nth_tile(tr, n); };
    // This chunk covers tiles [n_begin, n_end) of the item's tile sequence.
    const int n_begin = chunk * n_tiles / n_chunks, n_end = (chunk + 1) * n_tiles / n_chunks;
    const int n_steps = (n_end - n_begin + KSP - 1) / KSP;
    // The first tile's DMA goes out before the Q load, to overlap their latencies.
    if (n_begin + GRP < n_end) {
      const int j0 = tile_at(n_begin + GRP) * BN;
      dma_tile(tile_at(n_begin + GRP), Buf0{}, in_page(j0) ? p.page_ids[s.page0 + (j0 >> p.ps_log2)] : 0);
    }
    // Paged calls: the page id of the tile a step's DMA fetches is read one
    // step earlier, by a vector load issued after that step's DMA (so the
    // next step's wait for its tile covers it); the DMA then needs no
    // dependent load of its own.
    int page_v = 0;
    auto load_page = [&](int n) {
      if constexpr (PAGED) {
        const int j0 = tile_at(n) * BN;
        if (in_page(j0)) {
          int idx = s.page0 + (j0 >> p.ps_log2);
          asm volatile("" : "+v"(idx));  // a vector load, counted by vmcnt behind the DMA
          page_v = p.page_ids[idx];
        }
      }
    };
    if (n_begin + GRP + KSP < n_end) load_page(n_begin + GRP + KSP);

    // Q fragments (B operand of S^T = K Q^T), pre-scaled by c.
    V8 qf[KS];
    {
      const T* qrow = (const T*)p.q + ((size_t)(s.q_tok0 + q_loc) * p.Hq + h) * D + half * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4_t x = {0u, 0u, 0u, 0u};
        if (row_ok) x = *(const u32x4_t*)(qrow + ks * 16);
        const V8 raw = __builtin_bit_cast(V8, x);
        V8 sc;
#pragma unroll
        for (int e = 0; e < 8; ++e) sc[e] = (T)((float)raw[e] * p.c_q);
        qf[ks] = sc;
      }
    }
    // Row i sees keys [0, a_i] and [b_i, i] (second interval empty when b_i > i).
    const int hi_i = (i < s.nc) ? max(i, s.nc - 1) : i;
    const int tlo_i = (p.g <= 0) ? s.H : (i >= s.H ? s.H + ((i - s.H) / p.g) * p.g : INT_MAX);
    const int a_i = CAUSAL ? min(hi_i, s.H - 1) : s.L - 1;
    const int b_i = CAUSAL ? max(tlo_i, s.H) : INT_MAX;
    // Local window (p.win > 0, causal only): row i sees no key below
    // i - win + 1, and a tile is full only if every row of the item sees its
    // first key. Both are formed per tile from the kernel argument, so no
    // register holds them across the loop.
    const bool windowed = CAUSAL && p.win > 0;


    f32x16_t o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

    // rab and the user mask are [B, heads, S, S] (heads 1: shared by every
    // query head), indexed by absolute positions. Rows past the sequence
    // read its last row (always in bounds; their results are never stored).
    auto sq_row = [&](const void* base, int heads) -> const T* {
      const int row = s.Lh + min(q_loc, max(s.Lq - 1, 0));
      return (const T*)base + ((size_t)(b * heads + (heads == 1 ? 0 : h)) * p.max_seq_len + row) * p.max_seq_len;
    };
    const T* rrow = RAB ? sq_row(p.rab, p.rab_heads) : nullptr;
    const T* mrow = MSK ? sq_row(p.mask, p.mask_heads) : nullptr;
    // Ring DMA geometry of this lane: in block u it fills 16-byte slot
    // (blk * 64 + lane) of a tile, blk = wave + kWaves u, i.e. chunk cp of
    // row P, holding the 8 keys of chunk cp ^ swizzle(P) of pair P. Rows
    // past the sequence repeat its last row; chunks past max_seq_len repeat
    // the row's last chunk (those keys are masked).
    const T* ring_row[N_RING ? N_RING : 1][N_RING ? SQ_BLK_W : 1];
    int ring_col[N_RING ? SQ_BLK_W : 1];
    if constexpr (N_RING > 0) {
#pragma unroll
      for (int u = 0; u < SQ_BLK_W; ++u) {
        const int slot = (wave + kWaves * u) * 64 + lane;
        const int P = slot / SQ_CH, cp = slot % SQ_CH;
        ring_col[u] = 8 * (cp ^ ((P / SQ_G) % SQ_CH));
        const int w = P / kRowsPerWave;
        const int hh = hg * hpw + (w & (hpw - 1));
        const int qq = q_lo + (w >> p.hpw_log2) * kRowsPerWave + P % kRowsPerWave;
        const int row = s.Lh + min(qq, max(s.Lq - 1, 0));
        int t = 0;
        if constexpr (R_LDS)
          ring_row[t++][u] = (const T*)p.rab + ((size_t)(b * p.rab_heads + (p.rab_heads == 1 ? 0 : hh)) * p.max_seq_len + row) * p.max_seq_len;
        if constexpr (M_LDS)
          ring_row[t++][u] = (const T*)p.mask + ((size_t)(b * p.mask_heads + (p.mask_heads == 1 ? 0 : hh)) * p.max_seq_len + row) * p.max_seq_len;
      }
    }
    // DMA of the side tensors' tile n (of the chunk) into ring slot rs.
    auto ring_dma = [&](int n, int rs) {
      if constexpr (N_RING > 0) {
        const int j0 = tile_at(n) * BN;
#pragma unroll
        for (int t = 0; t < N_RING; ++t)
#pragma unroll
          for (int u = 0; u < SQ_BLK_W; ++u)
            dma16(ring_row[t][u] + min(j0 + ring_col[u], p.max_seq_len - 8),
                  smem_sq[t * RING + rs] + (wave + kWaves * u) * 1024);
      }
    };
    // This lane's rab / mask words of ring slot rs, in the register layout
    // of the prefetch below.
    const int ring_pair = lw * kRowsPerWave + l32;
    const int ring_off = ring_pair * SQ_ROW_B + 8 * half;
    const int ring_swz = (ring_pair / SQ_G) % SQ_CH;
    // rab (or mask) of the tile at key j0: lane holds row q_loc, keys
    // j0 + 32 jb + 8 a + 4 half + 0..3. Loaded one step ahead (issued right
    // after the next tile's DMA), so the step that uses it never waits for
    // memory in the middle. Keys past the sequence read 0.
    using RabRegs = u32x2_t[NJB][4];
    auto load_rab = [&](const T* row, int j0, RabRegs& rv) {
      if (j0 + BN <= s.L && p.rab_vec) {  // uniform: whole tile inside the sequence, 8-byte aligned rows
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
          for (int a = 0; a < 4; ++a) rv[jb][a] = *(const u32x2_t*)(row + j0 + jb * 32 + 8 * a + 4 * half);
      } else {
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int jj = j0 + jb * 32 + 8 * a + 4 * half;
            T t4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) t4[e] = (jj + e < s.L) ? row[jj + e] : (T)0.f;
            rv[jb][a] = *(const u32x2_t*)t4;
          }
      }
    };
    RabRegs rv_next, mv_next;
    if (n_begin + GRP < n_end) {
      if constexpr (RAB && !R_LDS) load_rab(rrow, tile_at(n_begin + GRP) * BN, rv_next);
      if constexpr (MSK && !M_LDS) load_rab(mrow, tile_at(n_begin + GRP) * BN, mv_next);
    }
    // The ring's first two tiles, after every other load of the prologue:
    // the first step then waits for all but the second.
    int ring_slot = 0;
    if constexpr (N_RING > 0) {
      asm volatile("" ::: "memory");
      ring_dma(n_begin, 0);
      if (n_begin + 1 < n_end) ring_dma(n_begin + 1, 1);
    }
    const int G = lane >> 4, sl = lane & 15;

    // One key tile: publish its LDS buffer, request the next tile into the
    // other buffer, then S^T, epilogue and O^T on this one.
    auto step = [&](int t, auto bufc) {
      constexpr int BUF = decltype(bufc)::value;
      const int n = n_begin + KSP * t + GRP;
      const bool has_tile = n < n_end;
      const int kt = tile_at(has_tile ? n : n_begin);
      const int cur = ring_slot;  // ring slot of this tile
      ring_slot = cur == RING - 1 ? 0 : cur + 1;
      if constexpr (N_RING > 0) {
        // This tile's K/V DMA and ring tile must have landed; the ring DMA
        // issued last after them (tile n + 1, when it exists) may stay in
        // flight. The ring DMAs are the last vector memory instructions a
        // step issues.
        constexpr int NRD = N_RING * SQ_BLK_W;
        static_assert(NRD < 16, "vmcnt field");
        if (n + 1 < n_end)
          __builtin_amdgcn_s_waitcnt(0x0F70 | NRD);  // vmcnt(NRD)
        else
          wait_vmem_all();
      } else {
        wait_vmem_all();
      }
      __syncthreads();
      const int j0 = kt * BN;

      // The next tile's DMA goes out first: it has a whole step to land;
      // then the next tile's rab (this tile's arrived last step), then the
      // ring tile two ahead, into the slot the last step read.
      // Jagged 64-key kernels at two waves per SIMD, no side-tensor ring: a
      // whole next tile's DMA instructions (K_BLK_W + V_BLK_W per wave) are
      // spread over the S^T MFMA groups below instead of going out back to
      // back, where the CU's 80 or so 1 KB LDS DMAs queue behind each other
      // and each wave stalls until its last one is accepted (GQA workload
      // about 2 % faster; the shorter steps of 32-key and paged kernels left
      // too little time after the spread DMAs, so they issue at once).
      constexpr bool SPREAD = WPE == 2 && N_RING == 0 && BN == 64 && !PAGED;
      constexpr int NQ = K_BLK_W + V_BLK_W;
      using NextBuf = std::integral_constant<int, BUF ^ 1>;
      const char *kb_n = nullptr, *vb_n = nullptr;
      bool spread = false;
      if (n + KSP < n_end) {
        const int kt_n = tile_at(n + KSP), pg = __builtin_amdgcn_readfirstlane(page_v);
        if (SPREAD && tile_bases(kt_n * BN, pg, kb_n, vb_n))
          spread = true;
        else
          dma_tile(kt_n, NextBuf{}, pg);
      }
      // DMA instruction q of this wave for the next tile (whole tiles only).
      auto dma_part = [&](int q) {
        if (q < K_BLK_W) {
          const int blk = wave + kWaves * q;
          if (K_BLK % kWaves == 0 || blk < K_BLK) dma16(kb_n + dma_k_off[q], kv_smem(NextBuf{}, 0) + blk * 1024);
        } else {
          const int u = q - K_BLK_W, blk = wave + kWaves * u;
          if (V_BLK % kWaves == 0 || blk < V_BLK) dma16(vb_n + dma_v_off[u], kv_smem(NextBuf{}, 1) + blk * 1024);
        }
      };
      if (n + 2 * KSP < n_end) load_page(n + 2 * KSP);
      RabRegs rv, mv;
      if constexpr (RAB && !R_LDS) {
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
          for (int a = 0; a < 4; ++a) rv[jb][a] = rv_next[jb][a];
        if (n + KSP < n_end) load_rab(rrow, tile_at(n + KSP) * BN, rv_next);
      }
      if constexpr (MSK && !M_LDS) {
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
          for (int a = 0; a < 4; ++a) mv[jb][a] = mv_next[jb][a];
        if (n + KSP < n_end) load_rab(mrow, tile_at(n + KSP) * BN, mv_next);
      }
      if constexpr (N_RING > 0) {
        asm volatile("" ::: "memory");
        if (n + 2 < n_end) ring_dma(n + 2, cur == 0 ? RING - 1 : cur - 1);
      }
      if (!wave_active || !has_tile) {
        if constexpr (SPREAD) {
          if (spread) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) dma_part(q);
          }
        }
        return;
      }
      // The ring tensors' words of this tile.
      if constexpr (N_RING > 0) {
        int t = 0;
        auto ring_read = [&](RabRegs& rg, int tt) {
          const char* base = smem_sq[tt * RING + cur] + ring_off;
#pragma unroll
          for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
            for (int a = 0; a < 4; ++a) rg[jb][a] = *(const u32x2_t*)(base + 16 * ((4 * jb + a) ^ ring_swz));
        };
        if constexpr (R_LDS) ring_read(rv, t++);
        if constexpr (M_LDS) ring_read(mv, t++);
      }

      const char* kbuf = kv_smem(bufc, 0);
      const char* vbuf = kv_smem(bufc, 1);

      // Full tiles skip the mask; the branch is uniform and taken once per
      // tile, so each variant below is straight-line code the scheduler can
      // interleave freely.
      const int j1 = min(j0 + BN, s.L);
      const bool full = (j0 + BN <= s.L) && (!windowed || j0 >= i_hi - p.win + 1) &&
                        (!CAUSAL || ((j1 - 1 <= i_lo) && (j1 <= s.H)) || ((i_hi < s.nc) && (j1 <= s.nc)));

      // K fragment (A operand of S^T) for key block jb, k step ks.
      auto k_frag = [&](int jb, int ks) -> V8 {
        const int row = jb * 32 + l32;
        return *(const V8*)(kbuf + row * KS_B + (2 * ks + half) * 16);
      };
      // V^T fragment (A operand of O^T += V^T P^T) for (jb, m, db): two
      // transposing reads; the 16-lane group G = lane/16 reads key rows
      // 32 jb + 16 m + 8 u + 4 (G/2) + (lane%16)/4 and features
      // 32 db + 16 (G%2) + 4 (lane%4) .. +3, and lane t of the group receives
      // feature 32 db + 16 (G%2) + t for those four keys.
      auto v_frag = [&](int jb, int m, int db) -> V8 {
        v4i16_t part[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int row = jb * 32 + 16 * m + 8 * u + 4 * (G >> 1) + (sl >> 2);
          const int col = db * 32 + 16 * (G & 1) + 4 * (sl & 3);
          part[u] = lds_read_tr16(vbuf + row * VS_B + col * 2);
        }
        return __builtin_bit_cast(V8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
      };

      // Visibility of the lane's keys in block jb as a bit mask over the
      // offset from its first key j = j0 + 32 jb + 4 half: bit o is set iff
      // key j + o is visible, i.e. o <= a_i - j or b_i - j <= o <= i - j,
      // and o >= i - win + 1 - j (the local window).
      // Built on masked tiles only (full tiles never read it).
      uint32_t vis[NJB];
      auto make_vis = [&]() {
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
          const int jbase = j0 + jb * 32 + 4 * half;
          const int lo_end = a_i - jbase + 1, hi_beg = b_i == INT_MAX ? 32 : b_i - jbase, hi_end = i - jbase + 1;
          vis[jb] = low_bits(lo_end) | (low_bits(hi_end) & ~low_bits(hi_beg));
          if (windowed) vis[jb] &= ~low_bits(i - p.win + 1 - jbase);
        }
      };
      f32x16_t sacc[NJB];
      V8 pf[NJB][2];
      // S block jb times y_mul (only when Q was scaled by c / y_mul).
      auto scale_s = [&](int jb) {
        if (p.y_mul != 1.f) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[jb][r] *= p.y_mul;
        }
      };
      // Epilogue of element r of block jb: rab, mask (masked tiles), SiLU, round.
      // rab and mask of element r of block jb: y (kept in sacc).
      // Element r of block jb of a prefetched rab / mask tile, as float.
      auto sq_val = [&](const RabRegs& rg, int jb, int r) -> float {
        const uint32_t wd = rg[jb][r / 4][(r % 4) / 2];
        if constexpr (std::is_same<T, __bf16>::value) {
          return __builtin_bit_cast(float, (r % 2) ? (wd & 0xffff0000u) : (wd << 16));
        } else {
          const T* t2 = (const T*)&wd;
          return (float)t2[r % 2];
        }
      };
      auto epi_pre = [&](auto masked, int jb, int r) -> float {
        float y = sacc[jb][r];
        if (RAB) y = __builtin_fmaf(sq_val(rv, jb, r), p.c_exp, y);
        if constexpr (MSK) {
          // A zero mask value removes the key: y = +0, so p = 0 exactly.
          const int keep = sq_val(mv, jb, r) != 0.f ? -1 : 0;
          y = __builtin_bit_cast(float, __builtin_bit_cast(int, y) & keep);
        }
        if constexpr (decltype(masked)::value) {
          // Masked keys get y = +0 (bitwise AND with the sign-extended
          // visibility bit), hence p = 0 * 1/2 = 0 exactly, and a NaN rab
          // there never reaches the arithmetic. Both variants run the same
          // arithmetic otherwise, so results do not depend on which tiles a
          // configuration classifies as full.
          const int off = 8 * (r / 4) + (r % 4);  // unrolled: a constant
          const int keep = (int)(vis[jb] << (31 - off)) >> 31;
          y = __builtin_bit_cast(float, __builtin_bit_cast(int, y) & keep);
        }
        return y;
      };
      // The user mask's value of element r of block jb. On masked tiles the
      // ring can hold bytes past the sequence (whatever the tensor holds
      // there): masked keys take 0 there, so P stays 0.
      auto mval = [&](auto masked, int jb, int r) -> float {
        float m = sq_val(mv, jb, r);
        if constexpr (M_LDS && decltype(masked)::value) {
          const int off = 8 * (r / 4) + (r % 4);
          const int keep = (int)(vis[jb] << (31 - off)) >> 31;
          m = __builtin_bit_cast(float, __builtin_bit_cast(int, m) & keep);
        }
        return m;
      };
      // Epilogue of element r of block jb: rab, mask (masked tiles), SiLU, round.
      auto epi = [&](auto masked, int jb, int r) {
        const float y = epi_pre(masked, jb, r);
        const float e = __builtin_amdgcn_exp2f(y);
        float pv = y * __builtin_amdgcn_rcpf(1.f + e);
        if constexpr (MSK) pv *= mval(masked, jb, r);
        pf[jb][r / 8][r % 8] = (T)pv;
      };
      // The same for the 16 elements of block jb, one operation at a time
      // across EB elements (each stage its own scheduling region): EB
      // independent chains, and every result is used EB instructions after
      // it is made.
      auto epi_block = [&](auto masked, int jb) {
        constexpr int EB = (RAB || MSK) ? 4 : 16;  // elements per pass (rab / mask values hold registers too)
#pragma unroll
        for (int r0 = 0; r0 < 16; r0 += EB) {
          float y[EB], e[EB];
#pragma unroll
          for (int r = 0; r < EB; ++r) y[r] = epi_pre(masked, jb, r0 + r);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int r = 0; r < EB; ++r) e[r] = __builtin_amdgcn_exp2f(y[r]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int r = 0; r < EB; ++r) e[r] = 1.f + e[r];
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int r = 0; r < EB; ++r) e[r] = __builtin_amdgcn_rcpf(e[r]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int r = 0; r < EB; ++r) {
            float pv = y[r] * e[r];
            if constexpr (MSK) pv *= mval(masked, jb, r0 + r);
            pf[jb][(r0 + r) / 8][(r0 + r) % 8] = (T)pv;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };

      if constexpr (WPE == 1) {
        // One wave per SIMD: overlap MFMA and VALU inside the wave. S^T of
        // block jb runs while the epilogue of block jb - 1 fills the VALU
        // slots; O^T of block 0 runs under the epilogue of the last block.
        // Fragment reads are issued one step ahead. The full / masked choice
        // selects one of two straight-line copies.
        auto body = [&](auto masked) {
          auto s_block = [&](int jb) {
            if (jb > 0) scale_s(jb - 1);
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[jb][r] = 0.f;
            V8 kf = k_frag(jb, 0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              V8 kn = kf;
              if (ks + 1 < KS) kn = k_frag(jb, ks + 1);
              sacc[jb] = F::mfma(kf, qf[ks], sacc[jb]);
              if (jb > 0) {
#pragma unroll
                for (int r = ks * 16 / KS; r < (ks + 1) * 16 / KS; ++r) epi(masked, jb - 1, r);
              }
              kf = kn;
            }
          };
          auto pv_block = [&](int jb, bool overlap) {
            constexpr int NSTEP = 2 * NDB;
            V8 vf = v_frag(jb, 0, 0);
#pragma unroll
            for (int st = 0; st < NSTEP; ++st) {
              const int m = st / NDB, db = st % NDB;
              V8 vn = vf;
              if (st + 1 < NSTEP) vn = v_frag(jb, (st + 1) / NDB, (st + 1) % NDB);
              o[db] = F::mfma(vf, pf[jb][m], o[db]);
              if (overlap) {
#pragma unroll
                for (int r = st * 16 / NSTEP; r < (st + 1) * 16 / NSTEP; ++r) epi(masked, NJB - 1, r);
              }
              vf = vn;
            }
          };
#pragma unroll
          for (int jb = 0; jb < NJB; ++jb) s_block(jb);
          scale_s(NJB - 1);
          if (NJB > 1) {
            pv_block(0, true);
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) epi(masked, 0, r);
            pv_block(0, false);
          }
#pragma unroll
          for (int jb = 1; jb < NJB; ++jb) pv_block(jb, false);
        };
        if (full) {
          body(std::false_type{});
        } else {
          make_vis();
          body(std::true_type{});
        }
      } else {
        // Two waves per SIMD: the other wave on the SIMD fills the gaps of
        // this one. The body is cut into small scheduling regions (by
        // sched_barrier) whose instruction order is written out here: left
        // to itself the scheduler chains the SiLU elements one at a time
        // and reads each MFMA operand just before its MFMA.
        //
        // S^T: groups of GS MFMAs (key blocks alternate, so consecutive
        // MFMAs are independent); the K fragments of group g+1 are read
        // while group g multiplies.
        constexpr int NS = KS * NJB;        // S MFMAs per tile
        constexpr int GS = (RAB || MSK) ? 1 : 2;  // MFMAs per group (rab / mask prefetch holds registers)
        constexpr int NGS = NS / GS;
        static_assert(NS % GS == 0, "S groups");
        auto s_kf = [&](int q) { return k_frag(q % NJB, q / NJB); };  // q-th S MFMA: ks = q / NJB, jb = q % NJB
        V8 kf[2][GS];
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[jb][r] = 0.f;
#pragma unroll
        for (int e = 0; e < GS; ++e) kf[0][e] = s_kf(e);
#pragma unroll
        for (int g = 0; g < NGS; ++g) {
          if (g + 1 < NGS) {
#pragma unroll
            for (int e = 0; e < GS; ++e) kf[(g + 1) & 1][e] = s_kf((g + 1) * GS + e);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int e = 0; e < GS; ++e) {
            const int q = g * GS + e;
            sacc[q % NJB] = F::mfma(kf[g & 1][e], qf[q / NJB], sacc[q % NJB]);
          }
          if constexpr (SPREAD) {
            if (spread) {
#pragma unroll
              for (int q = g * NQ / NGS; q < (g + 1) * NQ / NGS; ++q) dma_part(q);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // O^T operands: groups of GP MFMAs in (jb, m, db) order, V^T
        // fragments one group ahead; group 0 is read during the epilogue.
        constexpr int NP = NJB * 2 * NDB;
        constexpr int GP = (RAB || MSK || NDB < 2) ? 1 : 2;
        constexpr int NGP = NP / GP;
        static_assert(NDB % GP == 0, "PV groups");
        auto p_vf = [&](int q) { return v_frag(q / (2 * NDB), (q / NDB) % 2, q % NDB); };
        V8 vf[2][GP];
#pragma unroll
        for (int e = 0; e < GP; ++e) vf[0][e] = p_vf(e);
        auto epi_all = [&](auto masked) {
#pragma unroll
          for (int jb = 0; jb < NJB; ++jb) scale_s(jb);
#pragma unroll
          for (int jb = 0; jb < NJB; ++jb) epi_block(masked, jb);
        };
        if (full) {
          epi_all(std::false_type{});
        } else {
          make_vis();
          epi_all(std::true_type{});
        }
#pragma unroll
        for (int g = 0; g < NGP; ++g) {
          if (g + 1 < NGP) {
#pragma unroll
            for (int e = 0; e < GP; ++e) vf[(g + 1) & 1][e] = p_vf((g + 1) * GP + e);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int e = 0; e < GP; ++e) {
            const int q = g * GP + e, jb = q / (2 * NDB), m = (q / NDB) % 2, db = q % NDB;
            o[db] = F::mfma(vf[g & 1][e], pf[jb][m], o[db]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };

    // Step t of group g works on tile n_begin + KSP t + g; every group runs
    // the same number of steps (and barriers).
    for (int t = 0; t < n_steps; t += 2) {
      step(t, Buf0{});
      if (t + 1 < n_steps) step(t + 1, Buf1{});
    }

    // Every wave is done with the K/V buffers past this barrier; they serve
    // as exchange and staging space below.
    __syncthreads();
    if constexpr (KSP > 1) {
      // Group 1 hands its partial O^T to group 0 (same lane, same register).
      char* xch = wave == 0 ? smem_k0[KSP - 1] : wave == 1 ? smem_v0[KSP - 1] : wave == 2 ? smem_k1[KSP - 1] : smem_v1[KSP - 1];
      int ln = lane;
      asm volatile("" : "+v"(ln));
      if (GRP == 1) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            f32x4_t y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = o[db][4 * a + e];
            *(f32x4_t*)(xch + ((db * 4 + a) * 64 + ln) * 16) = y;
          }
      }
      __syncthreads();
      if (GRP == 0) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const f32x4_t y = *(const f32x4_t*)(xch + ((db * 4 + a) * 64 + ln) * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[db][4 * a + e] += y[e];
          }
      }
    }
    // Lane holds query l32, features d = 32 db + 8 a + 4 half + 0..3.
    if (GRP == 0 && n_chunks > 1) {
      // Split item: store this chunk's fp32 partial; the reduction kernel
      // sums the chunks in order (deterministic) and writes O.
      if (row_ok) {
        float* mine = p.partials + ((size_t)(slot0 + chunk) * p.n_hg + hg) * (kWaves * kRowsPerWave * D) +
                      (size_t)(lw * kRowsPerWave + l32) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            f32x4_t y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = o[db][4 * a + e];
            *(f32x4_t*)(mine + db * 32 + 8 * a + 4 * half) = y;
          }
      }
    } else if (GRP == 0) {
      // Stage the wave's 32 x D output rows through LDS (its own K/V
      // buffer) and write them back as whole rows, 16 bytes per lane.
      char* stg = wave == 0 ? smem_k0[0] : wave == 1 ? smem_v0[0] : wave == 2 ? smem_k1[0] : smem_v1[0];
      // The lane index is re-read here so that the address arithmetic below
      // is not hoisted out of the item loop (it would hold registers there).
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int r32 = ln & 31, hf = ln >> 5;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          T y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = (T)(o[db][4 * a + e] * p.out_mul);
          const int f0 = db * 32 + 8 * a + 4 * hf;
          *(u32x2_t*)(stg + r32 * ROW_B + (((f0 >> 3) ^ swz<D>(r32)) * 16) + (f0 & 7) * 2) = *(const u32x2_t*)y;
        }
      __builtin_amdgcn_wave_barrier();
      constexpr int CPR = D / 8;  // 16-byte chunks per output row
      const int row0 = q_lo + rb * kRowsPerWave;
#pragma unroll
      for (int it = 0; it < kRowsPerWave * CPR / 64; ++it) {
        const int idx = it * 64 + ln, row = idx / CPR, c = idx % CPR;
        const u32x4_t x = *(const u32x4_t*)(stg + row * ROW_B + ((c ^ swz<D>(row)) * 16));
        if (row0 + row < s.Lq) *(u32x4_t*)((T*)p.out + ((size_t)(s.q_tok0 + row0 + row) * p.Hq + h) * D + c * 8) = x;
      }
    }
    if (tid == 0) sh_item[parity] = w_next;
    __syncthreads();
    w = __builtin_amdgcn_readfirstlane(sh_item[parity]);  // uniform: keeps item state in SGPRs
    parity ^= 1;
  }
  };
  if (KSP == 1 || wave_id < kWaves)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, KSP - 1>{});
  if (dyn) leave_queue(p);
}

// ------------------------------------------------------------------------
// FP8 forward (the feature table's FP8 quantization row, "cast": element
// quantization with no scale). Q, K and V are OCP E4M3 (FN) bytes; both
// products run on v_mfma_f32_32x32x64_f8f6f4 with E4M3 operands and fp32
// accumulation; P = silu(alpha S) is cast to E4M3 in between (nearest, ties
// to even, saturating at 448: the convert rounds to nearest even but turns
// values past the format into NaN, so P is first clamped to 448); O is
// stored in bf16. head_dim 128, no rab or user mask, jagged calls with equal
// Q and K lengths.
//
// Layouts (checked on the device): the f8f6f4 MFMA maps the 32 bytes of a
// lane to k in the same way for A and B, so a product only needs A and B
// filled with the same key / feature order; its output layout is that of
// the 16-bit kernel's 32x32 MFMA (lane = query, 16 keys or features per
// lane). ds_read_b64_tr_b8 works on 16-lane groups: lane t of a group
// receives byte t % 8 of the 8-byte reads of lanes 2i + t / 8, i = 0..7.
//
// K and V tiles are 64 rows of 128 bytes in LDS, with no padding; the
// 16-byte chunk c of key row k sits at chunk slot c ^ swz(k) (the DMA loads
// the chunk its slot needs, so the swizzle costs nothing). K uses
// (k >> 1) & 7: the 16 rows of a 16-lane K-fragment read fill all 64 banks.
// V uses ((k >> 3) & 3) << 1 with P's key order below: the 8 rows x 2
// chunks a 32-lane half of a transposing V read touches fill all 64 banks.
//
// O^T += V^T P^T: lane (query n, half h) of the B operand holds, at byte
// 8 q + i (q, i = 0..7), P for key 32 (q/2) + 8 (i/2) + 4 h + 2 (q%2) + i%2
// -- which is element 4 (i/2) + 2 (q%2) + i%2 of S^T block q/2 in the same
// lane -- and the A operand's transposing reads bring V rows in that order.
// ------------------------------------------------------------------------
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

__device__ inline f32x16_t mfma_e4m3(i32x8_t a, i32x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ inline i32x2_t lds_read_tr8(const void* addr) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)addr);
#else
  return i32x2_t{};
#endif
}

__device__ inline int swz_k8(int k) { return (k >> 1) & 7; }
__device__ inline int swz_v8(int k) { return ((k >> 3) & 3) << 1; }

template <bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void fwd_fp8_kernel(KParams p) {
  using TO = __bf16;
  constexpr int D = 128, BN = 64, ROW = D;  // bytes per E4M3 row
  constexpr int TILE_B = BN * ROW;          // 8 KB per K or V tile
  constexpr int NBLK = TILE_B / 1024;       // 1 KB DMA blocks per tile
  constexpr int BLK_W = NBLK / kWaves;      // per wave
  constexpr int NDB = D / 32;               // 32-feature blocks of O^T
  constexpr int KS = D / 64;                // k steps of S^T
  constexpr int NJB = BN / 32;              // 32-key blocks per tile
  constexpr int OUT_ROW_B = D * 2;          // bf16 output row
  static_assert(NBLK % kWaves == 0, "DMA blocks per wave");

  __shared__ __attribute__((aligned(1024))) char smem_k0[TILE_B];
  __shared__ __attribute__((aligned(1024))) char smem_v0[TILE_B];
  __shared__ __attribute__((aligned(1024))) char smem_k1[TILE_B];
  __shared__ __attribute__((aligned(1024))) char smem_v1[TILE_B];
  __shared__ int sh_item[2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const bool direct = p.direct_items > 0;
  const int n_work = direct ? p.direct_items : *p.n_items * p.n_hg;
  const int hpw = 1 << p.hpw_log2;
  const uint32_t row_stride_b = (uint32_t)p.Hk * ROW;

  // DMA geometry of this lane: block blk = wave + kWaves u, 16-byte slot
  // blk * 64 + lane = key row slot / 8 of the tile, chunk slot slot % 8,
  // which receives chunk (slot % 8) ^ swz(row) of that row.
  uint32_t dma_k_off[BLK_W], dma_v_off[BLK_W];
#pragma unroll
  for (int u = 0; u < BLK_W; ++u) {
    const int sl = (wave + kWaves * u) * 64 + lane, row = sl >> 3, pos = sl & 7;
    dma_k_off[u] = (uint32_t)row * row_stride_b + 16u * (uint32_t)(pos ^ swz_k8(row));
    dma_v_off[u] = (uint32_t)row * row_stride_b + 16u * (uint32_t)(pos ^ swz_v8(row));
  }
  // Transposing V reads: lane t16 = lane % 16 of its 16-lane group G reads,
  // for read q, key row key8(q) at bytes 8 cs of chunk 2 db + (G & 1).
  const int G = lane >> 4, t16 = lane & 15, ki = t16 >> 1, cs = t16 & 1;
  auto key8 = [&](int q) { return 32 * (q >> 1) + 8 * (ki >> 1) + 4 * half + 2 * (q & 1) + (ki & 1); };

  const bool dyn = (int)gridDim.x < n_work;
  int w = blockIdx.x, parity = 0;
  while (w < n_work) {
    int w_next = n_work;
    if (dyn && tid == 0) w_next = (int)gridDim.x + atomicAdd(p.counter, 1);
    const int item = w / p.n_hg;
    const int hg = w - item * p.n_hg;
    int b, qt;
    if (direct) {
      qt = p.n_qt_max - 1 - item / p.batch;
      b = item - (p.n_qt_max - 1 - qt) * p.batch;
    } else {
      const int packed = p.items[2 * item];
      b = packed >> 16;
      qt = packed & 0xffff;
    }
    const Seq s = load_seq<false>(p, b, CAUSAL);
    if (direct && qt * p.bm >= s.Lq) break;
    const int h = hg * hpw + (wave & (hpw - 1));
    const int rb = wave >> p.hpw_log2;
    const int hk = (hg * hpw) / p.group;
    const int q_lo = qt * p.bm;
    const int q_hi = min(q_lo + p.bm, s.Lq);
    const int i_lo = s.Lh + q_lo, i_hi = s.Lh + q_hi - 1;
    const int q_loc = q_lo + rb * kRowsPerWave + l32;
    const bool row_ok = q_loc < s.Lq;
    const bool wave_active = q_lo + rb * kRowsPerWave < s.Lq;
    const int i = s.Lh + q_loc;

    // K and V tile kt into LDS; rows past the sequence repeat its last row
    // (finite, and P is zero there).
    auto dma_tile = [&](int kt, char* kbuf, char* vbuf) {
      const int j0 = kt * BN;
      if (j0 + BN <= s.L) {
        const char* kb = (const char*)p.k + ((size_t)(s.k_tok0 + j0) * p.Hk + hk) * ROW;
        const char* vb = (const char*)p.v + ((size_t)(s.k_tok0 + j0) * p.Hk + hk) * ROW;
#pragma unroll
        for (int u = 0; u < BLK_W; ++u) {
          const int blk = wave + kWaves * u;
          dma16(kb + dma_k_off[u], kbuf + blk * 1024);
          dma16(vb + dma_v_off[u], vbuf + blk * 1024);
        }
      } else {
#pragma unroll
        for (int u = 0; u < BLK_W; ++u) {
          const int blk = wave + kWaves * u;
          const int sl = blk * 64 + lane, row = sl >> 3, pos = sl & 7;
          const int j = min(j0 + row, s.L - 1);
          const char* base = (const char*)p.k + ((size_t)(s.k_tok0 + j) * p.Hk + hk) * ROW;
          const char* vbase = (const char*)p.v + ((size_t)(s.k_tok0 + j) * p.Hk + hk) * ROW;
          dma16(base + 16 * (pos ^ swz_k8(row)), kbuf + blk * 1024);
          dma16(vbase + 16 * (pos ^ swz_v8(row)), vbuf + blk * 1024);
        }
      }
    };

    const Tiles tr = tile_range(s, i_lo, i_hi, p.g, p.win, CAUSAL, BN);
    const int n_tiles = tile_count(tr);
    auto tile_at = [&](int n) { return nth_tile(tr, n); };
    if (n_tiles > 0) dma_tile(tile_at(0), smem_k0, smem_v0);

    // Q fragments (B operand of S^T = K Q^T): lane (query l32, half) holds
    // features 64 ks + 32 half .. + 31 of its row, as K's A operand does.
    i32x8_t qf[KS];
    {
      const char* qrow = (const char*)p.q + ((size_t)(s.q_tok0 + q_loc) * p.Hq + h) * ROW + 32 * half;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4_t x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
        if (row_ok) {
          x0 = *(const u32x4_t*)(qrow + 64 * ks);
          x1 = *(const u32x4_t*)(qrow + 64 * ks + 16);
        }
        qf[ks] = i32x8_t{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
      }
    }
    const int hi_i = (i < s.nc) ? max(i, s.nc - 1) : i;
    const int tlo_i = (p.g <= 0) ? s.H : (i >= s.H ? s.H + ((i - s.H) / p.g) * p.g : INT_MAX);
    const int a_i = CAUSAL ? min(hi_i, s.H - 1) : s.L - 1;
    const int b_i = CAUSAL ? max(tlo_i, s.H) : INT_MAX;
    // Local window (p.win > 0, causal only): row i sees no key below
    // i - win + 1, and a tile is full only if every row of the item sees its
    // first key. Both are formed per tile from the kernel argument, so no
    // register holds them across the loop.
    const bool windowed = CAUSAL && p.win > 0;

    f32x16_t o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

    auto step = [&](int n, auto bufc) {
      constexpr int BUF = decltype(bufc)::value;
      const bool has_tile = n < n_tiles;
      const int kt = tile_at(has_tile ? n : 0);
      wait_vmem_all();
      __syncthreads();
      if (n + 1 < n_tiles) {
        if constexpr (BUF == 0) dma_tile(tile_at(n + 1), smem_k1, smem_v1); else dma_tile(tile_at(n + 1), smem_k0, smem_v0);
      }
      if (!wave_active || !has_tile) return;
      const char* kbuf = BUF == 0 ? smem_k0 : smem_k1;
      const char* vbuf = BUF == 0 ? smem_v0 : smem_v1;
      const int j0 = kt * BN;
      const int j1 = min(j0 + BN, s.L);
      const bool full = (j0 + BN <= s.L) && (!windowed || j0 >= i_hi - p.win + 1) &&
                        (!CAUSAL || ((j1 - 1 <= i_lo) && (j1 <= s.H)) || ((i_hi < s.nc) && (j1 <= s.nc)));

      // S^T = K Q^T: lane (key row, half) reads features 64 ks + 32 half .. + 31.
      f32x16_t sacc[NJB];
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        const int row = jb * 32 + l32;
        const char* rbase = kbuf + row * ROW;
        const int sw = swz_k8(row);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int c0 = 4 * ks + 2 * half;
          const u32x4_t a0 = *(const u32x4_t*)(rbase + 16 * (c0 ^ sw));
          const u32x4_t a1 = *(const u32x4_t*)(rbase + 16 * ((c0 + 1) ^ sw));
          const i32x8_t kf = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
          const f32x16_t zero = {};
          sacc[jb] = mfma_e4m3(kf, qf[ks], ks == 0 ? zero : sacc[jb]);
        }
      }

      // Epilogue: P = min(silu(alpha s), 448), cast to E4M3, packed as the
      // B operand of O^T (byte order in the comment above the kernel). Full
      // tiles skip the visibility bit-select (two straight-line copies).
      uint32_t vis[NJB];
      i32x8_t pb = {};
      auto epilogue = [&](auto masked) {
        if constexpr (decltype(masked)::value) {
#pragma unroll
          for (int jb = 0; jb < NJB; ++jb) {
            const int jbase = j0 + jb * 32 + 4 * half;
            const int lo_end = a_i - jbase + 1, hi_beg = b_i == INT_MAX ? 32 : b_i - jbase, hi_end = i - jbase + 1;
            vis[jb] = low_bits(lo_end) | (low_bits(hi_end) & ~low_bits(hi_beg));
            if (windowed) vis[jb] &= ~low_bits(i - p.win + 1 - jbase);
          }
        }
        auto pval = [&](int jb, int r) -> float {
          float sv = sacc[jb][r];
          if constexpr (decltype(masked)::value) {
            // Masked keys get s = +0 (bitwise AND with the visibility bit), hence p = 0 exactly.
            const int off = 8 * (r / 4) + (r % 4);
            const int keep = (int)(vis[jb] << (31 - off)) >> 31;
            sv = __builtin_bit_cast(float, __builtin_bit_cast(int, sv) & keep);
          }
          const float a = sv * p.alpha;
          const float e = __builtin_amdgcn_exp2f(a * -kLog2e);
          const float pv = a * __builtin_amdgcn_rcpf(1.f + e);
          return __builtin_fminf(pv, 448.f);
        };
        // Word 2 q + w holds bytes 8 q + 4 w .. + 3, i.e. i2 = 2 w (low half)
        // and i2 = 2 w + 1 (high half) of the pairs (i, i + 1) = (2 i2, 2 i2 + 1).
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int wh = 0; wh < 2; ++wh) {
            const int jb = q >> 1, r_lo = 4 * (2 * wh) + 2 * (q & 1), r_hi = 4 * (2 * wh + 1) + 2 * (q & 1);
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(pval(jb, r_lo), pval(jb, r_lo + 1), 0, false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(pval(jb, r_hi), pval(jb, r_hi + 1), word, true);
            pb[2 * q + wh] = word;
          }
      };
      if (full)
        epilogue(std::false_type{});
      else
        epilogue(std::true_type{});

      // O^T += V^T P^T: four transposing reads per 32-feature block.
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        i32x2_t part[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = key8(q);
          part[q] = lds_read_tr8(vbuf + row * ROW + 16 * ((2 * db + (G & 1)) ^ swz_v8(row)) + 8 * cs);
        }
        const i32x8_t vf = {part[0][0], part[0][1], part[1][0], part[1][1], part[2][0], part[2][1], part[3][0], part[3][1]};
        o[db] = mfma_e4m3(vf, pb, o[db]);
      }
    };
    for (int t = 0; t < n_tiles; t += 2) {
      step(t, std::integral_constant<int, 0>{});
      if (t + 1 < n_tiles) step(t + 1, std::integral_constant<int, 1>{});
    }

    // Output: stage the wave's 32 x D bf16 rows through LDS (its own 8 KB
    // buffer) and store whole rows, 16 bytes per lane.
    __syncthreads();
    {
      char* stg = wave == 0 ? smem_k0 : wave == 1 ? smem_v0 : wave == 2 ? smem_k1 : smem_v1;
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int r32 = ln & 31, hf = ln >> 5;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          TO y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = (TO)(o[db][4 * a + e] * p.out_mul);
          const int f0 = db * 32 + 8 * a + 4 * hf;
          *(u32x2_t*)(stg + r32 * OUT_ROW_B + (((f0 >> 3) ^ swz<D>(r32)) * 16) + (f0 & 7) * 2) = *(const u32x2_t*)y;
        }
      __builtin_amdgcn_wave_barrier();
      constexpr int CPR = D / 8;
      const int row0 = q_lo + rb * kRowsPerWave;
#pragma unroll
      for (int it = 0; it < kRowsPerWave * CPR / 64; ++it) {
        const int idx = it * 64 + ln, row = idx / CPR, c = idx % CPR;
        const u32x4_t x = *(const u32x4_t*)(stg + row * OUT_ROW_B + ((c ^ swz<D>(row)) * 16));
        if (wave_active && row0 + row < s.Lq)
          *(u32x4_t*)((TO*)p.out + ((size_t)(s.q_tok0 + row0 + row) * p.Hq + h) * D + c * 8) = x;
      }
    }
    if (tid == 0) sh_item[parity] = w_next;
    __syncthreads();
    w = __builtin_amdgcn_readfirstlane(sh_item[parity]);
    parity ^= 1;
  }
  if (dyn) leave_queue(p);
}

// ------------------------------------------------------------------------
// Split-K reduction: for each split item and head group, O = out_mul *
// (partial of chunk 0 + chunk 1 + ...), summed in chunk order so the result
// does not depend on which workgroup finished first.
// ------------------------------------------------------------------------
template <typename T, int D, bool PAGED>
__global__ __launch_bounds__(kThreads) void reduce_kernel(KParams p) {
  constexpr int SLOT_FLOATS = kWaves * kRowsPerWave * D;
  const int hpw = 1 << p.hpw_log2;
  // Work unit: (split item, head group, 32-row block of the partial tile);
  // blocks without rows of the sequence are skipped whole. Each thread sums
  // its float4s over the chunks in chunk order (deterministic), with the
  // loads of four chunks in flight at a time. The first entry is read
  // together with the count (every workgroup's first entry lies inside the
  // split list's allocation: the grid is at most half the slots times the
  // head groups and row blocks), so the two loads overlap.
  auto entry = [&](int it) { return *(const u32x4_t*)(p.split_items + 4 * it); };
  u32x4_t e = entry(blockIdx.x / (p.n_hg * kWaves));
  const int n_work = *p.n_split * p.n_hg * kWaves;
  for (int w = blockIdx.x; w < n_work; w += gridDim.x) {
    const int it = w / (p.n_hg * kWaves), rest = w - it * (p.n_hg * kWaves);
    const int hg = rest / kWaves, wv = rest - hg * kWaves;
    if (w != (int)blockIdx.x) e = entry(it);
    const int packed = (int)e[0], meta = (int)e[1];
    const int qt = packed & 0xffff;
    const int nk = (meta >> 16) & 0xff, slot0 = meta & 0xffff;
    const int q_tok0 = (int)e[2], Lq = (int)e[3];
    const int rblk = wv >> p.hpw_log2;
    const int row0 = qt * p.bm + rblk * kRowsPerWave;
    const int rows = min(Lq - row0, kRowsPerWave);
    if (rows <= 0) continue;  // uniform: no rows of the sequence in this block
    const int h = hg * hpw + (wv & (hpw - 1));
    const float* base = p.partials + ((size_t)slot0 * p.n_hg + hg) * SLOT_FLOATS + (size_t)wv * kRowsPerWave * D;
    const size_t chunk_stride = (size_t)p.n_hg * SLOT_FLOATS;
    for (int f4 = threadIdx.x; f4 < rows * (D / 4); f4 += kThreads) {
      const int row = f4 / (D / 4), d = (f4 % (D / 4)) * 4;
      const float* src = base + (size_t)row * D + d;
      f32x4_t acc = *(const f32x4_t*)src;
      int k = 1;
      for (; k + 4 <= nk; k += 4) {
        f32x4_t x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = *(const f32x4_t*)(src + (k + u) * chunk_stride);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[c] += x[u][c];
      }
      for (; k < nk; ++k) {
        const f32x4_t x = *(const f32x4_t*)(src + k * chunk_stride);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] += x[c];
      }
      T y[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) y[c] = (T)(acc[c] * p.out_mul);
      *(u32x2_t*)((T*)p.out + ((size_t)(q_tok0 + row0 + row) * p.Hq + h) * D + d) = *(const u32x2_t*)y;
    }
  }
}

// ------------------------------------------------------------------------
// fp32 forward (v_mfma_f32_32x32x2f32). Same structure; V stays row-major in
// LDS because each k step of the second product takes one key per half-wave.
// ------------------------------------------------------------------------
template <int D, int BN, bool CAUSAL, bool RAB, bool PAGED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1))) void fwd_kernel_f32(KParams p) {
  using T = float;
  constexpr int KH = D / 2;    // features per half-wave; k step ks uses feature half*KH + ks
  constexpr int NJB = BN / 32;
  constexpr int NDB = D / 32;
  constexpr int KLD = D + 4;
  constexpr int VLD = D;
  constexpr int CPR = D / 4;   // 16-byte chunks per row
  constexpr int CHUNKS = BN * CPR;
  constexpr int PER_T = (CHUNKS + kThreads - 1) / kThreads;

  __shared__ __attribute__((aligned(16))) float Ks[BN * KLD];
  __shared__ __attribute__((aligned(16))) float Vs[BN * VLD];
  __shared__ int sh_item;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int n_work = *p.n_items * p.n_hg;
  const int hpw = 1 << p.hpw_log2;

  for (int w = next_item(&sh_item, p.counter); w < n_work; w = next_item(&sh_item, p.counter)) {
    const int item = w / p.n_hg;
    const int hg = w - item * p.n_hg;
    const int packed = p.items[2 * item];
    const int meta = p.items[2 * item + 1];
    const int b = packed >> 16, qt = packed & 0xffff;
    const int chunk = (int)((uint32_t)meta >> 24), n_chunks = (meta >> 16) & 0xff, slot0 = meta & 0xffff;
    const Seq s = load_seq<PAGED>(p, b, CAUSAL);
    const int h = hg * hpw + (wave & (hpw - 1));
    const int rb = wave >> p.hpw_log2;
    const int hk = (hg * hpw) / p.group;
    const int q_lo = qt * p.bm;
    const int q_hi = min(q_lo + p.bm, s.Lq);
    const int i_lo = s.Lh + q_lo, i_hi = s.Lh + q_hi - 1;
    const int q_loc = q_lo + rb * kRowsPerWave + l32;
    const bool row_ok = q_loc < s.Lq;
    const bool wave_active = q_lo + rb * kRowsPerWave < s.Lq;
    const int i = s.Lh + q_loc;

    float qf[KH];
    {
      const float* qrow = (const float*)p.q + ((size_t)(s.q_tok0 + q_loc) * p.Hq + h) * D + half * KH;
#pragma unroll
      for (int c = 0; c < KH / 4; ++c) {
        f32x4_t x = {0.f, 0.f, 0.f, 0.f};
        if (row_ok) x = *(const f32x4_t*)(qrow + 4 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[4 * c + e] = x[e];
      }
    }
    const int hi_i = (i < s.nc) ? max(i, s.nc - 1) : i;
    const int tlo_i = (p.g <= 0) ? s.H : (i >= s.H ? s.H + ((i - s.H) / p.g) * p.g : INT_MAX);
    // Local window: row i sees no key below w_i; every row of the item sees
    // the keys from w_full on (both far below 0 without a window).
    const int w_i = (CAUSAL && p.win > 0) ? i - p.win + 1 : -(1 << 30);
    const int w_full = (CAUSAL && p.win > 0) ? i_hi - p.win + 1 : -(1 << 30);
    const Tiles tr = tile_range(s, i_lo, i_hi, p.g, p.win, CAUSAL, BN);
    const int n_tiles = tile_count(tr);

    f32x4_t kreg[PER_T], vreg[PER_T];
    auto tile_at = [&](int n) { return nth_tile(tr, n); };
    auto load_tile = [&](int kt) {
      const int j0 = kt * BN;
#pragma unroll
      for (int u = 0; u < PER_T; ++u) {
        const int c = tid + u * kThreads;
        const int r = c / CPR, col = c % CPR;
        const int j = j0 + r;
        f32x4_t xk = {0.f, 0.f, 0.f, 0.f}, xv = {0.f, 0.f, 0.f, 0.f};
        if ((CHUNKS % kThreads == 0 || c < CHUNKS) && j < s.L) {
          xk = *(const f32x4_t*)(kv_row<float, D, PAGED>(p, s, hk, j, 0) + col * 4);
          xv = *(const f32x4_t*)(kv_row<float, D, PAGED>(p, s, hk, j, 1) + col * 4);
        }
        kreg[u] = xk;
        vreg[u] = xv;
      }
    };
    auto store_tile = [&]() {
#pragma unroll
      for (int u = 0; u < PER_T; ++u) {
        const int c = tid + u * kThreads;
        if (CHUNKS % kThreads == 0 || c < CHUNKS) {
          const int r = c / CPR, col = c % CPR;
          *(f32x4_t*)&Ks[r * KLD + col * 4] = kreg[u];
          *(f32x4_t*)&Vs[r * VLD + col * 4] = vreg[u];
        }
      }
    };

    f32x16_t o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

    if (n_tiles > 0) load_tile(tile_at(0));
    for (int n = 0; n < n_tiles; ++n) {
      const int kt = tile_at(n);
      __syncthreads();
      store_tile();
      __syncthreads();
      if (n + 1 < n_tiles) load_tile(tile_at(n + 1));
      if (!wave_active) continue;
      const int j0 = kt * BN;

      f32x16_t sacc[NJB];
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[jb][r] = 0.f;
#pragma unroll
        for (int c = 0; c < KH / 4; ++c) {
          const f32x4_t a4 = *(const f32x4_t*)&Ks[(jb * 32 + l32) * KLD + half * KH + 4 * c];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sacc[jb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[e], qf[4 * c + e], sacc[jb], 0, 0, 0);
        }
      }

      const int j1 = min(j0 + BN, s.L);
      const bool full = !CAUSAL || ((j0 >= w_full) &&
                                    (((j1 - 1 <= i_lo) && (j1 <= s.H)) || ((i_hi < s.nc) && (j1 <= s.nc))));
      const float* rrow =
          RAB ? (const float*)p.rab + ((size_t)(b * p.rab_heads + (p.rab_heads == 1 ? 0 : h)) * p.max_seq_len + s.Lh +
                 q_loc) * p.max_seq_len
              : nullptr;  // read for rows inside the sequence only
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + jb * 32 + 8 * (r / 4) + 4 * half + (r % 4);
          float x = sacc[jb][r];
          if (RAB) x += (row_ok && j < s.L) ? rrow[j] : 0.f;
          const float e = __builtin_amdgcn_exp2f(x * p.c_exp);
          float pv = x * __builtin_amdgcn_rcpf(1.f + e);
          if (CAUSAL && !full) {
            const bool vis = ((j < s.H) ? (j <= hi_i) : (j >= tlo_i && j <= i)) && (j >= w_i);
            pv = vis ? pv : 0.f;
          }
          sacc[jb][r] = pv;
        }

#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float a = Vs[(jb * 32 + 8 * (r / 4) + 4 * half + (r % 4)) * VLD + db * 32 + l32];
            o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, sacc[jb][r], o[db], 0, 0, 0);
          }
    }

    if (row_ok) {
      float* orow = (float*)p.out + ((size_t)(s.q_tok0 + q_loc) * p.Hq + h) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          f32x4_t y;
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = o[db][4 * a + e] * p.out_mul;
          *(f32x4_t*)(orow + db * 32 + 8 * a + 4 * half) = y;
        }
    }
  }
  leave_queue(p);
}

// ------------------------------------------------------------------------
// Validation of the device side inputs (debug mode): one workgroup checks
// what the page leaves to the caller -- seq_offsets (and seq_offsets_k)
// start at 0 and never decrease, every key sequence fits max_seq_len,
// queries never outnumber their keys; paged calls: page_offsets start at 0
// and never decrease, last_page_len is in [1, page_size] for requests that
// own pages, and history + new tokens fit max_seq_len. It writes 1 to *flag
// when anything fails, else 0.
// ------------------------------------------------------------------------
template <bool PAGED>
__global__ __launch_bounds__(256) void validate_kernel(KParams p, int32_t* flag) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  int mine = 0;
  if (threadIdx.x == 0) {
    mine |= p.seq_offsets[0] != 0;
    if (p.seq_offsets_k) mine |= p.seq_offsets_k[0] != 0;
    if (PAGED) mine |= p.page_offsets[0] != 0;
  }
  for (int b = threadIdx.x; b < p.batch; b += blockDim.x) {
    const int lq = p.seq_offsets[b + 1] - p.seq_offsets[b];
    mine |= lq < 0;
    int lk = lq;
    if (p.seq_offsets_k) {
      lk = p.seq_offsets_k[b + 1] - p.seq_offsets_k[b];
      mine |= lk < 0 || lq > lk;
    }
    if (PAGED) {
      const int np = p.page_offsets[b + 1] - p.page_offsets[b];
      mine |= np < 0;
      const int last = p.last_page_len[b];
      if (np > 0) mine |= last < 1 || last > (1 << p.ps_log2);
      const long long hist = np > 0 ? ((long long)(np - 1) << p.ps_log2) + last : 0;
      mine |= hist + lq > p.max_seq_len;
    } else {
      mine |= lk > p.max_seq_len;
    }
  }
  if (mine) atomicOr(&bad, 1);
  __syncthreads();
  if (threadIdx.x == 0) *flag = bad;
}

// ------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------
constexpr size_t kHeaderBytes = 256;

int heads_per_wg_log2(int group) {
  if (group % 4 == 0) return 2;
  if (group % 2 == 0) return 1;
  return 0;
}

int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

using KernelFn = void (*)(KParams);

// LDS bytes of fwd_kernel's two K/V buffers (the kernel's row padding and
// 1 KB DMA blocks), and whether n side-tensor rings of three tiles fit
// beside them at the kernel's occupancy (two workgroups per CU when WPE is
// 2, one when it is 1; 160 KB of LDS per CU).
template <int D, int BN>
constexpr int kv_lds_bytes() {
  constexpr int ROW_B = D * 2;
  constexpr int KS_B = ROW_B + 16, VS_B = ROW_B + (ROW_B % 256 == 64 ? 0 : 64);
  return 2 * ((BN * KS_B + 1023) / 1024 * 1024 + (BN * VS_B + 1023) / 1024 * 1024);
}
template <int D, int BN, int WPE>
constexpr bool ring_fits(int n) {
  return kv_lds_bytes<D, BN>() + n * 3 * kWaves * kRowsPerWave * BN * 2 + 256 <= (WPE == 2 ? 80 : 160) * 1024;
}

// sq16: rows of max_seq_len elements are 16-byte multiples, so rab and the
// user mask can go through the LDS ring (see fwd_kernel's SQL).
template <typename T, int D, bool PAGED>
KernelFn pick16(bool causal, bool rab, bool ksplit, bool user_mask, bool delta, bool sq16) {
  constexpr int BN = D >= 256 ? 32 : 64;
  constexpr int WPE = D >= 256 ? 1 : 2;
  if (PAGED) return causal ? fwd_kernel<T, D, BN, true, false, true, WPE, 1> : fwd_kernel<T, D, BN, false, false, true, WPE, 1>;
  if (user_mask) {
    // The user-mask kernels hold a second prefetched tile (the mask values).
    // At head_dim 128 they take 32-key tiles, which halves the prefetched
    // and S^T / P registers: measured 86 -> 67 us on the user-mask workload
    // (64-key tiles spilled at two waves per SIMD and ran best at one).
    constexpr int BNM = D == 128 ? 32 : BN;
    // The ring takes the mask, and rab too where both fit.
    constexpr int SQ2 = ring_fits<D, BNM, WPE>(2) ? 3 : ring_fits<D, BNM, WPE>(1) ? 2 : 0;
    constexpr int SQ1 = ring_fits<D, BNM, WPE>(1) ? 2 : 0;
    if (rab)
      return sq16 ? fwd_kernel<T, D, BNM, false, true, false, WPE, 1, true, SQ2>
                  : fwd_kernel<T, D, BNM, false, true, false, WPE, 1, true>;
    return sq16 ? fwd_kernel<T, D, BNM, false, false, false, WPE, 1, true, SQ1>
                : fwd_kernel<T, D, BNM, false, false, false, WPE, 1, true>;
  }
  if constexpr (BN == 64) {
    if (ksplit) {
      if (causal) return rab ? fwd_kernel<T, D, BN, true, true, false, WPE, 2> : fwd_kernel<T, D, BN, true, false, false, WPE, 2>;
      return rab ? fwd_kernel<T, D, BN, false, true, false, WPE, 2> : fwd_kernel<T, D, BN, false, false, false, WPE, 2>;
    }
  }
  // The rab kernels at head_dim 128 take 32-key tiles: half the prefetched
  // rab, S^T and P registers, which removes their register spills (measured
  // 150 -> 133 us on the rab workload). The other kernels measured slower
  // with 32-key tiles.
  constexpr int BNR = D == 128 ? 32 : BN;
  // Calls with separate key offsets (few queries, long key-split items)
  // measured 6 % faster on 32-key tiles at head_dim 128 as well.
  // rab through the LDS ring where it fits.
  constexpr int SQR = ring_fits<D, BNR, WPE>(1) ? 1 : 0;
  if (rab) {
    if (causal)
      return sq16 ? fwd_kernel<T, D, BNR, true, true, false, WPE, 1, false, SQR>
                  : fwd_kernel<T, D, BNR, true, true, false, WPE, 1>;
    return sq16 ? fwd_kernel<T, D, BNR, false, true, false, WPE, 1, false, SQR>
                : fwd_kernel<T, D, BNR, false, true, false, WPE, 1>;
  }
  if (delta) return causal ? fwd_kernel<T, D, BNR, true, false, false, WPE, 1> : fwd_kernel<T, D, BNR, false, false, false, WPE, 1>;
  return causal ? fwd_kernel<T, D, BN, true, false, false, WPE, 1> : fwd_kernel<T, D, BN, false, false, false, WPE, 1>;
}

template <int D, bool PAGED>
KernelFn pick32(bool causal, bool rab) {
  constexpr int BN = 64;
  if (PAGED) return causal ? fwd_kernel_f32<D, BN, true, false, true> : fwd_kernel_f32<D, BN, false, false, true>;
  if (causal) return rab ? fwd_kernel_f32<D, BN, true, true, false> : fwd_kernel_f32<D, BN, true, false, false>;
  return rab ? fwd_kernel_f32<D, BN, false, true, false> : fwd_kernel_f32<D, BN, false, false, false>;
}

// ksplit: use the 8-wave key-split kernel (16-bit, head_dim <= 128, jagged,
// built-in masks). user_mask: mask_type 3 (16-bit jagged only). delta:
// jagged with separate key offsets.
// On return, *wgs_per_cu and *threads give the launch shape.
template <bool PAGED>
KernelFn pick(DType dt, int D, bool causal, bool rab, bool ksplit, bool user_mask, bool delta, bool sq16,
              int* wgs_per_cu, int* threads) {
  if (dt == DType::FP8) {
    // FP8 cast: head_dim 128 jagged calls without rab, user mask or key offsets.
    if (PAGED || D != 128 || rab || user_mask || delta) return nullptr;
    *wgs_per_cu = 2;
    *threads = kThreads;
    return causal ? fwd_fp8_kernel<true> : fwd_fp8_kernel<false>;
  }
  ksplit = ksplit && !PAGED && dt != DType::F32 && D <= 128 && !user_mask;
  if (user_mask && (PAGED || dt == DType::F32)) return nullptr;
  *wgs_per_cu = ksplit ? 1 : ((dt == DType::F32 || D >= 256) ? 1 : 2);
  *threads = ksplit ? 2 * kThreads : kThreads;
  switch (dt) {
    case DType::BF16:
      switch (D) {
        case 32: return pick16<__bf16, 32, PAGED>(causal, rab, ksplit, user_mask, delta, sq16);
        case 64: return pick16<__bf16, 64, PAGED>(causal, rab, ksplit, user_mask, delta, sq16);
        case 128: return pick16<__bf16, 128, PAGED>(causal, rab, ksplit, user_mask, delta, sq16);
        case 256: return pick16<__bf16, 256, PAGED>(causal, rab, ksplit, user_mask, delta, sq16);
      }
      break;
    case DType::F16:
      switch (D) {
        case 32: return pick16<_Float16, 32, PAGED>(causal, rab, ksplit, user_mask, delta, sq16);
        case 64: return pick16<_Float16, 64, PAGED>(causal, rab, ksplit, user_mask, delta, sq16);
        case 128: return pick16<_Float16, 128, PAGED>(causal, rab, ksplit, user_mask, delta, sq16);
        case 256: return pick16<_Float16, 256, PAGED>(causal, rab, ksplit, user_mask, delta, sq16);
      }
      break;
    case DType::F32:
      switch (D) {
        case 32: return pick32<32, PAGED>(causal, rab);
        case 64: return pick32<64, PAGED>(causal, rab);
        case 128: return pick32<128, PAGED>(causal, rab);
      }
      break;
  }
  return nullptr;
}

KernelFn pick_reduce(DType dt, int D, bool paged) {
  switch (dt) {
    case DType::BF16:
      switch (D) {
        case 32: return paged ? reduce_kernel<__bf16, 32, true> : reduce_kernel<__bf16, 32, false>;
        case 64: return paged ? reduce_kernel<__bf16, 64, true> : reduce_kernel<__bf16, 64, false>;
        case 128: return paged ? reduce_kernel<__bf16, 128, true> : reduce_kernel<__bf16, 128, false>;
        case 256: return paged ? reduce_kernel<__bf16, 256, true> : reduce_kernel<__bf16, 256, false>;
      }
      break;
    case DType::F16:
      switch (D) {
        case 32: return paged ? reduce_kernel<_Float16, 32, true> : reduce_kernel<_Float16, 32, false>;
        case 64: return paged ? reduce_kernel<_Float16, 64, true> : reduce_kernel<_Float16, 64, false>;
        case 128: return paged ? reduce_kernel<_Float16, 128, true> : reduce_kernel<_Float16, 128, false>;
        case 256: return paged ? reduce_kernel<_Float16, 256, true> : reduce_kernel<_Float16, 256, false>;
      }
      break;
    default:
      break;
  }
  return nullptr;
}

// Workspace layout (all offsets 256-byte aligned):
//   header: n_items, queue counter, exit counter
//   work list: 2 ints per entry, at most items + split slots entries
//   split counters: one int per (split slot, head group)
//   partial sums: kWaves * 32 * head_dim floats per (split slot, head group)
struct WsLayout {
  size_t items, splits, partials, total;
  int split_slots, n_qt_max, n_hg;
};

constexpr int kSplitUnits = 1024;  // (slot, head group) pairs of partial sums

// Key-range splitting is used when few queries meet long key ranges: the
// paged variant (new tokens against cached histories) and jagged calls with
// their own key offsets. For jagged batches whose queries are the whole
// sequence, the fixed cost of each extra chunk (queue pop, sequence and Q
// loads, partial sums, the reduction launch) outweighed the shorter critical
// path on the measured workloads, so they are not split.
bool use_split(bool split_keys, DType dtype) { return split_keys && dtype != DType::F32 && dtype != DType::FP8; }

// cap > 0: a workspace of at most cap bytes (the static scratch of the
// allocation-free entry point). Split items then get as many partial-sum
// slots as fit, at least 2; the planner picks longer key chunks when slots
// are few, so the result stays correct (only the chunking changes).
WsLayout ws_layout(int32_t batch, int32_t max_q_len, int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                   DType dtype, bool split_keys, size_t cap = 0) {
  WsLayout w{};
  const int group = num_heads_q / num_heads_kv;
  const int hpw_log2 = heads_per_wg_log2(group);
  const int bm = kRowsPerWave * (kWaves >> hpw_log2);
  w.n_hg = num_heads_q >> hpw_log2;
  w.n_qt_max = (max_q_len + bm - 1) / bm;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  auto fill = [&](int slots) {
    w.split_slots = slots;
    const size_t entries = (size_t)batch * w.n_qt_max + slots;
    w.items = kHeaderBytes;
    w.splits = up(w.items + entries * 2 * sizeof(int32_t));
    w.partials = up(w.splits + (size_t)slots * 2 * sizeof(int32_t));
    w.total = w.partials + (size_t)slots * w.n_hg * kWaves * kRowsPerWave * head_dim * sizeof(float);
  };
  int slots = use_split(split_keys, dtype) ? max(2, kSplitUnits / w.n_hg) : 0;
  fill(slots);
  if (cap > 0 && w.total > cap && slots > 2) {
    int lo = 2, hi = slots;  // total grows with the slot count: the largest count that fits
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      fill(mid);
      if (w.total <= cap) lo = mid; else hi = mid - 1;
    }
    fill(lo);
  }
  return w;
}

}  // namespace

size_t fwd_workspace_bytes(int32_t batch, int32_t max_q_len, int32_t num_heads_q, int32_t num_heads_kv,
                           int32_t head_dim, DType dtype, bool split_keys, size_t cap) {
  if (batch < 0 || max_q_len < 0 || num_heads_q <= 0 || num_heads_kv <= 0 || head_dim <= 0) return 0;
  return ws_layout(batch, max_q_len, num_heads_q, num_heads_kv, head_dim, dtype, split_keys, cap).total;
}

namespace {


KParams make_params(const FwdArgs& a) {
  KParams p = {};
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.rab = a.rab;
  p.mask = a.user_mask ? a.mask : nullptr;
  p.seq_offsets_k = a.paged ? nullptr : a.seq_offsets_k;
  p.rab_heads = a.rab_heads == 1 ? 1 : a.num_heads_q;
  p.mask_heads = a.mask_heads == 1 ? 1 : a.num_heads_q;
  p.out = a.out;
  p.seq_offsets = a.seq_offsets;
  p.num_context = a.num_context;
  p.num_targets = a.num_targets;
  p.kv_cache = a.kv_cache;
  p.page_offsets = a.page_offsets;
  p.page_ids = a.page_ids;
  p.last_page_len = a.last_page_len;
  const WsLayout w = ws_layout(a.batch, a.max_seq_len, a.num_heads_q, a.num_heads_kv, a.head_dim, a.dtype,
                               a.paged || a.seq_offsets_k != nullptr, a.workspace_cap);
  char* ws = (char*)a.workspace;
  p.n_items = (int32_t*)ws;
  p.counter = (int32_t*)(ws + 64);
  p.exited = (int32_t*)(ws + 128);
  p.n_split = (int32_t*)(ws + 192);
  p.items = (int32_t*)(ws + w.items);
  p.split_items = (int32_t*)(ws + w.splits);
  p.partials = (float*)(ws + w.partials);
  p.split_slots = w.split_slots;
  p.batch = a.batch;
  p.max_seq_len = a.max_seq_len;
  p.Hq = a.num_heads_q;
  p.Hk = a.num_heads_kv;
  p.group = a.num_heads_q / a.num_heads_kv;
  p.hpw_log2 = heads_per_wg_log2(p.group);
  p.n_hg = a.num_heads_q >> p.hpw_log2;
  p.bm = kRowsPerWave * (kWaves >> p.hpw_log2);
  p.n_qt_max = w.n_qt_max;
  int ps_log2 = 0;
  while (a.paged && (1 << ps_log2) < a.page_size) ++ps_log2;
  p.ps_log2 = ps_log2;
  p.g = a.target_group_size;
  p.win = a.causal ? a.local_window : 0;
  p.rab_vec = (a.max_seq_len % 4) == 0;
  p.alpha = a.alpha;
  // Both kernels evaluate 2^(c s) with c = -alpha*log2(e). The fp32 kernel
  // multiplies by s and folds alpha into the output scale; the 16-bit kernel
  // multiplies by y = c s (Q pre-scaled) and folds -1/log2(e) instead.
  p.c_exp = -a.alpha * kLog2e;
  p.c_q = p.c_exp;
  p.y_mul = 1.f;
  if (a.dtype == DType::F16 && std::fabs(p.c_exp) > 1.f) {
    int k = 0;
    std::frexp(p.c_exp, &k);  // |c_exp| = m 2^k, m in [0.5, 1)
    p.y_mul = std::ldexp(1.f, k);
    p.c_q = std::ldexp(p.c_exp, -k);
  }
  // The fp32 kernel folds alpha into the output scale and the 16-bit kernels
  // -1/log2(e) (see the kernels); the FP8 kernel computes P itself.
  p.out_mul = a.dtype == DType::F32 ? a.out_scale * a.alpha : a.dtype == DType::FP8 ? a.out_scale
                                                                                     : -a.out_scale / kLog2e;
  const bool one_wave = a.dtype == DType::F32 || a.head_dim >= 256;
  // Paged calls: one chunk per two resident workgroups; jagged calls with
  // their own key offsets: one per resident workgroup. Measured on the paged
  // and delta-QK workloads against 1/4x to 8x that (cold, caches flushed by
  // a read): fewer chunks lengthen the critical path; more of them cost
  // chunk set-ups, partial-sum traffic and reduction time, and on the paged
  // workload slow every step (paged 92.8 us at 1x, 101.6 at 2x, 98.4 at 4x;
  // delta-QK 39.6 us at 1x, 38.1 at 2x, 51.7 at 4x).
  p.target_chunks = num_cus() * (one_wave ? 1 : 2) / 2 * (a.paged ? 1 : 2);
  return p;
}

int tile_n(const FwdArgs& a) { return (a.dtype != DType::F32 && a.head_dim >= 256) ? 32 : 64; }


// Items a run may have: (sequence, q tile, head group) plus split chunks.
long long item_bound(const FwdArgs& a, const KParams& p) {
  return ((long long)a.batch * p.n_qt_max + p.split_slots) * p.n_hg;
}

// Direct mode: when every possible item can have its own CU, the 16-bit
// jagged kernel takes item w = blockIdx.x from the full grid and no work
// list is built (the plan phase launches nothing).
bool use_direct(const FwdArgs& a, const KParams& p) {
  return !a.paged && a.dtype != DType::F32 && p.split_slots == 0 && item_bound(a, p) <= num_cus();
}

}  // namespace

hipError_t launch_validate(const FwdArgs& a, int32_t* flag) {
  const KParams p = make_params(a);
  if (a.paged)
    hipLaunchKernelGGL(validate_kernel<true>, dim3(1), dim3(256), 0, a.stream, p, flag);
  else
    hipLaunchKernelGGL(validate_kernel<false>, dim3(1), dim3(256), 0, a.stream, p, flag);
  return hipGetLastError();
}

hipError_t launch_plan(const FwdArgs& a) {
  const KParams p = make_params(a);
  if (use_direct(a, p)) return hipSuccess;
  const int causal = a.causal ? 1 : 0;
  if (tile_n(a) == 32) {
    if (a.paged)
      hipLaunchKernelGGL((plan_kernel<true, 32>), dim3(1), dim3(kPlanThreads), 0, a.stream, p, causal);
    else
      hipLaunchKernelGGL((plan_kernel<false, 32>), dim3(1), dim3(kPlanThreads), 0, a.stream, p, causal);
  } else {
    if (a.paged)
      hipLaunchKernelGGL((plan_kernel<true, 64>), dim3(1), dim3(kPlanThreads), 0, a.stream, p, causal);
    else
      hipLaunchKernelGGL((plan_kernel<false, 64>), dim3(1), dim3(kPlanThreads), 0, a.stream, p, causal);
  }
  return hipGetLastError();
}

hipError_t launch_run(const FwdArgs& a) {
  KParams p = make_params(a);
  const long long upper = item_bound(a, p);
  if (use_direct(a, p)) p.direct_items = (int32_t)upper;
  // A work list that cannot give every CU an item runs on the key-split
  // kernel: one 8-wave workgroup per CU, each item twice as fast.
  const bool ksplit = upper <= num_cus();
  int per_cu = 2, threads = kThreads;
  KernelFn fn = a.paged ? pick<true>(a.dtype, a.head_dim, a.causal, false, false, false, false, false, &per_cu, &threads)
                        : pick<false>(a.dtype, a.head_dim, a.causal, a.rab != nullptr, ksplit, a.user_mask,
                                      a.seq_offsets_k != nullptr, a.max_seq_len % 8 == 0, &per_cu, &threads);
  if (!fn) return hipErrorInvalidValue;
  const long long cap = (long long)num_cus() * per_cu;
  const int grid = (int)(upper < cap ? upper : cap);
  if (grid <= 0) return hipSuccess;
  if (p.direct_items > 0 && grid != p.direct_items) return hipErrorInvalidValue;  // one workgroup per item
  hipLaunchKernelGGL(fn, dim3(grid), dim3(threads), 0, a.stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.split_slots == 0) return err;
  KernelFn red = pick_reduce(a.dtype, a.head_dim, a.paged);
  if (!red) return hipErrorInvalidValue;
  const long long rupper = (long long)(p.split_slots / 2) * p.n_hg * kWaves;
  const long long rcap = (long long)num_cus() * 4;
  hipLaunchKernelGGL(red, dim3((int)(rupper < rcap ? rupper : rcap)), dim3(kThreads), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace hstu
