/*
 * HSTU attention forward: plain float64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or
 * call this file. Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it. It shares no code with the HIP library.
 *
 * What it computes. Source: the RecOps Running Case Documentation page on
 * the HSTU_V1 forward operator (hstu_dense_forward). Its feature table
 * (attention row) defines S = Q K^T, P = silu(S), O = P V per head; its
 * operator introduction lists the fused steps as the QK product, SiLU,
 * scaling, masking and the product with V; its inputs/outputs table defines
 * attn_bias [B, N, S, S], silu_scale (default 1/max_seq_len), alpha,
 * num_context, num_target, target_group_size, mask_type, seq_offsets and the
 * paged inputs kv_cache, page_offsets, page_ids and last_page_len:
 *
 *   O[s_b+i, h, :] = out_scale * sum_{j : vis_b(i,j)}
 *                       silu(alpha * (Q[s_b+i,h,:] . K[s_b+j,hk,:] + R[b,h,i,j]))
 *                       * V[s_b+j, hk, :]
 *   silu(x) = x / (1 + exp(-x)),   hk = floor(h * Hk / Hq)
 *
 * Readings taken where the page is silent (each one is a single place here):
 *   - rab is added to Q.K^T before the alpha scale;
 *   - silu_scale is out_scale, applied after SiLU (it is linear);
 *   - the causal mask with context and targets: clamp nt <= L, H = L - nt,
 *     nc <= H; history keys j < H are seen causally (j <= i) and context
 *     rows (i < nc) also see every context key; target keys j >= H are seen
 *     causally when target_group_size == 0, and otherwise only by target rows
 *     of the same group of target_group_size consecutive targets (j <= i);
 *   - rab is indexed by positions local to the sequence, row stride
 *     max_seq_len;
 *   - GQA maps query head h to kv head floor(h * Hk / Hq) (contiguous groups);
 *   - paged: the new tokens' queries sit right after the cached history,
 *     at absolute positions Lh + t; their keys/values come from k_new/v_new;
 *   - different Q and K lengths (the table's seq_offsets_k and is_delta_qk):
 *     the Lq queries of a sequence are its last Lq positions, i.e. query t
 *     sits at absolute position Lk - Lq + t among the Lk keys (Lq <= Lk);
 *   - rab and the user mask may have one head ([B, 1, S, S], the feature
 *     table's rab broadcast), which then serves every query head; they are
 *     indexed by absolute positions (i, j);
 *   - mask_type 3 (user mask, the table's mask input [B, N, S, S]): every key
 *     of the sequence is a candidate and the mask value m = mask[b,h,i,j]
 *     multiplies P; m == 0 removes the key entirely (it contributes exactly
 *     zero, whatever the score), as the built-in masks do;
 *   - local mask (the feature table's local-mask row, which names the
 *     feature only): a sliding window of W >= 1 positions on the causal
 *     mask -- query i sees key j only when the causal mask above lets it and
 *     i - j < W, for context, history and target pairs alike; W = 0 is no
 *     window, and the window is defined for the causal mask only;
 *   - FP8 "cast" (the feature table's FP8 quantization row): element-level
 *     quantization with no scale. Q, K and V arrive as OCP E4M3 (FN) values
 *     (callers pass them widened to float64), and P = silu(...) is cast to
 *     E4M3 before the product with V: round to nearest, ties to even, on the
 *     E4M3 grid (3 mantissa bits, exponent bias 7, subnormal step 2^-9),
 *     saturating to +-448 beyond the largest finite value (p_fp8 = 1).
 *
 * Every function is a direct loop over the definition; no blocking, no
 * reordering beyond summation order in j and e.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_MASK_CAUSAL 0
#define ORACLE_MASK_NONE 2
#define ORACLE_MASK_CUSTOM 3

/* SiLU, textbook form x * sigmoid(x). */
double hstu_oracle_silu(double x) { return x / (1.0 + exp(-x)); }

/* The OCP E4M3 (FN) value nearest to x, ties to even, saturating at +-448.
 * E4M3 holds sign * 2^(e-7) * (1 + m/8) for biased exponents e = 1..15
 * (the top code 0x7f is NaN, so the largest finite value is 1.75 * 2^8 =
 * 448) and sign * m * 2^-9 for e = 0: for |x| >= 2^-6 the grid step is
 * 2^(floor(log2 |x|) - 3), below it 2^-9. */
double hstu_oracle_e4m3(double x) {
  if (x != x) return x;
  const double a = fabs(x);
  if (a >= 448.0) return x < 0 ? -448.0 : 448.0;
  int e2 = 0;
  (void)frexp(a, &e2); /* a = f 2^e2, f in [0.5, 1): floor(log2 a) = e2 - 1 */
  const double step = (a >= ldexp(1.0, -6)) ? ldexp(1.0, e2 - 1 - 3) : ldexp(1.0, -9);
  double r = nearbyint(a / step) * step; /* the default rounding mode: nearest, ties to even */
  if (r > 448.0) r = 448.0;
  return x < 0 ? -r : r;
}

/* Visibility of key j to query i, both positions local to one sequence of
 * length L, under the reading stated in the header comment (w: the local
 * window, 0 for none). */
int hstu_oracle_vis(int32_t mask_type, int64_t L, int64_t nc, int64_t nt, int64_t g, int64_t w, int64_t i,
                    int64_t j) {
  if (i < 0 || j < 0 || i >= L || j >= L) return 0;
  if (mask_type != ORACLE_MASK_CAUSAL) return 1; /* none, or the user mask decides */
  if (w > 0 && i - j >= w) return 0;             /* outside the local window */
  if (nt < 0) nt = 0;
  if (nt > L) nt = L;
  int64_t H = L - nt;
  if (nc < 0) nc = 0;
  if (nc > H) nc = H;
  if (j < H) return (j <= i) || (i < nc && j < nc);
  if (g <= 0) return j <= i;
  return (i >= H) && ((i - H) / g == (j - H) / g) && (j <= i);
}

/* Fill an L x L 0/1 matrix with hstu_oracle_vis. */
void hstu_oracle_mask(int32_t mask_type, int64_t L, int64_t nc, int64_t nt, int64_t g, int64_t w, uint8_t* out) {
  for (int64_t i = 0; i < L; ++i)
    for (int64_t j = 0; j < L; ++j) out[i * L + j] = (uint8_t)hstu_oracle_vis(mask_type, L, nc, nt, g, w, i, j);
}

/* One output row: query row qrow (pointer to D values), keys/values given as
 * per-position row pointers through a callback-free array of row pointers. */
static void one_row(const double* qrow, const double* const* krows, const double* const* vrows,
                    const double* rabrow /* nullable, indexed by local j */,
                    const double* maskrow /* nullable (mask_type 3), indexed by local j */, int64_t L, int64_t D,
                    int32_t mask_type, int64_t nc, int64_t nt, int64_t g, int64_t w, int64_t i, double alpha,
                    double out_scale, int32_t p_fp8, double* out) {
  for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
  for (int64_t j = 0; j < L; ++j) {
    if (!hstu_oracle_vis(mask_type, L, nc, nt, g, w, i, j)) continue;
    if (maskrow && maskrow[j] == 0.0) continue;
    double s = 0.0;
    for (int64_t e = 0; e < D; ++e) s += qrow[e] * krows[j][e];
    if (rabrow) s += rabrow[j];
    double p = hstu_oracle_silu(alpha * s);
    if (p_fp8) p = hstu_oracle_e4m3(p); /* FP8 cast of P before the product with V */
    if (maskrow) p *= maskrow[j];
    for (int64_t d = 0; d < D; ++d) out[d] += p * vrows[j][d];
  }
  for (int64_t d = 0; d < D; ++d) out[d] *= out_scale;
}

/*
 * Jagged forward.
 *   q   [Tq, Hq, D], k, v [Tk, Hk, D]  (float64, contiguous)
 *   rab [B, rab_heads, max_seq_len, max_seq_len] or NULL (rab_heads 1 or Hq)
 *   mask [B, mask_heads, max_seq_len, max_seq_len], mask_type 3 only
 *   out [Tq, Hq, D]
 *   seq_offsets [B+1] (queries); seq_offsets_k [B+1] (keys) or NULL (same);
 *   num_context, num_targets [B] or NULL.
 * p_fp8 != 0: P is cast to E4M3 before the product with V (FP8 cast).
 * If rows != NULL, only the n_rows (token, head) pairs listed in rows[2*r],
 * rows[2*r+1] are computed, into out[r*D ...] (sampled mode); otherwise all.
 * Returns 0 on success, -1 on invalid arguments.
 */
int hstu_oracle_fwd(const double* q, const double* k, const double* v, const double* rab, const double* mask,
                    double* out, const int64_t* seq_offsets, const int64_t* seq_offsets_k,
                    const int64_t* num_context, const int64_t* num_targets, int64_t B, int64_t max_seq_len, int64_t Hq,
                    int64_t Hk, int64_t D, int64_t rab_heads, int64_t mask_heads, int32_t mask_type, int64_t g,
                    int64_t local_window, double alpha, double out_scale, int32_t p_fp8, const int64_t* rows,
                    int64_t n_rows) {
  if (B < 0 || Hq <= 0 || Hk <= 0 || D <= 0 || Hq % Hk != 0) return -1;
  if (local_window < 0 || (local_window > 0 && mask_type != ORACLE_MASK_CAUSAL)) return -1;
  if ((mask_type == ORACLE_MASK_CUSTOM) != (mask != NULL)) return -1;
  if (rab && rab_heads != 1 && rab_heads != Hq) return -1;
  if (mask && mask_heads != 1 && mask_heads != Hq) return -1;
  const int64_t* koff = seq_offsets_k ? seq_offsets_k : seq_offsets;
  const int64_t T = seq_offsets[B];
  int64_t n_items = rows ? n_rows : T * Hq;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t it = 0; it < n_items; ++it) {
    int64_t t = rows ? rows[2 * it] : it / Hq;
    int64_t h = rows ? rows[2 * it + 1] : it % Hq;
    double* o = rows ? out + it * D : out + (t * Hq + h) * D;
    if (t < 0 || t >= T || h < 0 || h >= Hq) {
      err = 1;
      continue;
    }
    int64_t b = 0;
    while (b < B && !(seq_offsets[b] <= t && t < seq_offsets[b + 1])) ++b;
    if (b == B) {
      err = 1;
      continue;
    }
    const int64_t q0 = seq_offsets[b], Lq = seq_offsets[b + 1] - q0;
    const int64_t k0 = koff[b], L = koff[b + 1] - k0;
    if (Lq > L) {
      err = 1;
      continue;
    }
    const int64_t i = L - Lq + (t - q0); /* absolute position among the keys */
    const int64_t hk = h * Hk / Hq;
    const int64_t nc = num_context ? num_context[b] : 0, nt = num_targets ? num_targets[b] : 0;
    const double** kr = (const double**)malloc(sizeof(double*) * (size_t)(L > 0 ? L : 1));
    const double** vr = (const double**)malloc(sizeof(double*) * (size_t)(L > 0 ? L : 1));
    for (int64_t j = 0; j < L; ++j) {
      kr[j] = k + ((k0 + j) * Hk + hk) * D;
      vr[j] = v + ((k0 + j) * Hk + hk) * D;
    }
    const int64_t hr = rab_heads == 1 ? 0 : h, hm = mask_heads == 1 ? 0 : h;
    const double* rabrow = rab ? rab + ((b * rab_heads + hr) * max_seq_len + i) * max_seq_len : NULL;
    const double* maskrow = mask ? mask + ((b * mask_heads + hm) * max_seq_len + i) * max_seq_len : NULL;
    one_row(q + (t * Hq + h) * D, kr, vr, rabrow, maskrow, L, D, mask_type, nc, nt, g, local_window, i, alpha,
            out_scale, p_fp8, o);
    free(kr);
    free(vr);
  }
  return err ? -1 : 0;
}

/*
 * Paged forward (kv_cache holds the cached history of each request).
 *   q, k_new, v_new [Tq, Hq|Hk, D]: the new tokens, jagged by seq_offsets_q [B+1]
 *   kv_cache [num_pages, 2, page_size, Hk, D]: slot 0 = K, slot 1 = V
 *   page_offsets [B+1], page_ids [page_offsets[B]], last_page_len [B]
 * History length of request b: (n_pages-1)*page_size + last_page_len[b]
 * (0 if it owns no page). Query t of request b sits at absolute position
 * Lh + t in a sequence of length Lh + Tq_b; the mask is applied on absolute
 * positions. rows / n_rows select (new-token index, head) pairs as above.
 */
int hstu_oracle_fwd_paged(const double* q, const double* k_new, const double* v_new, const double* kv_cache,
                          double* out, const int64_t* seq_offsets_q, const int64_t* page_offsets,
                          const int64_t* page_ids, const int64_t* last_page_len, const int64_t* num_context,
                          const int64_t* num_targets, int64_t B, int64_t page_size, int64_t Hq, int64_t Hk, int64_t D,
                          int32_t mask_type, int64_t g, int64_t local_window, double alpha, double out_scale,
                          const int64_t* rows, int64_t n_rows) {
  if (B < 0 || Hq <= 0 || Hk <= 0 || D <= 0 || Hq % Hk != 0 || page_size <= 0) return -1;
  if (local_window < 0 || (local_window > 0 && mask_type != ORACLE_MASK_CAUSAL)) return -1;
  const int64_t Tq = seq_offsets_q[B];
  int64_t n_items = rows ? n_rows : Tq * Hq;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t it = 0; it < n_items; ++it) {
    int64_t t = rows ? rows[2 * it] : it / Hq;
    int64_t h = rows ? rows[2 * it + 1] : it % Hq;
    double* o = rows ? out + it * D : out + (t * Hq + h) * D;
    if (t < 0 || t >= Tq || h < 0 || h >= Hq) {
      err = 1;
      continue;
    }
    int64_t b = 0;
    while (b < B && !(seq_offsets_q[b] <= t && t < seq_offsets_q[b + 1])) ++b;
    if (b == B) {
      err = 1;
      continue;
    }
    const int64_t np = page_offsets[b + 1] - page_offsets[b];
    const int64_t Lh = np > 0 ? (np - 1) * page_size + last_page_len[b] : 0;
    const int64_t q0 = seq_offsets_q[b], Lq = seq_offsets_q[b + 1] - q0;
    const int64_t L = Lh + Lq, i = Lh + (t - q0);
    const int64_t hk = h * Hk / Hq;
    const int64_t nc = num_context ? num_context[b] : 0, nt = num_targets ? num_targets[b] : 0;
    const double** kr = (const double**)malloc(sizeof(double*) * (size_t)(L > 0 ? L : 1));
    const double** vr = (const double**)malloc(sizeof(double*) * (size_t)(L > 0 ? L : 1));
    for (int64_t j = 0; j < Lh; ++j) {
      const int64_t page = page_ids[page_offsets[b] + j / page_size], slot = j % page_size;
      kr[j] = kv_cache + (((page * 2 + 0) * page_size + slot) * Hk + hk) * D;
      vr[j] = kv_cache + (((page * 2 + 1) * page_size + slot) * Hk + hk) * D;
    }
    for (int64_t j = 0; j < Lq; ++j) {
      kr[Lh + j] = k_new + ((q0 + j) * Hk + hk) * D;
      vr[Lh + j] = v_new + ((q0 + j) * Hk + hk) * D;
    }
    one_row(q + (t * Hq + h) * D, kr, vr, NULL, NULL, L, D, mask_type, nc, nt, g, local_window, i, alpha, out_scale,
            0, o);
    free(kr);
    free(vr);
  }
  return err ? -1 : 0;
}

/* Number of threads OpenMP would use (reported by the CPU baseline), and a
 * setter for it (the baseline also times one thread). Not arithmetic. */
#ifdef _OPENMP
#include <omp.h>
int hstu_oracle_num_threads(void) { return omp_get_max_threads(); }
void hstu_oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int hstu_oracle_num_threads(void) { return 1; }
void hstu_oracle_set_num_threads(int n) { (void)n; }
#endif
