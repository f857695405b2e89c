"""Work accounting for the fused HSTU forward: visible (q, k) pairs, the
effective-FLOP count and the algorithmic HBM bytes.

Effective FLOPs count 4 * head_dim per visible (query, key) pair per query
head: 2 * head_dim for the Q.K^T dot product and 2 * head_dim for the P.V
update. Masked pairs are not counted: the kernels skip them.

Row counts use the closed form of the mask (HSTU_V1 forward operator page,
feature table's causal-mask row; context/target geometry as read in the C
header): with nt clamped to [0, L], H = L - nt and nc clamped to [0, H], a
context row (i < nc) sees nc keys, a history row (nc <= i < H) sees i + 1,
and a target row (i >= H) sees i + 1 when target_group_size g == 0 and
H + ((i - H) mod g) + 1 otherwise. The bidirectional mask gives L per row.
A local window W (the feature table's local-mask row, read as: key j is
visible to query i only when i - j < W as well) keeps of those sets only the
keys j >= i - W + 1.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

MASK_CAUSAL = 0
MASK_NONE = 2


def visible_per_row(L: int, nc: int = 0, nt: int = 0, g: int = 0, mask_type: int = MASK_CAUSAL,
                    w: int = 0) -> np.ndarray:
    """Number of visible keys for each query row 0..L-1 of one sequence
    (w: the local window, 0 for none)."""
    L = int(L)
    if L <= 0:
        return np.zeros(0, dtype=np.int64)
    if mask_type == MASK_NONE:
        return np.full(L, L, dtype=np.int64)
    nt = min(max(int(nt), 0), L)
    H = L - nt
    nc = min(max(int(nc), 0), H)
    i = np.arange(L, dtype=np.int64)
    lo = np.maximum(i - int(w) + 1, 0) if w > 0 else np.zeros(L, dtype=np.int64)  # first key in the window
    out = i + 1 - lo
    out[:nc] = nc - lo[:nc]
    if g > 0 and nt > 0:
        t = i[H:]
        gs = H + ((t - H) // g) * g  # first row of the target's group
        out[H:] = np.maximum(H - lo[H:], 0) + t + 1 - np.maximum(gs, lo[H:])
    return out


def pairs_jagged(seq_offsets: Sequence[int], num_context: Optional[Sequence[int]],
                 num_targets: Optional[Sequence[int]], target_group_size: int, mask_type: int,
                 local_window: int = 0) -> int:
    """Visible pairs summed over sequences, for ONE query head."""
    off = np.asarray(seq_offsets, dtype=np.int64)
    total = 0
    for b in range(off.shape[0] - 1):
        L = int(off[b + 1] - off[b])
        nc = 0 if num_context is None else int(num_context[b])
        nt = 0 if num_targets is None else int(num_targets[b])
        total += int(visible_per_row(L, nc, nt, target_group_size, mask_type, local_window).sum())
    return total


def pairs_paged(history_lengths: Sequence[int], new_lengths: Sequence[int], num_context: Optional[Sequence[int]],
                num_targets: Optional[Sequence[int]], target_group_size: int, mask_type: int,
                local_window: int = 0) -> int:
    """Visible pairs of the new-token rows only (the queries), ONE query head."""
    total = 0
    for b in range(len(history_lengths)):
        Lh, Lq = int(history_lengths[b]), int(new_lengths[b])
        nc = 0 if num_context is None else int(num_context[b])
        nt = 0 if num_targets is None else int(num_targets[b])
        rows = visible_per_row(Lh + Lq, nc, nt, target_group_size, mask_type, local_window)
        total += int(rows[Lh:].sum())
    return total


def pairs_delta(key_lengths: Sequence[int], query_lengths: Sequence[int], num_context: Optional[Sequence[int]],
                num_targets: Optional[Sequence[int]], target_group_size: int, mask_type: int,
                local_window: int = 0) -> int:
    """Different Q and K lengths: the queries are the last Lq of Lk
    positions, so only those rows count (ONE query head)."""
    lk = np.asarray(key_lengths, dtype=np.int64)
    lq = np.asarray(query_lengths, dtype=np.int64)
    return pairs_paged(lk - lq, lq, num_context, num_targets, target_group_size, mask_type, local_window)


def user_mask_counts(mask: np.ndarray, lengths: Sequence[int], num_heads_q: int, rab_heads: int = 0):
    """User mask (mask_type 3) [B, Hm, S, S]: returns (visible pairs summed
    over all query heads, distinct rab entries those pairs read when a rab
    with rab_heads heads is given). A pair is visible where the mask value
    inside the sequence is non-zero."""
    total, rab_entries = 0, 0
    Hm = mask.shape[1]
    for b, L in enumerate(lengths):
        L = int(L)
        nz = mask[b, :, :L, :L] != 0  # [Hm, L, L]
        per_head = nz.reshape(Hm, -1).sum(axis=1)
        total += int(per_head.sum()) * (num_heads_q // Hm)
        if rab_heads == 1:
            rab_entries += int(nz.any(axis=0).sum())
        elif rab_heads:
            rab_entries += int(per_head.sum()) * (num_heads_q // Hm)
    return total, rab_entries


def effective_flops(pairs_one_head: int, num_heads_q: int, head_dim: int) -> float:
    return 4.0 * head_dim * float(pairs_one_head) * num_heads_q


def algorithmic_bytes_jagged(T: int, num_heads_q: int, num_heads_kv: int, head_dim: int, elem_bytes: int,
                             rab_pairs_one_head: int = 0, Tk: Optional[int] = None, extra_bytes: float = 0.0,
                             out_bytes: Optional[int] = None) -> float:
    """Compulsory HBM bytes: Q and O once (T query rows), K and V once (Tk
    key rows, default T), rab only for the visible pairs (the method never
    reads masked rab), plus extra_bytes (a user mask, whose every entry
    inside the sequences is read once per mask head). out_bytes: bytes per
    output element when they differ from the inputs' (the FP8 cast writes
    bf16)."""
    qo = T * num_heads_q * head_dim * (elem_bytes + (elem_bytes if out_bytes is None else out_bytes))
    kv = 2.0 * (T if Tk is None else Tk) * num_heads_kv * head_dim * elem_bytes
    rab = float(rab_pairs_one_head) * num_heads_q * elem_bytes
    return qo + kv + rab + extra_bytes


def algorithmic_bytes_paged(Tq: int, history_tokens: int, num_heads_q: int, num_heads_kv: int, head_dim: int,
                            elem_bytes: int) -> float:
    """Q, O, k_new, v_new once plus the cached history K and V once."""
    qo = 2.0 * Tq * num_heads_q * head_dim * elem_bytes
    kv_new = 2.0 * Tq * num_heads_kv * head_dim * elem_bytes
    kv_hist = 2.0 * history_tokens * num_heads_kv * head_dim * elem_bytes
    return qo + kv_new + kv_hist
