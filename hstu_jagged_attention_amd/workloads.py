"""Seeded synthetic inputs for the fused HSTU forward.

This module only draws inputs: it holds none of the method's arithmetic, and
both the HIP path and the float64 oracle consume what it returns. Every draw
uses ``numpy.random.default_rng(seed)`` in a fixed order -- sequence lengths,
num_context, num_targets, Q, K, V, rab, page permutation -- in float32, and
values are then rounded to the case dtype (round-to-nearest-even, via torch
on the CPU). The returned tensors live on the CPU; callers move them.

The five named workloads follow the shapes the HSTU_V1 forward operator page
describes (jagged q/k/v [T, N, D], rab [B, N, S, S], kv_cache
[num_pages, 2, page_size, N, D]); their sizes and distributions are fixed
here, with the readings noted on each function.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Dict, Optional, Sequence, Union

import numpy as np
import torch

MASK_CAUSAL = 0
MASK_NONE = 2
MASK_CUSTOM = 3

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}
# rab and the user mask of an FP8 case are bf16 (the FP8 cast quantizes the
# operands of the two products only).
SIDE_DTYPES = {"f32": "f32", "f16": "f16", "bf16": "bf16", "fp8": "bf16"}

IntSpec = Union[None, int, Sequence[int], tuple]


@dataclass
class JaggedCase:
    name: str
    dtype: str
    q: torch.Tensor  # [Tq, Hq, D]
    k: torch.Tensor  # [Tk, Hk, D]
    v: torch.Tensor  # [Tk, Hk, D]
    rab: Optional[torch.Tensor]  # [B, Hq or 1, S, S] or None
    seq_offsets: np.ndarray  # int64 [B+1], queries
    num_context: Optional[np.ndarray]  # int64 [B] or None
    num_targets: Optional[np.ndarray]  # int64 [B] or None
    max_seq_len: int
    mask_type: int
    target_group_size: int
    alpha: float
    out_scale: float
    seq_offsets_k: Optional[np.ndarray] = None  # int64 [B+1], keys (None: same as queries)
    mask: Optional[torch.Tensor] = None  # [B, Hq or 1, S, S], mask_type 3 only
    local_window: int = 0  # local mask window W (causal only; 0 = none)

    @property
    def batch(self) -> int:
        return int(self.seq_offsets.shape[0] - 1)

    @property
    def lengths(self) -> np.ndarray:
        """Query lengths."""
        return np.diff(self.seq_offsets)

    @property
    def key_lengths(self) -> np.ndarray:
        return self.lengths if self.seq_offsets_k is None else np.diff(self.seq_offsets_k)

    @property
    def num_heads_q(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_heads_kv(self) -> int:
        return int(self.k.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[2])


@dataclass
class PagedCase:
    name: str
    dtype: str
    q: torch.Tensor  # [Tq, Hq, D]
    k_new: torch.Tensor  # [Tq, Hk, D]
    v_new: torch.Tensor  # [Tq, Hk, D]
    kv_cache: torch.Tensor  # [num_pages, 2, page_size, Hk, D]
    seq_offsets_q: np.ndarray  # int64 [B+1]
    page_offsets: np.ndarray  # int64 [B+1]
    page_ids: np.ndarray  # int64 [page_offsets[-1]]
    last_page_len: np.ndarray  # int64 [B]
    history_lengths: np.ndarray  # int64 [B]
    num_context: Optional[np.ndarray]
    num_targets: Optional[np.ndarray]
    page_size: int
    max_seq_len: int
    mask_type: int
    target_group_size: int
    alpha: float
    out_scale: float
    local_window: int = 0

    @property
    def batch(self) -> int:
        return int(self.seq_offsets_q.shape[0] - 1)

    @property
    def new_lengths(self) -> np.ndarray:
        return np.diff(self.seq_offsets_q)

    @property
    def num_heads_q(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_heads_kv(self) -> int:
        return int(self.k_new.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[2])


def _draw_ints(rng: np.random.Generator, spec: IntSpec, n: int) -> Optional[np.ndarray]:
    """None -> None; int -> constant; (lo, hi) tuple -> uniform inclusive; sequence -> as given."""
    if spec is None:
        return None
    if isinstance(spec, (int, np.integer)):
        return np.full(n, int(spec), dtype=np.int64)
    if isinstance(spec, tuple) and len(spec) == 2:
        return rng.integers(spec[0], spec[1] + 1, size=n).astype(np.int64)
    arr = np.asarray(spec, dtype=np.int64)
    assert arr.shape == (n,), (arr.shape, n)
    return arr


def _normal(rng: np.random.Generator, shape, dtype: str, std: float = 1.0) -> torch.Tensor:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return torch.from_numpy(x).to(TORCH_DTYPES[dtype])


def jagged_case(seed: int, lengths: Sequence[int], num_heads_q: int, num_heads_kv: int, head_dim: int,
                dtype: str = "bf16", *, mask_type: int = MASK_CAUSAL, num_context: IntSpec = None,
                num_targets: IntSpec = None, target_group_size: int = 0, rab_std: Optional[float] = None,
                rab_padding_nan: bool = True, max_seq_len: Optional[int] = None, alpha: Optional[float] = None,
                out_scale: Optional[float] = None, name: str = "jagged", q_lengths: Optional[Sequence[int]] = None,
                rab_heads: Optional[int] = None, mask_keep: Optional[float] = None,
                mask_heads: Optional[int] = None, local_window: int = 0) -> JaggedCase:
    """A jagged case with the given sequence lengths.

    Q, K, V ~ N(0, 1). rab ~ N(0, rab_std^2) when rab_std is given, with
    rab_heads heads (default num_heads_q; 1 = one rab for every head); with
    rab_padding_nan the rab entries outside each sequence (row or column
    >= its length) are NaN, so any read of them poisons the output.
    q_lengths (optional, each <= the matching entry of lengths) gives the
    queries of each sequence when they are fewer than its keys: q then holds
    q_lengths[b] rows per sequence and seq_offsets_k the key offsets.
    mask_keep (with mask_type 3) draws a user mask [B, mask_heads, S, S] of
    ones with probability mask_keep, else zeros, NaN outside each sequence.
    alpha defaults to 1/sqrt(head_dim), out_scale to 1/max_seq_len.
    """
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    B = int(lengths.shape[0])
    S = int(max_seq_len if max_seq_len is not None else max(1, int(lengths.max(initial=1))))
    nc = _draw_ints(rng, num_context, B)
    nt = _draw_ints(rng, num_targets, B)
    offsets = np.zeros(B + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(lengths)
    T = int(offsets[-1])
    offsets_q, offsets_k, Tq = offsets, None, T
    if q_lengths is not None:
        ql = np.asarray(q_lengths, dtype=np.int64)
        assert ql.shape == (B,) and (ql <= lengths).all() and (ql >= 0).all()
        offsets_q = np.zeros(B + 1, dtype=np.int64)
        offsets_q[1:] = np.cumsum(ql)
        offsets_k, Tq = offsets, int(offsets_q[-1])
    q = _normal(rng, (Tq, num_heads_q, head_dim), dtype)
    k = _normal(rng, (T, num_heads_kv, head_dim), dtype)
    v = _normal(rng, (T, num_heads_kv, head_dim), dtype)

    def padded_nan(x):
        for b in range(B):
            x[b, :, lengths[b]:, :] = np.nan
            x[b, :, :, lengths[b]:] = np.nan
        return x

    rab = None
    if rab_std is not None:
        x = rng.standard_normal(size=(B, rab_heads or num_heads_q, S, S), dtype=np.float32)
        x *= np.float32(rab_std)
        if rab_padding_nan:
            padded_nan(x)
        rab = torch.from_numpy(x).to(TORCH_DTYPES[SIDE_DTYPES[dtype]])
    mask = None
    if mask_keep is not None:
        m = (rng.random(size=(B, mask_heads or num_heads_q, S, S), dtype=np.float32) < mask_keep).astype(np.float32)
        mask = torch.from_numpy(padded_nan(m)).to(TORCH_DTYPES[SIDE_DTYPES[dtype]])
    return JaggedCase(name=name, dtype=dtype, q=q, k=k, v=v, rab=rab, seq_offsets=offsets_q, num_context=nc,
                      num_targets=nt, max_seq_len=S, mask_type=mask_type, target_group_size=target_group_size,
                      alpha=float(alpha if alpha is not None else 1.0 / math.sqrt(head_dim)),
                      out_scale=float(out_scale if out_scale is not None else 1.0 / S), seq_offsets_k=offsets_k,
                      mask=mask, local_window=int(local_window))


def paged_case(seed: int, history_lengths: Sequence[int], new_lengths: Sequence[int], num_heads_q: int,
               num_heads_kv: int, head_dim: int, dtype: str = "bf16", *, page_size: int = 64,
               mask_type: int = MASK_CAUSAL, num_context: IntSpec = None, num_targets: IntSpec = "new",
               target_group_size: int = 1, max_seq_len: Optional[int] = None, alpha: Optional[float] = None,
               out_scale: Optional[float] = None, extra_pages: int = 0, name: str = "paged",
               local_window: int = 0) -> PagedCase:
    """A paged case: request b has history_lengths[b] cached tokens in
    ceil(h / page_size) pages and new_lengths[b] new tokens (the queries).

    The page pool holds exactly the pages the requests own (plus
    ``extra_pages`` unused ones, filled with NaN so a stray read poisons the
    output) under a seeded random permutation. num_targets="new" makes
    every new token a target (num_targets[b] = new_lengths[b]).
    """
    rng = np.random.default_rng(seed)
    hist = np.asarray(history_lengths, dtype=np.int64)
    newl = np.asarray(new_lengths, dtype=np.int64)
    B = int(hist.shape[0])
    nc = _draw_ints(rng, num_context, B)
    nt = newl.copy() if isinstance(num_targets, str) and num_targets == "new" else _draw_ints(rng, num_targets, B)
    offq = np.zeros(B + 1, dtype=np.int64)
    offq[1:] = np.cumsum(newl)
    Tq = int(offq[-1])
    q = _normal(rng, (Tq, num_heads_q, head_dim), dtype)
    k_new = _normal(rng, (Tq, num_heads_kv, head_dim), dtype)
    v_new = _normal(rng, (Tq, num_heads_kv, head_dim), dtype)
    n_pages_req = (hist + page_size - 1) // page_size
    page_offsets = np.zeros(B + 1, dtype=np.int64)
    page_offsets[1:] = np.cumsum(n_pages_req)
    n_used = int(page_offsets[-1])
    n_pool = n_used + int(extra_pages)
    cache = rng.standard_normal(size=(max(n_pool, 1), 2, page_size, num_heads_kv, head_dim), dtype=np.float32)
    perm = rng.permutation(max(n_pool, 1)).astype(np.int64)
    page_ids = perm[:n_used].copy()
    if extra_pages:
        cache[perm[n_used:]] = np.nan
    last = np.where(n_pages_req > 0, hist - (n_pages_req - 1) * page_size, page_size).astype(np.int64)
    S = int(max_seq_len if max_seq_len is not None else max(1, int((hist + newl).max(initial=1))))
    return PagedCase(name=name, dtype=dtype, q=q, k_new=k_new, v_new=v_new,
                     kv_cache=torch.from_numpy(cache).to(TORCH_DTYPES[dtype]), seq_offsets_q=offq,
                     page_offsets=page_offsets, page_ids=page_ids, last_page_len=last, history_lengths=hist,
                     num_context=nc, num_targets=nt, page_size=page_size, max_seq_len=S, mask_type=mask_type,
                     target_group_size=target_group_size,
                     alpha=float(alpha if alpha is not None else 1.0 / math.sqrt(head_dim)),
                     out_scale=float(out_scale if out_scale is not None else 1.0 / S),
                     local_window=int(local_window))


# ---------------------------------------------------------------------------
# The five named workloads. `batch_scale` < 1 keeps the distributions but
# draws fewer sequences (used for CPU-sized parity cases).
# ---------------------------------------------------------------------------

def tiny_fp32_bidirectional(seed: int = 1) -> JaggedCase:
    """batch 2, lengths {64, 100}, 2 heads MHA, d 32, fp32, no rab, no mask,
    alpha 1/sqrt(32), out_scale 1/100."""
    return jagged_case(seed, [64, 100], 2, 2, 32, "f32", mask_type=MASK_NONE, max_seq_len=100,
                       alpha=1.0 / math.sqrt(32), out_scale=1.0 / 100, name="tiny_fp32_bidirectional")


def bf16_mha_causal(seed: int = 2, batch: int = 8) -> JaggedCase:
    """batch 8, lengths ~ U{256..1024}, 4 heads MHA, d 128, bf16, plain causal
    mask, no rab, alpha 1/sqrt(128), out_scale 1/1024 (max_seq_len = the
    configured bound 1024)."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(256, 1024 + 1, size=batch)
    return jagged_case(seed + 1000, lengths, 4, 4, 128, "bf16", mask_type=MASK_CAUSAL, max_seq_len=1024,
                       alpha=1.0 / math.sqrt(128), out_scale=1.0 / 1024, name="bf16_mha_causal")


def bf16_rab_target(seed: int = 3, batch: int = 32) -> JaggedCase:
    """batch 32, lengths ~ U{512..2048}, 4 heads, d 128, bf16, rab
    [B, 4, 2048, 2048] ~ N(0, 0.1^2) (std 0.1), causal with num_context ~
    U{0..32}, num_targets ~ U{1..64}, target_group_size 1. No alpha/out_scale
    given: alpha 1/sqrt(128), out_scale 1/2048."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(512, 2048 + 1, size=batch)
    return jagged_case(seed + 1000, lengths, 4, 4, 128, "bf16", mask_type=MASK_CAUSAL, num_context=(0, 32),
                       num_targets=(1, 64), target_group_size=1, rab_std=0.1, max_seq_len=2048,
                       alpha=1.0 / math.sqrt(128), out_scale=1.0 / 2048, name="bf16_rab_target")


def fp16_gqa_causal(seed: int = 4, batch: int = 16) -> JaggedCase:
    """batch 16, lengths = clip(round(lognormal(ln 1500, sigma 0.5)), 128,
    4096) (sigma not given; 0.5 taken), 8 query heads on 2 kv heads, d 128,
    fp16, causal, num_targets ~ U{1..32}, target_group_size 1, no context, no
    rab, alpha 1/sqrt(128), out_scale 1/4096."""
    rng = np.random.default_rng(seed)
    lengths = np.clip(np.round(rng.lognormal(math.log(1500.0), 0.5, size=batch)), 128, 4096).astype(np.int64)
    return jagged_case(seed + 1000, lengths, 8, 2, 128, "f16", mask_type=MASK_CAUSAL, num_targets=(1, 32),
                       target_group_size=1, max_seq_len=4096, alpha=1.0 / math.sqrt(128), out_scale=1.0 / 4096,
                       name="fp16_gqa_causal")


def fp8_gqa_causal(seed: int = 8, batch: int = 16) -> JaggedCase:
    """The FP8 cast row on the GQA causal shape: as fp16_gqa_causal (batch
    16, lognormal lengths median 1500 clipped to [128, 4096], 8 query heads
    on 2 kv heads, d 128, causal, num_targets ~ U{1..32}, group size 1,
    alpha 1/sqrt(128), out_scale 1/4096) with Q, K, V drawn N(0, 1) and
    cast to OCP E4M3 (FN); the output is bf16."""
    rng = np.random.default_rng(seed)
    lengths = np.clip(np.round(rng.lognormal(math.log(1500.0), 0.5, size=batch)), 128, 4096).astype(np.int64)
    return jagged_case(seed + 1000, lengths, 8, 2, 128, "fp8", mask_type=MASK_CAUSAL, num_targets=(1, 32),
                       target_group_size=1, max_seq_len=4096, alpha=1.0 / math.sqrt(128), out_scale=1.0 / 4096,
                       name="fp8_gqa_causal")


def fp16_gqa_local(seed: int = 9, batch: int = 16) -> JaggedCase:
    """The local mask on the GQA causal shape: as fp16_gqa_causal (batch 16,
    lognormal lengths median 1500 clipped to [128, 4096], 8 query heads on 2
    kv heads, d 128, fp16, num_targets ~ U{1..32}, group size 1, alpha
    1/sqrt(128), out_scale 1/4096) with a local window of 512 positions (no
    window size is given; 512 keeps a third of the median sequence)."""
    rng = np.random.default_rng(seed)
    lengths = np.clip(np.round(rng.lognormal(math.log(1500.0), 0.5, size=batch)), 128, 4096).astype(np.int64)
    return jagged_case(seed + 1000, lengths, 8, 2, 128, "f16", mask_type=MASK_CAUSAL, num_targets=(1, 32),
                       target_group_size=1, max_seq_len=4096, alpha=1.0 / math.sqrt(128), out_scale=1.0 / 4096,
                       name="fp16_gqa_local", local_window=512)


def bf16_paged_target(seed: int = 5, batch: int = 64) -> PagedCase:
    """64 requests, cached history ~ U{512..4096} in 64-token pages under a
    seeded shuffled block table, 1..64 new target tokens as queries
    (num_targets = new tokens, group size 1), 4 heads, d 128, bf16, causal,
    no rab, alpha 1/sqrt(128), out_scale 1/4160 (4096 + 64)."""
    rng = np.random.default_rng(seed)
    hist = rng.integers(512, 4096 + 1, size=batch)
    newl = rng.integers(1, 64 + 1, size=batch)
    return paged_case(seed + 1000, hist, newl, 4, 4, 128, "bf16", page_size=64, mask_type=MASK_CAUSAL,
                      num_targets="new", target_group_size=1, max_seq_len=4160, alpha=1.0 / math.sqrt(128),
                      out_scale=1.0 / 4160, name="bf16_paged_target")


def bf16_custom_mask(seed: int = 6, batch: int = 16) -> JaggedCase:
    """The user-mask and rab-broadcast features: batch 16, lengths ~
    U{256..1024}, 4 heads, d 128, bf16, mask_type 3 with a mask [B, 4, 1024,
    1024] of ones with probability 1/2, rab [B, 1, 1024, 1024] ~ N(0, 0.1^2)
    shared by the 4 heads, alpha 1/sqrt(128), out_scale 1/1024."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(256, 1024 + 1, size=batch)
    return jagged_case(seed + 1000, lengths, 4, 4, 128, "bf16", mask_type=MASK_CUSTOM, rab_std=0.1, rab_heads=1,
                       mask_keep=0.5, max_seq_len=1024, alpha=1.0 / math.sqrt(128), out_scale=1.0 / 1024,
                       name="bf16_custom_mask")


def bf16_delta_qk(seed: int = 7, batch: int = 32) -> JaggedCase:
    """Different Q and K lengths without paging: batch 32, keys ~
    U{512..2048} per sequence, of which the last 1..64 are the queries
    (targets, group size 1), 4 heads, d 128, bf16, causal, no rab, alpha
    1/sqrt(128), out_scale 1/2048."""
    rng = np.random.default_rng(seed)
    lk = rng.integers(512, 2048 + 1, size=batch)
    lq = rng.integers(1, 64 + 1, size=batch)
    return jagged_case(seed + 1000, lk, 4, 4, 128, "bf16", mask_type=MASK_CAUSAL, num_targets=lq,
                       target_group_size=1, max_seq_len=2048, alpha=1.0 / math.sqrt(128), out_scale=1.0 / 2048,
                       q_lengths=lq, name="bf16_delta_qk")


WORKLOADS: Dict[str, Callable[..., object]] = {
    "tiny_fp32_bidirectional": tiny_fp32_bidirectional,
    "bf16_mha_causal": bf16_mha_causal,
    "bf16_rab_target": bf16_rab_target,
    "fp16_gqa_causal": fp16_gqa_causal,
    "bf16_paged_target": bf16_paged_target,
    "bf16_custom_mask": bf16_custom_mask,
    "bf16_delta_qk": bf16_delta_qk,
    "fp8_gqa_causal": fp8_gqa_causal,
    "fp16_gqa_local": fp16_gqa_local,
}
