"""Pins of the float64 oracle against things other than itself: closed forms,
library routines, hand-worked fixtures, brute force from the English mask
rules, and invariants. CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
from hstu_jagged_attention_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
CAUSAL, NONE = oracle.MASK_CAUSAL, oracle.MASK_NONE


def f64(t):
    return t.double().numpy() if hasattr(t, "double") else np.asarray(t, dtype=np.float64)


# ---------------------------------------------------------------- SiLU
def test_silu_against_library_sigmoid():
    xs = np.concatenate([np.linspace(-40, 40, 801), [-700.0, -1e-300, 0.0, 1e-300, 700.0]])
    for x in xs:
        ref = x * expit(x)
        got = oracle.silu(x)
        assert got == pytest.approx(ref, rel=1e-14, abs=1e-300)


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    for x in [0.1, 0.5, 1.0, 2.5, 7.0, 19.0]:
        # silu(x) - silu(-x) = x (sigma(x) + sigma(-x) = 1)
        assert oracle.silu(x) - oracle.silu(-x) == pytest.approx(x, rel=1e-14)
    assert oracle.silu(60.0) / 60.0 == pytest.approx(1.0, abs=1e-20 + 1e-15)
    # the minimum of x*sigma(x) sits where x*sigma(x) = 1 + x, x* = -1.2784645427610738
    xstar = -1.2784645427610738
    assert oracle.silu(xstar) == pytest.approx(1.0 + xstar, abs=1e-15)
    assert oracle.silu(xstar) <= min(oracle.silu(xstar - 1e-4), oracle.silu(xstar + 1e-4))


# ---------------------------------------------------------------- mask
def mask_from_rules(L, nc, nt, g, mask_type):
    """Sets built from the English rules, independent of the oracle's predicate."""
    if mask_type == NONE:
        return np.ones((L, L), dtype=bool)
    nt = min(max(nt, 0), L)
    H = L - nt
    nc = min(max(nc, 0), H)
    context = set(range(nc))
    history = set(range(nc, H))
    targets = list(range(H, L))
    groups = []
    if g > 0:
        for s in range(H, L, g):
            groups.append(set(range(s, min(s + g, L))))
    M = np.zeros((L, L), dtype=bool)
    for i in range(L):
        if i in context:
            seen = set(context)
        elif i in history:
            seen = set(range(i + 1))
        else:
            if g == 0:
                seen = set(range(i + 1))
            else:
                own = next(gr for gr in groups if i in gr)
                seen = context | history | {j for j in own if j <= i}
        for j in seen:
            M[i, j] = True
    return M


def test_mask_hand_fixtures():
    with open(os.path.join(GOLDEN, "mask_examples.json")) as f:
        data = json.load(f)
    for c in data["cases"]:
        got = oracle.mask_matrix(CAUSAL, c["L"], c["nc"], c["nt"], c["g"])
        np.testing.assert_array_equal(got, np.array(c["mask"], dtype=bool), err_msg=str(c))


def test_mask_bruteforce_random():
    rng = np.random.default_rng(11)
    for _ in range(400):
        L = int(rng.integers(1, 40))
        nc = int(rng.integers(-2, L + 4))
        nt = int(rng.integers(-2, L + 4))
        g = int(rng.choice([0, 1, 2, 3, 5]))
        got = oracle.mask_matrix(CAUSAL, L, nc, nt, g)
        np.testing.assert_array_equal(got, mask_from_rules(L, nc, nt, g, CAUSAL), err_msg=str((L, nc, nt, g)))
    np.testing.assert_array_equal(oracle.mask_matrix(NONE, 7), np.ones((7, 7), dtype=bool))


def closed_form_counts(L, nc, nt, g):
    nt = min(max(nt, 0), L)
    H = L - nt
    nc = min(max(nc, 0), H)
    out = []
    for i in range(L):
        if i < nc:
            out.append(nc)
        elif i < H or g == 0:
            out.append(i + 1)
        else:
            out.append(H + (i - H) % g + 1)
    return np.array(out)


def test_mask_row_counts_closed_form():
    rng = np.random.default_rng(12)
    for _ in range(300):
        L = int(rng.integers(1, 60))
        nc, nt = int(rng.integers(0, L + 2)), int(rng.integers(0, L + 2))
        g = int(rng.choice([0, 1, 3, 4]))
        M = oracle.mask_matrix(CAUSAL, L, nc, nt, g)
        np.testing.assert_array_equal(M.sum(1), closed_form_counts(L, nc, nt, g))


def test_target_never_sees_other_groups():
    for (L, nc, nt, g) in [(20, 3, 9, 1), (20, 0, 12, 3), (33, 5, 17, 4)]:
        M = oracle.mask_matrix(CAUSAL, L, nc, nt, g)
        H = L - nt
        for i in range(H, L):
            for j in range(H, L):
                if (i - H) // g != (j - H) // g:
                    assert not M[i, j]


# ---------------------------------------------------------------- forward
def small_case(seed, lengths, Hq=2, Hk=2, D=8, mask=CAUSAL, nc=None, nt=None, g=0, rab=False, S=None,
               local_window=0):
    return wl.jagged_case(seed, lengths, Hq, Hk, D, "f32", mask_type=mask, num_context=nc, num_targets=nt,
                          target_group_size=g, rab_std=0.5 if rab else None, max_seq_len=S, alpha=0.7,
                          local_window=local_window,
                          out_scale=0.3)


def run_oracle(c, q=None, k=None, v=None, **over):
    kw = dict(rab=None if c.rab is None else f64(c.rab), mask=None if c.mask is None else f64(c.mask),
              seq_offsets_k=c.seq_offsets_k, num_context=c.num_context, num_targets=c.num_targets,
              max_seq_len=c.max_seq_len, mask_type=c.mask_type, target_group_size=c.target_group_size,
              alpha=c.alpha, out_scale=c.out_scale, local_window=c.local_window)
    kw.update(over)
    return oracle.hstu_fwd(f64(c.q) if q is None else q, f64(c.k) if k is None else k,
                           f64(c.v) if v is None else v, c.seq_offsets, **kw)


def dense_library(c):
    """Per sequence and head: out_scale * (M * silu(alpha (Q K^T + R))) V with
    BLAS matmul and scipy's logistic function; the mask comes from the
    rule-based sets above."""
    q, k, v = f64(c.q), f64(c.k), f64(c.v)
    rab = None if c.rab is None else f64(c.rab)
    Hq, Hk = q.shape[1], k.shape[1]
    out = np.zeros_like(q)
    for b in range(c.batch):
        s0, s1 = c.seq_offsets[b], c.seq_offsets[b + 1]
        L = s1 - s0
        nc = 0 if c.num_context is None else c.num_context[b]
        nt = 0 if c.num_targets is None else c.num_targets[b]
        M = mask_from_rules(L, nc, nt, c.target_group_size, c.mask_type)
        if c.local_window:
            M &= window_band(L, c.local_window)
        for h in range(Hq):
            hk = h * Hk // Hq
            S = q[s0:s1, h, :] @ k[s0:s1, hk, :].T
            if rab is not None:
                S = S + np.where(M, rab[b, h, :L, :L], 0.0)
            X = c.alpha * S
            P = np.where(M, X * expit(X), 0.0)
            out[s0:s1, h, :] = c.out_scale * (P @ v[s0:s1, hk, :])
    return out


@pytest.mark.parametrize("kind", ["none", "causal", "ctx_tgt_g1", "ctx_tgt_g3_rab", "gqa", "empty_seq"])
def test_oracle_matches_dense_library(kind):
    if kind == "none":
        c = small_case(1, [5, 17, 9], mask=NONE)
    elif kind == "causal":
        c = small_case(2, [13, 1, 20])
    elif kind == "ctx_tgt_g1":
        c = small_case(3, [19, 24, 7], nc=(0, 5), nt=(0, 6), g=1)
    elif kind == "ctx_tgt_g3_rab":
        c = small_case(4, [19, 24, 7], nc=(0, 5), nt=(0, 9), g=3, rab=True, S=30)
    elif kind == "gqa":
        c = small_case(5, [11, 16], Hq=6, Hk=2, nt=(0, 4), g=1, rab=True)
    else:
        c = small_case(6, [9, 0, 12, 0], nc=2, nt=3, g=2)
    got = run_oracle(c)
    ref = dense_library(c)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_worked_example_by_hand():
    with open(os.path.join(GOLDEN, "hand_worked_3x2.json")) as f:
        g = json.load(f)
    for mask, key in [(CAUSAL, "expected_causal"), (NONE, "expected_bidirectional")]:
        out = oracle.hstu_fwd(g["q"], g["k"], g["v"], g["seq_offsets"], max_seq_len=3, mask_type=mask,
                              alpha=g["alpha"], out_scale=g["out_scale"])
        np.testing.assert_allclose(out, np.array(g[key]), rtol=1e-15, atol=1e-15)


def test_page_running_case_shape():
    with open(os.path.join(GOLDEN, "page_running_case.json")) as f:
        g = json.load(f)
    rng = np.random.default_rng(0)
    T, D = g["q_tokens"], g["head_dim"]
    q = rng.standard_normal((T, g["num_heads_q"], D))
    k = rng.standard_normal((T, g["num_heads_kv"], D))
    v = rng.standard_normal((T, g["num_heads_kv"], D))
    out = oracle.hstu_fwd(q, k, v, g["seq_offsets"], max_seq_len=g["max_seq_len"], mask_type=g["mask_type"],
                          out_scale=g["silu_scale"])
    assert list(out.shape) == g["output_shape"]
    assert np.all(out[g["seq_offsets"][-1]:] == 0.0)


# closed forms through the data path -----------------------------------------
def test_zero_query_no_rab_gives_zero():
    c = small_case(7, [12, 5], nc=2, nt=3, g=1)
    out = run_oracle(c, q=np.zeros(c.q.shape))
    assert np.all(out == 0.0)


def test_constant_rab_unit_values_counts_visible_keys():
    rng = np.random.default_rng(8)
    for (L, nc, nt, g) in [(23, 4, 6, 1), (17, 0, 5, 3), (9, 9, 0, 0), (30, 2, 30, 4)]:
        S, D, cst, alpha, osc = L + 3, 4, 0.9, 0.6, 0.25
        c = wl.jagged_case(int(rng.integers(1 << 30)), [L], 1, 1, D, "f32", mask_type=CAUSAL,
                           num_context=nc, num_targets=nt, target_group_size=g, max_seq_len=S)
        rab = np.full((1, 1, S, S), cst)
        out = oracle.hstu_fwd(np.zeros((L, 1, D)), f64(c.k), np.ones((L, 1, D)), [0, L], rab=rab,
                              num_context=[nc], num_targets=[nt], max_seq_len=S, mask_type=CAUSAL,
                              target_group_size=g, alpha=alpha, out_scale=osc)
        x = alpha * cst
        expect = osc * x * expit(x) * closed_form_counts(L, nc, nt, g)
        np.testing.assert_allclose(out[:, 0, :], np.repeat(expect[:, None], D, 1), rtol=1e-14)


def test_one_hot_values_read_out_the_mask():
    L, nc, nt, g = 12, 3, 5, 2
    D, cst, alpha, osc = 16, -1.3, 1.1, 0.5
    V = np.zeros((L, 1, D))
    V[np.arange(L), 0, np.arange(L)] = 1.0
    out = oracle.hstu_fwd(np.zeros((L, 1, D)), np.ones((L, 1, D)), V, [0, L], rab=np.full((1, 1, L, L), cst),
                          num_context=[nc], num_targets=[nt], max_seq_len=L, mask_type=CAUSAL,
                          target_group_size=g, alpha=alpha, out_scale=osc)
    x = alpha * cst
    M = mask_from_rules(L, nc, nt, g, CAUSAL)
    np.testing.assert_allclose(out[:, 0, :L], osc * x * expit(x) * M, rtol=1e-14, atol=0)
    assert np.all(out[:, 0, L:] == 0.0)


def test_query_key_orientation():
    # Only query row i0 is non-zero and every key lies on axis 0: S[i0, j] = x*y_j, S = 0 elsewhere.
    L, D, i0, x = 10, 12, 4, 1.7
    y = np.linspace(-2.0, 2.5, L)
    Q = np.zeros((L, 1, D))
    Q[i0, 0, 0] = x
    K = np.zeros((L, 1, D))
    K[:, 0, 0] = y
    V = np.zeros((L, 1, D))
    V[np.arange(L), 0, np.arange(L)] = 1.0
    out = oracle.hstu_fwd(Q, K, V, [0, L], max_seq_len=L, mask_type=NONE, alpha=0.8, out_scale=2.0)
    s = 0.8 * x * y
    expect = np.zeros((L, D))
    expect[i0, :L] = 2.0 * s * expit(s)
    np.testing.assert_allclose(out[:, 0, :], expect, rtol=1e-14, atol=1e-300)


def test_rab_orientation_batch_head_and_stride():
    lengths, Hq, S, D = [5, 7], 2, 9, 8  # S > every length: row stride is max_seq_len
    rng = np.random.default_rng(9)
    rab = rng.standard_normal((2, Hq, S, S))
    off = [0, 5, 12]
    T = 12
    V = np.zeros((T, 1, D))
    for b in range(2):
        for j in range(lengths[b]):
            V[off[b] + j, 0, j] = 1.0
    out = oracle.hstu_fwd(np.zeros((T, Hq, D)), np.zeros((T, 1, D)), V, off, rab=rab, max_seq_len=S,
                          mask_type=CAUSAL, alpha=0.9, out_scale=1.5)
    for b in range(2):
        L = lengths[b]
        M = mask_from_rules(L, 0, 0, 0, CAUSAL)
        for h in range(Hq):
            x = 0.9 * rab[b, h, :L, :L]
            np.testing.assert_allclose(out[off[b]:off[b] + L, h, :L], 1.5 * np.where(M, x * expit(x), 0.0),
                                       rtol=1e-14, atol=1e-300)


def test_gqa_head_mapping_closed_form():
    L, Hq, Hk, D = 9, 6, 3, 4
    c_h = np.linspace(-1.0, 1.5, Hq)
    rab = np.broadcast_to(c_h[None, :, None, None], (1, Hq, L, L)).copy()
    V = np.broadcast_to((np.arange(Hk) + 1.0)[None, :, None], (L, Hk, D)).copy()
    out = oracle.hstu_fwd(np.zeros((L, Hq, D)), np.zeros((L, Hk, D)), V, [0, L], rab=rab, num_targets=[3],
                          max_seq_len=L, mask_type=CAUSAL, target_group_size=1, alpha=1.0, out_scale=1.0)
    counts = closed_form_counts(L, 0, 3, 1)
    for h in range(Hq):
        expect = c_h[h] * expit(c_h[h]) * counts * (h * Hk // Hq + 1)
        np.testing.assert_allclose(out[:, h, 0], expect, rtol=1e-14)


# invariants ------------------------------------------------------------------
def test_gqa_equals_repeated_mha():
    c = small_case(10, [14, 9], Hq=4, Hk=2, nt=(1, 4), g=1, rab=True)
    got = run_oracle(c)
    krep = np.repeat(f64(c.k), 2, axis=1)
    vrep = np.repeat(f64(c.v), 2, axis=1)
    ref = oracle.hstu_fwd(f64(c.q), krep, vrep, c.seq_offsets, rab=f64(c.rab), num_targets=c.num_targets,
                          max_seq_len=c.max_seq_len, mask_type=CAUSAL, target_group_size=1, alpha=c.alpha,
                          out_scale=c.out_scale)
    np.testing.assert_array_equal(got, ref)


def test_batch_split_and_permutation_invariance():
    c = small_case(11, [7, 13, 4], nc=(0, 3), nt=(0, 4), g=2, rab=True, S=16)
    full = run_oracle(c)
    q, k, v, rab = f64(c.q), f64(c.k), f64(c.v), f64(c.rab)
    for b in range(3):
        s0, s1 = c.seq_offsets[b], c.seq_offsets[b + 1]
        one = oracle.hstu_fwd(q[s0:s1], k[s0:s1], v[s0:s1], [0, s1 - s0], rab=rab[b:b + 1],
                              num_context=c.num_context[b:b + 1], num_targets=c.num_targets[b:b + 1], max_seq_len=16,
                              mask_type=CAUSAL, target_group_size=2, alpha=c.alpha, out_scale=c.out_scale)
        np.testing.assert_array_equal(one, full[s0:s1])
    perm = [2, 0, 1]
    segs = [slice(c.seq_offsets[b], c.seq_offsets[b + 1]) for b in perm]
    lens = [c.lengths[b] for b in perm]
    off = np.concatenate([[0], np.cumsum(lens)])
    outp = oracle.hstu_fwd(np.concatenate([q[s] for s in segs]), np.concatenate([k[s] for s in segs]),
                           np.concatenate([v[s] for s in segs]), off, rab=rab[perm],
                           num_context=c.num_context[perm], num_targets=c.num_targets[perm], max_seq_len=16,
                           mask_type=CAUSAL, target_group_size=2, alpha=c.alpha, out_scale=c.out_scale)
    np.testing.assert_array_equal(outp, np.concatenate([full[s] for s in segs]))


def test_nan_in_masked_rab_is_never_read():
    c = small_case(12, [11, 6], nc=(1, 3), nt=(1, 4), g=1, rab=True, S=14)
    clean = f64(c.rab).copy()
    lengths = c.lengths
    for b in range(2):
        clean[b, :, lengths[b]:, :] = 0.0
        clean[b, :, :, lengths[b]:] = 0.0
    ref = run_oracle(c, rab=clean)
    poisoned = clean.copy()
    for b in range(2):
        L = lengths[b]
        M = mask_from_rules(L, c.num_context[b], c.num_targets[b], 1, CAUSAL)
        blk = poisoned[b, :, :L, :L]
        blk[:, ~M] = np.nan
        poisoned[b, :, L:, :] = np.nan
        poisoned[b, :, :, L:] = np.nan
    got = run_oracle(c, rab=poisoned)
    assert np.all(np.isfinite(got))
    np.testing.assert_array_equal(got, ref)


def test_other_target_groups_do_not_affect_a_target():
    for g in (1, 3):
        c = small_case(13, [20], nt=9, g=g)
        base = run_oracle(c)
        H = 20 - 9
        k, v = f64(c.k).copy(), f64(c.v).copy()
        # perturb the last target; rows of other groups must not move
        k[19] += 3.0
        v[19] -= 2.0
        pert = run_oracle(c, k=k, v=v)
        for i in range(H, 20):
            if (i - H) // g != (19 - H) // g:
                np.testing.assert_array_equal(pert[i], base[i])
        assert not np.array_equal(pert[19], base[19])


def test_sampled_rows_equal_full_rows():
    c = small_case(14, [10, 21, 3], Hq=4, Hk=2, nc=(0, 3), nt=(0, 5), g=1, rab=True)
    full = run_oracle(c)
    rows = [(0, 1), (30, 3), (12, 0), (33, 2), (9, 3)]
    got = run_oracle(c, rows=rows)
    for r, (t, h) in enumerate(rows):
        np.testing.assert_array_equal(got[r], full[t, h])


# paged -----------------------------------------------------------------------
def gather_paged(pc):
    """Contiguous K/V per request, gathered with numpy fancy indexing."""
    kv = f64(pc.kv_cache)
    ps = pc.page_size
    ks, vs, lens = [], [], []
    kn, vn = f64(pc.k_new), f64(pc.v_new)
    for b in range(pc.batch):
        Lh = int(pc.history_lengths[b])
        pages = pc.page_ids[pc.page_offsets[b]:pc.page_offsets[b + 1]]
        pos = np.arange(Lh)
        hk = kv[pages[pos // ps], 0, pos % ps]
        hv = kv[pages[pos // ps], 1, pos % ps]
        q0, q1 = pc.seq_offsets_q[b], pc.seq_offsets_q[b + 1]
        ks.append(np.concatenate([hk, kn[q0:q1]]))
        vs.append(np.concatenate([hv, vn[q0:q1]]))
        lens.append(Lh + q1 - q0)
    return np.concatenate(ks), np.concatenate(vs), np.concatenate([[0], np.cumsum(lens)])


def test_paged_equals_gathered_jagged():
    pc = wl.paged_case(21, [70, 0, 129, 64], [3, 5, 1, 4], 4, 2, 16, "f32", page_size=32, num_context=(0, 6),
                       target_group_size=2, extra_pages=3)
    out = oracle.hstu_fwd_paged(f64(pc.q), f64(pc.k_new), f64(pc.v_new), f64(pc.kv_cache), pc.seq_offsets_q,
                                pc.page_offsets, pc.page_ids, pc.last_page_len, num_context=pc.num_context,
                                num_targets=pc.num_targets, mask_type=CAUSAL, target_group_size=2, alpha=pc.alpha,
                                out_scale=pc.out_scale)
    assert np.all(np.isfinite(out))
    K, V, off = gather_paged(pc)
    Q = np.zeros((K.shape[0], 4, 16))
    for b in range(pc.batch):
        Lh = pc.history_lengths[b]
        q0, q1 = pc.seq_offsets_q[b], pc.seq_offsets_q[b + 1]
        Q[off[b] + Lh: off[b + 1]] = f64(pc.q)[q0:q1]
    ref = oracle.hstu_fwd(Q, K, V, off, num_context=pc.num_context, num_targets=pc.num_targets,
                          max_seq_len=int(np.diff(off).max()), mask_type=CAUSAL, target_group_size=2,
                          alpha=pc.alpha, out_scale=pc.out_scale)
    for b in range(pc.batch):
        Lh = pc.history_lengths[b]
        q0, q1 = pc.seq_offsets_q[b], pc.seq_offsets_q[b + 1]
        np.testing.assert_array_equal(out[q0:q1], ref[off[b] + Lh: off[b + 1]])


def test_paged_constant_scores_count_keys():
    hist, newl = [100, 33, 64], [4, 7, 2]
    pc = wl.paged_case(22, hist, newl, 2, 2, 8, "f32", page_size=32, num_context=(0, 5), target_group_size=3)
    a, bq = 0.8, -1.1
    q = np.zeros(pc.q.shape)
    q[:, :, 0] = a
    kn = np.zeros(pc.k_new.shape)
    kn[:, :, 0] = bq
    kv = np.zeros(pc.kv_cache.shape)
    kv[:, 0, :, :, 0] = bq
    kv[:, 1] = 1.0
    out = oracle.hstu_fwd_paged(q, kn, np.ones(pc.v_new.shape), kv, pc.seq_offsets_q, pc.page_offsets,
                                pc.page_ids, pc.last_page_len, num_context=pc.num_context, num_targets=pc.num_targets,
                                mask_type=CAUSAL, target_group_size=3, alpha=0.5, out_scale=0.1)
    x = 0.5 * a * bq
    for b in range(3):
        L = hist[b] + newl[b]
        counts = closed_form_counts(L, pc.num_context[b], pc.num_targets[b], 3)[hist[b]:]
        q0 = pc.seq_offsets_q[b]
        np.testing.assert_allclose(out[q0:q0 + newl[b], :, 0], 0.1 * x * expit(x) * counts[:, None] * np.ones((1, 2)),
                                   rtol=1e-14)


def test_paged_independent_of_page_permutation():
    pc = wl.paged_case(23, [90, 40], [3, 2], 2, 2, 8, "f32", page_size=32, target_group_size=1)
    kv = f64(pc.kv_cache)
    base = oracle.hstu_fwd_paged(f64(pc.q), f64(pc.k_new), f64(pc.v_new), kv, pc.seq_offsets_q, pc.page_offsets,
                                 pc.page_ids, pc.last_page_len, num_targets=pc.num_targets, target_group_size=1,
                                 alpha=pc.alpha, out_scale=pc.out_scale)
    perm = np.random.default_rng(1).permutation(kv.shape[0])
    inv = np.argsort(perm)
    kv2 = kv[perm]  # page p now lives at index inv[p]
    out = oracle.hstu_fwd_paged(f64(pc.q), f64(pc.k_new), f64(pc.v_new), kv2, pc.seq_offsets_q, pc.page_offsets,
                                inv[pc.page_ids], pc.last_page_len, num_targets=pc.num_targets, target_group_size=1,
                                alpha=pc.alpha, out_scale=pc.out_scale)
    np.testing.assert_array_equal(out, base)


# metrics closed form vs the oracle's mask ---------------------------------------
def test_metrics_counts_match_oracle_mask():
    from hstu_jagged_attention_amd import metrics
    rng = np.random.default_rng(15)
    for _ in range(100):
        L = int(rng.integers(0, 50))
        nc, nt, g = int(rng.integers(0, L + 2)), int(rng.integers(0, L + 2)), int(rng.choice([0, 1, 3]))
        for mt in (CAUSAL, NONE):
            M = oracle.mask_matrix(mt, L, nc, nt, g)
            np.testing.assert_array_equal(metrics.visible_per_row(L, nc, nt, g, mt), M.sum(1))


# ------------------------------------------ user mask, rab broadcast, delta-QK
CUSTOM = oracle.MASK_CUSTOM


def dense_general(c):
    """Per sequence and head, with BLAS matmul and scipy's logistic function:
    the queries are the last Lq of the Lk positions (rows Lk-Lq.. of the
    full score matrix); rab / mask heads broadcast when they have one head;
    the user mask M multiplies P where it is non-zero and removes the key
    where it is zero; the built-in mask comes from the rule-based sets."""
    q, k, v = f64(c.q), f64(c.k), f64(c.v)
    rab = None if c.rab is None else f64(c.rab)
    um = None if c.mask is None else f64(c.mask)
    koff = c.seq_offsets if c.seq_offsets_k is None else c.seq_offsets_k
    Hq, Hk = q.shape[1], k.shape[1]
    out = np.zeros_like(q)
    for b in range(c.batch):
        q0, q1, k0, k1 = c.seq_offsets[b], c.seq_offsets[b + 1], koff[b], koff[b + 1]
        Lq, L = q1 - q0, k1 - k0
        rows = np.arange(L - Lq, L)
        nc = 0 if c.num_context is None else c.num_context[b]
        nt = 0 if c.num_targets is None else c.num_targets[b]
        M = mask_from_rules(L, nc, nt, c.target_group_size, NONE if c.mask_type == CUSTOM else c.mask_type)[rows]
        for h in range(Hq):
            hk = h * Hk // Hq
            S = q[q0:q1, h, :] @ k[k0:k1, hk, :].T
            keep = M.copy()
            scale = np.ones_like(S)
            if um is not None:
                mm = um[b, 0 if um.shape[1] == 1 else h][np.ix_(rows, np.arange(L))]
                keep &= mm != 0
                scale = np.where(keep, mm, 0.0)
            if rab is not None:
                rr = rab[b, 0 if rab.shape[1] == 1 else h][np.ix_(rows, np.arange(L))]
                S = S + np.where(keep, rr, 0.0)
            X = c.alpha * S
            P = np.where(keep, X * expit(X) * scale, 0.0)
            out[q0:q1, h, :] = c.out_scale * (P @ v[k0:k1, hk, :])
    return out


def custom_case(seed, lengths, keep=0.5, Hq=2, Hk=2, rab=True, rab_heads=None, mask_heads=None, S=None):
    return wl.jagged_case(seed, lengths, Hq, Hk, 8, "f32", mask_type=CUSTOM, rab_std=0.5 if rab else None,
                          rab_heads=rab_heads, mask_keep=keep, mask_heads=mask_heads, max_seq_len=S, alpha=0.7,
                          out_scale=0.3)


@pytest.mark.parametrize("kind", ["mask", "mask_gqa_bcast", "mask_values", "delta_causal", "delta_ctx_tgt_rab",
                                  "delta_none_gqa", "delta_mask"])
def test_general_oracle_matches_dense_library(kind):
    """The user mask, rab broadcast and delta-QK paths of the oracle against
    the dense BLAS formulation (the inputs/outputs table: mask
    [B, N, S, S] with mask_type 3, rab broadcast [b, 1, s, s], seq_offsets_k
    with is_delta_qk)."""
    if kind == "mask":
        c = custom_case(11, [13, 1, 20, 0], S=24)
    elif kind == "mask_gqa_bcast":
        c = custom_case(12, [9, 16], Hq=4, Hk=2, rab_heads=1, mask_heads=1)
    elif kind == "mask_values":
        c = custom_case(13, [7, 12], keep=0.6)
        rng = np.random.default_rng(0)  # scale the kept entries by values other than 1, some negative
        c.mask = c.mask * torch.from_numpy(rng.choice([0.5, 2.0, -1.5], size=tuple(c.mask.shape)).astype(np.float32))
    elif kind == "delta_causal":
        c = wl.jagged_case(14, [17, 30, 5], 2, 2, 8, "f32", q_lengths=[4, 30, 1], alpha=0.7, out_scale=0.3)
    elif kind == "delta_ctx_tgt_rab":
        c = wl.jagged_case(15, [21, 26], 2, 2, 8, "f32", q_lengths=[9, 3], num_context=(0, 6), num_targets=(1, 8),
                           target_group_size=2, rab_std=0.5, max_seq_len=28, alpha=0.7, out_scale=0.3)
    elif kind == "delta_none_gqa":
        c = wl.jagged_case(16, [12, 19], 6, 2, 8, "f32", q_lengths=[12, 2], mask_type=NONE, alpha=0.7, out_scale=0.3)
    else:
        c = wl.jagged_case(17, [15, 22], 2, 2, 8, "f32", q_lengths=[6, 5], mask_type=CUSTOM, mask_keep=0.5,
                           rab_std=0.5, rab_heads=1, alpha=0.7, out_scale=0.3)
    np.testing.assert_allclose(run_oracle(c), dense_general(c), rtol=1e-12, atol=1e-13)


def test_user_mask_of_ones_is_no_mask():
    c = custom_case(21, [11, 17], keep=1.0, rab=False)
    got = run_oracle(c)
    ref = run_oracle(c, mask=None, mask_type=NONE)
    assert np.array_equal(got, ref)


def test_user_mask_of_rule_sets_is_the_builtin_mask():
    """A user mask holding the 0/1 matrix built from the English mask rules
    reproduces the built-in causal mask with context and target groups."""
    lengths, nc, nt, g = [19, 24, 7], [3, 0, 2], [5, 9, 0], 3
    c = wl.jagged_case(22, lengths, 2, 2, 8, "f32", mask_type=CAUSAL, num_context=nc, num_targets=nt,
                       target_group_size=g, alpha=0.7, out_scale=0.3)
    S = max(lengths)
    m = np.zeros((len(lengths), 1, S, S))
    for b, L in enumerate(lengths):
        m[b, 0, :L, :L] = mask_from_rules(L, nc[b], nt[b], g, CAUSAL)
    builtin = run_oracle(c)
    user = run_oracle(c, mask=m, mask_type=CUSTOM, num_context=None, num_targets=None, max_seq_len=S)
    assert np.array_equal(builtin, user)


def test_user_mask_scales_linearly():
    c = custom_case(23, [10, 14], keep=1.0)
    ones = run_oracle(c)
    twos = run_oracle(c, mask=2.0 * f64(c.mask))
    np.testing.assert_allclose(twos, 2.0 * ones, rtol=1e-14, atol=0)


def test_user_mask_zero_removes_nan_scores():
    """Zero mask entries contribute exactly zero even where rab is NaN."""
    c = custom_case(24, [12, 9], keep=0.5)
    clean = run_oracle(c)
    rab = f64(c.rab).copy()
    m = f64(c.mask)
    rab[np.nan_to_num(m, nan=1.0) == 0] = np.nan
    got = run_oracle(c, rab=rab)
    assert np.isfinite(got).all()
    assert np.array_equal(got, clean)


def test_zero_user_mask_gives_zero():
    c = custom_case(25, [8, 13], keep=0.0)
    assert not run_oracle(c).any()


def test_rab_broadcast_equals_repeated_rab():
    c = custom_case(26, [9, 14], Hq=3, Hk=1, rab_heads=1)
    rep = np.repeat(f64(c.rab), 3, axis=1)
    assert np.array_equal(run_oracle(c), run_oracle(c, rab=rep))


def test_delta_qk_equals_last_rows_of_full_sequence():
    """Queries right-aligned on the keys: the delta call equals the full
    call's rows for the last Lq positions (same keys, same mask inputs)."""
    lk, lq = [20, 33, 7], [5, 33, 1]
    full = wl.jagged_case(27, lk, 2, 2, 8, "f32", num_context=(0, 4), num_targets=(1, 6), target_group_size=1,
                          rab_std=0.5, max_seq_len=34, alpha=0.7, out_scale=0.3)
    qf = f64(full.q)
    rows = np.concatenate([np.arange(full.seq_offsets[b + 1] - lq[b], full.seq_offsets[b + 1]) for b in range(3)])
    offq = np.concatenate([[0], np.cumsum(lq)])
    ref = run_oracle(full)[rows]
    got = oracle.hstu_fwd(qf[rows], f64(full.k), f64(full.v), offq, seq_offsets_k=full.seq_offsets,
                          rab=f64(full.rab), num_context=full.num_context, num_targets=full.num_targets,
                          max_seq_len=34, mask_type=CAUSAL, target_group_size=1, alpha=0.7, out_scale=0.3)
    assert np.array_equal(got, ref)


def test_general_oracle_rejects_bad_arguments():
    c = custom_case(28, [5, 6])
    with pytest.raises(ValueError):  # mask_type 3 needs a mask
        run_oracle(c, mask=None)
    with pytest.raises(ValueError):  # a mask needs mask_type 3
        run_oracle(c, mask_type=NONE)
    d = wl.jagged_case(29, [4, 6], 2, 2, 8, "f32", alpha=0.7, out_scale=0.3)
    with pytest.raises(ValueError):  # more queries than keys
        oracle.hstu_fwd(f64(d.q), f64(d.k)[:8], f64(d.v)[:8], d.seq_offsets, seq_offsets_k=[0, 3, 8], max_seq_len=6)


# ---------------------------------------------------------------- FP8 cast
E4M3 = torch.float8_e4m3fn


def torch_e4m3(x):
    """torch's own E4M3 (FN) cast of float32 values: round to nearest, ties to
    even (NaN past the range, which the pins below stay inside)."""
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(E4M3).to(torch.float64).numpy()


def all_e4m3_values():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    vals = codes.view(E4M3).to(torch.float64).numpy()
    return vals[np.isfinite(vals)]


def test_e4m3_every_code_maps_to_itself():
    vals = all_e4m3_values()
    assert vals.size == 254 and vals.max() == 448.0 and vals.min() == -448.0
    for v in vals:
        assert oracle.e4m3(float(v)) == v


def test_e4m3_matches_library_cast():
    rng = np.random.default_rng(0)
    mag = np.exp(rng.uniform(np.log(1e-4), np.log(463.0), size=20000)).astype(np.float32)
    x = (mag * rng.choice([-1.0, 1.0], size=mag.size)).astype(np.float32)
    # exact midpoints between neighbouring codes (ties to even) and points just beside them
    vals = np.unique(all_e4m3_values())
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, np.nextafter(mids, np.float32(1e4)), np.nextafter(mids, np.float32(-1e4))])
    x = x[np.abs(x) < 464.0]
    got = np.array([oracle.e4m3(float(t)) for t in x])
    np.testing.assert_array_equal(got, torch_e4m3(x))


def test_e4m3_hand_values_and_saturation():
    # ties to even on the grid; subnormal step 2^-9; saturation beyond 448 (the stated reading)
    cases = {1.0625: 1.0, 1.1875: 1.25, 0.3: 0.3125, -2.7: -2.75, 2.0 ** -10: 0.0, 3 * 2.0 ** -10: 2.0 ** -8,
             0.001: 2.0 ** -9, 17.0: 16.0, 447.0: 448.0, 460.0: 448.0, 464.0: 448.0, 500.0: 448.0, 1e6: 448.0,
             -1e6: -448.0, 0.0: 0.0}
    for x, want in cases.items():
        assert oracle.e4m3(x) == want, (x, oracle.e4m3(x), want)
    assert math.isnan(oracle.e4m3(float("nan")))


def fp8_case(seed, lengths, Hq=2, Hk=2, mask=CAUSAL, nc=None, nt=None, g=0, rab=False, S=None):
    return wl.jagged_case(seed, lengths, Hq, Hk, 16, "fp8", mask_type=mask, num_context=nc, num_targets=nt,
                          target_group_size=g, rab_std=0.5 if rab else None, max_seq_len=S, alpha=0.35,
                          out_scale=0.3)


def dense_fp8(c):
    """Per sequence and head: out_scale * (M * E4M3(silu(alpha (Q K^T + R)))) V
    with BLAS matmul, scipy's logistic function and torch's E4M3 cast; the
    mask comes from the rule-based sets."""
    q, k, v = f64(c.q), f64(c.k), f64(c.v)
    rab = None if c.rab is None else f64(c.rab)
    Hq, Hk = q.shape[1], k.shape[1]
    out = np.zeros_like(q)
    for b in range(c.batch):
        s0, s1 = c.seq_offsets[b], c.seq_offsets[b + 1]
        L = s1 - s0
        nc = 0 if c.num_context is None else c.num_context[b]
        nt = 0 if c.num_targets is None else c.num_targets[b]
        M = mask_from_rules(L, nc, nt, c.target_group_size, c.mask_type)
        if c.local_window:
            M &= window_band(L, c.local_window)
        for h in range(Hq):
            hk = h * Hk // Hq
            S = q[s0:s1, h, :] @ k[s0:s1, hk, :].T
            if rab is not None:
                S = S + np.where(M, rab[b, h, :L, :L], 0.0)
            X = c.alpha * S
            P = np.where(M, torch_e4m3(X * expit(X)), 0.0)
            out[s0:s1, h, :] = c.out_scale * (P @ v[s0:s1, hk, :])
    return out


@pytest.mark.parametrize("kind", ["causal", "none", "ctx_tgt_g3", "gqa_rab"])
def test_fp8_oracle_matches_dense_library(kind):
    """The FP8 cast reading: E4M3 inputs, P cast to E4M3 before the product
    with V, against the dense formulation with the library cast."""
    if kind == "causal":
        c = fp8_case(21, [13, 1, 20])
    elif kind == "none":
        c = fp8_case(22, [5, 17, 9], mask=NONE)
    elif kind == "ctx_tgt_g3":
        c = fp8_case(23, [19, 24, 7], nc=(0, 5), nt=(0, 9), g=3)
    else:
        c = fp8_case(24, [11, 16], Hq=6, Hk=2, nt=(0, 4), g=1, rab=True)
    for t in (c.q, c.k, c.v):
        assert t.dtype == E4M3
    got = run_oracle(c, p_fp8=True)
    np.testing.assert_allclose(got, dense_fp8(c), rtol=1e-12, atol=1e-13)
    # the cast is real: without it the result moves by the E4M3 step of P
    plain = run_oracle(c)
    rel = np.linalg.norm(got - plain) / np.linalg.norm(plain)
    assert 1e-3 < rel < 0.2, rel


def test_fp8_constant_rab_unit_values_closed_form():
    """Q = 0, rab = c, V = 1: every visible term is E4M3(silu(alpha c)), so
    O[i, :] = out_scale * E4M3(silu(alpha c)) * (visible keys of row i)."""
    L, D, alpha, out_scale, cst = 23, 16, 0.35, 0.3, 1.7
    nc, nt, g = 3, 6, 2
    rab = np.full((1, 1, L, L), cst)
    out = oracle.hstu_fwd(np.zeros((L, 1, D)), np.zeros((L, 1, D)), np.ones((L, 1, D)), [0, L], rab=rab,
                          num_context=[nc], num_targets=[nt], max_seq_len=L, target_group_size=g, alpha=alpha,
                          out_scale=out_scale, p_fp8=True)
    p8 = float(torch_e4m3([alpha * cst * expit(alpha * cst)])[0])
    assert p8 != alpha * cst * expit(alpha * cst)
    counts = closed_form_counts(L, nc, nt, g)
    np.testing.assert_allclose(out[:, 0, :], out_scale * p8 * np.repeat(np.asarray(counts, float)[:, None], D, 1),
                               rtol=1e-14)


# ---------------------------------------------------------------- local mask
def window_band(L, w):
    """Pairs with i - j < w, from numpy's triangle routine (np.tri(L, L, -w)
    marks exactly the pairs with j <= i - w)."""
    return ~np.tri(L, L, -w, dtype=bool)


def test_local_mask_bruteforce_random():
    rng = np.random.default_rng(41)
    for _ in range(400):
        L = int(rng.integers(1, 40))
        nc = int(rng.integers(-2, L + 4))
        nt = int(rng.integers(-2, L + 4))
        g = int(rng.choice([0, 1, 2, 3, 5]))
        w = int(rng.integers(1, L + 3))
        got = oracle.mask_matrix(CAUSAL, L, nc, nt, g, w)
        ref = mask_from_rules(L, nc, nt, g, CAUSAL) & window_band(L, w)
        np.testing.assert_array_equal(got, ref, err_msg=str((L, nc, nt, g, w)))


def test_local_mask_hand_fixture():
    # L = 7, two context rows, two targets in groups of one, window 3: the
    # context rows see both context keys (the window bounds i - j only from
    # above), history row 4 sees keys 2..4, target 6 sees history 4 and itself.
    M = oracle.mask_matrix(CAUSAL, 7, 2, 2, 1, 3).astype(int)
    expect = np.array([[1, 1, 0, 0, 0, 0, 0],
                       [1, 1, 0, 0, 0, 0, 0],
                       [1, 1, 1, 0, 0, 0, 0],
                       [0, 1, 1, 1, 0, 0, 0],
                       [0, 0, 1, 1, 1, 0, 0],
                       [0, 0, 0, 1, 1, 1, 0],
                       [0, 0, 0, 0, 1, 0, 1]])
    np.testing.assert_array_equal(M, expect)


def closed_form_counts_window(L, nc, nt, g, w):
    """Row counts with the window, from interval lengths: each row's set is
    one or two intervals of keys, cut below at lo = max(0, i - w + 1)."""
    nt = min(max(nt, 0), L)
    H = L - nt
    nc = min(max(nc, 0), H)
    out = []
    for i in range(L):
        lo = max(0, i - w + 1)
        if i < nc:
            out.append(nc - lo)
        elif i < H or g == 0:
            out.append(min(i + 1, w))
        else:
            start = H + (i - H) // g * g
            out.append(max(0, H - lo) + i + 1 - max(start, lo))
    return np.array(out)


def test_local_mask_row_counts_closed_form():
    rng = np.random.default_rng(42)
    for _ in range(300):
        L = int(rng.integers(1, 60))
        nc, nt = int(rng.integers(0, L + 2)), int(rng.integers(0, L + 2))
        g = int(rng.choice([0, 1, 3, 4]))
        w = int(rng.integers(1, 70))
        M = oracle.mask_matrix(CAUSAL, L, nc, nt, g, w)
        np.testing.assert_array_equal(M.sum(1), closed_form_counts_window(L, nc, nt, g, w), err_msg=str((L, nc, nt, g, w)))


def test_local_window_covering_the_sequence_is_no_window():
    for (L, nc, nt, g) in [(17, 3, 5, 2), (30, 0, 0, 0), (9, 9, 0, 0)]:
        for w in (L, L + 1, 4 * L):
            np.testing.assert_array_equal(oracle.mask_matrix(CAUSAL, L, nc, nt, g, w),
                                          oracle.mask_matrix(CAUSAL, L, nc, nt, g))


def test_local_window_one_reads_only_the_diagonal():
    # With no context, a window of one leaves each query its own key:
    # O_i = out_scale * silu(alpha (q_i . k_i + rab_ii)) v_i, by hand.
    c = small_case(43, [13, 1, 20], Hq=4, Hk=2, nt=(0, 7), g=1, rab=True)
    got = run_oracle(c, local_window=1)
    q, k, v, rab = f64(c.q), f64(c.k), f64(c.v), f64(c.rab)
    ref = np.zeros_like(q)
    for b in range(c.batch):
        s0, s1 = c.seq_offsets[b], c.seq_offsets[b + 1]
        for i in range(s1 - s0):
            for h in range(4):
                x = c.alpha * (q[s0 + i, h] @ k[s0 + i, h // 2] + rab[b, h, i, i])
                ref[s0 + i, h] = c.out_scale * x * expit(x) * v[s0 + i, h // 2]
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("kind", ["w5", "w1_ctx", "w9_ctx_tgt_g3_rab", "w16_gqa_delta"])
def test_local_oracle_matches_dense_library(kind):
    if kind == "w5":
        c = small_case(44, [13, 1, 20, 0], local_window=5)
    elif kind == "w1_ctx":
        c = small_case(45, [19, 24, 7], nc=(0, 5), local_window=1)
    elif kind == "w9_ctx_tgt_g3_rab":
        c = small_case(46, [19, 24, 7], nc=(0, 5), nt=(0, 9), g=3, rab=True, S=30, local_window=9)
    else:
        full = small_case(47, [40, 33], Hq=6, Hk=2, nt=(0, 5), g=1, rab=True, local_window=16)
        ref = dense_library(full)
        lq = np.array([7, 12])
        rows = np.concatenate([np.arange(full.seq_offsets[b + 1] - lq[b], full.seq_offsets[b + 1]) for b in range(2)])
        offq = np.concatenate([[0], np.cumsum(lq)])
        got = oracle.hstu_fwd(f64(full.q)[rows], f64(full.k), f64(full.v), offq, seq_offsets_k=full.seq_offsets,
                              rab=f64(full.rab), num_targets=full.num_targets, max_seq_len=full.max_seq_len,
                              mask_type=CAUSAL, target_group_size=1, alpha=full.alpha, out_scale=full.out_scale,
                              local_window=16)
        np.testing.assert_allclose(got, ref[rows], rtol=1e-12, atol=1e-13)
        return
    np.testing.assert_allclose(run_oracle(c), dense_library(c), rtol=1e-12, atol=1e-13)


def test_local_window_paged_equals_gathered_jagged():
    pc = wl.paged_case(48, [70, 0, 129, 64], [3, 5, 1, 4], 4, 2, 16, "f32", page_size=32, num_context=(0, 6),
                       target_group_size=2, extra_pages=3, local_window=40)
    out = oracle.hstu_fwd_paged(f64(pc.q), f64(pc.k_new), f64(pc.v_new), f64(pc.kv_cache), pc.seq_offsets_q,
                                pc.page_offsets, pc.page_ids, pc.last_page_len, num_context=pc.num_context,
                                num_targets=pc.num_targets, mask_type=CAUSAL, target_group_size=2, alpha=pc.alpha,
                                out_scale=pc.out_scale, local_window=40)
    assert np.all(np.isfinite(out))
    K, V, off = gather_paged(pc)
    Q = np.zeros((K.shape[0], 4, 16))
    for b in range(pc.batch):
        q0, q1 = pc.seq_offsets_q[b], pc.seq_offsets_q[b + 1]
        Q[off[b] + pc.history_lengths[b]: off[b + 1]] = f64(pc.q)[q0:q1]
    ref = oracle.hstu_fwd(Q, K, V, off, num_context=pc.num_context, num_targets=pc.num_targets,
                          max_seq_len=int(np.diff(off).max()), mask_type=CAUSAL, target_group_size=2,
                          alpha=pc.alpha, out_scale=pc.out_scale, local_window=40)
    for b in range(pc.batch):
        q0, q1 = pc.seq_offsets_q[b], pc.seq_offsets_q[b + 1]
        np.testing.assert_array_equal(out[q0:q1], ref[off[b] + pc.history_lengths[b]: off[b + 1]])


def test_local_window_metrics_counts_match_oracle_mask():
    from hstu_jagged_attention_amd import metrics
    rng = np.random.default_rng(49)
    for _ in range(150):
        L = int(rng.integers(0, 50))
        nc, nt, g = int(rng.integers(0, L + 2)), int(rng.integers(0, L + 2)), int(rng.choice([0, 1, 3]))
        w = int(rng.integers(1, 60))
        M = oracle.mask_matrix(CAUSAL, L, nc, nt, g, w)
        np.testing.assert_array_equal(metrics.visible_per_row(L, nc, nt, g, CAUSAL, w), M.sum(1))


def test_local_window_rejected_outside_the_causal_mask():
    c = small_case(50, [5, 6], mask=NONE)
    with pytest.raises(ValueError):
        run_oracle(c, local_window=3)
    d = small_case(51, [5, 6])
    with pytest.raises(ValueError):
        run_oracle(d, local_window=-1)
