"""Shared helpers of the GPU parity tests: run a case through the C ABI (via
the binding) and through the float64 oracle, and compare."""
from __future__ import annotations

import numpy as np
import torch
from scipy.special import expit

import hstu_jagged_attention_amd as hj
import oracle

# Tolerances: max-abs bars as stated for the workloads (1e-4 fp32, 2e-2
# bf16/fp16 on unit-normal inputs), plus relative checks so that an
# all-zero output cannot pass (out_scale = 1/max_seq_len makes |O| ~ 1e-2).
TOL = {
    "f32": dict(max_abs=1e-4, rel_l2=1e-5, rel_max=1e-3),
    "f16": dict(max_abs=2e-2, rel_l2=1e-2, rel_max=2e-2),
    "bf16": dict(max_abs=2e-2, rel_l2=1e-2, rel_max=2e-2),
    # The FP8 cast writes bf16 and the oracle models its E4M3 cast of P, so
    # the bf16 bars apply (the cast itself moves O by about 2 % rel-L2, see
    # the FP8 parity test).
    "fp8": dict(max_abs=2e-2, rel_l2=1e-2, rel_max=2e-2),
}


def f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def gpu_device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    hj.load_library()
    return torch.device("cuda:0")


def run_jagged(c, dev, out=None, workspace=None, **over) -> torch.Tensor:
    kw = dict(rab=None if c.rab is None else c.rab.to(dev), mask=None if c.mask is None else c.mask.to(dev),
              seq_offsets_k=None if c.seq_offsets_k is None else torch.as_tensor(c.seq_offsets_k),
              num_context=c.num_context, num_targets=c.num_targets, max_seq_len=c.max_seq_len, mask_type=c.mask_type,
              target_group_size=c.target_group_size, alpha=c.alpha, out_scale=c.out_scale, out=out,
              workspace=workspace)
    if c.local_window:
        kw["local_window"] = c.local_window
    kw.update(over)
    return hj.hstu_fwd(c.q.to(dev), c.k.to(dev), c.v.to(dev), torch.as_tensor(c.seq_offsets), **kw)


def run_paged(pc, dev, **over) -> torch.Tensor:
    kw = dict(num_context=pc.num_context, num_targets=pc.num_targets, max_seq_len=pc.max_seq_len,
              mask_type=pc.mask_type, target_group_size=pc.target_group_size, alpha=pc.alpha,
              out_scale=pc.out_scale)
    if pc.local_window:
        kw["local_window"] = pc.local_window
    kw.update(over)
    return hj.hstu_fwd_paged(pc.q.to(dev), pc.k_new.to(dev), pc.v_new.to(dev), pc.kv_cache.to(dev),
                             torch.as_tensor(pc.seq_offsets_q), torch.as_tensor(pc.page_offsets),
                             torch.as_tensor(pc.page_ids), torch.as_tensor(pc.last_page_len), **kw)


def oracle_jagged(c, rows=None) -> np.ndarray:
    return oracle.hstu_fwd(f64(c.q), f64(c.k), f64(c.v), c.seq_offsets, rab=None if c.rab is None else f64(c.rab),
                           mask=None if c.mask is None else f64(c.mask), seq_offsets_k=c.seq_offsets_k,
                           num_context=c.num_context, num_targets=c.num_targets, max_seq_len=c.max_seq_len,
                           mask_type=c.mask_type, target_group_size=c.target_group_size, alpha=c.alpha,
                           out_scale=c.out_scale, rows=rows, p_fp8=c.dtype == "fp8",
                           local_window=c.local_window)


def oracle_jagged_sampled(c, picks):
    """picks: {b: [(local_row, head), ...]}. Each sequence is handed to the
    oracle on its own (the result of a sequence does not depend on the
    others), so the oracle never needs the whole batch in float64.
    Returns {b: (global token rows, heads, values [n, D])}."""
    res = {}
    koff = c.seq_offsets if c.seq_offsets_k is None else c.seq_offsets_k
    for b, rows in picks.items():
        s0, s1 = int(c.seq_offsets[b]), int(c.seq_offsets[b + 1])
        k0, k1 = int(koff[b]), int(koff[b + 1])
        rab = None if c.rab is None else f64(c.rab[b:b + 1])
        mask = None if c.mask is None else f64(c.mask[b:b + 1])
        vals = oracle.hstu_fwd(f64(c.q[s0:s1]), f64(c.k[k0:k1]), f64(c.v[k0:k1]), [0, s1 - s0], rab=rab, mask=mask,
                               seq_offsets_k=None if c.seq_offsets_k is None else [0, k1 - k0],
                               num_context=None if c.num_context is None else c.num_context[b:b + 1],
                               num_targets=None if c.num_targets is None else c.num_targets[b:b + 1],
                               max_seq_len=c.max_seq_len, mask_type=c.mask_type,
                               target_group_size=c.target_group_size, alpha=c.alpha, out_scale=c.out_scale,
                               rows=rows, p_fp8=c.dtype == "fp8", local_window=c.local_window)
        res[b] = (np.array([s0 + r for r, _ in rows]), np.array([h for _, h in rows]), vals)
    return res


def oracle_paged(pc, rows=None) -> np.ndarray:
    return oracle.hstu_fwd_paged(f64(pc.q), f64(pc.k_new), f64(pc.v_new), f64(pc.kv_cache), pc.seq_offsets_q,
                                 pc.page_offsets, pc.page_ids, pc.last_page_len, num_context=pc.num_context,
                                 num_targets=pc.num_targets, mask_type=pc.mask_type,
                                 target_group_size=pc.target_group_size, alpha=pc.alpha, out_scale=pc.out_scale,
                                 rows=rows, local_window=pc.local_window)


def fp8_cast_allowance(c, toks, heads, eps=2.0 ** -14):
    """Both roundings of an E4M3 cast of P are valid where P lies within a
    relative eps of a rounding midpoint: the kernel computes P in fp32 with
    the hardware exp2 / reciprocal (a few ulp), the oracle in float64, and
    the two can fall on either side. eps = 2^-14 is far above fp32's
    rounding (2^-24) and far below an E4M3 step (2^-4 relative at least).
    For the (token, head) pairs given, returns the largest change of O
    those casts can make: out_scale * sum over such keys of (the gap between
    the two candidate E4M3 values) * |V[j, :]|, shape [n, D]."""
    import oracle
    q, k, v = f64(c.q), f64(c.k), f64(c.v)
    koff = c.seq_offsets if c.seq_offsets_k is None else c.seq_offsets_k
    Hq, Hk = q.shape[1], k.shape[1]
    toks, heads = np.asarray(toks), np.asarray(heads)
    out = np.zeros((len(toks), q.shape[2]))
    cast = lambda x: torch.from_numpy(np.minimum(x, 448.0)).float().to(torch.float8_e4m3fn).double().numpy()
    b_of = np.searchsorted(c.seq_offsets, toks, side="right") - 1
    for b in np.unique(b_of):
        s0, s1, k0, k1 = int(c.seq_offsets[b]), int(c.seq_offsets[b + 1]), int(koff[b]), int(koff[b + 1])
        Lk = k1 - k0
        nc = 0 if c.num_context is None else int(c.num_context[b])
        nt = 0 if c.num_targets is None else int(c.num_targets[b])
        M = oracle.mask_matrix(c.mask_type, Lk, nc, nt, c.target_group_size, c.local_window)
        for h in np.unique(heads[b_of == b]):
            sel = np.nonzero((b_of == b) & (heads == h))[0]
            hk = int(h) * Hk // Hq
            pos = (Lk - (s1 - s0)) + toks[sel] - s0  # key positions of the queries
            a = c.alpha * (q[toks[sel], h, :] @ k[k0:k1, hk, :].T)
            p = a * expit(a)
            gap = np.where(M[pos], np.abs(cast(p * (1 + eps)) - cast(p * (1 - eps))), 0.0)
            out[sel] = c.out_scale * (gap @ np.abs(v[k0:k1, hk, :]))
    return out


def assert_parity_fp8(got, ref, c, toks=None, heads=None, what: str = ""):
    """The FP8 cast's comparison: the bars of the other 16-bit dtypes on the
    raw difference (max-abs, relative L2), and the relative max-abs bar on
    what remains after the cast-midpoint allowance of each element (see
    fp8_cast_allowance). toks / heads: the (token, head) of each row of
    got / ref ([n, D]); default, every row of a [T, H, D] output."""
    g, r = f64(got), np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    if toks is None:
        T, H = g.shape[0], g.shape[1]
        toks, heads = np.repeat(np.arange(T), H), np.tile(np.arange(H), T)
        g, r = g.reshape(T * H, -1), r.reshape(T * H, -1)
    max_abs, rel_l2, ref_max = errors(g, r)
    t = TOL["fp8"]
    allow = fp8_cast_allowance(c, np.asarray(toks), np.asarray(heads))
    excess = float(np.max(np.abs(g - r) - allow, initial=0.0))
    msg = (f"{what}: max_abs={max_abs:.3e} rel_l2={rel_l2:.3e} max|ref|={ref_max:.3e} "
           f"beyond cast allowance={excess:.3e} (rows with an ambiguous cast: {int((allow > 0).any(1).sum())})")
    assert max_abs <= t["max_abs"], msg
    assert rel_l2 <= t["rel_l2"], msg
    assert excess <= t["rel_max"] * max(ref_max, 1e-30), msg
    return max_abs, rel_l2


def errors(got, ref):
    g, r = f64(got), np.asarray(ref, dtype=np.float64)
    d = np.abs(g - r)
    max_abs = float(d.max()) if d.size else 0.0
    ref_norm = float(np.linalg.norm(r))
    rel_l2 = float(np.linalg.norm(g - r) / ref_norm) if ref_norm > 0 else float(np.linalg.norm(g - r))
    ref_max = float(np.abs(r).max()) if r.size else 0.0
    return max_abs, rel_l2, ref_max


def assert_parity(got, ref, dtype: str, what: str = ""):
    g = f64(got)
    assert g.shape == np.shape(ref), (what, g.shape, np.shape(ref))
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    max_abs, rel_l2, ref_max = errors(g, ref)
    t = TOL[dtype]
    msg = f"{what}: max_abs={max_abs:.3e} rel_l2={rel_l2:.3e} max|ref|={ref_max:.3e}"
    assert max_abs <= t["max_abs"], msg
    assert rel_l2 <= t["rel_l2"], msg
    assert max_abs <= t["rel_max"] * max(ref_max, 1e-30) or max_abs == 0.0, msg
    return max_abs, rel_l2
