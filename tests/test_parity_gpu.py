"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
the same seeded inputs. CPU-sized cases are compared element by element;
the full-size workloads, in the launch configuration the benchmark times,
are compared on sampled rows."""
import sys
import zlib

import numpy as np
import pytest
import torch

import hstu_jagged_attention_amd as hj
from hstu_jagged_attention_amd import workloads as wl
from _helpers import (assert_parity, assert_parity_fp8, f64, gpu_device, oracle_jagged, oracle_jagged_sampled,
                      oracle_paged, run_jagged, run_paged)

pytestmark = pytest.mark.gpu
CAUSAL, NONE = wl.MASK_CAUSAL, wl.MASK_NONE


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


# ------------------------------------------------------------ the five workloads, CPU-sized
def test_tiny_fp32_bidirectional_full(dev):
    c = wl.tiny_fp32_bidirectional()
    say("tiny_fp32_bidirectional", c.lengths.tolist())
    got = run_jagged(c, dev)
    assert_parity(got, oracle_jagged(c), "f32", "C1")


@pytest.mark.parametrize("name,batch", [("bf16_mha_causal", 3), ("bf16_rab_target", 2), ("fp16_gqa_causal", 2)])
def test_workload_reduced_batch(dev, name, batch):
    c = wl.WORKLOADS[name](batch=batch)
    say(name, "batch", batch, c.lengths.tolist())
    got = run_jagged(c, dev)
    assert_parity(got, oracle_jagged(c), c.dtype, name)


def test_paged_workload_reduced(dev):
    pc = wl.bf16_paged_target(batch=6)
    say("bf16_paged_target batch 6", pc.history_lengths.tolist(), pc.new_lengths.tolist())
    got = run_paged(pc, dev)
    assert_parity(got, oracle_paged(pc), "bf16", "C5 reduced")


# ------------------------------------------------------------ full sizes, sampled rows
def _picks(c, n_seq=3, n_rows=12, seed=0):
    rng = np.random.default_rng(seed)
    L = c.lengths
    seqs = {int(np.argmax(L)), int(np.argmin(L))}
    while len(seqs) < min(n_seq, c.batch):
        seqs.add(int(rng.integers(c.batch)))
    picks = {}
    for b in sorted(seqs):
        n = int(L[b])
        rows = {0, n - 1, n // 2}
        if c.num_targets is not None:
            nt = min(int(c.num_targets[b]), n)
            rows |= {n - nt, max(n - nt - 1, 0)}
        if c.num_context is not None:
            rows |= {max(min(int(c.num_context[b]), n) - 1, 0)}
        while len(rows) < min(n_rows, n):
            rows.add(int(rng.integers(n)))
        picks[b] = [(r, h) for r in sorted(rows) for h in range(c.num_heads_q)]
    return picks


@pytest.mark.parametrize("name", ["bf16_mha_causal", "bf16_rab_target", "fp16_gqa_causal"])
def test_workload_full_size_sampled(dev, name):
    c = wl.WORKLOADS[name]()
    say(name, "full size: B", c.batch, "T", int(c.seq_offsets[-1]))
    got = run_jagged(c, dev).cpu()
    ref = oracle_jagged_sampled(c, _picks(c))
    for b, (toks, heads, vals) in ref.items():
        assert_parity(got[torch.as_tensor(toks), torch.as_tensor(heads)], vals, c.dtype, f"{name} seq {b}")


def test_paged_workload_full_size_sampled(dev):
    pc = wl.bf16_paged_target()
    say("bf16_paged_target full size: B", pc.batch, "Tq", int(pc.seq_offsets_q[-1]))
    got = run_paged(pc, dev).cpu()
    rng = np.random.default_rng(3)
    reqs = set(rng.choice(pc.batch, 6, replace=False).tolist()) | {int(np.argmax(pc.history_lengths))}
    rows = []
    for b in sorted(reqs):
        q0, q1 = int(pc.seq_offsets_q[b]), int(pc.seq_offsets_q[b + 1])
        for t in sorted({q0, q1 - 1, (q0 + q1) // 2}):
            rows += [(t, h) for h in range(pc.num_heads_q)]
    ref = oracle_paged(pc, rows=rows)
    idx_t = torch.as_tensor([t for t, _ in rows])
    idx_h = torch.as_tensor([h for _, h in rows])
    assert_parity(got[idx_t, idx_h], ref, "bf16", "C5 full sampled")


# ------------------------------------------------------------ edge cases
EDGE = [
    # (name, lengths, Hq, Hk, D, dtype, mask, nc, nt, g, rab, S)
    ("single_token_seqs", [1, 1, 3], 2, 2, 64, "bf16", CAUSAL, None, None, 0, False, None),
    ("empty_seqs_inside", [0, 37, 0, 129, 0], 2, 1, 64, "bf16", CAUSAL, 3, 5, 1, True, None),
    ("ragged_tails", [31, 33, 65, 127, 129, 200], 4, 4, 128, "bf16", CAUSAL, None, None, 0, False, None),
    ("bidirectional_ragged", [17, 130, 64], 2, 2, 128, "f16", NONE, None, None, 0, True, None),
    ("context_targets_exceed_L", [10, 40, 70], 2, 2, 64, "bf16", CAUSAL, (5, 60), (20, 90), 1, True, None),
    ("group_size_3", [90, 150], 4, 2, 128, "bf16", CAUSAL, (0, 10), (10, 40), 3, True, None),
    ("group_size_0_with_targets", [90, 150], 4, 2, 128, "f16", CAUSAL, (0, 10), (10, 40), 0, False, None),
    ("all_targets", [50, 80], 2, 2, 64, "bf16", CAUSAL, 0, 200, 2, False, None),
    ("rab_odd_max_seq_len", [77, 101], 2, 2, 64, "bf16", CAUSAL, (0, 4), (1, 9), 1, True, 103),
    ("gqa_group_2", [150, 270], 4, 2, 128, "bf16", CAUSAL, None, (1, 16), 1, False, None),
    ("gqa_group_3", [150, 270], 6, 2, 64, "f16", CAUSAL, None, (1, 16), 1, True, None),
    ("gqa_group_8", [150, 270], 8, 1, 128, "f16", CAUSAL, (0, 8), (1, 16), 1, False, None),
    ("head_dim_32_bf16", [100, 260], 2, 2, 32, "bf16", CAUSAL, (0, 8), (1, 16), 1, True, None),
    ("head_dim_256_bf16", [100, 260], 2, 2, 256, "bf16", CAUSAL, (0, 8), (1, 16), 1, True, None),
    ("head_dim_256_f16", [70, 200], 4, 1, 256, "f16", NONE, None, None, 0, False, None),
    ("fp32_causal_d64", [70, 150], 2, 2, 64, "f32", CAUSAL, (0, 8), (1, 16), 1, True, None),
    ("fp32_gqa_d128", [70, 150], 4, 2, 128, "f32", CAUSAL, None, (1, 16), 2, False, None),
    ("fp32_bidirectional_d32", [5, 300], 2, 1, 32, "f32", NONE, None, None, 0, True, None),
]


@pytest.mark.parametrize("case", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(dev, case):
    name, lengths, Hq, Hk, D, dtype, mask, nc, nt, g, rab, S = case
    c = wl.jagged_case(zlib.crc32(name.encode()) % (1 << 30), lengths, Hq, Hk, D, dtype, mask_type=mask, num_context=nc,
                       num_targets=nt, target_group_size=g, rab_std=0.5 if rab else None, max_seq_len=S)
    say(name, lengths, Hq, Hk, D, dtype)
    got = run_jagged(c, dev)
    assert_parity(got, oracle_jagged(c), dtype, name)


# Batches too large for one item per CU run on the work-list path (plan kernel,
# 4-wave workgroups, queue); the small cases above run on the direct key-split
# path. The same edge shapes, many sequences at once, cover the former.
LENGTH_MIX = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 255, 256, 257, 300]
WORK_LIST = [
    # (name, Hq, Hk, D, dtype, mask, nc, nt, g, rab)
    ("mha_bf16_ctx_targets_rab", 2, 2, 128, "bf16", CAUSAL, (0, 12), (0, 40), 1, True),
    ("gqa_f16_targets_g3", 4, 2, 64, "f16", CAUSAL, None, (1, 30), 3, False),
    ("bidirectional_bf16_rab", 2, 1, 128, "bf16", NONE, None, None, 0, True),
]


@pytest.mark.parametrize("case", WORK_LIST, ids=[e[0] for e in WORK_LIST])
def test_work_list_path_edge_mix(dev, case):
    name, Hq, Hk, D, dtype, mask, nc, nt, g, rab = case
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    lengths = rng.permutation(np.resize(np.array(LENGTH_MIX), 96))
    c = wl.jagged_case(zlib.crc32(name.encode()) % (1 << 30), lengths, Hq, Hk, D, dtype, mask_type=mask,
                       num_context=nc, num_targets=nt, target_group_size=g, rab_std=0.5 if rab else None,
                       max_seq_len=300)
    group = Hq // Hk
    hpw = 4 if group % 4 == 0 else (2 if group % 2 == 0 else 1)
    bm = 32 * (4 // hpw)
    items = c.batch * -(-c.max_seq_len // bm) * (Hq // hpw)
    assert items > torch.cuda.get_device_properties(dev).multi_processor_count, "case must exceed one item per CU"
    say(name, "batch", c.batch, "items", items)
    got = run_jagged(c, dev)
    assert_parity(got, oracle_jagged(c), dtype, name)


# Work-list batches of 60 sequences with lengths from 0 to 700 (ragged tails
# around every tile boundary) over every mask kind, GQA groups 4, 2 and 1
# and head_dim 64 / 128, element by element.
WORK_LIST_MIX = [
    # (name, Hq, Hk, D, dtype, mask, nc, nt, g)
    ("gqa4_f16_d128_ctx_targets_g1", 8, 2, 128, "f16", CAUSAL, (0, 40), (0, 70), 1),
    ("gqa4_bf16_d128_targets_g3", 4, 1, 128, "bf16", CAUSAL, None, (1, 90), 3),
    ("gqa4_f16_d64_targets_g0", 8, 2, 64, "f16", CAUSAL, (0, 20), (0, 50), 0),
    ("gqa2_bf16_d128_causal", 4, 2, 128, "bf16", CAUSAL, None, None, 0),
    ("mha_bf16_d128_ctx_targets", 2, 2, 128, "bf16", CAUSAL, (0, 30), (1, 40), 1),
    ("mha_f16_d64_bidirectional", 2, 1, 64, "f16", NONE, None, None, 0),
    ("gqa4_bf16_d128_bidirectional", 8, 2, 128, "bf16", NONE, None, None, 0),
]
TG_LENGTHS = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 255, 256, 257, 300, 511, 513, 700]


@pytest.mark.parametrize("case", WORK_LIST_MIX, ids=[e[0] for e in WORK_LIST_MIX])
def test_work_list_ragged_mask_mix(dev, case):
    name, Hq, Hk, D, dtype, mask, nc, nt, g = case
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    lengths = rng.permutation(np.resize(np.array(TG_LENGTHS), 60))
    c = wl.jagged_case(zlib.crc32(name.encode()) % (1 << 30), lengths, Hq, Hk, D, dtype, mask_type=mask,
                       num_context=nc, num_targets=nt, target_group_size=g, max_seq_len=700, name=name)
    group = Hq // Hk
    hpw = 4 if group % 4 == 0 else (2 if group % 2 == 0 else 1)
    items_4w = c.batch * -(-c.max_seq_len // (32 * (4 // hpw))) * (Hq // hpw)
    assert items_4w > torch.cuda.get_device_properties(dev).multi_processor_count, "case must take the work-list path"
    say(name, "batch", c.batch, "items", items_4w)
    got = run_jagged(c, dev)
    assert_parity(got, oracle_jagged(c), dtype, name)


def test_gqa_work_list_graph_replay_and_determinism(dev):
    """The GQA work-list run's queue counters survive graph replays, and
    runs are bitwise deterministic."""
    c = wl.fp16_gqa_causal(batch=3)
    say("gqa work-list graph", c.lengths.tolist())
    s = torch.cuda.Stream(dev)
    with torch.cuda.stream(s):
        prep = _prepare(c, dev)
        prep.plan()
        prep.run()
        s.synchronize()
        eager = prep.out.clone()
        prep.run()
        s.synchronize()
        assert torch.equal(prep.out, eager)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            prep.plan()
            prep.run()
        for _ in range(3):
            prep.out.zero_()
            g.replay()
            s.synchronize()
            assert torch.equal(prep.out, eager)
    assert_parity(eager, oracle_jagged(c), c.dtype, "gqa work-list graph")


@pytest.mark.parametrize("batch", [2, 40])
def test_fp16_large_q_alpha_one(dev, batch):
    """fp16 with alpha = 1 and |q| entries near 6e4 (small k): alpha*log2(e)*q
    exceeds fp16's range, so Q is pre-scaled by c / 2^k and S restored by
    2^k; the result must match the oracle (no overflow to inf). batch 2 runs
    the direct key-split kernel, batch 40 the work-list kernel."""
    rng = np.random.default_rng(77)
    lengths = rng.integers(40, 300, size=batch)
    c = wl.jagged_case(78 + batch, lengths, 4, 4, 64, "f16", num_targets=(1, 9), target_group_size=1,
                       max_seq_len=300, name="large_q")
    q = c.q.float()
    big = torch.as_tensor(rng.uniform(5e4, 6.5e4, size=q.shape), dtype=torch.float32)
    sign = torch.as_tensor(rng.choice([-1.0, 1.0], size=q.shape), dtype=torch.float32)
    pick = torch.as_tensor(rng.random(q.shape) < 0.05)
    c.q = torch.where(pick, big * sign, q).half()
    c.k = (c.k.float() * 1e-4).half()
    c.alpha = 1.0
    say("large |q| fp16 alpha 1, batch", batch)
    got = run_jagged(c, dev)
    assert torch.isfinite(got.float()).all()
    assert_parity(got, oracle_jagged(c), "f16", "large q")


# ------------------------------------------------------------ FP8 cast (E4M3 inputs, P cast to E4M3, bf16 out)
FP8_CASES = [
    # (name, lengths, Hq, Hk, mask, nc, nt, g)
    ("fp8_direct_causal", [200, 77, 300, 1], 4, 4, CAUSAL, None, None, 0),
    ("fp8_direct_gqa_ctx_targets", [150, 270, 33], 8, 2, CAUSAL, (0, 20), (1, 40), 1),
    ("fp8_direct_bidirectional", [65, 129, 200], 2, 1, NONE, None, None, 0),
    ("fp8_work_list_targets_g3", [int(x) for x in np.resize([0, 1, 31, 33, 64, 65, 127, 129, 300, 257], 90)], 4, 2,
     CAUSAL, (0, 12), (1, 50), 3),
    ("fp8_work_list_mha", [int(x) for x in np.resize([63, 64, 65, 200, 255, 256, 511], 70)], 4, 4, CAUSAL, None,
     (0, 30), 1),
]


@pytest.mark.parametrize("case", FP8_CASES, ids=[e[0] for e in FP8_CASES])
def test_fp8_cast(dev, case):
    """FP8 cast on v_mfma_f32_32x32x64_f8f6f4, element by element against the
    oracle with its E4M3 cast of P; the oracle without that cast is much
    further away, so the kernel does cast P."""
    name, lengths, Hq, Hk, mask, nc, nt, g = case
    c = wl.jagged_case(zlib.crc32(name.encode()) % (1 << 30), lengths, Hq, Hk, 128, "fp8", mask_type=mask,
                       num_context=nc, num_targets=nt, target_group_size=g, name=name)
    say(name, "batch", c.batch, "heads", Hq, Hk)
    got = run_jagged(c, dev)
    assert got.dtype == torch.bfloat16
    _, rel_cast = assert_parity_fp8(got, oracle_jagged(c), c, what=name)
    import oracle as orc
    plain = orc.hstu_fwd(f64(c.q), f64(c.k), f64(c.v), c.seq_offsets, num_context=c.num_context,
                         num_targets=c.num_targets, max_seq_len=c.max_seq_len, mask_type=c.mask_type,
                         target_group_size=c.target_group_size, alpha=c.alpha, out_scale=c.out_scale)
    g64 = f64(got)
    rel_plain = float(np.linalg.norm(g64 - plain) / np.linalg.norm(plain))
    assert rel_plain > 3 * rel_cast, (rel_plain, rel_cast)


def test_fp8_workload_reduced_and_sampled(dev):
    c = wl.fp8_gqa_causal(batch=2)
    say("fp8_gqa_causal batch 2", c.lengths.tolist())
    assert_parity_fp8(run_jagged(c, dev), oracle_jagged(c), c, what="fp8_gqa_causal reduced")
    c = wl.fp8_gqa_causal()
    say("fp8_gqa_causal full size: B", c.batch, "T", int(c.seq_offsets[-1]))
    got = run_jagged(c, dev).cpu()
    ref = oracle_jagged_sampled(c, _picks(c))
    for b, (toks, heads, vals) in ref.items():
        assert_parity_fp8(got[torch.as_tensor(toks), torch.as_tensor(heads)], vals, c, toks, heads,
                          f"fp8_gqa_causal seq {b}")


def test_every_row_is_written(dev):
    c = wl.jagged_case(5, [45, 0, 200, 1], 4, 2, 128, "bf16", num_targets=(1, 9), target_group_size=1)
    say("every_row_is_written")
    out = torch.full(tuple(c.q.shape), float("nan"), dtype=c.q.dtype, device=dev)
    got = run_jagged(c, dev, out=out)
    assert torch.isfinite(got).all()
    assert_parity(got, oracle_jagged(c), "bf16", "nan-prefilled out")


@pytest.mark.parametrize("S", [140, 144])
def test_masked_rab_nan_is_never_read(dev, S):
    """NaN in masked rab entries and in the padding never reaches the output
    (bit-identical to the run with those entries zero). S = 144 stages rab
    through the LDS ring, which reads padding columns of the last tiles."""
    c = wl.jagged_case(6, [130, 70], 2, 2, 128, "bf16", num_context=(2, 6), num_targets=(3, 9), target_group_size=1,
                       rab_std=0.3, max_seq_len=S)
    say("masked_rab_nan S", S)
    import oracle
    clean = c.rab.clone()
    poisoned = c.rab.clone()
    for b in range(2):
        L = int(c.lengths[b])
        clean[b, :, L:, :] = 0
        clean[b, :, :, L:] = 0
        M = torch.as_tensor(oracle.mask_matrix(CAUSAL, L, int(c.num_context[b]), int(c.num_targets[b]), 1))
        blk = poisoned[b, :, :L, :L]
        blk[:, ~M] = float("nan")
    a = run_jagged(c, dev, rab=clean.to(dev))
    bq = run_jagged(c, dev, rab=poisoned.to(dev))
    assert torch.isfinite(bq).all()
    assert torch.equal(a, bq)


def test_run_to_run_bitwise_deterministic(dev):
    c = wl.bf16_rab_target(batch=3)
    say("determinism")
    a = run_jagged(c, dev)
    b = run_jagged(c, dev)
    assert torch.equal(a, b)


def test_gqa_equals_repeated_mha_on_gpu(dev):
    c = wl.jagged_case(7, [200, 90], 8, 2, 128, "f16", num_targets=(1, 9), target_group_size=1)
    say("gqa_vs_mha")
    a = run_jagged(c, dev)
    krep = c.k.repeat_interleave(4, dim=1).contiguous().to(dev)
    vrep = c.v.repeat_interleave(4, dim=1).contiguous().to(dev)
    b = hj.hstu_fwd(c.q.to(dev), krep, vrep, torch.as_tensor(c.seq_offsets), num_targets=c.num_targets,
                    max_seq_len=c.max_seq_len, target_group_size=1, alpha=c.alpha, out_scale=c.out_scale)
    # The two layouts tile and split the key range differently, so fp32
    # partial sums are grouped differently: equal up to output rounding.
    d = (a.double() - b.double()).abs().max().item()
    assert d <= 2e-3 * b.double().abs().max().item(), d


@pytest.mark.parametrize("page_size", [32, 64, 128, 256])
def test_paged_page_sizes(dev, page_size):
    pc = wl.paged_case(30 + page_size, [0, 1, 63, 64, 65, 300], [3, 1, 7, 64, 2, 33], 4, 2, 128, "bf16",
                       page_size=page_size, num_context=(0, 4), target_group_size=2, extra_pages=3)
    say("paged page_size", page_size)
    got = run_paged(pc, dev)
    assert_parity(got, oracle_paged(pc), "bf16", f"paged ps={page_size}")


@pytest.mark.parametrize("dtype,D", [("f16", 64), ("f32", 32), ("bf16", 256)])
def test_paged_dtypes(dev, dtype, D):
    pc = wl.paged_case(40, [100, 257], [5, 40], 2, 2, D, dtype, page_size=64, target_group_size=1)
    say("paged", dtype, D)
    got = run_paged(pc, dev)
    assert_parity(got, oracle_paged(pc), dtype, f"paged {dtype} D={D}")


# Key-split calls whose items split into about eight chunks each (the
# reduction's loads of four chunks at a time and their remainder; the
# planner's per-cost chunk positions), with query counts on both sides of
# every 32-row block of an item.
SPLIT_ROWS = [1, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 200]


def test_key_split_many_chunks_row_blocks_jagged(dev):
    lk = [4000 + 37 * i for i in range(len(SPLIT_ROWS))]
    c = wl.jagged_case(61, lk, 4, 4, 128, "bf16", num_targets=SPLIT_ROWS, target_group_size=1,
                       q_lengths=SPLIT_ROWS, max_seq_len=4500, name="split_many_jagged")
    say(c.name, "batch", c.batch)
    got = run_jagged(c, dev)
    assert_parity(got, oracle_jagged(c), "bf16", c.name)


@pytest.mark.parametrize("Hq,Hk", [(4, 4), (8, 4)])
def test_key_split_many_chunks_row_blocks_paged(dev, Hq, Hk):
    newl = [1, 31, 32, 33, 63, 64, 65, 100]
    hist = [3900 + 53 * i for i in range(len(newl))]
    pc = wl.paged_case(62 + Hq, hist, newl, Hq, Hk, 128, "f16", page_size=64, target_group_size=1)
    say("split_many_paged", Hq, Hk)
    got = run_paged(pc, dev)
    assert_parity(got, oracle_paged(pc), "f16", f"split_many_paged {Hq}/{Hk}")


def test_paged_equals_gathered_jagged_on_gpu(dev):
    pc = wl.paged_case(41, [130, 64, 5], [9, 3, 12], 4, 4, 128, "bf16", page_size=64, num_context=(0, 3),
                       target_group_size=1)
    say("paged_vs_gathered")
    got = run_paged(pc, dev).cpu()
    kv = pc.kv_cache
    ks, vs, qs, offs = [], [], [], [0]
    for b in range(pc.batch):
        Lh = int(pc.history_lengths[b])
        pages = torch.as_tensor(pc.page_ids[pc.page_offsets[b]:pc.page_offsets[b + 1]])
        pos = torch.arange(Lh)
        q0, q1 = int(pc.seq_offsets_q[b]), int(pc.seq_offsets_q[b + 1])
        ks.append(torch.cat([kv[pages[pos // 64], 0, pos % 64], pc.k_new[q0:q1]]))
        vs.append(torch.cat([kv[pages[pos // 64], 1, pos % 64], pc.v_new[q0:q1]]))
        qs.append(torch.cat([torch.zeros(Lh, 4, 128, dtype=pc.q.dtype), pc.q[q0:q1]]))
        offs.append(offs[-1] + Lh + q1 - q0)
    out = hj.hstu_fwd(torch.cat(qs).to(dev), torch.cat(ks).to(dev), torch.cat(vs).to(dev), torch.as_tensor(offs),
                      num_context=pc.num_context, num_targets=pc.num_targets, max_seq_len=pc.max_seq_len,
                      target_group_size=1, alpha=pc.alpha, out_scale=pc.out_scale).cpu()
    for b in range(pc.batch):
        Lh = int(pc.history_lengths[b])
        q0, q1 = int(pc.seq_offsets_q[b]), int(pc.seq_offsets_q[b + 1])
        a, bb = got[q0:q1].double(), out[offs[b] + Lh: offs[b + 1]].double()
        assert (a - bb).abs().max().item() <= 2e-2 * max(bb.abs().max().item(), 1e-30)


def test_page_running_case_shape(dev):
    # GQA running case of the operator page: B=2, S=256, 8 q heads, 2 kv heads, D=64, fp16,
    # offsets [0, 128, 256], causal, silu_scale 1/256; q holds 512 tokens, out has q's shape.
    g = torch.Generator().manual_seed(0)
    q = torch.randn(512, 8, 64, generator=g).half()
    k = torch.randn(512, 2, 64, generator=g).half()
    v = torch.randn(512, 2, 64, generator=g).half()
    say("page running case")
    out = hj.hstu_fwd(q.to(dev), k.to(dev), v.to(dev), torch.tensor([0, 128, 256]), max_seq_len=256,
                      mask_type=CAUSAL, out_scale=1.0 / 256)
    assert tuple(out.shape) == (512, 8, 64)
    import oracle
    ref = oracle.hstu_fwd(f64(q[:256]), f64(k[:256]), f64(v[:256]), [0, 128, 256], max_seq_len=256, mask_type=CAUSAL,
                          out_scale=1.0 / 256)
    assert_parity(out[:256], ref, "f16", "page running case")


# ------------------------------------------------------------ user mask, rab broadcast, delta-QK
CUSTOM = wl.MASK_CUSTOM
NEXT = [
    # (name, key lengths, query lengths or None, Hq, Hk, D, dtype, mask, nc, nt, g, rab_std, rab_heads,
    #  mask_keep, mask_heads, S)
    ("user_mask_bf16", [200, 77, 300], None, 4, 4, 128, "bf16", CUSTOM, None, None, 0, None, None, 0.5, None, None),
    ("user_mask_rab_bcast_f16", [130, 64, 257], None, 4, 2, 128, "f16", CUSTOM, None, None, 0, 0.1, 1, 0.3, 1, None),
    ("user_mask_gqa_d64_odd_S", [90, 150], None, 6, 2, 64, "bf16", CUSTOM, None, None, 0, 0.5, None, 0.7, 1, 151),
    ("user_mask_d256", [70, 130], None, 2, 2, 256, "bf16", CUSTOM, None, None, 0, 0.1, 2, 0.5, 2, None),
    ("user_mask_d32_empty_seq", [0, 40, 1], None, 2, 2, 32, "f16", CUSTOM, None, None, 0, None, None, 0.5, None, None),
    ("user_mask_many_seqs", [60 + 7 * i for i in range(40)], None, 4, 4, 128, "bf16", CUSTOM, None, None, 0, 0.1, 1,
     0.5, None, None),
    ("rab_bcast_causal", [150, 270], None, 4, 4, 128, "bf16", CAUSAL, (0, 8), (1, 16), 1, 0.5, 1, None, None, None),
    ("rab_bcast_gqa_f16", [150, 270], None, 8, 2, 128, "f16", CAUSAL, None, (1, 16), 1, 0.5, 1, None, None, None),
    ("delta_causal_targets", [600, 333, 1030], [40, 333, 1], 4, 4, 128, "bf16", CAUSAL, None, [40, 333, 1], 1, None,
     None, None, None, None),
    ("delta_ctx_rab", [500, 260], [70, 9], 4, 2, 128, "f16", CAUSAL, (0, 20), (1, 30), 2, 0.1, None, None, None, None),
    ("delta_none_gqa", [300, 129], [64, 129], 8, 2, 64, "bf16", NONE, None, None, 0, None, None, None, None, None),
    ("delta_d256", [300, 129], [64, 100], 2, 2, 256, "bf16", CAUSAL, None, (1, 30), 1, 0.1, 1, None, None, None),
    ("delta_f32_rab_bcast", [200, 90], [33, 90], 2, 2, 64, "f32", CAUSAL, None, (1, 20), 1, 0.5, 1, None, None, None),
    ("delta_user_mask", [400, 150], [50, 150], 4, 4, 128, "bf16", CUSTOM, None, None, 0, 0.1, 1, 0.5, 4, None),
    ("delta_many_seqs", [500 + 13 * i for i in range(48)], [1 + (5 * i) % 64 for i in range(48)], 4, 4, 128, "bf16",
     CAUSAL, None, [1 + (5 * i) % 64 for i in range(48)], 1, None, None, None, None, None),
]


@pytest.mark.parametrize("case", NEXT, ids=[e[0] for e in NEXT])
def test_user_mask_rab_broadcast_delta_qk(dev, case):
    """The table's user mask (mask_type 3), rab broadcast [b, 1, s, s] and
    different Q/K lengths (seq_offsets_k), element by element against the
    oracle; spans several tiles, ragged tails, the direct and work-list
    launch modes, head dims 32..256 and the f32 path for delta-QK."""
    name, lk, lq, Hq, Hk, D, dt, mask, nc, nt, g, rab_std, rab_h, keep, mask_h, S = case
    seed = zlib.crc32(name.encode()) & 0xffff
    say(name, "seed", seed, "keys", lk, "queries", lq)
    c = wl.jagged_case(seed, lk, Hq, Hk, D, dt, mask_type=mask, num_context=nc, num_targets=nt, target_group_size=g,
                       rab_std=rab_std, rab_heads=rab_h, mask_keep=keep, mask_heads=mask_h, max_seq_len=S,
                       q_lengths=lq, name=name)
    got = run_jagged(c, dev)
    assert_parity(got, oracle_jagged(c), dt, name)


def test_user_mask_zero_removes_nan_rab_on_gpu(dev):
    """Zero user-mask entries contribute exactly zero even where rab is NaN:
    the output equals the run with those rab entries finite, bit for bit."""
    c = wl.jagged_case(91, [150, 64, 200], 4, 4, 128, "bf16", mask_type=CUSTOM, rab_std=0.1, mask_keep=0.5,
                       name="nan_under_zero_mask")
    say("nan_under_zero_mask")
    clean = run_jagged(c, dev).cpu()
    rab = c.rab.clone()
    rab[torch.nan_to_num(c.mask.float(), nan=1.0) == 0] = float("nan")
    got = run_jagged(c, dev, rab=rab.to(dev)).cpu()
    assert torch.isfinite(got.float()).all()
    assert torch.equal(got, clean)


@pytest.mark.parametrize("name", ["bf16_custom_mask", "bf16_delta_qk"])
def test_next_workloads_reduced_batch(dev, name):
    c = wl.WORKLOADS[name](batch=3)
    say(name, "batch 3", c.lengths.tolist(), c.key_lengths.tolist())
    got = run_jagged(c, dev)
    assert_parity(got, oracle_jagged(c), c.dtype, name)


@pytest.mark.parametrize("name", ["bf16_custom_mask", "bf16_delta_qk"])
def test_next_workloads_full_size_sampled(dev, name):
    c = wl.WORKLOADS[name]()
    say(name, "full size: B", c.batch, "Tq", int(c.seq_offsets[-1]))
    got = run_jagged(c, dev).cpu()
    ref = oracle_jagged_sampled(c, _picks(c))
    for b, (toks, heads, vals) in ref.items():
        assert_parity(got[torch.as_tensor(toks), torch.as_tensor(heads)], vals, c.dtype, f"{name} seq {b}")


# ------------------------------------------------------------ HIP graph capture
def _prepare(c, dev):
    return hj.prepare_fwd(c.q.to(dev), c.k.to(dev), c.v.to(dev), torch.as_tensor(c.seq_offsets),
                          rab=None if c.rab is None else c.rab.to(dev),
                          seq_offsets_k=None if c.seq_offsets_k is None else torch.as_tensor(c.seq_offsets_k),
                          num_context=c.num_context, num_targets=c.num_targets, max_seq_len=c.max_seq_len,
                          mask_type=c.mask_type, target_group_size=c.target_group_size, alpha=c.alpha,
                          out_scale=c.out_scale)


@pytest.mark.parametrize("name,batch", [("bf16_mha_causal", 8), ("fp16_gqa_causal", 2), ("bf16_delta_qk", 6)])
def test_plan_and_run_replay_in_a_hip_graph(dev, name, batch):
    """plan + run captured in one HIP graph (direct mode, the work list with
    its queue counters, and key-split items with the ordered reduction):
    every replay, with eager launches of another call in between, equals the
    eager result bit for bit, so the counters the run rewinds and the plan
    rewrites survive replays."""
    c = wl.WORKLOADS[name](batch=batch)
    say("graph", name, "batch", batch)
    other = wl.bf16_mha_causal(batch=2)
    s = torch.cuda.Stream(dev)
    with torch.cuda.stream(s):
        prep = _prepare(c, dev)
        prep_other = _prepare(other, dev)
        prep.plan()
        prep.run()
        s.synchronize()
        eager = prep.out.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            prep.plan()
            prep.run()
        for _ in range(4):
            prep.out.zero_()
            g.replay()
            s.synchronize()
            assert torch.equal(prep.out, eager)
            prep_other.fwd()  # eager work on the same stream between replays
            s.synchronize()
    assert_parity(eager, oracle_jagged(c), c.dtype, f"graph {name}")


# ------------------------------------------------------------ seeded random configurations
def _random_case(i):
    """Configuration i of a seeded sweep over the ABI's space: dtype, head
    dim, head counts, ragged and empty lengths, the three mask kinds with
    context / targets / groups, rab with one or all heads, odd max_seq_len,
    and different Q/K lengths."""
    rng = np.random.default_rng(9000 + i)
    dt = ["bf16", "f16", "f32"][i % 3]
    D = int(rng.choice([32, 64, 128] if dt == "f32" else [32, 64, 128, 256]))
    Hq, Hk = [(1, 1), (2, 1), (4, 4), (4, 2), (6, 3), (8, 2)][int(rng.integers(6))]
    B = int(rng.integers(1, 6))
    lk = rng.integers(0, 300, size=B)
    lk[int(rng.integers(B))] = max(int(lk.max()), 1)
    mask = int(rng.choice([CAUSAL, NONE, CUSTOM] if dt != "f32" else [CAUSAL, NONE]))
    delta = bool(rng.integers(2))
    lq = np.minimum(rng.integers(1, 80, size=B), lk) if delta else None
    S = int(lk.max()) + int(rng.integers(0, 3))
    kw = {}
    if mask == CAUSAL:
        kw.update(num_context=(0, 40) if rng.integers(2) else None,
                  num_targets=(0, 60) if rng.integers(2) else None, target_group_size=int(rng.integers(0, 4)))
    if rng.integers(2):
        kw.update(rab_std=0.2, rab_heads=int(rng.choice([1, Hq])))
    if mask == CUSTOM:
        kw.update(mask_keep=float(rng.uniform(0.2, 0.9)), mask_heads=int(rng.choice([1, Hq])))
    return wl.jagged_case(9000 + i, lk, Hq, Hk, D, dt, mask_type=mask, max_seq_len=S, q_lengths=lq,
                          name=f"random_{i}", **kw)


@pytest.mark.parametrize("i", range(24))
def test_random_configurations(dev, i):
    c = _random_case(i)
    say(c.name, c.dtype, "D", c.head_dim, "heads", c.num_heads_q, c.num_heads_kv, "mask", c.mask_type,
        "keys", c.key_lengths.tolist(), "queries", c.lengths.tolist(), "rab", c.rab is not None,
        "S", c.max_seq_len)
    got = run_jagged(c, dev)
    assert_parity(got, oracle_jagged(c), c.dtype, c.name)


# ------------------------------------------------------------ debug validation, guard bands, block-table permutation
def _raw_fwd(c, dev, off, max_seq_len, offk=None, out=None):
    """hstu_fwd through the C ABI with explicit int32 device offsets (no
    marshalling checks on their contents); returns (status, out)."""
    lib = hj.load_library()
    import ctypes
    q, k, v = c.q.to(dev), c.k.to(dev), c.v.to(dev)
    out = torch.full(tuple(c.q.shape), 7.0, dtype=c.q.dtype, device=dev) if out is None else out
    offd = torch.as_tensor(off, dtype=torch.int32, device=dev)
    offkd = None if offk is None else torch.as_tensor(offk, dtype=torch.int32, device=dev)
    B = len(off) - 1
    Hq, Hk, D = c.num_heads_q, c.num_heads_kv, c.head_dim
    code = hj.DTYPE_CODES[c.q.dtype]
    need = int(lib.hstu_fwd_workspace_size(B, max_seq_len, Hq, Hk, D, code, 0 if offk is None else 1))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    P = ctypes.c_void_p
    st = lib.hstu_fwd(P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), None, None, P(out.data_ptr()),
                      P(offd.data_ptr()), None if offkd is None else P(offkd.data_ptr()), None, None, B, max_seq_len,
                      Hq, Hk, D, 1, 1, CAUSAL, 0, 0, c.alpha, c.out_scale, code, P(ws.data_ptr()), need,
                      P(torch.cuda.current_stream(dev).cuda_stream))
    torch.cuda.synchronize(dev)
    return st, out


@pytest.mark.parametrize("bad", ["first_not_zero", "decreasing", "too_long", "queries_exceed_keys"])
def test_validate_mode_rejects_malformed_offsets(dev, bad, monkeypatch):
    """HSTU_VALIDATE=1: malformed device offsets return HSTU_ERR_INVALID_ARG
    and no forward kernel runs (out keeps its fill value); the same call with
    valid offsets passes and matches the oracle."""
    c = wl.jagged_case(321, [40, 70, 33], 4, 2, 64, "bf16")
    good = [0, 40, 110, 143]
    off, offk, S = list(good), None, c.max_seq_len
    if bad == "first_not_zero":
        off = [3, 40, 110, 143]
    elif bad == "decreasing":
        off = [0, 40, 30, 143]
    elif bad == "too_long":
        S = 60  # the second sequence has 70 keys
    else:
        offk = [0, 40, 100, 143]  # sequence 1: 70 queries, 60 keys
    monkeypatch.setenv("HSTU_VALIDATE", "1")
    say("validate", bad)
    st, out = _raw_fwd(c, dev, off, S, offk=offk)
    assert st == hj.HSTU_ERR_INVALID_ARG, st
    assert bool((out == 7.0).all()), "a forward kernel ran on rejected inputs"
    st, out = _raw_fwd(c, dev, good, c.max_seq_len)
    assert st == hj.HSTU_OK
    assert_parity(out, oracle_jagged(c), "bf16", "validated call")
    monkeypatch.setenv("HSTU_VALIDATE", "0")
    st, _ = _raw_fwd(c, dev, good, c.max_seq_len)
    assert st == hj.HSTU_OK


GUARD = 4096  # bytes of canary before and after each buffer


def _guarded(nbytes, dev, fill):
    buf = torch.full((GUARD + nbytes + GUARD,), fill, dtype=torch.uint8, device=dev)
    return buf, buf[GUARD:GUARD + nbytes]


@pytest.mark.parametrize("kind", ["direct", "work_list", "delta_split", "paged_split", "fp8"])
def test_guard_bands_stay_intact(dev, kind):
    """Canary bytes around out and around the workspace are untouched by valid
    calls in every launch mode (direct, work list, key-split with the ordered
    reduction, paged, FP8)."""
    say("guard bands", kind)
    if kind == "paged_split":
        pc = wl.bf16_paged_target(batch=8)
        need = hj.hstu_fwd_paged_workspace_size(pc.batch, pc.page_size, pc.max_seq_len, pc.num_heads_q,
                                                pc.num_heads_kv, pc.head_dim, torch.bfloat16)
        wbuf, ws = _guarded(need, dev, 0xA5)
        obuf, ob = _guarded(pc.q.numel() * 2, dev, 0x5A)
        out = ob.view(torch.bfloat16).view(tuple(pc.q.shape))
        got = run_paged(pc, dev, out=out, workspace=ws)
        ref = oracle_paged(pc)
        assert_parity(got, ref, "bf16", "paged guarded")
    else:
        if kind == "direct":
            c = wl.jagged_case(401, [150, 1, 67, 300], 8, 2, 128, "bf16", num_targets=(1, 20), target_group_size=1)
        elif kind == "work_list":
            c = wl.jagged_case(402, np.resize([0, 31, 65, 129, 300], 80), 4, 2, 64, "f16", num_targets=(1, 9),
                               target_group_size=1, max_seq_len=300)
        elif kind == "delta_split":
            lk = [500 + 13 * i for i in range(48)]
            lq = [1 + (5 * i) % 64 for i in range(48)]
            c = wl.jagged_case(403, lk, 4, 4, 128, "bf16", num_targets=lq, target_group_size=1, q_lengths=lq)
        else:
            c = wl.jagged_case(404, np.resize([33, 200, 129], 60), 8, 2, 128, "fp8", num_targets=(1, 9),
                               target_group_size=1)
        odt = torch.bfloat16 if c.dtype == "fp8" else c.q.dtype
        need = hj.hstu_fwd_workspace_size(c.batch, c.max_seq_len, c.num_heads_q, c.num_heads_kv, c.head_dim,
                                          c.q.dtype, is_delta_qk=c.seq_offsets_k is not None)
        wbuf, ws = _guarded(need, dev, 0xA5)
        obuf, ob = _guarded(c.q.shape[0] * c.q.shape[1] * c.q.shape[2] * 2, dev, 0x5A)
        out = ob.view(odt).view(tuple(c.q.shape))
        got = run_jagged(c, dev, out=out, workspace=ws)
        if c.dtype == "fp8":
            assert_parity_fp8(got, oracle_jagged(c), c, what=f"guarded {kind}")
        else:
            assert_parity(got, oracle_jagged(c), c.dtype, f"guarded {kind}")
    torch.cuda.synchronize(dev)
    for buf, fill, what in ((wbuf, 0xA5, "workspace"), (obuf, 0x5A, "out")):
        head, tail = buf[:GUARD], buf[-GUARD:]
        assert bool((head == fill).all()) and bool((tail == fill).all()), f"{what} guard band overwritten"


def test_paged_block_table_permutation_bit_identical(dev):
    """Moving the pages of the pool under a random permutation of their ids
    (block table rewritten to match) leaves the paged output bit-identical."""
    pc = wl.paged_case(55, [300, 64, 1000, 5, 0], [9, 3, 40, 1, 7], 4, 2, 128, "bf16", page_size=64,
                       num_context=(0, 4), target_group_size=1, extra_pages=5)
    say("block-table permutation")
    a = run_paged(pc, dev)
    rng = np.random.default_rng(9)
    n_pool = pc.kv_cache.shape[0]
    perm = rng.permutation(n_pool)  # new slot of old page p is perm[p]
    kv2 = torch.empty_like(pc.kv_cache)
    kv2[torch.as_tensor(perm)] = pc.kv_cache
    pc.kv_cache = kv2
    pc.page_ids = perm[pc.page_ids]
    b = run_paged(pc, dev)
    assert torch.equal(a, b)


# ------------------------------------------------------------ local mask (sliding window on the causal mask)
LOCAL_MIX = [int(x) for x in np.resize([0, 1, 2, 31, 33, 63, 64, 65, 127, 129, 200, 256, 257, 300, 511, 700], 64)]
LOCAL = [
    # (name, key lengths, query lengths or None, Hq, Hk, D, dtype, nc, nt, g, rab_std, W)
    ("w1_bf16_direct", [200, 77, 300, 1], None, 4, 4, 128, "bf16", None, None, 0, None, 1),
    ("w64_f16_gqa_ctx_targets", [150, 270, 33], None, 8, 2, 128, "f16", (0, 20), (1, 40), 1, None, 64),
    ("w65_bf16_d64_ctx", [300, 129, 64], None, 2, 2, 64, "bf16", (0, 90), None, 0, None, 65),
    ("w100_bf16_rab_work_list", LOCAL_MIX, None, 2, 2, 128, "bf16", (0, 12), (0, 40), 1, 0.5, 100),
    ("w37_f16_d64_targets_g3_work_list", LOCAL_MIX, None, 8, 2, 64, "f16", None, (1, 90), 3, None, 37),
    ("w300_f16_gqa4_work_list", LOCAL_MIX, None, 8, 2, 128, "f16", None, (1, 32), 1, None, 300),
    ("w_ge_length_bf16", [200, 300], None, 2, 2, 128, "bf16", None, (0, 9), 1, None, 5000),
    ("w200_d256_bf16_rab", [300, 129], None, 2, 2, 256, "bf16", None, (1, 30), 1, 0.1, 200),
    ("w7_d32_f16_ctx", [0, 40, 1, 130], None, 2, 2, 32, "f16", (0, 5), None, 0, None, 7),
    ("w33_f32_rab", [200, 90], None, 2, 2, 64, "f32", None, (1, 20), 1, 0.5, 33),
    ("w129_delta_split", [600, 333, 1030], [40, 333, 1], 4, 4, 128, "bf16", None, [40, 333, 1], 1, None, 129),
    ("w64_delta_many", [500 + 13 * i for i in range(48)], [1 + (5 * i) % 64 for i in range(48)], 4, 4, 128, "bf16",
     None, [1 + (5 * i) % 64 for i in range(48)], 1, None, 64),
    ("w65_fp8_gqa_ctx_targets", [150, 270, 33], None, 8, 2, 128, "fp8", (0, 20), (1, 40), 1, None, 65),
    ("w100_fp8_work_list_g3", LOCAL_MIX, None, 4, 2, 128, "fp8", (0, 12), (1, 50), 3, None, 100),
]


@pytest.mark.parametrize("case", LOCAL, ids=[e[0] for e in LOCAL])
def test_local_window(dev, case):
    """The local mask (key j visible to query i only when the causal mask
    allows it and i - j < W), element by element against the oracle: windows
    of 1 to beyond the sequence, context and targets, GQA, head dims 32..256,
    every dtype, the direct and work-list modes and key-split delta-QK."""
    name, lk, lq, Hq, Hk, D, dt, nc, nt, g, rab_std, W = case
    seed = zlib.crc32(name.encode()) & 0xffff
    say(name, "seed", seed, "window", W, "batch", len(lk))
    c = wl.jagged_case(seed, lk, Hq, Hk, D, dt, mask_type=CAUSAL, num_context=nc, num_targets=nt,
                       target_group_size=g, rab_std=rab_std, q_lengths=lq, name=name, local_window=W)
    got = run_jagged(c, dev)
    if dt == "fp8":
        assert_parity_fp8(got, oracle_jagged(c), c, what=name)
    else:
        assert_parity(got, oracle_jagged(c), dt, name)
    if W >= int(c.key_lengths.max(initial=0)):
        # a window covering every sequence is no window, bit for bit
        assert torch.equal(got, run_jagged(c, dev, local_window=0))


def test_local_window_paged(dev):
    pc = wl.paged_case(57, [0, 1, 63, 64, 65, 300, 1000], [3, 1, 7, 64, 2, 33, 40], 4, 2, 128, "bf16", page_size=64,
                       num_context=(0, 4), target_group_size=1, extra_pages=2, local_window=70)
    say("paged local window 70")
    assert_parity(run_paged(pc, dev), oracle_paged(pc), "bf16", "paged local window")


def test_local_window_workload_reduced_and_sampled(dev):
    c = wl.fp16_gqa_local(batch=2)
    say("fp16_gqa_local batch 2", c.lengths.tolist())
    assert_parity(run_jagged(c, dev), oracle_jagged(c), "f16", "fp16_gqa_local reduced")
    c = wl.fp16_gqa_local()
    say("fp16_gqa_local full size: B", c.batch, "T", int(c.seq_offsets[-1]))
    got = run_jagged(c, dev).cpu()
    ref = oracle_jagged_sampled(c, _picks(c))
    for b, (toks, heads, vals) in ref.items():
        assert_parity(got[torch.as_tensor(toks), torch.as_tensor(heads)], vals, "f16", f"fp16_gqa_local seq {b}")


# ------------------------------------------------------------ rab / user mask through the LDS ring
# max_seq_len a multiple of 8 takes the ring (tiles of rab and the mask staged
# through LDS by DMA); 304 is not a multiple of the 32- or 64-key tile, so the
# last tiles reach past the row end (those chunks are clamped and masked).
RING_MIX = [int(x) for x in np.resize([0, 1, 7, 31, 32, 33, 63, 64, 65, 130, 200, 255, 257, 300, 304], 45)]
RING = [
    # (name, lengths, Hq, Hk, D, dtype, mask, nc, nt, g, rab_std, rab_heads, mask_keep, mask_heads, S)
    ("ring_rab_causal_ctx_targets", RING_MIX, 4, 4, 128, "bf16", CAUSAL, (0, 12), (0, 40), 1, 0.5, None, None, None, 304),
    ("ring_rab_gqa_f16", RING_MIX, 8, 2, 128, "f16", CAUSAL, None, (1, 30), 3, 0.5, None, None, None, 304),
    ("ring_rab_bcast_bidirectional", [150, 270, 33, 304], 4, 4, 128, "bf16", NONE, None, None, 0, 0.5, 1, None, None, 304),
    ("ring_rab_d32", [150, 270, 33, 1], 4, 2, 32, "bf16", CAUSAL, None, (1, 9), 1, 0.5, None, None, None, 272),
    ("ring_rab_d256", [150, 270, 33, 1], 2, 2, 256, "f16", CAUSAL, None, (1, 9), 1, 0.5, None, None, None, 272),
    ("ring_mask_only", RING_MIX, 4, 4, 128, "bf16", CUSTOM, None, None, 0, None, None, 0.5, None, 304),
    ("ring_mask_rab", RING_MIX, 4, 4, 128, "f16", CUSTOM, None, None, 0, 0.3, 1, 0.5, None, 304),
    ("ring_mask_gqa_d32", [150, 270, 33, 1, 64], 8, 2, 32, "bf16", CUSTOM, None, None, 0, 0.3, None, 0.6, 1, 272),
    ("ring_mask_d256", [150, 270, 33], 2, 2, 256, "bf16", CUSTOM, None, None, 0, 0.3, 2, 0.5, 2, 272),
]


@pytest.mark.parametrize("case", RING, ids=[e[0] for e in RING])
def test_ring_rab_and_mask(dev, case):
    """rab and the user mask staged through the LDS ring (max_seq_len a
    multiple of 8), element by element against the oracle; NaN fills the
    rab and mask entries outside each sequence, so any byte of the padding
    that reached the arithmetic would poison the output."""
    name, lengths, Hq, Hk, D, dt, mask, nc, nt, g, rab_std, rab_h, keep, mask_h, S = case
    seed = zlib.crc32(name.encode()) & 0xffff
    say(name, "seed", seed, "S", S, "batch", len(lengths))
    c = wl.jagged_case(seed, lengths, Hq, Hk, D, dt, mask_type=mask, num_context=nc, num_targets=nt,
                       target_group_size=g, rab_std=rab_std, rab_heads=rab_h, mask_keep=keep, mask_heads=mask_h,
                       max_seq_len=S, name=name)
    got = run_jagged(c, dev)
    assert_parity(got, oracle_jagged(c), dt, name)
