"""C-ABI checks that need no GPU: the library loads, exports every function
include/hstu.h declares, and rejects bad arguments on the host before any
launch. No call here reaches a kernel (each one fails validation first or is
an empty input that launches nothing)."""
import ctypes
import os
import re

import pytest

import hstu_jagged_attention_amd as hj

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hstu.h")

OK, INVAL, UNSUP, WS = hj.HSTU_OK, hj.HSTU_ERR_INVALID_ARG, hj.HSTU_ERR_UNSUPPORTED, hj.HSTU_ERR_WORKSPACE
BF16, F16, F32, FP8 = 2, 1, 0, 3
FAKE = 0x10000  # 16-byte aligned host integer, never dereferenced (calls fail validation first)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hstu_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return hj.load_library()


def test_header_and_binding_agree():
    assert declared_functions() == sorted(hj.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    for code in range(5):
        s = hj.status_string(code)
        assert s.startswith("HSTU_")
    assert "unknown" in hj.status_string(99)


def fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, rab=None, umask=None, out=FAKE, off=FAKE, offk=None, nc=None, nt=None, B=2,
             S=128, Hq=4, Hk=2, D=128, rab_h=4, mask_h=4, mask=0, g=0, win=0, alpha=1.0, osc=1.0, dt=BF16,
             ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.hstu_fwd(a["q"], a["k"], a["v"], a["rab"], a["umask"], a["out"], a["off"], a["offk"], a["nc"],
                        a["nt"], a["B"], a["S"], a["Hq"], a["Hk"], a["D"], a["rab_h"], a["mask_h"], a["mask"], a["g"],
                        a["win"], a["alpha"], a["osc"], a["dt"], a["ws"], a["wsb"], a["stream"])


def paged(lib, **kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, out=FAKE, offq=FAKE, cache=FAKE, poff=FAKE, pids=FAKE, lpl=FAKE, nc=None,
             nt=None, B=2, ps=64, S=128, Hq=4, Hk=4, D=128, mask=0, g=1, win=0, alpha=1.0, osc=1.0, dt=BF16,
             ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.hstu_fwd_paged(a["q"], a["kn"], a["vn"], a["out"], a["offq"], a["cache"], a["poff"], a["pids"],
                              a["lpl"], a["nc"], a["nt"], a["B"], a["ps"], a["S"], a["Hq"], a["Hk"], a["D"], a["mask"],
                              a["g"], a["win"], a["alpha"], a["osc"], a["dt"], a["ws"], a["wsb"], a["stream"])


def test_empty_inputs_are_a_noop(lib):
    # The page: a zero B, N or D means the operator does not run.
    assert fwd(lib, B=0, q=None, k=None, v=None, out=None, off=None, ws=None, wsb=0) == OK
    assert fwd(lib, Hq=0, q=None, k=None, v=None, out=None, off=None, ws=None, wsb=0) == OK
    assert fwd(lib, D=0, q=None, k=None, v=None, out=None, off=None, ws=None, wsb=0) == OK
    assert paged(lib, B=0, q=None, ws=None, wsb=0) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(Hk=3), INVAL),                      # Hq not a multiple of Hk
    (dict(Hk=0), INVAL),
    (dict(B=-1), INVAL),
    (dict(B=2049), INVAL),                    # the page's B range; work-list entries pack b in 16 bits
    (dict(B=40000), INVAL),
    (dict(g=-1), INVAL),
    (dict(S=0), INVAL),
    (dict(S=20481), INVAL),
    (dict(mask=1), UNSUP),                    # upper triangular: unsupported by the page itself
    (dict(mask=3), INVAL),                    # user mask code without the mask tensor
    (dict(umask=FAKE), INVAL),                # mask tensor without the user mask code
    (dict(mask=3, umask=FAKE, nt=FAKE), INVAL),  # built-in mask inputs with the user mask
    (dict(mask=3, umask=FAKE + 4), INVAL),    # not 16-byte aligned
    (dict(mask=3, umask=FAKE, mask_h=2), INVAL),  # mask heads neither 1 nor num_heads_q
    (dict(mask=3, umask=FAKE, D=64, dt=F32), UNSUP),  # the user mask is built for f16/bf16
    (dict(rab=FAKE, rab_h=3), INVAL),         # rab heads neither 1 nor num_heads_q
    (dict(offk=FAKE + 2), INVAL),
    (dict(offk=FAKE, wsb=1 << 20), WS),       # key offsets need the key-split partial sums
    (dict(mask=7), INVAL),
    (dict(D=48), UNSUP),
    (dict(D=256, dt=F32), UNSUP),
    (dict(dt=5), UNSUP),
    (dict(q=None), INVAL),
    (dict(off=None), INVAL),
    (dict(q=FAKE + 8), INVAL),                # not 16-byte aligned
    (dict(rab=FAKE + 2), INVAL),
    (dict(off=FAKE + 2), INVAL),
    (dict(mask=2, nt=FAKE), INVAL),           # targets with the bidirectional mask
    (dict(mask=2, nc=FAKE), INVAL),
    (dict(ws=None), WS),
    (dict(wsb=16), WS),
    (dict(dt=FP8, D=64), UNSUP),              # the FP8 cast is built for head_dim 128
    (dict(dt=FP8, rab=FAKE), UNSUP),          # ... without rab
    (dict(dt=FP8, mask=3, umask=FAKE), UNSUP),  # ... or the user mask
    (dict(dt=FP8, offk=FAKE), UNSUP),         # ... or separate key offsets
    (dict(dt=4), UNSUP),
    (dict(win=-1), INVAL),                    # negative local window
    (dict(win=-1, B=0), INVAL),               # ... even for an empty input
    (dict(win=8, mask=2), INVAL),             # the local window needs the causal mask
    (dict(win=8, mask=3, umask=FAKE), INVAL),
])
def test_fwd_rejects(lib, kw, code):
    assert fwd(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(ps=48), UNSUP),
    (dict(ps=512), UNSUP),
    (dict(ps=-1), INVAL),
    (dict(cache=None), INVAL),
    (dict(pids=None), INVAL),
    (dict(lpl=FAKE + 1), INVAL),
    (dict(Hk=3), INVAL),
    (dict(mask=3), UNSUP),
    (dict(wsb=8), WS),
    (dict(B=2049), INVAL),
    (dict(dt=FP8), UNSUP),                    # the FP8 cast is built for jagged calls
    (dict(win=-3), INVAL),
    (dict(win=16, mask=2), INVAL),
])
def test_paged_rejects(lib, kw, code):
    assert paged(lib, **kw) == code


def test_workspace_sizes(lib):
    small = hj.hstu_fwd_workspace_size(8, 1024, 4, 4, 128, __import__("torch").bfloat16)
    big = hj.hstu_fwd_workspace_size(8, 4096, 4, 4, 128, __import__("torch").bfloat16)
    assert 0 < small < big
    assert lib.hstu_fwd_workspace_size(2, 128, 4, 3, 128, BF16, 0) == 0
    assert lib.hstu_fwd_workspace_size(-1, 128, 4, 4, 128, BF16, 0) == 0
    # different Q/K lengths reserve the partial sums of key-split items
    assert hj.hstu_fwd_workspace_size(32, 2048, 4, 4, 128, __import__("torch").bfloat16, is_delta_qk=True) > \
        hj.hstu_fwd_workspace_size(32, 2048, 4, 4, 128, __import__("torch").bfloat16)
    assert lib.hstu_fwd_paged_workspace_size(64, 64, 4160, 4, 4, 128, BF16) > 0
    # batches past the page's B range have no workspace size
    assert lib.hstu_fwd_workspace_size(2048, 128, 4, 4, 128, BF16, 0) > 0
    assert lib.hstu_fwd_workspace_size(2049, 128, 4, 4, 128, BF16, 0) == 0
    assert lib.hstu_fwd_paged_workspace_size(2049, 64, 4160, 4, 4, 128, BF16) == 0


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        hj.load_library(str(tmp_path / "missing.so"))


def test_binding_requires_max_seq_len():
    # The binding never reads device arrays back, so the page's maximum
    # sequence length must be given (checked before anything is launched).
    import torch
    q = torch.zeros(4, 2, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="max_seq_len"):
        hj.prepare_fwd(q, q, q, [0, 4])
    kv = torch.zeros(1, 2, 32, 2, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="max_seq_len"):
        hj.prepare_fwd_paged(q, q, q, kv, [0, 4], [0, 1], [0], [1])
