"""MI355X (gfx950) fused HSTU attention forward.

Thin ctypes binding over the C ABI in ``include/hstu.h`` (library
``libhstu.so`` built in-tree from ``csrc/``). This module only marshals
arguments: it checks tensor dtypes/devices/contiguity, converts integer side
inputs to int32, allocates ``out`` and the workspace with torch when the
caller does not pass them, and hands raw device pointers plus the current
HIP stream to the library. Every step of the computation runs in the HIP
kernels; there is no fallback. If the library is missing, every call raises.

The operation is the HSTU_V1 forward operator of the RecOps Running Case
Documentation page (feature table, inputs/outputs table): per query head,
out = out_scale * (mask .* silu(alpha * (q k^T + rab))) v over jagged
sequences, MHA or GQA, bidirectional or causal (context / history / target)
masks, plus a paged-KV variant. ``out_scale`` defaults to 1/max_seq_len (the
page's silu_scale default) and ``alpha`` to 1.0 (the page gives none).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhstu.so")

MASK_CAUSAL = 0
MASK_NONE = 2
MASK_CUSTOM = 3

HSTU_OK = 0
HSTU_ERR_INVALID_ARG = 1
HSTU_ERR_UNSUPPORTED = 2
HSTU_ERR_WORKSPACE = 3
HSTU_ERR_HIP = 4

DTYPE_CODES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.float8_e4m3fn: 3}
# The FP8 cast (q, k, v in E4M3) writes bf16; rab and the user mask would be
# bf16 too (the library rejects them with FP8 inputs).
OUT_DTYPES = {torch.float8_e4m3fn: torch.bfloat16}

# Every symbol include/hstu.h declares.
EXPORTED = ("hstu_fwd_workspace_size", "hstu_fwd", "hstu_fwd_plan", "hstu_fwd_run", "hstu_fwd_paged_workspace_size",
            "hstu_fwd_paged", "hstu_fwd_paged_plan", "hstu_fwd_paged_run", "hstu_fwd_noalloc", "hstu_status_string")


class HstuError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


_lib = None


def load_library(path: Optional[str] = None):
    """Load libhstu.so (torch is imported first so the library binds to the
    HIP runtime torch already loaded). Raises if the library is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"HSTU HIP library not built: {p} is missing "
                           "(run `python -m hstu_jagged_attention_amd.build`)")
    lib = ctypes.CDLL(p)
    P, I32, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    E = ctypes.c_int
    lib.hstu_fwd_workspace_size.argtypes = [I32, I32, I32, I32, I32, E, I32]
    lib.hstu_fwd_workspace_size.restype = SZ
    lib.hstu_fwd_paged_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32, E]
    lib.hstu_fwd_paged_workspace_size.restype = SZ
    jag = [P, P, P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, E, I32, I32, F, F, E, P, SZ, P]
    pag = [P, P, P, P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, E, I32, I32, F, F, E, P, SZ, P]
    for name in ("hstu_fwd", "hstu_fwd_run"):
        getattr(lib, name).argtypes = jag
        getattr(lib, name).restype = E
    for name in ("hstu_fwd_paged", "hstu_fwd_paged_run"):
        getattr(lib, name).argtypes = pag
        getattr(lib, name).restype = E
    lib.hstu_fwd_noalloc.argtypes = jag[:23] + [P]
    lib.hstu_fwd_noalloc.restype = E
    lib.hstu_fwd_plan.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, E, I32, I32, E, P, SZ, P]
    lib.hstu_fwd_plan.restype = E
    lib.hstu_fwd_paged_plan.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, I32, E, I32, I32, E, P, SZ, P]
    lib.hstu_fwd_paged_plan.restype = E
    lib.hstu_status_string.argtypes = [E]
    lib.hstu_status_string.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().hstu_status_string(int(status)).decode()


def hstu_fwd_workspace_size(batch: int, max_seq_len: int, num_heads_q: int, num_heads_kv: int, head_dim: int,
                            dtype: torch.dtype, is_delta_qk: bool = False) -> int:
    return int(load_library().hstu_fwd_workspace_size(batch, max_seq_len, num_heads_q, num_heads_kv, head_dim,
                                                       DTYPE_CODES[dtype], int(bool(is_delta_qk))))


def hstu_fwd_paged_workspace_size(batch: int, page_size: int, max_seq_len: int, num_heads_q: int, num_heads_kv: int,
                                  head_dim: int, dtype: torch.dtype) -> int:
    return int(load_library().hstu_fwd_paged_workspace_size(batch, page_size, max_seq_len, num_heads_q, num_heads_kv,
                                                             head_dim, DTYPE_CODES[dtype]))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev_tensor(t: torch.Tensor, name: str, dtype: torch.dtype, device) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _int32(t, name: str, device) -> Optional[torch.Tensor]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        t = torch.as_tensor(t)
    if t.dtype not in (torch.int32, torch.int64):
        raise TypeError(f"{name} must be int32 or int64")
    return t.to(device=device, dtype=torch.int32).contiguous()


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class Prepared:
    """One forward call with its arguments marshalled once.

    ``plan()``, ``run()`` and ``fwd()`` call hstu_*_plan, hstu_*_run and the
    combined entry point with the stored pointers on the stream that was
    current at preparation time; the tensors stay referenced by this object.
    """

    def __init__(self, name: str, lib, fwd_args, plan_args, out: torch.Tensor, workspace: torch.Tensor, keep):
        self.name = name
        self._lib = lib
        self._fwd = getattr(lib, name)
        self._run = getattr(lib, name + "_run")
        self._plan = getattr(lib, name + "_plan")
        self._fwd_args = fwd_args
        self._plan_args = plan_args
        self.out = out
        self.workspace = workspace
        self._keep = keep

    def _check(self, st: int, what: str):
        if st != HSTU_OK:
            raise HstuError(st, what)

    def fwd(self) -> torch.Tensor:
        self._check(self._fwd(*self._fwd_args), self.name)
        return self.out

    def plan(self) -> None:
        self._check(self._plan(*self._plan_args), self.name + "_plan")

    def run(self) -> torch.Tensor:
        self._check(self._run(*self._fwd_args), self.name + "_run")
        return self.out

    __call__ = fwd


def prepare_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_offsets, *, rab: Optional[torch.Tensor] = None,
                mask: Optional[torch.Tensor] = None, seq_offsets_k=None, num_context=None, num_targets=None,
                max_seq_len: Optional[int] = None, mask_type: Optional[int] = None, target_group_size: int = 0,
                local_window: int = 0, alpha: float = 1.0, out_scale: Optional[float] = None,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> Prepared:
    """Marshal a jagged forward: q [Tq, Hq, D], k/v [Tk, Hk, D] on the GPU.

    seq_offsets addresses q; seq_offsets_k (optional) addresses k/v when the
    query and key lengths differ (queries are the last positions of each
    sequence). rab and mask are [B, Hq or 1, max_seq_len, max_seq_len].
    mask_type defaults to MASK_CUSTOM when a mask is given, else MASK_CAUSAL.
    local_window (causal mask only) is the local mask's window W: key j is
    visible to query i only when i - j < W as well (0: no window).
    max_seq_len (the page's maximum sequence length: the row stride of rab
    and mask, and the bound on every key sequence) is required: the binding
    never reads device arrays back."""
    lib = load_library()
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [tokens, heads, head_dim]")
    device, dtype = q.device, q.dtype
    if dtype not in DTYPE_CODES:
        raise TypeError(f"unsupported dtype {dtype}")
    _dev_tensor(q, "q", dtype, device)
    _dev_tensor(k, "k", dtype, device)
    _dev_tensor(v, "v", dtype, device)
    off = _int32(seq_offsets, "seq_offsets", device)
    offk = _int32(seq_offsets_k, "seq_offsets_k", device)
    B = int(off.shape[0]) - 1
    if offk is not None and int(offk.shape[0]) != B + 1:
        raise ValueError("seq_offsets_k must have batch + 1 entries")
    if mask_type is None:
        mask_type = MASK_CUSTOM if mask is not None else MASK_CAUSAL
    if max_seq_len is None:
        raise ValueError("max_seq_len is required")
    max_seq_len = int(max_seq_len)
    if out_scale is None:
        out_scale = 1.0 / max_seq_len
    heads = {}
    side = OUT_DTYPES.get(dtype, dtype)
    for name, t in (("rab", rab), ("mask", mask)):
        heads[name] = 1
        if t is not None:
            _dev_tensor(t, name, side, device)
            if t.dim() != 4 or t.shape[0] != B or t.shape[1] not in (1, q.shape[1]) or \
                    tuple(t.shape[2:]) != (max_seq_len, max_seq_len):
                raise ValueError(f"{name} must be [{B}, {q.shape[1]} or 1, {max_seq_len}, {max_seq_len}], "
                                 f"got {tuple(t.shape)}")
            heads[name] = int(t.shape[1])
    nc = _int32(num_context, "num_context", device)
    nt = _int32(num_targets, "num_targets", device)
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=side, device=device)
    else:
        _dev_tensor(out, "out", side, device)
    Hq, Hk, D = int(q.shape[1]), int(k.shape[1]), int(q.shape[2])
    code = DTYPE_CODES[dtype]
    need = int(lib.hstu_fwd_workspace_size(B, max_seq_len, Hq, Hk, D, code, 0 if offk is None else 1))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    wsb = workspace.numel() * workspace.element_size()
    stream = _stream(device)
    fwd_args = (_ptr(q), _ptr(k), _ptr(v), _ptr(rab), _ptr(mask), _ptr(out), _ptr(off), _ptr(offk), _ptr(nc),
                _ptr(nt), B, max_seq_len, Hq, Hk, D, heads["rab"], heads["mask"], int(mask_type),
                int(target_group_size), int(local_window), float(alpha), float(out_scale), code, _ptr(workspace),
                wsb, stream)
    plan_args = (_ptr(off), _ptr(offk), _ptr(nc), _ptr(nt), B, max_seq_len, Hq, Hk, D, int(mask_type),
                 int(target_group_size), int(local_window), code, _ptr(workspace), wsb, stream)
    return Prepared("hstu_fwd", lib, fwd_args, plan_args, out, workspace, (q, k, v, rab, mask, off, offk, nc, nt))


def hstu_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_offsets, **kw) -> torch.Tensor:
    """Jagged HSTU forward; returns out [T, Hq, D]. Keywords as prepare_fwd."""
    return prepare_fwd(q, k, v, seq_offsets, **kw).fwd()


def hstu_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_offsets, *, out: torch.Tensor,
                     **kw) -> torch.Tensor:
    """hstu_fwd through the allocation-free entry point: the library uses its
    static device scratch instead of a workspace, and the caller passes
    ``out`` (integer side inputs must already be int32 device tensors for
    the call itself to allocate nothing). Keywords as prepare_fwd."""
    prep = prepare_fwd(q, k, v, seq_offsets, out=out, workspace=torch.empty(0, dtype=torch.uint8, device=q.device),
                       **kw)
    st = prep._lib.hstu_fwd_noalloc(*prep._fwd_args[:23], prep._fwd_args[-1])
    if st != HSTU_OK:
        raise HstuError(st, "hstu_fwd_noalloc")
    return out


def prepare_fwd_paged(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, kv_cache: torch.Tensor,
                      seq_offsets_q, page_offsets, page_ids, last_page_len, *, num_context=None, num_targets=None,
                      max_seq_len: Optional[int] = None, mask_type: int = MASK_CAUSAL, target_group_size: int = 0,
                      local_window: int = 0, alpha: float = 1.0, out_scale: Optional[float] = None,
                      out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> Prepared:
    """Marshal a paged-KV forward. kv_cache [num_pages, 2, page_size, Hk, D].

    max_seq_len (the bound on history + new tokens of every request) is
    required: the binding never reads device arrays back."""
    lib = load_library()
    device, dtype = q.device, q.dtype
    if dtype not in DTYPE_CODES:
        raise TypeError(f"unsupported dtype {dtype}")
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("kv_cache", kv_cache)):
        _dev_tensor(t, name, dtype, device)
    if kv_cache.dim() != 5 or kv_cache.shape[1] != 2:
        raise ValueError("kv_cache must be [num_pages, 2, page_size, heads, head_dim]")
    offq = _int32(seq_offsets_q, "seq_offsets_q", device)
    poff = _int32(page_offsets, "page_offsets", device)
    pids = _int32(page_ids, "page_ids", device)
    lpl = _int32(last_page_len, "last_page_len", device)
    B = int(offq.shape[0]) - 1
    page_size = int(kv_cache.shape[2])
    if max_seq_len is None:
        raise ValueError("max_seq_len is required")
    max_seq_len = int(max_seq_len)
    if out_scale is None:
        out_scale = 1.0 / max_seq_len
    nc = _int32(num_context, "num_context", device)
    nt = _int32(num_targets, "num_targets", device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev_tensor(out, "out", dtype, device)
    Hq, Hk, D = int(q.shape[1]), int(k_new.shape[1]), int(q.shape[2])
    code = DTYPE_CODES[dtype]
    need = int(lib.hstu_fwd_paged_workspace_size(B, page_size, max_seq_len, Hq, Hk, D, code))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    wsb = workspace.numel() * workspace.element_size()
    stream = _stream(device)
    fwd_args = (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(offq), _ptr(kv_cache), _ptr(poff), _ptr(pids),
                _ptr(lpl), _ptr(nc), _ptr(nt), B, page_size, max_seq_len, Hq, Hk, D, int(mask_type),
                int(target_group_size), int(local_window), float(alpha), float(out_scale), code, _ptr(workspace),
                wsb, stream)
    plan_args = (_ptr(offq), _ptr(poff), _ptr(lpl), _ptr(nc), _ptr(nt), B, page_size, max_seq_len, Hq, Hk, D,
                 int(mask_type), int(target_group_size), int(local_window), code, _ptr(workspace), wsb, stream)
    return Prepared("hstu_fwd_paged", lib, fwd_args, plan_args, out, workspace,
                    (q, k_new, v_new, kv_cache, offq, poff, pids, lpl, nc, nt))


def hstu_fwd_paged(q, k_new, v_new, kv_cache, seq_offsets_q, page_offsets, page_ids, last_page_len,
                   **kw) -> torch.Tensor:
    """Paged-KV HSTU forward; returns out [Tq, Hq, D]. Keywords as prepare_fwd_paged."""
    return prepare_fwd_paged(q, k_new, v_new, kv_cache, seq_offsets_q, page_offsets, page_ids, last_page_len,
                             **kw).fwd()
