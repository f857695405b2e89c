"""Float64 CPU oracle for the fused HSTU attention forward.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package. The
HIP library never links, loads or calls it, and it imports nothing from the
HIP package. Its arithmetic lives in ``hstu_oracle.c`` (plain C loops over
the definition, float64, OpenMP over output rows); this module only marshals
numpy arrays into that library.

Source of the definition: the RecOps Running Case Documentation page on the
HSTU_V1 forward operator (hstu_dense_forward) -- feature table, operator
introduction and inputs/outputs table. The readings taken where that page is
silent are listed in the header of ``hstu_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hstu_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libhstu_oracle.so")

MASK_CAUSAL = 0
MASK_NONE = 2
MASK_CUSTOM = 3

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, float64, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I32 = ctypes.c_int32
    D = ctypes.c_double
    lib.hstu_oracle_silu.argtypes = [D]
    lib.hstu_oracle_silu.restype = D
    lib.hstu_oracle_vis.argtypes = [I32, I64, I64, I64, I64, I64, I64, I64]
    lib.hstu_oracle_vis.restype = ctypes.c_int
    lib.hstu_oracle_mask.argtypes = [I32, I64, I64, I64, I64, I64, P]
    lib.hstu_oracle_mask.restype = None
    lib.hstu_oracle_e4m3.argtypes = [D]
    lib.hstu_oracle_e4m3.restype = D
    lib.hstu_oracle_fwd.argtypes = [P, P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I64, I64, I32, I64, I64, D,
                                    D, I32, P, I64]
    lib.hstu_oracle_fwd.restype = ctypes.c_int
    lib.hstu_oracle_fwd_paged.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I32, I64, I64, D,
                                          D, P, I64]
    lib.hstu_oracle_fwd_paged.restype = ctypes.c_int
    lib.hstu_oracle_num_threads.argtypes = []
    lib.hstu_oracle_num_threads.restype = ctypes.c_int
    lib.hstu_oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.hstu_oracle_set_num_threads.restype = None
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i64(x) -> Optional[np.ndarray]:
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().hstu_oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads the oracle's OpenMP loops use from now on (timing only)."""
    _load().hstu_oracle_set_num_threads(int(n))


def silu(x: float) -> float:
    return float(_load().hstu_oracle_silu(float(x)))


def e4m3(x: float) -> float:
    """x cast to OCP E4M3 (FN): nearest, ties to even, saturating at +-448."""
    return float(_load().hstu_oracle_e4m3(float(x)))


def vis(mask_type: int, L: int, nc: int, nt: int, g: int, i: int, j: int, w: int = 0) -> bool:
    return bool(_load().hstu_oracle_vis(mask_type, L, nc, nt, g, w, i, j))


def mask_matrix(mask_type: int, L: int, nc: int = 0, nt: int = 0, g: int = 0, w: int = 0) -> np.ndarray:
    """The L x L visibility matrix of one sequence (bool); w: local window."""
    out = np.zeros((L, L), dtype=np.uint8)
    _load().hstu_oracle_mask(mask_type, L, nc, nt, g, w, _ptr(out))
    return out.astype(bool)


def hstu_fwd(q, k, v, seq_offsets, *, rab=None, mask=None, seq_offsets_k=None, num_context=None,
             num_targets=None, max_seq_len: int, mask_type: int = MASK_CAUSAL, target_group_size: int = 0,
             alpha: float = 1.0, out_scale: Optional[float] = None, rows: Optional[Sequence] = None,
             p_fp8: bool = False, local_window: int = 0) -> np.ndarray:
    """Jagged forward in float64.

    q [Tq, Hq, D], k/v [Tk, Hk, D]; seq_offsets for q and seq_offsets_k for
    k/v (None: the same). rab [B, Hq or 1, max_seq_len, max_seq_len] or None;
    mask (mask_type 3 only) [B, Hq or 1, max_seq_len, max_seq_len].
    p_fp8: the FP8 cast, P cast to E4M3 before the product with V (the
    inputs are then E4M3 values, passed widened). local_window: the local
    mask's window W (causal mask only; 0 = none).
    Returns out [Tq, Hq, D], or [len(rows), D] when ``rows`` lists (token, head) pairs.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    off = _i64(seq_offsets)
    offk = _i64(seq_offsets_k)
    B = off.shape[0] - 1
    T, Hq, D = q.shape
    Hk = k.shape[1]
    if out_scale is None:
        out_scale = 1.0 / max_seq_len
    rab_a = None if rab is None else _f64(rab)
    if rab_a is not None:
        assert rab_a.shape[0] == B and rab_a.shape[1] in (1, Hq) and rab_a.shape[2:] == (max_seq_len, max_seq_len), \
            rab_a.shape
    mask_a = None if mask is None else _f64(mask)
    if mask_a is not None:
        assert mask_a.shape[0] == B and mask_a.shape[1] in (1, Hq) and mask_a.shape[2:] == (max_seq_len, max_seq_len), \
            mask_a.shape
    nc, nt = _i64(num_context), _i64(num_targets)
    rows_a = None if rows is None else _i64(rows).reshape(-1, 2)
    out = np.zeros((T, Hq, D) if rows_a is None else (rows_a.shape[0], D), dtype=np.float64)
    rc = _load().hstu_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(rab_a), _ptr(mask_a), _ptr(out), _ptr(off),
                                 _ptr(offk), _ptr(nc), _ptr(nt), B, max_seq_len, Hq, Hk, D,
                                 1 if rab_a is None else rab_a.shape[1], 1 if mask_a is None else mask_a.shape[1],
                                 mask_type, target_group_size, int(local_window), float(alpha), float(out_scale),
                                 int(bool(p_fp8)),
                                 _ptr(rows_a), 0 if rows_a is None else rows_a.shape[0])
    if rc != 0:
        raise ValueError("oracle: invalid arguments")
    return out


def hstu_fwd_paged(q, k_new, v_new, kv_cache, seq_offsets_q, page_offsets, page_ids, last_page_len, *,
                   num_context=None, num_targets=None, mask_type: int = MASK_CAUSAL, target_group_size: int = 0,
                   alpha: float = 1.0, out_scale: float, rows: Optional[Sequence] = None,
                   local_window: int = 0) -> np.ndarray:
    """Paged forward in float64. kv_cache [num_pages, 2, page_size, Hk, D]."""
    q, kn, vn, kv = _f64(q), _f64(k_new), _f64(v_new), _f64(kv_cache)
    offq, poff, pids, lpl = _i64(seq_offsets_q), _i64(page_offsets), _i64(page_ids), _i64(last_page_len)
    B = offq.shape[0] - 1
    Tq, Hq, D = q.shape
    Hk = kn.shape[1]
    page_size = kv.shape[2]
    nc, nt = _i64(num_context), _i64(num_targets)
    rows_a = None if rows is None else _i64(rows).reshape(-1, 2)
    out = np.zeros((Tq, Hq, D) if rows_a is None else (rows_a.shape[0], D), dtype=np.float64)
    rc = _load().hstu_oracle_fwd_paged(_ptr(q), _ptr(kn), _ptr(vn), _ptr(kv), _ptr(out), _ptr(offq), _ptr(poff),
                                       _ptr(pids), _ptr(lpl), _ptr(nc), _ptr(nt), B, page_size, Hq, Hk, D, mask_type,
                                       target_group_size, int(local_window), float(alpha), float(out_scale), _ptr(rows_a),
                                       0 if rows_a is None else rows_a.shape[0])
    if rc != 0:
        raise ValueError("oracle: invalid arguments")
    return out
