"""fp64 CPU oracle for ragged, paged, prefix-cached attention.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it.  The GPU library never loads or
calls it and shares no code with it.

The arithmetic lives in ``rpkv_oracle.c`` (plain C, double precision); this module
builds it with gcc on first use and marshals numpy arrays through ctypes.  Every
function's source passage is cited in the C file.  Parity status: every function
here is pinned by CPU tests (``tests/test_oracle_pins.py``); none is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rpkv_oracle.c")
_LIB_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIB_DIR, "librpkv_oracle.so")
_lock = threading.Lock()
_lib = None

BF16, F32 = 0, 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no tuning).  Returns the .so path."""
    os.makedirs(_LIB_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-Wall", "-o", tmp,
                               _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("cu_q", ctypes.c_void_p), ("seqlens", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p), ("pt_stride", ctypes.c_int64),
        ("q", ctypes.c_void_p), ("kpool", ctypes.c_void_p), ("vpool", ctypes.c_void_p),
        ("scale", ctypes.c_double), ("key_lo", ctypes.c_int64), ("key_hi", ctypes.c_int64),
    ]


def lib():
    global _lib
    with _lock:
        if _lib is None:
            # RPKV_ORACLE_LIB lets the mutation test load a deliberately broken copy
            path = os.environ.get("RPKV_ORACLE_LIB") or build(force=False)
            L = ctypes.CDLL(path)
            L.rpkv_oracle_slot.restype = ctypes.c_int64
            L.rpkv_oracle_slot.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                           ctypes.c_int64, ctypes.c_int32]
            L.rpkv_oracle_store_kv.restype = None
            L.rpkv_oracle_store_kv.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64, ctypes.c_int64]
            L.rpkv_oracle_last_indices.restype = None
            L.rpkv_oracle_last_indices.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
            L.rpkv_oracle_build_batch.restype = ctypes.c_int32
            L.rpkv_oracle_build_batch.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                                  ctypes.c_int32] + [ctypes.c_void_p] * 5
            L.rpkv_oracle_attend.restype = ctypes.c_int32
            L.rpkv_oracle_attend.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
            L.rpkv_oracle_lse_merge.restype = None
            L.rpkv_oracle_lse_merge.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_void_p]
            _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def slot(page_table: np.ndarray, req: int, pos: int, page_size: int) -> int:
    pt = _c(page_table, np.int32)
    return int(lib().rpkv_oracle_slot(_p(pt), pt.shape[1], req, pos, page_size))


def store_kv(kpool: np.ndarray, vpool: np.ndarray, k: np.ndarray, v: np.ndarray,
             slot_mapping: np.ndarray) -> None:
    """In place: pool[slot_mapping[t]] = k[t] / v[t], bit for bit (negative slot skipped)."""
    assert kpool.flags.c_contiguous and vpool.flags.c_contiguous
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    sm = _c(slot_mapping, np.int32)
    T = sm.shape[0]
    row_bytes = int(np.prod(kpool.shape[1:])) * kpool.itemsize
    assert k.shape[0] == T and k.dtype == kpool.dtype and v.dtype == vpool.dtype
    if T:
        assert int(sm.max()) < kpool.shape[0]
    lib().rpkv_oracle_store_kv(_p(kpool), _p(vpool), _p(k), _p(v), _p(sm), T, row_bytes)


def last_indices(cu_q: np.ndarray) -> np.ndarray:
    cu = _c(cu_q, np.int32)
    out = np.zeros(cu.shape[0] - 1, dtype=np.int32)
    lib().rpkv_oracle_last_indices(_p(cu), cu.shape[0] - 1, _p(out))
    return out


def build_batch(num_computed, n, need_logits, block_tables=None, block_size: int = 1):
    """Packed metadata: (qsl, seq_lens, positions, slots or None, logits_indices)."""
    nc = _c(num_computed, np.int32)
    nn = _c(n, np.int32)
    nl = _c(need_logits, np.uint8)
    bs = nc.shape[0]
    T = int(nn.sum())
    qsl = np.zeros(bs + 1, np.int32)
    seq = np.zeros(bs, np.int32)
    pos = np.zeros(max(T, 1), np.int32)
    slots = np.zeros(max(T, 1), np.int32)
    lg = np.zeros(max(bs, 1), np.int32)
    bt = None if block_tables is None else _c(block_tables, np.int32)
    m = lib().rpkv_oracle_build_batch(bs, _p(nc), _p(nn), _p(nl), _p(bt),
                                      0 if bt is None else bt.shape[1], block_size,
                                      _p(qsl), _p(seq), _p(pos), _p(slots), _p(lg))
    return qsl, seq, pos[:T], (slots[:T] if bt is not None else None), lg[:m]


def attend(dtype: int, q: np.ndarray, kpool: np.ndarray, vpool: np.ndarray,
           page_table: np.ndarray, cu_q: np.ndarray, seqlens: np.ndarray, Hq: int, Hkv: int,
           D: int, page_size: int, scale: float, key_lo: int = 0, key_hi: int = 1 << 62,
           rows: Optional[np.ndarray] = None, nthreads: int = 1):
    """fp64 attention of the packed batch over the (already stored) pool.

    q: [T, Hq, D], pools [slots, Hkv, D] -- uint16 bf16 bit patterns (dtype=BF16)
    or float32 (dtype=F32).  rows: optional bool [T] selecting tokens to compute.
    Returns (out [T, Hq, D] float64, lse [T, Hq] float64); unselected rows are NaN.
    """
    el = np.uint16 if dtype == BF16 else np.float32
    q = _c(q, el)
    kpool = _c(kpool, el)
    vpool = _c(vpool, el)
    pt = _c(page_table, np.int32)
    cu = _c(cu_q, np.int32)
    sl = _c(seqlens, np.int32)
    T = int(cu[-1])
    out = np.full((max(T, 1), Hq, D), np.nan, dtype=np.float64)
    lse = np.full((max(T, 1), Hq), np.nan, dtype=np.float64)
    sel = None if rows is None else _c(rows, np.uint8)
    pb = _Problem(dtype, Hq, Hkv, D, page_size, cu.shape[0] - 1, _p(cu), _p(sl), _p(pt),
                  pt.shape[1] if pt.ndim == 2 else 0, _p(q), _p(kpool), _p(vpool),
                  float(scale), int(key_lo), int(key_hi))
    rc = lib().rpkv_oracle_attend(ctypes.byref(pb), _p(sel), _p(out), _p(lse), int(nthreads))
    if rc != 0:
        raise ValueError("oracle: input outside the definition (n > L, bad cu_q or Hq % Hkv)")
    return out[:T], lse[:T]


def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    """o_parts [S, rows, D], lse_parts [S, rows] -> (out [rows, D], lse [rows])."""
    o = _c(o_parts, np.float64)
    l = _c(lse_parts, np.float64)
    S, R, D = o.shape
    out = np.zeros((R, D), np.float64)
    lo = np.zeros(R, np.float64)
    lib().rpkv_oracle_lse_merge(S, R, D, _p(o), _p(l), _p(out), _p(lo))
    return out, lo


def store_then_attend(spec, tensors, rows=None, nthreads: int = 1, key_lo: int = 0,
                      key_hi: int = 1 << 62):
    """The whole step on copies of the host tensors: store this step's K/V by
    slot_mapping, then attend.  Returns (out, lse, kpool_after, vpool_after)."""
    kp = tensors.kpool.copy()
    vp = tensors.vpool.copy()
    store_kv(kp, vp, tensors.k, tensors.v, spec.slot_mapping)
    dt = BF16 if spec.dtype == "bf16" else F32
    out, lse = attend(dt, tensors.q, kp, vp, spec.page_table, spec.cu_q, spec.L, spec.Hq,
                      spec.Hkv, spec.D, spec.P, spec.scale, key_lo, key_hi, rows, nthreads)
    return out, lse, kp, vp
