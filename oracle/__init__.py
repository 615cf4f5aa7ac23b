"""fp64 CPU oracle for masked attention (forward and gradients), the KV-split merge and
tile classification.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` are the only callers.  The product path never imports this
package.  The arithmetic lives in ``oracle.c`` (plain C, fp64); this module only
compiles it and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


class _Slice(ctypes.Structure):
    _fields_ = [("q0", ctypes.c_int32), ("q1", ctypes.c_int32), ("k0", ctypes.c_int32),
                ("k1", ctypes.c_int32), ("type", ctypes.c_int32)]


# -O3 at the x86-64-v3 level (AVX2, FMA): the library is compiled on one host and may be
# run on another x86 host (-march=native would bind it to the first one's CPU);
# -ffp-contract=off keeps every multiply and add rounded separately, as the C source
# reads.
CFLAGS = ["-O3", "-march=x86-64-v3", "-ffp-contract=off", "-std=c99", "-fPIC", "-shared", "-pthread"]
MAX_THREADS = 16       # worker threads by default: at most the host's cores, at most 16


def default_threads() -> int:
    return max(1, min(os.cpu_count() or 1, MAX_THREADS))


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (host only)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc"] + CFLAGS + [_SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        lib.oracle_pair_count.restype = ctypes.c_int64
        lib.oracle_pair_count.argtypes = [P, ctypes.c_int32, ctypes.c_int32]
        lib.oracle_row_key_set.restype = ctypes.c_int32
        lib.oracle_row_key_set.argtypes = [P, ctypes.c_int32, ctypes.c_int64, P, P]
        lib.oracle_tile_csr.restype = ctypes.c_int32
        lib.oracle_tile_csr.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, P, P, P, ctypes.c_int64,
                                        ctypes.POINTER(ctypes.c_int64)]
        lib.oracle_attn_fwd.restype = ctypes.c_int32
        lib.oracle_attn_fwd.argtypes = [P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int32,
                                        ctypes.c_double, P, ctypes.c_int64, P, P, ctypes.c_int32]
        I32, D = ctypes.c_int32, ctypes.c_double
        lib.oracle_attn_fwd_f64.restype = I32
        lib.oracle_attn_fwd_f64.argtypes = [P, P, P, I32, I32, I32, I32, I32, P, I32, D, P, P, I32]
        lib.oracle_attn_bwd.restype = I32
        lib.oracle_attn_bwd.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, P, I32, D, P, P, P, I32]
        lib.oracle_attn_bwd_f64.restype = I32
        lib.oracle_attn_bwd_f64.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, P, I32, D, P, P, P]
        lib.oracle_attn_bwd_sampled.restype = I32
        lib.oracle_attn_bwd_sampled.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, P, I32, D, P,
                                                ctypes.c_int64, P, P, ctypes.c_int64, P, P, I32]
        lib.oracle_merge.restype = None
        lib.oracle_merge.argtypes = [P, P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, P, P]
        _lib = lib
    return _lib


def _slices(slices):
    arr = (_Slice * max(1, len(slices)))()
    for t, s in enumerate(slices):
        arr[t] = _Slice(*[int(x) for x in s])
    return arr


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def pair_count(slices, sq: int) -> int:
    """Number of admitted (query, key) pairs of one head."""
    return int(_load().oracle_pair_count(_slices(slices), len(slices), sq))


def row_key_set(slices, i: int):
    """U(i) as a list of disjoint sorted half-open intervals."""
    n = max(1, len(slices))
    lo = np.zeros(n, np.int64)
    hi = np.zeros(n, np.int64)
    m = _load().oracle_row_key_set(_slices(slices), len(slices), i, _ptr(lo), _ptr(hi))
    return [(int(lo[t]), int(hi[t])) for t in range(m)]


def tile_csr(slices, sq: int, sk: int, bq: int, bk: int):
    """(row_ptr int32, col int32, tag uint8) of the non-empty (bq x bk) tiles."""
    n_qt = (sq + bq - 1) // bq
    n_kt = (sk + bk - 1) // bk
    cap = n_qt * n_kt
    row_ptr = np.zeros(n_qt + 1, np.int32)
    col = np.zeros(max(1, cap), np.int32)
    tag = np.zeros(max(1, cap), np.uint8)
    nnz = ctypes.c_int64(0)
    rc = _load().oracle_tile_csr(_slices(slices), len(slices), sq, sk, bq, bk, _ptr(row_ptr),
                                 _ptr(col), _ptr(tag), cap, ctypes.byref(nnz))
    if rc != 0:
        raise RuntimeError("oracle_tile_csr: capacity")
    return row_ptr, col[:nnz.value].copy(), tag[:nnz.value].copy()


def attn_fwd(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, slices, scale: float,
             rows=None, n_threads: int | None = None):
    """fp64 attention.  q_bits [sq, hq, d], k_bits/v_bits [sk, hkv, d] as uint16 bf16 bits.

    rows=None -> (O [sq, hq, d], LSE [hq, sq]); rows=[(h, i), ...] -> (O [n, d], LSE [n]).
    """
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    k_bits = np.ascontiguousarray(k_bits, dtype=np.uint16)
    v_bits = np.ascontiguousarray(v_bits, dtype=np.uint16)
    sq, hq, d = q_bits.shape
    sk, hkv, d2 = k_bits.shape
    assert d2 == d and v_bits.shape == k_bits.shape
    if n_threads is None:
        n_threads = default_threads()
    if rows is None:
        o = np.zeros((sq, hq, d), np.float64)
        lse = np.zeros((hq, sq), np.float64)
        rows_arr, n_rows, rows_ptr = None, 0, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
        n_rows = rows_arr.shape[0]
        rows_ptr = _ptr(rows_arr)
        o = np.zeros((n_rows, d), np.float64)
        lse = np.zeros(n_rows, np.float64)
    rc = _load().oracle_attn_fwd(_ptr(q_bits), _ptr(k_bits), _ptr(v_bits), sq, sk, hq, hkv, d,
                                 _slices(slices), len(slices), float(scale), rows_ptr, n_rows,
                                 _ptr(o), _ptr(lse), int(n_threads))
    if rc != 0:
        raise ValueError("oracle_attn_fwd: bad head counts")
    return o, lse


def attn_fwd_f64(q: np.ndarray, k: np.ndarray, v: np.ndarray, slices, scale: float, n_threads: int = 1):
    """The same fp64 forward on fp64 inputs q [sq, hq, d], k/v [sk, hkv, d] -> (O, LSE [hq, sq])."""
    q, k, v = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v))
    sq, hq, d = q.shape
    sk, hkv, _ = k.shape
    o = np.zeros((sq, hq, d), np.float64)
    lse = np.zeros((hq, sq), np.float64)
    rc = _load().oracle_attn_fwd_f64(_ptr(q), _ptr(k), _ptr(v), sq, sk, hq, hkv, d, _slices(slices),
                                     len(slices), float(scale), _ptr(o), _ptr(lse), int(n_threads))
    if rc != 0:
        raise ValueError("oracle_attn_fwd_f64: bad head counts")
    return o, lse


def attn_bwd(q_bits, k_bits, v_bits, do_bits, slices, scale: float, n_threads: int | None = None):
    """fp64 gradients (dQ [sq, hq, d], dK [sk, hkv, d], dV [sk, hkv, d]) of the forward for
    an upstream gradient dO [sq, hq, d]; all inputs bf16 bit patterns (uint16)."""
    q_bits, k_bits, v_bits, do_bits = (np.ascontiguousarray(x, dtype=np.uint16)
                                       for x in (q_bits, k_bits, v_bits, do_bits))
    sq, hq, d = q_bits.shape
    sk, hkv, _ = k_bits.shape
    assert do_bits.shape == q_bits.shape and v_bits.shape == k_bits.shape
    dq = np.zeros((sq, hq, d), np.float64)
    dk = np.zeros((sk, hkv, d), np.float64)
    dv = np.zeros((sk, hkv, d), np.float64)
    if n_threads is None:
        n_threads = default_threads()
    rc = _load().oracle_attn_bwd(_ptr(q_bits), _ptr(k_bits), _ptr(v_bits), _ptr(do_bits), sq, sk, hq, hkv,
                                 d, _slices(slices), len(slices), float(scale), _ptr(dq), _ptr(dk),
                                 _ptr(dv), int(n_threads))
    if rc != 0:
        raise ValueError("oracle_attn_bwd: bad head counts")
    return dq, dk, dv


def attn_bwd_sampled(q_bits, k_bits, v_bits, do_bits, slices, scale: float, rows=(), keys=(),
                     n_threads: int | None = None):
    """fp64 gradients at sampled outputs: dQ at (h, i) pairs `rows` -> [n_rows, d];
    dK, dV at (g, j) pairs `keys` (g a key/value head) -> [n_keys, d] each."""
    q_bits, k_bits, v_bits, do_bits = (np.ascontiguousarray(x, dtype=np.uint16)
                                       for x in (q_bits, k_bits, v_bits, do_bits))
    sq, hq, d = q_bits.shape
    sk, hkv, _ = k_bits.shape
    rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
    keys_arr = np.ascontiguousarray(np.asarray(keys, dtype=np.int64).reshape(-1, 2))
    dq = np.zeros((rows_arr.shape[0], d), np.float64)
    dk = np.zeros((keys_arr.shape[0], d), np.float64)
    dv = np.zeros((keys_arr.shape[0], d), np.float64)
    if n_threads is None:
        n_threads = default_threads()
    rc = _load().oracle_attn_bwd_sampled(
        _ptr(q_bits), _ptr(k_bits), _ptr(v_bits), _ptr(do_bits), sq, sk, hq, hkv, d, _slices(slices),
        len(slices), float(scale), _ptr(rows_arr), rows_arr.shape[0], _ptr(dq), _ptr(keys_arr),
        keys_arr.shape[0], _ptr(dk), _ptr(dv), int(n_threads))
    if rc != 0:
        raise ValueError("oracle_attn_bwd_sampled: bad head counts")
    return dq, dk, dv


def attn_bwd_f64(q, k, v, do, slices, scale: float):
    """attn_bwd on fp64 inputs (for finite-difference checks)."""
    q, k, v, do = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, do))
    sq, hq, d = q.shape
    sk, hkv, _ = k.shape
    dq = np.zeros((sq, hq, d), np.float64)
    dk = np.zeros((sk, hkv, d), np.float64)
    dv = np.zeros((sk, hkv, d), np.float64)
    rc = _load().oracle_attn_bwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(do), sq, sk, hq, hkv, d,
                                     _slices(slices), len(slices), float(scale), _ptr(dq), _ptr(dk),
                                     _ptr(dv))
    if rc != 0:
        raise ValueError("oracle_attn_bwd_f64: bad head counts")
    return dq, dk, dv


def merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge n partials: o_parts [n, R, d] fp64, lse_parts [n, R] fp64 -> (O [R, d], LSE [R])."""
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    n, r, d = o_parts.shape
    assert lse_parts.shape == (n, r)
    o = np.zeros((r, d), np.float64)
    lse = np.zeros(r, np.float64)
    _load().oracle_merge(_ptr(o_parts), _ptr(lse_parts), n, r, d, _ptr(o), _ptr(lse))
    return o, lse
