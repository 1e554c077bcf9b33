"""fp64 CPU oracle for the DCP LSE merge and the MLA decode partials behind it.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are its only users.  The product library
(``context_lse_merge_amd``) never imports this package, and this package never
imports the product: the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64, one sequential loop per
output row); this module only builds it with gcc and marshals numpy arrays.
Which page passage each function follows is stated in ``oracle.c``.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (closed forms, invariants, hand-derived fixtures
under ``tests/golden/`` and brute force against scipy's softmax/logsumexp);
none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BASE_E = 0
BASE_2 = 1
LSE_BHC = 0  # [B, H/cp, cp]
LSE_BH1 = 1  # [B, H, 1]
_DTYPE = {"bf16": 0, "f16": 1}  # 16-bit payload types of the attention oracle

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def _configure(lib):
    """Declare the C signatures on a loaded oracle library."""
    i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.oracle_merge_f64.argtypes = [vp, vp, i64, i64, i64, i64, i32, i32, vp, vp, vp, i32]
    lib.oracle_merge_bf16.argtypes = [vp, vp, i64, i64, i64, i64, i32, i32, vp, vp, vp, i32]
    lib.oracle_merge_f16.argtypes = [vp, vp, i64, i64, i64, i64, i32, i32, vp, vp, vp, i32]
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = dbl
    lib.oracle_attention_partials.argtypes = [vp, vp, i64, i64, i64, i64, i64, i64, dbl, i32, i32, vp, i64,
                                              vp, vp, i32]
    lib.oracle_attention_full.argtypes = [vp, vp, i64, i64, i64, i64, i64, dbl, i32, i32, vp, i64, vp, vp, i32]
    lib.oracle_attention_partials_varlen.argtypes = [vp, vp, i64, i64, i64, vp, i32, i64, i64, i64, dbl, i32, i32,
                                                     vp, i64, vp, vp, i32]
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = dbl
    lib.oracle_max_threads.restype = i32
    for f in ("oracle_merge_f64", "oracle_merge_bf16", "oracle_merge_f16", "oracle_attention_partials",
              "oracle_attention_full", "oracle_attention_partials_varlen"):
        getattr(lib, f).restype = i32
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def bf16_to_f64(bits) -> np.ndarray:
    """Decode raw bf16 bits (uint16 array) to float64 with the oracle's own routine."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    lib = _load()
    flat = bits.reshape(-1)
    out = np.empty(flat.shape, dtype=np.float64)
    for i, b in enumerate(flat):
        out[i] = lib.oracle_bf16_to_f64(int(b))
    return out.reshape(bits.shape)


def f16_to_f64(bits) -> np.ndarray:
    """Decode raw IEEE binary16 bits (uint16 array) to float64 with the oracle's own routine."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    lib = _load()
    flat = bits.reshape(-1)
    out = np.empty(flat.shape, dtype=np.float64)
    for i, b in enumerate(flat):
        out[i] = lib.oracle_f16_to_f64(int(b))
    return out.reshape(bits.shape)


def merge(O, lse, cp: int, lse_layout: int, lse_mode: int, threads: int = 0, dtype: str = "bf16"):
    """LSE-weighted merge of cp shards.

    ``O``: [B, H, D], either uint16 (raw 16-bit payload bits: bf16, or IEEE
    binary16 with ``dtype="f16"``) or float64.
    ``lse``: contiguous [B, H/cp, cp] (``LSE_BHC``) or [B, H] / [B, H, 1]
    (``LSE_BH1``); float32 with bf16 ``O``, float64 with float64 ``O``.
    Returns ``(out [B, H/cp, D], lse [B, H/cp], abs_weighted [B, H/cp, D])`` in float64.
    """
    lib = _load()
    B, H, D = O.shape
    if H % cp:
        raise ValueError("H must be a multiple of cp")
    hl = H // cp
    if O.dtype == np.uint16:
        O = np.ascontiguousarray(O)
        lse = np.ascontiguousarray(lse, dtype=np.float32)
        if dtype not in ("bf16", "f16"):
            raise ValueError("dtype must be 'bf16' or 'f16'")
        fn = lib.oracle_merge_bf16 if dtype == "bf16" else lib.oracle_merge_f16
    else:
        O = np.ascontiguousarray(O, dtype=np.float64)
        lse = np.ascontiguousarray(lse, dtype=np.float64)
        fn = lib.oracle_merge_f64
    if lse.size != B * H:
        raise ValueError("lse has %d elements, expected B*H = %d" % (lse.size, B * H))
    out = np.empty((B, hl, D), dtype=np.float64)
    out_lse = np.empty((B, hl), dtype=np.float64)
    out_abs = np.empty((B, hl, D), dtype=np.float64)
    rc = fn(_ptr(O), _ptr(lse), B, H, cp, D, lse_layout, lse_mode, _ptr(out), _ptr(out_lse), _ptr(out_abs),
            threads)
    if rc:
        raise ValueError("oracle_merge rejected its arguments (rc=%d)" % rc)
    return out, out_lse, out_abs


def _rows_arg(rows, B, hq):
    if rows is None:
        return None, B * hq
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= B * hq):
        raise ValueError("row index out of range")
    return rows, rows.size


def attention_partials(q_bits, kv_bits, cp: int, scale: float, lse_mode: int, dv: int = 512, rows=None,
                       threads: int = 0, dtype: str = "bf16"):
    """Per-shard softmax partials.  ``q_bits`` [B, hq, dqk] and ``kv_bits`` [T, dqk]
    are uint16 bits of ``dtype`` ("bf16" or "f16").  Returns
    ``(o [n_rows, cp, dv], lse [n_rows, cp])``."""
    lib = _load()
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    kv_bits = np.ascontiguousarray(kv_bits, dtype=np.uint16)
    B, hq, dqk = q_bits.shape
    T = kv_bits.shape[0]
    assert kv_bits.shape[1] == dqk
    rows, n = _rows_arg(rows, B, hq)
    o = np.empty((n, cp, dv), dtype=np.float64)
    lse = np.empty((n, cp), dtype=np.float64)
    rc = lib.oracle_attention_partials(_ptr(q_bits), _ptr(kv_bits), B, hq, T, dqk, dv, cp, float(scale), lse_mode,
                                       _DTYPE[dtype], _ptr(rows), n, _ptr(o), _ptr(lse), threads)
    if rc:
        raise ValueError("oracle_attention_partials rejected its arguments (rc=%d)" % rc)
    return o, lse


def attention_partials_varlen(q_bits, kv_bits, seq_lens, cp: int, scale: float, lse_mode: int,
                              interleaved: bool = False, dv: int = 512, rows=None, threads: int = 0,
                              dtype: str = "bf16"):
    """Per-shard partials with one cache per query token.  ``q_bits`` [B, hq, dqk];
    ``kv_bits`` [B, Tmax, dqk] (token b's cache) or [Tmax, dqk] (one cache shared by
    every token); ``seq_lens`` [B] int.  Shard s owns a contiguous slice of token b's
    first seq_lens[b] rows, or (``interleaved``) the rows t with t mod cp == s.
    Returns ``(o [n_rows, cp, dv], lse [n_rows, cp])``."""
    lib = _load()
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    kv_bits = np.ascontiguousarray(kv_bits, dtype=np.uint16)
    seq = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B, hq, dqk = q_bits.shape
    if kv_bits.ndim == 2:
        kv_sb, tmax = 0, kv_bits.shape[0]
    else:
        assert kv_bits.shape[0] == B
        kv_sb, tmax = kv_bits.shape[1], kv_bits.shape[1]
    assert kv_bits.shape[-1] == dqk and seq.shape == (B,)
    if seq.size and (seq.min() < 0 or seq.max() > tmax):
        raise ValueError("seq_lens must lie in [0, %d]" % tmax)
    rows, n = _rows_arg(rows, B, hq)
    o = np.empty((n, cp, dv), dtype=np.float64)
    lse = np.empty((n, cp), dtype=np.float64)
    rc = lib.oracle_attention_partials_varlen(_ptr(q_bits), _ptr(kv_bits), B, hq, kv_sb, _ptr(seq), int(interleaved),
                                              dqk, dv, cp, float(scale), lse_mode, _DTYPE[dtype], _ptr(rows), n,
                                              _ptr(o), _ptr(lse), threads)
    if rc:
        raise ValueError("oracle_attention_partials_varlen rejected its arguments (rc=%d)" % rc)
    return o, lse


def attention_full(q_bits, kv_bits, scale: float, lse_mode: int, dv: int = 512, rows=None, threads: int = 0,
                   dtype: str = "bf16"):
    """Unsharded softmax decode attention.  Returns ``(o [n_rows, dv], lse [n_rows])``."""
    lib = _load()
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    kv_bits = np.ascontiguousarray(kv_bits, dtype=np.uint16)
    B, hq, dqk = q_bits.shape
    T = kv_bits.shape[0]
    rows, n = _rows_arg(rows, B, hq)
    o = np.empty((n, dv), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = lib.oracle_attention_full(_ptr(q_bits), _ptr(kv_bits), B, hq, T, dqk, dv, float(scale), lse_mode,
                                   _DTYPE[dtype], _ptr(rows), n, _ptr(o), _ptr(lse), threads)
    if rc:
        raise ValueError("oracle_attention_full rejected its arguments (rc=%d)" % rc)
    return o, lse
