"""Parallax attention oracle -- TEST INFRASTRUCTURE ONLY.

A plain double-precision CPU implementation of the Parallax readout (see
``oracle.c`` for the definition and the passages it follows). Only the tests,
``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may
import this package; the GPU library and its Python binding never do, and the
two share no code. Inputs are numpy arrays of float32, float64 or of
bf16 bit patterns (uint16); every result is float64.

Parity pins (tests/test_oracle_pins.py) tie this code to what the pages and
the mathematics fix: r = 0 against torch's float64 scaled_dot_product_attention,
the correction against numpy's weighted covariance and against the
cross-covariance matrix route, the plus sign against the intercept of a
weighted least-squares fit, closed forms for one and two keys, shift and
linearity invariants, and a 50-digit mpmath evaluation on tiny inputs. The
gradients (tests/test_oracle_backward_pins.py) are pinned by central finite
differences of the pinned forward, torch's float64 autograd through
scaled_dot_product_attention at r = 0, and exact identities of the forward
(key-shift invariance, linearity in v, the probe-scale derivative).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PLX_SANITIZED_HOST_LIBS=1 selects the AddressSanitizer + UBSan build
# (liboracle_san.so, from build(sanitize=True)); the process must then preload
# gcc's libasan and libubsan.
_SANITIZED = os.environ.get("PLX_SANITIZED_HOST_LIBS") == "1"
_LIB_PATH = os.path.join(_HERE, "liboracle_san.so" if _SANITIZED else "liboracle.so")
_lib = None

F32, BF16, F64 = 0, 1, 2


def build(sanitize: bool = False) -> str:
    """Compile ``liboracle.so`` (plain C, double, OpenMP; no fast-math).
    sanitize=True builds liboracle_san.so with AddressSanitizer and UBSan
    instead (host test tier)."""
    out = os.path.join(_HERE, "liboracle_san.so" if sanitize else "liboracle.so")
    opt = (["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=undefined"] if sanitize else ["-O2"])
    cmd = ["gcc", *opt, "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
           os.path.join(_HERE, "oracle.c"), "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _bind(path: str):
    lib = ctypes.CDLL(path)
    vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_decode.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, dbl, dbl,
                                  i64, vp, i64, i64, i64, vp, vp]
    lib.oracle_decode.restype = i32
    lib.oracle_prefill.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, dbl, dbl,
                                   i64, vp, i64, i64, vp, vp, vp, vp]
    lib.oracle_prefill.restype = i32
    lib.oracle_prefill_backward.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                            dbl, dbl, i64, vp, i64, i64, vp, vp, vp, vp, vp]
    lib.oracle_prefill_backward.restype = i32
    lib.oracle_set_num_threads.argtypes = [i32]
    lib.oracle_set_num_threads.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i32
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
        _lib = _bind(_LIB_PATH)
    return _lib


class _Using:
    """Temporarily route decode()/prefill() through another build of oracle.c
    (the mutation tests compile deliberately broken copies)."""

    def __init__(self, path):
        self.lib = _bind(path)

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = self.lib
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def using_library(path: str) -> _Using:
    return _Using(path)


def set_num_threads(n: int) -> None:
    """Threads of the oracle's OpenMP regions (for timing on a given core count)."""
    _load().oracle_set_num_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _dtype_of(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle inputs are float32, float64 or bf16 bits (uint16), got {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


BLOCK = 128  # block-sparse mask granularity of the GPU library (the oracle takes any)


def _mask(block_mask, shape):
    """A block mask as contiguous uint8 of the given shape (None stays None)."""
    if block_mask is None:
        return None
    m = np.ascontiguousarray(np.asarray(block_mask) != 0, dtype=np.uint8)
    assert m.shape == tuple(shape), f"block mask shape {m.shape}, expected {tuple(shape)}"
    return m


def decode(q, r, k, v, *, seq_start=None, seq_len=None, Hkv=None, qk_scale=None, rk_scale=1.0,
           rows=None, window=0, block_mask=None, block=BLOCK):
    """Parallax decode rows.

    q, r: [B, Hq, D] (r may be None: r = 0, plain softmax attention).
    k, v: [B, L, Hkv, D] dense, or [T, Hkv, D] packed with ``seq_start`` /
    ``seq_len`` giving each sequence's token range.
    rows: optional int array [n, 2] of (b, h); default all rows.
    window: W > 0 keeps each sequence's last W keys (0: all).
    block_mask: optional [B, Hkv, nkb] (nonzero: visible) over key blocks of
    ``block`` positions, nkb >= ceil(longest sequence / block); the block
    holding a sequence's last key is always visible.
    Returns float64 [B, Hq, D] (or [n, D] when rows is given).
    """
    dt = _dtype_of(q)
    for a in (r, k, v):
        if a is not None:
            assert _dtype_of(a) == dt and a.flags.c_contiguous
    assert q.flags.c_contiguous
    B, Hq, D = q.shape
    if k.ndim == 4:
        Bk, L, Hk, Dk = k.shape
        assert Bk == B and Dk == D
        if seq_start is None:
            seq_start = np.arange(B, dtype=np.int64) * L
        if seq_len is None:
            seq_len = np.full(B, L, dtype=np.int64)
    else:
        _, Hk, Dk = k.shape
        assert Dk == D and seq_start is not None and seq_len is not None
    Hkv = Hk if Hkv is None else Hkv
    seq_start = np.ascontiguousarray(seq_start, dtype=np.int64)
    seq_len = np.ascontiguousarray(seq_len, dtype=np.int64)
    tau = 1.0 / math.sqrt(D) if qk_scale is None else float(qk_scale)
    mcols = 0
    if block_mask is not None:
        mcols = np.asarray(block_mask).shape[-1]
        assert mcols * block >= int(seq_len.max(initial=0))
        block_mask = _mask(block_mask, (B, Hkv, mcols))
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 2)
        out = np.empty((rows.shape[0], D), dtype=np.float64)
        n = rows.shape[0]
    else:
        out = np.empty((B, Hq, D), dtype=np.float64)
        n = B * Hq
    rc = _load().oracle_decode(_ptr(q), _ptr(r), _ptr(k), _ptr(v), dt, _ptr(seq_start),
                               _ptr(seq_len), B, Hq, Hkv, D, tau, float(rk_scale), int(window),
                               _ptr(block_mask), int(block), int(mcols), n, _ptr(rows),
                               _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle_decode failed ({rc})")
    return out


def prefill(q, r, k, v, *, qk_scale=None, rk_scale=1.0, rows=None, stats=False, window=0,
            block_mask=None, block=BLOCK):
    """Causal Parallax prefill rows.

    q, r: [B, Hq, L, D] (r may be None); k, v: [B, Hkv, L, D].
    rows: optional int array [n, 3] of (b, h, i).
    window: W > 0 limits query i to keys i - W + 1 .. i (0: causal only).
    block_mask: optional [B, Hkv, nb, nb], nb = ceil(L / block): entry
    [qb, kb] (nonzero: visible) lets query block qb see key block kb; the
    diagonal block is always visible.
    Returns o float64 [B, Hq, L, D] (or [n, D]); with stats=True also lse and sbar.
    """
    dt = _dtype_of(q)
    for a in (q, r, k, v):
        if a is not None:
            assert _dtype_of(a) == dt and a.flags.c_contiguous
    B, Hq, L, D = q.shape
    Hkv = k.shape[1]
    tau = 1.0 / math.sqrt(D) if qk_scale is None else float(qk_scale)
    nb = -(-L // block)
    block_mask = _mask(block_mask, (B, Hkv, nb, nb))
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
        n = rows.shape[0]
        out = np.empty((n, D), dtype=np.float64)
        lse = np.empty(n, dtype=np.float64)
        sbar = np.empty(n, dtype=np.float64)
    else:
        n = B * Hq * L
        out = np.empty((B, Hq, L, D), dtype=np.float64)
        lse = np.empty((B, Hq, L), dtype=np.float64)
        sbar = np.empty((B, Hq, L), dtype=np.float64)
    rc = _load().oracle_prefill(_ptr(q), _ptr(r), _ptr(k), _ptr(v), dt, B, Hq, Hkv, L, D, tau,
                                float(rk_scale), int(window), _ptr(block_mask), int(block), n,
                                _ptr(rows), _ptr(out), _ptr(lse), _ptr(sbar))
    if rc != 0:
        raise RuntimeError(f"oracle_prefill failed ({rc})")
    return (out, lse, sbar) if stats else out


def prefill_backward(q, r, k, v, do, *, qk_scale=None, rk_scale=1.0, units=None, window=0,
                     block_mask=None, block=BLOCK):
    """Gradients of the causal Parallax prefill for the upstream gradient ``do``.

    q, r, do: [B, Hq, L, D] (r may be None: r = 0); k, v: [B, Hkv, L, D].
    units: optional int array [n, 2] of (b, hkv): only the query heads reading
    those KV heads (and those KV heads' keys) are differentiated.
    window, block_mask, block: as in prefill.
    Returns float64 (dq, dr, dk, dv): [B, Hq, L, D] and [B, Hkv, L, D], or with
    ``units`` [n, g, L, D] and [n, L, D].
    """
    dt = _dtype_of(q)
    for a in (q, r, k, v, do):
        if a is not None:
            assert _dtype_of(a) == dt and a.flags.c_contiguous
    B, Hq, L, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    tau = 1.0 / math.sqrt(D) if qk_scale is None else float(qk_scale)
    nb = -(-L // block)
    block_mask = _mask(block_mask, (B, Hkv, nb, nb))
    if units is not None:
        units = np.ascontiguousarray(units, dtype=np.int64).reshape(-1, 2)
        n = units.shape[0]
    else:
        n = B * Hkv
    dq = np.empty((n, g, L, D), dtype=np.float64)
    dr = np.empty((n, g, L, D), dtype=np.float64)
    dk = np.empty((n, L, D), dtype=np.float64)
    dv = np.empty((n, L, D), dtype=np.float64)
    rc = _load().oracle_prefill_backward(_ptr(q), _ptr(r), _ptr(k), _ptr(v), _ptr(do), dt, B, Hq,
                                         Hkv, L, D, tau, float(rk_scale), int(window),
                                         _ptr(block_mask), int(block), n, _ptr(units), _ptr(dq),
                                         _ptr(dr), _ptr(dk), _ptr(dv))
    if rc != 0:
        raise RuntimeError(f"oracle_prefill_backward failed ({rc})")
    if units is None:
        return (dq.reshape(B, Hq, L, D), dr.reshape(B, Hq, L, D), dk.reshape(B, Hkv, L, D),
                dv.reshape(B, Hkv, L, D))
    return dq, dr, dk, dv


def _seq_dense(x, s0, s1):
    """Packed [T, H, D] rows s0 .. s1 - 1 as a dense [1, H, n, D] array."""
    return np.ascontiguousarray(x[s0:s1].transpose(1, 0, 2)[None])


def _seq_mask(block_mask, b, n, block):
    """Sequence b's block mask for length n, from a [B, Hkv, nb, nb] mask over
    the longest sequence (None stays None)."""
    if block_mask is None:
        return None
    nb = -(-n // block)
    return np.ascontiguousarray(np.asarray(block_mask)[b:b + 1, :, :nb, :nb])


def prefill_varlen(q, r, k, v, cu_seqlens, *, qk_scale=None, rk_scale=1.0, window=0,
                   stats=False, block_mask=None, block=BLOCK):
    """Causal prefill of packed sequences (the pages' parallax_varlen_func): q, r
    [T, Hq, D], k, v [T, Hkv, D], sequence b = tokens cu[b] .. cu[b+1] - 1.
    Each sequence is an independent causal prefill (the dense oracle on its
    slice). block_mask: optional [B, Hkv, nb, nb] over sequence-local blocks,
    nb = ceil(longest length / block). Returns o [T, Hq, D] (and lse, sbar
    [T, Hq] with stats=True)."""
    T, Hq, D = q.shape
    o = np.zeros((T, Hq, D), dtype=np.float64)
    lse = np.zeros((T, Hq), dtype=np.float64)
    sbar = np.zeros((T, Hq), dtype=np.float64)
    for b, (s0, s1) in enumerate(zip(cu_seqlens[:-1], cu_seqlens[1:])):
        if s1 <= s0:
            continue
        res = prefill(_seq_dense(q, s0, s1), None if r is None else _seq_dense(r, s0, s1),
                      _seq_dense(k, s0, s1), _seq_dense(v, s0, s1), qk_scale=qk_scale,
                      rk_scale=rk_scale, window=window, stats=True,
                      block_mask=_seq_mask(block_mask, b, s1 - s0, block), block=block)
        o[s0:s1] = res[0][0].transpose(1, 0, 2)
        lse[s0:s1] = res[1][0].T
        sbar[s0:s1] = res[2][0].T
    return (o, lse, sbar) if stats else o


def prefill_varlen_backward(q, r, k, v, do, cu_seqlens, *, qk_scale=None, rk_scale=1.0,
                            window=0, block_mask=None, block=BLOCK):
    """Gradients of prefill_varlen: (dq, dr [T, Hq, D], dk, dv [T, Hkv, D])."""
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    dq = np.zeros((T, Hq, D)); dr = np.zeros((T, Hq, D))
    dk = np.zeros((T, Hkv, D)); dv = np.zeros((T, Hkv, D))
    for b, (s0, s1) in enumerate(zip(cu_seqlens[:-1], cu_seqlens[1:])):
        if s1 <= s0:
            continue
        g = prefill_backward(_seq_dense(q, s0, s1), None if r is None else _seq_dense(r, s0, s1),
                             _seq_dense(k, s0, s1), _seq_dense(v, s0, s1),
                             _seq_dense(do, s0, s1), qk_scale=qk_scale, rk_scale=rk_scale,
                             window=window, block_mask=_seq_mask(block_mask, b, s1 - s0, block),
                             block=block)
        dq[s0:s1] = g[0][0].transpose(1, 0, 2)
        dr[s0:s1] = g[1][0].transpose(1, 0, 2)
        dk[s0:s1] = g[2][0].transpose(1, 0, 2)
        dv[s0:s1] = g[3][0].transpose(1, 0, 2)
    return dq, dr, dk, dv
