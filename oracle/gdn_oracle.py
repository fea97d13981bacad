"""Python front end of the double-precision oracle (test infrastructure only).

Only the tests, the package's smoke check and the CPU-baseline leg of the
benchmark may import this module.  It loads ``liboracle_gdn.so`` built from
``gdn_oracle.c`` with the host C compiler and never touches the HIP library.

Arrays are numpy.  bf16 tensors travel as ``uint16`` bit patterns, OCP E4M3
tensors as ``uint8`` codes, fp32 as ``float32``.  Layouts: q, k, v, o are [B, H, T, S, D]; gamma, beta [B, H, T];
states [B, H, D, D] indexed [key][value].

The recurrence itself is documented in ``gdn_oracle.c`` (source: the SANA-WM
news article "NVIDIA Apresenta SANA-WM ...", section "1. Atencao Linear
Hibrida com Gated DeltaNet (GDN)").
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB = os.path.join(HERE, "liboracle_gdn.so")

ERASE, WRITE = 0, 1
_MODES = {"erase": ERASE, "write": WRITE, ERASE: ERASE, WRITE: WRITE}


def build(out: str = LIB, mutant: int = 0, quiet: bool = True, native: bool = False) -> str:
    """Compile the oracle with gcc (OpenMP, no fast-math, no floating-point
    contraction).  native=True builds it -O3 -march=native for timing on the
    host it runs on; the arithmetic is the same (every sum keeps its order:
    without -ffast-math gcc neither reassociates nor contracts)."""
    opt = ["-O3", "-march=native"] if native else ["-O2"]
    cmd = ["gcc", *opt, "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off",
           f"-DORACLE_MUTANT={int(mutant)}", SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, capture_output=quiet)
    os.replace(out + ".tmp", out)
    return out


_libs: dict = {}


def load(path: str = LIB) -> ctypes.CDLL:
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SRC):
        if path != LIB:
            raise FileNotFoundError(path)
        build(path)
    lib = ctypes.CDLL(path)
    lib.oracle_gdn_head.restype = ctypes.c_int
    lib.oracle_gdn_head.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int]
    lib.oracle_e4m3_decode.restype = None
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    _libs[path] = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def head(q, k, v, gamma, beta, state_in=None, beta_mode="erase", want_out=True,
         want_norms=False, threads: int = 0, lib_path: str = LIB):
    """One head: q, k, v [T, S, D] (float32, uint16 bf16 bits or uint8 E4M3 codes), gamma/beta [T].

    Returns (out [T,S,D] float64 or None, state_out [D,D] float64, norms [T] or None).
    """
    lib = load(lib_path)
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    if not (q.shape == k.shape == v.shape and q.ndim == 3):
        raise ValueError("q, k, v must share shape [T, S, D]")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share dtype")
    if q.dtype == np.float32:
        io = 0
    elif q.dtype == np.uint16:
        io = 1
    elif q.dtype == np.uint8:
        io = 2
    else:
        raise TypeError("inputs must be float32, uint16 (bf16 bit patterns) or uint8 (E4M3 codes)")
    T, S, D = q.shape
    g = np.ascontiguousarray(gamma, dtype=np.float32).reshape(T)
    b = np.ascontiguousarray(beta, dtype=np.float32).reshape(T)
    sin = None if state_in is None else np.ascontiguousarray(state_in, dtype=np.float64).reshape(D, D)
    out = np.empty((T, S, D), np.float64) if want_out else None
    sout = np.empty((D, D), np.float64)
    norms = np.empty((T,), np.float64) if want_norms else None
    rc = lib.oracle_gdn_head(T, S, D, io, _MODES[beta_mode], _ptr(q), _ptr(k), _ptr(v),
                             _ptr(g), _ptr(b), _ptr(sin), _ptr(out), _ptr(sout), _ptr(norms),
                             int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_gdn_head failed with code {rc}")
    return out, sout, norms


def forward(q, k, v, gamma, beta, state_in=None, beta_mode="erase", want_out=True,
            want_norms=False, threads: int = 0, lib_path: str = LIB):
    """All heads: q, k, v [B, H, T, S, D]; gamma/beta [B, H, T]; state_in [B, H, D, D] or None.

    Returns (out [B,H,T,S,D] float64 or None, state_out [B,H,D,D], norms [B,H,T] or None).
    """
    B, H, T, S, D = q.shape
    out = np.empty((B, H, T, S, D), np.float64) if want_out else None
    sout = np.empty((B, H, D, D), np.float64)
    norms = np.empty((B, H, T), np.float64) if want_norms else None
    for bi in range(B):
        for hi in range(H):
            o, s, n = head(q[bi, hi], k[bi, hi], v[bi, hi], gamma[bi, hi], beta[bi, hi],
                           None if state_in is None else state_in[bi, hi], beta_mode,
                           want_out, want_norms, threads, lib_path)
            if want_out:
                out[bi, hi] = o
            sout[bi, hi] = s
            if want_norms:
                norms[bi, hi] = n
    return out, sout, norms


def e4m3_to_f64(codes: np.ndarray, lib_path: str = LIB) -> np.ndarray:
    """Exact values of OCP E4M3 codes (uint8), decoded by the oracle's C decoder."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    load(lib_path).oracle_e4m3_decode(_ptr(c), _ptr(out), int(c.size))
    return out


def _e4m3_grid() -> np.ndarray:
    """Values of the non-negative finite E4M3 codes 0x00..0x7E, in code order
    (which is also increasing value order)."""
    return e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))


def round_e4m3(x: np.ndarray) -> np.ndarray:
    """E4M3 code (uint8) nearest to each double, ties to the even code.

    The grid is that of the format (OCP 8-bit float E4M3, "fn" variant): the
    126 non-negative finite values, 448 the largest.  A magnitude past 464,
    half-way to the first value the format lacks (480), has no nearest code and
    gives NaN; NaN gives NaN.  The sign goes to the top bit, so -0.0 is 0x80.
    This is the rounding used for an E4M3 output: one rounding of the exact
    value to the format.
    """
    x = np.asarray(x, dtype=np.float64)
    grid = _e4m3_grid()
    a = np.abs(x)
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, len(grid) - 1)   # first grid value >= a
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    dlo, dhi = a - grid[lo], grid[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a > 464.0, 0x7F, code).astype(np.uint8)
    code = np.where(np.isnan(x), 0x7F, code).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
