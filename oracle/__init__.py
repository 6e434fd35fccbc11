"""fp64 CPU oracle for 1.5-entmax attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it and
shares no code with it.  The arithmetic lives in ``entmax_oracle.c`` (plain C,
fp64, OpenMP over rows); this module only compiles it with gcc and marshals
numpy arrays through ctypes.

Definitions followed (see the header of ``entmax_oracle.c`` for the full list):
  * 1.5-entmax p = [(s - tau)/2]_+^2 with sum p = 1: "GPT-2 with AdaSplash
    Attention via NeuralOps", Mathematical Formulation item 2;
    "AdaSplash-2: Faster Differentiable Sparse Attention", sec. 2.3-2.4.
  * exact tau by sorting plus the quadratic in (S0, S1, S2): AdaSplash-2
    sec. 2.4 "Sorting-based solvers" and appendix C.3.
  * attention S = scale Q K^T, O = A V: AdaSplash-2 sec. 2.2.
  * backward restricted to the support: AdaSplash-2 sec. 3.3 "Backward pass".
  * block mask packing, 32 column blocks per word: AdaSplash-2 appendix C.4.
  * general alpha in (1, 2] (AdaSplash-2 sec. 2.3): p = [(alpha-1)(s - tau)]_+
    ^(1/(alpha-1)); exact by sorting at alpha = 2 (sparsemax), by bisection on
    the bracket of sec. 2.4 for other alpha.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "entmax_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib: Optional[ctypes.CDLL] = None

MASK_NONE, MASK_CAUSAL, MASK_WINDOW_SINK = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile entmax_oracle.c into liboracle.so with gcc (fp64, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_entmax15_tau.restype = ctypes.c_double
    lib.orc_entmax15_tau.argtypes = [P, i64, P, P]
    lib.orc_entmax15.restype = ctypes.c_double
    lib.orc_entmax15.argtypes = [P, i64, P, P]
    lib.orc_tau_rows.restype = None
    lib.orc_tau_rows.argtypes = [P, i64, i64, i64, P, P]
    lib.orc_key_active.restype = ctypes.c_int
    lib.orc_key_active.argtypes = [ctypes.c_int, i64, i64, i64]
    lib.orc_attn_fwd.restype = None
    lib.orc_attn_fwd.argtypes = [P, P, P, i64, i64, i64, ctypes.c_double,
                                 ctypes.c_int, i64, P, i64, P, P, P, P]
    lib.orc_block_mask_head.restype = None
    lib.orc_block_mask_head.argtypes = [P, P, i64, i64, ctypes.c_double,
                                        ctypes.c_int, i64, i64, i64,
                                        ctypes.c_double, P, P, P, P]
    lib.orc_attn_bwd_head.restype = None
    lib.orc_attn_bwd_head.argtypes = [P, P, P, P, i64, i64, ctypes.c_double,
                                      ctypes.c_int, i64, P, P, P, P, P]
    lib.orc_attn_bwd_rows.restype = None
    lib.orc_attn_bwd_rows.argtypes = [P, P, P, P, i64, i64, i64,
                                      ctypes.c_double, ctypes.c_int, i64, P,
                                      i64, P, P, P]
    D = ctypes.c_double
    lib.orc_entmax_tau_bisect.restype = D
    lib.orc_entmax_tau_bisect.argtypes = [P, i64, D]
    lib.orc_entmax_tau_histogram.restype = D
    lib.orc_entmax_tau_histogram.argtypes = [P, i64, ctypes.c_float, ctypes.c_int]
    lib.orc_entmax_alpha.restype = D
    lib.orc_entmax_alpha.argtypes = [P, i64, D, P, P]
    lib.orc_tau_rows_alpha.restype = None
    lib.orc_tau_rows_alpha.argtypes = [P, i64, i64, i64, D, P, P]
    lib.orc_attn_fwd_alpha.restype = None
    lib.orc_attn_fwd_alpha.argtypes = [P, P, P, i64, i64, i64, D, ctypes.c_int, i64, D,
                                       P, i64, P, P, P, P]
    lib.orc_block_mask_head_alpha.restype = None
    lib.orc_block_mask_head_alpha.argtypes = [P, P, i64, i64, D, ctypes.c_int, i64, D,
                                              i64, i64, D, P, P, P, P]
    lib.orc_attn_bwd_head_alpha.restype = None
    lib.orc_attn_bwd_head_alpha.argtypes = [P, P, P, P, i64, i64, D, ctypes.c_int, i64, D,
                                            P, P, P, P, P]
    lib.orc_attn_bwd_rows_alpha.restype = None
    lib.orc_attn_bwd_rows_alpha.argtypes = [P, P, P, P, i64, i64, i64, D, ctypes.c_int,
                                            i64, D, P, i64, P, P, P]
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def num_threads() -> int:
    return int(_load().orc_num_threads())


def entmax15(s) -> tuple[np.ndarray, float, int]:
    """1.5-entmax of one score vector (fp64; -inf entries are inactive).

    Returns (p, tau, support_size)."""
    s = np.ascontiguousarray(np.asarray(s, dtype=np.float64))
    p = np.empty_like(s)
    k = ctypes.c_int64(0)
    tau = _load().orc_entmax15(_ptr(s), s.size, _ptr(p), ctypes.byref(k))
    return p, float(tau), int(k.value)


def key_active(mask: int, window: int, i: int, j: int) -> bool:
    return bool(_load().orc_key_active(mask, window, i, j))


def entmax(s, alpha: float = 1.5) -> tuple[np.ndarray, float, int]:
    """alpha-entmax of one score vector for alpha in (1, 2] (fp64; -inf
    entries are inactive): p = [(alpha-1)(s - tau)]_+^(1/(alpha-1)).

    Returns (p, tau, support_size)."""
    s = np.ascontiguousarray(np.asarray(s, dtype=np.float64))
    p = np.empty_like(s)
    k = ctypes.c_int64(0)
    tau = _load().orc_entmax_alpha(_ptr(s), s.size, float(alpha), _ptr(p), ctypes.byref(k))
    return p, float(tau), int(k.value)


def tau_bisect(s, alpha: float) -> float:
    """tau by plain bisection on the bracket (any alpha in (1, 2])."""
    s = np.ascontiguousarray(np.asarray(s, dtype=np.float64))
    return float(_load().orc_entmax_tau_bisect(_ptr(s), s.size, float(alpha)))


def tau_histogram(s, alpha: float = 1.5, bins: int = 64) -> float:
    """Histogram threshold tau_h of one fp32 row (AdaSplash-2 sec. 3.1)."""
    s = _f32(s)
    return float(_load().orc_entmax_tau_histogram(_ptr(s), s.size, float(alpha), int(bins)))


def tau_rows(S, want_p: bool = True, alpha: float = 1.5) -> tuple[np.ndarray, Optional[np.ndarray]]:
    """Row-wise tau (and P) of a 2-D fp32 score matrix."""
    S = _f32(S)
    rows, cols = S.shape
    tau = np.empty(rows, dtype=np.float64)
    P = np.empty((rows, cols), dtype=np.float64) if want_p else None
    _load().orc_tau_rows_alpha(_ptr(S), rows, cols, cols, float(alpha), _ptr(tau),
                               _ptr(P) if P is not None else None)
    return tau, P


def attn_fwd(Q, K, V, scale: float, mask: int = MASK_NONE, window: int = 0,
             rows: Optional[np.ndarray] = None, alpha: float = 1.5):
    """Forward for the listed flattened query rows (all rows when None).

    Q, K, V: [B, H, L, d] (any float dtype holding exact values).
    Returns (O [n, d], tau [n], support [n], gsum [n]) in fp64."""
    Q, K, V = _f32(Q), _f32(K), _f32(V)
    B, H, L, d = Q.shape
    BH = B * H
    if rows is None:
        n = BH * L
        rp = None
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows.size
        rp = _ptr(rows)
    O = np.empty((n, d), dtype=np.float64)
    tau = np.empty(n, dtype=np.float64)
    nsup = np.empty(n, dtype=np.int64)
    gsum = np.empty(n, dtype=np.float64)
    _load().orc_attn_fwd_alpha(_ptr(Q), _ptr(K), _ptr(V), BH, L, d, float(scale),
                               int(mask), int(window), float(alpha), rp, n, _ptr(O),
                               _ptr(tau), _ptr(nsup), _ptr(gsum))
    return O, tau, nsup, gsum


def block_mask_head(Qh, Kh, scale: float, mask: int, window: int, br: int,
                    bc: int, tol: float = 1e-4, alpha: float = 1.5):
    """Packed block masks of one head ([L, d] inputs) at tile br x bc.

    Returns (exact, must, may, tau); each mask is uint32 [Tr, ceil(Tc/32)]."""
    Qh, Kh = _f32(Qh), _f32(Kh)
    L, d = Qh.shape
    Tr, Tc = -(-L // br), -(-L // bc)
    Wd = -(-Tc // 32)
    ex = np.empty((Tr, Wd), dtype=np.uint32)
    lo = np.empty((Tr, Wd), dtype=np.uint32)
    hi = np.empty((Tr, Wd), dtype=np.uint32)
    tau = np.empty(L, dtype=np.float64)
    _load().orc_block_mask_head_alpha(_ptr(Qh), _ptr(Kh), L, d, float(scale),
                                      int(mask), int(window), float(alpha), br, bc,
                                      float(tol), _ptr(ex), _ptr(lo), _ptr(hi), _ptr(tau))
    return ex, lo, hi, tau


def attn_bwd_head(Qh, Kh, Vh, dOh, scale: float, mask: int = MASK_NONE,
                  window: int = 0, alpha: float = 1.5):
    """Full backward of one head ([L, d] inputs).

    Returns (dQ, dK, dV, tau, delta) in fp64."""
    Qh, Kh, Vh, dOh = _f32(Qh), _f32(Kh), _f32(Vh), _f32(dOh)
    L, d = Qh.shape
    dQ = np.empty((L, d)); dK = np.empty((L, d)); dV = np.empty((L, d))
    tau = np.empty(L); delta = np.empty(L)
    _load().orc_attn_bwd_head_alpha(_ptr(Qh), _ptr(Kh), _ptr(Vh), _ptr(dOh), L, d,
                                    float(scale), int(mask), int(window), float(alpha),
                                    _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(tau), _ptr(delta))
    return dQ, dK, dV, tau, delta


def attn_bwd_rows(Q, K, V, dO, scale: float, mask: int, window: int, rows,
                  alpha: float = 1.5):
    """dQ, delta and tau for the listed flattened query rows of [B,H,L,d]."""
    Q, K, V, dO = _f32(Q), _f32(K), _f32(V), _f32(dO)
    B, H, L, d = Q.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = rows.size
    dQ = np.empty((n, d)); delta = np.empty(n); tau = np.empty(n)
    _load().orc_attn_bwd_rows_alpha(_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), B * H, L, d,
                                    float(scale), int(mask), int(window), float(alpha),
                                    _ptr(rows), n, _ptr(dQ), _ptr(delta), _ptr(tau))
    return dQ, delta, tau
