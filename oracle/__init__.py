"""The CPU oracle for matmul against GGUF block-quantized weights.

TEST INFRASTRUCTURE ONLY.  This package wraps ``qmm_oracle.c`` (plain C,
binary64, element-indexed decoders, a k-ascending matmul and the tolerance
bound sum |w||x|).  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import it.  It shares no code with the HIP
library and never calls it; the library never calls this.

Kinds are the GGUF type ids (Q4_0=2, Q5_0=6, Q8_0=8, Q2_K=10, Q3_K=11,
Q4_K=12, Q5_K=13, Q6_K=14, IQ4_NL=20, IQ4_XS=23, MXFP4=39) or their names.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "qmm_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

KINDS = {
    "Q8_0": 8, "Q4_0": 2, "Q5_0": 6, "Q2_K": 10, "Q3_K": 11, "Q4_K": 12,
    "Q5_K": 13, "Q6_K": 14, "IQ4_NL": 20, "IQ4_XS": 23, "MXFP4": 39,
}


def compile_library(src: str, out: str) -> str:
    """gcc -O2 with OpenMP; no fast-math and no FMA contraction."""
    tmp = out + ".tmp"
    subprocess.run(
        ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
         "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
         src, "-o", tmp, "-lm"],
        check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
        compile_library(SOURCE, LIBRARY)
    return LIBRARY


def _kind(kind) -> int:
    return KINDS[kind] if isinstance(kind, str) else int(kind)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _as_f64(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype not in (np.float32, np.float16, np.float64):
        raise TypeError(f"activations must be f16/f32/f64, got {x.dtype}")
    return np.ascontiguousarray(x.astype(np.float64))  # exact widening


class Oracle:
    """One loaded copy of the oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        lib.oracle_block_geometry.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                              ctypes.POINTER(ctypes.c_int)]
        lib.oracle_dequant.argtypes = [ctypes.c_int, P, I64, P]
        lib.oracle_matmul.argtypes = [ctypes.c_int, P, I64, P, I64, P, I64, P, P, ctypes.c_int]
        lib.oracle_moe.argtypes = [ctypes.c_int, P, I64, I64, I64, P, I64, I64, P, ctypes.c_int,
                                   P, I64, P, P, ctypes.c_int]
        lib.oracle_max_threads.argtypes = []
        self._lib = lib
        self.path = path

    def block_geometry(self, kind) -> tuple[int, int]:
        """(block_bytes, block_elems) from the oracle's own table."""
        b, e = ctypes.c_int(), ctypes.c_int()
        if self._lib.oracle_block_geometry(_kind(kind), ctypes.byref(b), ctypes.byref(e)) != 0:
            raise KeyError(kind)
        return b.value, e.value

    def max_threads(self) -> int:
        return int(self._lib.oracle_max_threads())

    def dequant(self, kind, W) -> np.ndarray:
        """Exact (binary64) values of every element of the whole blocks in W."""
        W = np.ascontiguousarray(W, dtype=np.uint8).reshape(-1)
        bb, be = self.block_geometry(kind)
        if W.size % bb:
            raise ValueError("W is not a whole number of blocks")
        n = (W.size // bb) * be
        out = np.empty(n, dtype=np.float64)
        rc = self._lib.oracle_dequant(_kind(kind), _ptr(W), n, _ptr(out))
        if rc != 0:
            raise RuntimeError(f"oracle_dequant failed ({rc})")
        return out

    def matmul(self, kind, W, K: int, X, rows=None, threads: int = 0):
        """(y, bound), each [M][n_sel]: y = x . W^T in binary64 for the
        selected rows (all rows when ``rows`` is None), bound = sum |w||x|."""
        W = np.ascontiguousarray(W, dtype=np.uint8)
        X = _as_f64(X)
        if X.ndim == 1:
            X = X[None, :]
        M = X.shape[0]
        if X.shape[1] != K:
            raise ValueError("X has the wrong K")
        bb, be = self.block_geometry(kind)
        row_bytes = (K // be) * bb
        n_rows = W.size // row_bytes
        if rows is None:
            sel, n_sel = None, n_rows
        else:
            sel = np.ascontiguousarray(rows, dtype=np.int64)
            if sel.size and (sel.min() < 0 or sel.max() >= n_rows):
                raise IndexError("row index out of range")
            n_sel = sel.size
        Y = np.empty((M, n_sel), dtype=np.float64)
        B = np.empty((M, n_sel), dtype=np.float64)
        rc = self._lib.oracle_matmul(_kind(kind), _ptr(W), K, None if sel is None else _ptr(sel),
                                     n_sel, _ptr(X), M, _ptr(Y), _ptr(B), int(threads))
        if rc != 0:
            raise RuntimeError(f"oracle_matmul failed ({rc})")
        return Y, B

    def moe(self, kind, W, E: int, N: int, K: int, ids, X, x_per_slot: bool,
            rows=None, threads: int = 0):
        """(y, bound), each [M][topk][n_sel]: y[t][s] = W_{ids[t][s]} . x."""
        W = np.ascontiguousarray(W, dtype=np.uint8)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        M, topk = ids.shape
        X = _as_f64(X)
        if rows is None:
            sel, n_sel = None, N
        else:
            sel = np.ascontiguousarray(rows, dtype=np.int64)
            n_sel = sel.size
        Y = np.empty((M, topk, n_sel), dtype=np.float64)
        B = np.empty((M, topk, n_sel), dtype=np.float64)
        rc = self._lib.oracle_moe(_kind(kind), _ptr(W), E, N, K, _ptr(ids), M, topk, _ptr(X),
                                  1 if x_per_slot else 0, None if sel is None else _ptr(sel),
                                  n_sel, _ptr(Y), _ptr(B), int(threads))
        if rc != 0:
            raise RuntimeError(f"oracle_moe failed ({rc})")
        return Y, B


    def moe_ffn(self, kind, W_gu, W_d, E: int, N_ff: int, K: int, ids, topk_w, X, rows=None,
                threads: int = 0):
        """Routed SiLU-gated expert FFN with a weighted top-k combine, in
        binary64.  Model semantics, not on the pages (which stop at the
        routed expert products): for token t and slot s with e = ids[t][s]
        in [0, E),

            g = W_gu[e][0 : N_ff] . X[t]        (gate: the first N_ff rows)
            u = W_gu[e][N_ff : 2 N_ff] . X[t]   (up: the next N_ff rows)
            h = silu(g) * u
            y[t] += topk_w[t][s] * (W_d[e] . h)

        W_gu holds E experts of 2 N_ff rows of K elements, W_d E experts of K
        rows of N_ff elements.  A pair whose id lies outside [0, E) adds
        nothing.  ``rows`` selects output columns of y.

        Returns (y, tol), each [M][n_sel].  tol bounds |y_gpu - y| for an
        implementation whose every matmul stays within 1e-3 sum|w||x| + 1e-6
        of its exact value (the workload bar), whose SiLU-product is
        evaluated in f32 to within 2^-20 relative, and whose combine sums the
        top-k terms in f32:
            a_g = 1e-3 Bg + 1e-6, a_u likewise            (gate, up errors)
            a_h = (|silu g| + 1.1 a_g) a_u + 1.1 a_g |u|  (|silu'| < 1.1)
                  + 2^-20 (|h| + that)
            a_d = (1 + 1e-3) sum|W_d| a_h + 1e-3 sum|W_d||h| + 1e-6
            tol = sum_s |w_s| a_d + topk 2^-23 sum_s |w_s| (|d_s| + a_d)
        """
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        M, topk = ids.shape
        valid = (ids >= 0) & (ids < E)
        safe = np.where(valid, ids, 0).astype(np.int32)
        G, BG = self.moe(kind, W_gu, E, 2 * N_ff, K, safe, X, False, threads=threads)
        g, u = G[..., :N_ff], G[..., N_ff:]
        a_g = 1e-3 * BG[..., :N_ff] + 1e-6
        a_u = 1e-3 * BG[..., N_ff:] + 1e-6
        sg = silu(g)
        h = sg * u
        a_h0 = (np.abs(sg) + 1.1 * a_g) * a_u + 1.1 * a_g * np.abs(u)
        a_h = a_h0 + 2.0 ** -20 * (np.abs(h) + a_h0)
        D, BD = self.moe(kind, W_d, E, K, N_ff, safe, h, True, rows=rows, threads=threads)
        _, BA = self.moe(kind, W_d, E, K, N_ff, safe, a_h, True, rows=rows, threads=threads)
        a_d = (1.0 + 1e-3) * BA + 1e-3 * BD + 1e-6
        w = np.where(valid, np.asarray(topk_w, dtype=np.float64), 0.0)[..., None]
        y = np.sum(w * D, axis=1)
        tol = np.sum(np.abs(w) * a_d, axis=1) + topk * 2.0 ** -23 * np.sum(np.abs(w) * (np.abs(D) + a_d), axis=1)
        return y, tol


def silu(v):
    """SiLU (the sigmoid-weighted linear unit) in binary64:
    silu(v) = v / (1 + exp(-v)), evaluated as v e^v / (1 + e^v) for v < 0 so
    that neither branch overflows."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    pos = v >= 0
    out[pos] = v[pos] / (1.0 + np.exp(-v[pos]))
    e = np.exp(v[~pos])
    out[~pos] = v[~pos] * e / (1.0 + e)
    return out


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        build(force=False)
        _default = Oracle(LIBRARY)
    return _default


def block_geometry(kind):
    return default().block_geometry(kind)


def max_threads():
    return default().max_threads()


def dequant(kind, W):
    return default().dequant(kind, W)


def matmul(kind, W, K, X, rows=None, threads=0):
    return default().matmul(kind, W, K, X, rows=rows, threads=threads)


def moe(kind, W, E, N, K, ids, X, x_per_slot, rows=None, threads=0):
    return default().moe(kind, W, E, N, K, ids, X, x_per_slot, rows=rows, threads=threads)


def moe_ffn(kind, W_gu, W_d, E, N_ff, K, ids, topk_w, X, rows=None, threads=0):
    return default().moe_ffn(kind, W_gu, W_d, E, N_ff, K, ids, topk_w, X, rows=rows, threads=threads)
