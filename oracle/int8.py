"""Integer activations: per-block int8 quantization of x and the product
against it, on the CPU.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU baseline leg of ``bench.py`` may use it.  It shares no code with the HIP
library and never calls it.

The ferrox-cuda mul_mm page ("Why this shape") names the integer dot-product
path of llama.cpp's mmq (activations quantized to 8-bit integers, products on
integer dot units) and leaves it out.  The pages give no activation format
for it, so the plainest reading is taken:

* per token and 32-element block (the weight block of Q8_0, Q4_0, Q5_0,
  IQ4_NL and MXFP4, whose values are integers up to the block scale),
  amax = max |x|, the scale d = amax / 127 rounded to f32, and each code
  q = x / d rounded to f32, then to the nearest integer, ties to even;
  an all-zero block has d = 0 and q = 0;
* the product is y[t][n] = sum over blocks of d_w d_x (sum_i w_i q_i) with
  the weights' own integer codes, i.e. the exact product of W with the
  rebuilt activations d_x * q.

The quantization decides integers from floating point, so it is taken in the
precision the kernel takes it: f32, with correctly rounded division (numpy's
float32 arithmetic is IEEE).  The kernel's codes and scales therefore equal
these bit for bit, and its product can be held to f32 accumulation against
``matmul_quantized``; the difference from the exact product of the original x
is bounded by ``quantization_bound``.
"""
from __future__ import annotations

import numpy as np

from . import matmul

BLOCK = 32


def quantize(X) -> tuple[np.ndarray, np.ndarray]:
    """(q int8 [M][K], d float32 [M][K/32]) for activations X [M][K] (f32 or f16)."""
    X = np.asarray(X)
    if X.dtype not in (np.float32, np.float16):
        raise TypeError("activations must be f32 or f16")
    X = np.atleast_2d(X).astype(np.float32)  # f16 -> f32 is exact
    M, K = X.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    xb = X.reshape(M, K // BLOCK, BLOCK)
    amax = np.max(np.abs(xb), axis=2)                          # exact
    d = (amax / np.float32(127.0)).astype(np.float32)          # one f32 rounding
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (xb / d[:, :, None]).astype(np.float32)            # one f32 rounding
    q = np.where(d[:, :, None] > 0, np.rint(r), 0.0)           # ties to even
    assert np.all(np.abs(q) <= 127)
    return q.astype(np.int8).reshape(M, K), d


def rebuilt(X) -> np.ndarray:
    """d_x * q as binary64 [M][K] (exact: an f32 times an integer)."""
    q, d = quantize(X)
    M, K = q.shape
    return (q.reshape(M, K // BLOCK, BLOCK).astype(np.float64) * d.astype(np.float64)[:, :, None]).reshape(M, K)


def matmul_quantized(kind, W, K: int, X, rows=None, threads: int = 0):
    """(y_q, bound_q): the exact product of W with the rebuilt activations,
    and sum |w| |d_x q| -- the reference the int8 path is held to."""
    return matmul(kind, W, K, rebuilt(X), rows=rows, threads=threads)


def quantization_bound(kind, W, K: int, X, rows=None, threads: int = 0) -> np.ndarray:
    """sum_k |w_k| (d_x(k) / 2) (1 + 2^-16): how far the product of the
    rebuilt activations may lie from the product of X itself (rounding x / d
    to an integer moves x by at most d / 2, and the f32 quotient adds at most
    127 ulp-halves of 2^-24 relative)."""
    q, d = quantize(X)
    M, Kx = q.shape
    half = np.repeat(d.astype(np.float64) * 0.5 * (1.0 + 2.0 ** -16), BLOCK, axis=1).reshape(M, Kx)
    _, B = matmul(kind, W, K, half, rows=rows, threads=threads)
    return B
