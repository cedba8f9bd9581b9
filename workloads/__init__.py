"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the
benchmark.

This module only draws random bytes and numbers.  It holds none of the
decoding or matmul arithmetic: it knows where each kind keeps its scale
fields (so that it can give them a chosen distribution), and nothing else
about the formats.

Every random stream comes from numpy's PCG64 seeded with SeedSequence(0) and
a spawn key derived from the (workload, tensor) names, so each tensor of each
workload has its own reproducible stream.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field

import numpy as np

# GGUF type id, block bytes, block elements.
KINDS = {
    "Q8_0": (8, 34, 32),
    "Q4_0": (2, 18, 32),
    "Q5_0": (6, 22, 32),
    "Q2_K": (10, 84, 256),
    "Q3_K": (11, 110, 256),
    "Q4_K": (12, 144, 256),
    "Q5_K": (13, 176, 256),
    "Q6_K": (14, 210, 256),
    "IQ4_NL": (20, 18, 32),
    "IQ4_XS": (23, 136, 256),
    "MXFP4": (39, 17, 32),
}
KIND_NAMES = {v[0]: k for k, v in KINDS.items()}

# Byte offsets of the f16 scale fields inside a block (d, and dmin where the
# kind has one), and of the E8M0 scale byte for MXFP4.
F16_FIELDS = {
    "Q8_0": (0,), "Q4_0": (0,), "Q5_0": (0,), "Q2_K": (80, 82), "Q3_K": (108,),
    "Q4_K": (0, 2), "Q5_K": (0, 2), "Q6_K": (208,), "IQ4_NL": (0,), "IQ4_XS": (0,),
    "MXFP4": (),
}
E8M0_FIELDS = {"MXFP4": (0,)}


def name_of(kind) -> str:
    return kind if isinstance(kind, str) else KIND_NAMES[int(kind)]


def geometry(kind) -> tuple[int, int]:
    _, bb, be = KINDS[name_of(kind)]
    return bb, be


def row_bytes(kind, K: int) -> int:
    bb, be = geometry(kind)
    if K % be:
        raise ValueError(f"K={K} is not a whole number of {name_of(kind)} blocks")
    return (K // be) * bb


def rng(workload: str, tensor: str, seed: int = 0) -> np.random.Generator:
    key = (zlib.crc32(workload.encode()), zlib.crc32(tensor.encode()))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def _f16_bits(values: np.ndarray) -> np.ndarray:
    return values.astype(np.float16).view(np.uint16)


def random_weights(kind, n_rows: int, K: int, g: np.random.Generator,
                   scales: str = "config", f16_range=(1e-3, 1e-2),
                   e8m0_range=(118, 130)) -> np.ndarray:
    """[n_rows, row_bytes] uint8: uniform random bytes for every code, high
    bit and packed sub-block scale, with the block's f16 scale fields and
    E8M0 byte redrawn:

    * scales="config": f16 fields are RN_f16(U[f16_range]), positive; the
      E8M0 byte is uniform over the integers of e8m0_range (inclusive).
    * scales="stress": f16 fields take a random sign, a random 10-bit
      mantissa and an exponent field uniform in 8..22 (about 2^-7..2^7), so
      no field is zero, subnormal, Inf or NaN; the E8M0 byte is uniform over
      0..252, so every decoded MXFP4 weight (at most 6 * 2^125) is finite
      in f32.
    """
    name = name_of(kind)
    bb, be = geometry(name)
    rb = row_bytes(name, K)
    nblk = n_rows * (K // be)
    raw = g.integers(0, 256, size=(nblk, bb), dtype=np.uint8)
    for off in F16_FIELDS[name]:
        if scales == "config":
            bits = _f16_bits(g.uniform(f16_range[0], f16_range[1], size=nblk))
        elif scales == "stress":
            sign = g.integers(0, 2, size=nblk, dtype=np.uint16) << 15
            expo = g.integers(8, 23, size=nblk, dtype=np.uint16) << 10
            mant = g.integers(0, 1024, size=nblk, dtype=np.uint16)
            bits = sign | expo | mant
        else:
            raise ValueError(scales)
        raw[:, off] = (bits & 0xFF).astype(np.uint8)
        raw[:, off + 1] = (bits >> 8).astype(np.uint8)
    for off in E8M0_FIELDS.get(name, ()):
        lo, hi = e8m0_range if scales == "config" else (0, 252)
        raw[:, off] = g.integers(lo, hi + 1, size=nblk, dtype=np.int64).astype(np.uint8)
    return raw.reshape(n_rows, rb)


def activations(shape, dtype, g: np.random.Generator) -> np.ndarray:
    """Standard normal values rounded to the given dtype (f32 or f16)."""
    return g.standard_normal(size=shape).astype(dtype)


def routing(M: int, E: int, topk: int, g: np.random.Generator) -> np.ndarray:
    """[M, topk] int32: for each token, topk distinct experts uniform at
    random."""
    ids = np.empty((M, topk), dtype=np.int32)
    for t in range(M):
        ids[t] = g.choice(E, size=topk, replace=False)
    return ids


@dataclass(frozen=True)
class Matmul:
    """One weight set multiplied by one activation batch."""
    name: str
    kind: str
    M: int
    N: int
    K: int
    x_dtype: str          # "f32" or "f16"

    def weights(self, scales="config"):
        return random_weights(self.kind, self.N, self.K, rng(self.name, "W"), scales=scales)

    def x(self):
        dt = np.float32 if self.x_dtype == "f32" else np.float16
        return activations((self.M, self.K), dt, rng(self.name, "x"))

    @property
    def weight_bytes(self) -> int:
        return self.N * row_bytes(self.kind, self.K)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


@dataclass(frozen=True)
class Experts:
    """Routed expert products: E experts of a gate/up [N_gu, K_gu] and a down
    [N_d, K_d] matrix; each token is routed to topk experts."""
    name: str
    kind: str
    M: int
    E: int = 128
    topk: int = 8
    N_gu: int = 1536
    K_gu: int = 2048
    N_d: int = 2048
    K_d: int = 768
    x_dtype: str = "f16"

    def ids(self):
        return routing(self.M, self.E, self.topk, rng(self.name, "ids"))

    def w_gu(self, scales="config"):
        return random_weights(self.kind, self.E * self.N_gu, self.K_gu, rng(self.name, "W_gu"),
                              scales=scales)

    def w_d(self, scales="config"):
        return random_weights(self.kind, self.E * self.N_d, self.K_d, rng(self.name, "W_d"),
                              scales=scales)

    def x(self):
        return activations((self.M, self.K_gu), np.float16, rng(self.name, "x"))

    def h(self):
        return activations((self.M, self.topk, self.K_d), np.float16, rng(self.name, "h"))

    def touched_bytes(self, ids) -> int:
        distinct = np.unique(ids).size
        return distinct * (self.N_gu * row_bytes(self.kind, self.K_gu)
                           + self.N_d * row_bytes(self.kind, self.K_d))


# The workloads: decode GEMVs, prefill GEMMs, codebook kinds, routed experts.
C1 = [Matmul("c1_q4_0_m1", "Q4_0", 1, 4096, 4096, "f32")]
C2 = [Matmul(f"c2_{k.lower()}_m{m}", k, m, 14336, 4096, "f32")
      for k in ("Q4_K", "Q6_K") for m in (1, 8)]
C3 = [Matmul(f"c3_{k.lower()}_m512", k, 512, 4096, 4096, "f16") for k in ("Q8_0", "Q5_0")]
C4 = ([Matmul(f"c4_{k.lower()}_m1", k, 1, 11008, 4096, "f32") for k in ("IQ4_NL", "IQ4_XS", "MXFP4")]
      + [Matmul(f"c4_{k.lower()}_m256", k, 256, 11008, 4096, "f16")
         for k in ("IQ4_NL", "IQ4_XS", "MXFP4")])
C5 = [Experts(f"c5_q4_k_m{m}", "Q4_K", m) for m in (1, 16, 256)]
