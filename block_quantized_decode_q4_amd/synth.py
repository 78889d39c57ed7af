"""Seeded synthetic inputs for the Q4_K and Q6_K GEMVs (shared by the tests, the
oracle's checks and the benchmark).

This module draws random fields and places their bits in the GGUF Q4_K byte
layout; it contains none of the method's arithmetic (no decode, no scaling,
no dot product).  The field layout it writes:

  offset 0   fp16 d      (little-endian)
  offset 2   fp16 dmin   (little-endian)
  offset 4   12 bytes of packed 6-bit (sc_j, m_j), j = 0..7
  offset 16  128 bytes of 4-bit codes; in 64-element chunk c, byte 32c+i holds
             element 64c+i in its low nibble and element 64c+32+i in its high
             nibble

Scale bytes s[0..11] (GGUF K-quant packing), for j = 0..3:
  s[j]   = sc_j | (sc_{j+4} >> 4) << 6
  s[j+4] = m_j  | (m_{j+4}  >> 4) << 6
  s[j+8] = (sc_{j+4} & 15) | (m_{j+4} & 15) << 4

Workloads: the five shapes below, with the value distributions of the
problem statement -- codes uniform 0..15, 6-bit scales and mins uniform 0..63,
d and dmin drawn uniform on [1e-4, 1e-2] and rounded to fp16 (numpy's
round-to-nearest-even cast), x ~ N(0, 1) in f32.  Generator:
numpy.random.default_rng(1000 + config index) (PCG64); draw order d, dmin,
sc, m, q, x.

Q6_K (210-byte superblocks, the GGUF layout):

  offset 0    ql: 128 bytes, the low four bits of the codes
  offset 128  qh: 64 bytes, the high two bits
  offset 192  16 signed 8-bit scales, scale s for elements 16s .. 16s+15
  offset 208  fp16 d (little-endian)

Element e = 128h + 32t + l (h < 2, t < 4, l < 32) keeps its low bits in ql
byte 64h + 32(t % 2) + l (low nibble for t < 2, high nibble for t >= 2) and
its high bits in bits 2t, 2t+1 of qh byte 32h + l.  Q6_K workloads: codes
uniform 0..63, scales uniform -128..127, d uniform on [2e-6, 2e-4] rounded
to fp16 (about a quarter of them fp16 subnormals, as in quantized weights
of that size), x ~ N(0, 1); numpy.random.default_rng(2000 + index), draw
order d, sc, q, x.  Rows may be placed at a row stride (bytes) above the
dense 210 k / 256, the padding bytes zero.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

QK = 256
SB_BYTES = 144


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    n: int
    k: int
    m: int

    @property
    def S(self) -> int:
        return self.k // QK

    @property
    def weight_bytes(self) -> int:
        return self.n * self.S * SB_BYTES


# The five shapes: a smoke case, the 7B attention projection, the 7B FFN-down
# projection (k above a 12288-float single-stage x tile), the 32000-row LM
# head and an m = 8 small-batch decode over the FFN gate/up shape.
WORKLOADS = (
    Workload(0, "q4k_gemv_n256_k1024_m1", 256, 1024, 1),
    Workload(1, "q4k_gemv_attn_proj_n4096_k4096_m1", 4096, 4096, 1),
    Workload(2, "q4k_gemv_ffn_down_n4096_k14336_m1", 4096, 14336, 1),
    Workload(3, "q4k_gemv_lm_head_n32000_k4096_m1", 32000, 4096, 1),
    Workload(4, "q4k_gemv_batched_n14336_k4096_m8", 14336, 4096, 8),
)


@dataclass
class Fields:
    """Per-superblock fields, shapes (n, S), (n, S), (n, S, 8), (n, S, 8),
    (n, S, 256); q is indexed by element position inside the superblock."""
    d_bits: np.ndarray
    dmin_bits: np.ndarray
    sc: np.ndarray
    m: np.ndarray
    q: np.ndarray


def draw_fields(rng: np.random.Generator, n: int, S: int,
                d_range=(1e-4, 1e-2)) -> Fields:
    d = rng.uniform(d_range[0], d_range[1], size=(n, S)).astype(np.float16)
    dmin = rng.uniform(d_range[0], d_range[1], size=(n, S)).astype(np.float16)
    sc = rng.integers(0, 64, size=(n, S, 8), dtype=np.uint8)
    mn = rng.integers(0, 64, size=(n, S, 8), dtype=np.uint8)
    q = rng.integers(0, 16, size=(n, S, QK), dtype=np.uint8)
    return Fields(d.view(np.uint16), dmin.view(np.uint16), sc, mn, q)


def pack(f: Fields) -> np.ndarray:
    """Place the fields' bits in the 144-byte superblock layout.
    Returns uint8 [n * S * 144]."""
    n, S = f.d_bits.shape
    out = np.zeros((n, S, SB_BYTES), dtype=np.uint8)
    d = f.d_bits.astype(np.uint16)
    dm = f.dmin_bits.astype(np.uint16)
    out[:, :, 0] = (d & 0xFF).astype(np.uint8)
    out[:, :, 1] = (d >> 8).astype(np.uint8)
    out[:, :, 2] = (dm & 0xFF).astype(np.uint8)
    out[:, :, 3] = (dm >> 8).astype(np.uint8)
    sc = f.sc.astype(np.uint8)
    mn = f.m.astype(np.uint8)
    lo_sc, hi_sc = sc[:, :, 0:4], sc[:, :, 4:8]
    lo_m, hi_m = mn[:, :, 0:4], mn[:, :, 4:8]
    out[:, :, 4:8] = lo_sc | ((hi_sc >> 4) << 6)
    out[:, :, 8:12] = lo_m | ((hi_m >> 4) << 6)
    out[:, :, 12:16] = (hi_sc & 0x0F) | ((hi_m & 0x0F) << 4)
    q = f.q.astype(np.uint8).reshape(n, S, 4, 2, 32)      # [chunk][nibble][byte]
    qs = q[:, :, :, 0, :] | (q[:, :, :, 1, :] << 4)        # (n, S, 4, 32)
    out[:, :, 16:144] = qs.reshape(n, S, 128)
    return out.reshape(-1)


def make_inputs(n: int, k: int, m: int, seed: int, d_range=(1e-4, 1e-2)):
    """Weights (packed bytes, uint8 [n*(k/256)*144]) and x (float32 [m, k])."""
    if k % QK != 0 or k <= 0 or n <= 0 or m <= 0:
        raise ValueError("bad shape")
    rng = np.random.default_rng(seed)
    f = draw_fields(rng, n, k // QK, d_range)
    w = pack(f)
    x = rng.standard_normal((m, k), dtype=np.float32)
    return w, x


def workload_inputs(index: int):
    wl = WORKLOADS[index]
    w, x = make_inputs(wl.n, wl.k, wl.m, seed=1000 + index)
    return wl, w, x


# ----------------------------------------------------------------- Q6_K
Q6K_SB_BYTES = 210

# An LM head stored as Q6_K (the 32000 x 4096 head), the FFN-down shape, and
# a small case.
Q6K_WORKLOADS = (
    Workload(0, "q6k_gemv_n256_k1024_m1", 256, 1024, 1),
    Workload(1, "q6k_gemv_lm_head_n32000_k4096_m1", 32000, 4096, 1),
    Workload(2, "q6k_gemv_ffn_down_n4096_k14336_m1", 4096, 14336, 1),
)


@dataclass
class Q6Fields:
    """Per-superblock fields, shapes (n, S), (n, S, 16), (n, S, 256); q is
    indexed by element position inside the superblock."""
    d_bits: np.ndarray
    sc: np.ndarray
    q: np.ndarray


def draw_q6k_fields(rng: np.random.Generator, n: int, S: int,
                    d_range=(2e-6, 2e-4)) -> Q6Fields:
    d = rng.uniform(d_range[0], d_range[1], size=(n, S)).astype(np.float16)
    sc = rng.integers(-128, 128, size=(n, S, 16), dtype=np.int16).astype(np.int8)
    q = rng.integers(0, 64, size=(n, S, QK), dtype=np.uint8)
    return Q6Fields(d.view(np.uint16), sc, q)


def q6k_row_bytes(k: int) -> int:
    return (k // QK) * Q6K_SB_BYTES


def pack_q6k(f: Q6Fields, row_stride: int = 0) -> np.ndarray:
    """Place the fields' bits in the 210-byte superblock layout, row r at
    byte r * row_stride (0: dense).  Returns uint8 [n * row_stride]."""
    n, S = f.d_bits.shape
    q = f.q.astype(np.uint8).reshape(n, S, 2, 4, 32)       # [h][t][l]
    lo = q & 0x0F
    hi = q >> 4
    blk = np.zeros((n, S, Q6K_SB_BYTES), dtype=np.uint8)
    # ql: per half, 32 bytes for t = 0 | t = 2 (high nibble), then 32 for
    # t = 1 | t = 3
    ql = np.stack([lo[:, :, :, 0, :] | (lo[:, :, :, 2, :] << 4),
                   lo[:, :, :, 1, :] | (lo[:, :, :, 3, :] << 4)], axis=3)   # (n, S, 2, 2, 32)
    blk[:, :, 0:128] = ql.reshape(n, S, 128)
    qh = (hi[:, :, :, 0, :] | (hi[:, :, :, 1, :] << 2) | (hi[:, :, :, 2, :] << 4)
          | (hi[:, :, :, 3, :] << 6))                                       # (n, S, 2, 32)
    blk[:, :, 128:192] = qh.reshape(n, S, 64)
    blk[:, :, 192:208] = f.sc.astype(np.int8).view(np.uint8)
    d = f.d_bits.astype(np.uint16)
    blk[:, :, 208] = (d & 0xFF).astype(np.uint8)
    blk[:, :, 209] = (d >> 8).astype(np.uint8)
    dense = S * Q6K_SB_BYTES
    stride = dense if row_stride == 0 else int(row_stride)
    if stride < dense:
        raise ValueError("row_stride below the row's bytes")
    out = np.zeros((n, stride), dtype=np.uint8)
    out[:, :dense] = blk.reshape(n, dense)
    return out.reshape(-1)


def make_q6k_inputs(n: int, k: int, m: int, seed: int, row_stride: int = 0,
                    d_range=(2e-6, 2e-4)):
    """Q6_K weights (packed bytes) and x (float32 [m, k])."""
    if k % QK != 0 or k <= 0 or n <= 0 or m <= 0:
        raise ValueError("bad shape")
    rng = np.random.default_rng(seed)
    f = draw_q6k_fields(rng, n, k // QK, d_range)
    w = pack_q6k(f, row_stride)
    x = rng.standard_normal((m, k), dtype=np.float32)
    return w, x


def q6k_workload_inputs(index: int, row_stride: int = 0):
    wl = Q6K_WORKLOADS[index]
    w, x = make_q6k_inputs(wl.n, wl.k, wl.m, seed=2000 + index, row_stride=row_stride)
    return wl, w, x
