"""Seeded inputs at the edges of the arithmetic (test infrastructure).

Each case is weights (packed Q4_K bytes), x (f32 [m, k]) and a description,
built from synth's seeded draws with chosen fields or x values placed by hand.
No method arithmetic happens here: fields are set to integers and powers of
two whose relations are stated, and the oracle computes every expected value.
Used by the CPU model tests and by the GPU parity tests, so the kernels meet
the same inputs.

strict_kind is False only where d or dmin is +-inf or NaN: the kernels then
return NaN or an infinity where the exact value is NaN or an infinity, but
not necessarily the same one.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from block_quantized_decode_q4_amd import synth


@dataclass
class Case:
    name: str
    w: np.ndarray
    x: np.ndarray
    n: int
    k: int
    strict_kind: bool = True

    @property
    def m(self) -> int:
        return self.x.shape[0]


def _fields(seed, n, S):
    return synth.draw_fields(np.random.default_rng(seed), n, S)


def tiny_x(n=64, k=2048):
    """x = N(0,1) * 2^-122: most values are f32 subnormals or just above."""
    rng = np.random.default_rng(501)
    w = synth.pack(_fields(502, n, k // 256))
    x = (rng.standard_normal((2, k)) * 2.0 ** -122).astype(np.float32)
    return Case("x N(0,1)*2^-122", w, x, n, k)


def subnormal_x(n=64, k=2048):
    """Every x an f32 subnormal (random significand bits and sign)."""
    rng = np.random.default_rng(503)
    w = synth.pack(_fields(504, n, k // 256))
    bits = rng.integers(1, 1 << 23, size=(2, k), dtype=np.uint32)
    bits |= (rng.integers(0, 2, size=(2, k), dtype=np.uint32) << 31)
    return Case("x subnormal", w, bits.view(np.float32), n, k)


def huge_x(n=64, k=2048):
    """x = N(0,1) * 2^120: products exceed the f32 range, y does not."""
    rng = np.random.default_rng(505)
    w = synth.pack(_fields(506, n, k // 256))
    x = (rng.standard_normal((2, k)) * 2.0 ** 120).astype(np.float32)
    return Case("x N(0,1)*2^120", w, x, n, k)


def overflow_y(n=32, k=2048):
    """x near the top of the f32 range with positive weights only (dmin = 0):
    most y exceed it and must be infinities of the right sign."""
    rng = np.random.default_rng(507)
    f = _fields(508, n, k // 256)
    f.dmin_bits[:] = 0
    f.d_bits[:] = np.float16(4.0).view(np.uint16)
    w = synth.pack(f)
    x = np.full((2, k), 2.0 ** 126, np.float32)
    x[1] = -x[1]
    x[:, : k // 2] *= rng.uniform(0.5, 1.0, size=(2, k // 2)).astype(np.float32)
    return Case("y beyond the f32 range", w, x, n, k)


def mixed_subblock(n=48, k=1024, rest="ones"):
    """One sub-block per row where x_0 = 2^23 sits on a zero weight (q = 0,
    m_j = 0) and the other 31 elements are 1.0 (or N(0,1)); every other x is
    0, so that sub-block alone makes y and its bound."""
    rng = np.random.default_rng(509)
    S = k // 256
    f = _fields(510, n, S)
    f.m[:, 0, 0] = 0
    f.q[:, 0, 0] = 0
    w = synth.pack(f)
    x = np.zeros((2, k), np.float32)
    if rest == "ones":
        x[:, 1:32] = 1.0
    else:
        x[:, 1:32] = rng.standard_normal((2, 31)).astype(np.float32)
    x[:, 0] = 2.0 ** 23
    x[1, 0] = -x[1, 0]
    return Case("x_0 = 2^23 over a zero weight, rest %s" % rest, w, x, n, k)


def outliers(n=64, k=4096, big=2.0e4):
    """One activation outlier of +-2e4 per superblock, on a zero weight of
    every row (q = 0, m_j = 0 there); other x N(0,1)."""
    rng = np.random.default_rng(511)
    S = k // 256
    f = _fields(512, n, S)
    pos = rng.integers(0, 256, size=S)
    for s in range(S):
        f.q[:, s, pos[s]] = 0
        f.m[:, s, pos[s] // 32] = 0
    w = synth.pack(f)
    x = rng.standard_normal((2, k)).astype(np.float32)
    for s in range(S):
        x[:, 256 * s + pos[s]] = big * (1 if s % 2 == 0 else -1)
    return Case("outlier %.0e per superblock on zero weights" % big, w, x, n, k)


def zero_bound(n=32, k=2048):
    """Every weight exactly zero with nonzero scale terms: d = dmin, every
    code of sub-block j equal to q*_j and m_j = sc_j * q*_j (<= 63), so
    d*sc_j*q - dmin*m_j = 0 for every element.  y must be +-0."""
    rng = np.random.default_rng(513)
    S = k // 256
    f = _fields(514, n, S)
    f.dmin_bits[:] = f.d_bits
    qstar = rng.integers(1, 8, size=(n, S, 8))
    sc = rng.integers(1, 64, size=(n, S, 8)) // qstar
    sc = np.maximum(sc, 1)
    f.sc[:] = sc
    f.m[:] = sc * qstar
    f.q[:] = np.repeat(qstar, 32, axis=2)
    w = synth.pack(f)
    x = rng.standard_normal((2, k)).astype(np.float32) * np.float32(1000.0)
    return Case("all weights zero, scale terms not", w, x, n, k)


def near_zero_bound(n=32, k=2048):
    """As zero_bound, but one code per sub-block differs from q*_j by one:
    the only nonzero weights (+-d*sc_j) sit among exactly cancelling ones."""
    c = zero_bound(n, k)
    rng = np.random.default_rng(515)
    S = k // 256
    b = c.w.reshape(n, S, 144).copy()
    for r in range(n):
        for s in range(S):
            byte = int(rng.integers(0, 128))
            hi = int(rng.integers(0, 2))
            v = int(b[r, s, 16 + byte])
            q = (v >> 4) if hi else (v & 15)
            q2 = q + 1 if q < 15 else q - 1
            v = (v & 0x0F) | (q2 << 4) if hi else (v & 0xF0) | q2
            b[r, s, 16 + byte] = v
    return Case("cancelling weights plus one nonzero weight per sub-block", b.reshape(-1), c.x,
                n, k)


def nonfinite_x(n=40, k=2048):
    """+inf, -inf and NaN in x (vector 0: one +inf; 1: +inf and -inf; 2: one
    NaN; 3: +inf next to values of every magnitude); some rows have zero
    weights under the infinity (0 * inf = NaN)."""
    rng = np.random.default_rng(517)
    S = k // 256
    f = _fields(518, n, S)
    f.q[: n // 4, 0, 5] = 0
    f.m[: n // 4, 0, 0] = 0
    w = synth.pack(f)
    x = rng.standard_normal((4, k)).astype(np.float32)
    x[0, 5] = np.inf
    x[1, 5] = np.inf
    x[1, 300] = -np.inf
    x[2, 700] = np.nan
    x[3, 5] = np.inf
    x[3, 6] = 1e-30
    x[3, 7] = 1e30
    return Case("inf and NaN in x", w, x, n, k)


def nonfinite_header(n=48, k=1024):
    """+-inf and NaN as d or dmin in some superblocks (every weight there is
    then NaN or an infinity), other rows ordinary."""
    S = k // 256
    f = _fields(520, n, S)
    specials = [0x7C00, 0xFC00, 0x7E00, 0x7C01]
    for i, sp in enumerate(specials):
        f.d_bits[i, 1] = sp
        f.dmin_bits[8 + i, 2] = sp
    f.sc[1, 1, :] = 0            # inf * 0 inside d * sc
    f.m[9, 2, :] = 0
    w = synth.pack(f)
    x = np.random.default_rng(519).standard_normal((2, k)).astype(np.float32)
    return Case("inf and NaN as d or dmin", w, x, n, k, strict_kind=False)


def wide_magnitudes(n=48, k=2048):
    """x = N(0,1) * 2^u, u uniform on -40..40 per element: most elements sit
    far below their sub-block's largest, so most columns hold many values
    that need their exact terms (more than a short list holds)."""
    rng = np.random.default_rng(521)
    w = synth.pack(_fields(522, n, k // 256))
    x = (rng.standard_normal((2, k)) * np.exp2(rng.integers(-40, 41, size=(2, k)))).astype(np.float32)
    return Case("x N(0,1) * 2^(-40..40)", w, x, n, k)


def few_small(n=48, k=2048):
    """N(0,1) x where column c (of eight) holds c elements of size 1e-12:
    zero up to seven values that the grid leaves out per column."""
    rng = np.random.default_rng(523)
    w = synth.pack(_fields(524, n, k // 256))
    x = rng.standard_normal((2, k)).astype(np.float32)
    for c in range(k // 256):
        pos = rng.choice(256, size=c, replace=False)
        x[:, 256 * c + pos] = np.float32(1e-12)
    return Case("N(0,1) x with 0..7 tiny values per column", w, x, n, k)


def all_cases():
    return [tiny_x(), subnormal_x(), huge_x(), overflow_y(), mixed_subblock(),
            mixed_subblock(rest="normal"), outliers(), outliers(big=3.0e9), zero_bound(),
            near_zero_bound(), nonfinite_x(), nonfinite_header(), wide_magnitudes(), few_small()]
