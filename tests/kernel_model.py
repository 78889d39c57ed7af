"""CPU model of the integer kernels' arithmetic (test infrastructure).

A numpy restatement of what the line-streamed integer kernels (3, 5, 6)
compute, used on the CPU to check their error analysis against the oracle
on inputs the workloads never produce.  It models the kernels, not the
method: the oracle stays the reference.

x representation, per 32-element sub-block of one vector:
  * mx = largest |x| (NaN left out); sigma = 30 - E for mx = f * 2^E, f in
    [1/2, 1) (so mx * 2^sigma lies in [2^29, 2^30)), 0 when mx = 0, 30 when
    mx is infinite (frexp gives it exponent 0);
  * v = x * 2^sigma (exact in f32 for every element that is not rounded to
    zero), xi = rint(v) (round to nearest even), |xi| < 2^30, written as four
    signed base-256 digits (the bytes of xi + 0x80808080, each minus 128);
  * an element is certified when x = 0 or 2^16 <= |x 2^sigma| <= 2^30
    (then |v - xi| <= 1/2 <= 2^-17 |v|); an uncertified element (a value
    below 2^-13 of the sub-block's largest, inf, NaN) is left out of the
    digits (xi := 0);
  * per sub-block constants: s = 2^-sigma (f64) and XI = sum xi (exact
    integer, certified elements only).

Per (row, sub-block) with D = d*sc_j and M = dmin*m_j (exact in f32):
  * T = sum q xi (exact integer from digit sums: low codes q, high codes
    16 q - 128 then T = (T' + 128 XI) / 16), then in f64 p1 = D*T,
    e1 = D*T - p1 (exact product error), p2 = M*XI (exact),
    r = (p1 - p2) + e1, contribution r * s;
  * every uncertified element adds fl32(D q_e - M) * x_e in f64 (its exact
    weight against its exact x).
A row's contributions add up in f64; y is that sum rounded once to f32.

Error (finite inputs): each certified element's x error is at most
2^-17 |x_e|, the weights differ from the exact D q - M by at most 2^-24 |w|,
the f64 steps add about 2^-52 of sum |w||x|, the final rounding 2^-24 |y|:
|y - y_ref| <= (2^-17 + 2^-23 + 2^-50) sum|w||x| < 1e-5 sum|w||x|.
"""
from __future__ import annotations

import numpy as np

CERT_REL = 2.0 ** -17


def two_prod(a: np.ndarray, b: np.ndarray):
    """p = fl(a*b) and the exact error e = a*b - p (f64, Dekker's product;
    exact barring overflow)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    p = a * b
    split = 134217729.0            # 2^27 + 1
    with np.errstate(invalid="ignore", over="ignore"):
        ta = split * a
        ah = ta - (ta - a)
        al = a - ah
        tb = split * b
        bh = tb - (tb - b)
        bl = b - bh
        e = ((ah * bh - p) + ah * bl + al * bh) + al * bl
    return p, e


class XRep:
    """The x representation of one vector: arrays over its k/32 sub-blocks."""

    def __init__(self, x: np.ndarray):
        xs = np.asarray(x, np.float32).reshape(-1, 32)
        self.x = xs
        finite = np.isfinite(xs)
        a = np.where(np.isnan(xs), np.float32(0), np.abs(xs))
        mx = a.max(axis=1)
        _, E = np.frexp(mx)             # an infinite mx: exponent 0, sigma = 30
        self.sigma = np.where(mx > 0, 30 - E, 0).astype(np.int64)
        with np.errstate(invalid="ignore", over="ignore"):
            v = np.ldexp(np.where(finite, xs, np.float32(0)), self.sigma[:, None].astype(np.int32))
        v = v.astype(np.float32)
        xi = np.rint(v).astype(np.float32)
        a = np.abs(np.ldexp(xs, self.sigma[:, None].astype(np.int32)).astype(np.float32))
        cert = ((a >= 65536.0) & (a <= 2.0 ** 30)) | (xs == 0)
        self.cert = cert
        self.xi = np.where(cert, xi, 0).astype(np.int64)
        assert np.all(np.abs(self.xi) < 2 ** 30)
        self.dirty = ~cert.all(axis=1)          # sub-blocks with an uncertified element
        self.uncertified = int((~cert).sum())
        self.XI = self.xi.sum(axis=1)
        self.s = np.ldexp(1.0, -self.sigma)
        u = (self.xi + 0x80808080).astype(np.uint64)
        assert np.all(u < 2 ** 32)
        self.digits = np.stack([((u >> (8 * l)) & 0xFF).astype(np.int64) - 128
                                for l in range(4)], axis=-1)       # [nsb, 32, 4]


def decode_fields(w: np.ndarray, n: int, k: int):
    """(d, dmin) as f32 [n, S] and (sc, m) [n, S, 8], codes q [n, S, 256]
    (element order), from the packed bytes."""
    S = k // 256
    b = np.asarray(w, np.uint8).reshape(n, S, 144)
    d = b[:, :, 0:2].copy().view(np.float16)[:, :, 0].astype(np.float32)
    dmin = b[:, :, 2:4].copy().view(np.float16)[:, :, 0].astype(np.float32)
    s = b[:, :, 4:16].astype(np.int64)
    sc = np.zeros((n, S, 8), np.int64)
    mn = np.zeros((n, S, 8), np.int64)
    for j in range(4):
        sc[:, :, j] = s[:, :, j] & 63
        mn[:, :, j] = s[:, :, j + 4] & 63
        sc[:, :, j + 4] = (s[:, :, j + 8] & 15) | ((s[:, :, j] >> 6) << 4)
        mn[:, :, j + 4] = (s[:, :, j + 8] >> 4) | ((s[:, :, j + 4] >> 6) << 4)
    qs = b[:, :, 16:144].reshape(n, S, 4, 32).astype(np.int64)
    q = np.stack([qs & 15, qs >> 4], axis=3).reshape(n, S, 256)
    return d, dmin, sc, mn, q


def gemv(w: np.ndarray, x: np.ndarray, n: int):
    """y [m, n] (f32) as the integer kernels compute it; also the number of
    dirty sub-blocks per vector."""
    x = np.asarray(x, np.float32)
    if x.ndim == 1:
        x = x[None, :]
    m, k = x.shape
    S = k // 256
    d, dmin, sc, mn, q = decode_fields(w, n, k)
    D = (d[:, :, None] * sc.astype(np.float32)).astype(np.float32)        # exact
    M = (dmin[:, :, None] * mn.astype(np.float32)).astype(np.float32)     # exact
    qsb = q.reshape(n, S, 8, 32)
    y = np.empty((m, n), np.float32)
    dirty = []
    for b in range(m):
        rep = XRep(x[b])
        dirty.append(int(rep.dirty.sum()))
        dig = rep.digits.reshape(S, 8, 32, 4)
        XI = rep.XI.reshape(S, 8).astype(np.float64)
        s = rep.s.reshape(S, 8)
        # digit sums: low sub-blocks (even j) with q, high (odd j) with 16q - 128
        hi = (np.arange(8) % 2 == 1)[None, None, :, None]
        code = np.where(hi, 16 * qsb - 128, qsb)                              # [n,S,8,32]
        Tl = np.einsum("nsje,sjel->nsjl", code, dig)                          # exact ints
        Tp = (Tl * (256 ** np.arange(4))).sum(axis=-1)                        # sum code*xi
        xi_sum = rep.xi.reshape(S, 8, 32).sum(axis=-1)                        # digits' own sum
        T = np.where(hi[..., 0], (Tp + 128 * xi_sum[None]) // 16, Tp).astype(np.float64)
        assert np.all(np.abs(T) < 2.0 ** 53)
        with np.errstate(invalid="ignore", over="ignore"):
            p1, e1 = two_prod(D, T)
            p2 = M.astype(np.float64) * XI[None]
            r = (p1 - p2) + e1
            acc = (r * s[None]).sum(axis=(1, 2))
            # uncertified elements: exact weights against exact x
            if rep.uncertified:
                xs = rep.x.reshape(S, 8, 32)
                unc = ~rep.cert.reshape(S, 8, 32)
                w32 = (D[..., None] * qsb.astype(np.float32) - M[..., None]).astype(np.float32)
                prod = w32.astype(np.float64) * np.where(unc, xs, 0)[None].astype(np.float64)
                acc = acc + np.where(unc[None], prod, 0.0).sum(axis=(1, 2, 3))
        y[b] = acc.astype(np.float32)
    return y, dirty
