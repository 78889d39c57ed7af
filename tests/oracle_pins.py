"""Pin checks of the CPU oracle against facts fixed outside it (CPU only).

Each test checks the oracle against something other than itself: numpy's
binary16 conversion, a hand-worked superblock, bytes placed by hand from the
layout, closed forms, exact rational arithmetic and a quantizer round-trip.
Together they are chosen so that a dropped term, a wrong sign, a swapped
nibble or sub-block index, or a transposed scale/min fails at least one test
(test_oracle_mutations.py plants such mistakes in a copy of the oracle and
checks exactly that).  test_oracle_pins.py runs every check on the oracle.
"""
from fractions import Fraction
import os

import numpy as np

from block_quantized_decode_q4_amd import synth  # seeded generator: draws and bit placement only

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers
def f32bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def block_bytes(d_bits, dmin_bits, s12, qs128):
    """Place header and quants at the offsets of the layout (0, 2, 4, 16)."""
    b = np.zeros(144, dtype=np.uint8)
    b[0] = d_bits & 0xFF
    b[1] = d_bits >> 8
    b[2] = dmin_bits & 0xFF
    b[3] = dmin_bits >> 8
    b[4:16] = np.asarray(s12, dtype=np.uint8)
    b[16:144] = np.asarray(qs128, dtype=np.uint8)
    return b


def scale_bytes_single(j, field):
    """Twelve scale bytes with exactly one 6-bit field equal to 1: sc_j
    (field='sc') or m_j (field='m'); placed by hand from the bit table."""
    s = np.zeros(12, dtype=np.uint8)
    if field == "sc":
        if j < 4:
            s[j] = 1                 # low six bits of s[j]
        else:
            s[j + 4] = 0x01          # low nibble of s[j+4]
    else:
        if j < 4:
            s[j + 4] = 1             # low six bits of s[j+4]
        else:
            s[j + 4] = 0x10          # high nibble of s[j+4]
    return s


def element_of(c, hi, i):
    return 64 * c + 32 * hi + i


F16_ONE = 0x3C00
F16_HALF = 0x3800


# ------------------------------------------------------- binary16 decoding
def check_f16_decode_exhaustive_matches_numpy(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle_mod.f16_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan_ours = np.isnan(ours)
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ours, nan_ref)
    keep = ~nan_ref
    assert np.array_equal(f32bits(ours[keep]), f32bits(ref[keep]))
    # spot values from the definition
    assert oracle_mod.f16_to_f32([0x0001])[0] == 2.0 ** -24
    assert oracle_mod.f16_to_f32([0x03FF])[0] == 1023 * 2.0 ** -24
    assert oracle_mod.f16_to_f32([0x0400])[0] == 2.0 ** -14
    assert oracle_mod.f16_to_f32([0x7BFF])[0] == 65504.0
    assert oracle_mod.f16_to_f32([0xC000])[0] == -2.0
    assert np.isinf(oracle_mod.f16_to_f32([0xFC00])[0]) and oracle_mod.f16_to_f32([0xFC00])[0] < 0
    assert f32bits(oracle_mod.f16_to_f32([0x8000]))[0] == 0x80000000


def check_f16_encode_rne_matches_numpy(oracle_mod):
    rng = np.random.default_rng(7)
    # random bit patterns across the whole float32 range plus the binary16
    # boundaries and every exact tie between neighbouring binary16 values
    vals = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    f16 = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    ties = ((f16[:-1] + f16[1:]) / 2).astype(np.float32)
    extra = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 2.0 ** -25, 2.0 ** -26, 3 * 2.0 ** -26,
                      np.inf, -np.inf, 1e-4, 1e-2], dtype=np.float32)
    allv = np.concatenate([vals, ties, -ties, extra])
    ours = oracle_mod.f32_to_f16_rne(allv)
    with np.errstate(over="ignore"):
        ref = allv.astype(np.float16).view(np.uint16)
    isn = np.isnan(allv)
    assert np.array_equal(ours[~isn], ref[~isn])
    assert np.all(np.isnan(ours[isn].view(np.float16)))


# ------------------------------------------------------------ scale bytes
def check_scale_unpack_handworked_golden(oracle_mod):
    header, sc, m, _, _ = load_golden()
    got_sc, got_m = oracle_mod.unpack_scales(header[4:16])
    assert got_sc.tolist() == sc
    assert got_m.tolist() == m


def check_scale_pack_unpack_exhaustive(oracle_mod):
    """Every (sc, m) pair at every j, with the other fields random, survives
    pack -> unpack; the oracle's packer and the generator's packer (two
    independent writings of the table) give identical bytes."""
    rng = np.random.default_rng(11)
    for j in range(8):
        for sc_v in range(64):
            others_sc = rng.integers(0, 64, size=(64, 8), dtype=np.uint8)
            others_m = rng.integers(0, 64, size=(64, 8), dtype=np.uint8)
            others_sc[:, j] = sc_v
            others_m[:, j] = np.arange(64, dtype=np.uint8)
            # generator packer, vectorised over the 64 m values
            f = synth.Fields(np.zeros((64, 1), np.uint16), np.zeros((64, 1), np.uint16),
                             others_sc.reshape(64, 1, 8), others_m.reshape(64, 1, 8),
                             np.zeros((64, 1, 256), np.uint8))
            gen = synth.pack(f).reshape(64, 144)[:, 4:16]
            for t in range(64):
                s = oracle_mod.pack_scales(others_sc[t], others_m[t])
                assert np.array_equal(s, gen[t])
                usc, um = oracle_mod.unpack_scales(s)
                assert np.array_equal(usc, others_sc[t])
                assert np.array_equal(um, others_m[t])


def check_scale_single_field_by_hand(oracle_mod):
    """One 6-bit field set to 1 via bytes placed by hand; only that field is 1."""
    for j in range(8):
        for field in ("sc", "m"):
            sc, m = oracle_mod.unpack_scales(scale_bytes_single(j, field))
            exp_sc = np.zeros(8, np.uint8)
            exp_m = np.zeros(8, np.uint8)
            (exp_sc if field == "sc" else exp_m)[j] = 1
            assert np.array_equal(sc, exp_sc), (j, field)
            assert np.array_equal(m, exp_m), (j, field)
    # top bits: s[0..3] bits 6-7 feed sc_4..sc_7 bits 4-5, s[4..7] feed m_4..m_7
    for j in range(4):
        s = np.zeros(12, np.uint8)
        s[j] = 0xC0
        sc, m = oracle_mod.unpack_scales(s)
        assert sc[j] == 0 and sc[j + 4] == 48 and m.sum() == 0
        s = np.zeros(12, np.uint8)
        s[j + 4] = 0x80
        sc, m = oracle_mod.unpack_scales(s)
        assert m[j] == 0 and m[j + 4] == 32 and sc.sum() == 0


# --------------------------------------------------------- golden block
def load_golden():
    header = []
    qs = []
    sc = m = None
    w = []
    with open(os.path.join(GOLDEN, "q4k_superblock_handbuilt.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            if key == "header":
                header = [int(t, 16) for t in val.split()]
            elif key == "qs":
                qs += [int(t, 16) for t in val.split()]
            elif key == "sc":
                sc = [int(t) for t in val.split()]
            elif key == "m":
                m = [int(t) for t in val.split()]
            elif key == "w":
                e, v = val.split()
                w.append((int(e), float(v)))
    blk = np.array(header + qs, dtype=np.uint8)
    assert blk.size == 144
    return blk, sc, m, w, qs


def check_golden_handbuilt_superblock(oracle_mod):
    blk, _, _, w, _ = load_golden()
    out = oracle_mod.dequant_superblock(blk)
    for e, v in w:
        assert out[e] == np.float32(v), (e, out[e], v)


def check_golden_superblock_through_gemv(oracle_mod):
    """x = e_i picks out weight i: the GEMV path agrees with the hand values."""
    blk, _, _, w, _ = load_golden()
    x = np.zeros((len(w), 256), np.float32)
    for t, (e, _) in enumerate(w):
        x[t, e] = 1.0
    y, bound = oracle_mod.gemv(blk, x, n=1)
    for t, (e, v) in enumerate(w):
        assert y[t, 0] == v
        assert bound[t, 0] == abs(v)


# ---------------------------------------------------------- layout, one-hot
def check_onehot_scale_layout_bruteforce(oracle_mod, js=range(8)):
    """d=1, dmin=0, sc_j=1 and every other scale 0: w equals the 4-bit code on
    sub-block j and 0 elsewhere.  All 16 codes at every position."""
    for j in js:
        s12 = scale_bytes_single(j, "sc")
        c, hi = j // 2, j % 2
        for v in range(16):
            qs = np.zeros(128, np.uint8)
            # code v in the nibble of sub-block j for every byte of chunk c,
            # and code 15-v in the other nibble of every byte
            other = 15 - v
            for cc in range(4):
                for i in range(32):
                    lo_code = v if (cc == c and hi == 0) else other
                    hi_code = v if (cc == c and hi == 1) else other
                    qs[32 * cc + i] = lo_code | (hi_code << 4)
            out = oracle_mod.dequant_superblock(block_bytes(F16_ONE, 0, s12, qs))
            expect = np.zeros(256, np.float32)
            for i in range(32):
                expect[element_of(c, hi, i)] = v
            assert np.array_equal(out, expect), (j, v)


def check_onehot_min_layout_bruteforce(oracle_mod, js=range(8)):
    """q=0, dmin=1, m_j=1 and every other min 0: w = -1 on sub-block j only."""
    for j in js:
        s12 = scale_bytes_single(j, "m")
        out = oracle_mod.dequant_superblock(block_bytes(F16_ONE, F16_ONE, s12, np.zeros(128, np.uint8)))
        expect = np.zeros(256, np.float32)
        c, hi = j // 2, j % 2
        for i in range(32):
            expect[element_of(c, hi, i)] = -1.0
        assert np.array_equal(out, expect), j


def check_position_map_every_byte(oracle_mod):
    """Each byte of the 128 quant bytes is decoded at the positions the layout
    names: a distinct code pattern per byte, all scales 1, dmin 0."""
    s12 = np.zeros(12, np.uint8)
    s12[0:4] = 1                                  # sc_0..sc_3 = 1
    s12[8:12] = 0x01                              # sc_4..sc_7 = 1 (low nibbles)
    rng = np.random.default_rng(3)
    for _ in range(8):
        qs = rng.integers(0, 256, size=128, dtype=np.uint8)
        out = oracle_mod.dequant_superblock(block_bytes(F16_ONE, 0, s12, qs))
        for c in range(4):
            for i in range(32):
                b = int(qs[32 * c + i])
                assert out[64 * c + i] == (b & 15)
                assert out[64 * c + 32 + i] == (b >> 4)


# ------------------------------------------------------------ closed forms
def check_closed_form_uniform_row_is_constant(oracle_mod):
    """Uniform q, sc, m and the same d, dmin in every superblock give a
    constant row c = d*sc*q - dmin*m, so y = c * sum(x)."""
    rng = np.random.default_rng(5)
    S, n = 6, 3
    k = 256 * S
    cases = [(0x2E66, 0x2A00, 37, 12, 9), (0x3C00, 0x3800, 5, 7, 3), (0x1400, 0x0C00, 63, 63, 15)]
    for d_bits, dm_bits, scv, mv, qv in cases:
        f = synth.Fields(np.full((n, S), d_bits, np.uint16), np.full((n, S), dm_bits, np.uint16),
                         np.full((n, S, 8), scv, np.uint8), np.full((n, S, 8), mv, np.uint8),
                         np.full((n, S, 256), qv, np.uint8))
        w = synth.pack(f)
        d = Fraction(float(np.uint16(d_bits).view(np.float16)))
        dm = Fraction(float(np.uint16(dm_bits).view(np.float16)))
        cval = np.float32(float(d * scv * qv - dm * mv))   # one RNE rounding
        deq = oracle_mod.dequant(w, n, k)
        assert np.all(deq == cval)
        x = rng.standard_normal((2, k)).astype(np.float32)
        y, bound = oracle_mod.gemv(w, x, n)
        for b in range(2):
            exact = float(sum(Fraction(float(cval)) * Fraction(float(v)) for v in x[b]))
            assert np.allclose(y[b], exact, rtol=0, atol=1e-12 * bound[b].max())


def check_closed_form_zero_quants(oracle_mod):
    """All codes 0: y = -sum_j dmin*m_j * (sum of x over sub-block j)."""
    rng = np.random.default_rng(6)
    n, S = 5, 4
    k = 256 * S
    f = synth.draw_fields(rng, n, S)
    f.q[:] = 0
    w = synth.pack(f)
    x = rng.standard_normal((3, k)).astype(np.float32)
    y, bound = oracle_mod.gemv(w, x, n)
    dmin = f.dmin_bits.view(np.float16).astype(np.float64)
    for b in range(3):
        xs = x[b].astype(np.float64).reshape(S, 4, 2, 32).sum(axis=3).reshape(S, 8)  # [sb][j]
        for r in range(n):
            exp = -np.sum(dmin[r][:, None] * f.m[r].astype(np.float64) * xs)
            assert abs(y[b, r] - exp) <= 1e-12 * bound[b, r]


def check_exact_dyadic_bruteforce(oracle_mod):
    """Dyadic d and dmin and small-integer x make every weight and every
    product exact, so y is known exactly; rational arithmetic from the
    fields, not from the oracle, gives it."""
    rng = np.random.default_rng(9)
    n, S = 4, 2
    k = 256 * S
    f = synth.draw_fields(rng, n, S)
    dyadic = np.array([0x3800, 0x3400, 0x3C00, 0x4000, 0x3000, 0x2C00], np.uint16)  # .5 .25 1 2 .125 .0625
    f.d_bits[:] = rng.choice(dyadic, size=(n, S))
    f.dmin_bits[:] = rng.choice(dyadic, size=(n, S))
    w = synth.pack(f)
    x = rng.integers(-8, 9, size=(2, k)).astype(np.float32)
    y, bound = oracle_mod.gemv(w, x, n)
    for r in range(n):
        for b in range(2):
            tot = Fraction(0)
            mag = Fraction(0)
            for s in range(S):
                d = Fraction(float(f.d_bits[r, s].view(np.float16)))
                dm = Fraction(float(f.dmin_bits[r, s].view(np.float16)))
                for e in range(256):
                    j = 2 * (e // 64) + (e % 64) // 32
                    wv = d * int(f.sc[r, s, j]) * int(f.q[r, s, e]) - dm * int(f.m[r, s, j])
                    xv = int(x[b, 256 * s + e])
                    tot += wv * xv
                    mag += abs(wv) * abs(xv)
            assert y[b, r] == float(tot)
            assert bound[b, r] == float(mag)


def check_single_rounding_of_the_subtraction(oracle_mod):
    """When d*sc*q - dmin*m needs more than 24 bits, the weight is the exact
    value rounded once to binary32 (round-to-nearest-even)."""
    rng = np.random.default_rng(12)
    n, S = 64, 1
    f = synth.draw_fields(rng, n, S)
    # tiny d (subnormal and near the bottom of the normal range), dmin near 1
    f.d_bits[:] = rng.choice(np.array([0x0001, 0x0155, 0x03FF, 0x0401, 0x07FF, 0x0ABC], np.uint16), size=(n, S))
    f.dmin_bits[:] = rng.choice(np.array([0x3C01, 0x3BFF, 0x3E7B, 0x4123], np.uint16), size=(n, S))
    w = synth.pack(f)
    deq = oracle_mod.dequant(w, n, 256)
    for r in range(n):
        d = Fraction(float(f.d_bits[r, 0].view(np.float16)))
        dm = Fraction(float(f.dmin_bits[r, 0].view(np.float16)))
        for e in range(256):
            j = 2 * (e // 64) + (e % 64) // 32
            exact = d * int(f.sc[r, 0, j]) * int(f.q[r, 0, e]) - dm * int(f.m[r, 0, j])
            # the exact value fits a double (< 53 significant bits); casting it
            # to float32 is the single RNE rounding
            assert Fraction(float(exact)) == exact
            assert deq[r, e] == np.float32(float(exact)), (r, e)


def check_special_d_values(oracle_mod):
    """Signed zeros, subnormal, largest finite, infinities and NaN in d/dmin
    follow IEEE arithmetic on the decoded values."""
    specials = np.array([0x0000, 0x8000, 0x0001, 0x03FF, 0x7BFF, 0xFBFF, 0x7C00, 0xFC00, 0x7E00,
                         0xBC00, 0x3C00], np.uint16)
    rng = np.random.default_rng(4)
    n = specials.size * specials.size
    f = synth.draw_fields(rng, n, 1)
    f.d_bits[:, 0] = np.repeat(specials, specials.size)
    f.dmin_bits[:, 0] = np.tile(specials, specials.size)
    w = synth.pack(f)
    deq = oracle_mod.dequant(w, n, 256)
    with np.errstate(invalid="ignore", over="ignore"):
        for r in range(n):
            d = np.float32(f.d_bits[r, 0].view(np.float16))
            dm = np.float32(f.dmin_bits[r, 0].view(np.float16))
            for e in range(0, 256, 7):
                j = 2 * (e // 64) + (e % 64) // 32
                exp = np.float32(np.float32(d * np.float32(f.sc[r, 0, j])) * np.float32(f.q[r, 0, e])) \
                    - np.float32(dm * np.float32(f.m[r, 0, j]))
                got = deq[r, e]
                if np.isnan(exp):
                    assert np.isnan(got)
                else:
                    assert f32bits(got) == f32bits(exp), (r, e, got, exp)


# ------------------------------------------------------ quantizer round trip
def check_quantizer_round_trip(oracle_mod):
    rng = np.random.default_rng(21)
    n, k = 48, 1024
    x = rng.standard_normal((n, k)).astype(np.float32)
    wq = oracle_mod.quantize_rows(x)
    deq = oracle_mod.dequant(wq, n, k)
    blocks = wq.reshape(n, k // 256, 144)
    checked = 0
    for r in range(n):
        for s in range(k // 256):
            blk = blocks[r, s]
            d = float(np.uint16(blk[0] | (blk[1].astype(np.uint16) << 8)).view(np.float16))
            dm = float(np.uint16(blk[2] | (blk[3].astype(np.uint16) << 8)).view(np.float16))
            sc, m = oracle_mod.unpack_scales(blk[4:16])
            assert sc.max() < 64 and m.max() < 64
            for e in range(256):
                j = 2 * (e // 64) + (e % 64) // 32
                lo = -dm * int(m[j])
                hi = 15 * d * int(sc[j]) - dm * int(m[j])
                xv = float(x[r, 256 * s + e])
                if lo <= xv <= hi and sc[j] > 0:
                    err = abs(xv - float(deq[r, 256 * s + e]))
                    assert err <= 0.5 * d * int(sc[j]) + 2.0 ** -20 * max(abs(xv), dm * int(m[j])), (r, s, e)
                    checked += 1
    assert checked > 0.9 * n * k


def check_shape_errors(oracle_mod):
    for args in ((np.zeros(144, np.uint8), 1, 255), (np.zeros(143, np.uint8), 1, 256)):
        try:
            oracle_mod.dequant(*args)
        except ValueError:
            pass
        else:
            raise AssertionError("bad shape accepted")
    y, bound = oracle_mod.gemv(np.zeros(0, np.uint8), np.zeros((1, 256), np.float32), 0)
    assert y.shape == (1, 0)


# ------------------------------------------------- Q8 activations (variant)
# The Q8 block format is a reading (see oracle/q4k_oracle.c): blocks of 32,
# d = amax/127, codes the nearest-even integer of x*(127/amax).  Pinned by
# facts that hold whatever the implementation: exact round trips of dyadic
# blocks, closed forms of constant, zero, one-hot and mirrored blocks, the
# rounding bound, non-finite blocks, and the Q8 GEMV equal to the pinned
# f32 GEMV where the quantized x is x itself.

def _dyadic_q8_blocks(rng, m, nblk):
    """x = j * 2^e, integer j in [-127, 127] with one |j| = 127 per block,
    e per block in -60..60: amax = 127 * 2^e, so d = 2^e and the codes are j."""
    j = rng.integers(-127, 128, size=(m, nblk, 32))
    pos = rng.integers(0, 32, size=(m, nblk))
    sign = rng.choice([-1, 1], size=(m, nblk))
    for b in range(m):
        for t in range(nblk):
            j[b, t, pos[b, t]] = 127 * sign[b, t]
    e = rng.integers(-60, 61, size=(m, nblk))
    x = (j * np.exp2(e)[:, :, None]).astype(np.float32).reshape(m, nblk * 32)
    return x, j.reshape(m, nblk * 32).astype(np.int8), np.exp2(e).astype(np.float32)


def check_q8_dyadic_round_trip(oracle_mod):
    rng = np.random.default_rng(901)
    x, j, d = _dyadic_q8_blocks(rng, 3, 40)
    q, dq = oracle_mod.quantize_q8(x)
    assert np.array_equal(q, j)
    assert np.array_equal(dq.view(np.uint32), d.view(np.uint32))


def check_q8_closed_forms(oracle_mod):
    # constant positive block: all codes 127, d = c / 127 (f32); zero block:
    # d = 0, codes 0; one nonzero element: its code +-127, the rest 0;
    # the mirrored block: codes negated, the same scale
    rng = np.random.default_rng(902)
    c = np.float32(rng.uniform(0.5, 3.0))
    x = np.zeros((1, 128), np.float32)
    x[0, :32] = c
    x[0, 64 + 5] = -np.float32(7.25)
    x[0, 96:] = rng.standard_normal(32).astype(np.float32)
    q, d = oracle_mod.quantize_q8(x)
    assert np.all(q[0, :32] == 127) and d[0, 0] == np.float32(c / np.float32(127.0))
    assert np.all(q[0, 32:64] == 0) and d[0, 1] == 0.0
    assert q[0, 64 + 5] == -127 and np.count_nonzero(q[0, 64:96]) == 1
    assert d[0, 2] == np.float32(np.float32(7.25) / np.float32(127.0))
    qn, dn = oracle_mod.quantize_q8(-x)
    assert np.array_equal(qn, -q) and np.array_equal(dn, d)


def check_q8_rounding_bound(oracle_mod):
    # |x - d q| <= d/2 (1 + 2^-20) + 2^-21 |x| and |q| <= 127, x spread over
    # many binades
    rng = np.random.default_rng(903)
    x = (rng.standard_normal((4, 2048)) * np.exp2(rng.integers(-30, 31, size=(4, 64, 1))).repeat(
        32, axis=2).reshape(4, 2048)).astype(np.float32)
    q, d = oracle_mod.quantize_q8(x)
    assert np.all(np.abs(q.astype(int)) <= 127)
    dd = np.repeat(d.astype(np.float64), 32, axis=1)
    err = np.abs(x.astype(np.float64) - dd * q)
    assert np.all(err <= dd / 2 * (1 + 2.0 ** -20) + 2.0 ** -21 * np.abs(x.astype(np.float64)))
    # the largest element of each block takes code +-127
    amax = np.abs(x).reshape(4, 64, 32).max(axis=2)
    qmax = np.abs(q.astype(int)).reshape(4, 64, 32).max(axis=2)
    assert np.all(qmax[amax > 0] == 127)


def check_q8_non_finite_blocks(oracle_mod):
    x = np.ones((1, 96), np.float32)
    x[0, 3] = np.nan
    x[0, 40] = np.inf
    q, d = oracle_mod.quantize_q8(x)
    assert np.isnan(d[0, 0]) and np.all(q[0, :32] == 0)
    assert np.isinf(d[0, 1]) and np.all(q[0, 32:64] == 0)
    assert d[0, 2] == np.float32(1.0 / np.float32(127.0)) and np.all(q[0, 64:] == 127)


def check_q8_gemv_equals_f32_gemv_on_dyadic_x(oracle_mod):
    # where d q = x exactly (dyadic blocks), the Q8 GEMV is the pinned f32 GEMV
    rng = np.random.default_rng(904)
    n, k, m = 7, 512, 2
    w = synth.pack(synth.draw_fields(np.random.default_rng(905), n, k // 256))
    x, j, d = _dyadic_q8_blocks(rng, m, k // 32)
    x = (x * np.float32(2.0 ** -70)).astype(np.float32)     # products well inside f64
    d = (d * np.float32(2.0 ** -70)).astype(np.float32)
    y, bound = oracle_mod.gemv(w, x, n)
    yq, bq = oracle_mod.gemv_q8(w, j, d, n)
    assert np.array_equal(y, yq) and np.array_equal(bound, bq)


# ------------------------------------------------------------------ Q6_K
# The Q6_K field layout is a reading (GGUF Q6_K; see oracle/q4k_oracle.c).
# Pinned by a hand-computed superblock, by bytes placed element by element
# from the layout table here (an inverse written apart from the oracle's
# decode and from the generator's vectorized packer), by exact products of
# the fields, closed forms, exact dyadic dots and IEEE special values.

def load_q6k_golden():
    fields = {"ql": [], "qh": [], "scales": [], "d": []}
    w = []
    with open(os.path.join(GOLDEN, "q6k_superblock_handbuilt.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("w "):
                _, e, v = line.split()
                w.append((int(e), float(v)))
                continue
            key, val = line.split(":", 1)
            fields[key] += [int(t, 16) for t in val.split()]
    blk = np.array(fields["ql"] + fields["qh"] + fields["scales"] + fields["d"], dtype=np.uint8)
    assert blk.size == 210
    return blk, w


def q6k_place(codes, scales, d_bits):
    """One 210-byte superblock from 256 codes (0..63), 16 int8 scales and the
    fp16 bits of d, each code's bits placed one element at a time."""
    b = np.zeros(210, dtype=np.uint8)
    for e in range(256):
        h, t, l = e // 128, (e % 128) // 32, e % 32
        q = int(codes[e])
        lo, hi = q & 15, q >> 4
        i = 64 * h + 32 * (t % 2) + l
        b[i] |= lo if t < 2 else lo << 4
        b[128 + 32 * h + l] |= hi << (2 * t)
    b[192:208] = np.asarray(scales, dtype=np.int8).view(np.uint8)
    b[208] = d_bits & 0xFF
    b[209] = d_bits >> 8
    return b


def check_q6k_golden_handbuilt_superblock(oracle_mod):
    blk, w = load_q6k_golden()
    out = oracle_mod.q6k_dequant_superblock(blk)
    for e, v in w:
        assert out[e] == np.float32(v), (e, out[e], v)


def check_q6k_golden_through_gemv(oracle_mod):
    """x = e_i picks out weight i, through the GEMV with two vectors."""
    blk, w = load_q6k_golden()
    x = np.zeros((len(w), 256), np.float32)
    for t, (e, _) in enumerate(w):
        x[t, e] = 1.0
    y, bound = oracle_mod.q6k_gemv(blk, x, n=1)
    for t, (e, v) in enumerate(w):
        assert y[t, 0] == v and bound[t, 0] == abs(v)


def check_q6k_onehot_every_element_and_bit(oracle_mod):
    """All codes 32 (weight 0) but element e, whose code is 32 with bit b
    flipped: the one nonzero weight sits at e and equals d sc[e/16] (q - 32)
    with distinct scales per group.  Every element, every code bit, one
    superblock per row, in one call."""
    scales = np.array([3, -5, 7, -11, 13, -17, 19, -23, 29, -31, 37, -41, 43, -47, 53, -59],
                      np.int8)
    rows = []
    expect = []
    for e in range(256):
        for bit in range(6):
            codes = np.full(256, 32, np.int64)
            codes[e] = 32 ^ (1 << bit)
            rows.append(q6k_place(codes, scales, F16_ONE))
            ex = np.zeros(256, np.float32)
            ex[e] = float(scales[e // 16]) * float(codes[e] - 32)
            expect.append(ex)
    w = np.concatenate(rows)
    out = oracle_mod.q6k_dequant(w, len(rows), 256)
    assert np.array_equal(out, np.array(expect))


def check_q6k_generator_layout_agrees(oracle_mod):
    """The generator's vectorized packer and the element-wise placement here
    give the same bytes; decoded, every weight is the exact product of its
    fields (d has 11 significant bits, |sc| <= 128, |q - 32| <= 32: exact in
    f32), checked with rational arithmetic."""
    rng = np.random.default_rng(611)
    f = synth.draw_q6k_fields(rng, 3, 2)
    # the extremes of every field in the first superblock
    f.q[0, 0, :4] = [0, 63, 32, 31]
    f.sc[0, 0, :2] = [-128, 127]
    f.d_bits[0, 0] = 0x7BFF                       # largest finite binary16
    f.d_bits[1, 0] = 0x0001                       # smallest subnormal
    w = synth.pack_q6k(f)
    by_hand = np.concatenate([q6k_place(f.q[r, s], f.sc[r, s], int(f.d_bits[r, s]))
                              for r in range(3) for s in range(2)])
    assert np.array_equal(w, by_hand)
    out = oracle_mod.q6k_dequant(w, 3, 512)
    d = f.d_bits.view(np.float16)
    for r in range(3):
        for s in range(2):
            dv = Fraction(float(d[r, s]))
            for e in range(256):
                exact = dv * int(f.sc[r, s, e // 16]) * (int(f.q[r, s, e]) - 32)
                assert Fraction(float(out[r, 256 * s + e])) == exact, (r, s, e)


def check_q6k_closed_forms(oracle_mod):
    """Codes all 32: W = 0, y = 0 and bound 0.  Uniform code c and scale s,
    d = 1/2: every weight is s (c - 32) / 2, so y = s (c - 32) / 2 * sum x,
    exactly for dyadic x."""
    n, k = 3, 768
    zero = np.concatenate([q6k_place(np.full(256, 32), np.arange(1, 17), F16_HALF)
                           for _ in range(n * k // 256)])
    x = np.random.default_rng(612).standard_normal((2, k)).astype(np.float32)
    y, bound = oracle_mod.q6k_gemv(zero, x, n)
    assert np.all(y == 0.0) and np.all(bound == 0.0)
    c, sv = 45, -9
    uni = np.concatenate([q6k_place(np.full(256, c), np.full(16, sv), F16_HALF)
                          for _ in range(n * k // 256)])
    xd = (np.random.default_rng(613).integers(-64, 65, size=(2, k)) / 8.0).astype(np.float32)
    y, bound = oracle_mod.q6k_gemv(uni, xd, n)
    wv = Fraction(sv * (c - 32), 2)
    for b in range(2):
        sx = sum(Fraction(float(v)) for v in xd[b])
        sa = sum(abs(Fraction(float(v))) for v in xd[b])
        assert all(Fraction(float(v)) == wv * sx for v in y[b])
        assert all(Fraction(float(v)) == abs(wv) * sa for v in bound[b])


def check_q6k_exact_dyadic_dot(oracle_mod):
    """d = 2^-10, random codes and scales, integer x: every product and sum is
    exact in f64, so y equals the dot product in integers."""
    rng = np.random.default_rng(614)
    n, k = 5, 512
    codes = rng.integers(0, 64, size=(n, k // 256, 256))
    scales = rng.integers(-128, 128, size=(n, k // 256, 16))
    w = np.concatenate([q6k_place(codes[r, s], scales[r, s], 0x1400)      # 2^-10
                        for r in range(n) for s in range(k // 256)])
    x = rng.integers(-1000, 1001, size=(3, k)).astype(np.float32)
    y, _ = oracle_mod.q6k_gemv(w, x, n)
    for r in range(n):
        wr = [int(scales[r, c // 256, (c % 256) // 16]) * (int(codes[r, c // 256, c % 256]) - 32)
              for c in range(k)]
        for b in range(3):
            exact = Fraction(sum(wv * int(xv) for wv, xv in zip(wr, x[b])), 1024)
            assert Fraction(float(y[b, r])) == exact, (r, b)


def check_q6k_special_d(oracle_mod):
    """d = +-0, +-inf, NaN: weights follow IEEE products (inf * 0 is NaN: a
    zero scale or a code of 32)."""
    codes = np.arange(256) % 64
    scales = np.array([0, 1, -1, 5, -128, 127, 2, -2, 0, 3, -3, 4, -4, 7, -7, 1], np.int8)
    for bits in (0x0000, 0x8000, 0x7C00, 0xFC00, 0x7E00, 0x3C01):
        out = oracle_mod.q6k_dequant_superblock(q6k_place(codes, scales, bits))
        d = np.array([bits], np.uint16).view(np.float16).astype(np.float32)[0]
        with np.errstate(invalid="ignore"):
            expect = (d * scales.astype(np.float32).repeat(16)) * (codes - 32).astype(np.float32)
        assert np.array_equal(out.view(np.uint32), expect.astype(np.float32).view(np.uint32)) or (
            np.array_equal(np.isnan(out), np.isnan(expect))
            and np.array_equal(out[~np.isnan(out)].view(np.uint32),
                               expect[~np.isnan(expect)].astype(np.float32).view(np.uint32))), bits


def check_q6k_row_stride(oracle_mod):
    """Rows at a stride above 210 k / 256 bytes decode as the dense rows;
    the padding bytes (here 0xff) are never read."""
    rng = np.random.default_rng(615)
    n, k = 4, 1024
    f = synth.draw_q6k_fields(rng, n, k // 256)
    dense = synth.pack_q6k(f)
    stride = 896
    padded = synth.pack_q6k(f, stride).reshape(n, stride)
    padded[:, 840:] = 0xFF
    padded = padded.reshape(-1)
    assert np.array_equal(oracle_mod.q6k_dequant(padded, n, k, stride),
                          oracle_mod.q6k_dequant(dense, n, k))
    x = rng.standard_normal((2, k)).astype(np.float32)
    y0, b0 = oracle_mod.q6k_gemv(dense, x, n)
    y1, b1 = oracle_mod.q6k_gemv(padded, x, n, stride)
    assert np.array_equal(y0, y1) and np.array_equal(b0, b1)


def check_q6k_shape_errors(oracle_mod):
    for args in ((np.zeros(210, np.uint8), 1, 255), (np.zeros(209, np.uint8), 1, 256)):
        try:
            oracle_mod.q6k_dequant(*args)
        except ValueError:
            pass
        else:
            raise AssertionError("bad shape accepted")
    try:
        oracle_mod.q6k_dequant(np.zeros(420, np.uint8), 2, 256, 200)
    except ValueError:
        pass
    else:
        raise AssertionError("row stride below the row accepted")


# ----------------------------------------------------- fp16 mirror and GEMM
# The mirror element is the pinned f32 weight rounded to binary16; numpy's
# float16 cast (round to nearest even, written apart from the oracle) must
# agree bit for bit.  The GEMM is pinned by integer-valued operands, whose
# products and sums are exact, against integer matrix products, and by
# one-hot rows that pick out one activation each (orientation).

def _f16_bits(a):
    return np.asarray(a, np.float32).astype(np.float16).view(np.uint16)


def check_mirror_f16_is_the_rounded_weight(oracle_mod):
    rng = np.random.default_rng(701)
    n, k = 6, 1024
    f = synth.draw_fields(rng, n, k // 256)
    f.d_bits[0, 0] = 0x7800          # d = 32768: weights beyond the binary16 range -> inf
    f.d_bits[1, 1] = 0x0001          # smallest subnormal d
    w4 = synth.pack(f)
    m4 = oracle_mod.mirror_f16(w4, 4, n, k)
    assert np.array_equal(m4, _f16_bits(oracle_mod.dequant(w4, n, k)))
    assert np.any(m4 == 0x7C00) or np.any(m4 == 0xFC00)
    f6 = synth.draw_q6k_fields(rng, n, k // 256)
    f6.d_bits[2, 0] = 0x7BFF         # largest finite d
    w6 = synth.pack_q6k(f6, 896)
    m6 = oracle_mod.mirror_f16(w6, 6, n, k, 896)
    assert np.array_equal(m6, _f16_bits(oracle_mod.q6k_dequant(w6, n, k, 896)))


def check_f16_cvt_matches_numpy(oracle_mod):
    rng = np.random.default_rng(702)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 20, size=20000))).astype(np.float32)
    x[:6] = [0.0, -0.0, 65504.0, 65520.0, -1e-8, 6.0e-8]
    assert np.array_equal(oracle_mod.f16_cvt(x), _f16_bits(x))


def check_f16_gemm_integer_exact(oracle_mod):
    rng = np.random.default_rng(703)
    m, n, k = 5, 7, 300
    wi = rng.integers(-64, 65, size=(n, k))
    xi = rng.integers(-64, 65, size=(m, k))
    y, bound = oracle_mod.f16_gemm(_f16_bits(wi), _f16_bits(xi))
    assert np.array_equal(y, (xi @ wi.T).astype(np.float64))
    assert np.array_equal(bound, (np.abs(xi) @ np.abs(wi).T).astype(np.float64))


def check_f16_gemm_orientation(oracle_mod):
    """Row r of W is one-hot at column (3 r + 1) mod k: y[b, r] is x[b] at
    that column."""
    rng = np.random.default_rng(704)
    m, n, k = 3, 11, 37
    w = np.zeros((n, k), np.float32)
    for r in range(n):
        w[r, (3 * r + 1) % k] = 1.0
    x = rng.standard_normal((m, k)).astype(np.float16).astype(np.float32)
    y, _ = oracle_mod.f16_gemm(_f16_bits(w), _f16_bits(x))
    for r in range(n):
        assert np.array_equal(y[:, r], x[:, (3 * r + 1) % k].astype(np.float64))


# fastest first: the mutation test stops at the first failing check
ALL_CHECKS = (
    check_golden_handbuilt_superblock,
    check_golden_superblock_through_gemv,
    check_scale_unpack_handworked_golden,
    check_scale_single_field_by_hand,
    check_onehot_min_layout_bruteforce,
    check_position_map_every_byte,
    check_onehot_scale_layout_bruteforce,
    check_closed_form_zero_quants,
    check_closed_form_uniform_row_is_constant,
    check_exact_dyadic_bruteforce,
    check_single_rounding_of_the_subtraction,
    check_special_d_values,
    check_f16_decode_exhaustive_matches_numpy,
    check_shape_errors,
    check_quantizer_round_trip,
    check_f16_encode_rne_matches_numpy,
    check_scale_pack_unpack_exhaustive,
    check_q8_dyadic_round_trip,
    check_q8_closed_forms,
    check_q8_rounding_bound,
    check_q8_non_finite_blocks,
    check_q8_gemv_equals_f32_gemv_on_dyadic_x,
    check_q6k_golden_handbuilt_superblock,
    check_q6k_golden_through_gemv,
    check_q6k_shape_errors,
    check_q6k_special_d,
    check_q6k_row_stride,
    check_q6k_closed_forms,
    check_q6k_exact_dyadic_dot,
    check_q6k_generator_layout_agrees,
    check_q6k_onehot_every_element_and_bit,
    check_f16_gemm_orientation,
    check_f16_gemm_integer_exact,
    check_f16_cvt_matches_numpy,
    check_mirror_f16_is_the_rounded_weight,
)
