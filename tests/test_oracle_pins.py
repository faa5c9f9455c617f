"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
the pages' definitions, closed forms, exact rational arithmetic or brute force
on tiny inputs.  They are run as tests here and again by
``test_oracle_mutations.py`` against deliberately broken copies of the oracle,
to show that a plausible mistake anywhere in it fails at least one pin.
"""

from __future__ import annotations

import itertools
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle.tq_oracle as tqo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# helpers written from IEEE 754 / integer arithmetic, not from the oracle
# ----------------------------------------------------------------------------

def rn32(q: Fraction) -> Fraction:
    """Round a rational to the nearest binary32 value, ties to even (IEEE 754)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)  # below the normal range the quantum stays 2^-149
    quantum = Fraction(2) ** (e - 23)
    m = round(a / quantum)  # Fraction rounding: nearest, ties to even
    return sign * m * quantum


def rne_int(v: Fraction) -> int:
    return round(v)  # ties to even for Fraction


def f32_hex(v) -> str:
    return "0x%08x" % int(np.asarray(v, dtype=np.float32).view(np.uint32))


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([p.strip() for p in line.split("|")])
    return rows


def bf16_all_finite() -> np.ndarray:
    """Every finite bf16 value (both signs), as float32."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    pos = (bits << 16).view(np.float32)
    return np.concatenate([pos, -pos[1:]])


def lossless_codes(rng, rows, k, qmax):
    """Integer codes in [-qmax, qmax] with one +-qmax in every row."""
    c = rng.integers(-qmax, qmax + 1, size=(rows, k)).astype(np.int64)
    j = rng.integers(0, k, size=rows)
    c[np.arange(rows), j] = np.where(rng.integers(0, 2, size=rows) == 1, qmax, -qmax)
    return c


# ----------------------------------------------------------------------------
# quantiser
# ----------------------------------------------------------------------------

def pin_quantizer_golden():
    for name, bits, vals, s_hex, codes in read_golden("quantizer_examples.txt"):
        row = np.array([[float(v) for v in vals.split()]], dtype=np.float32)
        c, s = tqo.quantize_rows(row, int(bits))
        assert f32_hex(s[0]) == s_hex.lower(), (name, f32_hex(s[0]), s_hex)
        assert c[0].tolist() == [int(v) for v in codes.split()], (name, c[0].tolist(), codes)


def pin_quantizer_bruteforce(amaxes=(3.0, 1.0, 0.69921875, 12.375, 1.5 * 2.0 ** -100), bits=4):
    """Every finite bf16 x with |x| <= amax, against exact rational arithmetic."""
    allv = bf16_all_finite()
    qmax = (1 << (bits - 1)) - 1
    for amax in amaxes:
        xs = allv[np.abs(allv) <= np.float32(amax)]
        rows = np.stack([np.full(xs.shape, amax, dtype=np.float32), xs], axis=1)
        c, s = tqo.quantize_rows(rows, bits)
        s_ref = rn32(Fraction(float(np.float32(amax))) / qmax)
        assert Fraction(float(s[0])) == s_ref, (amax, float(s[0]), s_ref)
        assert np.all(s == s[0])
        got = c[:, 1].astype(np.int64)
        exp = np.empty_like(got)
        for i, x in enumerate(xs.tolist()):
            v = rne_int(rn32(Fraction(x) / s_ref))
            exp[i] = min(max(v, -(qmax + 1)), qmax)
        bad = np.nonzero(got != exp)[0]
        assert bad.size == 0, (amax, xs[bad[:5]].tolist(), got[bad[:5]].tolist(), exp[bad[:5]].tolist())
        assert np.all(c[:, 0] == qmax)


def pin_quantizer_invariants(seed=7):
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal((64, 96)) * np.exp(rng.uniform(-6, 6, size=(64, 1)))).astype(np.float32)
    a[3, 17] *= 50  # an outlier
    for bits in (4, 8):
        qmax = (1 << (bits - 1)) - 1
        c, s = tqo.quantize_rows(a, bits)
        # absmax element maps to +-qmax; all codes within [-qmax, qmax]
        j = np.argmax(np.abs(a), axis=1)
        assert np.all(np.abs(c[np.arange(a.shape[0]), j]) == qmax)
        assert np.all(np.sign(c[np.arange(a.shape[0]), j]) == np.sign(a[np.arange(a.shape[0]), j]))
        assert np.abs(c).max() <= qmax
        # dequantisation error <= s/2 (+ the fp32 rounding of x/s), in exact fp64
        err = np.abs(a.astype(np.float64) - c.astype(np.float64) * s.astype(np.float64)[:, None])
        assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + 2.0 ** -21 * qmax))
        # scale is fl32(max|row| / qmax)
        amax = np.max(np.abs(a), axis=1)
        assert np.array_equal(s, (amax / np.float32(qmax)).astype(np.float32))
        # power-of-two scaling of a row leaves codes, scales by 2^k exactly
        for k in (-5, 3):
            c2, s2 = tqo.quantize_rows(a * np.float32(2.0 ** k), bits)
            assert np.array_equal(c2, c)
            assert np.array_equal(s2, (s * np.float32(2.0 ** k)).astype(np.float32))
        # negation flips codes (round-half-even is symmetric)
        c3, s3 = tqo.quantize_rows(-a, bits)
        assert np.array_equal(c3, -c) and np.array_equal(s3, s)
        # rows are independent: scaling one row does not touch the others
        b = a.copy()
        b[5] *= np.float32(1000.0)
        c4, s4 = tqo.quantize_rows(b, bits)
        keep = np.arange(a.shape[0]) != 5
        assert np.array_equal(c4[keep], c[keep]) and np.array_equal(s4[keep], s[keep])


def pin_weight_is_per_output_channel(seed=8):
    rng = np.random.default_rng(seed)
    d, m = 24, 10
    cw = lossless_codes(rng, m, d, 7)  # output channel j = row j of C_w
    sw = (2.0 ** rng.integers(-9, -3, size=m)).astype(np.float32)
    w = (cw * sw[:, None]).T.astype(np.float32)  # d x m, column j = channel j
    c, s = tqo.quantize_weight(w, 4)
    assert c.shape == (m, d)
    assert np.array_equal(c, cw)
    assert np.array_equal(s, sw)


# ----------------------------------------------------------------------------
# packing
# ----------------------------------------------------------------------------

def pin_pack_golden():
    g = dict((k, v) for k, v in read_golden("pack_example.txt"))
    codes = np.array([[int(t) for t in r.split()] for r in g["codes"].split(";")])
    expect = np.array([[int(t, 16) for t in r.split()] for r in g["bytes"].split(";")], dtype=np.uint8)
    assert np.array_equal(tqo.pack_int4(codes), expect)
    assert np.array_equal(tqo.unpack_int4(expect), codes)


def pin_pack_roundtrip(seed=9):
    rng = np.random.default_rng(seed)
    c = rng.integers(-8, 8, size=(7, 40))
    p = tqo.pack_int4(c)
    assert p.dtype == np.uint8 and p.shape == (7, 20)
    assert np.array_equal(tqo.unpack_int4(p), c)
    # every byte value decodes and re-encodes to itself
    allb = np.arange(256, dtype=np.uint8)[None, :]
    assert np.array_equal(tqo.pack_int4(tqo.unpack_int4(allb)), allb)
    c8 = rng.integers(-128, 128, size=(3, 9))
    assert np.array_equal(tqo.pack_codes(c8, 8).view(np.int8).astype(np.int64), c8)


# ----------------------------------------------------------------------------
# integer accumulation
# ----------------------------------------------------------------------------

def pin_accumulator_bruteforce(seed=10):
    rng = random.Random(seed)
    for (n, k, m, lo, hi) in ((3, 5, 4, -8, 7), (2, 33, 3, -128, 127), (1, 1, 1, -8, 7), (4, 64, 5, -7, 7)):
        cx = [[rng.randint(lo, hi) for _ in range(k)] for _ in range(n)]
        cw = [[rng.randint(lo, hi) for _ in range(k)] for _ in range(m)]
        exp = [[sum(cx[i][t] * cw[j][t] for t in range(k)) for j in range(m)] for i in range(n)]
        got = tqo.int_matmul(np.array(cx), np.array(cw))
        assert got.tolist() == exp


def pin_accumulator_invariants(seed=11):
    rng = np.random.default_rng(seed)
    cx = rng.integers(-7, 8, size=(6, 128))
    cw1 = rng.integers(-7, 8, size=(5, 128))
    cw2 = rng.integers(-7, 8, size=(5, 128))
    base = tqo.int_matmul(cx, cw1)
    perm = rng.permutation(128)
    assert np.array_equal(tqo.int_matmul(cx[:, perm], cw1[:, perm]), base)
    assert np.array_equal(tqo.int_matmul(cx, cw1 + cw2), base + tqo.int_matmul(cx, cw2))
    # extreme magnitudes stay exact
    big = tqo.int_matmul(np.full((1, 14336), -8), np.full((1, 14336), -8))
    assert int(big[0, 0]) == 64 * 14336


# ----------------------------------------------------------------------------
# the layer
# ----------------------------------------------------------------------------

def pin_linear_golden():
    g = dict((k, v) for k, v in read_golden("linear_example.txt"))

    def mat(s):
        return np.array([[float(t) for t in r.split()] for r in s.split(";")], dtype=np.float32)

    out = tqo.tq_linear_ref(mat(g["X"]), mat(g["R"]), mat(g["L1"]), mat(g["L2"]))
    assert int(out["acc"][0, 0]) == int(g["acc"])
    num, den = (int(t) for t in g["Y_num_den"].split())
    assert Fraction(float(out["Y"][0, 0])) == Fraction(num, den)


def _lossless_case(rng, n, d, m):
    cx = lossless_codes(rng, n, d, 7)
    sx = (2.0 ** rng.integers(-6, 3, size=n)).astype(np.float32)
    cw = lossless_codes(rng, m, d, 7)
    sw = (2.0 ** rng.integers(-10, -4, size=m)).astype(np.float32)
    x = (cx * sx[:, None]).astype(np.float32)
    r = (cw * sw[:, None]).T.astype(np.float32)
    return x, r, cx, sx, cw, sw


def pin_linear_lossless(seed=12):
    """Inputs that quantise without loss: Y(r=0) equals X R exactly."""
    rng = np.random.default_rng(seed)
    n, d, m = 5, 48, 7
    x, r, cx, sx, cw, sw = _lossless_case(rng, n, d, m)
    out = tqo.tq_linear_ref(x, r)
    assert np.array_equal(out["codes_x"], cx) and np.array_equal(out["s_x"], sx)
    assert np.array_equal(out["codes_w"], cw) and np.array_equal(out["s_w"], sw)
    assert np.array_equal(out["acc"], cx @ cw.T)
    assert np.array_equal(out["Y"], x.astype(np.float64) @ r.astype(np.float64))
    # r = 0 (empty low-rank factors) reduces to the same pure W4A4 output
    out0 = tqo.tq_linear_ref(x, r, np.zeros((d, 0), np.float32), np.zeros((0, m), np.float32))
    assert np.array_equal(out0["Y"], out["Y"])


def pin_linear_lowrank(seed=13):
    rng = np.random.default_rng(seed)
    n, d, m, rk = 6, 40, 9, 3
    x, r, *_ = _lossless_case(rng, n, d, m)
    l1 = rng.standard_normal((d, rk)).astype(np.float32)
    l2 = rng.standard_normal((rk, m)).astype(np.float32)
    x64, r64, l164, l264 = (a.astype(np.float64) for a in (x, r, l1, l2))
    full = tqo.tq_linear_ref(x, r, l1, l2)["Y"]
    ref = x64 @ r64 + x64 @ (l164 @ l264)
    assert np.allclose(full, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # R = 0: scales 0, codes 0, output = X (L1 L2) by associativity, from the
    # unquantised X (a generic X, whose quantisation is lossy)
    xg = rng.standard_normal((n, d)).astype(np.float32)
    z = tqo.tq_linear_ref(xg, np.zeros_like(r), l1, l2)
    assert np.all(z["s_w"] == 0) and np.all(z["codes_w"] == 0)
    lr = xg.astype(np.float64) @ (l164 @ l264)
    assert np.allclose(z["Y"], lr, rtol=1e-12, atol=1e-12 * np.abs(lr).max())
    # L2 = 0 gives the pure W4A4 output
    assert np.array_equal(tqo.tq_linear_ref(x, r, l1, np.zeros_like(l2))["Y"], tqo.tq_linear_ref(x, r)["Y"])


def pin_linear_sampling(seed=14):
    """Sampled rows / columns equal the corresponding entries of the full output."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((9, 64)).astype(np.float32)
    r = (rng.standard_normal((64, 11)) * 0.02).astype(np.float32)
    l1 = rng.standard_normal((64, 4)).astype(np.float32)
    l2 = rng.standard_normal((4, 11)).astype(np.float32)
    full = tqo.tq_linear_ref(x, r, l1, l2)
    rows, cols = np.array([8, 0, 3]), np.array([10, 2])
    part = tqo.tq_linear_ref(x, r, l1, l2, rows=rows, cols=cols)
    assert np.array_equal(part["Y"], full["Y"][np.ix_(rows, cols)])
    assert np.array_equal(part["acc"], full["acc"][np.ix_(rows, cols)])


# ----------------------------------------------------------------------------
# rotation and the two-subspace form
# ----------------------------------------------------------------------------

def pin_hadamard():
    for k in (1, 2, 8, 128):
        h = tqo.hadamard(k)
        assert np.array_equal(h @ h.T, k * np.eye(k, dtype=np.int64))
        idx = np.arange(k)
        pc = np.vectorize(lambda v: bin(int(v)).count("1"))(idx[:, None] & idx[None, :])
        assert np.array_equal(h, np.where(pc % 2 == 0, 1, -1))  # Sylvester form


def pin_rotation_identities(seed=15):
    rng = np.random.default_rng(seed)
    d, n, m, dh = 256, 5, 7, 32
    signs = np.where(rng.integers(0, 2, size=d) == 1, 1.0, -1.0)
    perm = rng.permutation(d)
    u = tqo.block_rotation(signs, 128, perm)
    assert np.allclose(u @ u.T, np.eye(d), atol=1e-13)
    x = rng.standard_normal((n, d))
    w = rng.standard_normal((d, m))
    xu, uw = tqo.rotate(x, w, u)
    assert np.allclose(xu @ uw, x @ w, rtol=1e-12, atol=1e-12)  # Eq. 3
    ul, uh = u[:, : d - dh], u[:, d - dh:]
    assert np.allclose(ul @ ul.T + uh @ uh.T, np.eye(d), atol=1e-13)  # Eq. 5
    xl, xh, wl, wh = tqo.subspace_split(x, w, u, dh)
    assert xl.shape == (n, d - dh) and xh.shape == (n, dh) and wl.shape == (d - dh, m) and wh.shape == (dh, m)
    assert np.allclose(xl @ wl + xh @ wh, x @ w, rtol=1e-12, atol=1e-12)  # Eq. 8
    # X_l, X_h are the column blocks of X U; W_l, W_h the row blocks of U^T W
    assert np.allclose(np.hstack([xl, xh]), xu, rtol=0, atol=1e-13)
    assert np.allclose(np.vstack([wl, wh]), uw, rtol=0, atol=1e-13)


def pin_two_subspace_lossless(seed=16):
    """Eq. 9 with inputs that quantise without loss is exactly X_l W_l + X_h W_h."""
    rng = np.random.default_rng(seed)
    n, dl, dh, m = 4, 64, 16, 6
    cxl = lossless_codes(rng, n, dl, 7)
    cxh = lossless_codes(rng, n, dh, 127)
    cwl = lossless_codes(rng, m, dl, 7)
    cwh = lossless_codes(rng, m, dh, 127)
    sxl = 2.0 ** rng.integers(-4, 2, size=n)
    sxh = 2.0 ** rng.integers(-9, -5, size=n)
    swl = 2.0 ** rng.integers(-8, -3, size=m)
    swh = 2.0 ** rng.integers(-12, -8, size=m)
    xl, xh = cxl * sxl[:, None], cxh * sxh[:, None]
    wl, wh = (cwl * swl[:, None]).T, (cwh * swh[:, None]).T
    xrot = np.hstack([xl, xh]).astype(np.float32)
    wrot = np.vstack([wl, wh]).astype(np.float32)
    out = tqo.tq_linear_mp_ref(xrot, wrot, dh)
    assert np.array_equal(out["codes_xl"], cxl) and np.array_equal(out["codes_xh"], cxh)
    assert np.array_equal(out["codes_wl"], cwl) and np.array_equal(out["codes_wh"], cwh)
    assert np.array_equal(out["acc_l"], cxl @ cwl.T) and np.array_equal(out["acc_h"], cxh @ cwh.T)
    assert np.array_equal(out["Y"], xl @ wl + xh @ wh)
    # d_hi = d is W8A8; d_hi = 0 is W4A4, both on the rotated data
    x8 = (cxh * sxh[:, None]).astype(np.float32)
    w8 = (cwh * swh[:, None]).T.astype(np.float32)
    assert np.array_equal(tqo.tq_linear_mp_ref(x8, w8, dh)["Y"], x8.astype(np.float64) @ w8)
    x4 = (cxl * sxl[:, None]).astype(np.float32)
    w4 = (cwl * swl[:, None]).T.astype(np.float32)
    assert np.array_equal(tqo.tq_linear_mp_ref(x4, w4, 0)["Y"], x4.astype(np.float64) @ w4)
    assert np.array_equal(tqo.tq_linear_mp_ref(x4, w4, 0)["Y"], tqo.tq_linear_ref(x4, w4)["Y"])


def pin_group_stacking(seed=17):
    """G layers on one X equal one layer whose weight stacks theirs side by side
    and whose low-rank factors are [L1_0 | L1_1 | ...] and blockdiag(L2_0, L2_1, ...):
    weight scales are per output channel, and the block-diagonal L2 keeps each
    layer's T columns to its own channels."""
    rng = np.random.default_rng(seed)
    n, d, rk, ms = 6, 48, 3, (5, 7, 4)
    x = rng.standard_normal((n, d)).astype(np.float32)
    rs = [(0.02 * rng.standard_normal((d, m))).astype(np.float32) for m in ms]
    l1s = [rng.standard_normal((d, rk)).astype(np.float32) for _ in ms]
    l2s = [(0.02 * rng.standard_normal((rk, m))).astype(np.float32) for m in ms]
    grp = tqo.tq_linear_group_ref(x, rs, l1s, l2s)
    l2bd = np.zeros((rk * len(ms), sum(ms)), np.float32)
    c0 = 0
    for g, m in enumerate(ms):
        l2bd[rk * g:rk * (g + 1), c0:c0 + m] = l2s[g]
        c0 += m
    one = tqo.tq_linear_ref(x, np.concatenate(rs, axis=1), np.concatenate(l1s, axis=1), l2bd)
    assert np.array_equal(grp["codes_x"], one["codes_x"]) and np.array_equal(grp["s_x"], one["s_x"])
    assert np.array_equal(np.concatenate([o["codes_w"] for o in grp["layers"]]), one["codes_w"])
    assert np.array_equal(np.concatenate([o["acc"] for o in grp["layers"]], axis=1), one["acc"])
    assert np.allclose(grp["Y"], one["Y"], rtol=1e-12, atol=1e-12 * np.abs(one["Y"]).max())
    # one layer alone is the plain layer
    assert np.array_equal(tqo.tq_linear_group_ref(x, rs[:1], l1s[:1], l2s[:1])["Y"],
                          tqo.tq_linear_ref(x, rs[0], l1s[0], l2s[0])["Y"])


def pin_rht_rows(seed=18):
    """The fp32 online rotation: exact on small integers (each butterfly and
    the final single rounding), within fp32 error of X U from the dense fp64
    basis, and H H = block I for the unscaled butterflies."""
    rng = np.random.default_rng(seed)
    n, d, block = 5, 512, 128
    signs = np.where(rng.integers(0, 2, size=d) == 1, 1.0, -1.0)
    perm = rng.permutation(d)
    # small integers: every butterfly sum is exact, so X' = fl32(fl32(H (x signs)) / sqrt(block) as fl32) exactly
    xi = rng.integers(-50, 51, size=(n, d)).astype(np.float32)
    h = tqo.hadamard(block)
    exact = np.concatenate([(xi[:, b:b + block].astype(np.int64) * signs[b:b + block].astype(np.int64)) @ h
                            for b in range(0, d, block)], axis=1)
    want = (exact.astype(np.float32) * np.float32(1.0 / np.sqrt(block)))[:, perm]
    assert np.array_equal(tqo.rht_rows(xi, signs, perm, block), want)
    # generic values: close to the fp64 dense rotation of block_rotation
    x = rng.standard_normal((n, d)).astype(np.float32)
    u = tqo.block_rotation(signs, block, perm)
    ref = x.astype(np.float64) @ u
    got = tqo.rht_rows(x, signs, perm, block).astype(np.float64)
    tol = 8 * np.finfo(np.float32).eps * np.sqrt(block) * np.abs(x).max()
    assert np.abs(got - ref).max() <= tol
    # H H = block I: the transform applied twice (signs +1, identity permutation) gives x back
    ones, ident = np.ones(d), np.arange(d)
    twice = tqo.rht_rows(tqo.rht_rows(xi, ones, ident, block), ones, ident, block)
    assert np.allclose(twice, xi, rtol=1e-6, atol=1e-4)


def pin_rht_layer_rotation_invariance(seed=19):
    """The two-subspace layer on unrotated X with the rotation done online
    equals X W up to the quantisers' error (CoQuant Eq. 3: (XU)(U^T W) = XW);
    at d_hi = d both sides are 8-bit, so the error is small."""
    rng = np.random.default_rng(seed)
    n, d, m, block = 6, 256, 40, 128
    signs = np.where(rng.integers(0, 2, size=d) == 1, 1.0, -1.0)
    perm = rng.permutation(d)
    x = rng.standard_normal((n, d)).astype(np.float32)
    w = (0.02 * rng.standard_normal((d, m))).astype(np.float32)
    u = tqo.block_rotation(signs, block, perm)
    wrot = (u.T @ w.astype(np.float64)).astype(np.float32)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    for d_hi, tol in ((d, 2e-2), (128, 3.5e-1)):  # half the dimensions at 4 bits: a loose bound
        y = tqo.tq_linear_mp_rht_ref(x, signs, perm, wrot, d_hi, block)["Y"]
        assert np.abs(y - ref).max() <= tol * np.abs(ref).max(), d_hi
    # the same codes as the pre-rotated layer fed with the fp32 rotated X
    out = tqo.tq_linear_mp_rht_ref(x, signs, perm, wrot, 128, block)
    pre = tqo.tq_linear_mp_ref(tqo.rht_rows(x, signs, perm, block), wrot, 128)
    assert np.array_equal(out["codes_xl"], pre["codes_xl"]) and np.array_equal(out["codes_xh"], pre["codes_xh"])


# ----------------------------------------------------------------------------
# fully quantised low-rank branch
# ----------------------------------------------------------------------------

def _qlr_lossless_case(rng, n, d, m, rk, a=-3):
    """X, R, V that quantise without loss, and U whose columns are one-hot
    (entry +-7 2^a at input channel k_j, k_0 = 0) with column 0 of every token's
    codes at +-7: then X U V is reproduced exactly by the two quantised stages."""
    x, r, cx, sx, cw, sw = _lossless_case(rng, n, d, m)
    cx[:, 0] = np.where(rng.integers(0, 2, size=n) == 1, 7, -7)
    x = (cx * sx[:, None]).astype(np.float32)
    ks = np.concatenate([[0], rng.choice(np.arange(1, d), size=rk - 1, replace=False)])
    sg = np.where(rng.integers(0, 2, size=rk) == 1, 7, -7)
    u = np.zeros((d, rk), np.float32)
    u[ks, np.arange(rk)] = sg * 2.0 ** a
    cv = lossless_codes(rng, m, rk, 7)
    sv = (2.0 ** rng.integers(-8, -3, size=m)).astype(np.float32)
    v = (cv * sv[:, None]).T.astype(np.float32)
    return x, r, u, v, cx, sx, ks, sg, cv, sv


def pin_qlr_lossless(seed=20):
    """Both branches quantised: with lossless inputs the first stage's integer
    sums, its per-token re-quantisation and the output are known in closed
    form, and Y equals X R + (X U) V exactly."""
    rng = np.random.default_rng(seed)
    n, d, m, rk, a = 5, 48, 7, 4, -3
    x, r, u, v, cx, sx, ks, sg, cv, sv = _qlr_lossless_case(rng, n, d, m, rk, a)
    out = tqo.tq_linear_qlr_ref(x, r, u, v)
    assert np.array_equal(out["codes_u"], np.diag(sg) @ np.eye(d, dtype=np.int64)[ks])
    assert np.array_equal(out["s_u"], np.full(rk, 2.0 ** a, np.float32))
    acc1 = cx[:, ks] * sg[None, :]
    assert np.array_equal(out["acc1"], acc1)
    # t = acc1 2^a, every token's max |t| = 49 2^a: s_t = 7 2^a, codes = acc1 / 7
    assert np.array_equal(out["s_t"], np.full(n, 7 * 2.0 ** a, np.float32))
    assert np.array_equal(out["codes_t"], acc1 // 7)
    x64, r64, u64, v64 = (t.astype(np.float64) for t in (x, r, u, v))
    assert np.array_equal(out["Y"], x64 @ r64 + (x64 @ u64) @ v64)
    # V = 0 leaves the plain W4A4 layer
    assert np.array_equal(tqo.tq_linear_qlr_ref(x, r, u, np.zeros_like(v))["Y"], tqo.tq_linear_ref(x, r)["Y"])
    # a lossy re-quantisation known in closed form: both rank columns read
    # input channel 0, the second at half the first (7 2^a and 3.5 2^a), so
    # every token's first stage is (t0, t0 / 2) with |t0| = 49 2^a: s_t = 7 2^a
    # and the codes are +-7 and +-4 (3.5 rounds half to even), i.e. the second
    # column comes back as 4/7 of the first instead of 1/2
    u2 = np.zeros((d, 2), np.float32)
    u2[0] = [7 * 2.0 ** a, 3.5 * 2.0 ** a]
    v2 = (lossless_codes(rng, m, 2, 7) * sv[:, None]).T.astype(np.float32)
    o2 = tqo.tq_linear_qlr_ref(x, r, u2, v2)
    sgn = np.sign(cx[:, 0])
    assert np.array_equal(o2["codes_t"], np.stack([7 * sgn, 4 * sgn], axis=1))
    that = np.stack([sgn * 49.0, sgn * 28.0], axis=1) * (sx.astype(np.float64) * 2.0 ** a)[:, None]
    want = x64 @ r64 + that @ v2.astype(np.float64)
    assert np.allclose(o2["Y"], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def pin_qlr_invariants(seed=21):
    """Power-of-two rescalings that the definition passes through exactly:
    a token row of X scales its row of Y; U -> 2^k U scales the low-rank term
    by 2^k; a column of U keeps its codes and scales only its own s_u (U is
    quantised per column); a column of V scales its column of the low-rank
    term and keeps its codes (V per column); a permutation of the rank
    columns (U's columns with V's rows) changes nothing; U = 0 removes the
    branch."""
    rng = np.random.default_rng(seed)
    n, d, m, rk = 6, 64, 9, 5
    x = rng.standard_normal((n, d)).astype(np.float32)
    r = (0.02 * rng.standard_normal((d, m))).astype(np.float32)
    u = rng.standard_normal((d, rk)).astype(np.float32) * (2.0 ** rng.integers(-3, 3, size=rk)).astype(np.float32)
    v = (0.05 * rng.standard_normal((rk, m))).astype(np.float32)
    out = tqo.tq_linear_qlr_ref(x, r, u, v)
    base = out["Y"]
    zr = np.zeros_like(r)
    lr = tqo.tq_linear_qlr_ref(x, zr, u, v)["Y"]
    assert np.abs(lr).max() > 0
    xs = x.copy()
    xs[2] *= 8.0
    xs[4] *= 0.25
    want = base.copy()
    want[2] *= 8.0
    want[4] *= 0.25
    assert np.array_equal(tqo.tq_linear_qlr_ref(xs, r, u, v)["Y"], want)
    assert np.array_equal(tqo.tq_linear_qlr_ref(x, zr, 4.0 * u, v)["Y"], 4.0 * lr)
    us = u.copy()
    us[:, 1] *= 16.0
    o2 = tqo.tq_linear_qlr_ref(x, r, us, v)
    assert np.array_equal(o2["codes_u"], out["codes_u"])
    want_su = out["s_u"].copy()
    want_su[1] *= 16.0
    assert np.array_equal(o2["s_u"], want_su)
    vs = v.copy()
    vs[:, 2] *= 4.0
    vs[:, 7] *= 0.125
    o3 = tqo.tq_linear_qlr_ref(x, zr, u, vs)
    assert np.array_equal(o3["codes_v"], out["codes_v"])
    want = lr.copy()
    want[:, 2] *= 4.0
    want[:, 7] *= 0.125
    assert np.array_equal(o3["Y"], want)
    p = rng.permutation(rk)
    assert np.allclose(tqo.tq_linear_qlr_ref(x, r, u[:, p], v[p])["Y"], base, rtol=0, atol=1e-12 * np.abs(base).max())
    assert np.array_equal(tqo.tq_linear_qlr_ref(x, r, np.zeros_like(u), v)["Y"], tqo.tq_linear_ref(x, r)["Y"])
    # sampled rows / columns equal the full evaluation
    rows, cols = np.array([5, 0, 3]), np.array([8, 1, 2])
    sub = tqo.tq_linear_qlr_ref(x, r, u, v, rows=rows, cols=cols)["Y"]
    assert np.array_equal(sub, base[np.ix_(rows, cols)])


def pin_qlr_requant_step(seed=22):
    """The re-quantised first stage is a per-token symmetric 4-bit grid: every
    code in [-8, 7], some code at +-7 in each token, and |c_t s_t - t| at most
    half a step (round to nearest), on generic data with an outlier channel."""
    rng = np.random.default_rng(seed)
    n, d, m, rk = 40, 96, 11, 16
    x = rng.standard_normal((n, d))
    x[:, 5] *= 20.0
    x = x.astype(np.float32)
    u = (rng.standard_normal((d, rk)) * np.linspace(0.2, 3.0, rk)).astype(np.float32)
    v = (0.1 * rng.standard_normal((rk, m))).astype(np.float32)
    out = tqo.tq_linear_qlr_ref(x, np.zeros((d, m), np.float32), u, v)
    ct, st, t = out["codes_t"].astype(np.int64), out["s_t"].astype(np.float64), out["t"].astype(np.float64)
    assert ct.min() >= -8 and ct.max() <= 7
    assert np.all(np.abs(ct).max(axis=1) == 7)
    err = np.abs(ct * st[:, None] - t)
    assert np.all(err <= 0.5 * st[:, None] * (1 + 1e-6))
    # the rounding is to nearest: most codes sit well inside half a step
    assert np.mean(err <= 0.25 * st[:, None]) > 0.45


# ----------------------------------------------------------------------------
# asymmetric per-token activations (two-subspace layer)
# ----------------------------------------------------------------------------

def pin_asym_quantizer_bruteforce(seed=23):
    """Rows with a given min and max: s = rn32(rn32(max - min) / (2^N - 1)),
    z = min, and each code rne(rn32(rn32(x - z) / s)) clipped to [0, 2^N - 1],
    evaluated in exact rational arithmetic with IEEE rounding (rn32)."""
    rng = np.random.default_rng(seed)
    for bits in (4, 8):
        qm = (1 << bits) - 1
        for mn, mx in ((-3.0, 5.0), (0.25, 0.75), (-1.0e-3, 7.0e-3), (-12.375, -0.5), (2.0 ** -100, 3 * 2.0 ** -99)):
            vals = np.concatenate([[mn, mx], rng.uniform(mn, mx, size=200)]).astype(np.float32)
            # ties: values exactly half-way between grid points
            f_mn, f_mx = Fraction(float(np.float32(mn))), Fraction(float(np.float32(mx)))
            srange = rn32(f_mx - f_mn)
            s = rn32(srange / qm)
            halfs = [float(np.float32(float(f_mn + (Fraction(2 * j + 1, 2)) * s))) for j in range(0, qm, max(1, qm // 7))]
            row = np.concatenate([vals, np.asarray(halfs, np.float32)]).astype(np.float32)[None, :]
            u, s_got, z_got = tqo.quantize_rows_asym(row, bits)
            assert Fraction(float(s_got[0])) == s and Fraction(float(z_got[0])) == f_mn
            for x, c in zip(row[0], u[0]):
                want = min(max(rne_int(rn32(rn32(Fraction(float(x)) - f_mn) / s)), 0), qm)
                assert int(c) == want, (bits, mn, mx, float(x), int(c), want)


def _asym_lossless(rng, n, k, qm, e_lo, e_hi):
    u = rng.integers(0, qm + 1, size=(n, k)).astype(np.int64)
    u[:, 0], u[:, 1] = 0, qm  # every row spans the whole grid
    s = 2.0 ** rng.integers(e_lo, e_hi, size=n)
    z = s * rng.integers(-3 * qm, 2 * qm, size=n)  # a multiple of the step: x - z is exact
    return u, s, z, (u * s[:, None] + z[:, None])


def pin_asym_two_subspace_lossless(seed=24):
    """Inputs that quantise without loss (each row z + u s with u spanning
    [0, 2^N - 1], s a power of two, z a multiple of s): codes, scales and
    zero-points are known and Y = X_l W_l + X_h W_h exactly; a per-row shift
    by a multiple of the step moves only z and adds shift * s_w * colsum(C_w);
    a constant row has s = 0, codes 0 and dequantises to its value."""
    rng = np.random.default_rng(seed)
    n, dl, dh, m = 5, 64, 32, 7
    ul, sl, zl, xl = _asym_lossless(rng, n, dl, 15, -5, 1)
    uh, sh, zh, xh = _asym_lossless(rng, n, dh, 255, -9, -4)
    cwl = lossless_codes(rng, m, dl, 7)
    cwh = lossless_codes(rng, m, dh, 127)
    swl = 2.0 ** rng.integers(-8, -3, size=m)
    swh = 2.0 ** rng.integers(-12, -8, size=m)
    wl, wh = (cwl * swl[:, None]).T, (cwh * swh[:, None]).T
    xrot = np.hstack([xl, xh]).astype(np.float32)
    wrot = np.vstack([wl, wh]).astype(np.float32)
    out = tqo.tq_linear_mp_asym_ref(xrot, wrot, dh)
    assert np.array_equal(out["codes_xl"], ul) and np.array_equal(out["codes_xh"], uh)
    assert np.array_equal(out["s_xl"], sl.astype(np.float32)) and np.array_equal(out["z_xl"], zl.astype(np.float32))
    assert np.array_equal(out["s_xh"], sh.astype(np.float32)) and np.array_equal(out["z_xh"], zh.astype(np.float32))
    assert np.array_equal(out["colsum_l"], cwl.sum(axis=1)) and np.array_equal(out["colsum_h"], cwh.sum(axis=1))
    assert np.array_equal(out["Y"], xl @ wl + xh @ wh)
    # shift row 2 of the 4-bit subspace by 5 steps
    xs = xrot.copy()
    xs[2, :dl] += np.float32(5 * sl[2])
    o2 = tqo.tq_linear_mp_asym_ref(xs, wrot, dh)
    assert np.array_equal(o2["codes_xl"], ul)
    want = out["Y"].copy()
    want[2] += 5 * sl[2] * (swl * cwl.sum(axis=1))
    assert np.array_equal(o2["Y"], want)
    # a constant row
    xc = xrot.copy()
    xc[1] = np.float32(0.375)
    o3 = tqo.tq_linear_mp_asym_ref(xc, wrot, dh)
    assert o3["s_xl"][1] == 0 and o3["s_xh"][1] == 0 and not o3["codes_xl"][1].any() and not o3["codes_xh"][1].any()
    assert np.array_equal(o3["Y"][1], 0.375 * (wl.sum(axis=0) + wh.sum(axis=0)))


def pin_asym_half_step(seed=25):
    """Generic rows (an outlier channel, all-positive rows): every code in
    [0, 2^N - 1], the row's minimum at code 0 and maximum at 2^N - 1, and the
    dequantised u s + z within half a step of x."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((30, 96))
    x[:, 7] *= 25.0
    x[::3] = np.abs(x[::3]) + 3.0
    x = x.astype(np.float32)
    for bits in (4, 8):
        qm = (1 << bits) - 1
        u, s, z = tqo.quantize_rows_asym(x, bits)
        assert u.min() >= 0 and u.max() <= qm
        assert np.all(u[np.arange(30), x.argmin(axis=1)] == 0) and np.all(u[np.arange(30), x.argmax(axis=1)] == qm)
        deq = u.astype(np.float64) * s.astype(np.float64)[:, None] + z.astype(np.float64)[:, None]
        assert np.all(np.abs(deq - x) <= 0.5 * s.astype(np.float64)[:, None] * (1 + 1e-5) + 1e-6 * np.abs(x))


# ----------------------------------------------------------------------------
# 6/3-bit two-subspace layer
# ----------------------------------------------------------------------------

def pin_two_subspace_6_3_lossless(seed=26):
    """CoQuant's other bit pair: the two-subspace output at 3 bits (low) and 6
    bits (high), q_max 3 and 31, with inputs that quantise without loss, is
    exactly X_l W_l + X_h W_h; codes at 4/8 bits of the same data differ."""
    rng = np.random.default_rng(seed)
    n, dl, dh, m = 5, 64, 16, 6
    cxl = lossless_codes(rng, n, dl, 3)
    cxh = lossless_codes(rng, n, dh, 31)
    cwl = lossless_codes(rng, m, dl, 3)
    cwh = lossless_codes(rng, m, dh, 31)
    sxl = 2.0 ** rng.integers(-4, 2, size=n)
    sxh = 2.0 ** rng.integers(-9, -5, size=n)
    swl = 2.0 ** rng.integers(-8, -3, size=m)
    swh = 2.0 ** rng.integers(-12, -8, size=m)
    xl, xh = cxl * sxl[:, None], cxh * sxh[:, None]
    wl, wh = (cwl * swl[:, None]).T, (cwh * swh[:, None]).T
    xrot = np.hstack([xl, xh]).astype(np.float32)
    wrot = np.vstack([wl, wh]).astype(np.float32)
    out = tqo.tq_linear_mp_ref(xrot, wrot, dh, bits_lo=3, bits_hi=6)
    assert np.array_equal(out["codes_xl"], cxl) and np.array_equal(out["codes_xh"], cxh)
    assert np.array_equal(out["codes_wl"], cwl) and np.array_equal(out["codes_wh"], cwh)
    assert np.array_equal(out["s_xl"], (sxl * 1.0).astype(np.float32))
    assert np.array_equal(out["Y"], xl @ wl + xh @ wh)
    assert not np.array_equal(tqo.tq_linear_mp_ref(xrot, wrot, dh)["codes_xl"], cxl)


def pin_asym_linear(seed=27):
    """The rank-augmented layer with asymmetric activations: with lossless
    inputs (rows z + u s spanning the 4-bit grid, R from codes) Y equals
    X R + (X L1) L2 up to the fp64 rounding of the low-rank branch, and
    exactly X R without it; its residual term is the one-subspace case of the
    asymmetric two-subspace layer; a shifted row adds shift * s_w * colsum."""
    rng = np.random.default_rng(seed)
    n, d, m, rk = 6, 64, 9, 4
    u, s, z, x = _asym_lossless(rng, n, d, 15, -5, 1)
    cw = lossless_codes(rng, m, d, 7)
    sw = 2.0 ** rng.integers(-8, -3, size=m)
    w = (cw * sw[:, None]).T
    x32, w32 = x.astype(np.float32), w.astype(np.float32)
    out = tqo.tq_linear_asym_ref(x32, w32)
    assert np.array_equal(out["codes_x"], u) and np.array_equal(out["z_x"], z.astype(np.float32))
    assert np.array_equal(out["s_x"], s.astype(np.float32)) and np.array_equal(out["colsum"], cw.sum(axis=1))
    assert np.array_equal(out["Y"], x @ w)
    l1 = rng.standard_normal((d, rk)).astype(np.float32)
    l2 = rng.standard_normal((rk, m)).astype(np.float32)
    full = tqo.tq_linear_asym_ref(x32, w32, l1, l2)["Y"]
    ref = x @ w + (x @ l1.astype(np.float64)) @ l2.astype(np.float64)
    assert np.allclose(full, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    xg = rng.standard_normal((n, d)).astype(np.float32)
    wg = (0.02 * rng.standard_normal((d, m))).astype(np.float32)
    assert np.array_equal(tqo.tq_linear_asym_ref(xg, wg)["Y"], tqo.tq_linear_mp_asym_ref(xg, wg, 0)["Y"])
    xs = x32.copy()
    xs[3] += np.float32(2 * s[3])
    o2 = tqo.tq_linear_asym_ref(xs, w32)
    want = out["Y"].copy()
    want[3] += 2 * s[3] * (sw * cw.sum(axis=1))
    assert np.array_equal(o2["codes_x"], u) and np.array_equal(o2["Y"], want)


ALL_PINS = [
    pin_quantizer_golden,
    pin_quantizer_invariants,
    pin_weight_is_per_output_channel,
    pin_pack_golden,
    pin_pack_roundtrip,
    pin_accumulator_bruteforce,
    pin_accumulator_invariants,
    pin_linear_golden,
    pin_linear_lossless,
    pin_linear_lowrank,
    pin_linear_sampling,
    pin_hadamard,
    pin_rotation_identities,
    pin_two_subspace_lossless,
    pin_group_stacking,
    pin_rht_rows,
    pin_rht_layer_rotation_invariance,
    pin_qlr_lossless,
    pin_qlr_invariants,
    pin_qlr_requant_step,
    pin_asym_quantizer_bruteforce,
    pin_asym_two_subspace_lossless,
    pin_asym_half_step,
    pin_two_subspace_6_3_lossless,
    pin_asym_linear,
]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


@pytest.mark.slow
def test_pin_quantizer_bruteforce_int4():
    pin_quantizer_bruteforce()


@pytest.mark.slow
@pytest.mark.parametrize("bits", [3, 6])
def test_pin_quantizer_bruteforce_3_6(bits):
    """The 3- and 6-bit grids of the 6/3-bit two-subspace layer, against exact rational arithmetic."""
    pin_quantizer_bruteforce(amaxes=(3.0, 0.69921875, 1.5 * 2.0 ** -100), bits=bits)


@pytest.mark.slow
def test_pin_quantizer_bruteforce_int8():
    pin_quantizer_bruteforce(amaxes=(100.0, 0.375), bits=8)
