"""Pins of the CPU oracle against facts the pages and mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle currently in use
(``oracle.lib()``) disagrees with something that does not come from the
oracle itself: the IEEE binary16 conversions of numpy, exact rational
arithmetic, hand-derived worked examples, closed forms of softmax, a
library attention routine (torch's scaled_dot_product_attention in float64)
and library sorts.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutants.py`` runs them on copies of the oracle with a planted
mistake and requires each copy to fail at least one pin.

Passages pinned:
* the codec -- "FlexGen研究学术报告", section 三.2(C) (group-wise asymmetric
  4-bit, 64 contiguous elements; the dequantised value min + code*scale, and
  the report's FP16 form of it), with binary32 and with binary16 min/scale
  planes;
* dense decode attention -- the FlexGen blog, section "解码阶段", with the
  1/sqrt(d_k) scale of eq. (2) in the efficient-inference survey notes;
* top-10% sparse attention -- the report's section 三.2(C);
* int4 weights of the decode projections -- the same report section (weights
  compressed with the same code, dequantised to FP16 before compute) and the
  blog's "解码阶段" projections;
* prefill attention -- the blog's "预填充阶段" equation, causal, over the fp16
  K and V.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers
def _expand(tokens):
    out = []
    for tok in tokens:
        if "*" in tok:
            v, n = tok.split("*")
            out += [v] * int(n)
        else:
            out.append(tok)
    return out


def load_codec_examples(name: str = "codec_examples.txt"):
    """Parse a codec fixture under tests/golden/ into a list of dicts."""
    ex, cur = [], None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            if key == "example":
                cur = {"name": rest[0]}
                ex.append(cur)
            elif key == "x":
                cur["x"] = np.array([float(v) for v in _expand(rest)], np.float16)
            elif key in ("min", "scale"):
                cur[key] = float(rest[0])
            elif key == "scale_bits":
                cur[key] = int(rest[0], 16)
            elif key == "codes":
                cur["codes"] = np.array([int(v) for v in _expand(rest)])
            elif key == "bytes":
                cur["bytes"] = np.array([int(v) for v in _expand(rest)], np.uint8)
    return ex


def unpack(codes_bytes: np.ndarray) -> np.ndarray:
    """uint8 [..., n] -> codes [..., 2n]: even element = low nibble."""
    lo = codes_bytes & 15
    hi = codes_bytes >> 4
    return np.stack([lo, hi], axis=-1).reshape(*codes_bytes.shape[:-1], -1).astype(np.int64)


def _groups(seed: int, n: int = 64) -> list[np.ndarray]:
    """Varied fp16 groups: normal, uniform, outliers, tiny, huge, ties, duplicates."""
    r = np.random.default_rng(seed)
    gs = []
    for _ in range(n):
        kind = r.integers(0, 7)
        if kind == 0:
            x = r.standard_normal(64)
        elif kind == 1:
            x = r.uniform(-5, 5, 64)
        elif kind == 2:
            x = r.standard_normal(64)
            x[r.integers(0, 64, 2)] *= 40.0
        elif kind == 3:
            x = r.standard_normal(64) * 1e-6          # fp16 subnormals
        elif kind == 4:
            x = r.uniform(-60000, 60000, 64)
        elif kind == 5:
            x = r.integers(-3, 4, 64).astype(float) * 0.25   # many duplicates
        else:
            x = np.full(64, r.standard_normal())
            x[r.integers(0, 64)] += 1.0
        gs.append(x.astype(np.float16))
    return gs


def _exact(x16) -> list[Fraction]:
    return [Fraction(float(v)) for v in np.asarray(x16, np.float16)]


# ------------------------------------------------------ binary16 conversions
def pin_f16_to_f32_exhaustive():
    """Every one of the 65536 binary16 bit patterns widens exactly as numpy's IEEE conversion."""
    L = oracle.lib()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([L.oracle_f16_to_f32(int(b)) for b in bits], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def pin_f32_to_f16_round_to_nearest_even():
    """Narrowing agrees with numpy's IEEE RNE conversion on every binary16 value, every
    midpoint between neighbours (exact ties), values one binary32 ulp off each midpoint,
    the overflow edge and random binary32 values across the whole range."""
    L = oracle.lib()
    all16 = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    fin = all16[np.isfinite(all16)].astype(np.float64)
    fin = np.unique(fin)
    mids = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)          # exact in binary32
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    edges = np.array([65504, 65519.996, 65520, 65536, 1e9, -65520, 2.0 ** -25, 2.0 ** -26,
                      3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25], np.float32)
    r = np.random.default_rng(7)
    rnd = (r.standard_normal(20000) * np.exp(r.uniform(-20, 12, 20000))).astype(np.float32)
    vals = np.concatenate([fin.astype(np.float32), mids, up, dn, edges, rnd])
    vals = vals[r.permutation(vals.size)[:60000]] if vals.size > 60000 else vals
    vals = np.concatenate([vals, edges, mids[::97], mids[-50:], mids[:50]])
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([L.oracle_f32_to_f16(float(v)) for v in vals], np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (vals[bad[:5]], got[bad[:5]], ref[bad[:5]])


# --------------------------------------------------------------------- codec
def pin_codec_worked_examples():
    """Hand-derived examples in tests/golden/codec_examples.txt (ties to even, signed
    zeros, constant groups, fp16 extremes, nibble order)."""
    for ex in load_codec_examples():
        codes, mn, sc = oracle.quantize_group(ex["x"])
        got = unpack(codes[None])[0]
        assert np.array_equal(got, ex["codes"]), (ex["name"], got, ex["codes"])
        assert np.float32(mn).tobytes() == np.float32(ex["min"]).tobytes(), (ex["name"], mn)
        if "scale" in ex:
            assert np.float32(sc).tobytes() == np.float32(ex["scale"]).tobytes(), (ex["name"], sc)
        else:
            xs = ex["x"].astype(np.float64)
            exact = Fraction(float(xs.max())) - Fraction(float(xs.min()))
            assert abs(Fraction(float(sc)) - exact / 15) <= exact / 15 * Fraction(1, 2 ** 22)
        if "bytes" in ex:
            assert np.array_equal(codes, ex["bytes"]), (ex["name"], codes)


def pin_codec_nearest_level_bruteforce():
    """Each code is the nearest of the 16 levels min + c*scale (exact rational distances);
    only values within 1e-5 of a level midpoint may take either neighbour."""
    for x in _groups(11, 80):
        codes, mn, sc = oracle.quantize_group(x)
        c = unpack(codes[None])[0]
        xs = _exact(x)
        lo, hi = min(xs), max(xs)
        if hi == lo:
            assert sc == 0 and not c.any()
            continue
        for xi, ci in zip(xs, c):
            r = (xi - lo) * 15 / (hi - lo)              # exact position on the code axis
            dist = [abs(r - k) for k in range(16)]
            best = min(dist)
            assert dist[ci] <= best + Fraction(1, 100000), (float(r), ci)
            if abs(r - math.floor(r) - Fraction(1, 2)) > Fraction(1, 100000):
                assert dist[ci] == best, (float(r), ci)


def pin_codec_extremes_and_scale():
    """Stored min is the exact group minimum; the minimum maps to code 0 and the maximum
    to code 15; scale is (max - min)/15 within two binary32 roundings."""
    for x in _groups(12, 80):
        codes, mn, sc = oracle.quantize_group(x)
        c = unpack(codes[None])[0]
        xs = _exact(x)
        lo, hi = min(xs), max(xs)
        assert Fraction(float(mn)) == lo
        if lo == 0:
            assert np.float32(mn).tobytes() == np.float32(0.0).tobytes()   # +0, never -0
        if hi == lo:
            continue
        assert c[int(np.argmin(x))] == 0 and c[int(np.argmax(x))] == 15
        exact = (hi - lo) / 15
        assert abs(Fraction(float(sc)) - exact) <= abs(exact) * Fraction(1, 2 ** 22)


def pin_codec_error_bound():
    """Dequantised error per element: |x - (min + c*scale)| <= scale/2 (+ binary32 slack)."""
    for x in _groups(13, 80):
        codes, mn, sc = oracle.quantize_group(x)
        xhat = oracle.dequant_rows(codes[None], np.array([[mn]], np.float32), np.array([[sc]], np.float32))[0]
        xs = x.astype(np.float64)
        c = unpack(codes[None])[0]
        big = max(abs(xs.max()), abs(xs.min()))
        assert np.array_equal(xhat, float(mn) + c * float(sc))
        assert np.all(np.abs(xs - xhat) <= float(sc) / 2 * (1 + 1e-5) + big * 2.0 ** -22)


def pin_codec_fp16_form():
    """The report's FP16 form of a dequantised value is the binary16 value nearest to
    fl32(fl32(c*scale) + min) (numpy's IEEE conversion), so within half an fp16 ulp."""
    for x in _groups(16, 40):
        codes, mn, sc = oracle.quantize_group(x)
        c = unpack(codes[None])[0]
        x16 = oracle.dequant_rows_f16(codes[None], np.array([[mn]], np.float32), np.array([[sc]], np.float32))[0]
        v32 = (c.astype(np.float32) * np.float32(sc)).astype(np.float32) + np.float32(mn)
        with np.errstate(over="ignore"):
            ref = v32.astype(np.float32).astype(np.float16)
        assert np.array_equal(x16.view(np.uint16), ref.view(np.uint16))


def pin_codec_constant_group_roundtrip():
    """A constant group stores scale 0 and codes 0 and dequantises to itself exactly."""
    r = np.random.default_rng(14)
    for v in list(r.standard_normal(20)) + [0.0, -0.0, 65504.0, -65504.0, 6e-8, -3.5]:
        x = np.full(64, v, np.float16)
        codes, mn, sc = oracle.quantize_group(x)
        assert sc == 0 and not codes.any()
        xhat = oracle.dequant_rows(codes[None], np.array([[mn]], np.float32), np.array([[sc]], np.float32))[0]
        assert np.array_equal(xhat, x.astype(np.float64))


def pin_codec_params_are_correctly_rounded_quotients():
    """The scale and inverse the codec stores / codes with ([FG-report] 三.2(C)): with binary32
    metadata the IEEE binary32 quotients rng/15 and 15/rng, with binary16 metadata rng/15
    rounded to binary16 by numpy and its binary32 reciprocal -- numpy's float32 division is
    the correctly rounded quotient.  Ranges: log-uniform over every binade the codec can meet
    (2^-24 .. 2^17) plus binade edges; and the same values appear in quantize_group's stored
    scale for groups {0, .., rng}."""
    rr = np.random.default_rng(2024)
    e = rr.uniform(-24.0, 17.0, 200_000)
    r = np.exp2(e).astype(np.float32)
    edges = np.array([2.0 ** k for k in range(-24, 18)], np.float32)
    r = np.concatenate([r, edges, np.nextafter(edges, np.float32(0)), np.nextafter(edges, np.float32(1e9))])
    r = r[(r >= np.float32(2.0 ** -24)) & (r <= np.float32(2.0 ** 17))].astype(np.float32)
    s32, i32 = oracle.codec_params(r, "f32")
    assert np.array_equal(s32, r / np.float32(15)), "binary32 scale is not rng/15"
    assert np.array_equal(i32, np.float32(15) / r), "binary32 inverse is not 15/rng"
    s16, i16 = oracle.codec_params(r, "f16")
    want_s = (r / np.float32(15)).astype(np.float16).astype(np.float32)
    assert np.array_equal(s16, want_s), "binary16 scale is not rng/15 rounded to binary16"
    with np.errstate(divide="ignore"):
        want_i = np.where(want_s != 0, np.float32(1) / want_s, np.float32(0)).astype(np.float32)
    assert np.array_equal(i16, want_i), "binary16-metadata inverse is not 1/scale (0 for scale 0)"
    # the group quantisers store these scales: a group {0, v} has range v
    for v in (np.float16(1.0), np.float16(0.3), np.float16(6.0e-8), np.float16(65504.0), np.float16(2.0e-5)):
        g = np.zeros(oracle.GROUP, np.float16)
        g[7] = v
        _, _, sc = oracle.quantize_group(g)
        assert sc == oracle.codec_params(np.array([np.float32(v)]), "f32")[0][0]
        _, _, sc16 = oracle.quantize_group_m16(g)
        assert np.float32(sc16) == oracle.codec_params(np.array([np.float32(v)]), "f16")[0][0]


def pin_codec_rows_are_groupwise():
    """A row of d = 64*G values is G independent groups of 64 contiguous head_dim elements
    (group axis = head_dim), laid out group after group."""
    r = np.random.default_rng(15)
    x = (r.standard_normal((3, 5, 256)) * r.uniform(0.1, 10, (3, 5, 1))).astype(np.float16)
    codes, mins, scales = oracle.quantize_rows(x)
    assert codes.shape == (3, 5, 128) and mins.shape == (3, 5, 4)
    for i in range(3):
        for j in range(5):
            for g in range(4):
                c1, m1, s1 = oracle.quantize_group(x[i, j, 64 * g:64 * g + 64])
                assert np.array_equal(codes[i, j, 32 * g:32 * g + 32], c1)
                assert mins[i, j, g] == m1 and scales[i, j, g] == s1


def pin_codec_m16_rows_are_groupwise():
    """With binary16 metadata too, a row of d = 64*G values is G independent groups of 64
    contiguous head_dim elements: every group of a [3, 5, 256] tensor (rows of different
    ranges, so neighbouring groups differ) equals the one-group codec on its own 64 values,
    its 32 code bytes at byte 32g of the row and its min and scale at slot g."""
    r = np.random.default_rng(25)
    x = (r.standard_normal((3, 5, 256)) * r.uniform(0.1, 10, (3, 5, 1))
         * np.repeat(r.uniform(0.2, 5, (3, 5, 4)), 64, axis=2)).astype(np.float16)
    x[1, 2, 64:128] = 0.5                                   # one constant group mid-row
    codes, mins, scales = oracle.quantize_rows_m16(x)
    assert codes.shape == (3, 5, 128) and mins.shape == (3, 5, 4) and scales.shape == (3, 5, 4)
    assert mins.dtype == np.float16 and scales.dtype == np.float16
    for i in range(3):
        for j in range(5):
            for g in range(4):
                c1, m1, s1 = oracle.quantize_group_m16(x[i, j, 64 * g:64 * g + 64])
                assert np.array_equal(codes[i, j, 32 * g:32 * g + 32], c1), (i, j, g)
                assert mins[i, j, g].view(np.uint16) == m1.view(np.uint16), (i, j, g)
                assert scales[i, j, g].view(np.uint16) == s1.view(np.uint16), (i, j, g)
    # the stored pair of each group is that group's own minimum and range (not a neighbour's)
    xs = x.astype(np.float32).reshape(3, 5, 4, 64)
    assert np.array_equal(mins.view(np.uint16), (xs.min(-1) + np.float32(0)).astype(np.float16).view(np.uint16))


# ------------------------------------------------ codec, binary16 metadata
def pin_codec_m16_worked_examples():
    """Hand-derived examples in tests/golden/codec_m16_examples.txt (scale rounded to
    binary16, codes against the stored scale, underflow to 0, subnormal-scale clamp)."""
    for ex in load_codec_examples("codec_m16_examples.txt"):
        codes, mn, sc = oracle.quantize_group_m16(ex["x"])
        got = unpack(codes[None])[0]
        assert np.array_equal(got, ex["codes"]), (ex["name"], got, ex["codes"])
        assert mn.view(np.uint16) == np.float16(ex["min"]).view(np.uint16), (ex["name"], mn)
        assert int(sc.view(np.uint16)) == ex["scale_bits"], (ex["name"], hex(int(sc.view(np.uint16))))
        assert float(sc) == ex["scale"], (ex["name"], sc)
        if "bytes" in ex:
            assert np.array_equal(codes, ex["bytes"]), (ex["name"], codes)


def pin_codec_m16_stored_pair_is_library_rounding():
    """The stored min is the group minimum (exact, +0 for a zero minimum) and the stored
    scale is numpy's IEEE binary16 rounding of the binary32 quotient (max - min)/15."""
    for x in _groups(17, 120):
        codes, mn, sc = oracle.quantize_group_m16(x)
        x32 = x.astype(np.float32)
        lo, hi = x32.min() + np.float32(0), x32.max() + np.float32(0)
        assert mn.view(np.uint16) == np.float16(lo).view(np.uint16)
        rng = np.float32(hi - lo)
        ref = np.float16(np.float32(rng / np.float32(15))) if rng != 0 else np.float16(0)
        assert sc.view(np.uint16) == ref.view(np.uint16), (sc, ref)


def pin_codec_m16_nearest_level_bruteforce():
    """Each code is the nearest of the 16 levels min + c*scale of the STORED binary16 pair
    (exact rational distances; values within 1e-5 of a midpoint may take either
    neighbour); a stored scale of 0 gives codes 0."""
    r = np.random.default_rng(18)
    groups = _groups(19, 80)
    for i in range(40):     # tiny ranges: subnormal scales, and (range < 7.5 * 2^-24) scales that underflow to 0
        g = np.zeros(64)
        g[r.integers(0, 64, 4)] = r.integers(1, 40 if i % 2 else 8, 4) * 2.0 ** -24
        groups.append(g.astype(np.float16))
    for x in groups:
        codes, mn, sc = oracle.quantize_group_m16(x)
        c = unpack(codes[None])[0]
        xs = _exact(x)
        s16 = Fraction(float(sc))
        assert Fraction(float(mn)) == min(xs)
        if s16 == 0:
            assert not c.any()
            continue
        for xi, ci in zip(xs, c):
            pos = (xi - min(xs)) / s16
            dist = [abs(pos - k) for k in range(16)]
            best = min(dist)
            assert dist[ci] <= best + Fraction(1, 100000), (float(pos), ci)
            if abs(pos - math.floor(pos) - Fraction(1, 2)) > Fraction(1, 100000):
                assert dist[ci] == best, (float(pos), ci)


def pin_codec_m16_error_bound():
    """|x - (min + c*scale)| <= scale/2 for the stored scale, plus what the clamp at code 15
    leaves when the binary16 scale rounded down (max - (min + 15*scale)); with a stored
    scale of 0 the error is at most the group's range."""
    for x in _groups(20, 80):
        codes, mn, sc = oracle.quantize_group_m16(x)
        c = unpack(codes[None])[0]
        xs = x.astype(np.float64)
        xhat = float(mn) + c * float(sc)
        rng = xs.max() - xs.min()
        if float(sc) == 0:
            assert np.all(np.abs(xs - xhat) <= rng)
            continue
        over = max(0.0, rng - 15 * float(sc))
        assert np.all(np.abs(xs - xhat) <= float(sc) / 2 * (1 + 1e-5) + over + abs(xs).max() * 2.0 ** -22)


# ------------------------------------------------------------- int4 weights
def _load_w_examples():
    out = []
    with open(os.path.join(GOLDEN, "w_dequant_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                c, mn, sc, exp = line.split()
                out.append((int(c), float(mn), float(sc), float(exp)))
    return out


def pin_w_dequant_worked_examples():
    """Hand-derived FP16 forms of dequantised weights (tests/golden/w_dequant_examples.txt):
    ties to even at both signs, exact cases, a subnormal scale, overflow to inf."""
    for c, mn, sc, exp in _load_w_examples():
        got = oracle.w_dequant(c, mn, sc)
        assert np.float16(mn) == mn and np.float16(sc) == sc
        assert got.view(np.uint16) == np.float16(exp).view(np.uint16), (c, mn, sc, got, exp)


def pin_w_dequant_is_library_rounding():
    """For weights quantised by the binary16-metadata codec, the dequantised value equals
    numpy's IEEE binary16 rounding of min + code*scale taken in binary64 (exact here: the
    terms' binary exponents differ by less than 30)."""
    r = np.random.default_rng(33)
    W = (r.standard_normal((40, 256)) * np.exp(r.uniform(-6, 6, (40, 1)))).astype(np.float16)
    codes, mins, scales = oracle.quantize_weight(W)
    c = unpack(codes)
    for n in range(0, 40, 3):
        for k in range(0, 256, 7):
            g = k // 64
            m64, s64 = float(mins[n, g]), float(scales[n, g])
            ref = np.float16(m64 + c[n, k] * s64)
            got = oracle.w_dequant(int(c[n, k]), mins[n, g], scales[n, g])
            assert got.view(np.uint16) == ref.view(np.uint16), (n, k, got, ref)


def _w_hat_numpy(codes, mins, scales):
    c = unpack(codes).astype(np.float64)
    g = np.repeat(np.arange(c.shape[1] // 64), 64)
    return (mins.astype(np.float64)[:, g] + c * scales.astype(np.float64)[:, g]).astype(np.float16)


def pin_w_gemm_matches_library_matmul():
    """y = x W^T equals numpy's float64 matmul with the dequantised binary16 weights
    (dequantised here by numpy's own conversion)."""
    r = np.random.default_rng(34)
    for M, N, K in [(1, 5, 64), (3, 16, 192), (9, 7, 512)]:
        W = r.standard_normal((N, K)).astype(np.float16)
        x = r.standard_normal((M, K)).astype(np.float16)
        codes, mins, scales = oracle.quantize_weight(W)
        ref = x.astype(np.float64) @ _w_hat_numpy(codes, mins, scales).astype(np.float64).T
        got = oracle.gemm_w4a16(x, codes, mins, scales)
        assert np.allclose(got, ref, rtol=1e-13, atol=1e-12), np.abs(got - ref).max()


def pin_w_gemm_one_hot_and_fractions():
    """x = e_k picks column k of W^ exactly; a tiny case equals the exact rational sum."""
    r = np.random.default_rng(35)
    N, K = 6, 128
    W = r.standard_normal((N, K)).astype(np.float16)
    codes, mins, scales = oracle.quantize_weight(W)
    What = _w_hat_numpy(codes, mins, scales)
    for k in (0, 63, 64, 127):
        x = np.zeros((1, K), np.float16)
        x[0, k] = 1.0
        assert np.array_equal(oracle.gemm_w4a16(x, codes, mins, scales)[0], What[:, k].astype(np.float64))
    x = r.standard_normal((2, K)).astype(np.float16)
    y = oracle.gemm_w4a16(x, codes, mins, scales)
    for m in range(2):
        for n in range(N):
            exact = sum(Fraction(float(x[m, k])) * Fraction(float(What[n, k])) for k in range(K))
            assert abs(Fraction(y[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 60)


# ----------------------------------------------------------------- attention
def _rand_head(seed: int, T: int, d: int, std=1.0, kfix=None):
    r = np.random.default_rng(seed)
    K = (r.standard_normal((T, d)) * std).astype(np.float16)
    if kfix is not None:
        K = kfix(K)
    V = (r.standard_normal((T, d)) * std).astype(np.float16)
    q = (r.standard_normal(d) * std).astype(np.float16)
    kc, kmin, ksc = oracle.quantize_rows(K)
    vc, vmin, vsc = oracle.quantize_rows(V)
    hc = oracle.HeadCache(kc, kmin, ksc, vc, vmin, vsc)
    Kh = oracle.dequant_rows(kc, kmin, ksc)
    Vh = oracle.dequant_rows(vc, vmin, vsc)
    return q, K, V, hc, Kh, Vh


def _sdpa(q, Kh, Vh, mask=None):
    """torch's attention routine in float64 on the CPU (default scale 1/sqrt(d))."""
    qt = torch.from_numpy(np.asarray(q, np.float64).reshape(1, 1, 1, -1))
    kt = torch.from_numpy(np.ascontiguousarray(Kh)).reshape(1, 1, *Kh.shape)
    vt = torch.from_numpy(np.ascontiguousarray(Vh)).reshape(1, 1, *Vh.shape)
    am = None
    if mask is not None:
        am = torch.from_numpy(mask).reshape(1, 1, 1, -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=am).reshape(-1).numpy()


def pin_attention_matches_library_sdpa():
    """Dense attention equals torch's float64 scaled_dot_product_attention on the
    dequantised K and V (pins the 1/sqrt(d) scale, the softmax and P.V)."""
    for seed, T, d, std in [(21, 1, 64, 1.0), (22, 7, 64, 1.0), (23, 33, 128, 0.5), (24, 130, 128, 3.0),
                            (25, 20, 256, 1.0), (26, 64, 64, 8.0)]:
        q, K, V, hc, Kh, Vh = _rand_head(seed, T, d, std)
        ref = _sdpa(q.astype(np.float64), Kh, Vh)
        got = oracle.attend(q, hc)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), np.abs(got - ref).max()
        for Tp in (1, max(1, T // 2)):
            ref = _sdpa(q.astype(np.float64), Kh[:Tp], Vh[:Tp])
            assert np.allclose(oracle.attend(q, hc, Tp), ref, rtol=1e-12, atol=1e-12)


def pin_scores_match_library_matmul():
    """Scores are q . k_t / sqrt(d) over the dequantised keys (library matmul in float64)."""
    q, K, V, hc, Kh, Vh = _rand_head(31, 50, 128, 1.0)
    ref = (Kh @ q.astype(np.float64)) / math.sqrt(128)
    assert np.allclose(oracle.scores(q, hc), ref, rtol=1e-13, atol=1e-13)


def pin_attention_single_token():
    """T = 1: softmax of one score is 1, so the output is the dequantised V row exactly."""
    for seed, d in [(41, 64), (42, 128)]:
        q, K, V, hc, Kh, Vh = _rand_head(seed, 5, d, 2.0)
        assert np.array_equal(oracle.attend(q, hc, 1), Vh[0])


def pin_attention_identical_keys_and_zero_query():
    """Identical keys (or q = 0) give a uniform softmax: the output is the mean of the
    dequantised V, and within the codec's error bound of the mean of V itself."""
    for seed, T, d in [(51, 9, 64), (52, 100, 128)]:
        q, K, V, hc, Kh, Vh = _rand_head(seed, T, d, 1.0, kfix=lambda K: np.repeat(K[:1], K.shape[0], 0))
        mean_hat = Vh.mean(axis=0)
        got = oracle.attend(q, hc)
        assert np.allclose(got, mean_hat, rtol=0, atol=1e-12)
        vc_, vmin, vsc = hc.vc, hc.vmin, hc.vsc
        bound = vsc.max() / 2 * (1 + 1e-5) + np.abs(V.astype(np.float64)).max() * 2.0 ** -22
        assert np.all(np.abs(got - V.astype(np.float64).mean(axis=0)) <= bound)
        z = np.zeros(d, np.float16)
        q2, K2, V2, hc2, Kh2, Vh2 = _rand_head(seed + 100, T, d, 1.0)
        assert np.allclose(oracle.attend(z, hc2), Vh2.mean(axis=0), rtol=0, atol=1e-12)


def pin_attention_two_token_closed_form():
    """T = 2: out = (v0 + e^D v1) / (1 + e^D) with D = (s1 - s0), s_t = q.k_t/sqrt(d)."""
    q, K, V, hc, Kh, Vh = _rand_head(61, 2, 128, 1.5)
    s = Kh @ q.astype(np.float64) / math.sqrt(128)
    D = s[1] - s[0]
    ref = (Vh[0] + math.exp(D) * Vh[1]) / (1 + math.exp(D))
    assert np.allclose(oracle.attend(q, hc), ref, rtol=1e-12, atol=1e-13)


def pin_attention_fp16_form_matches_library_sdpa():
    """Attention over the report's FP16 form of the cache (every dequantised element rounded
    to binary16 before compute) equals torch's float64 scaled_dot_product_attention on the
    FP16-form K and V; over a token subset it equals the same routine with the other keys
    masked out; one token gives its FP16-form V row exactly; identical keys give the mean
    of the FP16-form V rows."""
    for seed, T, d, std in [(2101, 1, 64, 1.0), (2102, 9, 64, 1.0), (2103, 70, 128, 0.5), (2104, 129, 128, 3.0),
                            (2105, 33, 256, 1.0)]:
        q, K, V, hc, Kh, Vh = _rand_head(seed, T, d, std)
        K16 = oracle.dequant_rows_f16(hc.kc, hc.kmin, hc.ksc).astype(np.float64)
        V16 = oracle.dequant_rows_f16(hc.vc, hc.vmin, hc.vsc).astype(np.float64)
        ref = _sdpa(q.astype(np.float64), K16, V16)
        got = oracle.attend_f16form(q, hc)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), np.abs(got - ref).max()
        assert np.array_equal(oracle.attend_f16form(q, hc, 1), V16[0])
        if T >= 4:
            sel = np.sort(np.random.default_rng(seed).choice(T, T // 3 + 1, replace=False))
            mask = np.full(T, -np.inf)
            mask[sel] = 0.0
            ref = _sdpa(q.astype(np.float64), K16, V16, mask)
            got = oracle.attend_f16form(q, hc, idx=sel)
            assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), np.abs(got - ref).max()
    q, K, V, hc, Kh, Vh = _rand_head(2106, 40, 128, 1.0, kfix=lambda K: np.repeat(K[:1], K.shape[0], 0))
    V16 = oracle.dequant_rows_f16(hc.vc, hc.vmin, hc.vsc).astype(np.float64)
    assert np.allclose(oracle.attend_f16form(q, hc), V16.mean(axis=0), rtol=0, atol=1e-12)


# --------------------------------------------------------------------- top-k
def pin_topk_selection_matches_library_sort():
    """Selection = first k of a stable library sort by (score descending, index ascending),
    returned ascending; exercised with heavy ties."""
    r = np.random.default_rng(71)
    for T, k in [(10, 1), (10, 10), (50, 5), (300, 31), (2048, 205)]:
        for tie in (False, True):
            s = r.standard_normal(T)
            if tie:
                s = np.round(s * 2) / 2
            order = np.lexsort((np.arange(T), -s))
            ref = np.sort(order[:k])
            assert np.array_equal(oracle.select_topk(s, k), ref)


def pin_topk_full_equals_dense_and_top1_is_argmax():
    """k = T reduces to dense attention; k = 1 returns the dequantised V row of the
    highest-scoring key (smallest index on ties)."""
    q, K, V, hc, Kh, Vh = _rand_head(81, 40, 128, 1.0)
    out, sel = oracle.attend_topk(q, hc, 40)
    assert np.array_equal(sel, np.arange(40))
    assert np.allclose(out, oracle.attend(q, hc), rtol=1e-13, atol=1e-14)
    s = Kh @ q.astype(np.float64)
    out1, sel1 = oracle.attend_topk(q, hc, 1)
    assert sel1[0] == int(np.argmax(s)) and np.array_equal(out1, Vh[sel1[0]])


def pin_topk_matches_masked_library_sdpa():
    """Top-k output equals torch's float64 attention with every unselected key masked
    out (-inf), i.e. the softmax renormalised over the kept keys."""
    boost = lambda K: K * np.where(np.random.default_rng(5).random((K.shape[0], 1)) < 0.05, 3, 1).astype(np.float16)
    for seed, T, d in [(91, 200, 128), (92, 64, 64), (93, 2048, 128)]:
        q, K, V, hc, Kh, Vh = _rand_head(seed, T, d, 1.0, kfix=boost)
        k = math.ceil(0.1 * T)
        out, sel = oracle.attend_topk(q, hc, k)
        s = Kh @ q.astype(np.float64)
        order = np.lexsort((np.arange(T), -s))
        assert np.array_equal(sel, np.sort(order[:k]))
        mask = np.full(T, -np.inf)
        mask[sel] = 0.0
        ref = _sdpa(q.astype(np.float64), Kh, Vh, mask)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
        assert np.allclose(oracle.attend_subset(q, hc, sel), ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ prefill attention
def _prompt(seed: int, s: int, d: int, std=1.0):
    r = np.random.default_rng(seed)
    return tuple((r.standard_normal((s, d)) * std).astype(np.float16) for _ in range(3))


def _causal_sdpa(Q, K, V):
    """torch's attention routine in float64 on the CPU with its causal mask."""
    t = [torch.from_numpy(np.ascontiguousarray(x, np.float64)).reshape(1, 1, *x.shape) for x in (Q, K, V)]
    return torch.nn.functional.scaled_dot_product_attention(*t, is_causal=True).reshape(Q.shape).numpy()


def pin_prefill_matches_library_causal_sdpa():
    """Prefill attention equals torch's float64 scaled_dot_product_attention with
    is_causal=True on the fp16 Q, K, V (pins the mask, the 1/sqrt(d) scale, the softmax
    and P.V), including a strided head of a [s][a][d] batch row."""
    for seed, s, d, std in [(1001, 1, 64, 1.0), (1002, 7, 64, 1.0), (1003, 65, 128, 0.5), (1004, 130, 128, 3.0),
                            (1005, 20, 256, 1.0), (1006, 64, 64, 8.0)]:
        Q, K, V = _prompt(seed, s, d, std)
        got = oracle.prefill_attend(Q, K, V)
        ref = _causal_sdpa(Q, K, V)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), np.abs(got - ref).max()
    r = np.random.default_rng(1007)
    X = [(r.standard_normal((40, 3, 64))).astype(np.float16) for _ in range(3)]
    got = oracle.prefill_attend(X[0][:, 1], X[1][:, 1], X[2][:, 1])
    assert np.allclose(got, _causal_sdpa(X[0][:, 1], X[1][:, 1], X[2][:, 1]), rtol=1e-12, atol=1e-12)


def pin_prefill_selected_rows_match_library_causal_sdpa():
    """The row-selected prefill attention returns, for each requested query row, that row of
    torch's float64 causal scaled_dot_product_attention (rows in any order, repeated, first
    and last)."""
    Q, K, V = _prompt(1031, 150, 128, 1.0)
    ref = _causal_sdpa(Q, K, V)
    rows = np.array([149, 0, 63, 64, 64, 127, 128, 1, 100], np.int32)
    got = oracle.prefill_attend_rows(Q, K, V, rows)
    assert np.allclose(got, ref[rows], rtol=1e-12, atol=1e-12), np.abs(got - ref[rows]).max()


def pin_prefill_rows_are_decode_steps():
    """With K and V the codec reproduces exactly (every group holds the levels
    min + c*scale for c = 0..15 with scale a power of two), prefill row i equals the
    pinned decode attention of q_i over the cache of tokens 0..i."""
    r = np.random.default_rng(1011)
    s, d = 37, 128
    def lossless():
        c = r.integers(0, 16, (s, d))
        c[:, 0::64], c[:, 1::64] = 0, 15                      # every group spans all 16 levels
        off = np.repeat(r.integers(-8, 8, (s, d // 64)), 64, axis=1)
        return ((c + off) * 0.25).astype(np.float16)
    K, V = lossless(), lossless()
    Q = r.standard_normal((s, d)).astype(np.float16)
    kc, kmin, ksc = oracle.quantize_rows(K)
    vc, vmin, vsc = oracle.quantize_rows(V)
    assert np.array_equal(oracle.dequant_rows(kc, kmin, ksc), K.astype(np.float64))
    assert np.array_equal(oracle.dequant_rows(vc, vmin, vsc), V.astype(np.float64))
    hc = oracle.HeadCache(kc, kmin, ksc, vc, vmin, vsc)
    got = oracle.prefill_attend(Q, K, V)
    for i in range(s):
        assert np.allclose(got[i], oracle.attend(Q[i], hc, i + 1), rtol=1e-12, atol=1e-12), i


def pin_prefill_closed_forms():
    """Row 0 is v_0 exactly; identical keys (or a zero query) give row i = the mean of
    v_0..v_i; two tokens give row 1 = (v0 + e^D v1)/(1 + e^D), D = (q1.k1 - q1.k0)/sqrt(d)."""
    Q, K, V = _prompt(1021, 50, 128, 1.5)
    Vd = V.astype(np.float64)
    got = oracle.prefill_attend(Q, K, V)
    assert np.array_equal(got[0], Vd[0])
    prefix_mean = np.cumsum(Vd, axis=0) / np.arange(1, 51)[:, None]
    Ksame = np.repeat(K[:1], 50, axis=0)
    assert np.allclose(oracle.prefill_attend(Q, Ksame, V), prefix_mean, rtol=0, atol=1e-12)
    Qzero = np.zeros_like(Q)
    assert np.allclose(oracle.prefill_attend(Qzero, K, V), prefix_mean, rtol=0, atol=1e-12)
    q1 = Q[1].astype(np.float64)
    D = (q1 @ K[1].astype(np.float64) - q1 @ K[0].astype(np.float64)) / math.sqrt(128)
    ref = (Vd[0] + math.exp(D) * Vd[1]) / (1 + math.exp(D))
    assert np.allclose(got[1], ref, rtol=1e-12, atol=1e-13)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
