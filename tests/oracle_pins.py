"""Pins of the CPU oracle to facts the pages and mathematics fix.

Each ``pin_*`` function takes the oracle module and raises AssertionError when
the oracle disagrees with something other than itself: hand-worked examples of
the pages' definitions, the numbers the pages print (tests/golden/), exact
rational arithmetic (fractions.Fraction, mpmath at 50 digits), closed forms,
invariants, identities the pages state, and special cases that reduce to a
library routine.  ``test_oracle_pins.py`` runs them on the oracle;
``test_oracle_mutations.py`` runs them on copies of the oracle with plausible
mistakes planted, and expects each mistake to be caught.

Pages: [P1] "KV Cache Quantization Perturbs Attention Through Stored Keys and
Values"; [P2] "KV cache quantization reduces cache bytes with separate accuracy
and kernel costs"; [P3] "KV Cache Quantization and Per-Token Scale Placement".
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import mpmath
import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# Exact helpers (independent of the oracle: rational arithmetic only)
# ---------------------------------------------------------------------------
def exact_round_float(fr: Fraction, p: int, emin: int) -> Fraction:
    """Round a rational to the nearest binary float with p significant bits and
    minimum normal exponent emin (subnormals included), ties to even."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (p - 1))
    return sign * round(a / quantum) * quantum   # round(): ties to even


def rn32(fr):
    return exact_round_float(Fraction(fr), 24, -126)


def rn16(fr):
    return exact_round_float(Fraction(fr), 11, -14)


def rn64(fr):
    return exact_round_float(Fraction(fr), 53, -1022)


def fr(x) -> Fraction:
    return Fraction(float(x))


def exact_sym(vec, bits, scale_round):
    """Symmetric quantizer of one vector in exact arithmetic.  scale_round maps
    the exact amax/qmax to the stored scale."""
    qmax = (1 << (bits - 1)) - 1
    xs = [fr(v) for v in vec]
    amax = max(abs(v) for v in xs)
    if amax == 0:
        return [0] * len(xs), Fraction(1)
    s = scale_round(amax / qmax)
    return [max(-qmax, min(qmax, round(v / s))) for v in xs], s


def exact_asym(vec, bits):
    qmax = (1 << bits) - 1
    xs = [fr(v) for v in vec]
    lo = min(min(xs), Fraction(0))
    hi = max(max(xs), Fraction(0))
    if hi == lo:
        return [0] * len(xs), Fraction(1), 0
    s = rn16((hi - lo) / qmax)
    z = max(0, min(qmax, round(-lo / s)))
    return [max(0, min(qmax, round(v / s) + z)) for v in xs], s, z


def _rng(seed):
    return np.random.default_rng(seed)


def _bf16(x):
    """Values exact in bf16, rounded by torch (a library routine, not the oracle)."""
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _f32(x):
    return np.asarray(x, np.float32).astype(np.float64)


def _random_vectors(n, d, seed, magnitudes=(1e-3, 1.0, 37.0, 1e4)):
    rng = _rng(seed)
    out = []
    for i in range(n):
        m = magnitudes[i % len(magnitudes)]
        v = rng.standard_normal(d) * m
        if i % 3 == 0:
            v[rng.integers(d)] *= 10.0      # an outlier entry sets the max
        out.append(_f32(v))
    return np.stack(out)


def _near_ties(s, n, seed):
    """fp32 values within a few ulps of (k + 1/2) * s, with s an fp32 scale."""
    rng = _rng(seed)
    k = rng.integers(-120, 120, n)
    x = ((k + 0.5) * s).astype(np.float32)
    steps = rng.integers(-3, 4, n)
    x = np.array([np.nextafter(np.float32(v), np.float32(np.sign(st) * np.inf)) if st else v
                  for v, st in zip(x, steps)], dtype=np.float32)
    return x.astype(np.float64)


# ---------------------------------------------------------------------------
# Hand-worked examples of the pages' definitions
# ---------------------------------------------------------------------------
def pin_hand_examples(O):
    """Small vectors whose scale is a power of two, worked by hand from P2
    "Quantization needs a scale convention" and P3 "The axis choice is a kernel
    decision" (scale = amax/qmax, round ties to even, clamp)."""
    # amax 127 -> scale exactly 1; halves go to the even neighbour.
    c, s = O.quantize_sym(np.array([127, -63.5, 31.75, 0.5, -1.5, 2.5, 0, -127.0]), 8, "f32")
    assert float(s) == 1.0 and c.tolist() == [127, -64, 32, 0, -2, 2, 0, -127], (c, s)
    # amax 254 -> scale exactly 2.
    c, s = O.quantize_sym(np.array([254.0, 3.0, -5.0, 1.0]), 8, "f32")
    assert float(s) == 2.0 and c.tolist() == [127, 2, -2, 0], (c, s)
    # all-zero vector: codes 0, scale 1.
    c, s = O.quantize_sym(np.zeros(6), 8, "f32")
    assert float(s) == 1.0 and c.tolist() == [0] * 6
    # 4-bit symmetric: qmax 7, amax 7 -> scale 1.
    c, s = O.quantize_sym(np.array([7.0, -3.5, 2.5, 0.5, 1.75, -7.0]), 4, "f32")
    assert float(s) == 1.0 and c.tolist() == [7, -4, 2, 0, 2, -7], (c, s)
    # zero point, range [-7.5, 7.5] -> s 1, z = rint(7.5) = 8; 7.5 -> 16 clamps.
    c, s, z = O.quantize_asym(np.array([-7.5, 0.0, 7.5, 3.75, -2.5]), 4, "f16")
    assert float(s) == 1.0 and float(z) == 8.0 and c.tolist() == [0, 8, 15, 12, 6], (c, s, z)
    # all-positive vector: the range is widened to include 0, so z = 0.
    c, s, z = O.quantize_asym(np.array([1.0, 2.0, 3.0, 15.0]), 4, "f16")
    assert float(s) == 1.0 and float(z) == 0.0 and c.tolist() == [1, 2, 3, 15]
    # odd zero point: rint(x/s) + z, not rint(x/s + z): 0.5 -> 0 + 3, 1.5 -> 2 + 3.
    c, s, z = O.quantize_asym(np.array([-3.0, 12.0, 0.5, 1.5]), 4, "f16")
    assert float(s) == 1.0 and float(z) == 3.0 and c.tolist() == [0, 15, 3, 5], (c, s, z)
    # per-channel key scales: channel absmax 127 and 254 -> scales 1 and 2.
    k = np.array([[127.0, -254.0], [-63.5, 127.0], [0.5, 3.0]])
    sc = O.channel_scales(k, 8)
    assert sc.tolist() == [1.0, 2.0], sc
    assert O.quantize_with_channel_scales(k, sc, 8).tolist() == [[127, -127], [-64, 64], [0, 2]]
    # super-scale: sigma = amax / 7 = [255, 0.5, 0] -> S = 255/255 = 1;
    # u = [255, rint(0.5)=0 -> clamp 1, 0 for the zero vector].
    v = np.array([[1785.0, -892.5, 0.0], [3.5, -1.0, 0.5], [0.0, 0.0, 0.0]])
    S = O.super_scale(v, 4)
    assert float(S) == 1.0, S
    codes, u = O.quantize_superscaled(v, S, 4)
    assert u.tolist() == [255, 1, 0], u
    assert codes.tolist() == [[7, -4, 0], [4, -1, 0], [0, 0, 0]], codes


def pin_rounding_ties(O):
    """The numbers tests/golden/rounding_ties.json lists for Python's round(),
    which P3's quantizer listing uses."""
    g = json.load(open(os.path.join(GOLDEN, "rounding_ties.json")))
    xs = np.array([c[0] for c in g["cases"]])
    want = [c[1] for c in g["cases"]]
    got = O.rne_quotient(xs, 1.0)
    assert [int(v) for v in got] == want, (got, want)
    assert [round(x) for x in xs.tolist()] == want   # the listing's primitive


# ---------------------------------------------------------------------------
# Exact rational arithmetic
# ---------------------------------------------------------------------------
def pin_sym_exact(O):
    """Symmetric codes and scales equal exact rational evaluation: with an fp64
    scale this is P3's quantizer listing evaluated exactly (Python's float
    division is correctly rounded, round() ties to even); with an fp32 scale the
    scale is the exactly rounded amax/qmax (R2)."""
    vecs = _random_vectors(48, 128, 11)
    for bits in (8, 4, 2):
        for scale, rnd in (("f64", rn64), ("f32", rn32)):
            codes, s = O.quantize_sym(vecs, bits, scale)
            for i, v in enumerate(vecs):
                ec, es = exact_sym(v, bits, rnd)
                assert Fraction(float(s[i])) == es, (bits, scale, i)
                assert codes[i].tolist() == ec, (bits, scale, i)


def pin_near_ties(O):
    """Quotients within a few ulps of a half-integer round like the exact
    quotient (R1): fp32 division would get some of these wrong."""
    rng = _rng(5)
    for trial in range(24):
        s = np.float32(rng.uniform(0.003, 0.03))
        x = _near_ties(s, 64, 100 + trial)
        x[0] = 127.0 * float(s) * (1 + 1e-7)       # keeps amax/127 close to s
        codes, st = O.quantize_sym(x, 8, "f32")
        ec, es = exact_sym(x, 8, rn32)
        assert Fraction(float(st)) == es
        assert codes.tolist() == ec, trial


def pin_exact_ties(O):
    """Exact ties (k + 1/2) * s go to the even neighbour, for both signs."""
    for e in range(-6, 7):
        s = 2.0 ** e
        k = np.arange(-126, 126)
        x = np.concatenate([[127 * s], (k + 0.5) * s])
        codes, st = O.quantize_sym(x, 8, "f32")
        assert float(st) == s
        want = [127] + [int(2 * round((kk + 0.5) / 2)) for kk in k]
        assert codes.tolist() == want, e


def pin_asym_exact(O):
    """Zero-point codes, fp16 scales and zero points equal exact evaluation of
    reading R6 (4 and 2 bits); x = 0 reconstructs exactly; codes stay in
    [0, 2^b - 1]; every unclamped element is within s/2 of its
    reconstruction."""
    vecs = _random_vectors(40, 128, 23, magnitudes=(0.05, 1.0, 9.0, 300.0))
    vecs[5] = np.abs(vecs[5])          # one-signed vectors
    vecs[6] = -np.abs(vecs[6])
    vecs[7, :] = 0.0
    vecs[8, 3] = 0.0
    for bits in (4, 2):
        top = (1 << bits) - 1
        codes, s, z = O.quantize_asym(vecs, bits, "f16")
        for i, v in enumerate(vecs):
            ec, es, ez = exact_asym(v, bits)
            assert Fraction(float(s[i])) == es, (bits, i)
            assert float(z[i]) == ez, (bits, i)
            assert codes[i].tolist() == ec, (bits, i)
        assert codes.min() >= 0 and codes.max() <= top
        xh = O.dequant_asym(codes, s, z)
        assert np.all(xh[vecs == 0.0] == 0.0)
        err = np.abs(xh - vecs)
        sd = s.astype(np.float64)[:, None]
        unclamped = (codes > 0) & (codes < top)
        assert np.all(err[unclamped] <= sd.repeat(128, 1)[unclamped] / 2 * (1 + 1e-12))


def _nearest_code(x: Fraction, s: Fraction, lo: int, hi: int, z: int = 0) -> int:
    """Brute force: the code c in [lo, hi] whose grid point s (c - z) is
    nearest to x, ties to the even c - z (independent of any rint / clamp)."""
    best = None
    for c in range(lo, hi + 1):
        d = abs(x - s * (c - z))
        key = (d, (c - z) % 2)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def pin_storage_limits(O):
    """Reading R4 at the storage types' limits, in exact arithmetic: a scale
    whose fp64 value rounds to 0 stores the type's smallest positive value
    (fp16 2^-24, fp32 2^-149), an fp16 scale above 65504 stores 65504, and
    fp16 scales in the subnormal range round to multiples of 2^-24.  Codes
    are then the nearest points of the grid of the stored scale (brute force
    over every code, ties to even, at 8, 4 and 2 bits, with and without a
    zero point), so x_hat = c s_stored stays exact."""
    F16_TINY, F32_TINY = Fraction(1, 2 ** 24), Fraction(1, 2 ** 149)
    cases = []
    for bits in (8, 4, 2):
        qs, qu = (1 << (bits - 1)) - 1, (1 << bits) - 1
        # fp16: underflow (exact quotient below 2^-25), the tie 2^-25, the
        # subnormal range (3.3 * 2^-24), overflow (beyond 65520) and the
        # largest finite value's neighbourhood (65510 rounds to 65504)
        for target, want in ((Fraction(1, 2 ** 27), F16_TINY), (Fraction(1, 2 ** 25), F16_TINY),
                             (Fraction(33, 10 * 2 ** 24), Fraction(3, 2 ** 24)),
                             (Fraction(10 ** 6), Fraction(65504)), (Fraction(65510), Fraction(65504))):
            cases += [("f16", bits, target, want, False), ("f16", bits, target, want, True)]
        # fp32 (inputs exact in fp32): amax = k 2^-149 with k < qmax / 2, so
        # amax / qmax lies below 2^-150 and rounds to 0; and a quotient in
        # the subnormal range (7 2^-147, exact)
        for zp, q in ((False, qs), (True, qu)):
            if q >= 3:
                cases.append(("f32", bits, Fraction((q - 1) // 2, q * 2 ** 149), F32_TINY, zp))
            cases.append(("f32", bits, Fraction(7, 2 ** 147), Fraction(7, 2 ** 147), zp))
    rng = _rng(211)
    ran = {"f16": 0, "f32": 0}
    for scale, bits, target, want, zp in cases:
        qs, qu = (1 << (bits - 1)) - 1, (1 << bits) - 1
        if True:
            qmax = qu if zp else qs
            amax = target * qmax            # exact: amax / qmax == target
            famax = float(amax)
            if Fraction(famax) != amax or (scale == "f32" and Fraction(float(np.float32(famax))) != amax):
                continue                    # only inputs exact in the input type
            # a vector with that max, negative entries and values on and
            # between grid points of the expected stored scale
            v = [famax, -famax / 3, famax / 7, 0.0]
            v += [float(Fraction(k, 2) * want) for k in range(-2 * qs, 2 * qs + 1, 3)
                  if abs(Fraction(k, 2) * want) <= amax]
            v += list(rng.uniform(-famax, famax, 6))
            if scale == "f32":
                v = [float(np.float32(x)) for x in v]
            xs = [Fraction(x) for x in v]
            if zp:
                c, st, z = O.quantize_asym(np.array(v), bits, scale)
                lo = min(min(xs), Fraction(0))
                hi = max(max(xs), Fraction(0))
                span = (hi - lo) / qmax
                # the zero-point scale is (hi - lo) / qmax; recompute the
                # expected stored value for that quotient from the same rule
                exp_s = _stored(span, scale)
                assert Fraction(float(st)) == exp_s, (scale, bits, float(span), float(st))
                ez = max(0, min(qmax, round(-lo / exp_s)))
                assert Fraction(float(z)) == ez, (scale, bits, float(z), ez)
                want_c = [_nearest_code(x, exp_s, 0, qmax, ez) for x in xs]
            else:
                c, st = O.quantize_sym(np.array(v), bits, scale)
                assert Fraction(float(st)) == want, (scale, bits, float(target), float(st))
                want_c = [_nearest_code(x, want, -qs, qs) for x in xs]
            assert [int(x) for x in c] == want_c, (scale, bits, zp, float(target))
            ran[scale] += 1
    assert ran["f16"] >= 24 and ran["f32"] >= 9, ran   # every limit case ran


def _stored(q: Fraction, scale: str) -> Fraction:
    """Reading R4 written out: RN to the type (subnormals included), 0 ->
    smallest positive value, fp16 above 65504 -> 65504."""
    if scale == "f16":
        r = rn16(q)
        if r == 0:
            return Fraction(1, 2 ** 24)
        return min(r, Fraction(65504))
    r = rn32(q)
    return Fraction(1, 2 ** 149) if r == 0 else r


def pin_sym_closed_form(O):
    """The largest-magnitude element maps to +-qmax, every element is within s/2
    of its reconstruction, codes never reach -2^(b-1), s = RN32(amax/qmax)."""
    vecs = _random_vectors(64, 128, 31)
    for bits in (8, 4, 2):
        qmax = (1 << (bits - 1)) - 1
        codes, s = O.quantize_sym(vecs, bits, "f32")
        xh = O.dequant_sym(codes, s)
        sd = s.astype(np.float64)[:, None]
        assert np.all(np.abs(xh - vecs) <= sd / 2 * (1 + 1e-12))
        assert codes.min() >= -qmax and codes.max() <= qmax
        imax = np.argmax(np.abs(vecs), axis=1)
        top = codes[np.arange(len(vecs)), imax]
        assert np.all(np.abs(top) == qmax)
        assert np.all(np.sign(top) == np.sign(vecs[np.arange(len(vecs)), imax]))
        for i in range(0, 64, 7):
            assert Fraction(float(s[i])) == rn32(Fraction(float(np.max(np.abs(vecs[i])))) / qmax)


def pin_channel(O):
    """Per-channel key scales (P3 "Per-token scales and where they can live",
    reading R9) equal RN32(channel absmax / 127) exactly; codes equal exact
    rounding; a later token beyond the prefill range clamps; and moving the
    scales onto the query (P3 "The axis choice is a kernel decision") gives the
    scores of the dequantized keys exactly in rational arithmetic."""
    rng = _rng(41)
    k = _f32(rng.standard_normal((9, 16)) * np.array([1.0] * 12 + [10.0] * 4))
    sc = O.channel_scales(k, 8)
    for d in range(16):
        assert Fraction(float(sc[d])) == rn32(Fraction(float(np.max(np.abs(k[:, d])))) / 127)
    codes = O.quantize_with_channel_scales(k, sc, 8)
    for t in range(9):
        for d in range(16):
            assert codes[t, d] == max(-127, min(127, round(fr(k[t, d]) / fr(sc[d]))))
    later = k[:1] * 3.0
    lc = O.quantize_with_channel_scales(later, sc, 8)
    assert np.all(np.abs(lc) <= 127) and np.any(np.abs(lc) == 127)
    q = _f32(rng.standard_normal(16))
    folded = [sum(fr(q[d]) * fr(sc[d]) * int(codes[t, d]) for d in range(16)) for t in range(9)]
    kh = O.dequant_channel(codes, sc)
    got = O.scores(q, kh) * math.sqrt(16)
    for t in range(9):
        assert abs(Fraction(float(got[t])) - folded[t]) <= abs(folded[t]) * Fraction(1, 10 ** 13) + Fraction(1, 10 ** 300)


def pin_superscale(O):
    """8-bit scale codes relative to a per-head super-scale (reading R10), at
    4 and 2 bits: S = RN32(max_t(amax_t/qmax)/255); u in [1, 255] for non-zero
    vectors and 0 for zero vectors; u equals exact rint(amax/(qmax S))
    clamped; codes equal exact rounding under u*S; metadata is 1 byte per
    token."""
    v = _f32(_rng(53).laplace(0, 1, (64, 128)) * np.exp(_rng(54).uniform(-6, 2, (64, 1))))
    v[10] = 0.0
    amax = [Fraction(float(np.max(np.abs(r)))) for r in v]
    for bits in (4, 2):
        qmax = (1 << (bits - 1)) - 1
        S = O.super_scale(v, bits)
        assert Fraction(float(S)) == rn32(max(a / qmax for a in amax) / 255)
        codes, u = O.quantize_superscaled(v, S, bits)
        for t in range(64):
            if amax[t] == 0:
                assert u[t] == 0 and not codes[t].any()
                continue
            eu = max(1, min(255, round(amax[t] / qmax / Fraction(float(S)))))
            assert u[t] == eu, (bits, t)
            se = eu * Fraction(float(S))
            assert codes[t].tolist() == [max(-qmax, min(qmax, round(fr(x) / se))) for x in v[t]], t
            if eu > 1:
                assert abs(se - amax[t] / qmax) <= Fraction(float(S)) / 2
        fmt = O.TensorFormat(bits, "token", False, "u8_super")
        assert O.meta_bytes_per_token(fmt) == 1


def pin_fold(O):
    """P3 "The axis choice is a kernel decision": with a per-token key scale,
    scaling the integer dot product once equals the dot product with the
    dequantized key.  The oracle's score of each dequantized key equals the
    folded score computed exactly, to 1e-13 relative."""
    rng = _rng(61)
    kv = _random_vectors(12, 64, 62)
    codes, s = O.quantize_sym(kv, 8, "f32")
    q = _f32(rng.standard_normal(64))
    got = O.scores(q, O.dequant_sym(codes, s))
    for t in range(12):
        acc = sum(fr(q[d]) * int(codes[t, d]) for d in range(64))   # integer-code dot
        want = acc * fr(s[t])                                       # one multiply per score
        g = Fraction(float(got[t])) * 8   # * sqrt(64)
        assert abs(g - want) <= abs(want) * Fraction(1, 10 ** 13), t


# ---------------------------------------------------------------------------
# Attention: library routine, identities, special cases, brute force
# ---------------------------------------------------------------------------
def _sdpa_reference(q, k, v):
    """torch's scaled_dot_product_attention on the CPU in fp64, one query."""
    import torch
    hq, d = q.shape
    hkv = k.shape[0]
    g = hq // hkv
    kk = torch.from_numpy(np.repeat(k, g, axis=0))[None]      # [1, Hq, T, D]
    vv = torch.from_numpy(np.repeat(v, g, axis=0))[None]
    qq = torch.from_numpy(q)[None, :, None, :]                # [1, Hq, 1, D]
    out = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)
    return out[0, :, 0, :].numpy()


def pin_exact_cache(O):
    """With stored unquantized values (bits 16), attention over the cache is
    standard attention (P1 "Key error acts before the softmax"): equal to
    torch's scaled_dot_product_attention in fp64 to 1e-12."""
    rng = _rng(71)
    for (hq, hkv, t) in ((4, 1, 33), (8, 2, 200), (2, 2, 1), (6, 3, 7)):
        k = _bf16(rng.standard_normal((hkv, t, 32)) * 3)
        v = _bf16(rng.standard_normal((hkv, t, 32)))
        q = rng.standard_normal((hq, 32))
        cache = O.OracleCache(1, hkv, 32, O.TensorFormat(16), O.TensorFormat(16))
        cache.append(0, k, v)
        got = cache.attend(0, q)
        assert np.max(np.abs(got - _sdpa_reference(q, k, v))) < 1e-12, (hq, hkv, t)


def pin_identity_key(O):
    """P1 "Key error acts before the softmax": with keys stored as K + E_K the
    scores are s + q E_K^T / sqrt(d)."""
    rng = _rng(81)
    k = _f32(rng.standard_normal((50, 128)) * 2)
    codes, s = O.quantize_sym(k, 4, "f32")
    kh = O.dequant_sym(codes, s)
    q = _f32(rng.standard_normal(128))
    ek = kh - k
    lhs = O.scores(q, kh)
    rhs = (k @ q) / math.sqrt(128) + (ek @ q) / math.sqrt(128)
    assert np.max(np.abs(lhs - rhs)) < 1e-12


def pin_identity_value(O):
    """P1 "Value error acts after attention weights are formed": with exact
    keys and values stored as V + E_V, the output is o + a E_V."""
    rng = _rng(91)
    k = rng.standard_normal((1, 70, 128))
    v = _f32(rng.standard_normal((1, 70, 128)))
    codes, s = O.quantize_sym(v, 4, "f32")
    vh = O.dequant_sym(codes, s)
    q = rng.standard_normal((1, 128))
    a = O.attention_weights(q, k)[0]
    o = O.attend(q, k, v)[0]
    o2 = O.attend(q, k, vh)[0]
    assert np.max(np.abs(o2 - (o + a @ (vh[0] - v[0])))) < 1e-12


def pin_softmax_weights(O):
    """Attention weights are non-negative and sum to one (the output is a
    convex combination, P3 "Keys and values are not symmetric")."""
    rng = _rng(101)
    for t in (1, 5, 300):
        a = O.attention_weights(rng.standard_normal((4, 64)), rng.standard_normal((2, t, 64)) * 5)
        assert np.all(a >= 0) and np.max(np.abs(a.sum(axis=1) - 1)) < 1e-12


def pin_single_token(O):
    """One cached token: its weight is 1 and the output is its value."""
    rng = _rng(111)
    cache = O.OracleCache(1, 2, 128, O.TensorFormat(8), O.TensorFormat(4, zero_point=True, scale="f16"))
    k = _f32(rng.standard_normal((2, 1, 128)))
    v = _f32(rng.standard_normal((2, 1, 128)))
    cache.append(0, k, v)
    _, vh = cache.reconstructed(0)
    out = cache.attend(0, rng.standard_normal((4, 128)))
    assert np.array_equal(out, np.repeat(vh[:, 0, :], 2, axis=0))


def pin_uniform_keys(O):
    """Identical keys give uniform weights: the output is the mean of v_hat."""
    rng = _rng(121)
    t = 37
    kv = np.repeat(_f32(rng.standard_normal((1, 1, 128))), t, axis=1)
    v = _f32(rng.standard_normal((1, t, 128)))
    cache = O.OracleCache(1, 1, 128, O.TensorFormat(8), O.TensorFormat(8))
    cache.append(0, kv, v)
    _, vh = cache.reconstructed(0)
    out = cache.attend(0, rng.standard_normal((1, 128)))
    assert np.max(np.abs(out[0] - vh[0].mean(axis=0))) < 1e-12


def pin_gqa_mapping(O):
    """Grouped-query heads (reading R8): query head h attends KV head h // G,
    the same as repeating each KV head G times and running one head each."""
    rng = _rng(125)
    k = rng.standard_normal((3, 20, 16))
    v = rng.standard_normal((3, 20, 16))
    q = rng.standard_normal((12, 16))
    got = O.attend(q, k, v)
    for h in range(12):
        one = O.attend(q[h:h + 1], k[h // 4:h // 4 + 1], v[h // 4:h // 4 + 1])
        assert np.array_equal(got[h], one[0])
    assert np.max(np.abs(got - _sdpa_reference(q, k, v))) < 1e-12


def pin_brute_force(O):
    """Whole pipeline on tiny shapes against exact arithmetic: codes by
    rational rounding, scores and softmax with mpmath at 50 digits."""
    mpmath.mp.dps = 50
    rng = _rng(131)
    for d in (1, 2, 4):
        for t in (1, 2, 3):
            for trial in range(3):
                k = np.round(rng.standard_normal((1, t, d)) * 64) / 16     # dyadic
                v = np.round(rng.standard_normal((1, t, d)) * 64) / 16
                q = np.round(rng.standard_normal((2, d)) * 64) / 16
                cache = O.OracleCache(1, 1, d, O.TensorFormat(8), O.TensorFormat(4, zero_point=True, scale="f16"))
                cache.append(0, k, v)
                got = cache.attend(0, q)
                kh, vh = [], []
                for i in range(t):
                    c, s = exact_sym(k[0, i], 8, rn32)
                    kh.append([ci * s for ci in c])
                    c, s, z = exact_asym(v[0, i], 4)
                    vh.append([(ci - z) * s for ci in c])
                for h in range(2):
                    sc = [mpmath.mpf(sum(fr(q[h, j]) * kh[i][j] for j in range(d)).numerator)
                          / sum(fr(q[h, j]) * kh[i][j] for j in range(d)).denominator / mpmath.sqrt(d)
                          for i in range(t)]
                    m = max(sc)
                    e = [mpmath.exp(x - m) for x in sc]
                    z_ = sum(e)
                    for j in range(d):
                        o = sum(e[i] * mpmath.mpf(vh[i][j].numerator) / vh[i][j].denominator
                                for i in range(t)) / z_
                        assert abs(float(o) - got[h, j]) <= 1e-13 * max(1.0, abs(float(o))), (d, t, h, j)


def pin_drift(O):
    """P3 "What degrades first": per-token scales follow drifting magnitudes by
    construction.  Scaling a vector by a power of two scales its scale and
    leaves its codes unchanged, for magnitudes growing along the sequence."""
    rng = _rng(141)
    base = _f32(rng.standard_normal((40, 128)))
    growth = 2.0 ** np.arange(0, 40, 1)[:, None] / 2 ** 20   # x ~1e-6 .. ~5e5
    x = base * growth
    c0, s0 = O.quantize_sym(base, 8, "f32")
    c1, s1 = O.quantize_sym(x, 8, "f32")
    assert np.array_equal(c0, c1)
    assert np.array_equal(s1.astype(np.float64), s0.astype(np.float64) * growth[:, 0])
    ca, sa, za = O.quantize_asym(base, 4, "f16")
    cb, sb, zb = O.quantize_asym(base * 4.0, 4, "f16")
    assert np.array_equal(ca, cb) and np.array_equal(za, zb)
    assert np.array_equal(sb.astype(np.float64), sa.astype(np.float64) * 4)


def pin_window(O):
    """Reading R11 of P1 "Cache growth changes the serving trade": after a
    prefill and single-token appends, exactly the newest min(W, n) tokens are
    unquantized; the rest reconstruct as their own per-token quantization."""
    rng = _rng(151)
    w = 8
    cache = O.OracleCache(1, 2, 128, O.TensorFormat(8), O.TensorFormat(8), window=w)
    allk = _bf16(rng.standard_normal((2, 30, 128)))
    allv = _bf16(rng.standard_normal((2, 30, 128)))
    cache.append(0, allk[:, :5], allv[:, :5])          # shorter than the window
    kh, vh = cache.reconstructed(0)
    assert np.array_equal(kh, allk[:, :5]) and np.array_equal(vh, allv[:, :5])
    cache.append(0, allk[:, 5:20], allv[:, 5:20])      # crosses the window
    for t in range(20, 30):
        cache.append(0, allk[:, t:t + 1], allv[:, t:t + 1])
    kh, vh = cache.reconstructed(0)
    ck, sk = O.quantize_sym(allk[:, :30 - w], 8, "f32")
    assert np.array_equal(kh[:, :30 - w], O.dequant_sym(ck, sk))
    assert np.array_equal(kh[:, 30 - w:], allk[:, 30 - w:])
    assert np.array_equal(cache.stored(0, "k").codes, ck)


def pin_group_scales_exact(O):
    """Token groups (reading R20 of P3 "Per-token scales and where they can
    live": several tokens under one scale): each group's stored scale (and
    zero point) and its codes equal exact rational quantization of the
    group's g*D values taken as one vector, at 8, 4 and 2 bits."""
    rng = _rng(171)
    d = 8
    for g in (2, 4, 16):
        x = _bf16(rng.standard_normal((2, 3 * g, d)) * np.exp(rng.uniform(-3, 3, (2, 3 * g, 1))))
        x[0, 0:g] = 0.0                                  # an all-zero group
        for fmt in (O.TensorFormat(8), O.TensorFormat(4), O.TensorFormat(2),
                    O.TensorFormat(4, "token", True, "f16"), O.TensorFormat(2, "token", True, "f16")):
            cache = O.OracleCache(1, 2, d, fmt, fmt, group=g)
            cache.append(0, x, x)
            st = cache.stored(0, "k")
            assert st.codes.shape == (2, 3 * g, d) and st.s.shape == (2, 3)
            for h in range(2):
                for j in range(3):
                    vec = x[h, j * g:(j + 1) * g].reshape(-1)
                    codes = st.codes[h, j * g:(j + 1) * g].reshape(-1).tolist()
                    if fmt.zero_point:
                        ec, es, ez = exact_asym(vec, fmt.bits)
                        assert float(st.z[h, j]) == ez, (g, fmt, h, j)
                    else:
                        ec, es = exact_sym(vec, fmt.bits, rn32)
                    assert Fraction(float(st.s[h, j])) == es, (g, fmt, h, j)
                    assert codes == ec, (g, fmt, h, j)


def pin_group_residual(O):
    """Token groups with a window: after every append exactly
    Q = floor(max(n - W, 0) / g) * g positions are quantized and the newest
    n - Q are their bf16 values; with bf16-exact inputs the records do not
    depend on how the tokens were split into appends; g = 1 is per token."""
    rng = _rng(173)
    d = 16
    allk = _bf16(rng.standard_normal((2, 70, d)))
    allv = _bf16(rng.standard_normal((2, 70, d)) * 3)
    fmt = O.TensorFormat(2, "token", True, "f16")
    for w, g in ((0, 4), (8, 16), (16, 2)):
        one = O.OracleCache(1, 2, d, fmt, fmt, window=w, group=g)
        one.append(0, allk, allv)
        many = O.OracleCache(1, 2, d, fmt, fmt, window=w, group=g)
        n = 0
        for step in (5, 1, 1, 17, 2, 3, 1, 40):
            many.append(0, allk[:, n:n + step], allv[:, n:n + step])
            n += step
            q = O.quantized_count(n, w, g)
            assert q == max(n - w, 0) // g * g and q % g == 0
            assert many.stored(0, "k").codes.shape[1] == q, (w, g, n)
            kh, vh = many.reconstructed(0)
            assert np.array_equal(kh[:, q:], allk[:, q:n]) and np.array_equal(vh[:, q:], allv[:, q:n])
        for t in ("k", "v"):
            a, b = one.stored(0, t), many.stored(0, t)
            assert np.array_equal(a.codes, b.codes) and np.array_equal(a.s, b.s) and np.array_equal(a.z, b.z)
    per_tok = O.OracleCache(1, 2, d, fmt, fmt, window=8)
    g1 = O.OracleCache(1, 2, d, fmt, fmt, window=8, group=1)
    per_tok.append(0, allk, allv)
    g1.append(0, allk, allv)
    assert np.array_equal(per_tok.reconstructed(0)[0], g1.reconstructed(0)[0])


def pin_group_bytes(O):
    """Byte accounting with token groups: g tokens share one metadata element,
    so 2-bit codes with a 4-byte scale per 16 tokens carry 12.5 % / 16 of
    metadata at D = 128 ([P3]'s 12 % case, divided by the group size)."""
    f = O.TensorFormat(2)
    lens = [16 * 37 + 5, 16, 3, 0]
    for g in (1, 2, 16):
        b = O.cache_bytes(f, f, 1, 1, 128, lens, window=0, group=g)
        q = [O.quantized_count(n, 0, g) for n in lens]
        assert b["payload"] == sum(q) * 2 * 32
        assert b["metadata"] == sum(x // g for x in q) * 2 * 4
        assert b["window"] == sum(n - x for n, x in zip(lens, q)) * 128 * 4
    b = O.cache_bytes(f, f, 1, 1, 128, [16 * 100], group=16)
    assert Fraction(b["metadata"], b["payload"]) == Fraction(125, 1000) / 16


def pin_int_query(O):
    """Integer query (reading R21 of P3 "Precision floors and mixed cache
    formats", quantized by P3's listing in "The axis choice is a kernel
    decision"): s is the correctly rounded fp64 quotient amax/127, kept in
    fp64; each code is the round-half-even of the correctly rounded fp64
    quotient q/s, clamped (checked on constructed near-ties too, where an
    fp32 quotient or an fp32 scale rounds some codes the other way); the
    largest element maps to +-127; |q - Q s| <= s/2; an all-zero head gets
    s = 1, codes 0; and attention on the integer path is attention on Q s."""
    rng = _rng(181)
    q = _f32(rng.standard_normal((6, 64)) * np.exp(rng.uniform(-4, 4, (6, 1))))
    q[2] = 0.0
    near = []
    for trial in range(10):                       # quotients within ulps of k + 1/2
        st = np.float32(rng.uniform(0.003, 0.03))
        row = _near_ties(st, 64, 300 + trial)
        row[0] = np.float32(127.0 * float(st) * (1 + 1e-7))  # amax/127 close to st
        near.append(row)
    q = np.concatenate([q, np.stack(near)])
    codes, s = O.quantize_query_int8(q)
    flips = 0
    for h in range(len(q)):
        amax = max(abs(fr(x)) for x in q[h])
        if amax == 0:
            assert float(s[h]) == 1.0 and not codes[h].any()
            continue
        s_exact = rn64(amax / 127)
        assert Fraction(float(s[h])) == s_exact, h
        for i in range(64):
            want = max(-127, min(127, round(rn64(fr(q[h, i]) / s_exact))))
            assert codes[h, i] == want, (h, i)
            # what an fp32 scale and fp32 quotient would give
            s32 = rn32(amax / 127)
            flips += want != max(-127, min(127, round(rn32(fr(q[h, i]) / s32))))
        top = int(np.argmax(np.abs(q[h])))
        assert abs(codes[h, top]) == 127
        err = np.abs(q[h] - codes[h] * np.float64(s[h]))
        # half a step, plus the fp64 quotient's rounding (|q / s| <= 127.5 < 2^7)
        assert np.all(err <= float(s[h]) * (0.5 + 2.0 ** -45))
    assert flips > 0, "the near-tie rows do not separate fp64 from fp32 evaluation"
    # attention on the integer path equals attention on the reconstructed query
    fmt = O.TensorFormat(8)
    cache = O.OracleCache(1, 2, 64, fmt, fmt)
    k = _bf16(rng.standard_normal((2, 40, 64)))
    cache.append(0, k, k)
    qq = _bf16(rng.standard_normal((4, 64)))
    c, sq = O.quantize_query_int8(qq)
    assert np.array_equal(cache.attend(0, qq, query_bits=8),
                          cache.attend(0, c * np.asarray(sq, np.float64)[:, None]))
    assert not np.array_equal(cache.attend(0, qq, query_bits=8), cache.attend(0, qq))


def pin_bf16_from_f64(O):
    """Rounding fp64 values once to bf16 equals exact rational rounding to 8
    significant bits (ties to even), including values a hair off a bf16
    midpoint, where rounding to fp32 first would round the other way."""
    rng = _rng(191)
    xs = list(rng.standard_normal(300) * np.exp(rng.uniform(-20, 20, 300)))
    for _ in range(200):                          # midpoints +- a few fp64 ulps
        m = np.float64(np.float32(rng.standard_normal()))
        e = math.frexp(m)[1]
        mid = math.ldexp(round(math.ldexp(m, 8 - e)) + 0.5, e - 8)
        xs += [mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf),
               mid + math.ldexp(1, e - 33), mid - math.ldexp(1, e - 33)]
    got = O.round_bf16_from_f64(np.array(xs))
    for x, g in zip(xs, got):
        f = Fraction(float(x))
        if f == 0:
            assert g == 0
            continue
        e = math.floor(math.log2(abs(f)))
        while Fraction(2) ** e > abs(f):
            e -= 1
        while Fraction(2) ** (e + 1) <= abs(f):
            e += 1
        ulp = Fraction(2) ** (e - 7)
        q = f / ulp
        n = math.floor(q)
        r = q - n
        n = n + 1 if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2) else n
        assert Fraction(float(g)) == n * ulp, (x, g)
    # rounding through fp32 first gets some of the near-midpoint values wrong
    near = np.array(xs[300:])
    assert np.count_nonzero(O.round_bf16_from_f64(near) != O.round_bf16(near)) > 0


def pin_channel_scales_with_window(O):
    """Per-channel key scales with a recent window (readings R9, R11): the
    scales come from every token of the first append, also when that append
    is shorter than the window, and tokens leaving the window later are
    quantized with them (clamped)."""
    rng = _rng(201)
    d = 16
    k = _bf16(rng.standard_normal((1, 40, d)) * np.array([1.0] * 12 + [10.0] * 4))
    v = _bf16(rng.standard_normal((1, 40, d)))
    fk, fv = O.TensorFormat(8, "channel"), O.TensorFormat(4, "token", False, "u8_super")
    cache = O.OracleCache(1, 1, d, fk, fv, window=16)
    cache.append(0, k[:, :10], v[:, :10])             # shorter than the window
    st = cache.stored(0, "k")
    assert st.codes.shape[1] == 0
    for c in range(d):
        assert Fraction(float(st.chan[0, c])) == rn32(max(abs(fr(x)) for x in k[0, :10, c]) / 127)
    assert Fraction(float(cache.stored(0, "v").S[0])) == rn32(
        max(max(abs(fr(x)) for x in v[0, t]) / 7 for t in range(10)) / 255)
    for t in range(10, 40):
        cache.append(0, k[:, t:t + 1], v[:, t:t + 1])
    st = cache.stored(0, "k")
    assert st.codes.shape[1] == 40 - 16
    for t in range(24):
        for c in range(d):
            assert st.codes[0, t, c] == max(-127, min(127, round(fr(k[0, t, c]) / fr(st.chan[0, c]))))
    kh, _ = cache.reconstructed(0)
    assert np.array_equal(kh[:, 24:], k[:, 24:40])


def pin_channel_growth(O):
    """Reading R22: a channel whose new keys exceed qmax * s gets
    s' = RN32(max / 127); its stored codes become clamp(round(c s / s'))
    exactly; other channels keep theirs; the new tokens are quantized with
    the grown scales and stay within s'/2."""
    rng = _rng(203)
    d = 8
    k1 = _bf16(rng.standard_normal((2, 20, d)))
    k2 = _bf16(rng.standard_normal((2, 5, d)) * np.array([1, 1, 1, 1, 5, 5, 0.1, 9.0]))
    v = _bf16(rng.standard_normal((2, 25, d)))
    f = O.TensorFormat(8, "channel_grow")
    cache = O.OracleCache(1, 2, d, f, O.TensorFormat(8), window=0)
    cache.append(0, k1, v[:, :20])
    old_s = cache.stored(0, "k").chan.copy()
    old_c = cache.stored(0, "k").codes.copy()
    cache.append(0, k2, v[:, 20:])
    st = cache.stored(0, "k")
    for h in range(2):
        for c in range(d):
            m = max(abs(fr(x)) for x in k2[h, :, c])
            s0 = Fraction(float(old_s[h, c]))
            if m > 127 * s0:
                s1 = rn32(m / 127)
                assert Fraction(float(st.chan[h, c])) == s1, (h, c)
                for t in range(20):
                    want = max(-127, min(127, round(int(old_c[h, t, c]) * s0 / s1)))
                    assert st.codes[h, t, c] == want, (h, c, t)
            else:
                s1 = s0
                assert st.chan[h, c] == old_s[h, c]
                assert np.array_equal(st.codes[h, :20, c], old_c[h, :, c])
            for t in range(5):
                x = fr(k2[h, t, c])
                code = int(st.codes[h, 20 + t, c])
                assert code == max(-127, min(127, round(x / s1)))
                assert abs(x - code * s1) <= s1 / 2
    assert (st.chan != old_s).any() and (st.chan == old_s).any()   # both cases exercised
    frozen = O.OracleCache(1, 2, d, O.TensorFormat(8, "channel"), O.TensorFormat(8))
    frozen.append(0, k1, v[:, :20])
    frozen.append(0, k2, v[:, 20:])
    assert np.array_equal(frozen.stored(0, "k").chan, old_s)       # "channel" stays frozen


def pin_channel_hold(O):
    """Reading R26: with axis "channel_hold" the keys stay in the bf16 window
    until the first position is quantized; the channel scales are then
    RN32(max |k| / 127) over every token held at that moment (the window's
    and the new ones), not over the first append alone (R9) nor over the
    leaving or the new tokens alone; later tokens clamp.  A first append
    longer than the window gives R9's scales and codes exactly."""
    rng = _rng(205)
    d, W = 8, 16
    # channel 7 is large only in tokens 3 (held) and 25 (new in the second
    # append, stays in the window); channel 6 only in token 12 (leaves with
    # the first quantization); channel 5 only in token 2 and channel 4 only
    # in token 0 (both held since the first append)
    k = _bf16(rng.standard_normal((1, 40, d)))
    k[0, 3, 7], k[0, 25, 7], k[0, 12, 6], k[0, 2, 5], k[0, 0, 4] = 40.0, -60.0, 30.0, 20.0, 25.0
    v = _bf16(rng.standard_normal((1, 40, d)))
    fk, fv = O.TensorFormat(8, "channel_hold"), O.TensorFormat(8)
    cache = O.OracleCache(1, 1, d, fk, fv, window=W)
    cache.append(0, k[:, :10], v[:, :10])            # inside the window: nothing quantized
    assert cache.stored(0, "k").codes.shape[1] == 0
    cache.append(0, k[:, 10:30], v[:, 10:30])        # 30 tokens: positions 0..13 leave
    st = cache.stored(0, "k")
    assert st.codes.shape[1] == 30 - W
    want = [rn32(max(abs(fr(k[0, t, c])) for t in range(30)) / 127) for c in range(d)]
    assert [Fraction(float(x)) for x in st.chan[0]] == want
    for t in range(30, 40):                          # later tokens clamp to the fixed scales
        cache.append(0, k[:, t:t + 1], v[:, t:t + 1])
    st = cache.stored(0, "k")
    assert np.array_equal(st.chan[0], np.array([float(x) for x in want], np.float32))
    for t in range(40 - W):
        for c in range(d):
            assert st.codes[0, t, c] == max(-127, min(127, round(fr(k[0, t, c]) / want[c])))
    # a first append longer than the window: exactly R9 ("channel")
    a = O.OracleCache(1, 1, d, fk, fv, window=W)
    b = O.OracleCache(1, 1, d, O.TensorFormat(8, "channel"), fv, window=W)
    for c_ in (a, b):
        c_.append(0, k[:, :25], v[:, :25])
        c_.append(0, k[:, 25:27], v[:, 25:27])
    assert np.array_equal(a.stored(0, "k").chan, b.stored(0, "k").chan)
    assert np.array_equal(a.stored(0, "k").codes, b.stored(0, "k").codes)


def pin_tier_counts(O):
    """Reading R24 by brute force: a position is in the cache's format when
    its whole block of 32 positions is at least M older than the first
    window position, in bf16 when it is among the W newest, in the middle
    tier otherwise; the middle tier then holds M..M+31 positions once full and
    never more than its ring.  Its bytes follow P2's 2 L H_kv D T b per tier
    ("Cache precision is separate from weight precision")."""
    for W in (0, 16, 100):
        for M in (32, 64, 96):
            for n in range(0, 420, 7):
                q = max(n - W, 0)
                main = sum(1 for p in range(q) if 32 * (p // 32 + 1) <= q - M)
                got = O.tier_counts(n, W, M)
                assert got == (main, q - main, n - q), (W, M, n, got)
                if q >= M:
                    assert M <= got[1] <= M + 31
                assert got[1] <= O.mid_ring_slots(M)
            assert O.tier_counts(50, W, 0) == (max(50 - W, 0), 0, min(W, 50))
    k4, v4 = O.TensorFormat(4), O.TensorFormat(4)
    lens = [300, 37, 1000]
    b = O.cache_bytes(k4, v4, 2, 8, 128, lens, window=16, mid=64)
    want = 0
    for n in lens:
        a, m, _ = O.tier_counts(n, 16, 64)
        want += 2 * 2 * 8 * 128 * (a * Fraction(1, 2) + m * 1)
    assert b["payload"] == want


def _tier_stream(seed, hkv, n, d=128):
    rng = _rng(seed)
    mags = np.exp(rng.uniform(-6, 6, (hkv, n, 1)))
    x = rng.standard_normal((hkv, n, d)) * mags
    x[:, ::5, 3] *= 12.0                       # outlier entries set some maxima
    x[:, 7] = 0.0                              # an all-zero token
    return _bf16(x)


def pin_tier_requantize(O):
    """Reading R24 in exact arithmetic: a middle-tier token holds the int8
    codes and RN32 scale of its value; a token in the cache's format holds
    that format's codes of the exact middle-tier value c * s (symmetric,
    zero point, 2 and 4 bits); window tokens hold their bf16 values."""
    d, W, M = 128, 16, 64
    x = _tier_stream(301, 1, 260)
    y = _tier_stream(302, 1, 260)
    fmts = [(O.TensorFormat(4), lambda v: exact_sym(v, 4, rn32)),
            (O.TensorFormat(4, zero_point=True, scale="f16"), lambda v: exact_asym(v, 4)),
            (O.TensorFormat(2, zero_point=True, scale="f16"), lambda v: exact_asym(v, 2))]
    for fmt, exact in fmts:
        cache = O.OracleCache(1, 1, d, fmt, fmt, window=W, mid=M)
        cache.append(0, x[:, :200], y[:, :200])
        cache.append(0, x[:, 200:], y[:, 200:])
        a, m, w = O.tier_counts(260, W, M)
        assert a > 0 and m > 0 and w == W
        for t, src in (("k", x), ("v", y)):
            st = cache.stored(0, t)
            mc, ms = cache.mid_stored(0, t)
            assert st.codes.shape[1] == a and mc.shape[1] == m
            for p in range(a + m):
                c8, s8 = exact_sym(src[0, p], 8, rn32)
                if p >= a:
                    assert list(mc[0, p - a]) == c8 and Fraction(float(ms[0, p - a])) == s8, (t, p)
                    continue
                rec = [float(c * s8) for c in c8]      # exact in fp64
                want = exact(rec)
                assert list(st.codes[0, p]) == want[0], (fmt, t, p)
                assert Fraction(float(st.s[0, p])) == want[1], (fmt, t, p)
                if fmt.zero_point:
                    assert int(st.z[0, p]) == want[2]
            assert np.array_equal(cache.window_values(0, t)[0], src[0, a + m:])


def pin_tier_chunking(O):
    """Reading R24: where a token is stored depends only on its age, so the
    stored records are the same whether a stream is appended at once, token
    by token, or in uneven pieces."""
    d, W, M, n = 128, 8, 32, 150
    x = _tier_stream(303, 2, n)
    y = _tier_stream(304, 2, n)
    fmt = O.TensorFormat(4, zero_point=True, scale="f16")
    cuts = [[0, n], list(range(n + 1)), [0, 3, 40, 41, 90, 131, n]]
    caches = []
    for cut in cuts:
        c = O.OracleCache(1, 2, d, fmt, fmt, window=W, mid=M)
        for lo, hi in zip(cut[:-1], cut[1:]):
            c.append(0, x[:, lo:hi], y[:, lo:hi])
        caches.append(c)
    ref = caches[0]
    for c in caches[1:]:
        for t in ("k", "v"):
            for f in ("codes", "s", "z"):
                assert np.array_equal(getattr(c.stored(0, t), f), getattr(ref.stored(0, t), f)), (t, f)
            for i in range(2):
                assert np.array_equal(c.mid_stored(0, t)[i], ref.mid_stored(0, t)[i])
            assert np.array_equal(c.window_values(0, t), ref.window_values(0, t))
        assert np.array_equal(c.reconstructed(0)[0], ref.reconstructed(0)[0])


def pin_tier_int8_identity(O):
    """Re-quantizing an int8 reconstruction to int8 with an fp32 scale gives
    back the same codes and scale (its largest code is 127, so the scale is
    RN32(127 s / 127) = s), so an int8 cache with a middle tier equals a plain
    int8 cache with the same window; and with fewer than M + 32 tokens past
    the window the cache's format holds nothing, whatever it is."""
    d, W, M = 128, 16, 64
    x = _tier_stream(305, 2, 300)
    y = _tier_stream(306, 2, 300)
    i8 = O.TensorFormat(8)
    tier = O.OracleCache(1, 2, d, i8, i8, window=W, mid=M)
    flat = O.OracleCache(1, 2, d, i8, i8, window=W)
    for lo, hi in ((0, 120), (120, 121), (121, 300)):
        tier.append(0, x[:, lo:hi], y[:, lo:hi])
        flat.append(0, x[:, lo:hi], y[:, lo:hi])
        for u, v in zip(tier.reconstructed(0), flat.reconstructed(0)):
            assert np.array_equal(u, v)
    a = O.tier_counts(300, W, M)[0]
    assert np.array_equal(tier.stored(0, "k").codes, flat.stored(0, "k").codes[:, :a])
    q4 = O.TensorFormat(4)
    short = O.OracleCache(1, 2, d, q4, q4, window=W, mid=M)
    short.append(0, x[:, :W + M + 31], y[:, :W + M + 31])
    assert short.stored(0, "k").codes.shape[1] == 0
    for u, v in zip(short.reconstructed(0), _flat_prefix(O, x, y, W, W + M + 31)):
        assert np.array_equal(u, v)


def _flat_prefix(O, x, y, W, n):
    c = O.OracleCache(1, x.shape[0], x.shape[2], O.TensorFormat(8), O.TensorFormat(8), window=W)
    c.append(0, x[:, :n], y[:, :n])
    return c.reconstructed(0)


def pin_window_stores_bf16(O):
    """Unquantized tokens (bits 16, or the recent window) are stored in bf16:
    fp32 inputs come back rounded to nearest-even bf16 (torch's conversion)."""
    rng = _rng(155)
    x = _f32(rng.standard_normal((1, 6, 128)))
    cache = O.OracleCache(1, 1, 128, O.TensorFormat(8), O.TensorFormat(8), window=16)
    cache.append(0, x, x)
    kh, _ = cache.reconstructed(0)
    assert np.array_equal(kh, _bf16(x)) and not np.array_equal(kh, x)
    c2 = O.OracleCache(1, 1, 128, O.TensorFormat(16), O.TensorFormat(16))
    c2.append(0, x, x)
    assert np.array_equal(c2.reconstructed(0)[1], _bf16(x))


def pin_zero_point_positive_zero(O):
    """A zero point of 0 is stored as +0 (its fp16 bits are 0x0000)."""
    _, _, z = O.quantize_asym(np.array([[0.0, 1.0, 2.0], [0.0, 0.0, 0.0]]), 4, "f16")
    assert z.view(np.uint16).tolist() == [0, 0]


def pin_prefill_then_decode(O):
    """Per-channel key scales and the value super-scale are fixed by the first
    append (reading R9/R10); later single-token appends reuse them."""
    rng = _rng(161)
    cache = O.OracleCache(1, 1, 128, O.TensorFormat(8, "channel"), O.TensorFormat(4, scale="u8_super"))
    k = _f32(rng.standard_normal((1, 40, 128)))
    v = _f32(rng.laplace(0, 1, (1, 40, 128)))
    cache.append(0, k[:, :32], v[:, :32])
    sc = O.channel_scales(k[0, :32], 8)
    S = O.super_scale(v[0, :32], 4)
    for t in range(32, 40):
        cache.append(0, k[:, t:t + 1], v[:, t:t + 1])
    st = cache.stored(0, "k")
    assert np.array_equal(st.chan[0], sc)
    assert np.array_equal(st.codes[0], O.quantize_with_channel_scales(k[0], sc, 8))
    sv = cache.stored(0, "v")
    assert float(sv.S[0]) == float(S)
    c, u = O.quantize_superscaled(v[0], S, 4)
    assert np.array_equal(sv.codes[0], c) and np.array_equal(sv.u[0], u)


# ---------------------------------------------------------------------------
# Byte accounting and intensity
# ---------------------------------------------------------------------------
def pin_byte_accounting(O):
    """P2 "Cache precision is separate from weight precision": payload
    KV_bytes = 2 L H_kv D T b; halving b halves it.  P3 "Per-token scales and
    where they can live": metadata 3 / 6 / 6 / 12 percent at D = 128 (golden
    file; the page truncates 3.125 / 6.25 / 6.25 / 12.5)."""
    for (L, H, D, T, bits) in ((1, 1, 128, 512, 8), (32, 8, 128, 4096, 8), (2, 4, 64, 100, 4), (3, 2, 128, 7, 16)):
        f = O.TensorFormat(bits)
        got = O.cache_bytes(f, f, L, H, D, [T])["payload"]
        assert got == 2 * L * H * D * T * bits // 8, (L, H, D, T, bits)
    f16 = O.cache_bytes(O.TensorFormat(16), O.TensorFormat(16), 4, 8, 128, [1000])["payload"]
    f8 = O.cache_bytes(O.TensorFormat(8), O.TensorFormat(8), 4, 8, 128, [1000])["payload"]
    assert f16 == 2 * f8
    g = json.load(open(os.path.join(GOLDEN, "metadata_overhead.json")))
    for case in g["cases"]:
        bits, mb = case["code_bits"], case["meta_bytes_per_token"]
        fmt = O.TensorFormat(bits, "token", mb == 8, "f32")
        assert O.meta_bytes_per_token(fmt) == mb
        b = O.cache_bytes(fmt, fmt, 1, 1, g["head_dim"], [1000])
        pct = 100.0 * b["metadata"] / b["payload"]
        assert int(pct) == case["printed_percent"], (case, pct)
        assert pct == 100.0 * mb * 8 / (g["head_dim"] * bits)
    # closed forms of the five workloads' decode traffic (one layer)
    i8 = O.TensorFormat(8)
    assert O.decode_traffic(i8, i8, 1, 128, [512]) == 131072 + 4096
    assert O.decode_traffic(i8, i8, 8, 128, [4096] * 8) == 67108864 + 2097152
    a4 = O.TensorFormat(4, "token", True, "f16")
    assert O.decode_traffic(a4, a4, 8, 128, [8192] * 32) == 268435456 + 16777216
    kc, vs = O.TensorFormat(8, "channel"), O.TensorFormat(4, scale="u8_super")
    assert O.decode_traffic(kc, vs, 8, 128, [65536] * 16) == 1073741824 + 536870912 + 8388608 + 128 * (512 + 4)
    lens = [1024, 5000, 32768]
    assert O.decode_traffic(i8, i8, 8, 128, lens, window=128) == sum(8 * (65536 + (n - 128) * 264) for n in lens)
    pad = O.cache_bytes(i8, i8, 1, 8, 128, [145], window=128, block_tokens=16)
    # 17 quantized positions in 2 blocks: 15 unused slots (each block's 16 K
    # and 16 V fp32 scales fill one 128-byte key row, R27)
    assert pad["padding"] == 8 * (16 - 17 % 16) * 264
    pad = O.cache_bytes(a4, a4, 1, 8, 128, [145], window=128, block_tokens=16)
    # uint4 rows of 64 B: a block's 2 x 16 fp16 scale + zero point pairs
    # (128 B) fill two key rows
    assert pad["padding"] == 8 * (16 - 17 % 16) * 136
    u8s = O.TensorFormat(2, scale="u8_super")
    pad = O.cache_bytes(u8s, u8s, 1, 8, 128, [145], window=128, block_tokens=16)
    # 2-bit rows of 32 B: 2 x 16 scale codes (32 B) fill one key row
    assert pad["padding"] == 8 * (16 - 17 % 16) * 66
    kc4 = O.cache_bytes(O.TensorFormat(8, "channel"), O.TensorFormat(4, scale="u8_super"), 1, 8, 128,
                        [145], window=128, block_tokens=16)
    # per-channel keys have no per-token element: the 16 value scale codes
    # take one 128-byte key row, 112 B of it unused, in each of the 2 blocks
    assert kc4["padding"] == 8 * ((16 - 17 % 16) * 193 + 2 * 112)


def pin_allocated_bytes(O):
    """P2 "Metadata and block layout remain part of physical memory use": the
    total of payload, metadata, window and padding is what the layout
    allocates, written here from the buffer shapes alone (no per-sequence
    tier split): per (sequence, head) and layer, a contiguous cache holds
    max_tokens code rows and max_tokens / g metadata elements, a bf16 ring of
    W (+ g) slots, a middle-tier ring of M + 32 int8 rows with fp32 scales,
    and its per-head side data; a paged one holds whole 16-token blocks of
    the quantized positions (counted by brute force, position by position),
    each block a key unit of 16 key code rows plus its key and value
    metadata elements rounded up to whole key rows and a value unit of 16
    value code rows (reading R27), the same ring and side data."""
    rng = _rng(223)
    fmts = [(O.TensorFormat(8), O.TensorFormat(8)),
            (O.TensorFormat(4, zero_point=True, scale="f16"), O.TensorFormat(4, zero_point=True, scale="f16")),
            (O.TensorFormat(8, "channel"), O.TensorFormat(4, scale="u8_super")),
            (O.TensorFormat(2, scale="u8_super"), O.TensorFormat(2, scale="u8_super")),
            (O.TensorFormat(2, zero_point=True, scale="f16"), O.TensorFormat(2, zero_point=True, scale="f16"))]
    side = {"channel": lambda d: 4 * d}
    for trial in range(60):
        kf, vf = fmts[trial % len(fmts)]
        per_token = kf.axis == "token" and kf.scale != "u8_super" and vf.scale != "u8_super"
        g = int(rng.choice([1, 2, 4, 16])) if per_token else 1
        W = int(rng.choice([0, 16, 128]))
        M = int(rng.choice([0, 32, 96])) if (per_token and g == 1 and trial % 5 in (0, 1, 4)) else 0
        paged = M == 0 and trial % 2 == 1
        L, H, d, T = int(rng.integers(1, 3)), int(rng.integers(1, 4)), 128, 512
        lens = [int(x) for x in rng.integers(0, T + W, 3)]
        if M:
            lens = [min(n, T + W + M) for n in lens]
        got = O.cache_bytes(kf, vf, L, H, d, lens, window=W, block_tokens=16 if paged else 0,
                            max_tokens=None if paged else T, group=g, mid=M)
        row = d * (kf.bits + vf.bits) // 8
        meta = O.meta_bytes_per_token(kf) + O.meta_bytes_per_token(vf)   # per metadata element
        sd = (4 * d if kf.axis != "token" else 4 if kf.scale == "u8_super" else 0) + \
             (4 if vf.scale == "u8_super" else 0)
        ring = W + (g if g > 1 else 0)
        mid_bytes = (M + 32) * (2 * d + 8) if M else 0
        want = 0
        for n in lens:
            if paged:
                # a position is stored quantized when its whole group is
                # older than the window
                nq = sum(1 for p in range(n) if (p // g) * g + g <= n - W)
                blocks = -(-nq // 16)
                rk, rv = d * kf.bits // 8, d * vf.bits // 8
                m = (16 // g) * meta
                main = blocks * (16 * rk + math.ceil(m / rk) * rk + 16 * rv)
            else:
                main = T * row + (T // g) * meta
            want += L * H * (main + ring * d * 4 + mid_bytes + sd)
        assert got["total"] == want, (trial, kf, vf, g, W, M, paged, lens, got, want)
        assert got["total"] == got["payload"] + got["metadata"] + got["window"] + got["padding"]


def pin_arithmetic_intensity(O):
    """P3 "What the cache holds and how it is read": about one multiply-add per
    byte at 8 bits and two at 4 bits for one query per key (golden file)."""
    g = json.load(open(os.path.join(GOLDEN, "arith_intensity.json")))
    for case in g["cases"]:
        ai = O.arithmetic_intensity(case["code_bits"])
        assert round(ai) == case["printed_ops_per_byte"], (case, ai)
    assert abs(O.arithmetic_intensity(8) - 256 / 264) < 1e-15
    assert abs(O.arithmetic_intensity(4) - 256 / 136) < 1e-15
    assert O.multiply_adds(32, 128, [4096] * 8) == 2 * 32 * 128 * 4096 * 8


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
