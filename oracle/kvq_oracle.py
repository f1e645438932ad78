"""Plain CPU oracle for single-query decode attention over a low-bit KV cache.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import or
call anything in this package.  It shares no code, table or helper with the HIP
library and imports nothing from it.

Everything is numpy in float64 (inputs stored as bf16/fp32 upcast exactly), on
purpose slow and unblocked so that it can be checked against the pages by eye.

Pages cited (titles as they appear on the pages):
  [P1] nalar.dev, "KV Cache Quantization Perturbs Attention Through Stored Keys
       and Values"
  [P2] nalar.dev, "KV cache quantization reduces cache bytes with separate
       accuracy and kernel costs" (the page's address slug; it prints no title)
  [P3] mercemay.com, "KV Cache Quantization and Per-Token Scale Placement"

What is computed (the method reaches exact attention on a dequantized cache):
  * write side: each new key/value vector is quantized as q = clamp(round(x/s))
    with a scale s (P2 section "Quantization needs a scale convention"); the
    scale is per token and head by default (P3 section "Per-token scales and
    where they can live"), optionally with an integer zero point (P1 section
    "Quantization granularity defines which values share a scale"), per channel
    for keys with the factor moved onto the query (P3 section "The axis choice
    is a kernel decision"), or as an 8-bit code relative to a per-head
    super-scale (P3 section "Per-token scales and where they can live").
  * read side: s_i = q.k_hat_i / sqrt(D), a = softmax(s), o = sum_i a_i v_hat_i
    (P1 section "Key error acts before the softmax"; P2 section "Keys and values
    need not have identical error sensitivity").

Readings where the pages leave a step open (each restated where it is used):
  R1  rounding is round-half-to-even of the quotient x / s_stored, evaluated as
      one IEEE fp64 division followed by rint (P3's listing uses Python's
      round(), which ties to even).
  R2  scales/zero points are evaluated in fp64 and rounded once to their
      storage type; codes are computed from the stored (rounded) scale.
  R3  clamp after rounding; symmetric range [-(2^(b-1)-1), 2^(b-1)-1],
      unsigned (zero-point) range [0, 2^b - 1].
  R5  an all-zero vector gets scale 1 and codes 0 (P3's listing).
  R6  zero point: the integer code that represents 0; the range is widened to
      include 0; a flat (all-zero) vector gets s = 1, z = 0.
  R7  1/sqrt(D) is applied (formulas in P1 and P2); P3's score listing only
      shows the scale fold.
  R8  grouped-query heads: query head h reads KV head h // G.
  R9  per-channel key scales come from the absmax over the first append of a
      sequence (its prefill; all of its tokens, also those that stay in the
      window) and are then frozen; later tokens clamp.  The same holds for
      super-scales (R10).
  R22 a per-channel key scale that tracks a running estimate (axis
      "channel_grow", P3 "Per-token scales and where they can live": the
      estimate must be updated as the sequence grows): before tokens are
      quantized, a channel whose largest |k| among them exceeds qmax * s gets
      s' = RN32(that max / qmax), and its stored codes become
      clamp(rint(fl64(c s / s'))) (re-quantized on growth); the recent
      window holds keys in bf16 until they leave it.
  R26 a per-channel key scale held back until its estimate settles (axis
      "channel_hold", P3 "Per-token scales and where they can live": the
      entries can be kept in floating point until the running estimate is
      stable).  The pages leave "stable" open; here the estimate counts as
      stable once the recent window overflows: until a sequence's first
      position is quantized its keys are all in the bf16 window, and the
      channel scales are then taken, once, from the absmax over every token
      the sequence holds at that moment (the window's as stored there, in
      bf16, and the new ones as input), and frozen as R9's are; later
      tokens clamp.  Without a window this is R9.
  R10 super-scaled values: per token sigma = fl64(amax/qmax); per head
      S = RN32(max sigma / 255) over the prefill, frozen afterwards;
      u = clamp(rint(fl64(sigma / S)), 1, 255) (0 for an all-zero vector);
      the effective scale is the exact product u*S.
  R11 with a recent window of W tokens, exactly the min(W, n) newest tokens
      are kept unquantized, stored in bf16 (fp32 inputs are rounded to bf16,
      ties to even); older tokens are quantized per token.  A token is
      quantized from its input value, or from its bf16 window copy when it
      leaves the window in a later append.
  R13 the output is fp32 on the device; here fp64.
  R21 integer query (P3 "Precision floors and mixed cache formats": an 8-bit
      query against integer key codes, the integer sum converted to float
      once before the exponential): each query head is quantized by the
      symmetric quantizer P3 prints in "The axis choice is a kernel
      decision", in that listing's precision: s = fl64(amax / 127), kept in
      fp64 as the listing keeps it, and Q = clamp(rint(fl64(q / s)), -127,
      127), the same fp64 quotient as R1; an all-zero head gets s = 1 and
      codes 0.  Attention then uses Q * s for every token.  The exact path
      (the default) never quantizes the query.
  R20 token groups (P3 "Per-token scales and where they can live": several
      tokens under one scale): with a group size g, one scale (and zero
      point) is taken over all g*D values of g consecutive positions of a
      (sequence, head), i.e. the group is quantized as one vector.  A group
      is quantized once it is complete and older than the window: positions
      [0, Q) with Q = floor(max(n - W, 0) / g) * g are quantized, the newest
      n - Q stay in bf16 as the window's do (R11).  g = 1 is per token.
  R24 precision by recency beyond one window (P3 "Precision floors and mixed
      cache formats": precision that depends on how recent an entry is; P1
      "Cache growth changes the serving trade": recent tokens kept wider than
      older ones): between the bf16 window and the cache's format sits a
      middle tier of M positions (M a positive multiple of 32) stored as int8,
      symmetric, one fp32 scale per token.  With Q = max(n - W, 0) and
      A = floor(max(Q - M, 0) / 32) * 32, positions [0, A) hold the cache's
      format, [A, Q) the middle tier and [Q, n) bf16.  A token leaves the
      window into the middle tier (quantized as R11 says); it leaves the
      middle tier, 32 positions at a time, re-quantized to the cache's format
      from its middle-tier reconstruction c * s (exact).  The cache's format
      is then a per-token one (no channel axes, no 8-bit scale codes, no token
      groups).
  R27 where a paged block keeps its metadata (P2 "Metadata and block layout
      remain part of physical memory use": the block layout is part of what
      is allocated; the pages fix no layout): each (block, KV head) of a
      paged cache is a key unit, its 16 key code rows followed by its 16 / g
      key and then 16 / g value metadata elements in whole key code rows,
      and a value unit of its 16 value code rows; the rest of the last
      metadata row is padding.
  Scale underflow: a scale that rounds to 0 in its storage type is replaced by
  that type's smallest positive value (fp32 2^-149, fp16 2^-24); an fp16 scale
  above 65504 saturates to 65504.
  An empty cache (0 tokens) attends to nothing: the output is all zeros.

Parity: every function below is pinned by tests under tests/ (exact rational
arithmetic, closed forms, special cases, identities from P1).  None is
"parity unpinned", but the zero-point convention (R6) and the super-scale
convention (R10) are readings: the pages fix their invariants (range, exact
zero, error bound, metadata size), not their every bit.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np

F32_TINY = 2.0 ** -149   # smallest positive fp32 (subnormal)
F16_TINY = 2.0 ** -24    # smallest positive fp16 (subnormal)
F16_MAX = 65504.0

_SCALE_DTYPES = {"f32": np.float32, "f16": np.float16, "f64": np.float64}


# --------------------------------------------------------------------------
# Format description (the oracle's own; the HIP library has its own structs)
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class TensorFormat:
    """How one of K or V is stored.

    bits:       16 = unquantized (bf16 values kept as is), 8, 4 or 2 (2-bit
                symmetric codes are -1, 0, 1; with a zero point 0..3).
    axis:       "token" (one scale per token per head, P3 "Per-token scales and
                where they can live"), "channel" (one scale per feature per
                head, keys only, moved onto the query per P3 "The axis choice is
                a kernel decision"), "channel_grow" (per channel, the scale
                grows with the running absmax and the stored codes are
                re-quantized, reading R22) or "channel_hold" (per channel, the
                keys held in the bf16 window until the scales are fixed,
                reading R26).
    zero_point: integer zero point (unsigned codes) when True.
    scale:      "f32", "f16" (scale and zero point stored in that type) or
                "u8_super" (8-bit code times a per-head fp32 super-scale).
    """

    bits: int
    axis: str = "token"
    zero_point: bool = False
    scale: str = "f32"


def round_bf16(x) -> np.ndarray:
    """Values as stored in bf16 (round to nearest, ties to even); finite input.
    Tokens kept unquantized (bits 16, or the recent window) are stored in bf16."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def round_bf16_from_f64(x) -> np.ndarray:
    """fp64 values rounded once to bf16 (nearest, ties to even), directly on
    the fp64 bit pattern: drop 45 of its 52 fraction bits.  For values that
    are not exact in fp32 (a dequantized code times a scale), rounding to
    fp32 first could round twice.  Finite values in the normal bf16 range."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float64)).view(np.uint64)
    u = ((u + np.uint64((1 << 44) - 1) + ((u >> np.uint64(45)) & np.uint64(1)))
         >> np.uint64(45)) << np.uint64(45)
    return u.view(np.float64).copy()


def qmax_symmetric(bits: int) -> int:
    """Largest magnitude of a symmetric code; -2^(b-1) is never produced (R3)."""
    return (1 << (bits - 1)) - 1


def qmax_unsigned(bits: int) -> int:
    return (1 << bits) - 1


def quantized_count(n: int, window: int = 0, group: int = 1) -> int:
    """Positions [0, Q) of an n-token sequence are quantized (readings R11,
    R20): the newest min(W, n) stay in bf16, and of the rest only whole groups
    of g positions are quantized."""
    return max(n - window, 0) // group * group


TIER_BLOCK = 32   # positions that leave the middle tier together (R24)
MID_BITS, MID_SCALE = 8, "f32"   # the middle tier's format (R24)


def tier_counts(n: int, window: int = 0, mid: int = 0, group: int = 1):
    """Reading R24: (main, middle, bf16) position counts of an n-token
    sequence; without a middle tier (mid = 0) the middle count is 0 and the
    split is R11's / R20's."""
    q = quantized_count(n, window, group)
    if not mid:
        return q, 0, n - q
    a = max(q - mid, 0) // TIER_BLOCK * TIER_BLOCK
    return a, q - a, n - q


def mid_ring_slots(mid: int) -> int:
    """Middle-tier slots per (sequence, head): M plus one block of 32, since
    the tier holds between M and M + 31 positions once full (R24)."""
    return mid + TIER_BLOCK if mid else 0


def round_to_storage(x64, scale: str) -> np.ndarray:
    """Round fp64 values once (ties to even) to the storage type (R2), then
    apply the underflow/overflow rule stated in the module docstring."""
    dt = _SCALE_DTYPES[scale]
    s = np.asarray(x64, dtype=np.float64).astype(dt)
    if dt is np.float32:
        s = np.where(s == 0, np.float32(F32_TINY), s).astype(np.float32)
    elif dt is np.float16:
        s64 = s.astype(np.float64)
        s64 = np.where(s64 == 0, F16_TINY, s64)
        s64 = np.where(s64 > F16_MAX, F16_MAX, s64)
        s = s64.astype(np.float16)
    return s


def rne_quotient(x, s) -> np.ndarray:
    """R1: round-half-to-even of x / s, as one IEEE fp64 division then rint.

    x and s hold at most 24 significant bits and |x/s| <= 2^8 (plus the
    clamp), so the fp64 quotient never crosses or lands on a half-integer that
    the exact quotient does not: a non-tie quotient lies at least 2^-26 away
    from any half-integer, while the fp64 rounding error is below 2^-44.  A
    middle-tier reconstruction x = c * s8 (R24; |c| <= 127) has up to 31
    significant bits, but its granule is s8's and s lies between s8 / 4 and
    128 s8, so a non-tie quotient still lies at least 2^-34 from a
    half-integer.
    """
    return np.rint(np.asarray(x, np.float64) / np.asarray(s, np.float64))


# --------------------------------------------------------------------------
# Quantizers (write side).  Each works on the last axis of x (one vector).
# --------------------------------------------------------------------------
def quantize_sym(x, bits: int, scale: str = "f32"):
    """Symmetric per-vector quantization, P2 "Quantization needs a scale
    convention" (q = clamp(round(x/s)), x_hat = q*s) with the scale taken from
    the vector's absolute maximum as in P3 "The axis choice is a kernel
    decision" (scale = amax / qmax; all-zero vector -> codes 0, scale 1).

    Returns (codes int32 [..., D], scale [...] in the storage type).
    """
    x = np.asarray(x, dtype=np.float64)
    qmax = qmax_symmetric(bits)
    amax = np.max(np.abs(x), axis=-1)
    zero = amax == 0.0
    s = round_to_storage(np.where(zero, 1.0, amax / qmax), scale)
    s = np.where(zero, np.asarray(1.0, s.dtype), s).astype(s.dtype)
    codes = np.clip(rne_quotient(x, s[..., None]), -qmax, qmax)
    codes = np.where(zero[..., None], 0.0, codes)
    return codes.astype(np.int32), s


def quantize_asym(x, bits: int, scale: str = "f16"):
    """Zero-point (unsigned) per-vector quantization, reading R6.

    lo = min(min x, 0), hi = max(max x, 0); s = RN((hi - lo) / (2^b - 1));
    z = clamp(rint(-lo / s), 0, 2^b - 1) is the code that represents 0;
    c = clamp(rint(x / s) + z, 0, 2^b - 1).  The rounding is applied to x/s
    before z is added: rint(y) + z differs from rint(y + z) at ties when z is
    odd.  Reconstruction: x_hat = s * (c - z).

    Returns (codes int32 [..., D], s [...], z [...]) with s and z in the
    storage type (z is an integer, exact in fp16/fp32).
    """
    x = np.asarray(x, dtype=np.float64)
    qmax = qmax_unsigned(bits)
    lo = np.minimum(np.min(x, axis=-1), 0.0)
    hi = np.maximum(np.max(x, axis=-1), 0.0)
    flat = hi == lo
    s = round_to_storage(np.where(flat, 1.0, (hi - lo) / qmax), scale)
    s = np.where(flat, np.asarray(1.0, s.dtype), s).astype(s.dtype)
    z = np.clip(rne_quotient(-lo, s), 0, qmax)
    z = np.where(flat | (z == 0), 0.0, z)      # a zero point of 0 is stored as +0
    codes = np.clip(rne_quotient(x, s[..., None]) + z[..., None], 0, qmax)
    return codes.astype(np.int32), s, z.astype(s.dtype)


def channel_scales(k_prefill, bits: int) -> np.ndarray:
    """Per-channel key scales (reading R9 of P3 "Per-token scales and where they
    can live"): absmax over the prefill tokens of each feature, divided by qmax,
    rounded once to fp32; an all-zero channel gets scale 1.

    k_prefill: [..., T, D]  ->  [..., D] fp32.
    """
    k = np.asarray(k_prefill, dtype=np.float64)
    qmax = qmax_symmetric(bits)
    amax = np.max(np.abs(k), axis=-2)
    zero = amax == 0.0
    s = round_to_storage(np.where(zero, 1.0, amax / qmax), "f32")
    return np.where(zero, np.float32(1.0), s).astype(np.float32)


def quantize_with_channel_scales(k, s_chan, bits: int) -> np.ndarray:
    """Codes of keys under frozen per-channel scales: c = clamp(rint(k / s_d))."""
    qmax = qmax_symmetric(bits)
    k = np.asarray(k, dtype=np.float64)
    codes = np.clip(rne_quotient(k, np.asarray(s_chan)[..., None, :]), -qmax, qmax)
    return codes.astype(np.int32)


def super_scale(v_prefill, bits: int) -> np.ndarray:
    """Per-head fp32 super-scale (reading R10 of P3 "Per-token scales and where
    they can live": 8-bit scales relative to a coarser super-scale).

    sigma_t = fl64(amax_t / qmax) per token; S = RN32(max_t sigma_t / 255);
    S = 1 when every prefill vector is zero.  v_prefill: [..., T, D] -> [...].
    """
    v = np.asarray(v_prefill, dtype=np.float64)
    qmax = qmax_symmetric(bits)
    sigma = np.max(np.abs(v), axis=-1) / qmax
    smax = np.max(sigma, axis=-1)
    zero = smax == 0.0
    S = round_to_storage(np.where(zero, 1.0, smax / 255.0), "f32")
    return np.where(zero, np.float32(1.0), S).astype(np.float32)


def quantize_superscaled(v, S, bits: int):
    """Codes and 8-bit scale codes under a frozen super-scale S (reading R10).

    u_t = clamp(rint(fl64(sigma_t / S)), 1, 255), 0 for an all-zero vector;
    effective scale u_t*S (exact in fp64); c = clamp(rint(v / (u_t*S))).
    v: [..., T, D], S: [...]  ->  (codes int32 [..., T, D], u uint8 [..., T]).
    """
    v = np.asarray(v, dtype=np.float64)
    qmax = qmax_symmetric(bits)
    S64 = np.asarray(S, dtype=np.float64)[..., None]
    amax = np.max(np.abs(v), axis=-1)
    sigma = amax / qmax
    u = np.clip(np.rint(sigma / S64), 1, 255)
    u = np.where(amax == 0.0, 0.0, u)
    s_eff = u * S64                        # exact: 8-bit times 24-bit significand
    safe = np.where(u == 0.0, 1.0, s_eff)
    codes = np.clip(rne_quotient(v, safe[..., None]), -qmax, qmax)
    codes = np.where((u == 0.0)[..., None], 0.0, codes)
    return codes.astype(np.int32), u.astype(np.uint8)


def quantize_query_int8(q):
    """Reading R21: the query quantized to int8 per head (last axis) by the
    quantizer listing of P3 "The axis choice is a kernel decision": scale
    amax / 127 and quotient q / scale, both IEEE fp64 (the listing's Python
    floats), rounded ties to even (R1) and clamped.  q holds values exact in
    fp32.  Returns (codes int32 [..., D], scale float64 [...])."""
    q64 = np.asarray(q, np.float64)
    amax = np.max(np.abs(q64), axis=-1)
    zero = amax == 0
    s = np.where(zero, 1.0, amax / 127.0)
    codes = np.clip(rne_quotient(q64, s[..., None]), -127, 127)
    codes = np.where(zero[..., None], 0.0, codes)
    return codes.astype(np.int32), s


# --------------------------------------------------------------------------
# Dequantization (read side), fp64
# --------------------------------------------------------------------------
def dequant_sym(codes, s) -> np.ndarray:
    return np.asarray(codes, np.float64) * np.asarray(s, np.float64)[..., None]


def dequant_asym(codes, s, z) -> np.ndarray:
    return np.asarray(s, np.float64)[..., None] * (
        np.asarray(codes, np.float64) - np.asarray(z, np.float64)[..., None])


def dequant_channel(codes, s_chan) -> np.ndarray:
    return np.asarray(codes, np.float64) * np.asarray(s_chan, np.float64)[..., None, :]


def dequant_superscaled(codes, u, S) -> np.ndarray:
    s_eff = np.asarray(u, np.float64) * np.asarray(S, np.float64)[..., None]
    return np.asarray(codes, np.float64) * s_eff[..., None]


# --------------------------------------------------------------------------
# Attention (read side), the plain definition in fp64
# --------------------------------------------------------------------------
def softmax(s) -> np.ndarray:
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - np.max(s))
    return e / np.sum(e)


def scores(q_head, k_hat_head) -> np.ndarray:
    """Scores of one query head against one KV head's keys: q . k_hat_i / sqrt(D)
    (P2 "Keys and values need not have identical error sensitivity")."""
    q_head = np.asarray(q_head, dtype=np.float64)
    return (np.asarray(k_hat_head, dtype=np.float64) @ q_head) / math.sqrt(q_head.shape[-1])


def attend(q, k_hat, v_hat) -> np.ndarray:
    """Exact single-query attention over a reconstructed cache.

    P1 "Key error acts before the softmax": s = q K^T / sqrt(d), a = softmax(s),
    o = a V; P2 "Keys and values need not have identical error sensitivity":
    score_i = q . k_hat_i / sqrt(D), output = sum_i softmax(score)_i v_hat_i.

    q: [Hq, D]; k_hat, v_hat: [Hkv, T, D]; query head h reads KV head h // G
    with G = Hq / Hkv (reading R8).  T = 0 gives zeros.  Returns [Hq, D] fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v_hat = np.asarray(v_hat, dtype=np.float64)
    hq, d = q.shape
    hkv, t, _ = k_hat.shape
    assert hq % hkv == 0
    g = hq // hkv
    out = np.zeros((hq, d), dtype=np.float64)
    if t == 0:
        return out
    for h in range(hq):
        kv = h // g
        a = softmax(scores(q[h], k_hat[kv]))
        out[h] = a @ v_hat[kv]
    return out


def attention_weights(q, k_hat) -> np.ndarray:
    """Softmax weights [Hq, T] for the same definition as ``attend``."""
    q = np.asarray(q, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    hq, d = q.shape
    hkv, t, _ = k_hat.shape
    g = hq // hkv
    return np.stack([softmax(scores(q[h], k_hat[h // g])) for h in range(hq)])


# --------------------------------------------------------------------------
# A logical cache for one layer: what is stored per token, in position order
# --------------------------------------------------------------------------
class _Side:
    """Stored records of one tensor (K or V) of one sequence: [Hkv, n, ...]."""

    def __init__(self, hkv: int, d: int):
        self.codes = np.zeros((hkv, 0, d), np.int32)
        self.s = None          # per-token (per-group) scale [Hkv, n / g]
        self.z = None          # per-token (per-group) zero point [Hkv, n / g]
        self.u = None          # per-token 8-bit scale code [Hkv, n]
        self.raw = np.zeros((hkv, 0, d), np.float64)   # bits == 16 formats
        self.chan = None       # per-channel scale [Hkv, D]
        self.S = None          # per-head super-scale [Hkv]


class OracleCache:
    """Logical contents of one layer's cache for a batch of sequences.

    Appends follow P3 "Per-token scales and where they can live" (each vector
    quantized from itself at write time and stored with its scale).  With a
    recent window (P1 "Cache growth changes the serving trade"), the newest
    min(W, n) tokens stay as their bf16 values and the rest are quantized per
    token (reading R11).  Paging (P2 "Metadata and block layout remain part of
    physical memory use") changes placement only, so this model has none.

    With a token group size g > 1 (reading R20) one scale covers g
    consecutive positions, and the positions of a group not yet complete stay
    in bf16 beside the window.

    With a middle tier of `mid` positions (reading R24) the tokens between the
    window and the cache's format are held as int8 with one fp32 scale each.
    """

    def __init__(self, batch: int, hkv: int, d: int, key: TensorFormat,
                 value: TensorFormat, window: int = 0, group: int = 1, mid: int = 0):
        if group > 1 and (key.axis != "token" or key.scale == "u8_super"
                          or value.scale == "u8_super"):
            raise ValueError("token groups are modelled for per-token formats only")
        if group < 1:
            raise ValueError("group size must be at least 1")
        if mid:
            if mid < 0 or mid % TIER_BLOCK:
                raise ValueError("the middle tier holds a positive multiple of 32 positions")
            if group > 1 or any(f.axis != "token" or f.scale == "u8_super" or f.bits == 16
                                for f in (key, value)):
                raise ValueError("a middle tier is modelled for per-token formats only")
        self.batch, self.hkv, self.d = batch, hkv, d
        self.fmt = {"k": key, "v": value}
        self.window = window
        self.group = group
        self.mid = mid
        # middle tier (R24): codes [Hkv, n_mid, D] and fp32 scales [Hkv, n_mid]
        self.midq = [{t: (np.zeros((hkv, 0, d), np.int32), np.zeros((hkv, 0), np.float32))
                      for t in ("k", "v")} for _ in range(batch)]
        self.lens = [0] * batch
        self.side = [{"k": _Side(hkv, d), "v": _Side(hkv, d)} for _ in range(batch)]
        self.win = [{"k": np.zeros((hkv, 0, d)), "v": np.zeros((hkv, 0, d))}
                    for _ in range(batch)]

    # -- write side ---------------------------------------------------------
    def _quantize_into(self, side: _Side, fmt: TensorFormat, x: np.ndarray,
                       first: bool):
        """Quantize vectors x [Hkv, n, D] (position order, n a multiple of the
        group size) and append them."""
        n = x.shape[1]
        if n == 0:
            return
        if fmt.bits == 16:
            side.raw = np.concatenate([side.raw, round_bf16(x)], axis=1)
            return
        g = self.group
        if g > 1:
            # reading R20: each group of g positions is one vector of g*D values
            assert n % g == 0
            xg = x.reshape(x.shape[0], n // g, g * x.shape[2])
            if fmt.zero_point:
                c, s, z = quantize_asym(xg, fmt.bits, fmt.scale)
                side.z = z if side.z is None else np.concatenate([side.z, z], axis=1)
            else:
                c, s = quantize_sym(xg, fmt.bits, fmt.scale)
            side.s = s if side.s is None else np.concatenate([side.s, s], axis=1)
            side.codes = np.concatenate([side.codes, c.reshape(x.shape)], axis=1)
            return
        if fmt.axis != "token":
            c = quantize_with_channel_scales(x, side.chan, fmt.bits)
        elif fmt.scale == "u8_super":
            c, u = quantize_superscaled(x, side.S, fmt.bits)
            side.u = u if side.u is None else np.concatenate([side.u, u], axis=1)
        elif fmt.zero_point:
            c, s, z = quantize_asym(x, fmt.bits, fmt.scale)
            side.s = s if side.s is None else np.concatenate([side.s, s], axis=1)
            side.z = z if side.z is None else np.concatenate([side.z, z], axis=1)
        else:
            c, s = quantize_sym(x, fmt.bits, fmt.scale)
            side.s = s if side.s is None else np.concatenate([side.s, s], axis=1)
        side.codes = np.concatenate([side.codes, c], axis=1)

    def append(self, b: int, k_new, v_new):
        """Append n tokens (k_new, v_new: [Hkv, n, D], values exactly
        representable in the input dtype) to sequence b."""
        k_new = np.asarray(k_new, np.float64)
        v_new = np.asarray(v_new, np.float64)
        n = k_new.shape[1]
        first = self.lens[b] == 0
        total = self.lens[b] + n
        for t, x in (("k", k_new), ("v", v_new)):
            side, fmt = self.side[b][t], self.fmt[t]
            if first and n and fmt.bits != 16:
                # readings R9, R10: side data from every token of the first append
                if fmt.axis in ("channel", "channel_grow"):
                    side.chan = channel_scales(x, fmt.bits)
                elif fmt.axis == "token" and fmt.scale == "u8_super":
                    side.S = super_scale(x, fmt.bits)
            if self.window or self.group > 1:
                pool = np.concatenate([self.win[b][t], x], axis=1)
                keep = total - quantized_count(total, self.window, self.group)
                leave = pool.shape[1] - keep
                q, self.win[b][t] = pool[:, :leave], round_bf16(pool[:, leave:])
            else:
                pool = q = x
            if fmt.axis == "channel_hold" and fmt.bits != 16 and side.chan is None and q.shape[1]:
                side.chan = self._hold_scales(pool, q, fmt)
            if self.mid:
                # reading R24: the tokens leaving the window enter the middle
                # tier; its oldest whole blocks of 32 leave it for the cache's
                # format, re-quantized from their exact reconstruction c * s
                c8, s8 = quantize_sym(q, MID_BITS, MID_SCALE)
                mc, ms = self.midq[b][t]
                mc = np.concatenate([mc, c8], axis=1)
                ms = np.concatenate([ms, s8], axis=1)
                n_out = (tier_counts(total, self.window, self.mid)[0]
                         - tier_counts(self.lens[b], self.window, self.mid)[0])
                q = self._mid_reconstruction(mc[:, :n_out], ms[:, :n_out])
                self.midq[b][t] = (mc[:, n_out:], ms[:, n_out:])
            if fmt.axis == "channel_grow" and not first and q.shape[1]:
                self._grow_channels(side, fmt, q)
            self._quantize_into(side, fmt, q, first)
        self.lens[b] = total

    @staticmethod
    def _hold_scales(held, leaving, fmt: TensorFormat):
        """Reading R26: the channel scales fixed when a sequence's first
        positions leave the window, from every token it holds at that moment
        (held [Hkv, n, D]: the window's tokens and the new ones; leaving: the
        first of them, about to be quantized)."""
        return channel_scales(held, fmt.bits)

    @staticmethod
    def _mid_reconstruction(codes, s):
        """Reading R24: the exact value c * s of middle-tier tokens (fp64 holds
        it: 7 bits times 24), from which they are re-quantized."""
        return dequant_sym(codes, s)

    @staticmethod
    def _grow_channels(side: _Side, fmt: TensorFormat, x: np.ndarray):
        """Reading R22: channels whose new absmax exceeds qmax * s get the
        scale of that absmax, and their stored codes are re-quantized."""
        qmax = qmax_symmetric(fmt.bits)
        amax = np.max(np.abs(x), axis=1)                          # [Hkv, D]
        old = side.chan.astype(np.float64)
        grown = amax > qmax * old                                 # exact in fp64
        if not grown.any():
            return
        new = np.where(grown, round_to_storage(np.where(grown, amax, 1.0) / qmax, "f32"),
                       side.chan).astype(np.float32)
        c = np.asarray(side.codes, np.float64)
        requant = np.clip(rne_quotient(c * old[:, None, :], new.astype(np.float64)[:, None, :]),
                          -qmax, qmax)
        side.codes = np.where(grown[:, None, :], requant, c).astype(np.int32)
        side.chan = new

    # -- read side ----------------------------------------------------------
    def _dequant(self, side: _Side, fmt: TensorFormat) -> np.ndarray:
        if fmt.bits == 16:
            return side.raw.copy()
        if side.codes.shape[1] == 0:
            return np.zeros((self.hkv, 0, self.d))
        if fmt.axis != "token":
            return dequant_channel(side.codes, side.chan)
        if fmt.scale == "u8_super":
            return dequant_superscaled(side.codes, side.u, side.S)
        # per-group metadata applies to each of the group's positions
        s = np.repeat(side.s, self.group, axis=1)
        if fmt.zero_point:
            return dequant_asym(side.codes, s, np.repeat(side.z, self.group, axis=1))
        return dequant_sym(side.codes, s)

    def reconstructed(self, b: int):
        """(k_hat, v_hat) [Hkv, len, D] fp64 in position order."""
        out = []
        for t in ("k", "v"):
            q = self._dequant(self.side[b][t], self.fmt[t])
            if self.mid:
                mc, ms = self.midq[b][t]
                q = np.concatenate([q, dequant_sym(mc, ms)], axis=1)
            if self.window or self.group > 1:
                q = np.concatenate([q, self.win[b][t]], axis=1)
            out.append(q)
        return out[0], out[1]

    def stored(self, b: int, t: str) -> _Side:
        """The stored records of sequence b for t in {"k", "v"} (for bit-exact
        comparison of codes and metadata)."""
        return self.side[b][t]

    def mid_stored(self, b: int, t: str):
        """Middle-tier codes [Hkv, n_mid, D] and fp32 scales [Hkv, n_mid] of
        sequence b, oldest first (reading R24)."""
        return self.midq[b][t]

    def window_values(self, b: int, t: str) -> np.ndarray:
        return self.win[b][t]

    def attend(self, b: int, q, query_bits: int = 0) -> np.ndarray:
        """Attention of the queries q [Hq, D] of sequence b; query_bits = 8
        takes the integer-query path (reading R21)."""
        k_hat, v_hat = self.reconstructed(b)
        if query_bits == 8:
            codes, s = quantize_query_int8(q)
            q = dequant_sym(codes, s)
        elif query_bits != 0:
            raise ValueError("query_bits is 0 (exact) or 8")
        return attend(q, k_hat, v_hat)


# --------------------------------------------------------------------------
# Byte accounting
# --------------------------------------------------------------------------
def meta_bytes_per_token(fmt: TensorFormat) -> int:
    """Per-token, per-head metadata bytes (P3 "Per-token scales and where they
    can live" prices a 4-byte scale, and a scale plus zero point)."""
    if fmt.bits == 16 or fmt.axis != "token":
        return 0
    if fmt.scale == "u8_super":
        return 1
    width = {"f32": 4, "f16": 2, "f64": 8}[fmt.scale]
    return width * (2 if fmt.zero_point else 1)


def side_bytes_per_head(fmt: TensorFormat, d: int) -> int:
    """Per-(sequence, head) metadata: channel scales or the super-scale."""
    if fmt.bits == 16:
        return 0
    if fmt.axis != "token":
        return 4 * d
    if fmt.scale == "u8_super":
        return 4
    return 0


def ring_slots(window: int = 0, group: int = 1) -> int:
    """bf16 slots per (sequence, head): the window plus room for the
    positions of an incomplete token group (at most g - 1)."""
    return window + (group if group > 1 else 0)


def _unit_pad(row: int, meta_block: int) -> int:
    """Reading R27: a paged block keeps its key and value metadata in whole
    key code rows after its 16 key rows; the unused end of the last of those
    rows is padding."""
    return -(-meta_block // row) * row - meta_block


def cache_bytes(key: TensorFormat, value: TensorFormat, layers: int, hkv: int,
                d: int, lens: Sequence[int], window: int = 0,
                block_tokens: int = 0, max_tokens: Optional[int] = None,
                group: int = 1, mid: int = 0) -> Dict[str, int]:
    """Bytes of a cache holding sequences of the given lengths.

    payload   P2 "Cache precision is separate from weight precision":
              KV_bytes = 2 * L * H_kv * D * T * b, generalised to separate key
              and value widths: L * H_kv * D * T_q * (b_K + b_V) over the
              quantized tokens T_q of each sequence.
    metadata  per-token (per-group) scales / zero points / 8-bit scale codes
              plus per-head channel scales or super-scales (P3 "Per-token
              scales and where they can live"; P2 "Metadata and block layout
              remain part of physical memory use").
    window    the bf16 tokens (window and incomplete group), 2 bytes per
              element for K and V.
    A middle tier (R24) adds its int8 codes to payload and its fp32 scales
    to metadata; its unused ring slots are padding.
    padding   allocated but unused slots: the unfilled tail of the last block
              of a paged sequence, or max_tokens - T_q quantized slots of a
              contiguous one, and the unused bf16 ring slots of either (the
              ring is one fixed-size buffer per sequence and head in both
              layouts: P2 "Metadata and block layout remain part of physical
              memory use" counts what is allocated, not only what is used);
              in a paged cache, the rest of the key code rows that hold each
              block's metadata (reading R27).
    total     the sum of the four.
    """
    def row(fmt):  # bytes of one token's codes
        return d * fmt.bits // 8

    out = dict(payload=0, metadata=0, window=0, padding=0)
    codes = row(key) + row(value)
    meta = meta_bytes_per_token(key) + meta_bytes_per_token(value)   # per group
    ring = ring_slots(window, group)
    mid_row, mid_meta = 2 * d, 2 * 4   # int8 K and V rows, fp32 scale each
    for n in lens:
        n_q, n_m, n_w = tier_counts(n, window, mid, group)
        out["payload"] += layers * hkv * (n_q * codes + n_m * mid_row)
        out["metadata"] += layers * hkv * (
            n_q // group * meta + n_m * mid_meta
            + side_bytes_per_head(key, d) + side_bytes_per_head(value, d))
        if mid:
            out["padding"] += layers * hkv * (mid_ring_slots(mid) - n_m) * (mid_row + mid_meta)
        out["window"] += layers * hkv * n_w * d * 2 * 2
        if block_tokens:
            alloc_q = -(-n_q // block_tokens) * block_tokens
        else:
            alloc_q = max_tokens if max_tokens is not None else n_q
        out["padding"] += layers * hkv * ((alloc_q - n_q) * codes + (alloc_q - n_q) // group * meta)
        if block_tokens:
            out["padding"] += layers * hkv * (alloc_q // block_tokens) * _unit_pad(
                row(key), block_tokens // group * meta)
        if ring:
            out["padding"] += layers * hkv * (ring - n_w) * d * 2 * 2
    out["total"] = out["payload"] + out["metadata"] + out["window"] + out["padding"]
    return out


def decode_traffic(key: TensorFormat, value: TensorFormat, hkv: int, d: int,
                   lens: Sequence[int], window: int = 0, group: int = 1,
                   mid: int = 0) -> int:
    """Bytes one decode step must read from the cache (one layer): codes,
    per-token (per-group) metadata, middle-tier codes and scales, bf16 values
    and per-head side data; no padding."""
    b = cache_bytes(key, value, 1, hkv, d, lens, window, group=group, mid=mid)
    return b["payload"] + b["metadata"] + b["window"]


def dequantized_bf16(cache: "OracleCache", b: int):
    """Reconstructed keys and values of sequence b rounded once to bf16: the
    cache a dequantize-into-temporary-storage path attends over."""
    k_hat, v_hat = cache.reconstructed(b)
    return round_bf16_from_f64(k_hat), round_bf16_from_f64(v_hat)


def multiply_adds(hq: int, d: int, lens: Sequence[int]) -> int:
    """Multiply-adds of one decode step: q.k and a.v, D each per token and
    query head (P3 "What the cache holds and how it is read")."""
    return sum(2 * hq * d * n for n in lens)


def arithmetic_intensity(bits: int, d: int = 128, group: int = 1,
                         meta_bytes: int = 4) -> float:
    """Multiply-adds per cache byte for one token of one KV head read by
    ``group`` query heads: 2*G*D MACs over 2*D*b/8 code bytes plus a key and a
    value scale (P3 "What the cache holds and how it is read")."""
    return (2 * group * d) / (2 * d * bits / 8 + 2 * meta_bytes)
