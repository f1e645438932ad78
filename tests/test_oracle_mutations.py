"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one of them (a pin set that a dropped term, a wrong sign or index,
or a transposed operand slips through is too weak to trust the oracle on)."""
import importlib.util
import os
import sys

import numpy as np
import pytest

import oracle_pins

ORACLE_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "oracle", "kvq_oracle.py")
_count = [0]


def fresh_oracle():
    _count[0] += 1
    spec = importlib.util.spec_from_file_location(f"kvq_oracle_mut{_count[0]}", ORACLE_FILE)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod
    spec.loader.exec_module(mod)
    return mod


def _q(x, s):
    return np.asarray(x, np.float64) / np.asarray(s, np.float64)


def m_round_half_up(O):
    O.rne_quotient = lambda x, s: np.floor(_q(x, s) + 0.5)


def m_round_half_away(O):
    O.rne_quotient = lambda x, s: np.trunc(_q(x, s) + np.copysign(0.5, _q(x, s)))


def m_fp32_division(O):
    O.rne_quotient = lambda x, s: np.rint((np.asarray(x, np.float32) / np.asarray(s, np.float32)).astype(np.float64))


def m_reciprocal_multiply(O):
    O.rne_quotient = lambda x, s: np.rint(np.asarray(x, np.float64) * (1.0 / np.asarray(s, np.float32)).astype(np.float32))


def m_scale_not_rounded(O):
    O.round_to_storage = lambda x64, scale: np.asarray(x64, np.float64)


def m_qmax_128(O):
    O.qmax_symmetric = lambda b: 1 << (b - 1)


def m_group_count_ignores_window(O):
    O.quantized_count = lambda n, window=0, group=1: n // group * group


def m_group_count_rounds_up(O):
    O.quantized_count = lambda n, window=0, group=1: -(-max(n - window, 0) // group) * group


def m_int_query_fp32_division(O):
    def qq(q):
        q32 = np.asarray(q, np.float32)
        amax = np.max(np.abs(q32), axis=-1)
        s = np.where(amax == 0, np.float32(1.0), amax / np.float32(127.0)).astype(np.float32)
        return np.clip(np.rint(q32 / s[..., None]), -127, 127).astype(np.int32), s
    O.quantize_query_int8 = qq


def m_int_query_fp32_scale(O):
    def qq(q):
        q = np.asarray(q, np.float64)
        amax = np.max(np.abs(q), axis=-1)
        s = np.where(amax == 0, 1.0, amax / 127.0).astype(np.float32).astype(np.float64)
        return np.clip(np.rint(q / s[..., None]), -127, 127).astype(np.int32), s
    O.quantize_query_int8 = qq


def m_growth_requant_truncates(O):
    orig = O.OracleCache._grow_channels

    def grow(side, fmt, x):
        saved = O.rne_quotient
        O.rne_quotient = lambda a, b: np.trunc(np.asarray(a, np.float64) / np.asarray(b, np.float64))
        try:
            orig(side, fmt, x)
        finally:
            O.rne_quotient = saved
    O.OracleCache._grow_channels = staticmethod(grow)


def m_growth_never(O):
    O.OracleCache._grow_channels = staticmethod(lambda side, fmt, x: None)


def m_tier_reconstruction_fp32(O):
    O.OracleCache._mid_reconstruction = staticmethod(
        lambda c, s: O.dequant_sym(c, s).astype(np.float32).astype(np.float64))


def m_tier_mid_scale_fp16(O):
    O.MID_SCALE = "f16"


def m_tier_unaligned(O):
    def tier_counts(n, window=0, mid=0, group=1):
        q = O.quantized_count(n, window, group)
        a = max(q - mid, 0) if mid else q
        return a, q - a, n - q
    O.tier_counts = tier_counts


def m_tier_ignores_window(O):
    orig = O.tier_counts
    O.tier_counts = lambda n, window=0, mid=0, group=1: (
        orig(n, 0, mid, group)[0] if mid else orig(n, window, mid, group)[0],) + orig(n, window, mid, group)[1:]


def m_no_inv_sqrt_d(O):
    O.scores = lambda q, k: np.asarray(k, np.float64) @ np.asarray(q, np.float64)


def m_inv_d_not_sqrt(O):
    O.scores = lambda q, k: (np.asarray(k, np.float64) @ np.asarray(q, np.float64)) / np.asarray(q).shape[-1]


def m_gqa_modulo(O):
    def attend(q, k_hat, v_hat):
        hq, d = q.shape
        hkv = k_hat.shape[0]
        out = np.zeros((hq, d))
        if k_hat.shape[1] == 0:
            return out
        for h in range(hq):
            a = O.softmax(O.scores(q[h], k_hat[h % hkv]))
            out[h] = a @ v_hat[h % hkv]
        return out
    O.attend = attend


def m_zero_point_inside_round(O):
    orig = O.quantize_asym

    def quantize_asym(x, bits, scale="f16"):
        c, s, z = orig(x, bits, scale)
        qmax = (1 << bits) - 1
        c2 = np.clip(np.rint(_q(x, s[..., None]) + z.astype(np.float64)[..., None]), 0, qmax)
        return c2.astype(np.int32), s, z
    O.quantize_asym = quantize_asym


def m_dequant_asym_sign(O):
    O.dequant_asym = lambda c, s, z: np.asarray(s, np.float64)[..., None] * (
        np.asarray(c, np.float64) + np.asarray(z, np.float64)[..., None])


def m_softmax_unnormalised(O):
    O.softmax = lambda s: np.exp(np.asarray(s) - np.max(s))


def m_channel_scale_per_token(O):
    def channel_scales(k, bits):
        amax = np.max(np.abs(np.asarray(k, np.float64)), axis=-1)
        return np.resize(O.round_to_storage(amax / O.qmax_symmetric(bits), "f32"), np.asarray(k).shape[-1]).astype(np.float32)
    O.channel_scales = channel_scales


def m_super_code_floor(O):
    orig = O.quantize_superscaled

    def quantize_superscaled(v, S, bits):
        v = np.asarray(v, np.float64)
        qmax = O.qmax_symmetric(bits)
        amax = np.max(np.abs(v), axis=-1)
        u = np.clip(np.floor(amax / qmax / np.asarray(S, np.float64)[..., None]), 1, 255)
        u = np.where(amax == 0, 0, u)
        s = np.where(u == 0, 1.0, u * np.asarray(S, np.float64)[..., None])
        c = np.clip(np.rint(v / s[..., None]), -qmax, qmax)
        c = np.where((u == 0)[..., None], 0, c)
        return c.astype(np.int32), u.astype(np.uint8)
    O.quantize_superscaled = quantize_superscaled


def m_dequant_drops_scale(O):
    O.dequant_sym = lambda c, s: np.asarray(c, np.float64)


def m_amax_whole_tensor(O):
    orig = O.quantize_sym

    def quantize_sym(x, bits, scale="f32"):
        x = np.asarray(x, np.float64)
        qmax = O.qmax_symmetric(bits)
        amax = np.full(x.shape[:-1], np.max(np.abs(x)))
        s = O.round_to_storage(np.where(amax == 0, 1.0, amax / qmax), scale)
        c = np.clip(O.rne_quotient(x, s[..., None]), -qmax, qmax)
        return c.astype(np.int32), s
    O.quantize_sym = quantize_sym


def m_asym_range_without_zero(O):
    def quantize_asym(x, bits, scale="f16"):
        x = np.asarray(x, np.float64)
        qmax = (1 << bits) - 1
        lo, hi = np.min(x, axis=-1), np.max(x, axis=-1)
        flat = hi == lo
        s = O.round_to_storage(np.where(flat, 1.0, (hi - lo) / qmax), scale)
        z = np.clip(O.rne_quotient(-lo, s), 0, qmax)
        c = np.clip(O.rne_quotient(x, s[..., None]) + z[..., None], 0, qmax)
        return c.astype(np.int32), s, z.astype(s.dtype)
    O.quantize_asym = quantize_asym


def m_value_uses_keys(O):
    def attend(q, k_hat, v_hat):
        hq, d = q.shape
        g = hq // k_hat.shape[0]
        out = np.zeros((hq, d))
        for h in range(hq):
            out[h] = O.softmax(O.scores(q[h], k_hat[h // g])) @ k_hat[h // g]
        return out
    O.attend = attend


def m_meta_bytes_ignores_zero_point(O):
    O.meta_bytes_per_token = lambda fmt: 0 if (fmt.bits == 16 or fmt.axis == "channel") else (
        1 if fmt.scale == "u8_super" else {"f32": 4, "f16": 2, "f64": 8}[fmt.scale])


def m_payload_single_tensor(O):
    orig = O.cache_bytes

    def cache_bytes(*a, **k):
        out = dict(orig(*a, **k))
        out["payload"] //= 2
        return out
    O.cache_bytes = cache_bytes


def m_window_keeps_one_more(O):
    orig_append = O.OracleCache.append

    def append(self, b, k_new, v_new):
        self.window += 1
        try:
            orig_append(self, b, k_new, v_new)
        finally:
            self.window -= 1
    O.OracleCache.append = append


def m_super_scale_over_255_times_qmax(O):
    orig = O.super_scale
    O.super_scale = lambda v, bits: (orig(v, bits).astype(np.float64) * 7 / 8).astype(np.float32)


def m_f16_underflow_to_min_normal(O):
    orig = O.round_to_storage

    def rts(x64, scale):
        r = orig(x64, scale)
        if scale == "f16":
            r = np.where(r.astype(np.float64) == 2.0 ** -24, np.float16(2.0 ** -14), r).astype(np.float16)
        return r
    O.round_to_storage = rts


def m_f16_overflow_not_saturated(O):
    O.F16_MAX = np.inf


def m_f32_underflow_kept_zero(O):
    O.F32_TINY = 0.0


def m_f16_flush_subnormal_scales(O):
    orig = O.round_to_storage

    def rts(x64, scale):
        r = orig(x64, scale)
        if scale == "f16":
            r64 = r.astype(np.float64)
            r = np.where(r64 < 2.0 ** -14, np.float16(2.0 ** -24), r).astype(np.float16)
        return r
    O.round_to_storage = rts


def m_ring_padding_contiguous_only(O):
    orig = O.cache_bytes

    def cb(key, value, layers, hkv, d, lens, window=0, block_tokens=0, max_tokens=None,
           group=1, mid=0):
        out = orig(key, value, layers, hkv, d, lens, window, block_tokens, max_tokens, group, mid)
        if block_tokens:
            ring = O.ring_slots(window, group)
            for n in lens:
                nw = O.tier_counts(n, window, mid, group)[2]
                out["padding"] -= layers * hkv * (ring - nw) * d * 4
            out["total"] = out["payload"] + out["metadata"] + out["window"] + out["padding"]
        return out
    O.cache_bytes = cb


def m_mid_ring_without_spare_block(O):
    O.mid_ring_slots = lambda mid: mid


def m_hold_scales_from_leaving_tokens(O):
    O.OracleCache._hold_scales = staticmethod(lambda held, leaving, fmt: O.channel_scales(leaving, fmt.bits))


def m_hold_scales_skip_oldest(O):
    O.OracleCache._hold_scales = staticmethod(lambda held, leaving, fmt: O.channel_scales(held[:, 1:], fmt.bits))


def m_paged_meta_rows_not_rounded(O):
    O._unit_pad = lambda row, meta_block: 0


def m_paged_meta_padded_to_lines(O):
    O._unit_pad = lambda row, meta_block: -(-meta_block // 128) * 128 - meta_block


MUTATIONS = [v for k, v in sorted(globals().items()) if k.startswith("m_")]


@pytest.mark.parametrize("mutate", MUTATIONS, ids=lambda f: f.__name__)
def test_mutation_is_caught(mutate):
    O = fresh_oracle()
    mutate(O)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(O)
        except Exception:   # AssertionError, or a crash the mistake causes
            caught.append(pin.__name__)
    assert caught, f"no pin catches {mutate.__name__}"
