"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, validates arguments before touching the GPU, and its byte
accounting agrees with the oracle.  No compute call runs here."""
import ctypes
import os
import re

import numpy as np
import pytest

from decode_attention_quantized_kvq_amd import kvq as K
from decode_attention_quantized_kvq_amd import synth
from oracle import kvq_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert len(names) >= 9, names
    lib = K.lib()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(K.EXPORTS) == names


def test_status_strings():
    for s in range(5):
        assert K.status_string(s).startswith("KVQ_")
    assert K.status_string(99) == "KVQ_ERR_UNKNOWN"


def cfg_of(wl, **kw):
    d = dict(batch=wl["batch"], num_q_heads=wl["hq"], num_kv_heads=wl["hkv"], head_dim=wl["d"],
             max_tokens=wl["tokens"], key=wl["key"], value=wl["value"], window=wl["window"],
             block_tokens=wl["block_tokens"], in_dtype=wl["in_dtype"],
             group_tokens=wl.get("group", 1), mid_tokens=wl.get("mid", 0))
    if wl["block_tokens"]:
        d["num_blocks"] = 100
        d["max_blocks_per_seq"] = -(-(wl["tokens"] - wl["window"]) // 16)
    d.update(kw)
    return K.make_config(**d)


def oracle_fmt(spec):
    return O.TensorFormat(spec["bits"], spec.get("axis", "token"), bool(spec.get("zero_point")),
                          spec.get("scale", "f32"))


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5, 6, 7, 8])
def test_workloads_validate(wid):
    assert K.validate(cfg_of(synth.workload(wid))) == K.KVQ_OK


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5, 6, 7, 8])
def test_cache_bytes_match_oracle(wid):
    wl = synth.workload(wid)
    lens = synth.seq_lengths(wl)
    cfg = cfg_of(wl)
    got = K.cache_bytes(cfg, lens)
    # the per-call decode workspace at the library's split for the longest sequence
    assert got.pop("workspace") == K.decode_workspace_bytes(cfg, max(lens))
    want = O.cache_bytes(oracle_fmt(wl["key"]), oracle_fmt(wl["value"]), 1, wl["hkv"], wl["d"],
                         lens, wl["window"], wl["block_tokens"],
                         None if wl["block_tokens"] else wl["tokens"], group=wl.get("group", 1),
                         mid=wl.get("mid", 0))
    assert got == want
    traffic = O.decode_traffic(oracle_fmt(wl["key"]), oracle_fmt(wl["value"]), wl["hkv"], wl["d"],
                               lens, wl["window"], group=wl.get("group", 1), mid=wl.get("mid", 0))
    assert K.decode_traffic_bytes(cfg, lens) == traffic


@pytest.mark.parametrize("window,mid", [(0, 32), (16, 64), (128, 256)])
def test_middle_tier_bytes_match_oracle(window, mid):
    """Byte accounting and buffer sizes of a cache with a middle tier: the
    int8 codes and fp32 scales of the tier, and its unused ring slots."""
    spec = dict(bits=4, zero_point=True, scale="f16")
    wl = synth.workload(2, key=spec, value=spec, window=window, mid=mid, batch=4, tokens=2048)
    lens = [0, window + mid + 31, window + mid + 32, 2000]
    cfg = cfg_of(wl, mid_tokens=mid, num_layers=3)
    got = K.cache_bytes(cfg, lens)
    assert got.pop("workspace") == K.decode_workspace_bytes(cfg, max(lens))
    want = O.cache_bytes(oracle_fmt(spec), oracle_fmt(spec), 3, wl["hkv"], wl["d"], lens, window,
                         0, wl["tokens"], mid=mid)
    assert got == want
    assert K.decode_traffic_bytes(cfg, lens) == O.decode_traffic(
        oracle_fmt(spec), oracle_fmt(spec), wl["hkv"], wl["d"], lens, window, mid=mid)
    sz = K.buffer_sizes(cfg)
    slots = mid + 32
    assert sz.k_mid == sz.v_mid == 3 * 4 * wl["hkv"] * slots * 128
    assert sz.k_mid_scale == sz.v_mid_scale == 3 * 4 * wl["hkv"] * slots * 4
    assert K.buffer_sizes(cfg_of(wl, mid_tokens=0)).k_mid == 0


def test_cache_bytes_metadata_cases():
    """The overhead cases the metadata section prices (scale; scale + zero
    point; 4-bit; 2-bit), through the C accounting, several layers."""
    cases = [(8, False), (8, True), (4, False), (2, False)]
    for bits, zp in cases:
        spec = dict(bits=bits, axis="token", zero_point=zp, scale="f32")
        cfg = K.make_config(batch=3, num_q_heads=4, num_kv_heads=2, head_dim=128, max_tokens=64,
                            key=spec, value=spec, num_layers=5)
        lens = [64, 10, 0]
        got = K.cache_bytes(cfg, lens)
        assert got.pop("workspace") == K.decode_workspace_bytes(cfg, 64)
        want = O.cache_bytes(oracle_fmt(spec), oracle_fmt(spec), 5, 2, 128, lens, 0, 0, 64)
        assert got == want
        assert got["payload"] == 2 * 5 * 2 * 128 * 74 * bits // 8


def test_paged_unit_sizes():
    """Paged units as the header documents them: a key unit of 16 key rows
    plus the block's key and value metadata in whole key rows, a value unit
    of 16 value rows."""
    def paged(key, value, group=1):
        cfg = K.make_config(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, max_tokens=0,
                            key=key, value=value, block_tokens=16, num_blocks=10,
                            max_blocks_per_seq=5, group_tokens=group)
        return K.buffer_sizes(cfg)
    units = 10 * 2
    # uint4 with fp16 scale + zero point: 64-byte rows, 2 x 16 x 4 B = two rows
    z4 = dict(bits=4, zero_point=True, scale="f16")
    s = paged(z4, z4)
    assert s.k_codes == units * 18 * 64 and s.v_codes == units * 16 * 64 and s.k_meta == s.v_meta == 0
    # int2 with 8-bit scale codes: 32-byte rows, 2 x 16 x 1 B = one row
    u2 = dict(bits=2, scale="u8_super")
    s = paged(u2, u2)
    assert s.k_codes == units * 17 * 32 and s.v_codes == units * 16 * 32
    # per-channel int8 keys (no per-token element), int4 values with 8-bit
    # scale codes: the 16 value codes take one 128-byte key row
    s = paged(dict(bits=8, axis="channel"), dict(bits=4, scale="u8_super"))
    assert s.k_codes == units * 17 * 128 and s.v_codes == units * 16 * 64
    # uint2 with one fp16 scale + zero point per 16-token group: 2 x 4 B in
    # one 32-byte key row
    s = paged(dict(bits=2, zero_point=True, scale="f16"), dict(bits=2, zero_point=True, scale="f16"), 16)
    assert s.k_codes == units * 17 * 32 and s.v_codes == units * 16 * 32


def test_buffer_sizes():
    wl = synth.workload(4)
    cfg = cfg_of(wl, num_layers=2)
    sz = K.buffer_sizes(cfg)
    # paged: per (block, KV head) a key unit of 16 code rows of 128 B and one
    # more row holding the block's 16 key and 16 value fp32 scales, and a
    # value unit of 16 rows; no separate metadata buffers
    assert sz.k_codes == 2 * 100 * 8 * 17 * 128 and sz.k_meta == 0
    assert sz.v_codes == 2 * 100 * 8 * 16 * 128 and sz.v_meta == 0
    assert sz.k_win == 2 * 64 * 8 * 128 * 128 * 2 and sz.k_chan_scale == 0
    wl5 = synth.workload(5)
    sz5 = K.buffer_sizes(cfg_of(wl5))
    assert sz5.k_chan_scale == 16 * 8 * 128 * 4 and sz5.v_super == 16 * 8 * 4
    assert sz5.v_codes == 16 * 8 * 65536 * 64 and sz5.v_meta == 16 * 8 * 65536
    assert sz5.k_super == 0
    # 2-bit codes with 8-bit scale codes for keys and values
    s2 = dict(bits=2, scale="u8_super")
    cfg2 = K.make_config(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, max_tokens=64,
                         key=s2, value=s2, num_layers=2)
    sz2 = K.buffer_sizes(cfg2)
    assert sz2.k_codes == sz2.v_codes == 2 * 3 * 2 * 64 * 32
    assert sz2.k_meta == sz2.v_meta == 2 * 3 * 2 * 64
    assert sz2.k_super == sz2.v_super == 2 * 3 * 2 * 4


def test_validation_errors():
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, max_tokens=64,
                key=dict(bits=8), value=dict(bits=8))
    ok = K.make_config(**base)
    assert K.validate(ok) == K.KVQ_OK
    bad = [
        (dict(num_q_heads=6, num_kv_heads=4), K.KVQ_ERR_INVALID_ARG),
        (dict(batch=0), K.KVQ_ERR_INVALID_ARG),
        (dict(key=dict(bits=3)), K.KVQ_ERR_INVALID_ARG),
        (dict(key=dict(bits=8, axis="channel", scale="f16")), K.KVQ_ERR_INVALID_ARG),
        (dict(value=dict(bits=4, scale="u8_super", zero_point=True)), K.KVQ_ERR_INVALID_ARG),
        (dict(head_dim=64), K.KVQ_ERR_UNSUPPORTED),
        (dict(num_q_heads=32, num_kv_heads=2), K.KVQ_ERR_UNSUPPORTED),   # G = 16
        (dict(max_tokens=40), K.KVQ_ERR_UNSUPPORTED),
        (dict(key=dict(bits=2), value=dict(bits=8)), K.KVQ_ERR_UNSUPPORTED),   # no such pair
        (dict(key=dict(bits=2, axis="channel"), value=dict(bits=2)), K.KVQ_ERR_UNSUPPORTED),
        (dict(key=dict(bits=2, scale="u8_super"), value=dict(bits=2, scale="u8_super"),
              group_tokens=4), K.KVQ_ERR_UNSUPPORTED),
        (dict(key=dict(bits=8, axis="channel_grow"), value=dict(bits=4, scale="u8_super"),
              group_tokens=2), K.KVQ_ERR_UNSUPPORTED),
        (dict(key=dict(bits=16), value=dict(bits=8)), K.KVQ_ERR_UNSUPPORTED),   # mixed pair
        (dict(key=dict(bits=16), value=dict(bits=16), window=16), K.KVQ_ERR_UNSUPPORTED),
        (dict(key=dict(bits=16), value=dict(bits=16), block_tokens=16, num_blocks=8,
              max_blocks_per_seq=4), K.KVQ_ERR_UNSUPPORTED),
        (dict(value=dict(bits=8, axis="channel")), K.KVQ_ERR_UNSUPPORTED),
        (dict(value=dict(bits=8, axis="channel_hold")), K.KVQ_ERR_UNSUPPORTED),   # keys only
        (dict(key=dict(bits=8, axis="channel_hold", zero_point=True)), K.KVQ_ERR_INVALID_ARG),
        (dict(key=dict(bits=8, axis="channel_hold"), value=dict(bits=4, scale="u8_super"),
              group_tokens=2), K.KVQ_ERR_UNSUPPORTED),
        (dict(mid_tokens=32, key=dict(bits=8, axis="channel_hold"),
              value=dict(bits=4, scale="u8_super")), K.KVQ_ERR_UNSUPPORTED),
        (dict(window=20), K.KVQ_ERR_UNSUPPORTED),
        (dict(block_tokens=16, num_blocks=0, max_blocks_per_seq=4), K.KVQ_ERR_INVALID_ARG),
        (dict(block_tokens=32, num_blocks=8, max_blocks_per_seq=4), K.KVQ_ERR_UNSUPPORTED),
        (dict(mid_tokens=-32), K.KVQ_ERR_INVALID_ARG),
        (dict(mid_tokens=48), K.KVQ_ERR_INVALID_ARG),                    # not a multiple of 32
        (dict(mid_tokens=32, block_tokens=16, num_blocks=8, max_blocks_per_seq=4),
         K.KVQ_ERR_UNSUPPORTED),                                         # middle tier: contiguous
        (dict(mid_tokens=32, group_tokens=2), K.KVQ_ERR_UNSUPPORTED),
        (dict(mid_tokens=32, key=dict(bits=8), value=dict(bits=4)), K.KVQ_ERR_UNSUPPORTED),
        (dict(mid_tokens=32, key=dict(bits=2, scale="u8_super"), value=dict(bits=2, scale="u8_super")),
         K.KVQ_ERR_UNSUPPORTED),
        (dict(mid_tokens=32, key=dict(bits=8, axis="channel"), value=dict(bits=4, scale="u8_super")),
         K.KVQ_ERR_UNSUPPORTED),
        (dict(mid_tokens=32, key=dict(bits=16), value=dict(bits=16)), K.KVQ_ERR_UNSUPPORTED),
    ]
    for over, want in bad:
        cfg = K.make_config(**{**base, **over})
        assert K.validate(cfg) == want, over
    good = [
        dict(key=dict(bits=16), value=dict(bits=16)),   # unquantized, contiguous
        dict(key=dict(bits=8, axis="channel_grow"), value=dict(bits=4, scale="u8_super"),
             window=32),
        dict(key=dict(bits=8, axis="channel_hold"), value=dict(bits=4, scale="u8_super"),
             window=32),
        dict(key=dict(bits=8, axis="channel_hold"), value=dict(bits=4, scale="u8_super"),
             window=16, block_tokens=16, num_blocks=8, max_blocks_per_seq=4),
        dict(key=dict(bits=2, scale="u8_super"), value=dict(bits=2, scale="u8_super"), window=16),
        dict(key=dict(bits=2), value=dict(bits=2)),
        dict(key=dict(bits=2, scale="u8_super"), value=dict(bits=2, scale="u8_super")),
        dict(key=dict(bits=2, zero_point=True, scale="f16"),
             value=dict(bits=2, zero_point=True, scale="f16")),
        dict(mid_tokens=32),
        dict(mid_tokens=256, window=16, key=dict(bits=4), value=dict(bits=4)),
        dict(mid_tokens=64, key=dict(bits=4, zero_point=True, scale="f16"),
             value=dict(bits=4, zero_point=True, scale="f16")),
        dict(mid_tokens=64, window=128, key=dict(bits=2, zero_point=True, scale="f16"),
             value=dict(bits=2, zero_point=True, scale="f16")),
    ]
    for over in good:
        assert K.validate(K.make_config(**{**base, **over})) == K.KVQ_OK, over


def test_calls_fail_before_launch():
    """Invalid arguments come back as status codes without any GPU call."""
    cfg = K.make_config(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, max_tokens=64,
                        key=dict(bits=8), value=dict(bits=8))
    desc = K.CacheDesc()
    lib = K.lib()
    # missing cache buffers
    st = lib.kvq_quantize_append(ctypes.byref(cfg), ctypes.byref(desc), 0, 1, 1, 4, None, None)
    assert st == K.KVQ_ERR_INVALID_ARG
    # layer out of range
    st = lib.kvq_decode_attn(ctypes.byref(cfg), ctypes.byref(desc), 3, 1, 1, None, 0, 64, None)
    assert st == K.KVQ_ERR_INVALID_ARG
    # workspace too small (cache pointers are fake; validation stops first)
    fake = K.CacheDesc(*([256] * 8), None, 256, 256)
    st = lib.kvq_decode_attn(ctypes.byref(cfg), ctypes.byref(fake), 0, 256, 256, 256, 16, 64, None)
    assert st == K.KVQ_ERR_WORKSPACE
    # misaligned workspace
    need = K.decode_workspace_bytes(cfg, 64)
    st = lib.kvq_decode_attn(ctypes.byref(cfg), ctypes.byref(fake), 0, 256, 256, 260, need, 64, None)
    assert st == K.KVQ_ERR_WORKSPACE
    # bad split option
    opts = K.DecodeOpts(100)
    st = lib.kvq_decode_attn_ex(ctypes.byref(cfg), ctypes.byref(fake), 0, 256, 256, 256, need, 64,
                                ctypes.byref(opts), None)
    assert st == K.KVQ_ERR_INVALID_ARG
    assert K.decode_workspace_bytes(cfg, 64, 100) == 0
    # query_bits: 0 or 8, and 8 is not run with per-channel keys
    opts = K.DecodeOpts(0)
    opts.query_bits = 4
    st = lib.kvq_decode_attn_ex(ctypes.byref(cfg), ctypes.byref(fake), 0, 256, 256, 256, need, 64,
                                ctypes.byref(opts), None)
    assert st == K.KVQ_ERR_INVALID_ARG
    cfg_ch = K.make_config(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, max_tokens=64,
                           key=dict(bits=8, axis="channel"), value=dict(bits=4, scale="u8_super"))
    opts.query_bits = 8
    st = lib.kvq_decode_attn_ex(ctypes.byref(cfg_ch), ctypes.byref(fake), 0, 256, 256, 256, need, 64,
                                ctypes.byref(opts), None)
    assert st == K.KVQ_ERR_UNSUPPORTED
    # n_new == 0 is a no-op
    st = lib.kvq_quantize_append(ctypes.byref(cfg), ctypes.byref(fake), 0, 256, 256, 0, None, None)
    assert st == K.KVQ_OK


def test_cache_bytes_workspace_field():
    """kvq_bytes.workspace is the decode workspace at the library's split for
    the longest sequence (max_tokens each without host lengths); it is not
    part of the cache's total, and 0 for a configuration the kernels do not
    run."""
    cfg = cfg_of(synth.workload(2))
    b = K.cache_bytes(cfg, None)
    assert b["workspace"] == K.decode_workspace_bytes(cfg, 4096) > 0
    assert b["total"] == b["payload"] + b["metadata"] + b["window"] + b["padding"]
    assert K.cache_bytes(cfg, [100] * 8)["workspace"] == K.decode_workspace_bytes(cfg, 100)
    odd = K.make_config(batch=1, num_q_heads=1, num_kv_heads=1, head_dim=64, max_tokens=64,
                        key=dict(bits=8), value=dict(bits=8))
    assert K.validate(odd) == K.KVQ_ERR_UNSUPPORTED
    ob = K.cache_bytes(odd, None)
    assert ob["total"] > 0 and ob["workspace"] == 0


@pytest.mark.parametrize("over", [
    dict(window=16),                                                    # append kernels, ring
    dict(mid_tokens=32, window=16),                                     # middle tier
    dict(key=dict(bits=8, axis="channel"), value=dict(bits=4, scale="u8_super")),
    dict(),                                                             # the one-kernel step
])
def test_decode_step_checks_before_launch(over):
    """kvq_decode_step checks every argument of its decode half before its
    append launches anything: a step with a workspace too small, a NULL
    query or output, or a misaligned workspace returns the error with no
    GPU call (here, with no GPU, a launch would return KVQ_ERR_HIP), so the
    cache is never changed by a rejected step."""
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, max_tokens=64,
                key=dict(bits=8), value=dict(bits=8))
    cfg = K.make_config(**{**base, **over})
    assert K.validate(cfg) == K.KVQ_OK
    fake = K.CacheDesc(*([256] * 8), None, 256, *([256] * 5))
    lib = K.lib()
    need = K.decode_workspace_bytes(cfg, 64)
    step = lambda q, out, ws, wsb: lib.kvq_decode_step(ctypes.byref(cfg), ctypes.byref(fake), 0,
                                                      256, 256, q, out, ws, wsb, 64, None)
    assert step(256, 256, 256, 16) == K.KVQ_ERR_WORKSPACE
    assert step(256, 256, 260, need) == K.KVQ_ERR_WORKSPACE
    assert step(None, 256, 256, need) == K.KVQ_ERR_INVALID_ARG
    assert step(256, None, 256, need) == K.KVQ_ERR_INVALID_ARG
    st = lib.kvq_decode_step(ctypes.byref(cfg), ctypes.byref(fake), 0, None, 256, 256, 256, 256,
                             need, 64, None)
    assert st == K.KVQ_ERR_INVALID_ARG


def test_workspace_grows_with_length():
    wl = synth.workload(2)
    cfg = cfg_of(wl)
    a = K.decode_workspace_bytes(cfg, 1024)
    b = K.decode_workspace_bytes(cfg, 4096, 256)
    assert 0 < a and 0 < b
    # partial outputs [B][Hq][splits][D] fp32, partial (max, sum) pairs and
    # one arrival counter per (sequence, KV head), each region 256-aligned
    hkv = cfg.num_kv_heads
    assert b == (-(-8 * 32 * 16 * 128 * 4 // 256) * 256 + -(-8 * 32 * 16 * 2 * 4 // 256) * 256
                 + -(-8 * hkv * 4 // 256) * 256)


def test_paged_split_limit():
    """A paged wave addresses at most 128 blocks, so explicit splits above
    8192 tokens are rejected for paged caches (contiguous ones accept them)."""
    wl = synth.workload(4)
    cfg = K.make_config(batch=2, num_q_heads=64, num_kv_heads=8, head_dim=128, max_tokens=32768,
                        key=wl["key"], value=wl["value"], window=128, block_tokens=16,
                        num_blocks=4096, max_blocks_per_seq=2048)
    assert K.decode_workspace_bytes(cfg, 32768, 8192) > 0
    assert K.decode_workspace_bytes(cfg, 32768, 8320) == 0
    cfg_c = cfg_of(synth.workload(2))
    assert K.decode_workspace_bytes(cfg_c, 4096, 16384) > 0


def _workspace_rows(cfg, max_len, nsp):
    """Workspace bytes for nsp partial rows per query head: the arrival
    counters, (max, sum) pairs and partial outputs, each region 256-aligned."""
    r = lambda x: -(-x // 256) * 256
    rows = cfg.batch * cfg.num_q_heads * nsp
    return r(cfg.batch * cfg.num_kv_heads * 4) + r(rows * 2 * 4) + r(rows * cfg.head_dim * 4)


@pytest.mark.parametrize("wid,nsp", [
    (1, 1),   # 512 tokens: one workgroup, which writes the output directly
    (2, 8),   # int8: 512 workgroups of 512 tokens over 64 (sequence, KV head) pairs
    (3, 3),   # uint4 on both sides: 768 workgroups, splits of 2816 tokens
    (5, 4),   # per-channel int8 keys: 512 workgroups of 16384 tokens
    (6, 3),   # int2 with 8-bit scale codes: 768 workgroups
    (8, 5),   # middle tier: splits of 3584 tokens (512 workgroups over the 7040 older
              # tokens); the plan counts splits over every token past the window (3),
              # then the window's row and the tier's row
])
def test_library_split_choice(wid, nsp):
    """The library's split aims at one round of workgroups at the decode
    kernel's occupancy: 768 for codes of at most 4 bits without a middle tier,
    512 otherwise (contiguous splits up to 16384 tokens); a cache of at most
    512 quantized tokens gets one split.  Checked through
    the workspace it asks for, which holds nsp partial rows per query head."""
    wl = synth.workload(wid)
    cfg = cfg_of(wl)
    max_len = max(synth.seq_lengths(wl))
    assert K.decode_workspace_bytes(cfg, max_len) == _workspace_rows(cfg, max_len, nsp)
