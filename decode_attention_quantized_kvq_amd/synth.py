"""Seeded synthetic inputs for the decode workloads.

This module only draws random numbers and rounds them to the input dtype; it
holds none of the quantization or attention arithmetic.  Both the HIP path and
the CPU oracle are fed from it.

Workloads (shapes and formats; the pages name no dataset, so every input is
synthetic):
  1 tiny_int8    batch 1, 1 query head / 1 KV head, D 128, 512 tokens, fp32
                 inputs, int8 symmetric per-token fp32 scale.
  2 gqa_int8     batch 8, 32/8 heads, 4096 tokens, bf16 inputs with 4 key
                 channels per KV head scaled x10, int8 symmetric per-token.
  3 int4_asym    batch 32, 32/8 heads, 8192 tokens, same values as 2, 4-bit
                 codes packed two per byte with fp16 scale + fp16 zero point.
  4 paged_mixed  batch 64, 64/8 heads, lengths uniform in [1024, 32768], the
                 newest 128 tokens kept bf16, older ones int8 per-token in
                 16-token blocks placed through a shuffled block table.
  5 asym_kv      batch 16, 32/8 heads, 65536 tokens; keys int8 per-channel
                 (outlier channels as in 2), values Laplace(0,1) int4 with an
                 8-bit scale relative to a per-head fp32 super-scale.
  6 int2_super   batch 32, 32/8 heads, 8192 tokens, same values as 2; keys and
                 values 2-bit symmetric with an 8-bit scale code relative to a
                 per-head fp32 super-scale (the 2-bit metadata remedy of "KV
                 Cache Quantization and Per-Token Scale Placement", section
                 "Per-token scales and where they can live").
  7 int2_group   batch 32, 32/8 heads, 8192 tokens, same values as 2; keys and
                 values uint2 with one fp16 scale + zero point per 16-token
                 group (the other 2-bit remedy of the same section: several
                 tokens under one scale).
  8 int4_tiered  batch 32, 32/8 heads, 8192 tokens, same values as 2; the
                 newest 128 in bf16, the next 1024 (to 1055) as int8 with fp32
                 scales, the older ones uint4 with fp16 scale + zero point
                 (precision that varies with recency, "KV Cache Quantization
                 and Per-Token Scale Placement", section "Precision floors and
                 mixed cache formats").

Recipe: every draw comes from ``np.random.default_rng(SeedSequence(key))``
with a key that names the workload, the replica and the tensor, so any
(sequence, KV head) slice can be regenerated on its own.  Values are drawn in
fp64, outlier key channels are multiplied by 10, and the result is rounded to
fp32 and then (bf16 workloads) to bf16, both ties-to-even.
"""

from __future__ import annotations

import copy
from typing import Dict, List

import numpy as np

_TOKEN_I8_F32 = dict(bits=8, axis="token", zero_point=False, scale="f32")

WORKLOADS: Dict[int, dict] = {
    1: dict(name="tiny_int8", batch=1, hq=1, hkv=1, d=128, tokens=512,
            lengths=None, in_dtype="f32", key=dict(_TOKEN_I8_F32),
            value=dict(_TOKEN_I8_F32), window=0, block_tokens=0,
            outlier_keys=0, value_dist="normal"),
    2: dict(name="gqa_int8", batch=8, hq=32, hkv=8, d=128, tokens=4096,
            lengths=None, in_dtype="bf16", key=dict(_TOKEN_I8_F32),
            value=dict(_TOKEN_I8_F32), window=0, block_tokens=0,
            outlier_keys=4, value_dist="normal"),
    3: dict(name="int4_asym", batch=32, hq=32, hkv=8, d=128, tokens=8192,
            lengths=None, in_dtype="bf16",
            key=dict(bits=4, axis="token", zero_point=True, scale="f16"),
            value=dict(bits=4, axis="token", zero_point=True, scale="f16"),
            window=0, block_tokens=0, outlier_keys=4, value_dist="normal"),
    4: dict(name="paged_mixed", batch=64, hq=64, hkv=8, d=128, tokens=32768,
            lengths=(1024, 32768), in_dtype="bf16", key=dict(_TOKEN_I8_F32),
            value=dict(_TOKEN_I8_F32), window=128, block_tokens=16,
            outlier_keys=4, value_dist="normal"),
    5: dict(name="asym_kv", batch=16, hq=32, hkv=8, d=128, tokens=65536,
            lengths=None, in_dtype="bf16",
            key=dict(bits=8, axis="channel", zero_point=False, scale="f32"),
            value=dict(bits=4, axis="token", zero_point=False, scale="u8_super"),
            window=0, block_tokens=0, outlier_keys=4, value_dist="laplace"),
    6: dict(name="int2_super", batch=32, hq=32, hkv=8, d=128, tokens=8192,
            lengths=None, in_dtype="bf16",
            key=dict(bits=2, axis="token", zero_point=False, scale="u8_super"),
            value=dict(bits=2, axis="token", zero_point=False, scale="u8_super"),
            window=0, block_tokens=0, outlier_keys=4, value_dist="normal"),
    7: dict(name="int2_group", batch=32, hq=32, hkv=8, d=128, tokens=8192,
            lengths=None, in_dtype="bf16",
            key=dict(bits=2, axis="token", zero_point=True, scale="f16"),
            value=dict(bits=2, axis="token", zero_point=True, scale="f16"),
            window=0, block_tokens=0, outlier_keys=4, value_dist="normal", group=16),
    8: dict(name="int4_tiered", batch=32, hq=32, hkv=8, d=128, tokens=8192,
            lengths=None, in_dtype="bf16",
            key=dict(bits=4, axis="token", zero_point=True, scale="f16"),
            value=dict(bits=4, axis="token", zero_point=True, scale="f16"),
            window=128, block_tokens=0, outlier_keys=4, value_dist="normal", mid=1024),
}


def workload(wid: int, **overrides) -> dict:
    """A copy of workload ``wid`` with some fields replaced (smaller parity
    cases keep the formats and value recipe of the full workload)."""
    wl = copy.deepcopy(WORKLOADS[wid])
    wl["id"] = wid
    for k, v in overrides.items():
        wl[k] = v
    return wl


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Round values ties-to-even to fp32, then (for "bf16") to bf16; returns
    float32 arrays whose values are exact in ``dtype``."""
    f = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return f
    assert dtype == "bf16"
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x_f32) -> np.ndarray:
    """The bf16 bit patterns (uint16) of float32 values exact in bf16."""
    return (np.asarray(x_f32, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def seq_lengths(wl: dict, replica: int = 0) -> List[int]:
    """Per-sequence token counts: fixed, or uniform on [lo, hi] inclusive."""
    if wl.get("lengths") is None:
        return [int(wl["tokens"])] * int(wl["batch"])
    lo, hi = wl["lengths"]
    rng = _rng(1000 + wl["id"], replica, 90)
    return [int(n) for n in rng.integers(lo, hi, size=wl["batch"], endpoint=True)]


def outlier_channels(wl: dict, h: int) -> np.ndarray:
    """The key channels of KV head h scaled x10 (same for every sequence)."""
    k = int(wl.get("outlier_keys", 0))
    if k == 0:
        return np.zeros(0, dtype=np.int64)
    rng = _rng(1000 + wl["id"], 7777, h)
    return np.sort(rng.choice(wl["d"], k, replace=False))


def kv_tokens(wl: dict, b: int, h: int, n: int, replica: int = 0, start: int = 0):
    """Keys and values of tokens [start, start+n) of sequence b, KV head h.

    Returns (K, V) float32 [n, D] holding values exact in the input dtype.
    Tokens are drawn in blocks of 4096 positions so that any token range of a
    sequence is reproducible without drawing the whole sequence.
    """
    d = wl["d"]
    out_k = np.empty((n, d), np.float32)
    out_v = np.empty((n, d), np.float32)
    chans = outlier_channels(wl, h)
    blk = 4096
    pos = start
    while pos < start + n:
        bi = pos // blk
        rng = _rng(1000 + wl["id"], replica, 1, b, h, bi)
        k = rng.standard_normal((blk, d))
        if wl["value_dist"] == "laplace":
            v = rng.laplace(0.0, 1.0, (blk, d))
        else:
            v = rng.standard_normal((blk, d))
        if chans.size:
            k[:, chans] *= 10.0
        lo = pos - bi * blk
        hi = min(blk, start + n - bi * blk)
        o = pos - start
        out_k[o:o + hi - lo] = round_to_dtype(k[lo:hi], wl["in_dtype"])
        out_v[o:o + hi - lo] = round_to_dtype(v[lo:hi], wl["in_dtype"])
        pos = bi * blk + hi
    return out_k, out_v


def queries(wl: dict, b: int, replica: int = 0, step: int = 0) -> np.ndarray:
    """Query vectors [Hq, D] of sequence b, N(0,1) in the input dtype."""
    rng = _rng(1000 + wl["id"], replica, 2, b, step)
    return round_to_dtype(rng.standard_normal((wl["hq"], wl["d"])), wl["in_dtype"])


def block_table(wl: dict, lens: List[int], replica: int = 0):
    """Shuffled placement of each sequence's quantized tokens in 16-token blocks.

    Sequence b needs ceil((len_b - W) / 16) blocks; the pool holds exactly the
    sum of those, handed out through one random permutation.  Returns
    (table int32 [B, max_blocks] padded with -1, pool block count).
    """
    bt = wl["block_tokens"]
    w = wl["window"]
    need = [-(-max(n - w, 0) // bt) for n in lens]
    max_blocks = -(-max(wl["tokens"] - w, 0) // bt)
    pool = int(sum(need))
    perm = _rng(1000 + wl["id"], replica, 3).permutation(pool).astype(np.int32)
    table = np.full((len(lens), max(max_blocks, 1)), -1, np.int32)
    off = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[off:off + nb]
        off += nb
    return table, pool


def kv_device(wl: dict, lens: List[int], replica: int = 0, device: str = "cuda"):
    """Keys and values of every sequence drawn on the device (for the full-size
    workloads, where drawing on the host takes minutes).

    Same recipe as ``kv_tokens`` (N(0,1) or Laplace(0,1), outlier key channels
    x10, rounded to the input dtype) but drawn by torch's Philox generator on
    the device, seeded from the workload and replica; positions past a
    sequence's length are zero.  Returns (K, V) [B, H_kv, max(lens), D] in the
    input dtype.  The values differ from ``kv_tokens``'s; tests that compare
    with the oracle copy the slices they need back to the host.
    """
    import torch
    B, H, D = wl["batch"], wl["hkv"], wl["d"]
    T = max(lens) if lens else 0
    dt = torch.bfloat16 if wl["in_dtype"] == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed(int(np.random.SeedSequence([1000 + wl["id"], replica, 5]).generate_state(1)[0]))
    k = torch.empty((B, H, T, D), dtype=dt, device=device)
    v = torch.empty((B, H, T, D), dtype=dt, device=device)
    for b in range(B):                    # one sequence at a time bounds the fp32 temporaries
        kb = torch.randn((H, T, D), generator=gen, device=device, dtype=torch.float32)
        for h in range(H):
            ch = torch.from_numpy(outlier_channels(wl, h)).to(device)
            if ch.numel():
                kb[h, :, ch] *= 10.0
        if wl["value_dist"] == "laplace":
            u = torch.rand((H, T, D), generator=gen, device=device, dtype=torch.float32) - 0.5
            # inverse CDF; rand() can return exactly 0 (u = -1/2, log 0), so the
            # tail is cut at the smallest nonzero draw, 2^-24
            vb = -torch.sign(u) * torch.log1p(-2.0 * u.abs()).clamp_min(-16.635532333438686)
        else:
            vb = torch.randn((H, T, D), generator=gen, device=device, dtype=torch.float32)
        kb[:, lens[b]:] = 0
        vb[:, lens[b]:] = 0
        k[b] = kb.to(dt)
        v[b] = vb.to(dt)
    return k, v
