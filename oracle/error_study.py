"""Attention-error study on synthetic data, with the oracle only.

TEST INFRASTRUCTURE / STUDY, NOT PRODUCT CODE.  It imports the oracle and the
seeded input generators, nothing from the HIP library.

What it measures, for symmetric quantization at 8, 4 and 2 bits with fp32
scales (values per token; keys per token or per channel), of the keys only,
the values only, or both, on three input cases (keys with 4 outlier channels
x10 per head with per-token or per-channel key scales, and plain Gaussian
keys):
  * reconstruction error of the quantized tensor, ||X_hat - X||_F / ||X||_F;
  * score error s' - s with s = q.k / sqrt(D) (RMS and max |.|);
  * attention-distribution error: total variation 1/2 sum |a' - a|, the
    change of entropy H(a') - H(a) (positive = flatter), and whether the
    most attended position is still the same;
  * output error ||o' - o|| / ||o||.
The pages say where each error acts: key error before the softmax, value
error after the weights are formed ([P1] "Key error acts before the
softmax", "Value error acts after attention weights are formed"), and what
degrades first as bits drop: the softmax's discrimination between similar
scores, flatter distributions at 4 bits, a missed position at 2 bits ([P3]
"What degrades first").  This study measures those quantities on the
synthetic inputs; it asserts none of the pages' claims.

Run: python -m oracle.error_study [--pairs N] [--tokens T] [--out FILE]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys

import numpy as np

if __package__ in (None, ""):
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from oracle import kvq_oracle as O  # noqa: E402
from decode_attention_quantized_kvq_amd import synth  # noqa: E402


def _entropy(a):
    a = a[a > 0]
    return float(-(a * np.log(a)).sum())


CASES = (
    # name, workload whose key/value recipe is used, key axis
    ("outlier keys, per-token scales", 2, "token"),
    ("outlier keys, per-channel key scales", 2, "channel"),
    ("gaussian keys, per-token scales", 1, "token"),
)


def _quant(x, bits, axis):
    """Reconstruction of x [T, D] quantized symmetrically with fp32 scales."""
    if axis == "channel":
        sc = O.channel_scales(x, bits)          # over all T tokens, as one prefill
        return O.dequant_channel(O.quantize_with_channel_scales(x, sc, bits), sc)
    c, s = O.quantize_sym(x, bits, "f32")
    return O.dequant_sym(c, s)


def study(pairs: int = 4, tokens: int = 4096, bits_list=(8, 4, 2)):
    """Returns {"cases": {name: {bits: {"K"|"V"|"KV": metrics}}}, ...}."""
    out = {}
    for name, wid, axis in CASES:
        wl = synth.workload(wid, tokens=tokens)
        G = wl["hq"] // wl["hkv"]
        acc = {b: {w: {} for w in ("K", "V", "KV")} for b in bits_list}
        for p in range(pairs):
            bq, h, rep = p % wl["batch"], (p * 3) % wl["hkv"], p // (wl["batch"] * wl["hkv"])
            k, v = synth.kv_tokens(wl, bq, h, tokens, replica=rep)
            q = synth.queries(wl, bq, replica=rep)[h * G:(h + 1) * G]
            s_ref = np.stack([O.scores(q[i], k) for i in range(G)])
            a_ref = np.stack([O.softmax(s) for s in s_ref])
            o_ref = a_ref @ v
            for b in bits_list:
                k_hat, v_hat = _quant(k, b, axis), _quant(v, b, "token")
                for which, kk, vv in (("K", k_hat, v), ("V", k, v_hat), ("KV", k_hat, v_hat)):
                    s = np.stack([O.scores(q[i], kk) for i in range(G)])
                    a = np.stack([O.softmax(x) for x in s])
                    o = a @ vv
                    m = dict(
                        recon_K=float(np.linalg.norm(kk - k) / np.linalg.norm(k)),
                        recon_V=float(np.linalg.norm(vv - v) / np.linalg.norm(v)),
                        score_rms=float(np.sqrt(np.mean((s - s_ref) ** 2))),
                        score_max=float(np.max(np.abs(s - s_ref))),
                        tv=float(np.mean(0.5 * np.abs(a - a_ref).sum(axis=1))),
                        dH=float(np.mean([_entropy(a[i]) - _entropy(a_ref[i]) for i in range(G)])),
                        top1=float(np.mean(np.argmax(a, 1) == np.argmax(a_ref, 1))),
                        out_rel=float(np.mean(np.linalg.norm(o - o_ref, axis=1)
                                              / np.linalg.norm(o_ref, axis=1))),
                    )
                    for key, val in m.items():
                        acc[b][which].setdefault(key, []).append(val)
        out[name] = {str(b): {w: {k2: float(np.mean(v2)) for k2, v2 in acc[b][w].items()}
                              for w in ("K", "V", "KV")} for b in bits_list}
    return {"tokens": tokens, "pairs": pairs, "values": "per-token symmetric, fp32 scale",
            "cases": out}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--pairs", type=int, default=4)
    ap.add_argument("--tokens", type=int, default=4096)
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    res = study(args.pairs, args.tokens)
    txt = json.dumps(res, indent=1)
    if args.out:
        with open(args.out, "w") as f:
            f.write(txt + "\n")
    print(txt)


if __name__ == "__main__":
    main()
