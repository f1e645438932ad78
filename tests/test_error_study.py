"""The attention-error study (oracle/error_study.py): its stored table
reproduces, and the structure that does not depend on the draw holds."""
import json
import os

import pytest

from oracle import error_study as ES

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "error_study.json")


def _flat(x, prefix=""):
    if isinstance(x, dict):
        for k, v in x.items():
            yield from _flat(v, f"{prefix}/{k}")
    else:
        yield prefix, x


def test_golden_table_reproduces():
    want = dict(_flat(json.load(open(GOLDEN))))
    got = dict(_flat(json.loads(json.dumps(ES.study(want["/pairs"], want["/tokens"])))))
    assert got.keys() == want.keys()
    for k, v in want.items():
        if isinstance(v, float):
            assert got[k] == pytest.approx(v, rel=1e-9, abs=1e-15), k
        else:
            assert got[k] == v, k


@pytest.mark.parametrize("case", [c[0] for c in ES.CASES])
def test_error_structure(case):
    r = ES.study(pairs=2, tokens=512)["cases"][case]
    for which in ("K", "V", "KV"):
        e = {b: r[b][which] for b in ("8", "4", "2")}
        assert e["8"]["out_rel"] < e["4"]["out_rel"] < e["2"]["out_rel"], which
        if which != "V":      # key error acts before the softmax
            for key in ("recon_K", "score_rms", "tv"):
                assert e["8"][key] < e["4"][key] < e["2"][key], (which, key)
        else:                 # value error leaves scores and weights exact
            assert all(e[b]["score_rms"] == 0 and e[b]["tv"] == 0 and e[b]["top1"] == 1 for b in e)
        if which != "K":
            assert e["8"]["recon_V"] < e["4"]["recon_V"] < e["2"]["recon_V"]
        else:
            assert all(e[b]["recon_V"] == 0 for b in e)


def test_channel_scales_help_outlier_keys_at_8_and_4_bits():
    r = ES.study(pairs=2, tokens=512)["cases"]
    tok, ch = r["outlier keys, per-token scales"], r["outlier keys, per-channel key scales"]
    for b in ("8", "4"):
        assert ch[b]["K"]["recon_K"] < tok[b]["K"]["recon_K"]
        assert ch[b]["K"]["tv"] < tok[b]["K"]["tv"]
