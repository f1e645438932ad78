"""kvq_decode_attn_noalloc (the allocation-free decode) against
kvq_decode_attn through the C ABI: the same kernels and split plan over the
library's own per-GPU scratch, so the outputs must be bit for bit those of
the call with a caller workspace.  Two calls in a row, the second with a
smaller input (and a third back at the first size, after a rejected call),
so counters and partials left by one call must not leak into the next."""
import numpy as np
import pytest
import torch

import gpu_harness as H
from decode_attention_quantized_kvq_amd import kvq as K
from decode_attention_quantized_kvq_amd import synth

pytestmark = pytest.mark.gpu


def _case(wid, over, lens, decode_steps=0):
    wl = synth.workload(wid, **over)
    bt = H.build(wl, lens, decode_steps=decode_steps)
    q = H.to_device(H.queries(wl), wl["in_dtype"])
    return bt, q


def _compare(bt, q, what):
    max_len = max(bt.lens)
    want = K.decode_attn(bt.cache, 0, q, max_len)
    out = torch.full_like(want, float("nan"))
    got = K.decode_attn_noalloc(bt.cache, 0, q, max_len, out)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got, want), f"{what}: allocation-free output differs"
    ref = np.stack([bt.oracle.attend(b, H.queries(bt.wl)[b]) for b in range(bt.wl["batch"])])
    H.check_close(got.cpu().numpy().astype(np.float64), ref, what)


def test_noalloc_matches_workspace_call():
    H.log("case: allocation-free decode, large then small then paged")
    # 1. workload 2's format, 8 sequences of ragged lengths up to 4096
    big, qb = _case(2, dict(batch=8, tokens=4096), [4096, 4000, 3333, 2500, 4096, 17, 0, 1234])
    _compare(big, qb, "noalloc gqa_int8 batch 8")
    # 2. a smaller input right after: 3 sequences, uint4 with zero points
    small, qs = _case(3, dict(batch=3, tokens=1024), [1000, 77, 513], decode_steps=2)
    _compare(small, qs, "noalloc int4 batch 3")
    # 3. a call beyond the scratch is rejected before anything launches: 64
    #    sequences x 64 query heads planned for 2^20 tokens need 64 splits of
    #    16384, 262144 partial rows (128 MiB) against 16 MiB
    cfg = K.make_config(batch=64, num_q_heads=64, num_kv_heads=8, head_dim=128, max_tokens=16,
                        key=dict(bits=8), value=dict(bits=8))
    tiny = K.KvqCache(cfg)
    qh = torch.zeros((64, 64, 128), dtype=torch.bfloat16, device="cuda")
    oh = torch.zeros((64, 64, 128), dtype=torch.float32, device="cuda")
    assert K.decode_workspace_bytes(cfg, 1 << 20) > (16 << 20)
    with pytest.raises(K.KvqError) as e:
        K.decode_attn_noalloc(tiny, 0, qh, 1 << 20, oh)
    assert e.value.status == K.KVQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert int(oh.count_nonzero()) == 0
    # 4. paged with a bf16 window, then the first case again
    paged, qp = _case(4, dict(batch=3, tokens=1024), [1000, 300, 131], decode_steps=2)
    _compare(paged, qp, "noalloc paged window")
    _compare(big, qb, "noalloc gqa_int8 batch 8 again")
