"""The allocation-free decode attention (fixed library scratch) against the
workspace entry point: the same kernels, so the outputs must be identical,
on two calls in a row, the second with a smaller input (the scratch keeps
the first call's contents)."""
import sys

import numpy as np
import pytest
import torch

from tests.parity import to_dev
from trainable_sparse_attention_amd import inputs, qsa

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _decode_case(B, n_q, lens, seed):
    d = inputs.small(B=B, n=max(lens), hq=16, hkv=2, dtype="bf16", seed=seed)
    p = qsa.params()
    t = {k: to_dev(d[k]) for k in ("q_idx", "k_idx", "q", "k", "v")}
    nb = max(lens) // 4
    kbar = torch.empty((B, nb, 128), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_pool_keys(p, t["k_idx"], kbar, 0, nb)
    seq_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    qi = torch.stack([t["q_idx"][b, L - n_q:L] for b, L in enumerate(lens)]).contiguous()
    qq = torch.stack([t["q"][b, L - n_q:L] for b, L in enumerate(lens)]).contiguous()
    kB = qsa.k_blocks(p)
    idx = torch.empty((B, n_q, kB), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, n_q), dtype=torch.int32, device="cuda")
    ws = qsa.workspace(qsa.qsa_index_topk_workspace(p, qsa.QSA_BF16, B, n_q, nb, True))
    qsa.qsa_index_topk(p, qi, kbar, idx, cnt, ws, 0, seq_len)
    return p, t, qq, seq_len, idx, cnt


def test_noalloc_decode_equals_workspace_decode():
    outs = []
    for B, n_q, lens, seed in [(4, 4, (12000, 9001, 20003, 4099), 61), (2, 1, (6000, 3001), 62)]:
        say("noalloc decode B=%d n_q=%d lens=%s" % (B, n_q, lens))
        p, t, qq, seq_len, idx, cnt = _decode_case(B, n_q, list(lens), seed)
        ref = torch.empty_like(qq)
        ws = qsa.workspace(qsa.qsa_sparse_attn_decode_workspace(p, B, n_q, 16, 2))
        qsa.qsa_sparse_attn_decode(p, qq, t["k"], t["v"], seq_len, idx, cnt, ref, ws)
        got = torch.full_like(qq, 7.0)
        qsa.qsa_sparse_attn_decode_noalloc(p, qq, t["k"], t["v"], seq_len, idx, cnt, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), "allocation-free decode differs from the workspace form"
        assert torch.isfinite(got.float()).all()
        outs.append(got)
    say("noalloc decode: both calls equal the workspace entry point")


def test_noalloc_rejects_sizes_beyond_the_scratch():
    p = qsa.params()
    need = qsa.qsa_sparse_attn_decode_workspace(p, 512, 4, 16, 2)
    assert need > 64 << 20
    q = torch.empty((512, 4, 16, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((512, 2, 8, 128), dtype=torch.bfloat16, device="cuda")
    seq_len = torch.full((512,), 8, dtype=torch.int32, device="cuda")
    idx = torch.empty((512, 4, 512), dtype=torch.int32, device="cuda")
    cnt = torch.empty((512, 4), dtype=torch.int32, device="cuda")
    with pytest.raises(qsa.QSAError) as e:
        qsa.qsa_sparse_attn_decode_noalloc(p, q, kv, kv, seq_len, idx, cnt, torch.empty_like(q))
    assert e.value.status == 5
