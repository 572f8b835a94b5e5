"""GPU parity of the training path against the oracle ([hub] "Key ideas",
native-trainability bullet): the sparse-attention backward (stage 2, joint
sparse training), the indexer distillation loss and its gradients (stage 1),
and the pooling backward that carries the pooled-key gradient to the raw
indexer keys.

Tolerances: gradients and losses are accumulated in float32 from bf16
inputs (the attention backward rounds P and dS to bf16 for its MFMA
products, as the forward rounds P), so outputs are compared with the
max-abs relative error of the bf16 class, 2e-2, and the distillation
(float32 throughout, the student's query carried as bf16 hi + lo) with
2e-3.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL, rel_err, to_dev, to_host
from trainable_sparse_attention_amd import inputs, qsa

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _bf16(x):
    return inputs.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


# ReLU has no derivative at 0, and the pages fix no subgradient there: where
# an indexer pre-activation <q~_h, kbar_b> lies within rounding of 0, gating
# block b's gradient on or off are both correct results.  A gate is taken as
# such a near-tie when |<q~_h, kbar_b>| <= 1e-5 |q~_h| |kbar_b| (float32 and
# the bf16 hi + lo query carry errors of a few 1e-6 of that), and each one
# widens the bound of the entries it feeds by its whole contribution:
# |rotated-back g_b kbar_b| for dq_idx of that (row, head), |g_b q~_h| for
# dkbar of that block, g_b being the oracle's d loss / d I_b.
GATE_EPS = 1e-5


def _gate_slack(q_idx_rows, kbar_h, pos, g):
    """Elementwise allowances (dq_idx [m][h][d], dkbar [nb_cap][d]) and the
    number of near-tie gates of rows q_idx_rows at positions pos."""
    m, h, dd = q_idx_rows.shape
    pos = np.asarray(pos, dtype=np.int64)
    q = oracle.rope_rows(inputs.bf16_bits_to_f32(q_idx_rows.reshape(m * h, dd)).astype(np.float64),
                         np.repeat(pos, h)).reshape(m, h, dd)
    kb = inputs.bf16_bits_to_f32(kbar_h).astype(np.float64)
    kn = np.linalg.norm(kb, axis=1)
    dq_slack = np.zeros((m, h, dd))
    dkb_slack = np.zeros_like(kb)
    count = 0
    for u in range(m):
        nb = int(pos[u] + 1) // 4
        if nb == 0:
            continue
        dots = q[u] @ kb[:nb].T                                    # [h][nb]
        near = np.abs(dots) <= GATE_EPS * np.linalg.norm(q[u], axis=1)[:, None] * kn[None, :nb]
        for hh, blk in zip(*np.nonzero(near)):
            v = oracle.rope_rows((g[u, blk] * kb[blk])[None], np.array([-pos[u]]))[0]
            dq_slack[u, hh] += np.abs(v)
            dkb_slack[blk] += np.abs(g[u, blk] * q[u, hh])
            count += 1
    return dq_slack, dkb_slack, count


def _assert_close_slack(got, ref, tol, slack, what):
    """|got - ref| <= tol max|ref| + slack elementwise."""
    bad = np.abs(got - ref) > tol * np.max(np.abs(ref)) + slack
    assert not bad.any(), "%s: %d entries beyond the bound, worst excess %.3e of max|ref|" % (
        what, int(bad.sum()), float(np.max((np.abs(got - ref) - slack)[bad]) / np.max(np.abs(ref))))


@pytest.mark.parametrize("r,n,K,q_pos0,hq,hkv", [(4, 1200, 256, 0, 16, 2), (8, 1500, 512, 0, 16, 2),
                                                  (4, 2000, 512, 1300, 16, 2),
                                                  (1, 700, 256, 0, 8, 2), (16, 3001, 512, 0, 16, 1),
                                                  (2, 1003, 128, 500, 6, 2), (4, 777, 64, 0, 2, 2)])
def test_sparse_attn_backward(r, n, K, q_pos0, hq, hkv):
    """Query-side dq and key-side dk, dv (16 / G rows per key-side step:
    G = hq / hkv of 8, 4, 16, 3 (not a divisor of 16) and 1)."""
    say("sparse attention backward r=%d n=%d K=%d q_pos0=%d hq=%d hkv=%d" % (r, n, K, q_pos0, hq,
                                                                          hkv))
    B = 2
    d = inputs.small(B=B, n=n, hq=hq, hkv=hkv, dtype="bf16", r=r, K=K, seed=600 + r)
    p = qsa.params(r=r, K=K)
    kB = qsa.k_blocks(p)
    t = {k_: to_dev(d[k_]) for k_ in ("q_idx", "k_idx", "q", "k", "v")}
    nb = n // r
    kbar = torch.empty((B, nb, 128), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_pool_keys(p, t["k_idx"], kbar, 0, nb)
    n_q = n - q_pos0
    qi = t["q_idx"][:, q_pos0:].contiguous()
    qq = t["q"][:, q_pos0:].contiguous()
    idx = torch.empty((B, n_q, kB), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, n_q), dtype=torch.int32, device="cuda")
    ws = qsa.workspace(qsa.qsa_index_topk_workspace(p, qsa.QSA_BF16, B, n_q, nb, False))
    qsa.qsa_index_topk(p, qi, kbar, idx, cnt, ws, q_pos0)
    out = torch.empty_like(qq)
    qsa.qsa_sparse_attn_prefill(p, qq, t["k"], t["v"], idx, cnt, out, q_pos0)
    rng = np.random.default_rng(7)
    dout_h = _bf16(rng.standard_normal((B, n_q, hq, 128)) * 0.1)
    dout = to_dev(dout_h)
    dq = torch.empty((B, n_q, hq, 128), dtype=torch.float32, device="cuda")
    dk = torch.zeros((B, hkv, n, 128), dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    wsb = qsa.workspace(qsa.qsa_sparse_attn_backward_workspace(p, B, n_q, q_pos0, hq))
    qsa.qsa_sparse_attn_backward(p, qq, t["k"], t["v"], idx, cnt, out, dout, dq, dk, dv, wsb,
                                 q_pos0)
    # a second call into fresh buffers reproduces the first bit for bit (the
    # key side sums each key's rows in ascending row order)
    dq2 = torch.empty_like(dq)
    dk2, dv2 = torch.zeros_like(dk), torch.zeros_like(dv)
    qsa.qsa_sparse_attn_backward(p, qq, t["k"], t["v"], idx, cnt, out, dout, dq2, dk2, dv2, wsb,
                                 q_pos0)
    torch.cuda.synchronize()
    g_idx, g_cnt = to_host(idx), to_host(cnt)
    g_dq, g_dk, g_dv = dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    pos = q_pos0 + np.arange(n_q)
    for b in range(B):
        dout_f = inputs.bf16_bits_to_f32(dout_h[b]).astype(np.float64)
        o_dq, o_dk, o_dv = oracle.attend_backward(d["q"][b][pos], d["k"][b], d["v"][b], pos,
                                                  g_idx[b], g_cnt[b], dout_f, r=r)
        errs = [rel_err(g_dq[b], o_dq), rel_err(g_dk[b], o_dk), rel_err(g_dv[b], o_dv)]
        say("seq %d: dq %.2e dk %.2e dv %.2e" % (b, *errs))
        assert max(errs) <= TOL["bf16"]
        # key rows no query attended keep their cleared value
        untouched = np.all(o_dk == 0.0, axis=2)
        assert np.all(g_dk[b][untouched] == 0.0) and np.all(g_dv[b][untouched] == 0.0)


@pytest.mark.parametrize("n,q_pos0,hq,hkv", [(1000, 0, 16, 2), (1500, 900, 16, 2),
                                             (777, 0, 8, 1), (900, 100, 16, 8)])
def test_index_distill(n, q_pos0, hq, hkv):
    say("distillation n=%d q_pos0=%d hq=%d hkv=%d" % (n, q_pos0, hq, hkv))
    B = 2
    d = inputs.small(B=B, n=n, hq=hq, hkv=hkv, dtype="bf16", seed=700 + n, planted=0)
    p = qsa.params()
    t = {k_: to_dev(d[k_]) for k_ in ("q_idx", "k_idx", "q", "k")}
    nb = n // 4
    kbar = torch.empty((B, nb, 128), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_pool_keys(p, t["k_idx"], kbar, 0, nb)
    n_q = n - q_pos0
    qq = t["q"][:, q_pos0:].contiguous()
    qi = t["q_idx"][:, q_pos0:].contiguous()
    loss = torch.full((B, n_q), -1.0, dtype=torch.float32, device="cuda")
    dq = torch.empty((B, n_q, 4, 128), dtype=torch.float32, device="cuda")
    dkb = torch.zeros((B, nb, 128), dtype=torch.float32, device="cuda")
    # the workspace needs no clearing: start it as NaN bit patterns
    ws = qsa.workspace(qsa.qsa_index_distill_workspace(p, B, n_q, q_pos0))
    ws.fill_(255)
    qsa.qsa_index_distill(p, qq, t["k"], qi, kbar, loss, dq, dkb, ws, q_pos0)
    # the pooled-key gradient carried to the raw indexer keys
    dk_idx = torch.zeros((B, n, 128), dtype=torch.float32, device="cuda")
    qsa.qsa_pool_keys_backward(p, dkb, dk_idx, 0, nb)
    torch.cuda.synchronize()
    kbar_h = to_host(kbar)
    g_loss, g_dq, g_dkb, g_dk = (x.cpu().numpy() for x in (loss, dq, dkb, dk_idx))
    pos = q_pos0 + np.arange(n_q)
    for b in range(B):
        o_loss, o_dq, o_dkb, o_g = oracle.distill_rows(d["q"][b][pos], d["k"][b],
                                                       d["q_idx"][b][pos], kbar_h[b], pos,
                                                       return_g=True)
        dq_slack, dkb_slack, ngate = _gate_slack(d["q_idx"][b][pos], kbar_h[b], pos, o_g)
        _assert_close_slack(g_dq[b], o_dq, 2e-3, dq_slack, "seq %d dq_idx" % b)
        _assert_close_slack(g_dkb[b], o_dkb, 2e-3, dkb_slack, "seq %d dkbar" % b)
        errs = [rel_err(g_loss[b], o_loss), rel_err(g_dq[b], o_dq), rel_err(g_dkb[b], o_dkb)]
        say("seq %d: loss %.2e dq_idx %.2e dkbar %.2e (mean loss %.4f; %d near-tie gates)" % (
            b, *errs, float(o_loss.mean()), ngate))
        assert errs[0] <= 2e-3  # the loss has no gate: compared as is
        assert np.all(g_loss[b][pos < 3] == 0.0)
        o_dk = oracle.pool_backward(g_dkb[b].astype(np.float64))
        assert rel_err(g_dk[b][:nb * 4], o_dk) <= 1e-6


def test_training_full_size_sampled():
    """The training kernels at the 32K-token workload the bench times, in its
    launch configuration (B = 1, n = 32768, 16 q / 2 kv heads).  Per row:
    distillation loss and dq_idx and the backward's dq on sampled rows (the
    first, the last, around 2048 and 16384, and random ones).  Per key: keys
    of the last 8 blocks are reached only by rows n - 32 .. n - 1 (selected
    blocks lie below a row's position and tails start at it), so the
    oracle over those rows gives their whole dkbar, dk and dv."""
    say("full-size training kernels, train_32k")
    d = inputs.make("train_32k", seed=8, backend="torch")
    p = qsa.params()
    B, n, hq, hkv = d["B"], d["n"], d["hq"], d["hkv"]
    nb = n // 4
    kbar, idx, cnt, out = qsa.prefill(p, d["k_idx"], d["q_idx"], d["q"], d["k"], d["v"])
    loss = torch.empty((B, n), dtype=torch.float32, device="cuda")
    dqi = torch.empty((B, n, 4, 128), dtype=torch.float32, device="cuda")
    dkb = torch.zeros((B, nb, 128), dtype=torch.float32, device="cuda")
    wsd = qsa.workspace(qsa.qsa_index_distill_workspace(p, B, n, 0))
    qsa.qsa_index_distill(p, d["q"], d["k"], d["q_idx"], kbar, loss, dqi, dkb, wsd, 0)
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    dout = (torch.randn(out.shape, generator=g, device="cuda") * 0.1).to(torch.bfloat16)
    dq = torch.empty((B, n, hq, 128), dtype=torch.float32, device="cuda")
    dk = torch.zeros((B, hkv, n, 128), dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    wsb = qsa.workspace(qsa.qsa_sparse_attn_backward_workspace(p, B, n, 0, hq))
    qsa.qsa_sparse_attn_backward(p, d["q"], d["k"], d["v"], idx, cnt, out, dout, dq, dk, dv, wsb,
                                 0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    tail = np.arange(n - 32, n)
    rows = np.unique(np.concatenate([np.arange(6), [2046, 2047, 2048, 16383, 16384], tail,
                                     rng.choice(n, 16, replace=False)])).astype(np.int64)
    rt = torch.from_numpy(rows).cuda()
    q_h, k_h, v_h = to_host(d["q"][0]), to_host(d["k"][0]), to_host(d["v"][0])
    qi_h, kbar_h = to_host(d["q_idx"][0]), to_host(kbar[0])
    # distillation: loss and dq_idx per row; dkbar of the last 8 blocks
    o_loss, o_dq, o_dkb, o_g = oracle.distill_rows(q_h[rows], k_h, qi_h[rows], kbar_h, rows,
                                                   return_g=True)
    _, _, o_dkb_tail, o_g_tail = oracle.distill_rows(q_h[tail], k_h, qi_h[tail], kbar_h, tail,
                                                     return_g=True)
    g_loss = loss[0][rt].cpu().numpy()
    d_loss = float(np.max(np.abs(g_loss - o_loss)))
    dq_slack, _, ngate = _gate_slack(qi_h[rows], kbar_h, rows, o_g)
    _, dkb_slack, ngate_tail = _gate_slack(qi_h[tail], kbar_h, tail, o_g_tail)
    g_dqi, g_dkb_tail = dqi[0][rt].cpu().numpy(), dkb[0][nb - 8:].cpu().numpy()
    _assert_close_slack(g_dqi, o_dq, 2e-3, dq_slack, "dq_idx")
    _assert_close_slack(g_dkb_tail, o_dkb_tail[nb - 8:], 2e-3, dkb_slack[nb - 8:], "dkbar")
    say("near-tie gates: %d over the sampled rows, %d over the tail rows" % (ngate, ngate_tail))
    errs = [rel_err(g_dqi, o_dq), rel_err(g_dkb_tail, o_dkb_tail[nb - 8:])]
    say("distillation over %d rows: loss max |err| %.2e (max |loss| %.2e), dq_idx %.2e, "
        "dkbar (last 8 blocks) %.2e" % (rows.size, d_loss, float(np.max(np.abs(o_loss))), *errs))
    # The loss (a KL divergence, >= 0 and small) is a difference of per-row
    # terms of size ln(blocks) + max I, up to about 20 here.  Each lane sums
    # at most 512 blocks in float32 (a random-walk error near
    # sqrt(512) * 2^-24 = 1.3e-6 relative) before the lanes are combined, so
    # the loss carries an absolute error near 2e-5 even when every term is
    # right to float32 precision.
    assert d_loss <= 2e-3 * float(np.max(np.abs(o_loss))) + 2e-5
    # backward: dq per row; dk, dv of the keys of the last 8 blocks
    g_idx, g_cnt = to_host(idx[0]), to_host(cnt[0])
    dout_f = inputs.bf16_bits_to_f32(to_host(dout[0])).astype(np.float64)
    o_dq, _, _ = oracle.attend_backward(q_h[rows], k_h, v_h, rows, g_idx[rows], g_cnt[rows],
                                        dout_f[rows])
    _, o_dk, o_dv = oracle.attend_backward(q_h[tail], k_h, v_h, tail, g_idx[tail], g_cnt[tail],
                                           dout_f[tail])
    keys = slice(n - 32, n)
    errs = [rel_err(dq[0][rt].cpu().numpy(), o_dq),
            rel_err(dk[0][:, keys].cpu().numpy(), o_dk[:, keys]),
            rel_err(dv[0][:, keys].cpu().numpy(), o_dv[:, keys])]
    say("backward over %d rows: dq %.2e; last 32 keys: dk %.2e dv %.2e" % (rows.size, *errs))
    assert max(errs) <= TOL["bf16"]


def _random_backward_config(i):
    rng = np.random.default_rng(6000 + i)
    r = int(rng.choice([1, 2, 4, 8, 16]))
    K = int(rng.choice([64, 128, 256, 512, 1024, 2048]))
    hq, hkv = [(16, 2), (8, 2), (16, 1), (6, 2), (2, 2), (16, 4), (12, 4)][int(rng.integers(0, 7))]
    n = int(rng.integers(300, 3500))
    q_pos0 = int(rng.integers(0, n // 2)) if rng.random() < 0.5 else 0
    return r, n, K, q_pos0, hq, hkv


@pytest.mark.parametrize("i", range(10))
def test_random_backward_configurations(i):
    """The sparse-attention backward over a seeded sweep of micro-block
    sizes, K, query/KV head ratios, lengths and chunk offsets (the checks of
    test_sparse_attn_backward: dq, dk, dv against the oracle, untouched keys
    exactly zero, a second call equal bit for bit)."""
    test_sparse_attn_backward(*_random_backward_config(i))


@pytest.mark.parametrize("i", range(6))
def test_random_distill_configurations(i):
    """The distillation and the pooling backward over a seeded sweep of
    lengths, chunk offsets and query/KV head ratios (r = 4 and 4 indexer
    heads, the form the distillation is built for)."""
    rng = np.random.default_rng(7000 + i)
    hq, hkv = [(16, 2), (8, 1), (16, 8), (4, 4), (12, 6), (16, 16 // 2)][int(rng.integers(0, 6))]
    n = int(rng.integers(200, 2500))
    q_pos0 = int(rng.integers(0, n // 2)) if rng.random() < 0.5 else 0
    test_index_distill(n, q_pos0, hq, hkv)
