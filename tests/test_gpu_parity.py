"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Stage isolation: each GPU stage is compared with the oracle stage fed the
same bytes the GPU stage read (the oracle selects on the GPU's pooled keys;
the oracle attends with the GPU's selection), so a near-tie difference in
one stage cannot leak into the next.  Sets use the near-tie rule and outputs
the max-abs relative error of tests/parity.py.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL, as_f64, check_sets, rel_err, to_dev, to_host
from trainable_sparse_attention_amd import inputs, qsa

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _params(K=2048, rope_dims=64):
    return qsa.params(K=K, rope_dims=rope_dims)


def _dev_inputs(d):
    return {k: to_dev(d[k]) for k in ("q_idx", "k_idx", "q", "k", "v")}


def _pool_gpu(p, k_idx, nb):
    kbar = torch.empty((k_idx.shape[0], nb, 128), dtype=k_idx.dtype, device=k_idx.device)
    qsa.qsa_pool_keys(p, k_idx, kbar, 0, nb)
    return kbar


def _index_gpu(p, q_idx, kbar, q_pos0=0, seq_len=None):
    B, n_q = q_idx.shape[:2]
    kB = qsa.k_blocks(p)
    idx = torch.full((B, n_q, kB), -7, dtype=torch.int32, device=q_idx.device)
    cnt = torch.full((B, n_q), -7, dtype=torch.int32, device=q_idx.device)
    ws = qsa.workspace(qsa.qsa_index_topk_workspace(p, qsa.dtype_code(q_idx), B, n_q,
                                                    kbar.shape[1], seq_len is not None))
    qsa.qsa_index_topk(p, q_idx, kbar, idx, cnt, ws, q_pos0, seq_len)
    _assert_ids_valid(p, idx, cnt, q_pos0, seq_len)
    return idx, cnt


def _assert_ids_valid(p, idx, cnt, q_pos0, seq_len):
    """Every row's count is min(k_B, visible blocks) and its ids are distinct,
    ascending and visible, padded with -1: checked on the host before any
    kernel gathers through them."""
    B, n_q, kB = idx.shape
    g_idx, g_cnt = to_host(idx), to_host(cnt)
    lens = to_host(seq_len) if seq_len is not None else None
    for b in range(B):
        off = int(lens[b]) - n_q if lens is not None else q_pos0
        nvis = (off + np.arange(n_q) + 1) // p.r
        k = np.minimum(kB, nvis)
        assert np.array_equal(g_cnt[b], k), "index counts"
        col = np.arange(kB)[None, :]
        ids = g_idx[b]
        live = col < k[:, None]
        assert np.all(ids[~live] == -1), "index padding"
        assert np.all((ids >= 0) & (ids < nvis[:, None]) | ~live), "index ids out of range"
        assert np.all((np.diff(ids, axis=1) > 0) | ~live[:, 1:]), "index ids not ascending"


def _intact_plants(plants):
    """Planted matches whose keys no later plant of the same sequence
    overwrote (plants land on uniformly drawn blocks, so two can share one;
    the later one then holds the block's keys)."""
    last = {}
    for u, (b, i, blk, *_r) in enumerate(plants):
        last[(b, blk)] = u
    return [pl for u, pl in enumerate(plants) if last[(pl[0], pl[2])] == u]


def _attn_gpu(p, q, k, v, idx, cnt, q_pos0=0):
    out = torch.empty_like(q)
    qsa.qsa_sparse_attn_prefill(p, q, k, v, idx, cnt, out, q_pos0)
    return out


def _check_index_rows(b, rows, g_idx, g_cnt, q_idx_h, kbar_h, K, q_pos0=0, rope_dims=64):
    o_idx, o_cnt = oracle.index_rows(q_idx_h, kbar_h, rows, q_pos0, K=K, rope_dims=rope_dims)
    gi, gc = g_idx[b][rows], g_cnt[b][rows]
    differ = [u for u in range(len(rows)) if not np.array_equal(gi[u], o_idx[u])]
    scores = [None] * len(rows)
    if differ:
        sc = oracle.score_rows(q_idx_h, kbar_h, [rows[u] for u in differ], q_pos0,
                               rope_dims=rope_dims)
        for j, u in enumerate(differ):
            scores[u] = sc[j]
    sub = differ if differ else []
    assert np.array_equal(gc, o_cnt), "counts differ"
    near = check_sets(gi[sub], gc[sub], o_idx[sub], o_cnt[sub], [scores[u] for u in sub])
    return near, o_idx, o_cnt


# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_pool_parity(dtype):
    say("pool", dtype)
    d = inputs.small(B=2, n=1030, dtype=dtype, seed=21)
    p = _params()
    k_idx = to_dev(d["k_idx"])
    nb = 1030 // 4
    kbar = torch.zeros((2, nb + 3, 128), dtype=k_idx.dtype, device="cuda")
    qsa.qsa_pool_keys(p, k_idx, kbar, 0, 100)
    qsa.qsa_pool_keys(p, k_idx, kbar, 100, nb)
    torch.cuda.synchronize()
    got = to_host(kbar)
    for b in range(2):
        ref = oracle.pool(d["k_idx"][b])
        g, o = as_f64(got[b, :nb]), as_f64(ref)
        if dtype == "bf16":
            ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(o), 1e-30))) - 7)
            assert np.all(np.abs(g - o) <= ulp), np.max(np.abs(g - o) / ulp)
        else:
            scale = np.max(np.abs(o), axis=1, keepdims=True)
            assert np.all(np.abs(g - o) <= 4 * 2.0 ** -24 * scale)
        assert np.all(got[b, nb:] == 0), "rows beyond the range were written"


def _assert_pooled_close(got, ref, dtype):
    """The kernel normalises and rotates in float32, the oracle in float64
    with one final rounding.  Bound: one ulp of the stored value plus the
    float32 error of the normalise-and-rotate steps, a few 2^-24 of the
    key's largest element (a rotated pair that nearly cancels can sit many
    of its own bf16 ulps below that)."""
    floor = 8 * 2.0 ** -24 * np.max(np.abs(ref), axis=1, keepdims=True)
    if dtype == "bf16":
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        bad = np.abs(got - ref) > ulp + floor
    else:
        bad = np.abs(got - ref) > floor
    assert not np.any(bad), "pooled keys differ at %s" % (np.argwhere(bad)[:4].tolist(),)


@pytest.mark.parametrize("dtype,r", [("bf16", 4), ("fp32", 4), ("bf16", 16), ("bf16", 1)])
def test_pool_rmsnorm_parity(dtype, r):
    """Pooled keys RMS-normalised with a gain before the rotation, at
    positions up to 2^20 (blocks near the end of a 1M-token sequence are
    pooled through a range offset), then the selection of a few rows."""
    say("pool rmsnorm", dtype, r)
    n = 6000
    d = inputs.small(B=2, n=n, dtype=dtype, r=r, seed=23)
    p = qsa.params(r=r)
    nb = n // r
    rng = np.random.default_rng(5)
    gamma_h = rng.uniform(0.25, 2.0, 128).astype(np.float32)
    gamma = torch.from_numpy(gamma_h).cuda()
    k_idx = to_dev(d["k_idx"])
    kbar = torch.zeros((2, nb, 128), dtype=k_idx.dtype, device="cuda")
    qsa.qsa_pool_keys_rmsnorm(p, k_idx, gamma, 1e-6, kbar, 0, nb)
    torch.cuda.synchronize()
    got = to_host(kbar)
    for b in range(2):
        ref = as_f64(oracle.pool_rmsnorm(d["k_idx"][b], gamma_h.astype(np.float64), 1e-6, r=r))
        _assert_pooled_close(as_f64(got[b]), ref, dtype)
    # far positions: a sequence whose first 2^20 - 4096 tokens are absent
    # (their blocks are never pooled) -- only the last blocks are pooled
    big = (1 << 20) // r
    kb2 = torch.zeros((1, big, 128), dtype=k_idx.dtype, device="cuda")
    kfar = torch.zeros((1, big * r, 128), dtype=k_idx.dtype, device="cuda")
    kfar[0, big * r - n:] = k_idx[0]
    qsa.qsa_pool_keys_rmsnorm(p, kfar, gamma, 1e-6, kb2, big - nb, big)
    torch.cuda.synchronize()
    kfar_h = to_host(kfar[0])
    ref = as_f64(oracle.pool_rmsnorm(kfar_h, gamma_h.astype(np.float64), 1e-6, r=r, b0=big - 64,
                                     b1=big))
    _assert_pooled_close(as_f64(to_host(kb2[0, big - 64:])), ref, dtype)
    # the indexer consumes normalised keys like any others
    idx, cnt = _index_gpu(p, to_dev(d["q_idx"]), kbar)
    torch.cuda.synchronize()
    rows = np.array([0, 3, n // 2, n - 5, n - 1])
    if r == 4:
        _check_index_rows(0, rows, to_host(idx), to_host(cnt), d["q_idx"][0], got[0], 2048)


def test_prefill_4k_fp32_end_to_end_all_rows():
    """The 4K-token float32 workload (4 q heads / 1 kv head, 16 planted), every row."""
    say("4K fp32 end to end")
    d = inputs.make("prefill_4k_fp32", seed=100)
    p = _params()
    t = _dev_inputs(d)
    kbar = _pool_gpu(p, t["k_idx"], 1024)
    idx, cnt = _index_gpu(p, t["q_idx"], kbar)
    out = _attn_gpu(p, t["q"], t["k"], t["v"], idx, cnt)
    torch.cuda.synchronize()
    kbar_h, g_idx, g_cnt, g_out = to_host(kbar), to_host(idx), to_host(cnt), to_host(out)
    # pool stage
    ref = oracle.pool(d["k_idx"][0])
    np.testing.assert_allclose(kbar_h[0], ref, rtol=0, atol=4 * 2.0 ** -24 * np.abs(ref).max())
    rows = np.arange(4096)
    near, _, _ = _check_index_rows(0, rows, g_idx, g_cnt, d["q_idx"][0], kbar_h[0], 2048)
    say("4K fp32 near-tie differences:", near)
    for (_, i, blk, *_r) in _intact_plants(d["plants"]):
        assert blk in set(g_idx[0, i, :g_cnt[0, i]].tolist())
    o = oracle.attend_rows(d["q"][0], d["k"][0], d["v"][0], rows, g_idx[0], g_cnt[0])
    err = rel_err(g_out[0], o)
    say("4K fp32 attention rel err", err)
    assert err <= TOL["fp32"]


@pytest.mark.parametrize("n,dtype,K", [(1, "fp32", 16), (3, "bf16", 16), (5, "fp32", 8),
                                       (130, "bf16", 16), (1003, "fp32", 64),
                                       (1003, "bf16", 2048), (2500, "bf16", 100)])
def test_small_and_ragged(n, dtype, K):
    say("small/ragged n=%d %s K=%d" % (n, dtype, K))
    d = inputs.small(B=2, n=n, hq=8, hkv=2, dtype=dtype, K=K, seed=n)
    p = _params(K=K)
    t = _dev_inputs(d)
    nb = n // 4
    kbar = _pool_gpu(p, t["k_idx"], max(nb, 1)) if nb else torch.zeros(
        (2, 1, 128), dtype=t["k_idx"].dtype, device="cuda")
    idx, cnt = _index_gpu(p, t["q_idx"], kbar)
    out = _attn_gpu(p, t["q"], t["k"], t["v"], idx, cnt)
    torch.cuda.synchronize()
    kbar_h, g_idx, g_cnt, g_out = to_host(kbar), to_host(idx), to_host(cnt), to_host(out)
    rows = np.arange(n)
    for b in range(2):
        _check_index_rows(b, rows, g_idx, g_cnt, d["q_idx"][b], kbar_h[b], K)
        o = oracle.attend_rows(d["q"][b], d["k"][b], d["v"][b], rows, g_idx[b], g_cnt[b])
        assert rel_err(g_out[b], o) <= TOL[dtype]


@pytest.mark.parametrize("n", [600, 3000])
def test_large_K_is_dense(n):
    # n = 3000 gives rows with up to 751 slots, more than one LDS window of
    # slot ids in the bf16 attention kernel
    say("K >= n: dense causal, n=%d" % n)
    d = inputs.small(B=1, n=n, hq=16, hkv=2, dtype="bf16", K=4096, seed=5)
    p = _params(K=4096)
    t = _dev_inputs(d)
    kbar = _pool_gpu(p, t["k_idx"], n // 4)
    idx, cnt = _index_gpu(p, t["q_idx"], kbar)
    out = _attn_gpu(p, t["q"], t["k"], t["v"], idx, cnt)
    torch.cuda.synchronize()
    g_idx, g_cnt = to_host(idx)[0], to_host(cnt)[0]
    for i in range(n):
        nb = (i + 1) // 4
        assert g_cnt[i] == nb and np.array_equal(g_idx[i, :nb], np.arange(nb))
    rows = np.arange(n)
    o = oracle.attend_rows(d["q"][0], d["k"][0], d["v"][0], rows, g_idx, g_cnt)
    assert rel_err(to_host(out)[0], o) <= TOL["bf16"]


def test_bf16_medium_end_to_end_and_chunking():
    """n=16384, two sequences, 16 q / 2 kv heads, planted matches; chunked
    prefill (two halves through q_pos0) equals the full run bit for bit."""
    say("bf16 medium")
    n = 16384
    d = inputs.small(B=2, n=n, hq=16, hkv=2, dtype="bf16", planted=32, seed=33)
    p = _params()
    t = _dev_inputs(d)
    kbar = _pool_gpu(p, t["k_idx"], n // 4)
    idx, cnt = _index_gpu(p, t["q_idx"], kbar)
    out = _attn_gpu(p, t["q"], t["k"], t["v"], idx, cnt)
    # second half as its own chunk
    h = n // 2
    idx2, cnt2 = _index_gpu(p, t["q_idx"][:, h:].contiguous(), kbar, q_pos0=h)
    out2 = _attn_gpu(p, t["q"][:, h:].contiguous(), t["k"], t["v"], idx2, cnt2, q_pos0=h)
    # determinism
    idx3, cnt3 = _index_gpu(p, t["q_idx"], kbar)
    out3 = _attn_gpu(p, t["q"], t["k"], t["v"], idx3, cnt3)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx3) and torch.equal(cnt, cnt3) and torch.equal(out, out3)
    assert torch.equal(idx[:, h:], idx2) and torch.equal(cnt[:, h:], cnt2)
    assert torch.equal(out[:, h:], out2)
    kbar_h, g_idx, g_cnt, g_out = to_host(kbar), to_host(idx), to_host(cnt), to_host(out)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(2040, 2062),
                                     rng.integers(0, n, 256), np.arange(n - 8, n),
                                     [pl[1] for pl in d["plants"]]]))
    for b in range(2):
        near, _, _ = _check_index_rows(b, rows, g_idx, g_cnt, d["q_idx"][b], kbar_h[b], 2048)
        say("medium seq", b, "near-tie differences", near)
        o = oracle.attend_rows(d["q"][b], d["k"][b], d["v"][b], rows, g_idx[b][rows],
                               g_cnt[b][rows])
        err = rel_err(g_out[b][rows], o)
        say("medium seq", b, "attention rel err", err)
        assert err <= TOL["bf16"]
    for (b, i, blk, *_r) in _intact_plants(d["plants"]):
        assert blk in set(g_idx[b, i, :g_cnt[b, i]].tolist())


@pytest.mark.parametrize("n_q,dtype,K,lens", [
    (1, "bf16", 2048, (9000, 9001, 5003)), (4, "bf16", 2048, (9000, 9001, 5003)),
    (1, "fp32", 2048, (9000, 9001, 5003)), (6, "bf16", 2048, (9000, 9001, 5003)),
    # short sequences (at most 64 pooled blocks: one 16-block tile per scan
    # wave) with k_B = 16, so most rows still select
    (1, "bf16", 64, (256, 201, 90)), (4, "bf16", 64, (256, 201, 90)),
    # k_B = 4: selection and tail fit one split, which writes the output
    # without the merge
    (1, "bf16", 16, (256, 201, 90)), (4, "fp32", 16, (256, 201, 90))])
def test_decode_parity(n_q, dtype, K, lens):
    """Ragged sequence lengths; n_q new tokens per sequence (4 = the pages'
    next_n); decode equals the prefill rows at the same positions."""
    say("decode n_q=%d %s K=%d lens=%s" % (n_q, dtype, K, lens))
    lens = list(lens)
    n = max(lens)
    d = inputs.small(B=3, n=n, hq=16, hkv=2, dtype=dtype, seed=40 + n_q)
    p = _params(K=K)
    t = _dev_inputs(d)
    nbc = n // 4
    kbar = _pool_gpu(p, t["k_idx"], nbc)
    seq_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    qi = torch.stack([t["q_idx"][b, L - n_q:L] for b, L in enumerate(lens)]).contiguous()
    qq = torch.stack([t["q"][b, L - n_q:L] for b, L in enumerate(lens)]).contiguous()
    idx, cnt = _index_gpu(p, qi, kbar, seq_len=seq_len)
    out = torch.empty_like(qq)
    ws = qsa.workspace(qsa.qsa_sparse_attn_decode_workspace(p, 3, n_q, 16, 2))
    qsa.qsa_sparse_attn_decode(p, qq, t["k"], t["v"], seq_len, idx, cnt, out, ws)
    # the same rows through the prefill entry points
    pidx, pcnt = _index_gpu(p, t["q_idx"], kbar)
    torch.cuda.synchronize()
    kbar_h, g_idx, g_cnt, g_out = to_host(kbar), to_host(idx), to_host(cnt), to_host(out)
    p_idx, p_cnt = to_host(pidx), to_host(pcnt)
    for b, L in enumerate(lens):
        rows = np.arange(L - n_q, L)
        assert np.array_equal(g_idx[b], p_idx[b][rows]) and np.array_equal(g_cnt[b], p_cnt[b][rows])
        o_idx, o_cnt = oracle.index_rows(d["q_idx"][b], kbar_h[b], rows, K=K)
        sc = oracle.score_rows(d["q_idx"][b], kbar_h[b], rows)
        check_sets(g_idx[b], g_cnt[b], o_idx, o_cnt, sc)
        o = oracle.attend_rows(d["q"][b], d["k"][b], d["v"][b], rows, g_idx[b], g_cnt[b])
        assert rel_err(g_out[b], o) <= TOL[dtype]


def _random_config(i):
    """One seeded configuration: micro-block size, indexer heads, rotated
    dims, K (k_B within the many-row limit), batch, length, chunk offset,
    attention heads and dtype, drawn independently."""
    rng = np.random.default_rng(4000 + i)
    r = int(rng.choice([1, 2, 4, 8, 16]))
    K = int(rng.choice([64, 256, 1024, 2048, 4096]))
    while -(-K // r) > 3072:
        K //= 2
    hq, hkv = [(4, 1), (8, 2), (16, 2), (6, 3), (16, 16)][int(rng.integers(0, 5))]
    return dict(r=r, K=K, h=int(rng.choice([1, 2, 4])), R=int(rng.choice([0, 32, 64])),
                B=int(rng.integers(1, 3)), n=int(rng.integers(200, 14000)),
                chunk=bool(rng.integers(0, 2)), hq=hq, hkv=hkv,
                dtype="fp32" if rng.random() < 0.25 else "bf16", seed=4000 + i)


def _small_k(c, i):
    """The same configuration with K of a few blocks (at least r tokens): the
    selection is then shorter than one attention chunk and one decode
    split."""
    rng = np.random.default_rng(7000 + i)
    c = dict(c)
    c["K"] = max(c["r"], int(rng.choice([1, 8, 16, 32, 48, 100])))
    return c


@pytest.mark.parametrize("i", range(24))
def test_random_configurations(i):
    """A seeded sweep across the parameters the fixed cases vary one at a
    time ([hub] "Key ideas", QSA bullet: r, the indexer heads and the
    rotated share of the dims are the method's parameters; [glide] "QSA
    Ablations and Efficiency", Figure 5, sweeps r and the head count):
    pooling, selection and attention of one prefill pass, or of its second
    half run as a chunk at q_pos0, against the oracle on sampled rows."""
    _run_random_prefill(_random_config(i), i)


@pytest.mark.parametrize("i", range(8))
def test_random_small_k_configurations(i):
    """The seeded prefill sweep with K of a few blocks."""
    _run_random_prefill(_small_k(_random_config(i), i), i)


def _run_random_prefill(c, i):
    say("random configuration %d: %s" % (i, c))
    r, K, h, R, B, n = c["r"], c["K"], c["h"], c["R"], c["B"], c["n"]
    p = qsa.params(r=r, K=K, h_idx=h, rope_dims=R)
    kB = qsa.k_blocks(p)
    d = inputs.small(B=B, n=n, hq=c["hq"], hkv=c["hkv"], dtype=c["dtype"], r=r, K=K,
                     seed=c["seed"], planted=4 if n > (kB + 2) * r else 0)
    q_idx = np.ascontiguousarray(d["q_idx"][:, :, :h])
    t = _dev_inputs(d)
    nb = n // r
    kbar = torch.zeros((B, max(nb, 1), 128), dtype=t["k_idx"].dtype, device="cuda")
    if nb:
        qsa.qsa_pool_keys(p, t["k_idx"], kbar, 0, nb)
    n0 = (n // 3) if c["chunk"] else 0  # rows [n0, n) run as one chunk
    qi = to_dev(np.ascontiguousarray(q_idx[:, n0:]))
    qq = t["q"][:, n0:].contiguous()
    idx, cnt = _index_gpu(p, qi, kbar, q_pos0=n0)
    out = torch.empty_like(qq)
    qsa.qsa_sparse_attn_prefill(p, qq, t["k"], t["v"], idx, cnt, out, n0)
    torch.cuda.synchronize()
    kbar_h, g_idx, g_cnt, g_out = to_host(kbar), to_host(idx), to_host(cnt), to_host(out)
    m = n - n0
    rng = np.random.default_rng(c["seed"])
    first = kB * r + r - 1 - n0  # first chunk row that sees more than k_B blocks
    rows = np.concatenate([np.arange(4), np.arange(first - 3, first + 3),
                           rng.integers(0, m, 48), np.arange(m - 4, m)])
    rows = np.unique(rows[(rows >= 0) & (rows < m)]).astype(np.int64)
    for b in range(B):
        if nb:
            ref = as_f64(oracle.pool(d["k_idx"][b], r=r, rope_dims=R))
            _assert_pooled_close(as_f64(kbar_h[b, :nb]), ref, c["dtype"])
        qb = np.ascontiguousarray(q_idx[b, n0:])
        o_idx, o_cnt = oracle.index_rows(qb, kbar_h[b], rows, n0, r=r, K=K, rope_dims=R)
        sc = oracle.score_rows(qb, kbar_h[b], rows, n0, r=r, rope_dims=R)
        gi, gc = g_idx[b][rows], g_cnt[b][rows]
        check_sets(gi, gc, o_idx, o_cnt, sc)
        o = oracle.attend_rows(d["q"][b][n0:], d["k"][b], d["v"][b], rows, gi, gc, n0, r=r)
        err = rel_err(g_out[b][rows], o)
        assert err <= TOL[c["dtype"]], "sequence %d: attention error %g" % (b, err)


@pytest.mark.parametrize("i", range(12))
def test_random_decode_configurations(i):
    """The decode calls over a seeded sweep of batch, new tokens per
    sequence, ragged lengths (some at or below k_B blocks), micro-block
    size, indexer heads, rotated dims, K and attention heads ([glide] "QSA
    Ablations and Efficiency", Figure 6(d): decode with next_n new tokens,
    and index reuse across them): the selection of every new token, its
    attention, and the shared-selection attention, against the oracle."""
    _run_random_decode(_random_decode_config(i), i)


@pytest.mark.parametrize("i", range(8))
def test_random_small_k_decode(i):
    """The seeded decode sweep with K of a few blocks: selection and tail
    within one attention split for most draws."""
    _run_random_decode(_small_k(_random_decode_config(i), i), i)


def _random_decode_config(i):
    rng = np.random.default_rng(5000 + i)
    r = int(rng.choice([1, 2, 4, 8, 16]))
    K = int(rng.choice([64, 256, 2048, 4096]))
    while -(-K // r) > 4096:
        K //= 2
    h, R = int(rng.choice([1, 2, 4])), int(rng.choice([0, 32, 64]))
    hq, hkv = [(4, 1), (8, 2), (16, 2), (6, 3)][int(rng.integers(0, 4))]
    B, n_q = int(rng.integers(1, 7)), int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(n_q + r, 12000, B)]
    return dict(r=r, K=K, h=h, R=R, hq=hq, hkv=hkv, B=B, n_q=n_q, lens=lens)


def _run_random_decode(c, i):
    r, K, h, R, hq, hkv, B, n_q, lens = (c[k] for k in ("r", "K", "h", "R", "hq", "hkv", "B",
                                                         "n_q", "lens"))
    say("random decode %d: r=%d K=%d h=%d R=%d heads %d/%d B=%d n_q=%d lens=%s"
        % (i, r, K, h, R, hq, hkv, B, n_q, lens))
    n = max(lens)
    p = qsa.params(r=r, K=K, h_idx=h, rope_dims=R)
    d = inputs.small(B=B, n=n, hq=hq, hkv=hkv, dtype="bf16", r=r, K=K, seed=5000 + i)
    q_idx = np.ascontiguousarray(d["q_idx"][:, :, :h])
    t = _dev_inputs(d)
    t_qidx = to_dev(q_idx)
    kbar = torch.empty((B, n // r, 128), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_pool_keys(p, t["k_idx"], kbar, 0, n // r)
    seq_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    qi = torch.stack([t_qidx[b, L - n_q:L] for b, L in enumerate(lens)]).contiguous()
    qq = torch.stack([t["q"][b, L - n_q:L] for b, L in enumerate(lens)]).contiguous()
    idx, cnt = _index_gpu(p, qi, kbar, seq_len=seq_len)
    ws = qsa.workspace(qsa.qsa_sparse_attn_decode_workspace(p, B, n_q, hq, hkv))
    out = torch.empty_like(qq)
    qsa.qsa_sparse_attn_decode(p, qq, t["k"], t["v"], seq_len, idx, cnt, out, ws)
    first_len = torch.tensor([L - n_q + 1 for L in lens], dtype=torch.int32, device="cuda")
    sidx, scnt = _index_gpu(p, qi[:, :1].contiguous(), kbar, seq_len=first_len)
    sout = torch.empty_like(qq)
    qsa.qsa_sparse_attn_decode_shared(p, qq, t["k"], t["v"], seq_len, sidx, scnt, sout, ws)
    torch.cuda.synchronize()
    kbar_h, g_idx, g_cnt, g_out = to_host(kbar), to_host(idx), to_host(cnt), to_host(out)
    s_idx, s_cnt, s_out = to_host(sidx), to_host(scnt), to_host(sout)
    for b, L in enumerate(lens):
        pos = np.arange(L - n_q, L)
        o_idx, o_cnt = oracle.index_at(q_idx[b][pos], kbar_h[b], pos, r=r, K=K, rope_dims=R)
        sc = oracle.score_at(q_idx[b][pos], kbar_h[b], pos, r=r, rope_dims=R)
        check_sets(g_idx[b], g_cnt[b], o_idx, o_cnt, sc)
        o = oracle.attend_at(d["q"][b][pos], d["k"][b], d["v"][b], pos, g_idx[b], g_cnt[b], r=r)
        assert rel_err(g_out[b], o) <= TOL["bf16"], "sequence %d" % b
        f = L - n_q
        fo_idx, fo_cnt = oracle.index_at(q_idx[b][[f]], kbar_h[b], np.array([f]), r=r, K=K,
                                         rope_dims=R)
        fsc = oracle.score_at(q_idx[b][[f]], kbar_h[b], np.array([f]), r=r, rope_dims=R)
        check_sets(s_idx[b], s_cnt[b], fo_idx, fo_cnt, fsc)
        os_ = oracle.attend_shared(d["q"][b][pos], d["k"][b], d["v"][b], f, pos, s_idx[b, 0],
                                   s_cnt[b, 0], r=r)
        assert rel_err(s_out[b], os_) <= TOL["bf16"], "sequence %d (shared)" % b


def test_decode_multi_chunk_splits():
    """A batch large enough that each decode split covers several 32-key
    chunks (24 sequences x 2 KV heads: 4 chunks per split, 17 splits per
    row), with 4 new tokens per sequence, 4 query heads and ragged lengths,
    some below the k_B-block selection (empty splits), and a last split
    holding only the tail; every sequence's selection and output against
    the oracle."""
    say("decode multi-chunk splits")
    B, n_q = 24, 4
    rng = np.random.default_rng(61)
    lens = [int(x) for x in rng.integers(300, 6000, B)]
    lens[0], lens[1], lens[2] = 6000, 2055, 131
    n = max(lens)
    d = inputs.small(B=B, n=n, hq=4, hkv=2, dtype="bf16", seed=61)
    p = _params()
    t = _dev_inputs(d)
    kbar = _pool_gpu(p, t["k_idx"], n // 4)
    seq_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    qi = torch.stack([t["q_idx"][b, L - n_q:L] for b, L in enumerate(lens)]).contiguous()
    qq = torch.stack([t["q"][b, L - n_q:L] for b, L in enumerate(lens)]).contiguous()
    idx, cnt = _index_gpu(p, qi, kbar, seq_len=seq_len)
    out = torch.empty_like(qq)
    ws = qsa.workspace(qsa.qsa_sparse_attn_decode_workspace(p, B, n_q, 4, 2))
    qsa.qsa_sparse_attn_decode(p, qq, t["k"], t["v"], seq_len, idx, cnt, out, ws)
    torch.cuda.synchronize()
    kbar_h, g_idx, g_cnt, g_out = to_host(kbar), to_host(idx), to_host(cnt), to_host(out)
    for b, L in enumerate(lens):
        rows = np.arange(L - n_q, L)
        o_idx, o_cnt = oracle.index_rows(d["q_idx"][b], kbar_h[b], rows)
        sc = oracle.score_rows(d["q_idx"][b], kbar_h[b], rows)
        check_sets(g_idx[b], g_cnt[b], o_idx, o_cnt, sc)
        o = oracle.attend_rows(d["q"][b], d["k"][b], d["v"][b], rows, g_idx[b], g_cnt[b])
        assert rel_err(g_out[b], o) <= TOL["bf16"], "sequence %d (length %d)" % (b, L)


@pytest.mark.parametrize("n_q,lens", [(4, (9000, 9001, 5003)), (4, (20003, 256, 4098)),
                                      (2, (9002, 7000, 513))])
def test_decode_shared_selection(n_q, lens):
    """The pages' decode setting: n_q new tokens per sequence share the one
    selection made at the first new token (index reuse across speculative
    steps); each token attends to it plus every token from the first
    token's block boundary up to its own position."""
    say("decode shared selection n_q=%d lens=%s" % (n_q, lens))
    lens = list(lens)
    n = max(lens)
    d = inputs.small(B=3, n=n, hq=16, hkv=2, dtype="bf16", seed=50 + n_q)
    p = _params()
    t = _dev_inputs(d)
    kbar = _pool_gpu(p, t["k_idx"], n // 4)
    seq_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    first_len = torch.tensor([L - n_q + 1 for L in lens], dtype=torch.int32, device="cuda")
    qi = torch.stack([t["q_idx"][b, L - n_q:L - n_q + 1] for b, L in enumerate(lens)]).contiguous()
    qq = torch.stack([t["q"][b, L - n_q:L] for b, L in enumerate(lens)]).contiguous()
    idx, cnt = _index_gpu(p, qi, kbar, seq_len=first_len)
    ws = qsa.workspace(qsa.qsa_sparse_attn_decode_workspace(p, 3, n_q, 16, 2))
    out = torch.empty_like(qq)
    qsa.qsa_sparse_attn_decode_shared(p, qq, t["k"], t["v"], seq_len, idx, cnt, out, ws)
    # the first token alone through the ordinary decode call: same set, same bits
    out1 = torch.empty_like(qq[:, :1])
    ws1 = qsa.workspace(qsa.qsa_sparse_attn_decode_workspace(p, 3, 1, 16, 2))
    qsa.qsa_sparse_attn_decode(p, qq[:, :1].contiguous(), t["k"], t["v"], first_len, idx, cnt,
                               out1, ws1)
    torch.cuda.synchronize()
    assert torch.equal(out1[:, 0], out[:, 0])
    kbar_h, g_idx, g_cnt, g_out = to_host(kbar), to_host(idx), to_host(cnt), to_host(out)
    for b, L in enumerate(lens):
        f = L - n_q
        _check_index_at("shared seq %d" % b, d["q_idx"][b][[f]], kbar_h[b], np.array([f]),
                        g_idx[b], g_cnt[b])
        pos = np.arange(f, L)
        o = oracle.attend_shared(d["q"][b][pos], d["k"][b], d["v"][b], f, pos, g_idx[b, 0],
                                 g_cnt[b, 0])
        err = rel_err(g_out[b], o)
        say("shared seq", b, "attention rel err", err)
        assert err <= TOL["bf16"]


# ---- micro-block sizes other than 4 ([glide] "QSA Ablations and Efficiency",
# Figure 5(a) and Figure 6(a,b) sweep the micro-block size / compression) ----

def _transition_rows(n, kB, r, nrand=192, seed=3):
    first = kB * r + r - 1  # first row that sees more than k_B blocks
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.arange(8), np.arange(first - 6, first + 6), rng.integers(0, n, nrand),
                           np.arange(n - 8, n)])
    return np.unique(rows[(rows >= 0) & (rows < n)]).astype(np.int64)


@pytest.mark.parametrize("r,dtype,n", [(1, "bf16", 5003), (2, "bf16", 6001), (8, "bf16", 9001),
                                       (16, "bf16", 20003), (2, "fp32", 3001),
                                       (16, "fp32", 9000), (8, "bf16", 300)])
def test_block_size_variants_prefill(r, dtype, n):
    say("block size r=%d %s n=%d" % (r, dtype, n))
    K = 2048
    p = qsa.params(r=r, K=K)
    kB = qsa.k_blocks(p)
    d = inputs.small(B=2, n=n, hq=8, hkv=2, dtype=dtype, r=r, K=K, seed=200 + r,
                     planted=8 if n > K + r else 0)
    t = _dev_inputs(d)
    nb = n // r
    kbar = torch.zeros((2, max(nb, 1), 128), dtype=t["k_idx"].dtype, device="cuda")
    if nb:
        qsa.qsa_pool_keys(p, t["k_idx"], kbar, 0, nb)
    idx, cnt = _index_gpu(p, t["q_idx"], kbar)
    out = _attn_gpu(p, t["q"], t["k"], t["v"], idx, cnt)
    torch.cuda.synchronize()
    kbar_h, g_idx, g_cnt, g_out = to_host(kbar), to_host(idx), to_host(cnt), to_host(out)
    rows = _transition_rows(n, kB, r)
    for b in range(2):
        if nb:
            ref = as_f64(oracle.pool(d["k_idx"][b], r=r))
            _assert_pooled_close(as_f64(kbar_h[b, :nb]), ref, dtype)
        o_idx, o_cnt = oracle.index_rows(d["q_idx"][b], kbar_h[b], rows, r=r, K=K)
        gi, gc = g_idx[b][rows], g_cnt[b][rows]
        assert np.array_equal(gc, o_cnt), "counts differ"
        differ = [u for u in range(len(rows)) if not np.array_equal(gi[u], o_idx[u])]
        if differ:
            sc = oracle.score_rows(d["q_idx"][b], kbar_h[b], rows[differ], r=r)
            check_sets(gi[differ], gc[differ], o_idx[differ], o_cnt[differ], sc)
        o = oracle.attend_rows(d["q"][b], d["k"][b], d["v"][b], rows, gi, gc, r=r)
        err = rel_err(g_out[b][rows], o)
        say("r=%d seq %d: %d rows, %d differ, attention rel err %.2e" % (r, b, len(rows),
                                                                        len(differ), err))
        assert err <= TOL[dtype]


@pytest.mark.parametrize("rope_dims", [0, 32])
def test_rope_dims_variants_prefill(rope_dims):
    """Partial RoPE on fewer of the 128 indexer dims ([hub] "Key ideas",
    QSA bullet: the rotation covers only part of the dims): no rotated dim
    (the bf16 queries are exact, no low part is scored) and 32 (low parts on
    the first two 16-dim steps only), through the many-row indexer at a
    length whose later tiles take the sampled threshold; pooled keys and
    sampled selections against the oracle."""
    say("rope_dims=%d" % rope_dims)
    n, K = 20480, 2048
    p = _params(K=K, rope_dims=rope_dims)
    d = inputs.small(B=1, n=n, hq=4, hkv=1, dtype="bf16", planted=8, seed=300 + rope_dims)
    t = _dev_inputs(d)
    kbar = _pool_gpu(p, t["k_idx"], n // 4)
    idx, cnt = _index_gpu(p, t["q_idx"], kbar)
    torch.cuda.synchronize()
    kbar_h, g_idx, g_cnt = to_host(kbar), to_host(idx), to_host(cnt)
    ref = as_f64(oracle.pool(d["k_idx"][0], rope_dims=rope_dims))
    _assert_pooled_close(as_f64(kbar_h[0]), ref, "bf16")
    rows = _transition_rows(n, qsa.k_blocks(p), 4)
    near, _, _ = _check_index_rows(0, rows, g_idx, g_cnt, d["q_idx"][0], kbar_h[0], K,
                                   rope_dims=rope_dims)
    say("rope_dims=%d: %d rows, %d near-tie blocks" % (rope_dims, len(rows), near))


@pytest.mark.parametrize("r,n_q,lens", [(1, 1, (9000, 4097, 2050)), (8, 4, (9000, 9001, 5003)),
                                        (16, 1, (40000, 1999, 16391)),
                                        (2, 4, (9002, 7000, 1027))])
def test_block_size_variants_decode(r, n_q, lens):
    say("block size decode r=%d n_q=%d lens=%s" % (r, n_q, lens))
    lens = list(lens)
    n = max(lens)
    K = 2048
    p = qsa.params(r=r, K=K)
    d = inputs.small(B=3, n=n, hq=16, hkv=2, dtype="bf16", r=r, K=K, seed=300 + r)
    t = _dev_inputs(d)
    kbar = torch.empty((3, n // r, 128), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_pool_keys(p, t["k_idx"], kbar, 0, n // r)
    seq_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    qi = torch.stack([t["q_idx"][b, L - n_q:L] for b, L in enumerate(lens)]).contiguous()
    qq = torch.stack([t["q"][b, L - n_q:L] for b, L in enumerate(lens)]).contiguous()
    idx, cnt = _index_gpu(p, qi, kbar, seq_len=seq_len)
    ws = qsa.workspace(qsa.qsa_sparse_attn_decode_workspace(p, 3, n_q, 16, 2))
    out = torch.empty_like(qq)
    qsa.qsa_sparse_attn_decode(p, qq, t["k"], t["v"], seq_len, idx, cnt, out, ws)
    # the same tokens sharing the first token's selection
    first_len = torch.tensor([L - n_q + 1 for L in lens], dtype=torch.int32, device="cuda")
    sidx, scnt = _index_gpu(p, qi[:, :1].contiguous(), kbar, seq_len=first_len)
    sout = torch.empty_like(qq)
    qsa.qsa_sparse_attn_decode_shared(p, qq, t["k"], t["v"], seq_len, sidx, scnt, sout, ws)
    torch.cuda.synchronize()
    kbar_h, g_idx, g_cnt, g_out = to_host(kbar), to_host(idx), to_host(cnt), to_host(out)
    s_idx, s_cnt, s_out = to_host(sidx), to_host(scnt), to_host(sout)
    for b, L in enumerate(lens):
        pos = np.arange(L - n_q, L)
        o_idx, o_cnt = oracle.index_at(d["q_idx"][b][pos], kbar_h[b], pos, r=r, K=K)
        sc = oracle.score_at(d["q_idx"][b][pos], kbar_h[b], pos, r=r)
        check_sets(g_idx[b], g_cnt[b], o_idx, o_cnt, sc)
        o = oracle.attend_at(d["q"][b][pos], d["k"][b], d["v"][b], pos, g_idx[b], g_cnt[b], r=r)
        assert rel_err(g_out[b], o) <= TOL["bf16"]
        os_ = oracle.attend_shared(d["q"][b][pos], d["k"][b], d["v"][b], L - n_q, pos,
                                   s_idx[b, 0], s_cnt[b, 0], r=r)
        assert rel_err(s_out[b], os_) <= TOL["bf16"]


@pytest.mark.parametrize("h,dtype,n", [(1, "bf16", 9000), (2, "bf16", 9000), (2, "fp32", 3000),
                                        (1, "fp32", 3000)])
def test_indexer_head_counts_prefill(h, dtype, n):
    """Indexers with fewer query heads ([hub] "Key ideas": the ReLU-sum runs
    over the indexer's own heads): selections against the oracle with h heads."""
    say("indexer heads h=%d %s n=%d" % (h, dtype, n))
    K = 2048
    p = qsa.params(K=K, h_idx=h)
    d = inputs.small(B=2, n=n, hq=4, hkv=1, dtype=dtype, K=K, seed=500 + h, planted=0)
    q_idx = np.ascontiguousarray(d["q_idx"][:, :, :h])
    kbar = torch.empty((2, n // 4, 128), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                       device="cuda")
    qsa.qsa_pool_keys(p, to_dev(d["k_idx"]), kbar, 0, n // 4)
    idx, cnt = _index_gpu(p, to_dev(q_idx), kbar)
    torch.cuda.synchronize()
    kbar_h, g_idx, g_cnt = to_host(kbar), to_host(idx), to_host(cnt)
    rows = _transition_rows(n, qsa.k_blocks(p), 4)
    for b in range(2):
        o_idx, o_cnt = oracle.index_rows(q_idx[b], kbar_h[b], rows, K=K)
        gi, gc = g_idx[b][rows], g_cnt[b][rows]
        assert np.array_equal(gc, o_cnt), "counts differ"
        sc = oracle.score_rows(q_idx[b], kbar_h[b], rows)
        check_sets(gi, gc, o_idx, o_cnt, sc)


@pytest.mark.parametrize("h,n_q", [(1, 1), (2, 4)])
def test_indexer_head_counts_decode(h, n_q):
    say("indexer heads decode h=%d n_q=%d" % (h, n_q))
    lens = [9000, 4099, 30001]
    n = max(lens)
    K = 2048
    p = qsa.params(K=K, h_idx=h)
    d = inputs.small(B=3, n=n, hq=4, hkv=1, dtype="bf16", K=K, seed=510 + h, planted=0)
    kbar = torch.empty((3, n // 4, 128), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_pool_keys(p, to_dev(d["k_idx"]), kbar, 0, n // 4)
    q_idx = np.ascontiguousarray(np.stack([d["q_idx"][b, L - n_q:L, :h] for b, L in enumerate(lens)]))
    seq_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    idx, cnt = _index_gpu(p, to_dev(q_idx), kbar, seq_len=seq_len)
    torch.cuda.synchronize()
    kbar_h, g_idx, g_cnt = to_host(kbar), to_host(idx), to_host(cnt)
    for b, L in enumerate(lens):
        pos = np.arange(L - n_q, L)
        o_idx, o_cnt = oracle.index_at(q_idx[b], kbar_h[b], pos, K=K)
        sc = oracle.score_at(q_idx[b], kbar_h[b], pos)
        check_sets(g_idx[b], g_cnt[b], o_idx, o_cnt, sc)


# ---- dense causal GQA attention (QSA with every block selected; the
# pages' dense baseline, [glide] "QSA Ablations and Efficiency", Figure 6) ----

def _dense_ref(q_rows, k, v, pos):
    """The oracle's attention with every complete block selected: T = 0..pos."""
    pos = np.asarray(pos, dtype=np.int64)
    nbmax = int((pos.max() + 1) // 4)
    idx = np.full((pos.size, max(nbmax, 1)), -1, dtype=np.int32)
    cnt = ((pos + 1) // 4).astype(np.int32)
    for u, c in enumerate(cnt):
        idx[u, :c] = np.arange(c)
    return oracle.attend_at(q_rows, k, v, pos, idx, cnt)


@pytest.mark.parametrize("n,q_pos0,n_q,hq,hkv", [(3000, 0, 3000, 16, 2), (20000, 12000, 5001, 16, 2),
                                                 (1003, 0, 1003, 8, 2), (4500, 100, 4400, 16, 1),
                                                 (700, 650, 50, 2, 2)])
def test_dense_prefill(n, q_pos0, n_q, hq, hkv):
    say("dense prefill n=%d q_pos0=%d n_q=%d hq=%d hkv=%d" % (n, q_pos0, n_q, hq, hkv))
    d = inputs.small(B=2, n=n, hq=hq, hkv=hkv, dtype="bf16", seed=400 + n_q)
    t = _dev_inputs(d)
    q = t["q"][:, q_pos0:q_pos0 + n_q].contiguous()
    out = torch.empty_like(q)
    qsa.qsa_dense_attn_prefill(q, t["k"], t["v"], out, q_pos0)
    torch.cuda.synchronize()
    g = to_host(out)
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([np.arange(min(8, n_q)), rng.integers(0, n_q, 96),
                                     np.arange(max(0, n_q - 8), n_q)]))
    for b in range(2):
        o = _dense_ref(d["q"][b][q_pos0 + rows], d["k"][b], d["v"][b], q_pos0 + rows)
        err = rel_err(g[b][rows], o)
        say("dense prefill seq %d: %d rows, rel err %.2e" % (b, rows.size, err))
        assert err <= TOL["bf16"]


@pytest.mark.parametrize("n_q,lens,hq,hkv", [(1, (9000, 4097, 100), 16, 2),
                                             (4, (9000, 9001, 5003), 16, 2),
                                             (4, (300, 8191, 4096), 8, 2),
                                             (6, (5000, 2000, 6001), 16, 2),
                                             # every length within one split
                                             (2, (3113, 1653, 187), 16, 16),
                                             (1, (4096, 1000, 5), 8, 2)])
def test_dense_decode(n_q, lens, hq, hkv):
    say("dense decode n_q=%d lens=%s" % (n_q, lens))
    lens = list(lens)
    n = max(lens)
    d = inputs.small(B=3, n=n, hq=hq, hkv=hkv, dtype="bf16", seed=500 + n_q)
    t = _dev_inputs(d)
    seq_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    qq = torch.stack([t["q"][b, L - n_q:L] for b, L in enumerate(lens)]).contiguous()
    out = torch.empty_like(qq)
    ws = qsa.workspace(qsa.qsa_dense_attn_decode_workspace(3, n_q, hkv, n))
    qsa.qsa_dense_attn_decode(qq, t["k"], t["v"], seq_len, out, ws)
    torch.cuda.synchronize()
    g = to_host(out)
    for b, L in enumerate(lens):
        pos = np.arange(L - n_q, L)
        o = _dense_ref(d["q"][b][pos], d["k"][b], d["v"][b], pos)
        assert rel_err(g[b], o) <= TOL["bf16"]


def test_decode_step_graph_replays():
    """A decode step (pool the newest block, index, attend) captured in a HIP
    graph: every replay, with eager work and synchronizations between the
    replays, equals the eager step bit for bit."""
    say("decode step graph replays")
    lens = [20000, 17001, 9003]
    n = max(lens)
    d = inputs.small(B=3, n=n, hq=16, hkv=2, dtype="bf16", seed=77)
    p = _params()
    t = _dev_inputs(d)
    nbc = n // 4
    kB = qsa.k_blocks(p)
    kbar = _pool_gpu(p, t["k_idx"], nbc)
    seq_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    qi = torch.stack([t["q_idx"][b, L - 1:L] for b, L in enumerate(lens)]).contiguous()
    qq = torch.stack([t["q"][b, L - 1:L] for b, L in enumerate(lens)]).contiguous()
    idx = torch.empty((3, 1, kB), dtype=torch.int32, device="cuda")
    cnt = torch.empty((3, 1), dtype=torch.int32, device="cuda")
    out = torch.empty_like(qq)
    ws_i = qsa.workspace(qsa.qsa_index_topk_workspace(p, qsa.QSA_BF16, 3, 1, nbc, True))
    ws_a = qsa.workspace(qsa.qsa_sparse_attn_decode_workspace(p, 3, 1, 16, 2))

    def step():
        qsa.qsa_pool_keys(p, t["k_idx"], kbar, nbc - 1, nbc)
        qsa.qsa_index_topk(p, qi, kbar, idx, cnt, ws_i, 0, seq_len)
        qsa.qsa_sparse_attn_decode(p, qq, t["k"], t["v"], seq_len, idx, cnt, out, ws_a)

    step()
    torch.cuda.synchronize()
    _assert_ids_valid(p, idx, cnt, 0, seq_len)
    ref = [x.clone() for x in (idx, cnt, out)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the capture stream as torch asks
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        idx.fill_(-5)
        cnt.fill_(-5)
        out.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, r in zip(("idx", "cnt", "out"), (idx, cnt, out), ref):
            assert torch.equal(x, r), "replay %d differs in %s" % (rep, name)


def test_decode_exact_route_on_ties():
    """Decode rows whose scores tie in bulk: sequence 0 has a zero indexer
    query (every score is +0), sequence 1 a pooled cache whose keys are all
    equal and unrotated (one score everywhere).  Far more blocks than fit the
    candidate list share the k_B-th score, so the selection takes the exact
    route; ties go to the smaller block id.  Sequence 2 is ordinary."""
    say("decode exact route on ties")
    L = 30000  # 7500 blocks
    d = inputs.small(B=3, n=L, hq=16, hkv=2, dtype="bf16", seed=91)
    d["q_idx"][0, L - 1] = 0
    # every key = head 0's query on the unrotated dims, zero on the rotated
    # ones: all pooled keys are equal and score the same positive value
    d["k_idx"][1, :, :64] = 0
    d["k_idx"][1, :, 64:] = d["q_idx"][1, L - 1, 0, 64:]
    p = _params()
    t = _dev_inputs(d)
    nb = L // 4
    kbar = _pool_gpu(p, t["k_idx"], nb)
    seq_len = torch.full((3,), L, dtype=torch.int32, device="cuda")
    qi = t["q_idx"][:, L - 1:L].contiguous()
    idx, cnt = _index_gpu(p, qi, kbar, seq_len=seq_len)
    torch.cuda.synchronize()
    kbar_h, g_idx, g_cnt = to_host(kbar), to_host(idx), to_host(cnt)
    for b in range(3):
        o_idx, o_cnt = oracle.index_rows(d["q_idx"][b, L - 1:L], kbar_h[b], [0], L - 1)
        if b < 2:
            assert np.array_equal(o_idx[0], np.arange(512))
            assert np.array_equal(g_idx[b], o_idx) and np.array_equal(g_cnt[b], o_cnt)
        else:
            sc = oracle.score_rows(d["q_idx"][b, L - 1:L], kbar_h[b], [0], L - 1)
            check_sets(g_idx[b], g_cnt[b], o_idx, o_cnt, sc)


# ---- full-size configurations, sampled rows --------------------------------

def _sample_rows(n, plants, nrand, seed=0):
    """Rows 0-7, the dense -> sparse transition 2040-2061, nrand uniform rows,
    the last 8 rows and the query row of every planted match."""
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(8), np.arange(2040, 2062),
                                     rng.integers(0, n, nrand), np.arange(n - 8, n),
                                     [pl[1] for pl in plants]])).astype(np.int64)


def _sample_blocks(nb, seed=1):
    """Pooled-key blocks checked at full size: the first and last 64, six
    more runs of 64 spread over the sequence, 256 uniform singles."""
    rng = np.random.default_rng(seed)
    runs = [0, nb - 64] + [int(x) for x in rng.integers(0, nb - 64, 6)]
    blocks = np.concatenate([np.arange(b0, b0 + 64) for b0 in runs] +
                            [rng.integers(0, nb, 256)])
    return np.unique(blocks).astype(np.int64)


def _check_pool_sampled(tag, kbar_h, k_idx_h, nb):
    """GPU pooled keys of sampled blocks (positions up to the sequence end)
    within one bf16 ulp of the oracle's."""
    blocks = _sample_blocks(nb)
    # contiguous runs go to the oracle as ranges [b0, b1)
    splits = np.nonzero(np.diff(blocks) != 1)[0] + 1
    worst = 0.0
    for run in np.split(blocks, splits):
        b0, b1 = int(run[0]), int(run[-1]) + 1
        ref = as_f64(oracle.pool(k_idx_h, b0=b0, b1=b1))
        got = as_f64(kbar_h[b0:b1])
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        ratio = np.abs(got - ref) / ulp
        worst = max(worst, float(ratio.max()))
        assert np.all(ratio <= 1.0), "%s: pooled keys of blocks [%d, %d) differ by %.2f ulp" % (
            tag, b0, b1, ratio.max())
    say(tag, "pooled keys: %d blocks up to block %d, max %.2f bf16 ulp" % (
        blocks.size, int(blocks.max()), worst))


def _check_index_at(tag, q_rows_h, kbar_h, pos, g_idx, g_cnt):
    """Selections of rows given with their positions against the oracle, with
    the near-tie rule; returns the oracle selection."""
    o_idx, o_cnt = oracle.index_at(q_rows_h, kbar_h, pos)
    assert np.array_equal(g_cnt, o_cnt), "%s: counts differ" % tag
    differ = np.array([u for u in range(len(pos)) if not np.array_equal(g_idx[u], o_idx[u])],
                      dtype=np.int64)
    near = 0
    if differ.size:
        sc = oracle.score_at(q_rows_h[differ], kbar_h, pos[differ])
        near = check_sets(g_idx[differ], g_cnt[differ], o_idx[differ], o_cnt[differ], sc)
    say(tag, "%d rows, %d differ, %d near-tie blocks" % (len(pos), differ.size, near))
    return o_idx, o_cnt


# the 1M-token prefill (8192 query tiles) runs the indexer in four groups of
# tiles that reuse one workspace; 64K and 256K fit one group
@pytest.mark.parametrize("cfg,nrand", [("prefill_64k", 1024), ("prefill_256k", 1024),
                                       ("prefill_1m", 256)])
def test_full_size_prefill_sampled(cfg, nrand):
    say("full-size prefill", cfg)
    d = inputs.make(cfg, seed={"prefill_64k": 101, "prefill_256k": 102, "prefill_1m": 104}[cfg],
                    backend="torch")
    p = _params()
    n = d["n"]
    kbar, idx, cnt, out = qsa.prefill(p, d["k_idx"], d["q_idx"], d["q"], d["k"], d["v"])
    torch.cuda.synchronize()
    kbar_h = to_host(kbar[0])
    _check_pool_sampled(cfg, kbar_h, to_host(d["k_idx"][0]), n // 4)
    rows = _sample_rows(n, d["plants"], nrand)
    rt = torch.from_numpy(rows).cuda()
    qi_h = to_host(d["q_idx"][0][rt])
    g_idx, g_cnt = to_host(idx[0][rt]), to_host(cnt[0][rt])
    _check_index_at(cfg, qi_h, kbar_h, rows, g_idx, g_cnt)
    intact = _intact_plants(d["plants"])
    say(cfg, "%d of %d planted matches intact" % (len(intact), len(d["plants"])))
    for (_, i, blk, *_r) in intact:
        u = int(np.searchsorted(rows, i))
        assert blk in set(g_idx[u, :g_cnt[u]].tolist()), "planted block %d of row %d" % (blk, i)
    k_h, v_h = to_host(d["k"][0]), to_host(d["v"][0])
    o = oracle.attend_at(to_host(d["q"][0][rt]), k_h, v_h, rows, g_idx, g_cnt)
    err = rel_err(to_host(out[0][rt]), o)
    say(cfg, "attention rel err over %d rows" % rows.size, err)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("cfg", ["decode_64x256k", "decode_8x1m"])
def test_full_size_decode_sampled(cfg):
    say("full-size decode", cfg)
    d = inputs.make(cfg, seed={"decode_64x256k": 103, "decode_8x1m": 104}[cfg], backend="torch")
    p = _params()
    B, L = d["B"], d["n"]
    nb = L // 4
    # 64 x 256K: 17 of the 64 sequences (every fourth, and the last); 8 x 1M: all 8
    check = list(range(0, B, 4)) + [B - 1] if B > 8 else list(range(B))
    kbar = _pool_gpu(p, d["k_idx"], nb)
    seq_len = torch.full((B,), L, dtype=torch.int32, device="cuda")
    idx, cnt = _index_gpu(p, d["q_idx"], kbar, seq_len=seq_len)
    out = torch.empty_like(d["q"])
    ws = qsa.workspace(qsa.qsa_sparse_attn_decode_workspace(p, B, 1, 16, 2))
    qsa.qsa_sparse_attn_decode(p, d["q"], d["k"], d["v"], seq_len, idx, cnt, out, ws)
    torch.cuda.synchronize()
    for b in check:
        kbar_h = to_host(kbar[b])
        if b in (check[0], check[-1]):
            _check_pool_sampled("%s seq %d" % (cfg, b), kbar_h, to_host(d["k_idx"][b]), nb)
        qi = to_host(d["q_idx"][b, 0])
        g_idx, g_cnt = to_host(idx[b]), to_host(cnt[b])
        _check_index_at("%s seq %d" % (cfg, b), qi[None], kbar_h, np.array([L - 1]), g_idx,
                        g_cnt)
        # planted blocks outscore every noise block; when a sequence has more
        # planted blocks than k_B, the selection holds k_B of them
        planted = {blk for (bb, i, blk, *_r) in d["plants"] if bb == b}
        sel = set(g_idx[0, :g_cnt[0]].tolist())
        assert len(sel & planted) == min(len(planted), int(g_cnt[0]))
        o = oracle.attend_at(to_host(d["q"][b]), to_host(d["k"][b]), to_host(d["v"][b]),
                             np.array([L - 1]), g_idx, g_cnt)
        err = rel_err(to_host(out[b]), o)
        say(cfg, "seq", b, "attention rel err", err)
        assert err <= TOL["bf16"]


def test_threshold_fallback_rescan():
    """White-box: a tile whose rows see more than 3072 blocks first scores a
    strided sample of m = ceil(16 nbmin / k_B) blocks, u * nbmin // m, where
    nbmin is what its first row sees; lane u % 32 keeps its four largest
    sample scores per row, and the row's threshold is the
    ceil(E + 5 sqrt(E) + 2)-th largest kept value (E = m k_B / visible,
    about 16, so the 38th).  Planting high scores on the first 100 sampled
    blocks for the last row puts three or four planted scores in every
    lane, all of them kept, so the threshold lands among the planted scores
    and fewer than k_B blocks pass it: the tile is flagged and recomputed by
    the exact kernel, and the selection must still equal the oracle's."""
    say("threshold fallback")
    n = 20480
    d = inputs.small(B=1, n=n, hq=4, hkv=1, dtype="bf16", seed=77)
    i = n - 1
    row0 = (n - 1) // 128 * 128
    nbmin = (row0 + 1) // 4
    m = min(max(-(-16 * nbmin // 512), 64), nbmin)
    sample = [u * nbmin // m for u in range(m)]
    planted = sample[:100]  # distinct high scores; three or four in every lane
    qf = inputs.bf16_bits_to_f32(d["q_idx"][0, i, 0])
    kf = inputs.bf16_bits_to_f32(d["k_idx"][0])
    for u, blk in enumerate(planted):
        kf[4 * blk:4 * blk + 4, :64] = 0.0
        kf[4 * blk:4 * blk + 4, 64:] = (3.0 + 0.01 * u) * qf[64:]
    d["k_idx"][0] = inputs.f32_to_bf16_bits(kf)
    p = _params()
    t = _dev_inputs(d)
    kbar = _pool_gpu(p, t["k_idx"], n // 4)
    kB = qsa.k_blocks(p)
    idx = torch.empty((1, n, kB), dtype=torch.int32, device="cuda")
    cnt = torch.empty((1, n), dtype=torch.int32, device="cuda")
    ws = qsa.workspace(qsa.qsa_index_topk_workspace(p, qsa.QSA_BF16, 1, n, n // 4, False))
    qsa.qsa_index_topk(p, t["q_idx"], kbar, idx, cnt, ws)
    torch.cuda.synchronize()
    _assert_ids_valid(p, idx, cnt, 0, None)
    # the workspace ends with one flag per tile of the group (256-byte
    # aligned); the tiles run longest first, so the last tile is flag 0
    ntiles = n // 128
    flags_off = ws.numel() - (ntiles * 4 + 255) // 256 * 256
    flags = to_host(ws[flags_off:flags_off + ntiles * 4]).view(np.uint32)
    assert flags[0] != 0, "the planted tile was not flagged for the exact kernel"
    kbar_h, g_idx, g_cnt = to_host(kbar), to_host(idx), to_host(cnt)
    rows = np.arange(row0, n)
    near, o_idx, _ = _check_index_rows(0, rows, g_idx, g_cnt, d["q_idx"][0], kbar_h[0], 2048)
    # the exact kernel recovers all planted blocks plus the best noise blocks
    assert set(planted) <= set(g_idx[0, i, :g_cnt[0, i]].tolist())
    assert g_cnt[0, i] == 512
