"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test ties one oracle function to something other than itself: a worked
example of the pages (tests/golden), a closed form, a library routine on a
special case, brute force on tiny inputs, or an algebraic identity.  Each is
chosen so that a plausible mistake (a dropped head, a wrong sign, a wrong
pairing or index, an off-by-one in the causal rule) fails.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from trainable_sparse_attention_amd import inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(x):
    return inputs.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _f(x):
    return inputs.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x


# --------------------------------------------------------------------------
# Pooling ([hub] keys average-pooled into blocks of r; [glide] block 0 gets
# (k0 + k1) / 2)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_pool_without_rope_is_block_mean(dtype):
    rng = np.random.default_rng(1)
    k = rng.standard_normal((64, 128)).astype(np.float32)
    kin = _bf16(k) if dtype == "bf16" else k
    got = _f(oracle.pool(kin, r=4, rope_dims=0))
    mean = _f(kin).astype(np.float64).reshape(16, 4, 128).mean(axis=1)
    if dtype == "fp32":
        # float64 -> float32 cast is round-to-nearest-even: the closed form
        np.testing.assert_array_equal(got, mean.astype(np.float32))
    else:
        # a bf16 value within half a bf16 ulp of the exact mean
        assert np.array_equal(_bf16(got), inputs.f32_to_bf16_bits(got))
        ulp = 2.0 ** (np.floor(np.log2(np.abs(mean))) - 7)
        assert np.all(np.abs(got - mean) <= 0.5 * ulp + 1e-300)


def test_pool_toy_pairs_of_two():
    g = json.load(open(os.path.join(GOLD, "toy_qsa_walkthrough.json")))
    k = np.array(g["k_idx"], dtype=np.float32)
    got = oracle.pool(k, r=2, rope_dims=0)
    np.testing.assert_array_equal(got, np.array(g["expected"]["pooled"], dtype=np.float32))


def test_pool_partial_rope_leaves_upper_dims_and_norms():
    rng = np.random.default_rng(2)
    k = rng.standard_normal((4096, 128)).astype(np.float32)
    got = oracle.pool(k, r=4, rope_dims=64).astype(np.float64)
    mean = k.astype(np.float64).reshape(1024, 4, 128).mean(axis=1)
    # dims 64..127 are not rotated: the rounded block mean
    np.testing.assert_array_equal(got[:, 64:], mean[:, 64:].astype(np.float32))
    # each rotated pair (j, j+32) keeps its length
    n_got = got[:, :32] ** 2 + got[:, 32:64] ** 2
    n_ref = mean[:, :32] ** 2 + mean[:, 32:64] ** 2
    np.testing.assert_allclose(n_got, n_ref, rtol=1e-6, atol=1e-12)
    # block 0 sits at position r-1 = 3, so it IS rotated: pair 0 turns by 3 rad
    a, b = mean[0, 0], mean[0, 32]
    np.testing.assert_allclose(got[0, 0], a * math.cos(3) - b * math.sin(3), rtol=1e-6)


# --------------------------------------------------------------------------
# RoPE ([hub] partial RoPE on 64 of 128 dims)
# --------------------------------------------------------------------------

# RMS-normalised pooling ([glide] "Qwen Sparse Attention" toy: average-pool,
# then RMSNorm)

def test_pool_rmsnorm_closed_form_without_rope():
    """rope_dims = 0, eps = 0: every pooled key is the block mean divided by
    its root mean square, times the gain (float32 storage: one rounding)."""
    rng = np.random.default_rng(21)
    k = rng.standard_normal((64, 128)).astype(np.float32)
    gamma = rng.uniform(0.5, 2.0, 128)
    got = oracle.pool_rmsnorm(k, gamma, eps=0.0, r=4, rope_dims=0)
    mean = k.astype(np.float64).reshape(16, 4, 128).mean(axis=1)
    rms = np.sqrt((mean ** 2).mean(axis=1, keepdims=True))
    np.testing.assert_array_equal(got, (mean / rms * gamma).astype(np.float32))


def test_pool_rmsnorm_invariances():
    """Scaling every key by c > 0 leaves the normalised keys unchanged
    (eps = 0); with unit gain every pooled key has RMS 1 up to one float32
    rounding (the rotation keeps the sum of squares); eps > 0 only shrinks
    it; the unrotated dims equal those of the unrotated result."""
    rng = np.random.default_rng(22)
    k = (rng.standard_normal((64, 128)) * 0.1).astype(np.float32)
    ones = np.ones(128)
    a = oracle.pool_rmsnorm(k, ones, eps=0.0)
    b = oracle.pool_rmsnorm((k * np.float32(8.0)).astype(np.float32), ones, eps=0.0)
    np.testing.assert_allclose(a, b, rtol=3e-7, atol=0)
    rms = np.sqrt((a.astype(np.float64) ** 2).mean(axis=1))
    np.testing.assert_allclose(rms, 1.0, rtol=2e-7)
    c = oracle.pool_rmsnorm(k, ones, eps=1e-2)
    assert np.all(np.sqrt((c.astype(np.float64) ** 2).mean(axis=1)) < rms)
    d0 = oracle.pool_rmsnorm(k, ones, eps=0.0, rope_dims=0)
    np.testing.assert_array_equal(a[:, 64:], d0[:, 64:])


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(3).standard_normal((5, 128))
    np.testing.assert_array_equal(oracle.rope_rows(x, [0] * 5), x)


def test_rope_quarter_turn_closed_form():
    # theta chosen so that pair j=1 turns by exactly pi/2 per position:
    # theta^(-2/64) = pi/2  <=>  theta = (pi/2)^(-32)
    theta = (math.pi / 2) ** (-32)
    x = np.zeros((1, 128))
    x[0, 1], x[0, 33] = 3.0, 5.0
    y = oracle.rope_rows(x, [1], theta=theta)
    np.testing.assert_allclose([y[0, 1], y[0, 33]], [-5.0, 3.0], atol=1e-12)
    # pair j=0 has frequency 1: one radian per position
    x = np.zeros((1, 128))
    x[0, 0] = 1.0
    y = oracle.rope_rows(x, [2], theta=theta)
    np.testing.assert_allclose([y[0, 0], y[0, 32]], [math.cos(2), math.sin(2)], atol=1e-14)
    # upper half untouched, other dims inside the rotated range untouched
    assert np.count_nonzero(y[0, 64:]) == 0


def test_rope_composition_and_relative_position():
    rng = np.random.default_rng(4)
    a = rng.standard_normal((1, 128))
    b = rng.standard_normal((1, 128))
    # rotating by p then by q equals rotating by p + q
    np.testing.assert_allclose(oracle.rope_rows(oracle.rope_rows(a, [37]), [1000]),
                               oracle.rope_rows(a, [1037]), atol=1e-12)
    # <R_m a, R_n b> depends on m - n only
    d1 = float((oracle.rope_rows(a, [5000]) @ oracle.rope_rows(b, [4000]).T)[0, 0])
    d2 = float((oracle.rope_rows(a, [123456]) @ oracle.rope_rows(b, [122456]).T)[0, 0])
    np.testing.assert_allclose(d1, d2, rtol=1e-10)
    np.testing.assert_allclose(np.linalg.norm(oracle.rope_rows(a, [99999])), np.linalg.norm(a),
                               rtol=1e-14)


# --------------------------------------------------------------------------
# Block scores ([hub] I_ib = sum_h ReLU(<q_i^h, kbar_b>); [glide] block-causal)
# --------------------------------------------------------------------------

def _brute_scores(q_row, kbar, pos, r, rope_dims=64, theta=10000.0):
    """Matrix-product route: rotate (pinned above), one matmul per head,
    ReLU, sum; visibility from the block end position."""
    qr = oracle.rope_rows(q_row.astype(np.float64), [pos] * q_row.shape[0], rope_dims, theta)
    ends = (np.arange(kbar.shape[0]) + 1) * r - 1
    vis = kbar[ends <= pos].astype(np.float64)
    return np.maximum(qr @ vis.T, 0.0).sum(axis=0)


def test_scores_toy():
    g = json.load(open(os.path.join(GOLD, "toy_qsa_walkthrough.json")))
    kbar = oracle.pool(np.array(g["k_idx"], dtype=np.float32), r=2, rope_dims=0)
    for t in ("4", "5", "7"):
        q = np.array(g["q_idx"][t], dtype=np.float32)
        s = oracle.scores(q, kbar, int(t), r=2, rope_dims=0)
        assert s.shape[0] == g["expected"][t]["visible"]
        np.testing.assert_array_equal(s, g["expected"][t]["scores"])


@pytest.mark.parametrize("r", [1, 2, 4])
def test_scores_brute_force(r):
    rng = np.random.default_rng(10 + r)
    n = 48
    k = rng.standard_normal((n, 128)).astype(np.float32)
    kbar = oracle.pool(k, r=r)
    q = rng.standard_normal((n, 4, 128)).astype(np.float32)
    for pos in range(n):
        s = oracle.scores(q[pos], kbar, pos, r=r)
        assert s.shape[0] == (pos + 1) // r
        np.testing.assert_allclose(s, _brute_scores(q[pos], kbar, pos, r), rtol=1e-12, atol=1e-12)


def test_scores_relu_identity_heads_and_scaling():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((256, 128)).astype(np.float32)
    kbar = oracle.pool(k, r=4)
    q = rng.standard_normal((4, 128)).astype(np.float32)
    pos = 255
    s = oracle.scores(q, kbar, pos)
    # ReLU(x) - ReLU(-x) = x: s(q) - s(-q) is the plain sum of dot products
    lin = (oracle.rope_rows(q.astype(np.float64), [pos] * 4) @ kbar.astype(np.float64).T).sum(0)
    np.testing.assert_allclose(s - oracle.scores(-q, kbar, pos), lin, rtol=1e-10, atol=1e-12)
    # the 4-head score is the sum of single-head scores (no head dropped)
    per_head = sum(oracle.scores(q[h:h + 1], kbar, pos) for h in range(4))
    np.testing.assert_allclose(s, per_head, rtol=1e-12, atol=1e-14)
    # positively homogeneous, non-negative
    np.testing.assert_allclose(oracle.scores(2 * q, kbar, pos), 2 * s, rtol=1e-12)
    assert np.all(s >= 0)


# --------------------------------------------------------------------------
# Selection ([hub] top-k_B = ceil(K/r) blocks; ties: smaller block id first)
# --------------------------------------------------------------------------

def test_select_brute_force_subsets():
    rng = np.random.default_rng(6)
    for trial in range(200):
        nb = int(rng.integers(1, 12))
        kB = int(rng.integers(1, 5))
        s = rng.random(nb)
        idx, c = oracle.select(s, kB)
        assert c == min(kB, nb)
        best = max(itertools.combinations(range(nb), c), key=lambda S: sum(s[list(S)]))
        assert list(idx[:c]) == sorted(best)
        assert np.all(idx[c:] == -1)


def test_select_ties_prefer_smaller_ids_and_zero_scores_count():
    idx, c = oracle.select(np.zeros(10), 4)
    assert c == 4 and list(idx) == [0, 1, 2, 3]
    s = np.array([0.0, 2.0, 1.0, 2.0, 1.0, 0.0, 1.0])
    idx, c = oracle.select(s, 4)
    assert list(idx) == [1, 2, 3, 4]
    idx, c = oracle.select(np.ones(3), 8)
    assert c == 3 and list(idx) == [0, 1, 2, -1, -1, -1, -1, -1]


def test_toy_selection_and_token_sets():
    g = json.load(open(os.path.join(GOLD, "toy_qsa_walkthrough.json")))
    kbar = oracle.pool(np.array(g["k_idx"], dtype=np.float32), r=2, rope_dims=0)
    q_idx = np.zeros((8, 2, 4), dtype=np.float32)
    for t, v in g["q_idx"].items():
        q_idx[int(t)] = v
    rows = [4, 5, 7]
    idx, cnt = oracle.index_rows(q_idx, kbar, rows, r=2, K=g["K"], rope_dims=0)
    for u, t in enumerate(rows):
        e = g["expected"][str(t)]
        assert list(idx[u, :cnt[u]]) == e["selected"]
        nb = (t + 1) // 2
        toks = sorted([b * 2 + j for b in idx[u, :cnt[u]] for j in range(2)] +
                      list(range(nb * 2, t + 1)))
        assert toks == e["tokens"]


def test_planted_blocks_are_selected():
    d = inputs.make("prefill_4k_fp32", seed=100)
    kbar = oracle.pool(d["k_idx"][0])
    rows = sorted({p[1] for p in d["plants"]})
    idx, cnt = oracle.index_rows(d["q_idx"][0], kbar, rows)
    for (_, i, blk, *_rest) in d["plants"]:
        u = rows.index(i)
        assert blk in set(idx[u, :cnt[u]].tolist())
        assert cnt[u] == 512


def test_counts_and_id_invariants():
    d = inputs.small(n=300, r=4, K=32, seed=7)
    kbar = oracle.pool(d["k_idx"][0], r=4)
    rows = np.arange(300)
    idx, cnt = oracle.index_rows(d["q_idx"][0], kbar, rows, r=4, K=32)
    for t in rows:
        nb = (t + 1) // 4
        c = cnt[t]
        assert c == min(8, nb)
        ids = idx[t, :c]
        assert np.all(np.diff(ids) > 0) and (c == 0 or (ids[0] >= 0 and ids[-1] < nb))
        assert np.all(idx[t, c:] == -1)


# --------------------------------------------------------------------------
# Sparse core attention ([glide] Figure 3)
# --------------------------------------------------------------------------

def _sdpa(q, k, v, hq, hkv, mask=None, causal=False, scale=None):
    """torch's scaled_dot_product_attention in float64 on the CPU, KV heads
    repeated for GQA.  q: [n][hq][D]; k, v: [hkv][n][D]."""
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)[None]
    rep = hq // hkv
    kt = torch.from_numpy(k.astype(np.float64)).repeat_interleave(rep, 0)[None]
    vt = torch.from_numpy(v.astype(np.float64)).repeat_interleave(rep, 0)[None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m,
                                                         is_causal=causal, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("r,hq,hkv", [(4, 4, 1), (2, 8, 2), (1, 4, 4)])
def test_large_K_is_dense_causal_attention(r, hq, hkv):
    n = 40
    d = inputs.small(n=n, hq=hq, hkv=hkv, r=r, K=4096, seed=8)
    kbar = oracle.pool(d["k_idx"][0], r=r)
    rows = np.arange(n)
    idx, cnt = oracle.index_rows(d["q_idx"][0], kbar, rows, r=r, K=4096)
    out = oracle.attend_rows(d["q"][0], d["k"][0], d["v"][0], rows, idx, cnt, r=r)
    ref = _sdpa(d["q"][0], d["k"][0], d["v"][0], hq, hkv, causal=True)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-13)


def test_masked_dense_equivalence():
    # Figure 3 view: the selection as an n x n 0/1 mask over tokens.
    n, r, K = 64, 4, 16
    d = inputs.small(n=n, hq=8, hkv=2, r=r, K=K, seed=9)
    kbar = oracle.pool(d["k_idx"][0], r=r)
    rows = np.arange(n)
    idx, cnt = oracle.index_rows(d["q_idx"][0], kbar, rows, r=r, K=K)
    mask = np.zeros((n, n), dtype=bool)
    for t in rows:
        for b in idx[t, :cnt[t]]:
            mask[t, b * r:b * r + r] = True
        nb = (t + 1) // r
        mask[t, nb * r:t + 1] = True
    assert not np.any(np.triu(mask, 1)), "selection must be causal"
    out = oracle.attend_rows(d["q"][0], d["k"][0], d["v"][0], rows, idx, cnt, r=r)
    ref = _sdpa(d["q"][0], d["k"][0], d["v"][0], 8, 2, mask=mask)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-13)


# --------------------------------------------------------------------------
# Index reuse across a decode step's new tokens ([glide] "QSA Ablations and
# Efficiency": top-k indices reused across speculative decoding steps)
# --------------------------------------------------------------------------

def test_shared_selection_at_its_own_position_is_the_ordinary_rule():
    n = 300
    d = inputs.small(n=n, hq=8, hkv=2, r=4, K=32, seed=15)
    kbar = oracle.pool(d["k_idx"][0])
    for f in (130, 131, 132, 135):
        idx, cnt = oracle.index_rows(d["q_idx"][0], kbar, [f], K=32)
        a = oracle.attend_rows(d["q"][0], d["k"][0], d["v"][0], [f], idx, cnt)
        b = oracle.attend_shared(d["q"][0][[f]], d["k"][0], d["v"][0], f, [f], idx[0], cnt[0])
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("r", [4, 2])
def test_shared_selection_with_every_block_is_dense_causal(r):
    """K >= n: the first token selects every complete block, so each later
    token attends to all of 0..pos -- torch's causal SDPA in float64."""
    n, n_q = 41, 4
    d = inputs.small(n=n, hq=8, hkv=2, r=r, K=4096, seed=16)
    kbar = oracle.pool(d["k_idx"][0], r=r)
    ref = _sdpa(d["q"][0], d["k"][0], d["v"][0], 8, 2, causal=True)
    for f in (n - n_q, n - n_q - 1, n - n_q - 2):
        idx, cnt = oracle.index_rows(d["q_idx"][0], kbar, [f], r=r, K=4096)
        pos = np.arange(f, f + n_q)
        out = oracle.attend_shared(d["q"][0][pos], d["k"][0], d["v"][0], f, pos, idx[0], cnt[0],
                                   r=r)
        np.testing.assert_allclose(out, ref[pos], rtol=1e-11, atol=1e-13)


def test_shared_selection_masked_dense_equivalence():
    """The shared token sets written as an explicit 0/1 mask (selected blocks
    of the first token, then every token from its block boundary up to the
    row) and run through masked SDPA: the same outputs, and the mask is
    causal for every new token."""
    n, r, K, n_q = 96, 4, 16, 4
    d = inputs.small(n=n, hq=4, hkv=1, r=r, K=K, seed=17)
    kbar = oracle.pool(d["k_idx"][0], r=r)
    for f in (n - n_q, n - n_q - 2):
        idx, cnt = oracle.index_rows(d["q_idx"][0], kbar, [f], r=r, K=K)
        pos = np.arange(f, f + n_q)
        mask = np.zeros((n, n), dtype=bool)
        mask[np.arange(n), np.arange(n)] = True  # rows not checked: any valid mask
        for p_ in pos:
            mask[p_] = False
            for b in idx[0, :cnt[0]]:
                mask[p_, b * r:b * r + r] = True
            mask[p_, (f + 1) // r * r:p_ + 1] = True
        assert not np.any(np.triu(mask, 1)), "shared sets must be causal"
        ref = _sdpa(d["q"][0], d["k"][0], d["v"][0], 4, 1, mask=mask)
        out = oracle.attend_shared(d["q"][0][pos], d["k"][0], d["v"][0], f, pos, idx[0], cnt[0],
                                   r=r)
        np.testing.assert_allclose(out, ref[pos], rtol=1e-11, atol=1e-13)


def test_attention_constant_values_and_first_token():
    n = 32
    d = inputs.small(n=n, hq=4, hkv=1, r=4, K=8, seed=11)
    v = np.ones_like(d["v"][0]) * np.float32(0.375)
    kbar = oracle.pool(d["k_idx"][0], r=4)
    rows = np.arange(n)
    idx, cnt = oracle.index_rows(d["q_idx"][0], kbar, rows, r=4, K=8)
    out = oracle.attend_rows(d["q"][0], d["k"][0], v, rows, idx, cnt, r=4)
    np.testing.assert_allclose(out, 0.375, rtol=1e-14)
    out0 = oracle.attend_rows(d["q"][0], d["k"][0], d["v"][0], [0], idx[:1], cnt[:1], r=4)
    np.testing.assert_array_equal(out0[0], np.broadcast_to(d["v"][0][0, 0], (4, 128)))


def test_decode_equals_last_prefill_row():
    n = 4096
    d = inputs.small(n=n, hq=4, hkv=1, dtype="bf16", seed=12)
    kbar = oracle.pool(d["k_idx"][0])
    rows = [n - 1]
    idx, cnt = oracle.index_rows(d["q_idx"][0], kbar, rows)
    out = oracle.attend_rows(d["q"][0], d["k"][0], d["v"][0], rows, idx, cnt)
    di, dc, do = oracle.decode(d["q_idx"][0, n - 1], d["q"][0, n - 1], kbar, d["k"][0],
                               d["v"][0], seq_len=n)
    assert dc == cnt[0] and np.array_equal(di, idx[0])
    np.testing.assert_array_equal(do, out[0])


def test_rows_given_by_position_equal_prefill_rows():
    """index_at / score_at / attend_at take a compacted set of rows with
    their positions (sampled parity of long sequences); they must address
    the same rows as the prefill-row functions."""
    n = 3000
    d = inputs.small(n=n, hq=8, hkv=2, dtype="bf16", seed=14, planted=4)
    kbar = oracle.pool(d["k_idx"][0])
    rows = np.array([0, 5, 2050, 2051, 2999, 1234])
    idx, cnt = oracle.index_rows(d["q_idx"][0], kbar, rows, K=512)
    ia, ca = oracle.index_at(d["q_idx"][0][rows], kbar, rows, K=512)
    assert np.array_equal(idx, ia) and np.array_equal(cnt, ca)
    sc = oracle.score_rows(d["q_idx"][0], kbar, rows)
    sa = oracle.score_at(d["q_idx"][0][rows], kbar, rows)
    for x, y in zip(sc, sa):
        assert np.array_equal(x, y)
    out = oracle.attend_rows(d["q"][0], d["k"][0], d["v"][0], rows, idx, cnt)
    oa = oracle.attend_at(d["q"][0][rows], d["k"][0], d["v"][0], rows, ia, ca)
    assert np.array_equal(out, oa)


def test_generator_is_deterministic():
    import hashlib
    a = inputs.small(n=128, dtype="bf16", seed=3, planted=0)
    b = inputs.small(n=128, dtype="bf16", seed=3, planted=0)
    for name in ("q_idx", "k_idx", "q", "k", "v"):
        assert hashlib.sha256(a[name].tobytes()).digest() == \
            hashlib.sha256(b[name].tobytes()).digest()
