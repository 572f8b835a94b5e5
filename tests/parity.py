"""Helpers of the GPU parity tests: host<->device transfer of the exact
stored bits, the near-tie rule for block sets, and the error metric.

Tolerances (fixed by the method's statement of the problem):
  - block-index sets: identical, except that a block may differ between the
    two sets when its oracle score lies within 1e-3 relative of the k-th
    largest oracle score (near-tie); an absolute floor of 1e-6 times the
    row's largest score covers a k-th score of exactly zero (ReLU floor);
    counts must be identical;
  - outputs: max|o - o_ref| / max|o_ref| <= 2e-2 for bf16 inputs, 1e-4 for
    float32 inputs.
"""
import numpy as np
import torch

TOL = {"bf16": 2e-2, "fp32": 1e-4}


def to_dev(a, device="cuda"):
    """NumPy float32 or bf16 bits (uint16) -> torch tensor with the same bits."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def to_host(t):
    """torch tensor -> NumPy with the same bits (bf16 -> uint16 bits)."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def rel_err(o, ref):
    o, ref = as_f64(o), as_f64(ref)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(o - ref)) / (den if den > 0 else 1.0))


def check_sets(g_idx, g_cnt, o_idx, o_cnt, o_scores, rel=1e-3, floor=1e-6):
    """Compare GPU and oracle selections row by row.  o_scores: list of the
    oracle's score vectors of the same rows.  Returns the number of near-tie
    differences; raises AssertionError on any other difference."""
    g_idx, o_idx = np.asarray(g_idx), np.asarray(o_idx)
    g_cnt, o_cnt = np.asarray(g_cnt), np.asarray(o_cnt)
    assert np.array_equal(g_cnt, o_cnt), "counts differ at rows %s" % \
        np.nonzero(g_cnt != o_cnt)[0][:10]
    near = 0
    for u in range(g_idx.shape[0]):
        c = int(o_cnt[u])
        g, o = g_idx[u, :c], o_idx[u, :c]
        assert np.all(g_idx[u, c:] == -1), "row %d: padding is not -1" % u
        assert np.all(np.diff(g) > 0), "row %d: ids not strictly ascending" % u
        if np.array_equal(g, o):
            continue
        s = o_scores[u]
        assert g.min() >= 0 and g.max() < s.shape[0], "row %d: id out of the visible range" % u
        sk = np.sort(s)[::-1][c - 1]
        diff = np.setxor1d(g, o)
        tol = rel * abs(sk) + floor * float(s.max())
        bad = diff[np.abs(s[diff] - sk) > tol]
        assert bad.size == 0, "row %d: blocks %s differ beyond the near-tie band (s_k=%g, s=%s)" % (
            u, bad[:8], sk, s[bad[:8]])
        near += diff.size
    return near
