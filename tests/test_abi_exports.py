"""The C-ABI library loads and exports every entry point include/qsa.h
declares; host-side validation rejects bad arguments before any launch (no
GPU needed: every case below fails validation on the host)."""
import ctypes
import os
import re

import pytest

from trainable_sparse_attention_amd import qsa

INC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")


def _declared():
    names = set()
    for f in sorted(os.listdir(INC)):
        if f.endswith(".h"):
            src = re.sub(r"/\*.*?\*/", "", open(os.path.join(INC, f)).read(), flags=re.S)
            names.update(re.findall(r"\b(qsa_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


def test_header_and_binding_agree():
    assert sorted(qsa.EXPORTS) == _declared()


def test_library_exports_every_declared_symbol():
    lib = qsa.lib()
    for name in _declared():
        assert hasattr(lib, name), name


def test_defaults_and_status_strings():
    lib = qsa.lib()
    p = qsa.Params()
    lib.qsa_default_params(ctypes.byref(p))
    assert (p.r, p.K, p.h_idx, p.d_idx, p.rope_dims, p.rope_theta) == (4, 2048, 4, 128, 64, 10000.0)
    assert qsa.k_blocks(p) == 512
    for code, name in qsa.STATUS.items():
        assert lib.qsa_status_str(code).decode() == name


def _expect(status, code, lib):
    assert status == code, (qsa.STATUS.get(status), lib.qsa_last_error().decode())
    assert lib.qsa_last_error().decode() != ""


def test_host_validation_errors():
    lib = qsa.lib()
    p = qsa.params()
    P = ctypes.byref(p)
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    _expect(lib.qsa_pool_keys(P, 1, None, 64, fake, 16, 1, 0, 16, None), 1, lib)
    _expect(lib.qsa_pool_keys(P, 7, fake, 64, fake, 16, 1, 0, 16, None), 3, lib)
    _expect(lib.qsa_pool_keys(P, 1, fake, 60, fake, 16, 1, 0, 16, None), 2, lib)
    _expect(lib.qsa_pool_keys(P, 1, fake, 64, fake, 15, 1, 0, 16, None), 2, lib)
    _expect(lib.qsa_pool_keys(P, 1, fake, 64, fake, 16, 1, 5, 4, None), 2, lib)
    for r in (3, 32, 0):  # built for r in {1, 2, 4, 8, 16}
        bad = qsa.params(r=r)
        _expect(lib.qsa_pool_keys(ctypes.byref(bad), 1, fake, 64, fake, 16, 1, 0, 8, None), 4,
                lib)
    # RMS-normalised pooling: gain and eps checked
    _expect(lib.qsa_pool_keys_rmsnorm(P, 1, fake, 64, None, 1e-6, fake, 16, 1, 0, 16, None), 1,
            lib)
    _expect(lib.qsa_pool_keys_rmsnorm(P, 1, fake, 64, fake, -1.0, fake, 16, 1, 0, 16, None), 2,
            lib)
    _expect(lib.qsa_pool_keys_rmsnorm(P, 1, fake, 60, fake, 1e-6, fake, 16, 1, 0, 16, None), 2,
            lib)
    _expect(lib.qsa_pool_keys(None, 1, fake, 64, fake, 16, 1, 0, 8, None), 1, lib)
    # index: too few blocks for the positions; workspace missing; n_q < 1
    _expect(lib.qsa_index_topk(P, 1, fake, fake, 10, 1, 64, 0, None, fake, fake, fake, 1 << 30,
                               None), 2, lib)
    _expect(lib.qsa_index_topk(P, 1, fake, fake, 16, 1, 0, 0, None, fake, fake, fake, 1 << 30,
                               None), 2, lib)
    _expect(lib.qsa_index_topk(P, 1, fake, fake, 16, 1, 64, 0, None, fake, fake, None, 0, None),
            5, lib)
    # attention: head dim, GQA ratio, positions beyond the cache
    _expect(lib.qsa_sparse_attn_prefill(P, 1, fake, fake, fake, 64, fake, fake, 1, 8, 0, 16, 2,
                                        64, 0.0, fake, None), 4, lib)
    _expect(lib.qsa_sparse_attn_prefill(P, 1, fake, fake, fake, 64, fake, fake, 1, 8, 0, 16, 3,
                                        128, 0.0, fake, None), 2, lib)
    _expect(lib.qsa_sparse_attn_prefill(P, 1, fake, fake, fake, 64, fake, fake, 1, 8, 0, 64, 2,
                                        128, 0.0, fake, None), 4, lib)
    _expect(lib.qsa_sparse_attn_prefill(P, 1, fake, fake, fake, 64, fake, fake, 1, 8, 60, 16, 2,
                                        128, 0.0, fake, None), 2, lib)
    _expect(lib.qsa_sparse_attn_decode(P, 1, fake, fake, fake, 64, None, fake, fake, 1, 1, 16, 2,
                                       128, 0.0, fake, fake, 1 << 30, None), 1, lib)
    _expect(lib.qsa_sparse_attn_decode(P, 1, fake, fake, fake, 64, fake, fake, fake, 1, 1, 16, 2,
                                       128, 0.0, fake, fake, 0, None), 5, lib)


def test_host_validation_of_built_limits():
    """Sizes valid for the method but beyond what the kernels are built for
    are refused on the host: k_B above the candidate-list bounds, and KV
    capacities whose bf16 byte offsets would not fit 32 bits."""
    lib = qsa.lib()
    fake = ctypes.c_void_p(16)
    big = qsa.params(K=4 * 3073)           # k_B = 3073: many-row lists too small
    _expect(lib.qsa_index_topk(ctypes.byref(big), 1, fake, fake, 1 << 16, 1, 4096, 0, None,
                               fake, fake, fake, 1 << 40, None), 4, lib)
    ok = qsa.params(K=4 * 3072)            # k_B = 3072 passes this check (fails on workspace)
    _expect(lib.qsa_index_topk(ctypes.byref(ok), 1, fake, fake, 1 << 16, 1, 4096, 0, None,
                               fake, fake, None, 0, None), 5, lib)
    dec = qsa.params(K=4 * 4097)           # decode form: k_B = 4097
    _expect(lib.qsa_index_topk(ctypes.byref(dec), 1, fake, fake, 1 << 16, 2, 1, 0, fake, fake,
                               fake, fake, 1 << 40, None), 4, lib)
    # indexer head counts: 1, 2 and 4 are built (absent heads are zero
    # queries), 3 and 8 are not
    for h, want in ((3, 4), (8, 4)):
        ph = qsa.params(h_idx=h)
        _expect(lib.qsa_index_topk(ctypes.byref(ph), 1, fake, fake, 1 << 16, 1, 4096, 0, None,
                                   fake, fake, fake, 1 << 40, None), want, lib)
    for h in (1, 2):
        ph = qsa.params(h_idx=h)        # passes to the workspace check
        _expect(lib.qsa_index_topk(ctypes.byref(ph), 1, fake, fake, 1 << 16, 1, 4096, 0, None,
                                   fake, fake, None, 0, None), 5, lib)
    p = qsa.params()
    P = ctypes.byref(p)
    cap = (1 << 24) + 4
    _expect(lib.qsa_sparse_attn_prefill(P, 1, fake, fake, fake, cap, fake, fake, 1, 8, 0, 16, 2,
                                        128, 0.0, fake, None), 4, lib)
    _expect(lib.qsa_sparse_attn_decode(P, 1, fake, fake, fake, cap, fake, fake, fake, 1, 1, 16,
                                       2, 128, 0.0, fake, fake, 1 << 30, None), 4, lib)
    # fp32 addresses rows in 64 bits: the same capacity passes to the
    # positions check (q_pos0 + n_q beyond n_cap fails instead)
    _expect(lib.qsa_sparse_attn_prefill(P, 0, fake, fake, fake, cap, fake, fake, 1, 8, cap, 16, 2,
                                        128, 0.0, fake, None), 2, lib)


def test_workspace_sizes_grow_with_work():
    p = qsa.params()
    a = qsa.qsa_index_topk_workspace(p, 1, 1, 4096, 1024, False)
    b = qsa.qsa_index_topk_workspace(p, 1, 1, 1 << 18, 1 << 16, False)
    assert 0 < a <= b
    d = qsa.qsa_index_topk_workspace(p, 1, 8, 1, 1 << 18, True)
    assert d >= 8 * (1 << 18) * 4  # one score per block per sequence
    assert qsa.qsa_sparse_attn_decode_workspace(p, 8, 1, 16, 2) > 0
    # distillation: one float per (sequence, row, visible block), rows packed
    for B, n_q, q_pos0 in ((1, 1, 0), (2, 37, 5), (3, 1000, 4093), (1, 4096, 0)):
        blocks = sum((q + 1) // 4 for q in range(q_pos0, q_pos0 + n_q))
        assert qsa.qsa_index_distill_workspace(p, B, n_q, q_pos0) == B * blocks * 4


def test_distill_rejects_small_workspace():
    lib = qsa.lib()
    p = qsa.params()
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    need = qsa.qsa_index_distill_workspace(p, 1, 64, 0)
    assert need > 0
    for ws, nbytes in ((None, 0), (fake, need - 4)):
        _expect(lib.qsa_index_distill(ctypes.byref(p), 1, fake, fake, 64, fake, fake, 16, 1, 64, 0,
                                      16, 2, 128, 0.0, fake, fake, fake, ws, nbytes, None), 5, lib)
