"""ctypes wrapper around the C oracle (``qsa_oracle.c``) -- test infrastructure.

Arrays are NumPy arrays holding either float32 values or bfloat16 bit
patterns (``uint16``).  Every function reads the exact stored values and
computes in double precision; see the C source for the definitions and the
passages of the pages each one follows.
"""
import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_LIBDIR = os.path.join(_HERE, "lib")
_LIB = os.path.join(_LIBDIR, "libqsa_oracle.so")
_lib = None

F32, BF16 = 0, 1


def build(force=True):
    """Compile the oracle with the host C compiler (no GPU code involved)."""
    os.makedirs(_LIBDIR, exist_ok=True)
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P, I, L, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.orc_pool.argtypes = [P, I, I, I, I, D, L, L, P, I]
        lib.orc_pool.restype = None
        lib.orc_pool_rmsnorm.argtypes = [P, I, I, I, I, D, L, L, P, D, P, I]
        lib.orc_pool_rmsnorm.restype = None
        lib.orc_rope_rows.argtypes = [P, L, I, I, D, P]
        lib.orc_rope_rows.restype = None
        lib.orc_scores.argtypes = [P, P, I, I, I, I, I, D, L, P]
        lib.orc_scores.restype = L
        lib.orc_select.argtypes = [P, L, I, P]
        lib.orc_select.restype = I
        lib.orc_index_rows.argtypes = [P, P, I, I, I, I, I, D, I, L, P, L, P, P]
        lib.orc_index_rows.restype = None
        lib.orc_score_rows.argtypes = [P, P, I, I, I, I, I, D, L, P, L, P, L]
        lib.orc_score_rows.restype = None
        lib.orc_attend_rows.argtypes = [P, P, P, I, L, L, P, L, P, P, I, I, I, I, I, D, P]
        lib.orc_attend_rows.restype = None
        lib.orc_attend_shared.argtypes = [P, P, P, I, L, L, L, P, I, I, I, I, I, D, P]
        lib.orc_attend_shared.restype = L
        lib.orc_attend_backward.argtypes = [P, P, P, I, L, L, P, I, I, I, I, I, D, P, P, P, P]
        lib.orc_attend_backward.restype = None
        lib.orc_distill_row.argtypes = [P, P, I, L, I, I, I, D, P, P, I, I, I, I, D, L, P, P, P]
        lib.orc_distill_row.restype = D
        lib.orc_pool_backward.argtypes = [P, I, I, I, D, L, L, P]
        lib.orc_pool_backward.restype = None
        lib.orc_index_at.argtypes = [P, P, I, I, I, I, I, D, I, P, L, P, P]
        lib.orc_index_at.restype = None
        lib.orc_score_at.argtypes = [P, P, I, I, I, I, I, D, P, L, P, L]
        lib.orc_score_at.restype = None
        lib.orc_attend_at.argtypes = [P, P, P, I, L, P, L, P, P, I, I, I, I, I, D, P]
        lib.orc_attend_at.restype = None
        _lib = lib
    return _lib


def _dt(*arrs):
    kinds = {a.dtype for a in arrs}
    if len(kinds) != 1:
        raise TypeError("oracle inputs must share one storage type, got %s" % kinds)
    k = kinds.pop()
    if k == np.float32:
        return F32
    if k == np.uint16:
        return BF16
    raise TypeError("oracle takes float32 or bfloat16 bits (uint16), got %s" % k)


def _c(a):
    return np.ascontiguousarray(a)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def k_blocks(K, r):
    """k_B = ceil(K / r)."""
    return -(-K // r)


def pool(k_idx, r=4, rope_dims=64, theta=10000.0, b0=0, b1=None):
    """Pooled, partially rotated keys of blocks [b0, b1) of one sequence.

    k_idx: [n_tok][d].  Returns [(b1 - b0)][d] in the same storage type."""
    k_idx = _c(k_idx)
    dt = _dt(k_idx)
    n, d = k_idx.shape
    if b1 is None:
        b1 = n // r
    out = np.empty((b1 - b0, d), dtype=k_idx.dtype)
    load().orc_pool(_p(k_idx), dt, d, r, rope_dims, float(theta), b0, b1, _p(out), dt)
    return out


def pool_rmsnorm(k_idx, gamma, eps=1e-6, r=4, rope_dims=64, theta=10000.0, b0=0, b1=None):
    """Pooled keys of blocks [b0, b1) with the block mean RMS-normalised (gain
    gamma [d], float64) before the rotation; same storage type as k_idx."""
    k_idx = _c(k_idx)
    dt = _dt(k_idx)
    n, d = k_idx.shape
    if b1 is None:
        b1 = n // r
    g = _c(np.asarray(gamma, dtype=np.float64))
    assert g.shape == (d,)
    out = np.empty((b1 - b0, d), dtype=k_idx.dtype)
    load().orc_pool_rmsnorm(_p(k_idx), dt, d, r, rope_dims, float(theta), b0, b1, _p(g),
                            float(eps), _p(out), dt)
    return out


def rope_rows(x, pos, rope_dims=64, theta=10000.0):
    """Rotate rows of a float64 [n][d] array; row t at position pos[t]."""
    x = np.array(x, dtype=np.float64, copy=True, order="C")
    pos = _c(np.asarray(pos, dtype=np.int64))
    n, d = x.shape
    load().orc_rope_rows(_p(x), n, d, rope_dims, float(theta), _p(pos))
    return x


def scores(q_row, kbar, pos, r=4, rope_dims=64, theta=10000.0):
    """Block scores of one query at position pos: float64 [floor((pos+1)/r)]."""
    q_row, kbar = _c(q_row), _c(kbar)
    dt = _dt(q_row, kbar)
    h, d = q_row.shape
    nb = (pos + 1) // r
    if kbar.shape[0] < nb:
        raise ValueError("kbar holds %d blocks, query at %d sees %d" % (kbar.shape[0], pos, nb))
    out = np.empty(max(nb, 1), dtype=np.float64)
    load().orc_scores(_p(q_row), _p(kbar), dt, h, d, r, rope_dims, float(theta), pos, _p(out))
    return out[:nb]


def select(sc, kB):
    """Top-kB ids of a score vector (ascending ids, -1 padded) and the count."""
    sc = _c(np.asarray(sc, dtype=np.float64))
    idx = np.empty(kB, dtype=np.int32)
    c = load().orc_select(_p(sc), sc.shape[0], kB, _p(idx))
    return idx, c


def index_rows(q_idx, kbar, rows, pos0=0, r=4, K=2048, rope_dims=64, theta=10000.0):
    """Selections of listed query rows of one sequence.

    q_idx: [n_q][h][d]; kbar: [nb_cap][d].  Returns idx [nrows][k_B] int32 and
    cnt [nrows] int32."""
    q_idx, kbar = _c(q_idx), _c(kbar)
    dt = _dt(q_idx, kbar)
    _, h, d = q_idx.shape
    rows = _c(np.asarray(rows, dtype=np.int64))
    kB = k_blocks(K, r)
    need = (pos0 + int(rows.max()) + 1) // r if rows.size else 0
    if kbar.shape[0] < need:
        raise ValueError("kbar too short")
    idx = np.empty((rows.size, kB), dtype=np.int32)
    cnt = np.empty(rows.size, dtype=np.int32)
    load().orc_index_rows(_p(q_idx), _p(kbar), dt, h, d, r, rope_dims, float(theta), kB, pos0,
                          _p(rows), rows.size, _p(idx), _p(cnt))
    return idx, cnt


def score_rows(q_idx, kbar, rows, pos0=0, r=4, rope_dims=64, theta=10000.0):
    """Block scores of listed rows: list of float64 arrays."""
    q_idx, kbar = _c(q_idx), _c(kbar)
    dt = _dt(q_idx, kbar)
    _, h, d = q_idx.shape
    rows = _c(np.asarray(rows, dtype=np.int64))
    stride = max(1, (pos0 + int(rows.max()) + 1) // r) if rows.size else 1
    out = np.zeros((rows.size, stride), dtype=np.float64)
    load().orc_score_rows(_p(q_idx), _p(kbar), dt, h, d, r, rope_dims, float(theta), pos0,
                          _p(rows), rows.size, _p(out), stride)
    return [out[u, : (pos0 + int(t) + 1) // r] for u, t in enumerate(rows)]


def attend_rows(q, k, v, rows, idx, cnt, pos0=0, r=4, scale=None):
    """Attention outputs (float64 [nrows][hq][D]) of listed rows given their
    selections.  q: [n_q][hq][D]; k, v: [hkv][n_cap][D]."""
    q, k, v = _c(q), _c(k), _c(v)
    dt = _dt(q, k, v)
    _, hq, D = q.shape
    hkv, n_cap, _ = k.shape
    rows = _c(np.asarray(rows, dtype=np.int64))
    idx = _c(np.asarray(idx, dtype=np.int32))
    cnt = _c(np.asarray(cnt, dtype=np.int32))
    kB = idx.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if rows.size and pos0 + int(rows.max()) >= n_cap:
        raise ValueError("query position beyond the KV capacity")
    out = np.empty((rows.size, hq, D), dtype=np.float64)
    load().orc_attend_rows(_p(q), _p(k), _p(v), dt, n_cap, pos0, _p(rows), rows.size, _p(idx),
                           _p(cnt), kB, r, hq, hkv, D, float(scale), _p(out))
    return out


def prefill_rows(k_idx, q_idx, q, k, v, rows, r=4, K=2048, rope_dims=64, theta=10000.0,
                 scale=None):
    """Whole path for listed rows of one sequence starting at position 0:
    pool -> score -> select -> attend.  Returns (kbar, idx, cnt, out)."""
    kbar = pool(k_idx, r, rope_dims, theta)
    idx, cnt = index_rows(q_idx, kbar, rows, 0, r, K, rope_dims, theta)
    out = attend_rows(q, k, v, rows, idx, cnt, 0, r, scale)
    return kbar, idx, cnt, out


def decode(q_idx_row, q_row, kbar, k, v, seq_len, r=4, K=2048, rope_dims=64, theta=10000.0,
           scale=None):
    """One decode query at position seq_len - 1 (the new token is already in
    the caches).  q_idx_row: [h][d]; q_row: [hq][D]; kbar: [nb_cap][d];
    k, v: [hkv][n_cap][D].  Returns (idx [k_B], cnt, out [hq][D])."""
    pos = seq_len - 1
    idx, cnt = index_rows(np.asarray(q_idx_row)[None], kbar, [0], pos, r, K, rope_dims, theta)
    out = attend_rows(np.asarray(q_row)[None], k, v, [0], idx, cnt, pos, r, scale)
    return idx[0], int(cnt[0]), out[0]


def index_at(q_rows, kbar, pos, r=4, K=2048, rope_dims=64, theta=10000.0):
    """Selections of query rows given with their positions: q_rows [m][h][d],
    row u at token position pos[u]; kbar [nb_cap][d].  Returns idx [m][k_B]
    int32 and cnt [m] int32 (the steps of index_rows)."""
    q_rows, kbar = _c(q_rows), _c(kbar)
    dt = _dt(q_rows, kbar)
    m, h, d = q_rows.shape
    pos = _c(np.asarray(pos, dtype=np.int64))
    assert pos.shape == (m,)
    kB = k_blocks(K, r)
    if m and kbar.shape[0] < (int(pos.max()) + 1) // r:
        raise ValueError("kbar too short")
    idx = np.empty((m, kB), dtype=np.int32)
    cnt = np.empty(m, dtype=np.int32)
    load().orc_index_at(_p(q_rows), _p(kbar), dt, h, d, r, rope_dims, float(theta), kB, _p(pos),
                        m, _p(idx), _p(cnt))
    return idx, cnt


def score_at(q_rows, kbar, pos, r=4, rope_dims=64, theta=10000.0):
    """Block scores of query rows given with their positions: list of float64
    arrays, row u of length floor((pos[u] + 1) / r)."""
    q_rows, kbar = _c(q_rows), _c(kbar)
    dt = _dt(q_rows, kbar)
    m, h, d = q_rows.shape
    pos = _c(np.asarray(pos, dtype=np.int64))
    stride = max(1, (int(pos.max()) + 1) // r) if m else 1
    out = np.zeros((m, stride), dtype=np.float64)
    load().orc_score_at(_p(q_rows), _p(kbar), dt, h, d, r, rope_dims, float(theta), _p(pos), m,
                        _p(out), stride)
    return [out[u, : (int(p) + 1) // r] for u, p in enumerate(pos)]


def attend_at(q_rows, k, v, pos, idx, cnt, r=4, scale=None):
    """Attention outputs (float64 [m][hq][D]) of query rows given with their
    positions and selections.  q_rows [m][hq][D]; k, v [hkv][n_cap][D]."""
    q_rows, k, v = _c(q_rows), _c(k), _c(v)
    dt = _dt(q_rows, k, v)
    m, hq, D = q_rows.shape
    hkv, n_cap, _ = k.shape
    pos = _c(np.asarray(pos, dtype=np.int64))
    idx = _c(np.asarray(idx, dtype=np.int32))
    cnt = _c(np.asarray(cnt, dtype=np.int32))
    kB = idx.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if m and int(pos.max()) >= n_cap:
        raise ValueError("query position beyond the KV capacity")
    out = np.empty((m, hq, D), dtype=np.float64)
    load().orc_attend_at(_p(q_rows), _p(k), _p(v), dt, n_cap, _p(pos), m, _p(idx), _p(cnt), kB,
                         r, hq, hkv, D, float(scale), _p(out))
    return out


def attend_shared(q_rows, k, v, f, pos, idx_row, cnt, r=4, scale=None):
    """Attention (float64 [m][hq][D]) of a decode step's new tokens that
    share one selection made at position f: row u sits at pos[u] >= f and
    attends to the selected blocks (idx_row[:cnt]) and to the tokens
    floor((f+1)/r)*r .. pos[u].  q_rows [m][hq][D]; k, v [hkv][n_cap][D]."""
    q_rows, k, v = _c(q_rows), _c(k), _c(v)
    dt = _dt(q_rows, k, v)
    m, hq, D = q_rows.shape
    hkv, n_cap, _ = k.shape
    idx_row = _c(np.asarray(idx_row, dtype=np.int32))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.empty((m, hq, D), dtype=np.float64)
    step = hq * D * (2 if dt == BF16 else 4)
    base = q_rows.ctypes.data
    for u in range(m):
        p_u = int(pos[u])
        if p_u < f or p_u >= n_cap:
            raise ValueError("positions must lie in [f, n_cap)")
        load().orc_attend_shared(ctypes.c_void_p(base + u * step), _p(k), _p(v), dt, n_cap,
                                 int(f), p_u, _p(idx_row), int(cnt), r, hq, hkv, D, float(scale),
                                 out[u].ctypes.data_as(ctypes.c_void_p))
    return out


# ---- training path ---------------------------------------------------------

def attend_backward(q_rows, k, v, pos, idx, cnt, dout, r=4, scale=None):
    """Backward of the sparse attention of rows given with their positions
    and selections: dout [m][hq][D] (float64) -> dq [m][hq][D], dk, dv
    [hkv][n_cap][D] (float64; dk, dv summed over the rows)."""
    q_rows, k, v = _c(q_rows), _c(k), _c(v)
    dt = _dt(q_rows, k, v)
    m, hq, D = q_rows.shape
    hkv, n_cap, _ = k.shape
    idx = _c(np.asarray(idx, dtype=np.int32))
    cnt = _c(np.asarray(cnt, dtype=np.int32))
    dout = _c(np.asarray(dout, dtype=np.float64))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = np.zeros((m, hq, D), dtype=np.float64)
    dk = np.zeros((hkv, n_cap, D), dtype=np.float64)
    dv = np.zeros((hkv, n_cap, D), dtype=np.float64)
    step = hq * D * (2 if dt == BF16 else 4)
    for u in range(m):
        load().orc_attend_backward(ctypes.c_void_p(q_rows.ctypes.data + u * step), _p(k), _p(v),
                                   dt, n_cap, int(pos[u]), idx[u].ctypes.data_as(ctypes.c_void_p),
                                   int(cnt[u]), r, hq, hkv, D, float(scale),
                                   dout[u].ctypes.data_as(ctypes.c_void_p),
                                   dq[u].ctypes.data_as(ctypes.c_void_p), _p(dk), _p(dv))
    return dq, dk, dv


def distill_rows(q_rows, k, q_idx_rows, kbar, pos, r=4, rope_dims=64, theta=10000.0, scale=None,
                 return_g=False):
    """Indexer distillation of rows given with their positions: per-row KL of
    the indexer's block distribution to the block-max-pooled, head-summed
    dense attention.  q_rows [m][hq][D]; k [hkv][n_cap][D]; q_idx_rows
    [m][h][d] (not rotated); kbar [nb_cap][d] (as stored).  Returns loss [m],
    dq_idx [m][h][d] and dkbar [nb_cap][d] (float64, summed over the rows);
    with return_g also g [m][nb_cap], the loss gradient with respect to each
    visible block's score I_b (zero past the row's visible blocks)."""
    q_rows, k, q_idx_rows, kbar = _c(q_rows), _c(k), _c(q_idx_rows), _c(kbar)
    dt = _dt(q_rows, k, q_idx_rows, kbar)
    m, hq, D = q_rows.shape
    hkv, n_cap, _ = k.shape
    _, h, d = q_idx_rows.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    loss = np.zeros(m, dtype=np.float64)
    dq = np.zeros((m, h, d), dtype=np.float64)
    dkbar = np.zeros((kbar.shape[0], d), dtype=np.float64)
    g = np.zeros((m, kbar.shape[0]), dtype=np.float64)
    esz = 2 if dt == BF16 else 4
    for u in range(m):
        loss[u] = load().orc_distill_row(
            ctypes.c_void_p(q_rows.ctypes.data + u * hq * D * esz), _p(k), dt, n_cap, hq, hkv, D,
            float(scale), ctypes.c_void_p(q_idx_rows.ctypes.data + u * h * d * esz), _p(kbar), h,
            d, r, rope_dims, float(theta), int(pos[u]), dq[u].ctypes.data_as(ctypes.c_void_p),
            _p(dkbar), g[u].ctypes.data_as(ctypes.c_void_p))
    if return_g:
        return loss, dq, dkbar, g
    return loss, dq, dkbar


def pool_backward(dkbar, r=4, rope_dims=64, theta=10000.0, b0=0):
    """Gradient of the raw indexer keys of blocks [b0, b0 + len) from the
    gradient of their pooled keys: [(len) r][d] float64."""
    dkbar = _c(np.asarray(dkbar, dtype=np.float64))
    nbk, d = dkbar.shape
    out = np.empty((nbk * r, d), dtype=np.float64)
    load().orc_pool_backward(_p(dkbar), d, r, rope_dims, float(theta), b0, b0 + nbk, _p(out))
    return out
