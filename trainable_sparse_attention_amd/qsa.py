"""ctypes binding of libqsa (C ABI in include/qsa.h).

Argument marshalling only: tensors are torch CUDA (ROCm) tensors whose
device pointers are handed to the C entry points of the same names; every
step of the computation runs in the HIP kernels.  The library must be built
(``python -m trainable_sparse_attention_amd.build``); loading fails loudly
otherwise -- there is no CPU fallback.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libqsa.so")

QSA_FP32, QSA_BF16 = 0, 1
STATUS = {0: "QSA_OK", 1: "QSA_ERR_NULL", 2: "QSA_ERR_SHAPE", 3: "QSA_ERR_DTYPE",
          4: "QSA_ERR_UNSUPPORTED", 5: "QSA_ERR_WORKSPACE", 6: "QSA_ERR_LAUNCH"}

# every symbol the headers in include/ declare
EXPORTS = ["qsa_default_params", "qsa_k_blocks", "qsa_status_str", "qsa_last_error",
           "qsa_pool_keys", "qsa_pool_keys_rmsnorm", "qsa_index_topk",
           "qsa_index_topk_workspace",
           "qsa_sparse_attn_prefill", "qsa_sparse_attn_decode",
           "qsa_sparse_attn_decode_workspace", "qsa_sparse_attn_decode_shared",
           "qsa_sparse_attn_decode_noalloc", "qsa_sparse_attn_backward",
           "qsa_sparse_attn_backward_workspace", "qsa_index_distill",
           "qsa_index_distill_workspace",
           "qsa_pool_keys_backward",
           "qsa_dense_attn_prefill",
           "qsa_dense_attn_decode", "qsa_dense_attn_decode_workspace",
           "qsa_probe_gather"]


class QSAError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (STATUS.get(status, status), msg))
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [("r", ctypes.c_int32), ("K", ctypes.c_int32), ("h_idx", ctypes.c_int32),
                ("d_idx", ctypes.c_int32), ("rope_dims", ctypes.c_int32),
                ("rope_theta", ctypes.c_float)]


_lib = None


def lib():
    """Load libqsa.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libqsa.so not built at %s; run `python -m "
                              "trainable_sparse_attention_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ, F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                              ctypes.c_float)
        PP = ctypes.POINTER(Params)
        L.qsa_default_params.argtypes = [PP]
        L.qsa_default_params.restype = None
        L.qsa_k_blocks.argtypes = [PP]
        L.qsa_k_blocks.restype = I32
        L.qsa_status_str.argtypes = [ctypes.c_int]
        L.qsa_status_str.restype = ctypes.c_char_p
        L.qsa_last_error.argtypes = []
        L.qsa_last_error.restype = ctypes.c_char_p
        L.qsa_pool_keys.argtypes = [PP, ctypes.c_int, P, I64, P, I64, I32, I64, I64, P]
        L.qsa_pool_keys.restype = ctypes.c_int
        L.qsa_pool_keys_rmsnorm.argtypes = [PP, ctypes.c_int, P, I64, P, F, P, I64, I32, I64, I64,
                                            P]
        L.qsa_pool_keys_rmsnorm.restype = ctypes.c_int
        L.qsa_index_topk.argtypes = [PP, ctypes.c_int, P, P, I64, I32, I32, I64, P, P, P, P, SZ,
                                     P]
        L.qsa_index_topk.restype = ctypes.c_int
        L.qsa_index_topk_workspace.argtypes = [PP, ctypes.c_int, I32, I32, I64, I32]
        L.qsa_index_topk_workspace.restype = SZ
        L.qsa_sparse_attn_prefill.argtypes = [PP, ctypes.c_int, P, P, P, I64, P, P, I32, I32, I64,
                                              I32, I32, I32, F, P, P]
        L.qsa_sparse_attn_prefill.restype = ctypes.c_int
        L.qsa_sparse_attn_decode.argtypes = [PP, ctypes.c_int, P, P, P, I64, P, P, P, I32, I32,
                                             I32, I32, I32, F, P, P, SZ, P]
        L.qsa_sparse_attn_decode.restype = ctypes.c_int
        L.qsa_sparse_attn_decode_workspace.argtypes = [PP, I32, I32, I32, I32, I32]
        L.qsa_sparse_attn_decode_workspace.restype = SZ
        L.qsa_sparse_attn_decode_shared.argtypes = [PP, ctypes.c_int, P, P, P, I64, P, P, P, I32,
                                                    I32, I32, I32, I32, F, P, P, SZ, P]
        L.qsa_sparse_attn_decode_shared.restype = ctypes.c_int
        L.qsa_sparse_attn_decode_noalloc.argtypes = [PP, ctypes.c_int, P, P, P, I64, P, P, P,
                                                     I32, I32, I32, I32, I32, F, P, P]
        L.qsa_sparse_attn_decode_noalloc.restype = ctypes.c_int
        L.qsa_sparse_attn_backward.argtypes = [PP, ctypes.c_int, P, P, P, I64, P, P, P, P, I32,
                                               I32, I64, I32, I32, I32, F, P, P, P, P, SZ, P]
        L.qsa_sparse_attn_backward.restype = ctypes.c_int
        L.qsa_sparse_attn_backward_workspace.argtypes = [PP, I32, I32, I64, I32]
        L.qsa_sparse_attn_backward_workspace.restype = SZ
        L.qsa_index_distill.argtypes = [PP, ctypes.c_int, P, P, I64, P, P, I64, I32, I32, I64, I32,
                                        I32, I32, F, P, P, P, P, SZ, P]
        L.qsa_index_distill.restype = ctypes.c_int
        L.qsa_index_distill_workspace.argtypes = [PP, I32, I32, I64]
        L.qsa_index_distill_workspace.restype = SZ
        L.qsa_pool_keys_backward.argtypes = [PP, P, I64, P, I64, I32, I64, I64, P]
        L.qsa_pool_keys_backward.restype = ctypes.c_int
        L.qsa_dense_attn_prefill.argtypes = [ctypes.c_int, P, P, P, I64, I32, I32, I64, I32, I32,
                                             I32, F, P, P]
        L.qsa_dense_attn_prefill.restype = ctypes.c_int
        L.qsa_dense_attn_decode.argtypes = [ctypes.c_int, P, P, P, I64, P, I32, I32, I32, I32, I32,
                                            F, P, P, SZ, P]
        L.qsa_dense_attn_decode.restype = ctypes.c_int
        L.qsa_dense_attn_decode_workspace.argtypes = [I32, I32, I32, I64]
        L.qsa_dense_attn_decode_workspace.restype = SZ
        L.qsa_probe_gather.argtypes = [PP, P, P, I64, P, P, I32, I32, I64, I32, I32, I32, I32, P,
                                       P]
        L.qsa_probe_gather.restype = ctypes.c_int
        _lib = L
    return _lib


def params(r=4, K=2048, h_idx=4, d_idx=128, rope_dims=64, rope_theta=10000.0):
    return Params(r, K, h_idx, d_idx, rope_dims, rope_theta)


def _check(status):
    if status != 0:
        raise QSAError(status, lib().qsa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return QSA_FP32
    if t.dtype == torch.bfloat16:
        return QSA_BF16
    raise TypeError("QSA tensors are float32 or bfloat16, got %s" % t.dtype)


def k_blocks(p):
    return lib().qsa_k_blocks(ctypes.byref(p))


# ---- entry points (same names as the C ABI) --------------------------------

def qsa_pool_keys(p, k_idx, kbar, block_begin, block_end, stream=None):
    """k_idx [B][n_cap][128] -> kbar [B][nb_cap][128], blocks [begin, end)."""
    B, n_cap, _ = k_idx.shape
    _check(lib().qsa_pool_keys(ctypes.byref(p), dtype_code(k_idx), _ptr(k_idx), n_cap,
                               _ptr(kbar), kbar.shape[1], B, block_begin, block_end,
                               _stream(stream)))


def qsa_pool_keys_rmsnorm(p, k_idx, gamma, eps, kbar, block_begin, block_end, stream=None):
    """As qsa_pool_keys with the block mean RMS-normalised (gain gamma, a
    float32 [128] device tensor) before the rotation."""
    B, n_cap, _ = k_idx.shape
    _check(lib().qsa_pool_keys_rmsnorm(ctypes.byref(p), dtype_code(k_idx), _ptr(k_idx), n_cap,
                                       _ptr(gamma), eps, _ptr(kbar), kbar.shape[1], B,
                                       block_begin, block_end, _stream(stream)))


def qsa_index_topk_workspace(p, dtype, B, n_q, nb_cap, decode):
    return lib().qsa_index_topk_workspace(ctypes.byref(p), dtype, B, n_q, nb_cap, int(decode))


def qsa_index_topk(p, q_idx, kbar, idx, cnt, workspace, q_pos0=0, seq_len=None, stream=None):
    """q_idx [B][n_q][h_idx][128], kbar [B][nb_cap][128] -> idx [B][n_q][k_B], cnt [B][n_q]."""
    B, n_q = q_idx.shape[0], q_idx.shape[1]
    if q_idx.dim() != 4 or q_idx.shape[2] != p.h_idx:
        raise ValueError("q_idx must be [B][n_q][h_idx=%d][d]" % p.h_idx)
    _check(lib().qsa_index_topk(ctypes.byref(p), dtype_code(q_idx), _ptr(q_idx), _ptr(kbar),
                                kbar.shape[1], B, n_q, q_pos0, _ptr(seq_len), _ptr(idx),
                                _ptr(cnt), _ptr(workspace),
                                0 if workspace is None else workspace.numel(),
                                _stream(stream)))


def qsa_sparse_attn_prefill(p, q, k, v, idx, cnt, out, q_pos0=0, scale=0.0, stream=None):
    """q [B][n_q][hq][d], k/v [B][hkv][n_cap][d] -> out [B][n_q][hq][d]."""
    B, n_q, hq, d = q.shape
    hkv, n_cap = k.shape[1], k.shape[2]
    _check(lib().qsa_sparse_attn_prefill(ctypes.byref(p), dtype_code(q), _ptr(q), _ptr(k),
                                         _ptr(v), n_cap, _ptr(idx), _ptr(cnt), B, n_q, q_pos0,
                                         hq, hkv, d, scale, _ptr(out), _stream(stream)))


def qsa_sparse_attn_decode_workspace(p, B, n_q, hq, hkv, d=128):
    return lib().qsa_sparse_attn_decode_workspace(ctypes.byref(p), B, n_q, hq, hkv, d)


def qsa_sparse_attn_decode(p, q, k_cache, v_cache, seq_len, idx, cnt, out, workspace, scale=0.0,
                           stream=None):
    """q [B][n_q][hq][d], caches [B][hkv][n_cap][d], seq_len int32 [B] (device)."""
    B, n_q, hq, d = q.shape
    hkv, n_cap = k_cache.shape[1], k_cache.shape[2]
    _check(lib().qsa_sparse_attn_decode(ctypes.byref(p), dtype_code(q), _ptr(q), _ptr(k_cache),
                                        _ptr(v_cache), n_cap, _ptr(seq_len), _ptr(idx), _ptr(cnt),
                                        B, n_q, hq, hkv, d, scale, _ptr(out), _ptr(workspace),
                                        0 if workspace is None else workspace.numel(),
                                        _stream(stream)))


def qsa_sparse_attn_decode_shared(p, q, k_cache, v_cache, seq_len, idx, cnt, out, workspace,
                                  scale=0.0, stream=None):
    """n_q new tokens per sequence sharing the selection idx [B][1][k_B] made
    at the first new token (position seq_len[b] - n_q)."""
    B, n_q, hq, d = q.shape
    hkv, n_cap = k_cache.shape[1], k_cache.shape[2]
    _check(lib().qsa_sparse_attn_decode_shared(ctypes.byref(p), dtype_code(q), _ptr(q),
                                               _ptr(k_cache), _ptr(v_cache), n_cap, _ptr(seq_len),
                                               _ptr(idx), _ptr(cnt), B, n_q, hq, hkv, d, scale,
                                               _ptr(out), _ptr(workspace),
                                               0 if workspace is None else workspace.numel(),
                                               _stream(stream)))


def qsa_sparse_attn_decode_noalloc(p, q, k_cache, v_cache, seq_len, idx, cnt, out, scale=0.0,
                                   stream=None):
    """qsa_sparse_attn_decode with the library's fixed scratch (no workspace)."""
    B, n_q, hq, d = q.shape
    hkv, n_cap = k_cache.shape[1], k_cache.shape[2]
    _check(lib().qsa_sparse_attn_decode_noalloc(ctypes.byref(p), dtype_code(q), _ptr(q),
                                                _ptr(k_cache), _ptr(v_cache), n_cap,
                                                _ptr(seq_len), _ptr(idx), _ptr(cnt), B, n_q, hq,
                                                hkv, d, scale, _ptr(out), _stream(stream)))


def qsa_sparse_attn_backward_workspace(p, B, n_q, q_pos0, hq):
    return lib().qsa_sparse_attn_backward_workspace(ctypes.byref(p), B, n_q, q_pos0, hq)


def qsa_sparse_attn_backward(p, q, k, v, idx, cnt, out, dout, dq, dk, dv, workspace, q_pos0=0,
                             scale=0.0, stream=None):
    """Gradients of the sparse attention (bf16 inputs): dq [B][n_q][hq][d]
    float32 written; dk, dv [B][hkv][n_cap][d] float32 added to."""
    B, n_q, hq, d = q.shape
    hkv, n_cap = k.shape[1], k.shape[2]
    _check(lib().qsa_sparse_attn_backward(ctypes.byref(p), dtype_code(q), _ptr(q), _ptr(k),
                                          _ptr(v), n_cap, _ptr(idx), _ptr(cnt), _ptr(out),
                                          _ptr(dout), B, n_q, q_pos0, hq, hkv, d, scale, _ptr(dq),
                                          _ptr(dk), _ptr(dv), _ptr(workspace),
                                          0 if workspace is None else workspace.numel(),
                                          _stream(stream)))


def qsa_index_distill_workspace(p, B, n_q, q_pos0=0):
    return lib().qsa_index_distill_workspace(ctypes.byref(p), B, n_q, q_pos0)


def qsa_index_distill(p, q, k, q_idx, kbar, loss, dq_idx, dkbar, workspace, q_pos0=0, scale=0.0,
                      stream=None):
    """Stage-1 distillation of the indexer: loss [B][n_q] and dq_idx
    [B][n_q][4][128] written, dkbar [B][nb_cap][128] added to (float32);
    workspace of qsa_index_distill_workspace bytes."""
    B, n_q, hq, d = q.shape
    hkv, n_cap = k.shape[1], k.shape[2]
    _check(lib().qsa_index_distill(ctypes.byref(p), dtype_code(q), _ptr(q), _ptr(k), n_cap,
                                   _ptr(q_idx), _ptr(kbar), kbar.shape[1], B, n_q, q_pos0, hq, hkv,
                                   d, scale, _ptr(loss), _ptr(dq_idx), _ptr(dkbar),
                                   _ptr(workspace),
                                   0 if workspace is None else workspace.numel(),
                                   _stream(stream)))


def qsa_pool_keys_backward(p, dkbar, dk_idx, block_begin, block_end, stream=None):
    """dk_idx [B][n_cap][128] rows of blocks [begin, end) from dkbar
    [B][nb_cap][128] (float32)."""
    B = dkbar.shape[0]
    _check(lib().qsa_pool_keys_backward(ctypes.byref(p), _ptr(dkbar), dkbar.shape[1],
                                        _ptr(dk_idx), dk_idx.shape[1], B, block_begin, block_end,
                                        _stream(stream)))


def qsa_dense_attn_prefill(q, k, v, out, q_pos0=0, scale=0.0, stream=None):
    """Dense causal GQA attention: q [B][n_q][hq][d] at positions q_pos0 + t,
    k/v [B][hkv][n_cap][d] -> out [B][n_q][hq][d] (bf16)."""
    B, n_q, hq, d = q.shape
    hkv, n_cap = k.shape[1], k.shape[2]
    _check(lib().qsa_dense_attn_prefill(dtype_code(q), _ptr(q), _ptr(k), _ptr(v), n_cap, B, n_q,
                                        q_pos0, hq, hkv, d, scale, _ptr(out), _stream(stream)))


def qsa_dense_attn_decode_workspace(B, n_q, hkv, n_cap):
    return lib().qsa_dense_attn_decode_workspace(B, n_q, hkv, n_cap)


def qsa_dense_attn_decode(q, k_cache, v_cache, seq_len, out, workspace, scale=0.0, stream=None):
    """Dense causal GQA attention of n_q new tokens per sequence (positions
    seq_len[b] - n_q + t) against the caches."""
    B, n_q, hq, d = q.shape
    hkv, n_cap = k_cache.shape[1], k_cache.shape[2]
    _check(lib().qsa_dense_attn_decode(dtype_code(q), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                       n_cap, _ptr(seq_len), B, n_q, hq, hkv, d, scale,
                                       _ptr(out), _ptr(workspace),
                                       0 if workspace is None else workspace.numel(),
                                       _stream(stream)))


def qsa_probe_gather(p, k, v, idx, cnt, sink, waves_per_cu=8, depth=1, rows_per_wave=1,
                     q_pos0=0, stream=None):
    """Memory-only replay of the prefill attention's gathers (measurement
    aid; include/qsa_probe.h).  sink: uint32, one word per wave."""
    B, hkv, n_cap = k.shape[0], k.shape[1], k.shape[2]
    n_q = idx.shape[1]
    _check(lib().qsa_probe_gather(ctypes.byref(p), _ptr(k), _ptr(v), n_cap, _ptr(idx), _ptr(cnt),
                                  B, n_q, q_pos0, hkv, waves_per_cu, depth, rows_per_wave,
                                  _ptr(sink), _stream(stream)))


# ---- the whole path (sequences of the calls above) -------------------------

def workspace(nbytes, device="cuda"):
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def prefill(p, k_idx, q_idx, q, k, v, stream=None, ws=None):
    """pool -> index_topk -> sparse_attn_prefill for rows 0..n-1 of every
    sequence.  Returns (kbar, idx, cnt, out) as device tensors."""
    import torch
    B, n, d_idx = k_idx.shape
    nb = n // p.r
    dev = k_idx.device
    kB = k_blocks(p)
    kbar = torch.empty((B, nb, d_idx), dtype=k_idx.dtype, device=dev)
    qsa_pool_keys(p, k_idx, kbar, 0, nb, stream)
    n_q = q_idx.shape[1]
    idx = torch.empty((B, n_q, kB), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, n_q), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(qsa_index_topk_workspace(p, dtype_code(q_idx), B, n_q, nb, False), dev)
    qsa_index_topk(p, q_idx, kbar, idx, cnt, ws, 0, None, stream)
    out = torch.empty_like(q)
    qsa_sparse_attn_prefill(p, q, k, v, idx, cnt, out, 0, 0.0, stream)
    return kbar, idx, cnt, out
