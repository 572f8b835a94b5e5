// C ABI of libqsa: argument validation on the host, then kernel launches on
// the caller's stream.  Declared and documented in include/qsa.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "qsa_internal.h"
#include "../../include/qsa_probe.h"

using namespace qsa;

static thread_local char g_err[512];

static qsa_status fail(qsa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

static qsa_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(QSA_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  g_err[0] = 0;
  return QSA_OK;
}

static int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

static qsa_status check_params(const qsa_params* p) {
  if (!p) return fail(QSA_ERR_NULL, "params is NULL");
  if (p->r != 1 && p->r != 2 && p->r != 4 && p->r != 8 && p->r != 16)
    return fail(QSA_ERR_UNSUPPORTED, "r=%d: built for r in {1, 2, 4, 8, 16}", p->r);
  if (p->K < p->r) return fail(QSA_ERR_SHAPE, "K=%d must be >= r=%d", p->K, p->r);
  if (p->h_idx != 1 && p->h_idx != 2 && p->h_idx != 4)
    return fail(QSA_ERR_UNSUPPORTED, "h_idx=%d: built for 1, 2 or 4 indexer heads", p->h_idx);
  if (p->d_idx != 128) return fail(QSA_ERR_UNSUPPORTED, "d_idx=%d: only 128", p->d_idx);
  if (p->rope_dims < 0 || p->rope_dims > 128 || (p->rope_dims & 1))
    return fail(QSA_ERR_UNSUPPORTED, "rope_dims=%d must be even and <= 128", p->rope_dims);
  if (!(p->rope_theta > 0.f) || !isfinite(p->rope_theta))
    return fail(QSA_ERR_SHAPE, "rope_theta must be positive and finite");
  return QSA_OK;
}

static qsa_status check_dtype(qsa_dtype dt) {
  if (dt != QSA_FP32 && dt != QSA_BF16) return fail(QSA_ERR_DTYPE, "unknown dtype %d", (int)dt);
  return QSA_OK;
}

extern "C" {

void qsa_default_params(qsa_params* p) {
  if (!p) return;
  p->r = 4;
  p->K = 2048;
  p->h_idx = 4;
  p->d_idx = 128;
  p->rope_dims = 64;
  p->rope_theta = 10000.f;
}

int32_t qsa_k_blocks(const qsa_params* p) {
  if (!p || p->r <= 0) return 0;
  return (p->K + p->r - 1) / p->r;
}

const char* qsa_status_str(qsa_status s) {
  switch (s) {
    case QSA_OK: return "QSA_OK";
    case QSA_ERR_NULL: return "QSA_ERR_NULL";
    case QSA_ERR_SHAPE: return "QSA_ERR_SHAPE";
    case QSA_ERR_DTYPE: return "QSA_ERR_DTYPE";
    case QSA_ERR_UNSUPPORTED: return "QSA_ERR_UNSUPPORTED";
    case QSA_ERR_WORKSPACE: return "QSA_ERR_WORKSPACE";
    case QSA_ERR_LAUNCH: return "QSA_ERR_LAUNCH";
  }
  return "QSA_ERR_UNKNOWN";
}

const char* qsa_last_error(void) { return g_err; }

qsa_status qsa_pool_keys(const qsa_params* p, qsa_dtype dtype, const void* k_idx, int64_t n_cap,
                         void* kbar, int64_t nb_cap, int32_t B, int64_t block_begin,
                         int64_t block_end, void* stream) {
  qsa_status s = check_params(p);
  if (s) return s;
  if ((s = check_dtype(dtype))) return s;
  if (!k_idx || !kbar) return fail(QSA_ERR_NULL, "k_idx or kbar is NULL");
  if (B < 0 || n_cap < 0 || nb_cap < 0 || block_begin < 0 || block_begin > block_end)
    return fail(QSA_ERR_SHAPE, "bad sizes or block range");
  if (block_end * (int64_t)p->r > n_cap)
    return fail(QSA_ERR_SHAPE, "block_end*r=%lld exceeds n_cap=%lld",
                (long long)(block_end * p->r), (long long)n_cap);
  if (block_end > nb_cap)
    return fail(QSA_ERR_SHAPE, "block_end=%lld exceeds nb_cap=%lld", (long long)block_end,
                (long long)nb_cap);
  return launched(launch_pool(dtype, *p, k_idx, n_cap, kbar, nb_cap, B, block_begin, block_end,
                              nullptr, 0.f, (hipStream_t)stream),
                  "pool_keys");
}

qsa_status qsa_pool_keys_rmsnorm(const qsa_params* p, qsa_dtype dtype, const void* k_idx,
                                 int64_t n_cap, const float* gamma, float eps, void* kbar,
                                 int64_t nb_cap, int32_t B, int64_t block_begin,
                                 int64_t block_end, void* stream) {
  qsa_status s = check_params(p);
  if (s) return s;
  if ((s = check_dtype(dtype))) return s;
  if (!k_idx || !kbar || !gamma) return fail(QSA_ERR_NULL, "k_idx, gamma or kbar is NULL");
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(QSA_ERR_SHAPE, "eps must be finite and >= 0");
  if (B < 0 || n_cap < 0 || nb_cap < 0 || block_begin < 0 || block_begin > block_end)
    return fail(QSA_ERR_SHAPE, "bad sizes or block range");
  if (block_end * (int64_t)p->r > n_cap)
    return fail(QSA_ERR_SHAPE, "block_end*r=%lld exceeds n_cap=%lld",
                (long long)(block_end * p->r), (long long)n_cap);
  if (block_end > nb_cap)
    return fail(QSA_ERR_SHAPE, "block_end=%lld exceeds nb_cap=%lld", (long long)block_end,
                (long long)nb_cap);
  return launched(launch_pool(dtype, *p, k_idx, n_cap, kbar, nb_cap, B, block_begin, block_end,
                              gamma, eps, (hipStream_t)stream),
                  "pool_keys_rmsnorm");
}

static bool decode_split_path(int32_t n_q) { return n_q <= 4; }

size_t qsa_index_topk_workspace(const qsa_params* p, qsa_dtype dtype, int32_t B, int32_t n_q,
                                int64_t nb_cap, int32_t decode) {
  (void)dtype;
  if (!p || B <= 0 || n_q <= 0 || nb_cap < 0) return 0;
  const int kB = qsa_k_blocks(p);
  if (decode && decode_split_path(n_q)) return index_decode_workspace(B, n_q, nb_cap);
  return index_prefill_workspace(B, n_q, num_cus(), kB);
}

qsa_status qsa_index_topk(const qsa_params* p, qsa_dtype dtype, const void* q_idx,
                          const void* kbar, int64_t nb_cap, int32_t B, int32_t n_q,
                          int64_t q_pos0, const int32_t* d_seq_len, int32_t* idx, int32_t* cnt,
                          void* workspace, size_t workspace_bytes, void* stream) {
  qsa_status s = check_params(p);
  if (s) return s;
  if ((s = check_dtype(dtype))) return s;
  if (!q_idx || !kbar || !idx || !cnt) return fail(QSA_ERR_NULL, "NULL tensor argument");
  if (B < 0 || n_q < 1 || nb_cap < 0) return fail(QSA_ERR_SHAPE, "B>=0, n_q>=1, nb_cap>=0");
  if (nb_cap > (int64_t)0x7fffffff) return fail(QSA_ERR_UNSUPPORTED, "nb_cap beyond 2^31");
  if (!d_seq_len) {
    if (q_pos0 < 0) return fail(QSA_ERR_SHAPE, "q_pos0 < 0");
    if ((q_pos0 + n_q) / p->r > nb_cap)
      return fail(QSA_ERR_SHAPE, "queries up to position %lld see %lld blocks > nb_cap=%lld",
                  (long long)(q_pos0 + n_q - 1), (long long)((q_pos0 + n_q) / p->r),
                  (long long)nb_cap);
    if (q_pos0 + n_q > (int64_t)0x7fffffff) return fail(QSA_ERR_UNSUPPORTED, "positions >= 2^31");
  }
  const int kB = qsa_k_blocks(p);
  if (B == 0) return QSA_OK;
  const bool dec = d_seq_len && decode_split_path(n_q);
  // the candidate lists of the many-row kernels hold 4096 entries and are cut
  // back to k_B whenever a stage could overflow them: k_B must stay well
  // below that; the decode lists hold 6016
  if (!dec && kB > kMaxKBlocksRows)
    return fail(QSA_ERR_UNSUPPORTED, "k_B=%d: the many-row indexer is built for k_B <= %d", kB,
                kMaxKBlocksRows);
  if (dec && kB > kMaxKBlocksDecode)
    return fail(QSA_ERR_UNSUPPORTED, "k_B=%d: the decode indexer is built for k_B <= %d", kB,
                kMaxKBlocksDecode);
  const size_t need = qsa_index_topk_workspace(p, dtype, B, n_q, nb_cap, d_seq_len != nullptr);
  if (!workspace || workspace_bytes < need)
    return fail(QSA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  IndexArgs a;
  a.q_idx = q_idx;
  a.kbar = kbar;
  a.nb_cap = nb_cap;
  a.B = B;
  a.n_q = n_q;
  a.q_pos0 = q_pos0;
  a.seq_len = d_seq_len;
  a.idx = idx;
  a.cnt = cnt;
  a.kB = kB;
  a.r = p->r;
  a.R = p->rope_dims;
  a.h = p->h_idx;
  a.log2_theta = log2((double)p->rope_theta);
  hipError_t e = dec ? launch_index_decode(dtype, a, workspace, (hipStream_t)stream)
                     : launch_index_prefill(dtype, a, workspace, num_cus(), (hipStream_t)stream);
  return launched(e, "index_topk");
}

static qsa_status check_attn(const qsa_params* p, qsa_dtype dtype, const void* q, const void* k,
                             const void* v, const int32_t* idx, const int32_t* cnt, void* out,
                             int32_t B, int32_t n_q, int32_t hq, int32_t hkv, int32_t d,
                             int64_t n_cap) {
  qsa_status s = check_params(p);
  if (s) return s;
  if ((s = check_dtype(dtype))) return s;
  if (!q || !k || !v || !idx || !cnt || !out) return fail(QSA_ERR_NULL, "NULL tensor argument");
  if (B < 0 || n_q < 1 || hq < 1 || hkv < 1 || n_cap < 1)
    return fail(QSA_ERR_SHAPE, "B>=0, n_q>=1, hq>=1, hkv>=1, n_cap>=1");
  if (hq % hkv) return fail(QSA_ERR_SHAPE, "hq=%d not a multiple of hkv=%d", hq, hkv);
  if (hq / hkv > 16) return fail(QSA_ERR_UNSUPPORTED, "hq/hkv=%d > 16", hq / hkv);
  if (d != 128) return fail(QSA_ERR_UNSUPPORTED, "head dim %d: only 128", d);
  // the bf16 kernels address a head's K/V rows with 32-bit byte offsets
  if (dtype == QSA_BF16 && n_cap > kMaxCapBf16)
    return fail(QSA_ERR_UNSUPPORTED, "n_cap=%lld: bf16 attention is built for n_cap <= %lld",
                (long long)n_cap, (long long)kMaxCapBf16);
  return QSA_OK;
}

qsa_status qsa_sparse_attn_prefill(const qsa_params* p, qsa_dtype dtype, const void* q,
                                   const void* k, const void* v, int64_t n_cap,
                                   const int32_t* idx, const int32_t* cnt, int32_t B,
                                   int32_t n_q, int64_t q_pos0, int32_t hq, int32_t hkv,
                                   int32_t d, float scale, void* out, void* stream) {
  qsa_status s = check_attn(p, dtype, q, k, v, idx, cnt, out, B, n_q, hq, hkv, d, n_cap);
  if (s) return s;
  if (q_pos0 < 0 || q_pos0 + n_q > n_cap)
    return fail(QSA_ERR_SHAPE, "positions [%lld, %lld) exceed n_cap=%lld", (long long)q_pos0,
                (long long)(q_pos0 + n_q), (long long)n_cap);
  if (B == 0) return QSA_OK;
  AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.idx = idx;
  a.cnt = cnt;
  a.seq_len = nullptr;
  a.n_cap = n_cap;
  a.q_pos0 = q_pos0;
  a.B = B;
  a.n_q = n_q;
  a.hq = hq;
  a.hkv = hkv;
  a.kB = qsa_k_blocks(p);
  a.r = p->r;
  a.shared = 0;
  a.scale = scale > 0.f ? scale : 1.f / sqrtf((float)d);
  return launched(launch_attn_prefill(dtype, a, (hipStream_t)stream), "sparse_attn_prefill");
}

size_t qsa_sparse_attn_decode_workspace(const qsa_params* p, int32_t B, int32_t n_q, int32_t hq,
                                        int32_t hkv, int32_t d) {
  (void)hq;
  (void)d;
  if (!p || B <= 0 || n_q <= 0 || hkv <= 0) return 0;
  // sized for either form of the decode call (a shared selection can add a
  // tail slot)
  return attn_decode_workspace(B, n_q, hkv, qsa_k_blocks(p), p->r, true);
}

qsa_status qsa_sparse_attn_decode(const qsa_params* p, qsa_dtype dtype, const void* q,
                                  const void* k_cache, const void* v_cache, int64_t n_cap,
                                  const int32_t* d_seq_len, const int32_t* idx,
                                  const int32_t* cnt, int32_t B, int32_t n_q, int32_t hq,
                                  int32_t hkv, int32_t d, float scale, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  qsa_status s = check_attn(p, dtype, q, k_cache, v_cache, idx, cnt, out, B, n_q, hq, hkv, d,
                            n_cap);
  if (s) return s;
  if (!d_seq_len) return fail(QSA_ERR_NULL, "d_seq_len is NULL");
  if (B == 0) return QSA_OK;
  const size_t need = qsa_sparse_attn_decode_workspace(p, B, n_q, hq, hkv, d);
  if (!workspace || workspace_bytes < need)
    return fail(QSA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  AttnArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.out = out;
  a.idx = idx;
  a.cnt = cnt;
  a.seq_len = d_seq_len;
  a.n_cap = n_cap;
  a.q_pos0 = 0;
  a.B = B;
  a.n_q = n_q;
  a.hq = hq;
  a.hkv = hkv;
  a.kB = qsa_k_blocks(p);
  a.r = p->r;
  a.shared = 0;
  a.scale = scale > 0.f ? scale : 1.f / sqrtf((float)d);
  return launched(launch_attn_decode(dtype, a, workspace, (hipStream_t)stream),
                  "sparse_attn_decode");
}

qsa_status qsa_sparse_attn_decode_shared(const qsa_params* p, qsa_dtype dtype, const void* q,
                                         const void* k_cache, const void* v_cache, int64_t n_cap,
                                         const int32_t* d_seq_len, const int32_t* idx,
                                         const int32_t* cnt, int32_t B, int32_t n_q, int32_t hq,
                                         int32_t hkv, int32_t d, float scale, void* out,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  qsa_status s = check_attn(p, dtype, q, k_cache, v_cache, idx, cnt, out, B, n_q, hq, hkv, d,
                            n_cap);
  if (s) return s;
  if (!d_seq_len) return fail(QSA_ERR_NULL, "d_seq_len is NULL");
  if (B == 0) return QSA_OK;
  const size_t need = qsa_sparse_attn_decode_workspace(p, B, n_q, hq, hkv, d);
  if (!workspace || workspace_bytes < need)
    return fail(QSA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  AttnArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.out = out;
  a.idx = idx;
  a.cnt = cnt;
  a.seq_len = d_seq_len;
  a.n_cap = n_cap;
  a.q_pos0 = 0;
  a.B = B;
  a.n_q = n_q;
  a.hq = hq;
  a.hkv = hkv;
  a.kB = qsa_k_blocks(p);
  a.r = p->r;
  a.shared = 1;
  a.scale = scale > 0.f ? scale : 1.f / sqrtf((float)d);
  return launched(launch_attn_decode(dtype, a, workspace, (hipStream_t)stream),
                  "sparse_attn_decode_shared");
}

qsa_status qsa_sparse_attn_decode_noalloc(const qsa_params* p, qsa_dtype dtype, const void* q,
                                          const void* k_cache, const void* v_cache,
                                          int64_t n_cap, const int32_t* d_seq_len,
                                          const int32_t* idx, const int32_t* cnt, int32_t B,
                                          int32_t n_q, int32_t hq, int32_t hkv, int32_t d,
                                          float scale, void* out, void* stream) {
  qsa_status s = check_attn(p, dtype, q, k_cache, v_cache, idx, cnt, out, B, n_q, hq, hkv, d,
                            n_cap);
  if (s) return s;
  if (!d_seq_len) return fail(QSA_ERR_NULL, "d_seq_len is NULL");
  if (B == 0) return QSA_OK;
  const size_t need = qsa_sparse_attn_decode_workspace(p, B, n_q, hq, hkv, d);
  if (need > kDecodeScratchBytes)
    return fail(QSA_ERR_WORKSPACE, "needs %zu bytes of scratch, beyond the fixed %zu", need,
                kDecodeScratchBytes);
  void* ws = nullptr;
  hipError_t e = attn_static_scratch(&ws);
  if (e != hipSuccess) return launched(e, "sparse_attn_decode_noalloc: scratch lookup");
  AttnArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.out = out;
  a.idx = idx;
  a.cnt = cnt;
  a.seq_len = d_seq_len;
  a.n_cap = n_cap;
  a.q_pos0 = 0;
  a.B = B;
  a.n_q = n_q;
  a.hq = hq;
  a.hkv = hkv;
  a.kB = qsa_k_blocks(p);
  a.r = p->r;
  a.shared = 0;
  a.scale = scale > 0.f ? scale : 1.f / sqrtf((float)d);
  return launched(launch_attn_decode(dtype, a, ws, (hipStream_t)stream),
                  "sparse_attn_decode_noalloc");
}

qsa_status qsa_sparse_attn_backward(const qsa_params* p, qsa_dtype dtype, const void* q,
                                    const void* k, const void* v, int64_t n_cap,
                                    const int32_t* idx, const int32_t* cnt, const void* out,
                                    const void* dout, int32_t B, int32_t n_q, int64_t q_pos0,
                                    int32_t hq, int32_t hkv, int32_t d, float scale, float* dq,
                                    float* dk, float* dv, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  qsa_status s = check_attn(p, dtype, q, k, v, idx, cnt, dq, B, n_q, hq, hkv, d, n_cap);
  if (s) return s;
  if (dtype != QSA_BF16) return fail(QSA_ERR_UNSUPPORTED, "the backward is built for bf16");
  if (!out || !dout || !dk || !dv) return fail(QSA_ERR_NULL, "NULL tensor argument");
  if (q_pos0 < 0 || q_pos0 + n_q > n_cap)
    return fail(QSA_ERR_SHAPE, "positions [%lld, %lld) exceed n_cap=%lld", (long long)q_pos0,
                (long long)(q_pos0 + n_q), (long long)n_cap);
  // the transposed selection counts rows in 32-bit integers
  if ((int64_t)n_q * qsa_k_blocks(p) > INT32_MAX)
    return fail(QSA_ERR_UNSUPPORTED, "n_q * k_B beyond 2^31 entries per sequence");
  if (B == 0) return QSA_OK;
  const size_t need = attn_backward_workspace(B, n_q, q_pos0, hq, p->r, qsa_k_blocks(p));
  if (!workspace || workspace_bytes < need)
    return fail(QSA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  AttnArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = const_cast<void*>(out);
  a.idx = idx;
  a.cnt = cnt;
  a.n_cap = n_cap;
  a.q_pos0 = q_pos0;
  a.B = B;
  a.n_q = n_q;
  a.hq = hq;
  a.hkv = hkv;
  a.kB = qsa_k_blocks(p);
  a.r = p->r;
  a.scale = scale > 0.f ? scale : 1.f / sqrtf((float)d);
  return launched(launch_attn_backward(a, dout, dq, dk, dv, workspace, (hipStream_t)stream),
                  "sparse_attn_backward");
}

size_t qsa_sparse_attn_backward_workspace(const qsa_params* p, int32_t B, int32_t n_q,
                                          int64_t q_pos0, int32_t hq) {
  if (!p || check_params(p) || B < 0 || n_q < 1 || hq < 1 || q_pos0 < 0) return 0;
  return attn_backward_workspace(B, n_q, q_pos0, hq, p->r, qsa_k_blocks(p));
}

size_t qsa_index_distill_workspace(const qsa_params* p, int32_t B, int32_t n_q, int64_t q_pos0) {
  if (!p || p->r != 4 || B < 0 || n_q < 1 || q_pos0 < 0) return 0;
  return (size_t)B * (size_t)distill_blocks(q_pos0, n_q) * sizeof(float);
}

qsa_status qsa_index_distill(const qsa_params* p, qsa_dtype dtype, const void* q, const void* k,
                             int64_t n_cap, const void* q_idx, const void* kbar, int64_t nb_cap,
                             int32_t B, int32_t n_q, int64_t q_pos0, int32_t hq, int32_t hkv,
                             int32_t d, float scale, float* loss, float* dq_idx, float* dkbar,
                             void* workspace, size_t workspace_bytes, void* stream) {
  qsa_status s = check_params(p);
  if (s) return s;
  if ((s = check_dtype(dtype))) return s;
  if (dtype != QSA_BF16) return fail(QSA_ERR_UNSUPPORTED, "distillation is built for bf16");
  if (p->h_idx != 4) return fail(QSA_ERR_UNSUPPORTED, "distillation is built for 4 indexer heads");
  if (p->r != 4) return fail(QSA_ERR_UNSUPPORTED, "distillation is built for r = 4");
  if (p->rope_dims > 64) return fail(QSA_ERR_UNSUPPORTED, "distillation: rope_dims <= 64");
  if (!q || !k || !q_idx || !kbar || !loss || !dq_idx || !dkbar)
    return fail(QSA_ERR_NULL, "NULL tensor argument");
  if (B < 0 || n_q < 1 || hq < 1 || hkv < 1 || n_cap < 1 || nb_cap < 0)
    return fail(QSA_ERR_SHAPE, "B>=0, n_q>=1, hq>=1, hkv>=1, n_cap>=1, nb_cap>=0");
  if (hq % hkv) return fail(QSA_ERR_SHAPE, "hq=%d not a multiple of hkv=%d", hq, hkv);
  if (hq > 16 || hkv > 8) return fail(QSA_ERR_UNSUPPORTED, "distillation: hq <= 16, hkv <= 8");
  if (d != 128) return fail(QSA_ERR_UNSUPPORTED, "head dim %d: only 128", d);
  if (q_pos0 < 0 || q_pos0 + n_q > n_cap)
    return fail(QSA_ERR_SHAPE, "positions [%lld, %lld) exceed n_cap=%lld", (long long)q_pos0,
                (long long)(q_pos0 + n_q), (long long)n_cap);
  if ((q_pos0 + n_q) / p->r > nb_cap)
    return fail(QSA_ERR_SHAPE, "positions see more blocks than nb_cap=%lld", (long long)nb_cap);
  if (n_cap > kMaxCapBf16 || q_pos0 + n_q > (int64_t)0x7fffffff)
    return fail(QSA_ERR_UNSUPPORTED, "n_cap beyond %lld", (long long)kMaxCapBf16);
  if (B == 0) return QSA_OK;
  const size_t need = qsa_index_distill_workspace(p, B, n_q, q_pos0);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(QSA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  DistillArgs a;
  a.q = (const unsigned short*)q;
  a.k = (const unsigned short*)k;
  a.q_idx = (const unsigned short*)q_idx;
  a.kbar = (const unsigned short*)kbar;
  a.loss = loss;
  a.dq_idx = dq_idx;
  a.dkbar = dkbar;
  a.aws = (float*)workspace;
  a.aws_ld = distill_blocks(q_pos0, n_q);
  a.n_cap = n_cap;
  a.nb_cap = nb_cap;
  a.q_pos0 = q_pos0;
  a.B = B;
  a.n_q = n_q;
  a.hq = hq;
  a.hkv = hkv;
  a.R = p->rope_dims;
  a.scale = scale > 0.f ? scale : 1.f / sqrtf((float)d);
  a.log2_theta = log2((double)p->rope_theta);
  return launched(launch_distill(a, (hipStream_t)stream), "index_distill");
}

qsa_status qsa_pool_keys_backward(const qsa_params* p, const float* dkbar, int64_t nb_cap,
                                  float* dk_idx, int64_t n_cap, int32_t B, int64_t block_begin,
                                  int64_t block_end, void* stream) {
  qsa_status s = check_params(p);
  if (s) return s;
  if (!dkbar || !dk_idx) return fail(QSA_ERR_NULL, "dkbar or dk_idx is NULL");
  if (B < 0 || n_cap < 0 || nb_cap < 0 || block_begin < 0 || block_begin > block_end)
    return fail(QSA_ERR_SHAPE, "bad sizes or block range");
  if (block_end * (int64_t)p->r > n_cap || block_end > nb_cap)
    return fail(QSA_ERR_SHAPE, "block range beyond n_cap or nb_cap");
  return launched(launch_pool_backward(dkbar, nb_cap, dk_idx, n_cap, B, block_begin, block_end,
                                       p->r, p->rope_dims, log2((double)p->rope_theta),
                                       (hipStream_t)stream),
                  "pool_keys_backward");
}

static qsa_status check_dense(qsa_dtype dtype, const void* q, const void* k, const void* v,
                              void* out, int32_t B, int32_t n_q, int32_t hq, int32_t hkv,
                              int32_t d, int64_t n_cap) {
  qsa_status s = check_dtype(dtype);
  if (s) return s;
  if (dtype != QSA_BF16) return fail(QSA_ERR_UNSUPPORTED, "dense attention is built for bf16");
  if (!q || !k || !v || !out) return fail(QSA_ERR_NULL, "NULL tensor argument");
  if (B < 0 || n_q < 1 || hq < 1 || hkv < 1 || n_cap < 1)
    return fail(QSA_ERR_SHAPE, "B>=0, n_q>=1, hq>=1, hkv>=1, n_cap>=1");
  if (hq % hkv) return fail(QSA_ERR_SHAPE, "hq=%d not a multiple of hkv=%d", hq, hkv);
  if (16 % (hq / hkv))
    return fail(QSA_ERR_UNSUPPORTED, "hq/hkv=%d must divide 16", hq / hkv);
  if (d != 128) return fail(QSA_ERR_UNSUPPORTED, "head dim %d: only 128", d);
  if (n_cap > kMaxCapBf16)
    return fail(QSA_ERR_UNSUPPORTED, "n_cap=%lld: dense attention is built for n_cap <= %lld",
                (long long)n_cap, (long long)kMaxCapBf16);
  return QSA_OK;
}

qsa_status qsa_dense_attn_prefill(qsa_dtype dtype, const void* q, const void* k, const void* v,
                                  int64_t n_cap, int32_t B, int32_t n_q, int64_t q_pos0,
                                  int32_t hq, int32_t hkv, int32_t d, float scale, void* out,
                                  void* stream) {
  qsa_status s = check_dense(dtype, q, k, v, out, B, n_q, hq, hkv, d, n_cap);
  if (s) return s;
  if (q_pos0 < 0 || q_pos0 + n_q > n_cap)
    return fail(QSA_ERR_SHAPE, "positions [%lld, %lld) exceed n_cap=%lld", (long long)q_pos0,
                (long long)(q_pos0 + n_q), (long long)n_cap);
  if (B == 0) return QSA_OK;
  AttnArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.n_cap = n_cap;
  a.q_pos0 = q_pos0;
  a.B = B;
  a.n_q = n_q;
  a.hq = hq;
  a.hkv = hkv;
  a.scale = scale > 0.f ? scale : 1.f / sqrtf((float)d);
  return launched(launch_dense_prefill(a, (hipStream_t)stream), "dense_attn_prefill");
}

size_t qsa_dense_attn_decode_workspace(int32_t B, int32_t n_q, int32_t hkv, int64_t n_cap) {
  if (B <= 0 || n_q <= 0 || hkv <= 0 || n_cap <= 0) return 0;
  return dense_decode_workspace(B, n_q, hkv, n_cap);
}

qsa_status qsa_dense_attn_decode(qsa_dtype dtype, const void* q, const void* k_cache,
                                 const void* v_cache, int64_t n_cap, const int32_t* d_seq_len,
                                 int32_t B, int32_t n_q, int32_t hq, int32_t hkv, int32_t d,
                                 float scale, void* out, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  qsa_status s = check_dense(dtype, q, k_cache, v_cache, out, B, n_q, hq, hkv, d, n_cap);
  if (s) return s;
  if (!d_seq_len) return fail(QSA_ERR_NULL, "d_seq_len is NULL");
  if (n_q * (hq / hkv) > 64)
    return fail(QSA_ERR_UNSUPPORTED, "n_q * hq/hkv = %d > 64", n_q * (hq / hkv));
  if (B == 0) return QSA_OK;
  const size_t need = dense_decode_workspace(B, n_q, hkv, n_cap);
  if (!workspace || workspace_bytes < need)
    return fail(QSA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  AttnArgs a = {};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.out = out;
  a.seq_len = d_seq_len;
  a.n_cap = n_cap;
  a.B = B;
  a.n_q = n_q;
  a.hq = hq;
  a.hkv = hkv;
  a.scale = scale > 0.f ? scale : 1.f / sqrtf((float)d);
  return launched(launch_dense_decode(a, workspace, (hipStream_t)stream), "dense_attn_decode");
}

qsa_status qsa_probe_gather(const qsa_params* p, const void* k, const void* v, int64_t n_cap,
                            const int32_t* idx, const int32_t* cnt, int32_t B, int32_t n_q,
                            int64_t q_pos0, int32_t hkv, int32_t waves_per_cu, int32_t depth,
                            int32_t rows_per_wave, uint32_t* sink, void* stream) {
  qsa_status s = check_attn(p, QSA_BF16, k, k, v, idx, cnt, sink, B, n_q, hkv, hkv, 128, n_cap);
  if (s) return s;
  if (p->r != 4) return fail(QSA_ERR_UNSUPPORTED, "the probe reads 4-token blocks");
  if (qsa_k_blocks(p) % 8) return fail(QSA_ERR_UNSUPPORTED, "the probe needs k_B % 8 == 0");
  if (depth < 1 || depth > 4) return fail(QSA_ERR_SHAPE, "depth=%d outside 1..4", depth);
  if (rows_per_wave < 1 || rows_per_wave > 64)
    return fail(QSA_ERR_SHAPE, "rows_per_wave=%d outside 1..64", rows_per_wave);
  if (q_pos0 < 0 || q_pos0 + n_q > n_cap)
    return fail(QSA_ERR_SHAPE, "positions [%lld, %lld) exceed n_cap=%lld", (long long)q_pos0,
                (long long)(q_pos0 + n_q), (long long)n_cap);
  if (B == 0) return QSA_OK;
  AttnArgs a;
  a.q = nullptr;
  a.k = k;
  a.v = v;
  a.out = nullptr;
  a.idx = idx;
  a.cnt = cnt;
  a.seq_len = nullptr;
  a.n_cap = n_cap;
  a.q_pos0 = q_pos0;
  a.B = B;
  a.n_q = n_q;
  a.hq = hkv;
  a.hkv = hkv;
  a.kB = qsa_k_blocks(p);
  a.r = p->r;
  a.shared = 0;
  a.scale = 1.f;
  return launched(launch_probe_gather(a, waves_per_cu, depth, rows_per_wave, sink,
                                      (hipStream_t)stream),
                  "probe_gather");
}

}  // extern "C"
