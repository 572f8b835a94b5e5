/*
 * qsa.h -- C ABI of the MI355X (gfx950) Qwen Sparse Attention (QSA) hot path.
 *
 * The method (cited by site and section; every page describes the report
 * "On the Design of Qwen3.8-Next Architecture: Evaluation, Efficiency, and
 * Training Stability"):
 *   [hub]   gunjandhanuka.github.io research-hub note, "Key ideas", the QSA
 *           compressed-indexer bullet: MQA indexer with 4 query heads and one
 *           shared 128-dim key head; keys average-pooled into blocks of r;
 *           partial RoPE (64 of 128 dims) after compression;
 *           I_ib = sum_h ReLU(<q_i^h, kbar_b>); top-k_B = ceil(K/r) blocks
 *           plus the current-block tail; K = 2048, r = 4.
 *   [glide] paperglide.net reader, section "Qwen Sparse Attention": toy
 *           walk-through (pool, block-causal scores, top-K_B, expansion to
 *           token indices, incomplete-block tail) and Figure 3 (indexer ->
 *           top-k indices -> micro-block sparse mask -> sparse core
 *           attention); section "QSA Ablations and Efficiency", Figure 6
 *           (prefill and decode kernels: indexer + sparse core attention).
 *
 * Conventions shared by every entry point:
 *   - All tensor arguments are caller-owned DEVICE pointers, contiguous,
 *     16-byte aligned, in the layouts stated per argument (row-major, the
 *     last index fastest).  `dtype` selects float32 or bfloat16 storage for
 *     every floating-point tensor of the call; indices are int32.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call
 *     validates its arguments on the host, enqueues its kernels on `stream`
 *     and returns without synchronising.  Kernel faults surface at the
 *     caller's next synchronisation.
 *   - The library allocates no device memory.  Scratch memory comes only
 *     from the `workspace` arguments, sized by the *_workspace functions;
 *     its contents need no initialisation and are not preserved.
 *   - On error a call returns a non-zero qsa_status, launches nothing,
 *     writes no output, and records a message for qsa_last_error() (per host
 *     thread).  No C++ exception crosses this boundary.
 *   - Positions: query row t of sequence b sits at token position
 *     p = q_pos0 + t (prefill), or p = d_seq_len[b] - n_q + t when the
 *     device array d_seq_len is given (decode: the new tokens are already
 *     in the caches).  Block b is visible to position p iff (b+1)r-1 <= p.
 *   - Inputs must be finite; NaN or Inf give undefined selections.
 *   - Results are deterministic: identical inputs give identical bits.
 *   - Supported shapes: r in {1, 2, 4, 8, 16}, h_idx in {1, 2, 4} (q_idx
 *     then holds h_idx heads per token), d_idx = 128, rope_dims even and
 *     <= 128, K >= r, head dim d = 128, hq % hkv == 0, hq / hkv <= 16;
 *     k_B = ceil(K/r) <= 3072 for qsa_index_topk over more than 4 query rows
 *     per sequence and <= 4096 for its decode form (at most 4 new tokens);
 *     n_cap <= 2^24 tokens for bfloat16 attention.  Other values return
 *     QSA_ERR_UNSUPPORTED.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QSA_OK = 0,
  QSA_ERR_NULL = 1,        /* a required pointer is NULL */
  QSA_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes */
  QSA_ERR_DTYPE = 3,       /* unknown dtype */
  QSA_ERR_UNSUPPORTED = 4, /* valid by the method, not built here */
  QSA_ERR_WORKSPACE = 5,   /* workspace missing or too small */
  QSA_ERR_LAUNCH = 6       /* the HIP runtime refused a launch */
} qsa_status;

typedef enum { QSA_FP32 = 0, QSA_BF16 = 1 } qsa_dtype;

/* Method constants ([hub]): defaults r = 4, K = 2048 (k_B = 512),
 * h_idx = 4, d_idx = 128, rope_dims = 64, rope_theta = 10000. */
typedef struct {
  int32_t r;         /* micro-block size: tokens per pooled key */
  int32_t K;         /* token budget; k_B = ceil(K / r) selected blocks */
  int32_t h_idx;     /* indexer query heads */
  int32_t d_idx;     /* indexer head dimension */
  int32_t rope_dims; /* leading indexer dims rotated after pooling */
  float rope_theta;  /* RoPE base: pair (j, j + rope_dims/2) turns by
                        p * theta^(-2j / rope_dims) at position p */
} qsa_params;

/* Fills *p with the defaults above. */
void qsa_default_params(qsa_params* p);

/* k_B = ceil(K / r): the number of blocks each query selects at most. */
int32_t qsa_k_blocks(const qsa_params* p);

/* Human-readable name of a status code (static string). */
const char* qsa_status_str(qsa_status s);

/* Detail of the last error on this host thread ("" if none). */
const char* qsa_last_error(void);

/*
 * qsa_pool_keys -- pooled indexer keys ([hub]: average-pool the shared key
 * head over blocks of r tokens, then partial RoPE after compression;
 * [glide] toy: block 0 = (k0 + k1) / 2).
 *
 *   kbar[b][j][c] = RoPE_{(j+1)r-1}( (1/r) sum_{t<r} k_idx[b][j*r+t][c] )
 *   for every sequence b < B and block j in [block_begin, block_end); RoPE
 *   acts on dims c < rope_dims only.  Result rounded (nearest-even) to dtype.
 *
 *   k_idx : [B][n_cap][d_idx]   indexer keys of every token
 *   kbar  : [B][nb_cap][d_idx]  pooled key cache (rows outside the range
 *                               are left untouched)
 * Errors: NULL pointers; block_end * r > n_cap or block_end > nb_cap or
 * block_begin > block_end -> QSA_ERR_SHAPE.
 */
qsa_status qsa_pool_keys(const qsa_params* p, qsa_dtype dtype, const void* k_idx, int64_t n_cap,
                         void* kbar, int64_t nb_cap, int32_t B, int64_t block_begin,
                         int64_t block_end, void* stream);

/*
 * qsa_pool_keys_rmsnorm -- qsa_pool_keys with the block mean RMS-normalised
 * before the rotation ([glide] "Qwen Sparse Attention": the toy applies
 * RMSNorm to the average-pooled keys; [hub]: the partial RoPE comes after
 * the compression):
 *
 *   m = (1/r) sum_{t<r} k_idx[b][j*r+t],   y[c] = m[c] * gamma[c] / sqrt(mean_c(m^2) + eps)
 *   kbar[b][j] = RoPE_{(j+1)r-1}(y), rounded (nearest-even) to dtype.
 *
 *   gamma : device float32 [d_idx], the learned gain;  eps >= 0
 * Errors as for qsa_pool_keys; gamma NULL -> QSA_ERR_NULL; eps negative or
 * not finite -> QSA_ERR_SHAPE.
 */
qsa_status qsa_pool_keys_rmsnorm(const qsa_params* p, qsa_dtype dtype, const void* k_idx,
                                 int64_t n_cap, const float* gamma, float eps, void* kbar,
                                 int64_t nb_cap, int32_t B, int64_t block_begin,
                                 int64_t block_end, void* stream);

/*
 * qsa_index_topk -- compressed MQA indexer and top-k_B block selection
 * ([hub]: I_ib = sum_h ReLU(<q_i^h, kbar_b>) with partial RoPE on the query
 * at its position, top-k_B = ceil(K/r); [glide]: the compressed causal mask,
 * "select the top K_B blocks per query").
 *
 * For each query row: the min(k_B, visible) blocks with the largest score
 * under the total order (score descending, block id ascending), written as
 * ascending block ids, padded with -1.  The score matrix is never stored.
 * Precision: with bfloat16 the rotated query keeps float accuracy (each
 * element carried as a bf16 high part plus a bf16 low part on the rotated
 * dims) against the bf16 pooled keys, accumulated in float32; with float32
 * both operands stay float32.  Blocks whose scores differ by less than the
 * accumulation's rounding may be ordered either way.
 *
 *   q_idx : [B][n_q][h_idx][d_idx]  indexer queries, NOT rotated (h_idx
 *                                   is 1, 2 or 4)
 *   kbar  : [B][nb_cap][d_idx]      pooled keys from qsa_pool_keys
 *   d_seq_len : NULL (prefill: positions q_pos0 + t) or device int32 [B]
 *               (decode: positions d_seq_len[b] - n_q + t)
 *   idx   : [B][n_q][k_B] int32 out;  cnt : [B][n_q] int32 out
 *   workspace : device scratch of qsa_index_topk_workspace(...) bytes
 * Errors: NULL pointers; n_q < 1; a prefill position beyond nb_cap * r
 * -> QSA_ERR_SHAPE; workspace too small -> QSA_ERR_WORKSPACE; k_B above
 * 3072 (more than 4 rows per sequence) or 4096 (decode form) ->
 * QSA_ERR_UNSUPPORTED.  In decode
 * mode every d_seq_len[b] must lie in [n_q, nb_cap * r] (not checked on the
 * host: the values live on the device).
 */
qsa_status qsa_index_topk(const qsa_params* p, qsa_dtype dtype, const void* q_idx,
                          const void* kbar, int64_t nb_cap, int32_t B, int32_t n_q,
                          int64_t q_pos0, const int32_t* d_seq_len, int32_t* idx, int32_t* cnt,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes qsa_index_topk needs for these sizes on the current
 * device (decode != 0 when d_seq_len will be given). */
size_t qsa_index_topk_workspace(const qsa_params* p, qsa_dtype dtype, int32_t B, int32_t n_q,
                                int64_t nb_cap, int32_t decode);

/*
 * qsa_sparse_attn_prefill -- sparse core attention ([glide] Figure 3: the
 * selected blocks expanded to tokens, joined with the incomplete-block tail;
 * each query attends to that set only).
 *
 *   T_i = { j*r + u : j in idx[b][t][0..cnt), u < r } U { floor((p+1)/r)*r .. p }
 *   out[b][t][h] = sum_{s in T_i} softmax_s(scale <q[b][t][h], k[b][g][s]>) v[b][g][s]
 *   with g = floor(h * hkv / hq); scale <= 0 means 1/sqrt(d).
 *
 *   q   : [B][n_q][hq][d];  k, v : [B][hkv][n_cap][d] (head-major caches)
 *   idx, cnt : from qsa_index_topk (same n_q, positions)
 *   out : [B][n_q][hq][d]
 * Errors: NULL pointers; q_pos0 + n_q > n_cap -> QSA_ERR_SHAPE; d != 128,
 * hq / hkv > 16, or n_cap > 2^24 with bfloat16 -> QSA_ERR_UNSUPPORTED.
 */
qsa_status qsa_sparse_attn_prefill(const qsa_params* p, qsa_dtype dtype, const void* q,
                                   const void* k, const void* v, int64_t n_cap,
                                   const int32_t* idx, const int32_t* cnt, int32_t B,
                                   int32_t n_q, int64_t q_pos0, int32_t hq, int32_t hkv,
                                   int32_t d, float scale, void* out, void* stream);

/*
 * qsa_sparse_attn_decode -- the same attention for n_q new tokens per
 * sequence against the KV caches (the pages' decode benchmark, Figure 6(d),
 * uses next_n = 4), split over the selected blocks and combined
 * (flash-decoding).  Positions d_seq_len[b] - n_q + t.
 *
 *   q : [B][n_q][hq][d]; k_cache, v_cache : [B][hkv][n_cap][d];
 *   d_seq_len : device int32 [B], includes the new tokens; each length in
 *               [n_q, n_cap] (not checked on the host: the values live on
 *               the device; a length outside reads outside the caches)
 *   idx, cnt : from qsa_index_topk in decode mode for the same lengths;
 *   out : [B][n_q][hq][d]
 *   workspace : qsa_sparse_attn_decode_workspace(...) bytes
 * Errors as for the prefill call, plus QSA_ERR_WORKSPACE.
 */
qsa_status qsa_sparse_attn_decode(const qsa_params* p, qsa_dtype dtype, const void* q,
                                  const void* k_cache, const void* v_cache, int64_t n_cap,
                                  const int32_t* d_seq_len, const int32_t* idx,
                                  const int32_t* cnt, int32_t B, int32_t n_q, int32_t hq,
                                  int32_t hkv, int32_t d, float scale, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of qsa_sparse_attn_decode and qsa_sparse_attn_decode_shared
 * for these sizes (the same for both calls). */
size_t qsa_sparse_attn_decode_workspace(const qsa_params* p, int32_t B, int32_t n_q, int32_t hq,
                                        int32_t hkv, int32_t d);

/*
 * qsa_sparse_attn_decode_shared -- decode attention for n_q new tokens per
 * sequence that share ONE block selection ([glide] "QSA Ablations and
 * Efficiency": reusing the top-k indices across speculative decoding steps
 * leaves the accepted length unchanged, Table 4; Figure 1: the MTP module
 * reuses QSA indices across speculative steps).
 *
 * The selection is the one made for the step's first new token, at
 * position f = d_seq_len[b] - n_q: idx[b][0][..cnt[b][0]] from
 * qsa_index_topk with one query per sequence at that position (decode form
 * with lengths d_seq_len[b] - n_q + 1).  New token t (position f + t)
 * attends to the tokens of those blocks plus every token from
 * floor((f+1)/r)*r to f + t: its own incomplete block and, for the later
 * tokens, the blocks completed since the first token (which the shared
 * selection could not score).  Every selected block is complete at f, so
 * the set is causal for every token.
 *
 *   q : [B][n_q][hq][d]; caches [B][hkv][n_cap][d]; d_seq_len : device
 *   int32 [B] (includes the new tokens; each in [n_q, n_cap], not checked
 *   on the host); idx : [B][1][k_B]; cnt : [B][1];
 *   out : [B][n_q][hq][d]; workspace : qsa_sparse_attn_decode_workspace
 * Errors as for qsa_sparse_attn_decode.
 */
qsa_status qsa_sparse_attn_decode_shared(const qsa_params* p, qsa_dtype dtype, const void* q,
                                         const void* k_cache, const void* v_cache, int64_t n_cap,
                                         const int32_t* d_seq_len, const int32_t* idx,
                                         const int32_t* cnt, int32_t B, int32_t n_q, int32_t hq,
                                         int32_t hkv, int32_t d, float scale, void* out,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * qsa_sparse_attn_decode_noalloc -- qsa_sparse_attn_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same kernels and results,
 * with the split partials kept in a fixed 64 MiB device array of the library
 * instead of a caller workspace.  The call allocates nothing.
 *
 * Each device the library runs on holds one such array until the process
 * ends, and every call on that device shares it: calls that overlap on one
 * device (other streams, other host threads) race and give undefined
 * results; calls ordered on one stream are safe.  The array needs no
 * clearing (every partial a call reads was written by that call).
 * Arguments as for qsa_sparse_attn_decode, without the workspace.
 * Errors as for qsa_sparse_attn_decode; sizes whose partials exceed 64 MiB
 * (qsa_sparse_attn_decode_workspace(...) > 64 MiB) -> QSA_ERR_WORKSPACE.
 */
qsa_status qsa_sparse_attn_decode_noalloc(const qsa_params* p, qsa_dtype dtype, const void* q,
                                          const void* k_cache, const void* v_cache,
                                          int64_t n_cap, const int32_t* d_seq_len,
                                          const int32_t* idx, const int32_t* cnt, int32_t B,
                                          int32_t n_q, int32_t hq, int32_t hkv, int32_t d,
                                          float scale, void* out, void* stream);

/*
 * qsa_sparse_attn_backward -- gradients of the sparse core attention for
 * joint sparse training ([hub] "Key ideas": stage 2 trains the indexer and
 * the sparse attention together).  The block selection (idx, cnt, as given
 * to qsa_sparse_attn_prefill for the same rows) is a discrete choice and
 * gets no gradient.  With P the softmax weights of row t over T_t:
 *   dP_j = <dout, v_j>, Dsum = <dout, out>, dS_j = P_j (dP_j - Dsum),
 *   dq = scale sum_j dS_j k_j,  dk_j += scale dS_j q,  dv_j += P_j dout.
 *
 *   q, out, dout : [B][n_q][hq][d] bfloat16 (out as the forward wrote it);
 *   k, v : [B][hkv][n_cap][d] bfloat16;
 *   dq : [B][n_q][hq][d] float32, written;
 *   dk, dv : [B][hkv][n_cap][d] float32, ADDED to (the caller clears them;
 *            rows attended by no query are left untouched)
 *   workspace : device scratch of qsa_sparse_attn_backward_workspace(...)
 *               bytes (per-row log-sum-exp and <dout, out>, and the
 *               selection transposed to per-block lists of rows, so that
 *               each key row's gradient is summed by one owner: no float
 *               atomics; the sums run in ascending row order, so the result
 *               is deterministic while no block is selected by more than
 *               16384 rows of one call)
 * Errors as for qsa_sparse_attn_prefill; float32 inputs or n_q * k_B above
 * 2^31 -> QSA_ERR_UNSUPPORTED; workspace too small -> QSA_ERR_WORKSPACE.
 */
qsa_status qsa_sparse_attn_backward(const qsa_params* p, qsa_dtype dtype, const void* q,
                                    const void* k, const void* v, int64_t n_cap,
                                    const int32_t* idx, const int32_t* cnt, const void* out,
                                    const void* dout, int32_t B, int32_t n_q, int64_t q_pos0,
                                    int32_t hq, int32_t hkv, int32_t d, float scale, float* dq,
                                    float* dk, float* dv, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* Workspace bytes qsa_sparse_attn_backward needs for these sizes (0 for
 * invalid parameters). */
size_t qsa_sparse_attn_backward_workspace(const qsa_params* p, int32_t B, int32_t n_q,
                                          int64_t q_pos0, int32_t hq);

/*
 * qsa_index_distill -- stage-1 indexer distillation ([hub] "Key ideas",
 * native-trainability bullet: KL divergence of the indexer's scores to the
 * teacher's dense attention max-pooled over micro-blocks, the indexer
 * trained alone).  For query row t at position p = q_pos0 + t with
 * nb = floor((p+1)/r) complete blocks:
 *   teacher  a_b = max over the block's r tokens of sum_h softmax_{j<=p}(
 *            scale <q^h, k_j^{g(h)}>), normalised over b < nb;
 *   student  softmax over b < nb of I_b = sum_h ReLU(<q~^h, kbar_b>)
 *            (q~ = q_idx rotated at p, kbar as stored);
 *   loss[t]  = KL(teacher || student)  (0 when nb = 0);
 *   dq_idx   gradient of loss[t] w.r.t. the row's raw indexer queries
 *            (teacher fixed), written;
 *   dkbar    gradient of sum_t loss[t] w.r.t. the pooled keys, ADDED to.
 *
 *   q : [B][n_q][hq][d] bfloat16; k : [B][hkv][n_cap][d] bfloat16 (the
 *   attention keys); q_idx : [B][n_q][4][128] and kbar : [B][nb_cap][128]
 *   bfloat16; loss : [B][n_q], dq_idx : [B][n_q][4][128], dkbar :
 *   [B][nb_cap][128], all float32.  Built for r = 4, rope_dims <= 64,
 *   hq <= 16, hkv <= 8, d = 128.
 *   workspace : device scratch of qsa_index_distill_workspace(...) bytes,
 *   owned by the caller: the teacher's block values a_b of every row, kept
 *   from the normaliser pass for the gradient pass (which then needs
 *   neither the keys nor the teacher's logits).  Needs no clearing.
 * Errors: NULL pointers; positions beyond n_cap or seeing more than nb_cap
 * blocks -> QSA_ERR_SHAPE; other dtypes or sizes -> QSA_ERR_UNSUPPORTED;
 * workspace too small -> QSA_ERR_WORKSPACE.
 */
qsa_status qsa_index_distill(const qsa_params* p, qsa_dtype dtype, const void* q, const void* k,
                             int64_t n_cap, const void* q_idx, const void* kbar, int64_t nb_cap,
                             int32_t B, int32_t n_q, int64_t q_pos0, int32_t hq, int32_t hkv,
                             int32_t d, float scale, float* loss, float* dq_idx, float* dkbar,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes qsa_index_distill needs: 4 bytes per (sequence, row,
 * visible block) of the call's rows, i.e. B * sum over positions p of
 * floor((p+1)/4) (0 for invalid parameters). */
size_t qsa_index_distill_workspace(const qsa_params* p, int32_t B, int32_t n_q, int64_t q_pos0);

/*
 * qsa_pool_keys_backward -- gradient of the raw indexer keys from the
 * gradient of the pooled keys (qsa_pool_keys is linear: each of block j's r
 * keys receives (1/r) times dkbar[j] rotated back by the block's angle).
 *   dkbar : [B][nb_cap][d_idx] float32; dk_idx : [B][n_cap][d_idx] float32,
 *   rows of blocks [block_begin, block_end) written.
 * Errors as for qsa_pool_keys.
 */
qsa_status qsa_pool_keys_backward(const qsa_params* p, const float* dkbar, int64_t nb_cap,
                                  float* dk_idx, int64_t n_cap, int32_t B, int64_t block_begin,
                                  int64_t block_end, void* stream);

/*
 * qsa_dense_attn_prefill -- dense causal GQA attention: every query attends
 * to all tokens 0 .. its position.  This is QSA with every block selected
 * (k_B at least the visible blocks), and the dense baseline of the pages'
 * kernel comparison ([glide] "QSA Ablations and Efficiency", Figure 6(c):
 * chunked prefill, 16K-token chunks, batch 1, dense GQA vs QSA).
 *
 *   out[b][t][h] = sum_{j <= q_pos0 + t} softmax_j(scale <q[b][t][h], k[b][g][j]>) v[b][g][j]
 *   q : [B][n_q][hq][d] (rows at positions q_pos0 + t); k, v : [B][hkv][n_cap][d]
 *   out : [B][n_q][hq][d]; bfloat16 only; hq / hkv must divide 16; scale <= 0
 *   means 1/sqrt(d).
 * Errors: NULL pointers; q_pos0 + n_q > n_cap -> QSA_ERR_SHAPE; float32,
 * d != 128 or hq/hkv not dividing 16 -> QSA_ERR_UNSUPPORTED.
 */
qsa_status qsa_dense_attn_prefill(qsa_dtype dtype, const void* q, const void* k, const void* v,
                                  int64_t n_cap, int32_t B, int32_t n_q, int64_t q_pos0,
                                  int32_t hq, int32_t hkv, int32_t d, float scale, void* out,
                                  void* stream);

/*
 * qsa_dense_attn_decode -- the same for n_q new tokens per sequence at
 * positions d_seq_len[b] - n_q + t against the KV caches ([glide] Figure
 * 6(d): decode, batch 4, next_n = 4), split over the context in pieces of
 * 4096 keys and combined.
 *   q : [B][n_q][hq][d]; caches [B][hkv][n_cap][d]; d_seq_len device int32
 *   [B] (includes the new tokens; each in [n_q, n_cap], not checked on
 *   the host); out : [B][n_q][hq][d];
 *   workspace : qsa_dense_attn_decode_workspace(B, n_q, hkv, n_cap) bytes.
 * Errors as for qsa_dense_attn_prefill, plus n_q * hq/hkv > 64 ->
 * QSA_ERR_UNSUPPORTED and a small workspace -> QSA_ERR_WORKSPACE.
 */
qsa_status qsa_dense_attn_decode(qsa_dtype dtype, const void* q, const void* k_cache,
                                 const void* v_cache, int64_t n_cap, const int32_t* d_seq_len,
                                 int32_t B, int32_t n_q, int32_t hq, int32_t hkv, int32_t d,
                                 float scale, void* out, void* workspace, size_t workspace_bytes,
                                 void* stream);

size_t qsa_dense_attn_decode_workspace(int32_t B, int32_t n_q, int32_t hkv, int64_t n_cap);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
