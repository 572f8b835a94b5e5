/*
 * qsa_probe.h -- measurement aid of libqsa: the memory ceiling of the sparse
 * attention's gathers on the current device.
 *
 * The sparse core attention ([glide] "Qwen Sparse Attention", Figure 3:
 * selected micro-blocks expanded to tokens, plus the incomplete-block tail)
 * reads 1 KB of K and 1 KB of V per selected block and KV head (bfloat16,
 * r = 4, head dim 128).  qsa_probe_gather reads exactly those bytes, in the
 * attention kernel's launch order and chunk order, and computes nothing with
 * them; timing it gives the rate this access pattern reaches without the
 * attention's arithmetic.  Not part of the method.
 *
 *   k, v     : [B][hkv][n_cap][128] bfloat16 device buffers
 *   idx, cnt : a selection from qsa_index_topk (positions q_pos0 + t)
 *   waves_per_cu : the per-wave LDS request is the CU's LDS / waves_per_cu
 *                  (<= 0: no extra request, occupancy set by registers)
 *   depth    : chunks of 8 slots kept in flight per wave, 1..4
 *   rows_per_wave : 1..64 consecutive query rows per wave, swept in lock
 *                  step (each step reads one chunk of every row); 1 is the
 *                  attention kernel's own mapping
 *   sink     : device uint32 [B * ceil(n_q / rows_per_wave) * hkv], one word
 *              written per wave
 * Errors: NULL pointers, sizes as for qsa_sparse_attn_prefill, r != 4,
 * k_B not a multiple of 8, depth or rows_per_wave out of range -> non-zero
 * status (see qsa.h), nothing launched.
 */
#ifndef QSA_PROBE_H
#define QSA_PROBE_H

#include "qsa.h"

#ifdef __cplusplus
extern "C" {
#endif

qsa_status qsa_probe_gather(const qsa_params* p, const void* k, const void* v, int64_t n_cap,
                            const int32_t* idx, const int32_t* cnt, int32_t B, int32_t n_q,
                            int64_t q_pos0, int32_t hkv, int32_t waves_per_cu, int32_t depth,
                            int32_t rows_per_wave, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_PROBE_H */
