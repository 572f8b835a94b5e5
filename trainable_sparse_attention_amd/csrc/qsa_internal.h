// Internal declarations shared by the HIP translation units of libqsa.
// Device helpers (bf16 storage, RoPE angles) and the host-side launchers
// that the C ABI (abi.hip) calls after validating arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qsa.h"

namespace qsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---- bfloat16 storage: values travel as raw 16-bit patterns -------------

__device__ __forceinline__ float bf16_to_f32(unsigned short h) {
  return __uint_as_float(((unsigned int)h) << 16);
}

// Round-to-nearest-even float -> bfloat16 bits (finite inputs; NaN kept NaN).
__device__ __forceinline__ unsigned short f32_to_bf16(float f) {
  unsigned int u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (unsigned short)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

template <typename T> struct Elt;
template <> struct Elt<float> {
  __device__ __forceinline__ static float ld(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void st(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elt<unsigned short> {
  __device__ __forceinline__ static float ld(const unsigned short* p, int64_t i) {
    return bf16_to_f32(p[i]);
  }
  __device__ __forceinline__ static void st(unsigned short* p, int64_t i, float v) {
    p[i] = f32_to_bf16(v);
  }
};

// ---- RoPE angle ----------------------------------------------------------
// Pair (j, j + R/2) turns by pos * theta^(-2j/R).  The angle is formed and
// reduced in double (positions reach 2^20, where float spacing would be
// 0.06 rad), then cos/sin are taken in double and rounded to float.
__device__ __forceinline__ void rope_cs(int64_t pos, int j, int R, double log2_theta, float* c,
                                        float* s) {
  double inv = exp2(-2.0 * (double)j / (double)R * log2_theta);
  double a = (double)pos * inv;
  double sn, cs;
  sincos(a, &sn, &cs);
  *c = (float)cs;
  *s = (float)sn;
}

// ---- limits the host checks before any launch ----------------------------
// Largest k_B of the many-row indexer (candidate lists of 4096 entries, cut
// back to k_B whenever one more LDS stage of blocks could overflow them).
constexpr int kMaxKBlocksRows = 3072;
// Largest k_B of the few-token decode indexer (candidate lists of 6016).
constexpr int kMaxKBlocksDecode = 4096;
// Largest KV capacity of the bf16 attention: a token row's byte offset
// within one head, row * 256, is formed in 32 bits.
constexpr int64_t kMaxCapBf16 = (int64_t)1 << 24;

// ---- host launchers (defined in the kernel translation units) ------------

// gamma == nullptr: plain block mean; else RMS-normalised mean * gamma
hipError_t launch_pool(qsa_dtype dt, const qsa_params& p, const void* k_idx, int64_t n_cap,
                       void* kbar, int64_t nb_cap, int B, int64_t b0, int64_t b1,
                       const float* gamma, float eps, hipStream_t st);

struct IndexArgs {
  const void* q_idx;
  const void* kbar;
  int64_t nb_cap;
  int B, n_q;
  int64_t q_pos0;
  const int32_t* seq_len;  // nullptr in prefill
  int32_t* idx;
  int32_t* cnt;
  int kB, r, R;
  // indexer query heads (1, 2 or 4); the kernels score 4 head slots, the
  // ones at or above h read as zero queries (ReLU(0) adds nothing)
  int h;
  double log2_theta;
};

size_t index_prefill_workspace(int B, int n_q, int num_cu, int kB);
// the self-contained exact indexer over 128-row tiles [g0, g0 + count) (longest
// first), optionally only those with only[tile - g0] != 0
size_t index_exact_workspace(int B, int n_q, int num_cu);
hipError_t launch_index_exact(qsa_dtype dt, const IndexArgs& a, void* ws, int num_cu, int g0,
                              int count, const uint32_t* only, hipStream_t st);
hipError_t launch_index_prefill(qsa_dtype dt, const IndexArgs& a, void* ws, int num_cu,
                                hipStream_t st);
size_t index_decode_workspace(int B, int n_q, int64_t nb_cap);
hipError_t launch_index_decode(qsa_dtype dt, const IndexArgs& a, void* ws, hipStream_t st);

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const int32_t* idx;
  const int32_t* cnt;
  const int32_t* seq_len;  // nullptr in prefill
  int64_t n_cap;
  int64_t q_pos0;
  int B, n_q, hq, hkv, kB, r;
  // decode: the n_q new tokens of a sequence share the one selection idx[b][0]
  // made at the first new token (its tail then runs from that token's block)
  int shared;
  float scale;
  // decode: slots per split (whole chunks), set by the decode launcher
  int split_slots;
};

// split partial per (sequence, token, KV head, split): m[16], l[16],
// o[16][128] floats (16 query heads per KV head at most); m in log2 units,
// o and l relative to 2^m
constexpr int kPartFloats = 16 + 16 + 16 * 128;

hipError_t launch_attn_prefill(qsa_dtype dt, const AttnArgs& a, hipStream_t st);
// merge nsplit partials per (sequence, token, KV head) into a.out
hipError_t launch_attn_combine(qsa_dtype dt, const AttnArgs& a, int nsplit, const float* part,
                               hipStream_t st);
// sparse attention backward (bf16 inputs): dq written, dk / dv added to;
// the workspace holds per-(row, head) lse and <dout, out> and the selection
// transposed to per-block row lists
size_t attn_backward_workspace(int B, int n_q, int64_t q_pos0, int hq, int r, int kB);
hipError_t launch_attn_backward(const AttnArgs& a, const void* dout, float* dq, float* dk,
                                float* dv, void* ws, hipStream_t st);
// indexer distillation (r = 4, bf16): loss and dq_idx written, dkbar added to
struct DistillArgs {
  const unsigned short* q;      // [B][n_q][hq][128]
  const unsigned short* k;      // [B][hkv][n_cap][128]
  const unsigned short* q_idx;  // [B][n_q][4][128]
  const unsigned short* kbar;   // [B][nb_cap][128]
  float* loss;                  // [B][n_q]
  float* dq_idx;                // [B][n_q][4][128]
  float* dkbar;                 // [B][nb_cap][128], added to
  float* aws;                   // [B][aws_ld] teacher block values a_b of each row
  int64_t aws_ld;               // floats per sequence: the rows' visible blocks
  int64_t n_cap, nb_cap, q_pos0;
  int B, n_q, hq, hkv, R;
  float scale;
  double log2_theta;
};
size_t distill_lds(int hkv);
// visible blocks summed over positions q_pos0 .. q_pos0 + n_q - 1 (r = 4)
int64_t distill_blocks(int64_t q_pos0, int n_q);
hipError_t launch_distill(const DistillArgs& a, hipStream_t st);
// pooling backward: dk rows of blocks [b0, b1) written from dkbar
hipError_t launch_pool_backward(const float* dkbar, int64_t nb_cap, float* dk, int64_t n_cap,
                                int B, int64_t b0, int64_t b1, int r, int R, double log2_theta,
                                hipStream_t st);
// dense causal GQA attention (bf16; hq/hkv divides 16)
hipError_t launch_dense_prefill(const AttnArgs& a, hipStream_t st);
size_t dense_decode_workspace(int B, int n_q, int hkv, int64_t n_cap);
hipError_t launch_dense_decode(const AttnArgs& a, void* ws, hipStream_t st);
size_t attn_decode_workspace(int B, int n_q, int hkv, int kB, int r, bool shared);
hipError_t launch_attn_decode(qsa_dtype dt, const AttnArgs& a, void* ws, hipStream_t st);
// Size of the fixed device array behind qsa_sparse_attn_decode_noalloc: the
// split partials of up to 8066 (sequence, new token, KV head, split) slots,
// e.g. 8 sequences x 4 new tokens x 2 KV heads at k_B = 512 (65 splits).
constexpr size_t kDecodeScratchBytes = (size_t)64 << 20;
// This device's address of that array (looked up once per device).
hipError_t attn_static_scratch(void** out);
hipError_t launch_probe_gather(const AttnArgs& a, int waves_per_cu, int depth, int rg,
                               uint32_t* sink, hipStream_t st);

}  // namespace qsa
