// Dense causal GQA attention (flash-style), bf16 inputs, fp32 softmax and
// accumulation.  It is what QSA reduces to when every block is selected
// (k_B >= visible blocks: T_i = {0 .. i}), and the baseline the pages time
// QSA against (paperglide reader, "QSA Ablations and Efficiency", Figure 6(c,d):
// chunked prefill with 16K-token chunks at batch 1, and decode at batch 4 with
// next_n = 4, dense GQA vs QSA; research-hub note, "Key ideas": about 7.6x
// prefill and 4.9x decode at 1M).
//
// Layout of the work: a column is one (query token, query head) pair; the
// hq/hkv heads that share a KV head are consecutive columns, so with 8 query
// heads per KV head one 16-column MFMA group holds two tokens and nothing is
// padded.  Each wave owns NCG groups of 16 columns.  A workgroup of W waves
// shares one stream of 32-key K/V tiles: every tile is copied once into LDS
// (global -> LDS, 16 bytes per lane, two tiles in flight ahead of the one
// computed) and read by all its
// waves.  Per tile a wave computes S^T = K Q^T (v_mfma_f32_16x16x32_bf16, 16
// keys x 16 columns per call), an online softmax in base 2 against a
// reference maximum that moves only when the running maximum grows by more
// than 2^8, and O^T += V^T P^T with P kept in registers (the k index of the
// PV call is permuted to match the S^T accumulator layout; V^T comes from
// transposing LDS reads).  Per tile the S^T calls of all column groups come
// first, then the softmax, then the PV calls, so that the MFMA chains are
// independent; the column sum is kept per lane and reduced once at the end.
//
// Prefill: one workgroup per (sequence, KV head, tile of query tokens),
// keys 0 .. the tile's last position.  Decode: one wave per (sequence, KV
// head, split of the context); the split's partial (max, sum, unnormalised
// output) per token and head is merged by the split-combine kernel of the
// sparse decode.
#include <math.h>

#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr int kKT = 32;              // keys per tile
constexpr int kPrefetch = 1;         // tiles loaded ahead of the computed one
constexpr int kTileBytes = kKT * 256;  // one K or V tile in bf16

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// K tile in LDS: key row kk (256 bytes) keeps its 16-byte chunk c at chunk
// c ^ (kk & 15): the 16 rows an A-operand read touches then hit 16 distinct
// bank groups.
__device__ __forceinline__ int kswz(int kk, int c) { return c ^ (kk & 15); }
// V tile in LDS: chunk c of key row kk at c ^ 2(kk & 7), so a transposed
// read (16 key rows x two neighbouring chunks) touches every bank twice.
__device__ __forceinline__ int vswz(int kk, int c) { return c ^ ((kk & 7) << 1); }

__device__ __forceinline__ s16x4 lds_tr16(const unsigned short* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

__device__ __forceinline__ float wmax16(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wsum16(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

}  // namespace

// NCG: 16-column groups per wave; W: waves per workgroup (sharing the K/V
// stream).  part == nullptr: prefill, each column's output written here;
// else decode: nsplit splits of split_keys keys each write partials to
// `part` (also when nsplit is 1), merged by the combine kernel.
template <int NCG, int W>
__global__ __launch_bounds__(64 * W) void dense_attn_kernel(AttnArgs a, int nsplit,
                                                            int split_keys, float* part) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_dense[];
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hl = lane & 15, gq = lane >> 4;
  const int G = a.hq / a.hkv;
  constexpr int kCols = 16 * NCG * W;  // columns of the workgroup

  // ---- work unit --------------------------------------------------------
  int b, g, split = 0, t0;
  int64_t k_lo, k_hi;  // keys [k_lo, k_hi) of this unit
  const bool prefill = part == nullptr;
  if (prefill) {
    const int tokens = kCols / G;  // query tokens per workgroup
    const int ntiles = (a.n_q + tokens - 1) / tokens;
    int64_t w = blockIdx.x;
    // longest tiles (latest tokens) first
    const int tile = ntiles - 1 - (int)(w % ntiles);
    w /= ntiles;
    g = (int)(w % a.hkv);
    b = (int)(w / a.hkv);
    t0 = tile * tokens;
    const int t_last = min(a.n_q, t0 + tokens) - 1;
    k_lo = 0;
    k_hi = a.q_pos0 + t_last + 1;
  } else {
    int64_t w = blockIdx.x;
    split = (int)(w % nsplit);
    w /= nsplit;
    g = (int)(w % a.hkv);
    b = (int)(w / a.hkv);
    t0 = 0;
    const int64_t L = a.seq_len[b];
    k_lo = (int64_t)split * split_keys;
    k_hi = min(k_lo + (int64_t)split_keys, L);
  }
  const int64_t pos0 = prefill ? a.q_pos0 : (int64_t)a.seq_len[b] - a.n_q;

  // ---- this lane's columns: token, head, position ------------------------
  // positions stay below 2^31 (checked on the host): 32-bit compares
  int col_t[NCG], col_h[NCG], col_pos[NCG];
  bool col_ok[NCG];
#pragma unroll
  for (int c = 0; c < NCG; ++c) {
    const int col = 16 * (NCG * wv + c) + hl;
    col_t[c] = t0 + col / G;
    col_h[c] = col % G;
    col_ok[c] = col_t[c] < a.n_q && (prefill || col < 16 * NCG);
    col_pos[c] = (int)(pos0 + col_t[c]);
  }
  // every key below this position is visible to all of the wave's columns
  const int wave_min_pos = (int)(pos0 + t0 + (16 * NCG * wv) / G);
  // Q^T operands: column hl of group c, dims 32cc + 8gq .. + 7
  bf16x8 qf[NCG][4];
#pragma unroll
  for (int c = 0; c < NCG; ++c) {
    const unsigned short* qrow =
        (const unsigned short*)a.q +
        (((int64_t)b * a.n_q + (col_ok[c] ? col_t[c] : 0)) * a.hq + g * G + col_h[c]) * 128;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (col_ok[c]) v = *(const u16x8*)(qrow + 32 * cc + 8 * gq);
      qf[c][cc] = __builtin_bit_cast(bf16x8, v);
    }
  }

  const char* kbase = (const char*)a.k + ((int64_t)b * a.hkv + g) * a.n_cap * 256;
  const char* vbase = (const char*)a.v + ((int64_t)b * a.hkv + g) * a.n_cap * 256;

  // Copy the tile of keys k0 .. k0 + 31 into LDS buffer `dst` (K then V):
  // 16 instructions of 1 KB (4 keys each) dealt over the W waves; rows past
  // k_hi read row 0 (masked later).
  auto issue = [&](int64_t k0, unsigned char* dst) {
#pragma unroll
    for (int j = 0; j < 16 / W; ++j) {
      const int ins = W * j + wv;  // 0..7: K keys 4ins.., 8..15: V keys 4(ins-8)..
      const bool isv = ins >= 8;
      const int kk = 4 * (ins & 7) + (lane >> 4);
      const int64_t key = k0 + kk;
      const uint64_t row = key < k_hi ? (uint64_t)key : 0ull;
      const int ch = isv ? vswz(kk, lane & 15) : kswz(kk, lane & 15);
      const char* src = (isv ? vbase : kbase) + row * 256 + 16 * ch;
      __builtin_amdgcn_global_load_lds((glb_void_t*)src,
                                       (lds_void_t*)(dst + (isv ? kTileBytes : 0) +
                                                     (ins & 7) * 1024),
                                       16, 0, 0);
    }
  };

  const float sl2 = a.scale * 1.4426950408889634f;
  f32x4 o[NCG][8];
  float m[NCG], l[NCG];
#pragma unroll
  for (int c = 0; c < NCG; ++c) {
    m[c] = -INFINITY;
    l[c] = 0.f;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) o[c][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // kPrefetch tiles in flight ahead of the one computed, in a ring of
  // kPrefetch + 1 LDS buffers
  const int ntile = k_hi > k_lo ? (int)((k_hi - k_lo + kKT - 1) / kKT) : 0;
  auto bufp = [&](int it) { return smem_dense + (it % (kPrefetch + 1)) * 2 * kTileBytes; };
#pragma unroll
  for (int j = 0; j < kPrefetch; ++j)
    if (j < ntile) issue(k_lo + (int64_t)j * kKT, bufp(j));
  for (int it = 0; it < ntile; ++it) {
    const int64_t k0 = k_lo + (int64_t)it * kKT;
    const unsigned char* cur = bufp(it);
    // tile `it` has landed for every wave: this wave's later tiles (16 / W
    // loads each) may still be in flight
    if (it + kPrefetch - 1 < ntile) {
      if constexpr (kPrefetch == 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if constexpr (kPrefetch == 2 && W == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      if constexpr (kPrefetch == 2 && W == 8) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
      if constexpr (kPrefetch == 2 && W == 1) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      if constexpr (kPrefetch == 3 && W == 4) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      if constexpr (kPrefetch == 3 && W == 8) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      if constexpr (kPrefetch == 3 && W == 1) asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    // V^T operands of O^T tile tt (dims 16tt..): k index 8gq + j <-> key
    // (j < 4 ? 4gq + j : 16 + 4gq + j - 4); lane hl reads key 4gq + hl/4
    // (+16), dims 16tt + 4(hl%4) .. + 3, transposed
    s16x4 vr[16];
    {
      const unsigned short* vs = (const unsigned short*)(cur + kTileBytes);
      const int kk = 4 * gq + (hl >> 2);
      const int e0 = 4 * (hl & 1);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int c = 2 * tt + ((hl & 3) >> 1);
        vr[2 * tt] = lds_tr16(vs + kk * 128 + vswz(kk, c) * 8 + e0);
        vr[2 * tt + 1] = lds_tr16(vs + (kk + 16) * 128 + vswz(kk + 16, c) * 8 + e0);
      }
    }
    const bool full_tile = k0 + kKT <= k_hi && k0 + kKT - 1 <= wave_min_pos;
    // S^T of every column group first (independent MFMA chains)
    f32x4 sacc[NCG][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int c = 0; c < NCG; ++c) sacc[c][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        // K operand, read just before its calls: key row hl of 16-key tile
        // kt, dims 32cc + 8gq
        const int kk = 16 * kt + hl;
        const bf16x8 kf = *(const bf16x8*)(cur + kk * 256 + 16 * kswz(kk, 4 * cc + gq));
#pragma unroll
        for (int c = 0; c < NCG; ++c)
          sacc[c][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[c][cc], sacc[c][kt], 0,
                                                                0, 0);
      }
    // every operand of this tile is in registers (V^T above, K just now): the
    // next tile may land in another buffer while this one is computed
    if (it + kPrefetch < ntile) issue(k0 + (int64_t)kPrefetch * kKT, bufp(it + kPrefetch));
    bf16x8 pf[NCG];
#pragma unroll
    for (int c = 0; c < NCG; ++c) {
      // lane holds keys k0 + 16kt + 4gq + i of column hl; tiles wholly below
      // every column's position and k_hi need no mask (wave-uniform)
      float sv[8];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = (int)k0 + 16 * kt + 4 * gq + i;
          const bool ok = full_tile || (key < (int)k_hi && key <= col_pos[c]);
          sv[4 * kt + i] = ok ? sacc[c][kt][i] * sl2 : -INFINITY;
        }
      float mx = sv[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sv[j]);
      // the column's reference moves only if some lane's values exceed it
      // by more than 2^8 (then the column maximum is formed across lanes)
      if (__ballot(mx > m[c] + 8.f)) {
        const float mn = fmaxf(m[c], wmax16(mx));
        const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[c] - mn);
        l[c] *= alpha;
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) o[c][tt] = o[c][tt] * alpha;
        m[c] = mn;
      }
      // l: this lane's share of the column sum (summed across lanes at the
      // end).  A reference still at -inf here means every value of the lane
      // is -inf (a finite one would have moved it), so 0 stands in for it.
      const float mref = m[c] == -INFINITY ? 0.f : m[c];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // hardware v_exp_f32 (exp2f wraps it in a range fix-up): results
        // below 2^-126 of the reference are negligible in the sums
        const float pj = __builtin_amdgcn_exp2f(sv[j] - mref);
        l[c] += pj;
        pf[c][j] = (__bf16)pj;
      }
    }
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const s16x8 vv = __builtin_shufflevector(vr[2 * tt], vr[2 * tt + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int c = 0; c < NCG; ++c)
        o[c][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pf[c],
                                                           o[c][tt], 0, 0, 0);
    }
  }
#pragma unroll
  for (int c = 0; c < NCG; ++c) l[c] = wsum16(l[c]);

  // ---- write out --------------------------------------------------------
  // O^T tile tt: lane (hl, gq) holds dims 16tt + 4gq .. + 3 of column hl
#pragma unroll
  for (int c = 0; c < NCG; ++c) {
    if (!col_ok[c]) continue;
    if (prefill) {
      const float inv = l[c] > 0.f ? 1.f / l[c] : 0.f;
      unsigned short* orow = (unsigned short*)a.out +
                             (((int64_t)b * a.n_q + col_t[c]) * a.hq + g * G + col_h[c]) * 128;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        bf16x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (__bf16)(o[c][tt][i] * inv);
        *(bf16x4*)(orow + 16 * tt + 4 * gq) = w;
      }
    } else {
      float* pp = part +
                  ((((int64_t)b * a.n_q + col_t[c]) * a.hkv + g) * nsplit + split) * kPartFloats;
      if (gq == 0) {
        pp[col_h[c]] = m[c];
        pp[16 + col_h[c]] = l[c];
      }
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
        *(f32x4*)(pp + 32 + col_h[c] * 128 + 16 * tt + 4 * gq) = o[c][tt];
    }
  }
}

// ---- host side ------------------------------------------------------------

constexpr int kPrefillNCG = 2, kPrefillW = 8;
constexpr int kDecodeSplitKeys = 4096;

static size_t dense_lds() { return (kPrefetch + 1) * 2 * (size_t)kTileBytes; }

hipError_t launch_dense_prefill(const AttnArgs& a, hipStream_t st) {
  const int G = a.hq / a.hkv;
  const int tokens = 16 * kPrefillNCG * kPrefillW / G;
  const int64_t ntiles = (a.n_q + tokens - 1) / tokens;
  const int64_t grid = ntiles * a.hkv * a.B;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((dense_attn_kernel<kPrefillNCG, kPrefillW>), dim3((unsigned)grid),
                     dim3(64 * kPrefillW), dense_lds(), st, a, 1, 0, (float*)nullptr);
  return hipGetLastError();
}

int dense_decode_splits(int64_t n_cap) {
  const int64_t s = (n_cap + kDecodeSplitKeys - 1) / kDecodeSplitKeys;
  return (int)(s < 1 ? 1 : s);
}

size_t dense_decode_workspace(int B, int n_q, int hkv, int64_t n_cap) {
  return (size_t)B * n_q * hkv * dense_decode_splits(n_cap) * kPartFloats * sizeof(float);
}

hipError_t launch_dense_decode(const AttnArgs& a, void* ws, hipStream_t st) {
  const int G = a.hq / a.hkv;
  const int cols = a.n_q * G;
  const int nsplit = dense_decode_splits(a.n_cap);
  const int64_t grid = (int64_t)a.B * a.hkv * nsplit;
  if (grid == 0) return hipSuccess;
  float* part = (float*)ws;
  if (cols <= 16)
    hipLaunchKernelGGL((dense_attn_kernel<1, 1>), dim3((unsigned)grid), dim3(64), dense_lds(), st,
                       a, nsplit, kDecodeSplitKeys, part);
  else if (cols <= 32)
    hipLaunchKernelGGL((dense_attn_kernel<2, 1>), dim3((unsigned)grid), dim3(64), dense_lds(), st,
                       a, nsplit, kDecodeSplitKeys, part);
  else
    hipLaunchKernelGGL((dense_attn_kernel<4, 1>), dim3((unsigned)grid), dim3(64), dense_lds(), st,
                       a, nsplit, kDecodeSplitKeys, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attn_combine(QSA_BF16, a, nsplit, part, st);
}

}  // namespace qsa
