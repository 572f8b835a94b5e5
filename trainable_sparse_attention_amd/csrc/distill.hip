// Indexer distillation loss and its gradients (research-hub note, "Key
// ideas", native-trainability bullet: stage 1 trains the indexer alone on a
// KL divergence to the teacher's dense attention, max-pooled over each
// micro-block).
//
// For query row i (position p, nb = floor((p+1)/4) complete blocks):
//   teacher  P_j^h = softmax_{j <= p}(scale <q^h, k_j^{g(h)}>),
//            a_b = max_{t<4} sum_h P_{4b+t}^h,  t_b = a_b / sum_b a_b  (b < nb)
//   student  I_b = sum_{h<4} ReLU(<q~^h, kbar_b>),  s_b = softmax_{b < nb}(I_b)
//   loss     KL(t || s);  g_b = s_b - t_b
//   grads    dq~^h = sum_b g_b [<q~^h, kbar_b> > 0] kbar_b (rotated back to
//            dq_idx), dkbar_b += g_b sum_h [...] q~^h.
//
// A workgroup of 8 waves takes 8 consecutive rows (one wave each) and walks
// the history in lock step, 64 keys (16 blocks) a step; each step's K rows of
// every KV head and the 16 pooled keys are copied once into LDS.  Per wave:
// teacher logits S = Q K^T on v_mfma_f32_16x16x32_bf16 (16 rows = the query
// heads, one call per KV head, each row keeping its own head's product), so
// that a lane holds one key against 4 heads: the head sum is 3 adds in the
// lane and 2 shuffles across the lane groups, the block maximum 2 shuffles
// within a lane quad.  Student scores on the same MFMA with the rotated
// indexer queries carried as bf16 hi + lo (float-level accuracy).  Three
// passes over the history: the teacher's log-sum-exp per head; the
// normalisers (sum of a_b, the student's log-sum-exp) and the loss, with
// every a_b stored to a workspace; the gradients, which read a_b back and
// so stage only the pooled keys and recompute only the student.  Both gradients of a step are small float matrix products with
// the step's g values over the workgroup's (row, head) pairs: dkbar of the
// step's blocks (the rotated queries stay in LDS), added to global memory
// with float atomics, and dq~, kept in registers.
//
// Built for r = 4, bfloat16 inputs, hq <= 16, 4 indexer heads of 128 dims,
// rope_dims <= 64.
#include <math.h>

#include "index_common.h"

namespace qsa {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

constexpr int kDW = 8;         // waves (rows) per workgroup
constexpr int kStepKeys = 64;  // keys per step
constexpr int kStepBlk = 16;   // blocks per step (r = 4)
constexpr int kMaxKv = 16;
static_assert(kDW * 16 == 128, "one 16-dim slice of dkbar per wave");

__device__ __forceinline__ int dswz(int kk, int c) { return c ^ (kk & 15); }

__device__ __forceinline__ float xsum16(float x) {  // over the 16 lanes of a group
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  return x + __shfl_xor(x, 8);
}
__device__ __forceinline__ float xmax16(float x) {  // over the 16 lanes of a group
  x = fmaxf(x, __shfl_xor(x, 1));
  x = fmaxf(x, __shfl_xor(x, 2));
  x = fmaxf(x, __shfl_xor(x, 4));
  return fmaxf(x, __shfl_xor(x, 8));
}
// The reductions of the inner loops use DPP quad permutes (lanes l ^ 1,
// l ^ 2) and the permlane swaps (lanes l ^ 16, l ^ 32), which leave every
// lane of a pair with the pair's two values (the even row's first), so
// both lanes combine them in the same order.  No LDS traffic.
__device__ __forceinline__ float dpp_x1(float x) {  // lane l ^ 1
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_x2(float x) {  // lane l ^ 2
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ float xsum4(float x) {  // over lanes hl = 0..3 of a group
  x += dpp_x1(x);
  return x + dpp_x2(x);
}
__device__ __forceinline__ float xmax4(float x) {  // over lanes hl = 0..3 of a group
  x = fmaxf(x, dpp_x1(x));
  return fmaxf(x, dpp_x2(x));
}
// hardware exponential (base 2) for the teacher's probabilities: results
// below 2^-126 are negligible next to the normalised values they are summed
// with.  The student's softmax and the loss keep the library functions: the
// gradient g_b = s_b - t_b is a difference of close values, which a
// relative error of 1e-6 in s_b would show at the 1e-3 level.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
// sum over j = 1 .. P of floor(j / 4): the blocks visible to positions
// 0 .. P - 1 together (r = 4), so that a row's a_b start at
// blocks_upto(p) - blocks_upto(q_pos0) in the packed workspace
__host__ __device__ __forceinline__ int64_t blocks_upto(int64_t P) {
  const int64_t Q = P >> 2, R = P & 3;
  return 2 * Q * (Q - 1) + Q * (R + 1);
}
__device__ __forceinline__ float sel4(const float* v, int i) {  // v[i] without scratch
  return i == 0 ? v[0] : (i == 1 ? v[1] : (i == 2 ? v[2] : v[3]));
}
__device__ __forceinline__ float xmaxg(float x) {  // over the 4 lane groups
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float xsumg(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

}  // namespace

// Two workgroups per CU (two waves per SIMD each) keep one workgroup's
// compute running over the other's staging wait; that needs <= 128 VGPRs.
__global__ __launch_bounds__(64 * kDW) __attribute__((amdgpu_waves_per_eu(4))) void distill_kernel(
    DistillArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_dist[];
  // K rows of the step: [hkv][64 keys][128] bf16, then the step's pooled
  // keys [16][128] bf16, then per-wave scratch, then the dkbar sums
  unsigned short* kls = (unsigned short*)smem_dist;
  unsigned short* kbs = kls + (size_t)a.hkv * kStepKeys * 128;
  float* scr = (float*)(kbs + kStepBlk * 128);  // [kDW][4][128] rotated queries (kept)
  float* wscr = scr + kDW * 4 * 128;           // [kDW][32] per-wave a and g values
  float* gmat = wscr + kDW * 32;               // [16 blocks][kDW * 4]: g where the head's score > 0
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hl = lane & 15, gq = lane >> 4;
  const int ntiles = (a.n_q + kDW - 1) / kDW;
  const int tile = ntiles - 1 - (int)(blockIdx.x % ntiles);  // longest rows first
  const int b = (int)(blockIdx.x / ntiles);
  const int t0 = tile * kDW;
  const int t = t0 + wv;
  const bool live = t < a.n_q;
  const int64_t pos = a.q_pos0 + (live ? t : a.n_q - 1);
  const int64_t nb = live ? (pos + 1) / 4 : 0;
  const int t_last = min(a.n_q, t0 + kDW) - 1;
  const int64_t pos_last = a.q_pos0 + t_last;
  const int64_t nb_last = (pos_last + 1) / 4;
  const int G = a.hq / a.hkv;
  const float sl2 = a.scale * 1.4426950408889634f;
  // the fields the lambdas below read, as locals (a kernel argument
  // captured by reference would be kept in scratch memory)
  const unsigned short* const kglob = a.k;
  const unsigned short* const kbglob = a.kbar;
  const int64_t n_cap = a.n_cap, nb_cap = a.nb_cap;
  const int hkv = a.hkv, hq = a.hq, R = a.R;

  // ---- prologue: Q^T operands (column hl = head), rotated indexer query
  bf16x8 qb[4];
  {
    const unsigned short* qr = a.q + (((int64_t)b * a.n_q + (live ? t : 0)) * a.hq + hl) * 128;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      u16x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
      if (live && hl < a.hq) x = *(const u16x8*)(qr + 32 * cc + 8 * gq);
      qb[cc] = __builtin_bit_cast(bf16x8, x);
    }
  }
  float* qs = scr + wv * 4 * 128;  // q~ [4][128] of this wave's row
  {
    const int half = a.R / 2;
    const unsigned short* qi = a.q_idx + ((int64_t)b * a.n_q + (live ? t : 0)) * 512;
    for (int e = lane; e < 512; e += 64) {
      const int d = e & 127;
      const float x = live ? bf16_to_f32(qi[e]) : 0.f;
      float val = x;
      if (d < a.R) {
        const int j = d < half ? d : d - half;
        float c, s;
        rope_cs(pos, j, a.R, a.log2_theta, &c, &s);
        const float y = live ? bf16_to_f32(qi[(e & ~127) + (d < half ? d + half : d - half)]) : 0.f;
        val = d < half ? (x * c - y * s) : (y * s + x * c);
      }
      qs[e] = val;
    }
  }
  wave_sync();
  // student B operands: column hl < 4 = indexer head, dims 32cc + 8gq; hi
  // part, and a lo part for the rotated dims (cc < NLO)
  bf16x8 ib[4], ibl[2];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    u16x8 h = {0, 0, 0, 0, 0, 0, 0, 0}, lo = h;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = hl < 4 ? qs[hl * 128 + 32 * cc + 8 * gq + e] : 0.f;
      unsigned short hh, ll;
      split_bf16(v, &hh, &ll);
      h[e] = hh;
      lo[e] = 32 * cc + 8 * gq + e < a.R ? ll : (unsigned short)0;
    }
    ib[cc] = __builtin_bit_cast(bf16x8, h);
    if (cc < 2) ibl[cc] = __builtin_bit_cast(bf16x8, lo);
  }
  __syncthreads();

  // ---- a step's K rows (every KV head) and pooled keys into LDS ---------
  auto stage = [&](int64_t k0, int64_t klim, bool with_k, bool with_kbar) {
    const int nkv_ins = with_k ? hkv * kStepKeys / 4 : 0;  // 1 KB instructions for K
    const int nins = nkv_ins + (with_kbar ? kStepBlk / 4 : 0);
    for (int ins = wv; ins < nins; ins += kDW) {
      if (ins < nkv_ins) {
        const int gg = ins / (kStepKeys / 4), kk = 4 * (ins % (kStepKeys / 4)) + (lane >> 4);
        const int64_t key = k0 + kk;
        const uint64_t row = key < klim ? (uint64_t)key : 0ull;
        const unsigned short* src = kglob + (((int64_t)b * hkv + gg) * n_cap + row) * 128 +
                                    8 * dswz(kk, lane & 15);
        __builtin_amdgcn_global_load_lds((glb_void_t*)src,
                                         (lds_void_t*)(kls + ((size_t)gg * kStepKeys + kk - (lane >> 4)) * 128),
                                         16, 0, 0);
      } else {
        const int bb = 4 * (ins - nkv_ins) + (lane >> 4);
        const int64_t blk = k0 / 4 + bb;
        const uint64_t row = blk < nb_cap ? (uint64_t)blk : 0ull;
        const unsigned short* src = kbglob + ((int64_t)b * nb_cap + row) * 128 +
                                    8 * dswz(bb, lane & 15);
        __builtin_amdgcn_global_load_lds((glb_void_t*)src,
                                         (lds_void_t*)(kbs + (bb - (lane >> 4)) * 128), 16, 0, 0);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  // teacher logits S = Q K^T of key tile kt (16 keys) of the step (not yet
  // scaled): lane (hl, gq) holds key 16 kt + hl against heads 4 gq + i.
  // One product per KV head; each of the lane's heads keeps its own KV
  // head's value (heads >= hq keep 0 and are masked by the callers).
  auto teacher = [&](int kt, f32x4& out) {
    out = f32x4{0.f, 0.f, 0.f, 0.f};
    const int kk = 16 * kt + hl;
    for (int gg = 0; gg < hkv; ++gg) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const unsigned short* rowp = kls + ((size_t)gg * kStepKeys + kk) * 128;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const bf16x8 kv = *(const bf16x8*)(rowp + 8 * dswz(kk, 4 * cc + gq));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb[cc], kv, acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((4 * gq + i) / G == gg) out[i] = acc[i];
    }
  };

  // ---- pass 1: teacher log-sum-exp per head (base 2), keys 0 .. p -------
  // per lane: a running maximum and sum for each of its 4 heads over the
  // keys of its column hl; the 16 columns are merged after the sweep
  float lm[4], ll[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lm[i] = -INFINITY;
    ll[i] = 0.f;
  }
  const int nstep1 = (int)((pos_last + 1 + kStepKeys - 1) / kStepKeys);
  for (int st = 0; st < nstep1; ++st) {
    const int64_t k0 = (int64_t)st * kStepKeys;
    stage(k0, pos_last + 1, true, false);
    float x[4][4];  // [key tile][head], future keys at -inf
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4 s;
      teacher(kt, s);
      const bool ok = live && k0 + 16 * kt + hl <= pos;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[kt][i] = ok ? s[i] * sl2 : -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mx = fmaxf(fmaxf(lm[i], fmaxf(x[0][i], x[1][i])), fmaxf(x[2][i], x[3][i]));
      if (mx != -INFINITY) {
        float acc = lm[i] == -INFINITY ? 0.f : ll[i] * fexp2(lm[i] - mx);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) acc += fexp2(x[kt][i] - mx);
        ll[i] = acc;
        lm[i] = mx;
      }
    }
    __syncthreads();
  }
  float lse[4];  // of heads 4 gq + i (-inf for absent rows and heads)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float mm = xmax16(lm[i]);
    const float l = xsum16(lm[i] == -INFINITY ? 0.f : ll[i] * exp2f(lm[i] - mm));
    lse[i] = mm == -INFINITY ? -INFINITY : mm + log2f(l);
  }

  float* wsc = wscr + wv * 32;  // this wave's [16] a values, then [16] g values
  // student: 16 blocks x 4 heads (columns hl < 4); lane (hl, gq) ends with
  // I of blocks 4gq + i and the sign bits of the 4 heads
  auto student_terms = [&](float* iv, uint64_t* sgn) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int bb = hl;  // A row: block hl of the step
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const bf16x8 kv = *(const bf16x8*)(kbs + bb * 128 + 8 * dswz(bb, 4 * cc + gq));
      if (cc < 2 && R > 0)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, ibl[cc], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, ib[cc], acc, 0, 0, 0);
    }
    // lane (hl, gq) holds <q~^hl, kbar> of blocks 4gq + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sgn[i] = __ballot(hl < 4 && acc[i] > 0.f);
      iv[i] = xsum4(hl < 4 ? relu(acc[i]) : 0.f);
    }
  };
  // per step: a_b and I_b of the step's 16 blocks; lane (hl, gq) ends with
  // a and I of blocks 4gq + i (i < 4) and the sign bits of the 4 heads
  auto block_terms = [&](int64_t k0, float* av, float* iv, uint64_t* sgn) {
    // teacher: head-summed probabilities, maximum over the block's 4 keys
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4 s;
      teacher(kt, s);
      const bool ok = live && k0 + 16 * kt + hl <= pos;
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sum += (ok && 4 * gq + i < hq) ? fexp2(fmaf(s[i], sl2, -lse[i])) : 0.f;
      sum = xsumg(sum);  // all heads of key 16 kt + hl
      // block 4 kt + hl / 4: its 4 keys sit in lanes hl & ~3 .. (hl & ~3) + 3
      const float mx = xmax4(sum);
      if (lane < 16 && (hl & 3) == 0) wsc[4 * kt + (hl >> 2)] = mx;
    }
    wave_sync();
    student_terms(iv, sgn);
#pragma unroll
    for (int i = 0; i < 4; ++i) av[i] = wsc[4 * gq + i];
    wave_sync();
  };


  // ---- pass 2: normalisers and the loss ----------------------------------
  const int nstep2 = (int)((nb_last + kStepBlk - 1) / kStepBlk);
  float asum = 0.f, alog = 0.f, aI = 0.f, zm = -INFINITY, zl = 0.f;
  // this row's a_b, blocks 0 .. nb - 1, in the workspace (rows packed)
  float* const arow = a.aws + (int64_t)b * a.aws_ld + (blocks_upto(pos) - blocks_upto(a.q_pos0));
  for (int st = 0; st < nstep2; ++st) {
    const int64_t k0 = (int64_t)st * kStepKeys;
    stage(k0, pos_last + 1, true, true);
    float av[4], iv[4];
    uint64_t sgn[4];
    block_terms(k0, av, iv, sgn);
    // lane (hl < 4, gq) takes block 4 gq + hl of the step
    if (hl < 4) {
      const float ab = sel4(av, hl), ib_ = sel4(iv, hl);
      const int64_t blk = (int64_t)st * kStepBlk + 4 * gq + hl;
      if (blk < nb) {
        arow[blk] = ab;
        asum += ab;
        alog += ab > 0.f ? ab * logf(ab) : 0.f;
        aI += ab * ib_;
        if (ib_ > zm) {
          zl = zl * expf(zm - ib_) + 1.f;
          zm = ib_;
        } else {
          zl += expf(ib_ - zm);
        }
      }
    }
    __syncthreads();
  }
  // combine the 16 lanes hl < 4 (the others carry 0)
  asum = xsumg(xsum4(hl < 4 ? asum : 0.f));
  alog = xsumg(xsum4(hl < 4 ? alog : 0.f));
  aI = xsumg(xsum4(hl < 4 ? aI : 0.f));
  float lnz;
  {
    const float zz = hl < 4 ? zm : -INFINITY;
    const float mz = xmaxg(xmax4(zz));
    const float s = xsumg(xsum4(hl < 4 && zm != -INFINITY ? zl * expf(zm - mz) : 0.f));
    lnz = mz + logf(s);
  }
  const bool has = live && nb > 0;
  if (live && lane == 0)
    a.loss[(int64_t)b * a.n_q + t] =
        has ? alog / asum - logf(asum) - aI / asum + lnz : 0.f;

  // ---- pass 3: gradients -------------------------------------------------
  // Both gradients are small products with the step's G[b][(row, h)] = g_b
  // where head h's score of block b is positive (else 0), over the
  // workgroup's 8 rows x 4 heads: every wave writes its row's 16 x 4 column
  // of G to LDS, then wave wv forms dims 16 wv .. 16 wv + 15 of
  //   dkbar[b][d]     = sum_(row, h) G[b][(row, h)] q~[(row, h)][d]  (k = (row, h))
  //   dq~[(row, h)][d] += sum_b kbar[b][d] G[b][(row, h)]            (k = b)
  // on v_mfma_f32_16x16x4f32 (float operands).  dq~ stays in registers
  // across the steps (dims of every row of the workgroup) and is regrouped
  // by row through LDS at the end.
  static_assert(kDW * 4 == 32, "two 16-column tiles of (row, head) pairs");
  f32x4 dacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  const float inv_a = has ? 1.f / asum : 0.f;
  for (int st = 0; st < nstep2; ++st) {
    const int64_t k0 = (int64_t)st * kStepKeys;
    stage(k0, pos_last + 1, false, true);  // the pooled keys only
    float iv[4];
    uint64_t sgn[4];
    student_terms(iv, sgn);
    // g of block 4 gq + hl (lanes hl < 4, which stored its a_b in pass 2),
    // shared through the wave's scratch
    if (hl < 4) {
      const int64_t blk = (int64_t)st * kStepBlk + 4 * gq + hl;
      wsc[16 + 4 * gq + hl] =
          (has && blk < nb) ? expf(sel4(iv, hl) - lnz) - arow[blk] * inv_a : 0.f;
    }
    wave_sync();
    {
      // this row's column of G: lane (block lane / 4, head lane % 4)
      const int bb = lane >> 2, h = lane & 3, i = bb & 3, grp = bb >> 2;
      const uint64_t sg = i == 0 ? sgn[0] : (i == 1 ? sgn[1] : (i == 2 ? sgn[2] : sgn[3]));
      const bool on = (sg >> (16 * grp + h)) & 1ull;
      gmat[bb * (kDW * 4) + wv * 4 + h] = on ? wsc[16 + bb] : 0.f;
    }
    __syncthreads();
    f32x4 cacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kDW; ++c) {
      const float ga = gmat[hl * (kDW * 4) + 4 * c + gq];
      const float qv = scr[(4 * c + gq) * 128 + 16 * wv + hl];
      cacc = __builtin_amdgcn_mfma_f32_16x16x4f32(ga, qv, cacc, 0, 0, 0);
    }
    // dq~: lane (hl, gq) brings kbar[4c + gq][16 wv + hl] and G[4c + gq][16 nt + hl]
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int bq = 4 * c + gq, dd = 16 * wv + hl;
      const float kv = bf16_to_f32(kbs[bq * 128 + 8 * dswz(bq, dd >> 3) + (dd & 7)]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        dacc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv, gmat[bq * (kDW * 4) + 16 * nt + hl],
                                                        dacc[nt], 0, 0, 0);
    }
    // cacc: lane holds blocks 4gq + e of the step at dim 16 wv + hl
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t blk = (int64_t)st * kStepBlk + 4 * gq + e;
      if (blk < nb_last && cacc[e] != 0.f)
        unsafeAtomicAdd(a.dkbar + ((int64_t)b * a.nb_cap + blk) * 128 + 16 * wv + hl, cacc[e]);
    }
    __syncthreads();
  }
  // dacc[nt]: lane (hl, gq) holds dims 16 wv + 4 gq + e of pair 16 nt + hl;
  // regroup by row through the (now free) rotated-query scratch
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int e = 0; e < 4; ++e) scr[(16 * nt + hl) * 128 + 16 * wv + 4 * gq + e] = dacc[nt][e];
  __syncthreads();
  float dq[4][2];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    dq[h][0] = scr[(wv * 4 + h) * 128 + lane];
    dq[h][1] = scr[(wv * 4 + h) * 128 + 64 + lane];
  }
  // dq_idx: rotate back (angle -p) on the rotated dims; pair (j, j + R/2)
  // lives in lanes j and j + R/2 (R <= 64)
  if (live) {
    const int half = a.R / 2;
    float* out = a.dq_idx + ((int64_t)b * a.n_q + t) * 512;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float v0 = dq[h][0];
      const float partner = __shfl(v0, lane < a.R ? (lane < half ? lane + half : lane - half) : lane);
      if (lane < a.R) {
        const int j = lane < half ? lane : lane - half;
        float c, s;
        rope_cs(pos, j, a.R, a.log2_theta, &c, &s);
        // inverse rotation: x' = x c + y s, y' = -x s + y c for the pair (x, y)
        v0 = lane < half ? (v0 * c + partner * s) : (v0 * c - partner * s);
      }
      out[h * 128 + lane] = v0;
      out[h * 128 + 64 + lane] = dq[h][1];
    }
  }
}

int64_t distill_blocks(int64_t q_pos0, int n_q) {
  return blocks_upto(q_pos0 + n_q) - blocks_upto(q_pos0);
}

size_t distill_lds(int hkv) {
  return (size_t)hkv * kStepKeys * 128 * 2 + kStepBlk * 128 * 2 + kDW * 4 * 128 * 4 +
         kDW * 32 * 4 + kStepBlk * kDW * 4 * 4;
}

hipError_t launch_distill(const DistillArgs& a, hipStream_t st) {
  const int ntiles = (a.n_q + kDW - 1) / kDW;
  const int64_t grid = (int64_t)ntiles * a.B;
  if (grid == 0) return hipSuccess;
  const size_t lds = distill_lds(a.hkv);
  hipError_t e = hipFuncSetAttribute((const void*)distill_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(distill_kernel, dim3((unsigned)grid), dim3(64 * kDW), lds, st, a);
  return hipGetLastError();
}

// Pooling backward: dk_idx rows of blocks [b0, b1) from dkbar: each of the
// block's 4 keys gets dkbar rotated back (angle -(4b + 3)) divided by 4.
__global__ __launch_bounds__(256) void pool_backward_kernel(const float* dkbar, int64_t nb_cap,
                                                            float* dk, int64_t n_cap, int B,
                                                            int64_t b0, int64_t nblk, int r,
                                                            int R, double log2_theta) {
  const int lane = threadIdx.x & 63;
  const int64_t job = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (job >= (int64_t)B * nblk) return;
  const int64_t b = job / nblk, j = b0 + job % nblk;
  const float* src = dkbar + (b * nb_cap + j) * 128;
  const int half = R / 2;
  float v[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = lane + 64 * i;
    float x = src[c];
    if (c < R) {
      const int jj = c < half ? c : c - half;
      float cs, sn;
      rope_cs((j + 1) * r - 1, jj, R, log2_theta, &cs, &sn);
      const float y = src[c < half ? c + half : c - half];
      x = c < half ? (x * cs + y * sn) : (x * cs - y * sn);
    }
    v[i] = x / (float)r;
  }
  for (int t = 0; t < r; ++t) {
    float* dst = dk + (b * n_cap + j * r + t) * 128;
    dst[lane] = v[0];
    dst[lane + 64] = v[1];
  }
}

hipError_t launch_pool_backward(const float* dkbar, int64_t nb_cap, float* dk, int64_t n_cap,
                                int B, int64_t b0, int64_t b1, int r, int R, double log2_theta,
                                hipStream_t st) {
  const int64_t jobs = (int64_t)B * (b1 - b0);
  if (jobs == 0) return hipSuccess;
  hipLaunchKernelGGL(pool_backward_kernel, dim3((unsigned)((jobs + 3) / 4)), dim3(256), 0, st,
                     dkbar, nb_cap, dk, n_cap, B, b0, b1 - b0, r, R, log2_theta);
  return hipGetLastError();
}

}  // namespace qsa
