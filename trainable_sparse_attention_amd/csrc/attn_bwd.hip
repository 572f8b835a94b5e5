// Backward of the sparse core attention (joint sparse training, research-hub
// note, "Key ideas", native-trainability bullet; paperglide reader, "Qwen
// Sparse Attention", Figure 3 for the token sets).  The block selection is a
// discrete choice and receives no gradient.
//
// One 64-lane wave per (sequence, query row, KV head), as in the forward: the
// hq/hkv query heads of the KV head are the 16 columns of the MFMA tiles.
// The row's token set is walked twice in chunks of 32 keys, each chunk's K
// and V copied into LDS (1 KB per global->LDS instruction):
//   pass 1: S^T = K Q^T (v_mfma_f32_16x16x32_bf16), per-column log-sum-exp;
//   pass 2: S^T again, P^T = 2^(S^T log2(e) scale - lse), dP^T = V dO^T,
//           dS^T = P^T (dP^T - Dsum) with Dsum = <dO, O> per head,
//           dQ^T += K^T dS^T (K^T read transposed from LDS, dS^T as the B
//           operand under the same key permutation as P in the forward),
//           dV^T = dO^T P and dK^T = Q^T dS (v_mfma_f32_16x16x16_bf16, P and
//           dS transposed through a small LDS tile), added to dv / dk with
//           float atomics (a key row is shared by every query that selected
//           its block).
// Inputs bf16; dq written, dk and dv accumulated, all float32.
#include <math.h>

#include "qsa_internal.h"

namespace qsa {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kBwdKeys = 32;  // keys per chunk

// chunk c of key row kk at c ^ 2(kk & 7) (rows read straight and transposed)
__device__ __forceinline__ int bswz(int kk, int c) { return c ^ ((kk & 7) << 1); }

__device__ __forceinline__ s16x4 tr16(const unsigned short* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

__device__ __forceinline__ float xmax(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float xsum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

}  // namespace

// RR: tokens per block (r); SPC = 32 / RR slots per chunk.
template <int RR>
__global__ __launch_bounds__(64) void attn_bwd_kernel(AttnArgs a, const unsigned short* dout,
                                                      float* dq, float* dk, float* dv) {
  constexpr int SPC = kBwdKeys / RR;
  __shared__ __attribute__((aligned(16))) unsigned short kl[kBwdKeys * 128];
  __shared__ __attribute__((aligned(16))) unsigned short vl[kBwdKeys * 128];
  __shared__ __attribute__((aligned(16))) unsigned short pl[kBwdKeys * 16];   // P[key][head]
  __shared__ __attribute__((aligned(16))) unsigned short dsl[kBwdKeys * 16];  // dS[key][head]
  const int lane = threadIdx.x, hl = lane & 15, gq = lane >> 4;
  int64_t w = blockIdx.x;
  const int g = (int)(w % a.hkv);
  w /= a.hkv;
  const int t = (int)(w % a.n_q);
  const int b = (int)(w / a.n_q);
  const int G = a.hq / a.hkv;
  const int head = g * G + hl;
  const bool hv = hl < G;
  const int64_t pos = a.q_pos0 + t;
  const int64_t nb = (pos + 1) / RR;
  const int ntail = (int)(pos + 1 - nb * RR);
  const int cnt = a.cnt[(int64_t)b * a.n_q + t];
  const int nslots = cnt + (ntail > 0 ? 1 : 0);
  const int32_t* ids = a.idx + ((int64_t)b * a.n_q + t) * a.kB;
  const char* kb = (const char*)a.k + ((int64_t)b * a.hkv + g) * a.n_cap * 256;
  const char* vb = (const char*)a.v + ((int64_t)b * a.hkv + g) * a.n_cap * 256;
  const int64_t rowq = (((int64_t)b * a.n_q + t) * a.hq + head) * 128;

  auto slot_ntok = [&](int u) { return u < cnt ? RR : (u < nslots ? ntail : 0); };
  auto slot_blk = [&](int u) -> int64_t { return u < cnt ? (int64_t)ids[u] : nb; };
  // key kk of the chunk at slot s: in the set?
  auto key_ok = [&](int s, int kk) { return kk % RR < slot_ntok(s + kk / RR); };

  // Q^T and dO^T as B operands (column hl = head, dims 32cc + 8gq) and as
  // the A operands of the 16x16x16 products (dim row, heads 4gq .. + 3)
  bf16x8 qb[4], ob[4];
  float dsum = 0.f;
  {
    const unsigned short* qr = (const unsigned short*)a.q + rowq;
    const unsigned short* orow = (const unsigned short*)a.out + rowq;
    const unsigned short* dr = dout + rowq;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      u16x8 x = {0, 0, 0, 0, 0, 0, 0, 0}, y = x, z = x;
      if (hv) {
        x = *(const u16x8*)(qr + 32 * cc + 8 * gq);
        y = *(const u16x8*)(dr + 32 * cc + 8 * gq);
        z = *(const u16x8*)(orow + 32 * cc + 8 * gq);
      }
      qb[cc] = __builtin_bit_cast(bf16x8, x);
      ob[cc] = __builtin_bit_cast(bf16x8, y);
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum += bf16_to_f32(y[e]) * bf16_to_f32(z[e]);
    }
  }
  dsum = xsum(dsum);  // <dO, O> of head hl
  // (bf16 bit patterns: the 16x16x16 product takes 16-bit integer vectors)
  s16x4 qa[8], oa[8];
  {
    const int h0 = g * G + 4 * gq;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const int dim = 16 * tt + hl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = 4 * gq + e < G;
        const int64_t off = (((int64_t)b * a.n_q + t) * a.hq + (ok ? h0 + e : 0)) * 128 + dim;
        qa[tt][e] = ok ? (short)((const unsigned short*)a.q)[off] : (short)0;
        oa[tt][e] = ok ? (short)dout[off] : (short)0;
      }
    }
  }

  // chunk at slot s: K and V into LDS (instruction i moves keys 4i .. 4i+3)
  auto load_chunk = [&](int s, bool with_v) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kk = 4 * i + (lane >> 4);
      const int u = s + kk / RR;
      const bool ok = key_ok(s, kk);
      const uint64_t row = ok ? (uint64_t)(slot_blk(u) * RR + kk % RR) : 0ull;
      const uint64_t off = row * 256 + 16 * bswz(kk, lane & 15);
      __builtin_amdgcn_global_load_lds((glb_void_t*)(kb + off), (lds_void_t*)(kl + i * 512), 16,
                                       0, 0);
      if (with_v)
        __builtin_amdgcn_global_load_lds((glb_void_t*)(vb + off), (lds_void_t*)(vl + i * 512),
                                         16, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  // S^T-shaped product of the chunk's rows (K or V) with a 16-column B
  auto rows_times = [&](const unsigned short* src, const bf16x8* bop, f32x4* acc) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int kk = 16 * kt + hl;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const bf16x8 av = *(const bf16x8*)(src + kk * 128 + 8 * bswz(kk, 4 * cc + gq));
        acc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bop[cc], acc[kt], 0, 0, 0);
      }
    }
  };

  const float sl2 = a.scale * 1.4426950408889634f;
  const int nch = (nslots + SPC - 1) / SPC;

  // ---- pass 1: log-sum-exp (base 2) of each head's logits --------------
  float m = -INFINITY, l = 0.f;
  for (int c = 0; c < nch; ++c) {
    const int s = SPC * c;
    load_chunk(s, false);
    f32x4 sacc[2];
    rows_times(kl, qb, sacc);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!key_ok(s, 16 * kt + 4 * gq + i)) continue;
        const float x = sacc[kt][i] * sl2;
        if (x > m) {
          l = l * exp2f(m - x) + 1.f;
          m = x;
        } else {
          l += exp2f(x - m);
        }
      }
    __syncthreads();
  }
  const float mm = xmax(m);
  const float lse = mm + log2f(xsum(m == -INFINITY ? 0.f : l * exp2f(m - mm)));

  // ---- pass 2: gradients -------------------------------------------------
  f32x4 dqa[8];
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) dqa[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float* dkb = dk + ((int64_t)b * a.hkv + g) * a.n_cap * 128;
  float* dvb = dv + ((int64_t)b * a.hkv + g) * a.n_cap * 128;
  for (int c = 0; c < nch; ++c) {
    const int s = SPC * c;
    load_chunk(s, true);
    f32x4 sacc[2], dpacc[2];
    rows_times(kl, qb, sacc);
    rows_times(vl, ob, dpacc);
    // P and dS for column hl, keys 16kt + 4gq + i
    float p[8], ds[8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = hv && key_ok(s, 16 * kt + 4 * gq + i);
        const float pv = ok ? exp2f(sacc[kt][i] * sl2 - lse) : 0.f;
        p[4 * kt + i] = pv;
        ds[4 * kt + i] = pv * (dpacc[kt][i] - dsum);
      }
    // dQ^T += K^T dS^T: B = dS^T with k index 8gq + j <-> key
    // (j < 4 ? 4gq + j : 16 + 4gq + j - 4); A = K^T read transposed
    bf16x8 dsb;
#pragma unroll
    for (int j = 0; j < 8; ++j) dsb[j] = (__bf16)ds[j];
    {
      const int kk = 4 * gq + (hl >> 2);
      const int e0 = 4 * (hl & 1);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int ch = 2 * tt + ((hl & 3) >> 1);
        const s16x4 x0 = tr16(kl + kk * 128 + bswz(kk, ch) * 8 + e0);
        const s16x4 x1 = tr16(kl + (kk + 16) * 128 + bswz(kk + 16, ch) * 8 + e0);
        const s16x8 kv = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
        dqa[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv), dsb,
                                                          dqa[tt], 0, 0, 0);
      }
    }
    // P and dS transposed through LDS: [key][head]
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * kt + 4 * gq + i;
        pl[key * 16 + hl] = __builtin_bit_cast(unsigned short, (__bf16)p[4 * kt + i]);
        dsl[key * 16 + hl] = __builtin_bit_cast(unsigned short, (__bf16)ds[4 * kt + i]);
      }
    __syncthreads();
    // dV^T = dO^T P, dK^T = scale Q^T dS: 16 dims x 16 keys per call, k =
    // 16 heads; lane (key hl, dims 4gq + e)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = 16 * kt + hl;
      const s16x4 pb = *(const s16x4*)(pl + key * 16 + 4 * gq);
      const s16x4 db = *(const s16x4*)(dsl + key * 16 + 4 * gq);
      const int u = s + key / RR;
      const bool ok = key_ok(s, key);
      const int64_t row = ok ? slot_blk(u) * RR + key % RR : 0;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 dva = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(oa[tt], pb, z, 0, 0, 0);
        const f32x4 dka = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(qa[tt], db, z, 0, 0, 0);
        if (ok) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int dim = 16 * tt + 4 * gq + e;
            unsafeAtomicAdd(dvb + row * 128 + dim, dva[e]);
            unsafeAtomicAdd(dkb + row * 128 + dim, dka[e] * a.scale);
          }
        }
      }
    }
    __syncthreads();
  }
  // dQ^T tile tt: lane (head hl, dims 16tt + 4gq + e)
  if (hv) {
    float* dqr = dq + rowq;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      f32x4 x = dqa[tt] * a.scale;
      *(f32x4*)(dqr + 16 * tt + 4 * gq) = x;
    }
  }
}

hipError_t launch_attn_backward(const AttnArgs& a, const void* dout, float* dq, float* dk,
                                float* dv, hipStream_t st) {
  const int64_t waves = (int64_t)a.B * a.n_q * a.hkv;
  if (waves == 0) return hipSuccess;
  const unsigned short* d = (const unsigned short*)dout;
  switch (a.r) {
    case 1:
      hipLaunchKernelGGL(attn_bwd_kernel<1>, dim3((unsigned)waves), dim3(64), 0, st, a, d, dq, dk,
                         dv);
      break;
    case 2:
      hipLaunchKernelGGL(attn_bwd_kernel<2>, dim3((unsigned)waves), dim3(64), 0, st, a, d, dq, dk,
                         dv);
      break;
    case 8:
      hipLaunchKernelGGL(attn_bwd_kernel<8>, dim3((unsigned)waves), dim3(64), 0, st, a, d, dq, dk,
                         dv);
      break;
    case 16:
      hipLaunchKernelGGL(attn_bwd_kernel<16>, dim3((unsigned)waves), dim3(64), 0, st, a, d, dq,
                         dk, dv);
      break;
    default:
      hipLaunchKernelGGL(attn_bwd_kernel<4>, dim3((unsigned)waves), dim3(64), 0, st, a, d, dq, dk,
                         dv);
  }
  return hipGetLastError();
}

}  // namespace qsa
