// Backward of the sparse core attention (joint sparse training, research-hub
// note, "Key ideas", native-trainability bullet; paperglide reader, "Qwen
// Sparse Attention", Figure 3 for the token sets).  The block selection is a
// discrete choice and receives no gradient.
//
// The gradient of a key row gathers over every query that attended it, so
// the work is split by who owns the output:
//   query side, one 64-lane wave per (sequence, query row, KV head), as in
//   the forward (the hq/hkv query heads of the KV head are the 16 columns
//   of the MFMA tiles); the row's token set is walked twice in chunks of 32
//   keys (cyclically from a phase that grows with the position, as in the
//   forward), each chunk's K and V copied into LDS:
//     pass 1: S^T = K Q^T (v_mfma_f32_16x16x32_bf16), per-head log-sum-exp;
//     pass 2: S^T again, P^T = 2^(S^T log2(e) scale - lse), dP^T = V dO^T,
//             dS^T = P^T (dP^T - Dsum) with Dsum = <dO, O> per head, and
//             dQ^T += K^T dS^T (K^T read transposed from LDS);
//     the row's lse and Dsum per head go to the workspace.
//   the selection transposed: per sequence, the rows that selected each
//   block, as lists in ascending row order (count, scan, scatter, sort);
//   key side, one wave per (sequence, KV head, block): the block's r keys
//   against its rows, 16 (row, head) pairs a step staged in LDS, the next
//   step's rows in flight while a step is computed:
//     S = Q K^T and dP = dO V^T (16x16x32), P and dS from the staged lse and
//     Dsum, then dK^T += Q^T dS and dV^T += dO^T P (v_mfma_f32_16x16x16_bf16,
//     Q^T and dO^T read transposed from LDS); the rows whose incomplete block
//     is this one add their tails (key position <= row position).  A key
//     row is owned by one wave, so dK and dV take one plain add each.
// Inputs bf16; dq written, dk and dv added to, all float32.
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
constexpr int kSortCap = 16384;  // longest block row list sorted in LDS

// chunk c of key row kk at c ^ 2(kk & 7) (rows read straight and transposed)
__device__ __forceinline__ int bswz(int kk, int c) { return c ^ ((kk & 7) << 1); }

// LDS byte address of a pointer into workgroup memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(p);
}

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

struct BwdWs {
  float* lse;      // [B][n_q][hq] base-2 log-sum-exp of the scaled logits
  float* dsum;     // [B][n_q][hq] <dout, out>
  int32_t* cnt;    // [B][nbk + 1] rows per block, then the scatter's cursors
  int32_t* off;    // [B][nbk + 1] start of each block's row list
  int32_t* rows;   // [B][ld] the row lists, block after block
  int64_t nbk;     // blocks holding keys some row attends
  int64_t ld;      // list entries per sequence (n_q * k_B)
};

// Query side.  RR: tokens per block (r); SPC = 32 / RR slots per chunk.
template <int RR>
__global__ __launch_bounds__(64) void attn_bwd_q_kernel(AttnArgs a, const unsigned short* dout,
                                                        float* dq, float* lse_out,
                                                        float* dsum_out, int resident) {
  constexpr int SPC = kBwdKeys / RR;
  __shared__ __attribute__((aligned(16))) unsigned short kl[kBwdKeys * 128];
  __shared__ __attribute__((aligned(16))) unsigned short vl[kBwdKeys * 128];
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
  const int64_t rowh = ((int64_t)b * a.n_q + t) * a.hq + head;  // (row, head) index
  const int64_t rowq = rowh * 128;

  auto slot_ntok = [&](int u) { return u < cnt ? RR : (u < nslots ? ntail : 0); };
  auto slot_blk = [&](int u) -> int64_t { return u < cnt ? (int64_t)ids[u] : nb; };
  // key kk of the chunk at slot s: in the set?
  auto key_ok = [&](int s, int kk) { return kk % RR < slot_ntok(s + kk / RR); };

  // Q^T and dO^T as B operands (column hl = head, dims 32cc + 8gq)
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
  // Chunks are visited cyclically from a phase that grows with the row's
  // position (and so with the launch order), as in the forward: the
  // resident waves then read the same narrow window of the history at a
  // time and share it in the caches.  The phase depends on the position and
  // the device's occupancy only, so repeated calls sum in the same order.
  int ph = 0;
  if (resident > 0 && nch > 0) ph = (int)(((pos * a.hkv + g) * nch / resident) % nch);
  auto chunk_at = [&](int cc) { return cc + ph < nch ? cc + ph : cc + ph - nch; };

  // ---- pass 1: log-sum-exp (base 2) of each head's logits --------------
  // a running maximum and sum per lane, rescaled once per chunk
  float m = -INFINITY, l = 0.f;
  for (int cc = 0; cc < nch; ++cc) {
    const int s = SPC * chunk_at(cc);
    load_chunk(s, false);
    f32x4 sacc[2];
    rows_times(kl, qb, sacc);
    float x[8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        x[4 * kt + i] = key_ok(s, 16 * kt + 4 * gq + i) ? sacc[kt][i] * sl2 : -INFINITY;
    float mx = m;
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = fmaxf(mx, x[j]);
    if (mx != -INFINITY) {
      float acc = m == -INFINITY ? 0.f : l * exp2f(m - mx);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += exp2f(x[j] - mx);
      l = acc;
      m = mx;
    }
    __syncthreads();
  }
  const float mm = xmax(m);
  const float lse = mm + log2f(xsum(m == -INFINITY ? 0.f : l * exp2f(m - mm)));
  if (hv && gq == 0) {
    lse_out[rowh] = lse;
    dsum_out[rowh] = dsum;
  }

  // ---- pass 2: dq --------------------------------------------------------
  f32x4 dqa[8];
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) dqa[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int cc = 0; cc < nch; ++cc) {
    const int s = SPC * chunk_at(cc);
    load_chunk(s, true);
    f32x4 sacc[2], dpacc[2];
    rows_times(kl, qb, sacc);
    rows_times(vl, ob, dpacc);
    // dS for column hl, keys 16kt + 4gq + i
    float ds[8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = hv && key_ok(s, 16 * kt + 4 * gq + i);
        const float pv = ok ? exp2f(sacc[kt][i] * sl2 - lse) : 0.f;
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

// ---- the selection transposed ----------------------------------------------
// Per sequence: cnt[j] rows selected block j, off[j] the start of block j's
// list in rows[] (off[nbk] = the sequence's total), rows[] the row indices.

__global__ __launch_bounds__(256) void bwd_clear_kernel(int32_t* p, int64_t n) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256)
    p[e] = 0;
}

// one wave per query row: count (or, with scatter, place) its selected blocks
template <bool SCATTER>
__global__ __launch_bounds__(256) void bwd_count_kernel(AttnArgs a, BwdWs w) {
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)a.B * a.n_q;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows;
       row += (int64_t)gridDim.x * 4) {
    const int b = (int)(row / a.n_q), t = (int)(row % a.n_q);
    const int c = a.cnt[row];
    const int32_t* ids = a.idx + row * a.kB;
    int32_t* cb = w.cnt + (int64_t)b * (w.nbk + 1);
    for (int u = lane; u < c; u += 64) {
      const int j = ids[u];
      if (j < 0 || j >= w.nbk) continue;  // not a block of these rows (never from index_topk)
      if (SCATTER) {
        const int at = atomicAdd(&cb[j], 1);
        w.rows[(int64_t)b * w.ld + at] = t;
      } else {
        atomicAdd(&cb[j], 1);
      }
    }
  }
}

// one workgroup per sequence: off = exclusive scan of cnt; cnt = off (the
// scatter's cursors)
__global__ __launch_bounds__(1024) void bwd_scan_kernel(BwdWs w) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t carry;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int32_t* cb = w.cnt + (int64_t)blockIdx.x * (w.nbk + 1);
  int32_t* ob = w.off + (int64_t)blockIdx.x * (w.nbk + 1);
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int64_t j0 = 0; j0 <= w.nbk; j0 += 1024) {
    const int64_t j = j0 + tid;
    const int32_t v = j < w.nbk ? cb[j] : 0;
    int32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int32_t before = carry;
    for (int x = 0; x < wv; ++x) before += wsum[x];
    if (j <= w.nbk) {
      ob[j] = before + incl - v;
      cb[j] = before + incl - v;
    }
    __syncthreads();
    if (tid == 1023) carry = before + incl;
    __syncthreads();
  }
}

// one workgroup per (sequence, block): the block's list in ascending row
// order (a bitonic sort in LDS), so that the key side sums in a fixed order;
// longer lists than kSortCap stay in the scatter's order
__global__ __launch_bounds__(1024) void bwd_sort_kernel(BwdWs w) {
  __shared__ int32_t v[kSortCap];
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x / w.nbk, j = blockIdx.x % w.nbk;
  const int32_t* ob = w.off + b * (w.nbk + 1);
  const int32_t o0 = ob[j], L = ob[j + 1] - o0;
  if (L < 2 || L > kSortCap) return;
  int n2 = 2;
  while (n2 < L) n2 <<= 1;
  int32_t* src = w.rows + b * w.ld + o0;
  for (int e = tid; e < n2; e += 1024) v[e] = e < L ? src[e] : 0x7fffffff;
  __syncthreads();
  for (int k = 2; k <= n2; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int e = tid; e < n2; e += 1024) {
        const int p = e ^ jj;
        if (p > e) {
          const bool up = (e & k) == 0;
          const int32_t x = v[e], y = v[p];
          if ((x > y) == up) {
            v[e] = y;
            v[p] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int e = tid; e < L; e += 1024) src[e] = v[e];
}

// Key side.  One wave per (sequence, KV head, block j).  16 (row, head) pairs
// per step: RB = floor(16 / G) rows, pair i = (row i / G, head g G + i % G);
// Q and dO rows staged in LDS [pair][128] under the bswz swizzle.
template <int RR>
__global__ __launch_bounds__(64) void attn_bwd_kv_kernel(AttnArgs a, const unsigned short* dout,
                                                         BwdWs w, float* dk, float* dv) {
  // two step buffers: one step's Q and dO rows are computed on while the
  // next step's are in flight.  buf[s] holds step buffer s: Q rows, then dO
  // rows (16 pairs x 256 bytes each).  The compute reads them in inline asm
  // (the compiler would otherwise wait for the loads into the other buffer
  // before every read), after an explicit wait for the step's own loads.
  __shared__ __attribute__((aligned(16))) unsigned short buf[2][2 * 16 * 128];
  __shared__ __attribute__((aligned(16))) float stat[2][2][16];  // [buffer][lse, Dsum][pair]
  __shared__ __attribute__((aligned(16))) int32_t rid[2][16];    // list entries of a step
  const int lane = threadIdx.x, hl = lane & 15, gq = lane >> 4;
  int64_t wi = blockIdx.x;
  const int64_t j = wi % w.nbk;
  wi /= w.nbk;
  const int g = (int)(wi % a.hkv);
  const int b = (int)(wi / a.hkv);
  const int G = a.hq / a.hkv;
  const int RB = 16 / G;
  const int64_t key0 = j * RR;  // first key position of the block
  // the block's rows: its list, then the rows whose incomplete block it is
  // (positions key0 .. key0 + RR - 2 within the call's rows)
  const int32_t* ob = w.off + (int64_t)b * (w.nbk + 1);
  const int32_t L = ob[j + 1] - ob[j];
  const int32_t* list = w.rows + (int64_t)b * w.ld + ob[j];
  const int64_t tp0 = key0 > a.q_pos0 ? key0 : a.q_pos0;
  int64_t tp1 = key0 + RR - 2;
  if (tp1 > a.q_pos0 + a.n_q - 1) tp1 = a.q_pos0 + a.n_q - 1;
  const int ntr = tp1 >= tp0 ? (int)(tp1 - tp0 + 1) : 0;
  const int total = L + ntr;
  if (total == 0) return;
  const int nsteps = (total + RB - 1) / RB;
  const char* kb = (const char*)a.k + ((int64_t)b * a.hkv + g) * a.n_cap * 256;
  const char* vb = (const char*)a.v + ((int64_t)b * a.hkv + g) * a.n_cap * 256;
  // K and V of the block as B operands: column hl = key hl (zero past RR
  // and past the cache's end), dims 32c + 8gq
  const bool kin = hl < RR && key0 + hl < a.n_cap;
  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    u16x8 x = {0, 0, 0, 0, 0, 0, 0, 0}, y = x;
    if (kin) {
      x = *(const u16x8*)(kb + (key0 + hl) * 256 + (32 * c + 8 * gq) * 2);
      y = *(const u16x8*)(vb + (key0 + hl) * 256 + (32 * c + 8 * gq) * 2);
    }
    kf[c] = __builtin_bit_cast(bf16x8, x);
    vf[c] = __builtin_bit_cast(bf16x8, y);
  }
  f32x4 dka[8], dva[8];
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) dka[tt] = dva[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sl2 = a.scale * 1.4426950408889634f;
  const unsigned short* qg = (const unsigned short*)a.q;

  // A step takes RB rows x G heads = 16 (row, head) pairs; lane hl (of every
  // lane group) stands for pair hl: row slot hl / G, head g G + hl % G.
  // The row of pair hl at step n (index within the call's rows; -1: none).
  auto step_row = [&](int n) -> int32_t {
    const int k = n * RB + hl / G;
    if (n >= nsteps || hl / G >= RB || k >= total) return -1;
    return k < L ? list[k] : (int32_t)(tp0 - a.q_pos0) + (k - L);
  };
  // the same from the list entry v that fetch_rows brought for step n
  auto row_from = [&](int n, int32_t v) -> int32_t {
    const int k = n * RB + hl / G;
    if (n >= nsteps || hl / G >= RB || k >= total) return -1;
    return k < L ? v : (int32_t)(tp0 - a.q_pos0) + (k - L);
  };
  // lanes 0..15 copy pair hl's list entry of step n into rid[sl] (any
  // valid word when the pair has none).  1 vector memory instruction.
  auto fetch_rows = [&](int n, int sl) {
    if (lane < 16) {
      const int k = n * RB + hl / G;
      const int32_t* src = L > 0 ? list + (k < L ? k : L - 1) : ob + j;
      __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)rid[sl], 4, 0, 0);
    }
  };
  auto pair_index = [&](int32_t t, int pr) -> int64_t {  // (row, head) index
    return ((int64_t)b * a.n_q + (t >= 0 ? t : 0)) * a.hq + g * G + pr % G;
  };
  // the step's Q and dO rows into buffer bf: instruction i moves pairs
  // 4i + lane / 16 (chunk lane & 15 of each row; absent rows read row 0
  // of the sequence and are masked later), then lanes 0..15 move their
  // pair's lse and Dsum.  10 vector memory instructions.
  auto issue = [&](int32_t t, int bf) {
    unsigned short* qd = buf[bf];
    unsigned short* od = buf[bf] + 16 * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pr = 4 * i + (lane >> 4);
      const uint64_t off = (uint64_t)pair_index(__shfl(t, pr), pr) * 256 + 16 * bswz(pr, lane & 15);
      __builtin_amdgcn_global_load_lds((glb_void_t*)((const char*)qg + off),
                                       (lds_void_t*)(qd + i * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((glb_void_t*)((const char*)dout + off),
                                       (lds_void_t*)(od + i * 512), 16, 0, 0);
    }
    if (lane < 16) {
      const int64_t rh = pair_index(t, hl);
      __builtin_amdgcn_global_load_lds((glb_void_t*)(w.lse + rh), (lds_void_t*)stat[bf][0], 4, 0,
                                       0);
      __builtin_amdgcn_global_load_lds((glb_void_t*)(w.dsum + rh), (lds_void_t*)stat[bf][1], 4,
                                       0, 0);
    }
  };

  // Pipeline: at step n, the rows of step n + 1 are known (their list
  // entries were fetched a step earlier), step n + 2's list entries and
  // step n + 1's rows, lse and Dsum are fetched, then step n is computed
  // once its own loads (the vector memory instructions before the newest
  // 11) have landed.  Inside the loop every global read goes straight to
  // LDS and is read back in inline asm after an explicit wait, so no
  // register waits on a load in flight.
  int32_t t_cur = step_row(0);
  fetch_rows(1, 1);
  issue(t_cur, 0);
  for (int n = 0; n < nsteps; ++n) {
    const int cur = n & 1;
    int32_t t_n1 = -1;
    if (n + 1 < nsteps) {
      // step n + 1's list entries (fetched before step n's 10 loads)
      int32_t v;
      asm volatile(
          "s_waitcnt vmcnt(10)\n"
          "ds_read_b32 %0, %1\n"
          "s_waitcnt lgkmcnt(0)\n"
          : "=&v"(v)
          : "v"(lds_addr(&rid[(n + 1) & 1][hl]))
          : "memory");
      t_n1 = row_from(n + 1, v);
      fetch_rows(n + 2, n & 1);  // 1 instruction
      issue(t_n1, cur ^ 1);      // 10
      asm volatile("s_waitcnt vmcnt(11)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    const unsigned short* qc = buf[cur];
    // S = Q K^T, dP = dO V^T: lane (key hl, pairs 4gq + e); A rows = pair
    // hl, dims 32c + 8gq (the dO rows sit 4096 bytes after the Q rows)
    s16x8 qa[4], oa[4];
    f32x4 lsev, dsv;  // lse and Dsum of pairs 4gq + e
    {
      uint32_t ad[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) ad[c] = lds_addr(qc + hl * 128 + 8 * bswz(hl, 4 * c + gq));
      const uint32_t as = lds_addr(&stat[cur][0][4 * gq]);
      asm volatile(
          "ds_read_b128 %0, %10\n"
          "ds_read_b128 %1, %11\n"
          "ds_read_b128 %2, %12\n"
          "ds_read_b128 %3, %13\n"
          "ds_read_b128 %4, %10 offset:4096\n"
          "ds_read_b128 %5, %11 offset:4096\n"
          "ds_read_b128 %6, %12 offset:4096\n"
          "ds_read_b128 %7, %13 offset:4096\n"
          "ds_read_b128 %8, %14\n"
          "ds_read_b128 %9, %14 offset:64\n"
          "s_waitcnt lgkmcnt(0)\n"
          : "=&v"(qa[0]), "=&v"(qa[1]), "=&v"(qa[2]), "=&v"(qa[3]), "=&v"(oa[0]), "=&v"(oa[1]),
            "=&v"(oa[2]), "=&v"(oa[3]), "=&v"(lsev), "=&v"(dsv)
          : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(as)
          : "memory");
    }
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, dpa = sa;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[c]), kf[c], sa,
                                                   0, 0, 0);
      dpa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, oa[c]), vf[c], dpa,
                                                    0, 0, 0);
    }
    s16x4 pb, db;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pr = 4 * gq + e, rr = pr / G;
      const int32_t t = __shfl(t_cur, pr);
      const float lse = lsev[e], dsm = dsv[e];
      // a listed row attends the whole block; a tail row the keys up to
      // its own position
      const bool ok = kin && t >= 0 && (n * RB + rr < L || key0 + hl <= a.q_pos0 + t);
      const float p = ok ? exp2f(sa[e] * sl2 - lse) : 0.f;
      const float d = p * (dpa[e] - dsm);
      pb[e] = __builtin_bit_cast(short, (__bf16)p);
      db[e] = __builtin_bit_cast(short, (__bf16)d);
    }
    // dK^T += Q^T dS, dV^T += dO^T P: A = Q^T / dO^T read transposed (dims
    // 16tt + hl, pairs 4gq .. 4gq + 3), B = dS / P (pairs, key hl)
    // (ds_read_b64_tr_b16, as tr16: lane i of a 16-lane group receives
    // element i % 4 of the 8-byte rows addressed by lanes 4j + i / 4)
    {
      const int kk = 4 * gq + (hl >> 2);
      const int e0 = 4 * (hl & 1);
      uint32_t ad[8];
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
        ad[tt] = lds_addr(qc + kk * 128 + bswz(kk, 2 * tt + ((hl & 3) >> 1)) * 8 + e0);
      s16x4 qt[8], ot[8];
      asm volatile(
          "ds_read_b64_tr_b16 %0, %16\n"
          "ds_read_b64_tr_b16 %1, %17\n"
          "ds_read_b64_tr_b16 %2, %18\n"
          "ds_read_b64_tr_b16 %3, %19\n"
          "ds_read_b64_tr_b16 %4, %20\n"
          "ds_read_b64_tr_b16 %5, %21\n"
          "ds_read_b64_tr_b16 %6, %22\n"
          "ds_read_b64_tr_b16 %7, %23\n"
          "ds_read_b64_tr_b16 %8, %16 offset:4096\n"
          "ds_read_b64_tr_b16 %9, %17 offset:4096\n"
          "ds_read_b64_tr_b16 %10, %18 offset:4096\n"
          "ds_read_b64_tr_b16 %11, %19 offset:4096\n"
          "ds_read_b64_tr_b16 %12, %20 offset:4096\n"
          "ds_read_b64_tr_b16 %13, %21 offset:4096\n"
          "ds_read_b64_tr_b16 %14, %22 offset:4096\n"
          "ds_read_b64_tr_b16 %15, %23 offset:4096\n"
          "s_waitcnt lgkmcnt(0)\n"
          : "=&v"(qt[0]), "=&v"(qt[1]), "=&v"(qt[2]), "=&v"(qt[3]), "=&v"(qt[4]), "=&v"(qt[5]),
            "=&v"(qt[6]), "=&v"(qt[7]), "=&v"(ot[0]), "=&v"(ot[1]), "=&v"(ot[2]), "=&v"(ot[3]),
            "=&v"(ot[4]), "=&v"(ot[5]), "=&v"(ot[6]), "=&v"(ot[7])
          : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
            "v"(ad[7])
          : "memory");
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        dka[tt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(qt[tt], db, dka[tt], 0, 0, 0);
        dva[tt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ot[tt], pb, dva[tt], 0, 0, 0);
      }
    }
    t_cur = t_n1;
    // the next iteration refills this step's buffers
    __builtin_amdgcn_wave_barrier();
  }
  // dK^T tile tt: lane (key hl, dims 16tt + 4gq + e); one owner per key row
  if (kin) {
    const int64_t row = ((int64_t)b * a.hkv + g) * a.n_cap + key0 + hl;
    float* dkr = dk + row * 128;
    float* dvr = dv + row * 128;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const int d0 = 16 * tt + 4 * gq;
      f32x4 x = *(f32x4*)(dkr + d0), y = *(f32x4*)(dvr + d0);
      x += dka[tt] * a.scale;
      y += dva[tt];
      *(f32x4*)(dkr + d0) = x;
      *(f32x4*)(dvr + d0) = y;
    }
  }
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static BwdWs carve_bwd(void* ws, int B, int n_q, int64_t q_pos0, int hq, int r, int kB,
                       size_t* total) {
  BwdWs w;
  w.nbk = (q_pos0 + n_q) / r + 1;
  w.ld = (int64_t)n_q * kB;
  char* p = (char*)ws;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* q = p ? p + off : nullptr;
    off += align256(bytes);
    return q;
  };
  w.lse = (float*)take((size_t)B * n_q * hq * sizeof(float));
  w.dsum = (float*)take((size_t)B * n_q * hq * sizeof(float));
  w.cnt = (int32_t*)take((size_t)B * (w.nbk + 1) * sizeof(int32_t));
  w.off = (int32_t*)take((size_t)B * (w.nbk + 1) * sizeof(int32_t));
  w.rows = (int32_t*)take((size_t)B * w.ld * sizeof(int32_t));
  if (total) *total = off;
  return w;
}

size_t attn_backward_workspace(int B, int n_q, int64_t q_pos0, int hq, int r, int kB) {
  size_t total = 0;
  carve_bwd(nullptr, B, n_q, q_pos0, hq, r, kB, &total);
  return total;
}

// The period of the query side's chunk phase: its waves resident on the
// whole device at once (occupancy of the current device), times 0.9 as for
// the forward (slots refill with a lag).  0 if the query fails: no phase.
template <int RR>
static int bwd_resident_waves() {
  static thread_local int dev_cached = -1, res_cached = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev == dev_cached) return res_cached;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_bwd_q_kernel<RR>, 64, 0) !=
          hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  dev_cached = dev;
  res_cached = per_cu * cus * 9 / 10;
  return res_cached;
}

template <int RR>
static hipError_t launch_bwd_r(const AttnArgs& a, const unsigned short* d, float* dq, float* dk,
                               float* dv, const BwdWs& w, hipStream_t st) {
  const int64_t waves = (int64_t)a.B * a.n_q * a.hkv;
  hipLaunchKernelGGL(attn_bwd_q_kernel<RR>, dim3((unsigned)waves), dim3(64), 0, st, a, d, dq,
                     w.lse, w.dsum, bwd_resident_waves<RR>());
  const int64_t rows = (int64_t)a.B * a.n_q;
  const unsigned cg = (unsigned)((rows + 3) / 4 < 65536 ? (rows + 3) / 4 : 65536);
  const int64_t ncnt = (int64_t)a.B * (w.nbk + 1);
  hipLaunchKernelGGL(bwd_clear_kernel, dim3((unsigned)((ncnt + 255) / 256 < 4096
                                                           ? (ncnt + 255) / 256 : 4096)),
                     dim3(256), 0, st, w.cnt, ncnt);
  hipLaunchKernelGGL(bwd_count_kernel<false>, dim3(cg), dim3(256), 0, st, a, w);
  hipLaunchKernelGGL(bwd_scan_kernel, dim3((unsigned)a.B), dim3(1024), 0, st, w);
  hipLaunchKernelGGL(bwd_count_kernel<true>, dim3(cg), dim3(256), 0, st, a, w);
  hipLaunchKernelGGL(bwd_sort_kernel, dim3((unsigned)(a.B * w.nbk)), dim3(1024), 0, st, w);
  hipLaunchKernelGGL(attn_bwd_kv_kernel<RR>, dim3((unsigned)(a.B * a.hkv * w.nbk)), dim3(64), 0,
                     st, a, d, w, dk, dv);
  return hipGetLastError();
}

hipError_t launch_attn_backward(const AttnArgs& a, const void* dout, float* dq, float* dk,
                                float* dv, void* ws, hipStream_t st) {
  if ((int64_t)a.B * a.n_q * a.hkv == 0) return hipSuccess;
  const BwdWs w = carve_bwd(ws, a.B, a.n_q, a.q_pos0, a.hq, a.r, a.kB, nullptr);
  const unsigned short* d = (const unsigned short*)dout;
  switch (a.r) {
    case 1: return launch_bwd_r<1>(a, d, dq, dk, dv, w, st);
    case 2: return launch_bwd_r<2>(a, d, dq, dk, dv, w, st);
    case 8: return launch_bwd_r<8>(a, d, dq, dk, dv, w, st);
    case 16: return launch_bwd_r<16>(a, d, dq, dk, dv, w, st);
    default: return launch_bwd_r<4>(a, d, dq, dk, dv, w, st);
  }
}

}  // namespace qsa
