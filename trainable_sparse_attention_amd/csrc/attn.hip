// Sparse core attention over gathered micro-blocks (paperglide reader,
// "Qwen Sparse Attention", Figure 3: selected block indices expanded into a
// micro-block sparse mask; the incomplete-block tail is always attended).
//
// One 64-lane wave handles one (sequence, query row, KV head, split) and the
// hq/hkv query heads that share the KV head (GQA).  The token set is walked
// in chunks of 32 keys: 32/r slots (a slot is one selected block of r keys,
// or a tail slot); each chunk gathers 8 KB of K and 8 KB of V (r * 256 bytes
// contiguous per block per head in the head-major caches).  r is 1, 2, 4, 8
// or 16 (the micro-block sizes the pages sweep).
//
// bf16: S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16 (16 keys x
//   16 heads per tile, heads beyond hq/hkv are zero); K and V are copied
//   global -> LDS one chunk ahead of the compute (V read transposed for the
//   A operand).  Softmax and accumulation in float (online, base 2).  P is
//   rounded to bf16 for the PV product.
// fp32: the same on v_mfma_f32_16x16x4f32, whose one-element-per-lane
//   operands need no transpose (the output dims are permuted instead).
//
// Decode splits the slots over `nsplit` waves per (row, KV head) and writes
// partial (max, sum, unnormalised output) that attn_combine merges.
#include <math.h>

#include <mutex>

#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr int kChunkKeys = 32;   // keys per chunk: two 16-key MFMA tiles
constexpr int kIdWin = 576;     // slot ids staged in LDS at a time (whole chunks)

struct Row {
  int64_t pos;
  int64_t nb;
  int ntail;
  int cnt;
  int nslots;
  const int32_t* ids;
};

// A row's token set: the cnt selected blocks, then the tail slots, which
// hold the tokens nb*r .. pos (block nb + j is tail slot j).  Ordinarily nb
// is the row's own complete-block count and the tail is its incomplete
// block; when a decode step's new tokens share one selection (made at the
// step's first new token), nb is the first token's count, so a later token's
// tail also covers the blocks completed since.
__device__ __forceinline__ Row row_ctx(const AttnArgs& a, int b, int t) {
  Row R;
  R.pos = a.seq_len ? (int64_t)a.seq_len[b] - a.n_q + t : a.q_pos0 + t;
  const int ts = a.shared ? 0 : t;  // row of the selection this token uses
  const int64_t psel = a.shared ? R.pos - t : R.pos;
  R.nb = (psel + 1) / a.r;
  R.ntail = (int)(R.pos + 1 - R.nb * a.r);
  const int nsel = a.shared ? 1 : a.n_q;
  R.cnt = a.cnt[(int64_t)b * nsel + ts];
  R.nslots = R.cnt + (R.ntail + a.r - 1) / a.r;
  R.ids = a.idx + ((int64_t)b * nsel + ts) * a.kB;
  return R;
}

// Tokens of slot u (< nslots) in the token set: r for a selected block, the
// rest of the tail for a tail slot.
__device__ __forceinline__ int slot_tokens(const Row& R, int u, int r) {
  return u < R.cnt ? r : min(r, R.ntail - (u - R.cnt) * r);
}
// Block of slot u (< nslots).
__device__ __forceinline__ int64_t slot_block(const Row& R, int u) {
  return u < R.cnt ? (int64_t)R.ids[u] : R.nb + (u - R.cnt);
}

// Token row of key `tok` (< r) of slot u; false if the key is not in T_i.
__device__ __forceinline__ bool slot_row(const Row& R, int u, int s1, int tok, int r,
                                         int64_t* row) {
  if (u >= s1 || tok >= slot_tokens(R, u, r)) {
    *row = 0;
    return false;
  }
  *row = slot_block(R, u) * r + tok;
  return true;
}

__device__ __forceinline__ float wave_max_xor(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float wave_sum_xor(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ void decode_job(const AttnArgs& a, int nsplit, int* b, int* t, int* g,
                                           int* split) {
  int64_t w = blockIdx.x;
  *split = (int)(w % nsplit);
  w /= nsplit;
  *g = (int)(w % a.hkv);
  w /= a.hkv;
  *t = (int)(w % a.n_q);
  *b = (int)(w / a.n_q);
}

}  // namespace


typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// V chunk layout in LDS: key row kk (256 bytes) keeps its 16-byte chunk c at
// chunk c ^ 2(kk & 7), so that a transposed read (16 key rows x two
// neighbouring chunks) touches every bank exactly twice.
__device__ __forceinline__ int vswz(int kk, int c) { return c ^ ((kk & 7) << 1); }
// K chunk layout in LDS: key row kk keeps its 16-byte chunk c at c ^ (kk & 15),
// so the 16 key rows one operand read touches fall in 16 distinct bank groups.
__device__ __forceinline__ int kswz(int kk, int c) { return c ^ (kk & 15); }
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i%4
// of the 8-byte rows addressed by lanes 4j + i/4 (j = 0..3), i.e. a 4 x 16
// block of 16-bit values arrives transposed.
__device__ __forceinline__ s16x4 lds_read_tr16(const unsigned short* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}
// LDS byte address of a pointer into workgroup memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(p);
}

// WIN: the row's slots may exceed one LDS window of ids (refilled as the
// scan advances); otherwise every slot id is staged once.  RR: tokens per
// block (r); a chunk holds SPC = 32 / RR slots.
template <bool WIN, int RR>
__global__ __launch_bounds__(64) void attn_bf16_kernel(AttnArgs a, int nsplit, float* part,
                                                       int resident) {
  constexpr int SPC = kChunkKeys / RR;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_attn[];
  unsigned short* vbuf = (unsigned short*)smem_attn;      // V: [32 keys][128]
  unsigned char* kbuf = smem_attn + 32 * 128 * 2;            // K: [32 keys][256 B]
  int* ids = (int*)(smem_attn + 2 * 32 * 128 * 2);          // block of each slot
  const int lane = threadIdx.x;
  const int hl = lane & 15, gq = lane >> 4;
  int b, t, g, split;
  decode_job(a, nsplit, &b, &t, &g, &split);
  const Row R = row_ctx(a, b, t);
  int s0 = 0, s1 = R.nslots;
  if (nsplit > 1) {
    s0 = split * a.split_slots;
    s1 = min(R.nslots, s0 + a.split_slots);
  }
  // Block ids of a window of kIdWin slots from `base` (tail slot j is block
  // nb + j; slots past the set read block 0 and are masked).
  int base = s0;
  // (at most the window, and no further than the chunk that holds slot s1 - 1)
  const int fill_n = min(kIdWin, (s1 - s0 + SPC - 1) / SPC * SPC);
  auto fill_ids = [&](int b0) {
    for (int u = lane; u < fill_n; u += 64) {
      const int sl = b0 + u;
      ids[u] = sl < s1 ? (int)slot_block(R, sl) : 0;
    }
  };
  fill_ids(base);
  __syncthreads();
  // Token row of key tok of slot u with block id `id`, 0 if the key is not
  // in T_i (branch-free).
  auto row_sel = [&](int u, int id, int tok) -> uint32_t {
    const bool ok = u < s1 && tok < slot_tokens(R, u, RR);
    return ok ? (uint32_t)id * (uint32_t)RR + (uint32_t)tok : 0u;
  };
  const int G = a.hq / a.hkv;
  const int head = g * G + hl;
  // K/V rows of this (sequence, KV head); byte offsets within fit 32 bits
  const char* kb = (const char*)a.k + ((int64_t)b * a.hkv + g) * a.n_cap * 256;
  const char* vb = (const char*)a.v + ((int64_t)b * a.hkv + g) * a.n_cap * 256;

  bf16x8 qf[4];
  {
    const unsigned short* qrow =
        (const unsigned short*)a.q + (((int64_t)b * a.n_q + t) * a.hq + head) * 128;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (hl < G) v = *(const u16x8*)(qrow + 32 * cc + 8 * gq);
      qf[cc] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // Block id behind each of a chunk's 8 load instructions (instruction i
  // moves keys 4i .. 4i + 3), read from the id window in LDS.  The reads are
  // waited for inside the asm, so no LDS access the compiler sees overlaps
  // the chunk copies in flight into kbuf / vbuf (it would otherwise wait for
  // them).  r >= 4: one id covers whole instructions (broadcast reads);
  // r < 4: each lane group reads the id of its own key.
  auto chunk_bids = [&](int s, int* bid) {
    const uint32_t a0 = lds_addr(ids + (s - base));
    if constexpr (RR == 4) {
      u32x4 x0, x1;
      asm volatile(
          "s_waitcnt lgkmcnt(0)\n"
          "ds_read_b128 %0, %2\n"
          "ds_read_b128 %1, %2 offset:16\n"
          "s_waitcnt lgkmcnt(0)\n"
          : "=&v"(x0), "=&v"(x1)
          : "v"(a0)
          : "memory");
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bid[i] = (int)x0[i];
        bid[4 + i] = (int)x1[i];
      }
    } else if constexpr (RR == 8) {
      u32x4 x0;
      asm volatile(
          "s_waitcnt lgkmcnt(0)\n"
          "ds_read_b128 %0, %1\n"
          "s_waitcnt lgkmcnt(0)\n"
          : "=&v"(x0)
          : "v"(a0)
          : "memory");
#pragma unroll
      for (int i = 0; i < 8; ++i) bid[i] = (int)x0[i / 2];
    } else if constexpr (RR == 16) {
      u32x2 x0;
      asm volatile(
          "s_waitcnt lgkmcnt(0)\n"
          "ds_read_b64 %0, %1\n"
          "s_waitcnt lgkmcnt(0)\n"
          : "=&v"(x0)
          : "v"(a0)
          : "memory");
#pragma unroll
      for (int i = 0; i < 8; ++i) bid[i] = (int)x0[i / 4];
    } else {
      // key 4i + lane / 16 is slot (4i + lane / 16) / RR: instruction i's id
      // sits 4i / RR words past the lane's first
      const uint32_t al = a0 + 4u * (uint32_t)((lane >> 4) / RR);
      constexpr int kStep = 16 / RR;  // bytes between instructions' ids
      uint32_t x[8];
      asm volatile(
          "s_waitcnt lgkmcnt(0)\n"
          "ds_read_b32 %0, %8\n"
          "ds_read_b32 %1, %8 offset:%9\n"
          "ds_read_b32 %2, %8 offset:%10\n"
          "ds_read_b32 %3, %8 offset:%11\n"
          "ds_read_b32 %4, %8 offset:%12\n"
          "ds_read_b32 %5, %8 offset:%13\n"
          "ds_read_b32 %6, %8 offset:%14\n"
          "ds_read_b32 %7, %8 offset:%15\n"
          "s_waitcnt lgkmcnt(0)\n"
          : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
            "=&v"(x[6]), "=&v"(x[7])
          : "v"(al), "i"(kStep), "i"(2 * kStep), "i"(3 * kStep), "i"(4 * kStep), "i"(5 * kStep),
            "i"(6 * kStep), "i"(7 * kStep)
          : "memory");
#pragma unroll
      for (int i = 0; i < 8; ++i) bid[i] = (int)x[i];
    }
  };
  // One chunk of K or V straight into LDS: instruction i moves keys
  // 4i .. 4i + 3 (1 KB); lane l's 16 bytes land at key 4i + l/16, chunk
  // position l%16 of that key row, so the lane fetches the logical chunk the
  // layout stores there.  Keys outside T_i read row 0 (masked later).
  auto load_chunk = [&](int s, const int* bid, const char* src, unsigned char* dst, bool isk) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kk = 4 * i + (lane >> 4);
      const int pos = isk ? kswz(kk, lane & 15) : vswz(kk, lane & 15);
      const uint32_t off = row_sel(s + kk / RR, bid[i], kk % RR) * 256u + 16u * pos;
      __builtin_amdgcn_global_load_lds((glb_void_t*)(src + off), (lds_void_t*)(dst + i * 1024),
                                       16, 0, 0);
    }
  };
  // K operand addresses: key row hl of tile kt (+4096 bytes for kt = 1),
  // dims 32cc + 8gq .. + 7 = logical chunk 4cc + gq
  uint32_t ka[4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) ka[cc] = lds_addr(kbuf + hl * 256 + 16 * kswz(hl, 4 * cc + gq));
  // V^T operand addresses (see the PV step)
  uint32_t va[8];
  {
    const int kk = 4 * gq + (hl >> 2);
    const int e0 = 4 * (hl & 1);
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const int c = 2 * tt + ((hl & 3) >> 1);
      va[tt] = lds_addr(vbuf + kk * 128 + vswz(kk, c) * 8 + e0);
    }
  }

  const float sl2 = a.scale * 1.4426950408889634f;
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // m is the reference the exponentials are taken against: it follows the
  // running maximum only when that grows by more than 2^8, so P <= 256 and
  // the rescale of o and l is rare.
  float m = -INFINITY, l = 0.f;

  // Chunks are visited cyclically from a phase that grows with the query
  // position (and so with the launch order): block lists are ascending, so
  // the resident waves then read the same narrow window of the history at a
  // time and share it in the caches.  The phase depends on the position, not
  // on the launch index, so a chunked prefill sums in the same order.
  // Copies run one chunk ahead, staggered: the next chunk's K is issued once
  // this chunk's K is in registers, its V once this chunk's V is, so a copy
  // is in flight while the wave computes.
  const int nch = (s1 - s0 + SPC - 1) / SPC;
  int ph = 0;
  if (!WIN && nsplit == 1 && resident > 0 && nch > 0)
    ph = (int)(((R.pos * a.hkv + g) * nch / resident) % nch);
  auto slot_of = [&](int cc) {
    int c = ph + cc;
    if (c >= nch) c -= nch;
    return s0 + SPC * c;
  };
  // make sure the ids of the chunk at slot s are in the window
  auto window = [&](int s) {
    if constexpr (WIN) {
      if (s + SPC - base > kIdWin) {
        base = s;
        fill_ids(base);
      }
    }
  };
  int bid[8];
  if (nch > 0) {
    const int s = slot_of(0);
    window(s);
    chunk_bids(s, bid);
    load_chunk(s, bid, kb, kbuf, true);
    load_chunk(s, bid, vb, (unsigned char*)vbuf, false);
  }
  for (int cc = 0; cc < nch; ++cc) {
    const int s = slot_of(cc);
    const bool more = cc + 1 < nch;
    // this chunk's K has landed (its V, the 8 newest copies, may not have)
    u32x4 kr[8];
    asm volatile(
        "s_waitcnt vmcnt(8)\n"
        "ds_read_b128 %0, %8\n"
        "ds_read_b128 %1, %8 offset:4096\n"
        "ds_read_b128 %2, %9\n"
        "ds_read_b128 %3, %9 offset:4096\n"
        "ds_read_b128 %4, %10\n"
        "ds_read_b128 %5, %10 offset:4096\n"
        "ds_read_b128 %6, %11\n"
        "ds_read_b128 %7, %11 offset:4096\n"
        "s_waitcnt lgkmcnt(0)\n"
        : "=&v"(kr[0]), "=&v"(kr[1]), "=&v"(kr[2]), "=&v"(kr[3]), "=&v"(kr[4]), "=&v"(kr[5]),
          "=&v"(kr[6]), "=&v"(kr[7])
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3])
        : "memory");
    int sn = s;
    if (more) {
      sn = slot_of(cc + 1);
      window(sn);
      chunk_bids(sn, bid);
      load_chunk(sn, bid, kb, kbuf, true);
    }
    // S^T tiles: lane holds head hl, keys 16kt + 4gq + i.
    f32x4 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4)
        sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, kr[2 * c4 + kt]), qf[c4], sacc[kt], 0, 0, 0);
    }
    // key 16kt + 4gq + i of the chunk: slot s + key / RR, token key % RR
    float sv[8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * kt + 4 * gq + i;
        const int u = s + key / RR;
        const bool ok = u < s1 && key % RR < slot_tokens(R, u, RR);
        sv[4 * kt + i] = ok ? sacc[kt][i] * sl2 : -INFINITY;
      }
    }
    float mx = sv[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sv[j]);
    mx = wave_max_xor(mx);
    if (__ballot(mx > m + 8.f)) {
      const float mn = fmaxf(m, mx);
      const float alpha = exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) o[tt] = o[tt] * alpha;
      m = mn;
    }
    float p[8], rs = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = exp2f(sv[j] - m);
      rs += p[j];
    }
    l += wave_sum_xor(rs);
    bf16x8 pf;
#pragma unroll
    for (int j = 0; j < 8; ++j) pf[j] = (__bf16)p[j];
    // O^T tile tt: A row = dim 16tt + hl, k index 8gq + j <-> key
    // (j < 4 ? 4gq + j : 16 + 4gq + j - 4), read transposed: lane hl of group
    // gq addresses key 4gq + hl/4 (+16), dims 16tt + 4(hl%4) .. +3.
    // This chunk's V has landed once at most the next chunk's K copies (8)
    // remain; all of it is read before the next chunk's V is issued.
    s16x4 vr[16];
    if (more) {
      asm volatile(
          "s_waitcnt vmcnt(8)\n"
          "ds_read_b64_tr_b16 %0, %16\n"
          "ds_read_b64_tr_b16 %1, %16 offset:4096\n"
          "ds_read_b64_tr_b16 %2, %17\n"
          "ds_read_b64_tr_b16 %3, %17 offset:4096\n"
          "ds_read_b64_tr_b16 %4, %18\n"
          "ds_read_b64_tr_b16 %5, %18 offset:4096\n"
          "ds_read_b64_tr_b16 %6, %19\n"
          "ds_read_b64_tr_b16 %7, %19 offset:4096\n"
          "ds_read_b64_tr_b16 %8, %20\n"
          "ds_read_b64_tr_b16 %9, %20 offset:4096\n"
          "ds_read_b64_tr_b16 %10, %21\n"
          "ds_read_b64_tr_b16 %11, %21 offset:4096\n"
          "ds_read_b64_tr_b16 %12, %22\n"
          "ds_read_b64_tr_b16 %13, %22 offset:4096\n"
          "ds_read_b64_tr_b16 %14, %23\n"
          "ds_read_b64_tr_b16 %15, %23 offset:4096\n"
          "s_waitcnt lgkmcnt(0)\n"
          : "=&v"(vr[0]), "=&v"(vr[1]), "=&v"(vr[2]), "=&v"(vr[3]), "=&v"(vr[4]), "=&v"(vr[5]),
            "=&v"(vr[6]), "=&v"(vr[7]), "=&v"(vr[8]), "=&v"(vr[9]), "=&v"(vr[10]), "=&v"(vr[11]),
            "=&v"(vr[12]), "=&v"(vr[13]), "=&v"(vr[14]), "=&v"(vr[15])
          : "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]),
            "v"(va[7])
          : "memory");
      load_chunk(sn, bid, vb, (unsigned char*)vbuf, false);
    } else {
      asm volatile(
          "s_waitcnt vmcnt(0)\n"
          "ds_read_b64_tr_b16 %0, %16\n"
          "ds_read_b64_tr_b16 %1, %16 offset:4096\n"
          "ds_read_b64_tr_b16 %2, %17\n"
          "ds_read_b64_tr_b16 %3, %17 offset:4096\n"
          "ds_read_b64_tr_b16 %4, %18\n"
          "ds_read_b64_tr_b16 %5, %18 offset:4096\n"
          "ds_read_b64_tr_b16 %6, %19\n"
          "ds_read_b64_tr_b16 %7, %19 offset:4096\n"
          "ds_read_b64_tr_b16 %8, %20\n"
          "ds_read_b64_tr_b16 %9, %20 offset:4096\n"
          "ds_read_b64_tr_b16 %10, %21\n"
          "ds_read_b64_tr_b16 %11, %21 offset:4096\n"
          "ds_read_b64_tr_b16 %12, %22\n"
          "ds_read_b64_tr_b16 %13, %22 offset:4096\n"
          "ds_read_b64_tr_b16 %14, %23\n"
          "ds_read_b64_tr_b16 %15, %23 offset:4096\n"
          "s_waitcnt lgkmcnt(0)\n"
          : "=&v"(vr[0]), "=&v"(vr[1]), "=&v"(vr[2]), "=&v"(vr[3]), "=&v"(vr[4]), "=&v"(vr[5]),
            "=&v"(vr[6]), "=&v"(vr[7]), "=&v"(vr[8]), "=&v"(vr[9]), "=&v"(vr[10]), "=&v"(vr[11]),
            "=&v"(vr[12]), "=&v"(vr[13]), "=&v"(vr[14]), "=&v"(vr[15])
          : "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]),
            "v"(va[7])
          : "memory");
    }
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const s16x8 vv = __builtin_shufflevector(vr[2 * tt], vr[2 * tt + 1], 0, 1, 2, 3, 4, 5, 6, 7);
      o[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pf, o[tt],
                                                      0, 0, 0);
    }
  }
  if (nsplit == 1) {
    if (hl < G) {
      const float inv = 1.f / l;
      unsigned short* orow =
          (unsigned short*)a.out + (((int64_t)b * a.n_q + t) * a.hq + head) * 128;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        bf16x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (__bf16)(o[tt][i] * inv);
        *(bf16x4*)(orow + 16 * tt + 4 * gq) = w;
      }
    }
  } else {
    float* pp = part + ((((int64_t)b * a.n_q + t) * a.hkv + g) * nsplit + split) * kPartFloats;
    if (gq == 0) {
      pp[hl] = m;
      pp[16 + hl] = l;
    }
    if (hl < G) {  // padding heads are never read
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) *(f32x4*)(pp + 32 + hl * 128 + 16 * tt + 4 * gq) = o[tt];
    }
  }
}

__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a, int nsplit, float* part) {
  const int lane = threadIdx.x;
  const int hl = lane & 15, gq = lane >> 4;
  int b, t, g, split;
  decode_job(a, nsplit, &b, &t, &g, &split);
  const Row R = row_ctx(a, b, t);
  // key k of a chunk at slot s: slot s + k / r, token k % r
  const int r = a.r, spc = kChunkKeys / r;
  int s0 = 0, s1 = R.nslots;
  if (nsplit > 1) {
    s0 = split * a.split_slots;
    s1 = min(R.nslots, s0 + a.split_slots);
  }
  const int G = a.hq / a.hkv;
  const int head = g * G + hl;
  const float* ks = (const float*)a.k + ((int64_t)b * a.hkv + g) * a.n_cap * 128;
  const float* vsrc = (const float*)a.v + ((int64_t)b * a.hkv + g) * a.n_cap * 128;

  // k index of MFMA call cc in lane group gq <-> dim 32 gq + cc.
  float qr[32];
  {
    const float* qrow = (const float*)a.q + (((int64_t)b * a.n_q + t) * a.hq + head) * 128;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (hl < G) v = *(const f32x4*)(qrow + 32 * gq + 4 * e);
      qr[4 * e + 0] = v[0];
      qr[4 * e + 1] = v[1];
      qr[4 * e + 2] = v[2];
      qr[4 * e + 3] = v[3];
    }
  }
  const float sl2 = a.scale * 1.4426950408889634f;
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  for (int s = s0; s < s1; s += spc) {
    f32x4 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      int64_t row;
      const int key = 16 * kt + hl;
      slot_row(R, s + key / r, s1, key % r, r, &row);
      const float* kr = ks + row * 128 + 32 * gq;
      sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const f32x4 kv = *(const f32x4*)(kr + 4 * e);
#pragma unroll
        for (int z = 0; z < 4; ++z)
          sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[z], qr[4 * e + z], sacc[kt], 0, 0, 0);
      }
    }
    float sv[8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int64_t row;
        const int key = 16 * kt + 4 * gq + i;
        const bool ok = slot_row(R, s + key / r, s1, key % r, r, &row);
        sv[4 * kt + i] = ok ? sacc[kt][i] * sl2 : -INFINITY;
      }
    }
    float mx = sv[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sv[j]);
    mx = wave_max_xor(mx);
    const float mn = fmaxf(m, mx);
    const float alpha = exp2f(m - mn);
    float p[8], rs = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = exp2f(sv[j] - mn);
      rs += p[j];
    }
    rs = wave_sum_xor(rs);
    l = l * alpha + rs;
    m = mn;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) o[tt] = o[tt] * alpha;
    // PV: call cc covers keys key(cc, gq) = cc < 4 ? 4gq + cc : 16 + 4gq + cc - 4;
    // output tile tt row m <-> dim 8 m + tt, so each lane reads 8 dims of a key.
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const int key = (cc < 4) ? (4 * gq + cc) : (16 + 4 * gq + cc - 4);
      int64_t row;
      slot_row(R, s + key / r, s1, key % r, r, &row);
      const float* vr = vsrc + row * 128 + 8 * hl;
      const f32x4 v0 = *(const f32x4*)vr;
      const f32x4 v1 = *(const f32x4*)(vr + 4);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const float av = tt < 4 ? v0[tt] : v1[tt - 4];
        o[tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, p[cc], o[tt], 0, 0, 0);
      }
    }
  }

  // Output tile tt row 4gq + i <-> dim 8(4gq + i) + tt.
  if (nsplit == 1) {
    if (hl < G) {
      const float inv = 1.f / l;
      float* orow = (float*)a.out + (((int64_t)b * a.n_q + t) * a.hq + head) * 128;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 lo, hi;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          lo[tt] = o[tt][i] * inv;
          hi[tt] = o[tt + 4][i] * inv;
        }
        *(f32x4*)(orow + 8 * (4 * gq + i)) = lo;
        *(f32x4*)(orow + 8 * (4 * gq + i) + 4) = hi;
      }
    }
  } else {
    float* pp = part + ((((int64_t)b * a.n_q + t) * a.hkv + g) * nsplit + split) * kPartFloats;
    if (gq == 0) {
      pp[hl] = m;
      pp[16 + hl] = l;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 lo, hi;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        lo[tt] = o[tt][i];
        hi[tt] = o[tt + 4][i];
      }
      *(f32x4*)(pp + 32 + hl * 128 + 8 * (4 * gq + i)) = lo;
      *(f32x4*)(pp + 32 + hl * 128 + 8 * (4 * gq + i) + 4) = hi;
    }
  }
}

// Merge split partials: one workgroup per (b, t, query head) of kCombGroups
// groups of 128 threads, thread = output dim; group j sums the splits
// j, j + kCombGroups, ...  Every partial load is issued before the split
// weights 2^(m_s - M) are known, so the merge waits on one round of loads.
constexpr int kCombGroups = 4;
constexpr int kCombUnroll = 17;  // splits per thread kept in registers (65 splits: 17 per group)
template <typename T>
__global__ __launch_bounds__(128 * kCombGroups) void attn_combine_kernel(
    AttnArgs a, int nsplit, const float* __restrict__ part) {
  constexpr int NT = 128 * kCombGroups, NW = NT / 64;
  extern __shared__ float wgt[];  // [nsplit]
  __shared__ float red[2 * NW];
  __shared__ float osum[kCombGroups - 1][128];
  const int tid = threadIdx.x, dim = tid & 127, grp = tid >> 7, lane = tid & 63, wv = tid >> 6;
  int64_t w = blockIdx.x;
  const int h = (int)(w % a.hq);
  w /= a.hq;
  const int t = (int)(w % a.n_q);
  const int b = (int)(w / a.n_q);
  const int G = a.hq / a.hkv;
  const int g = h / G, hl = h % G;
  const float* base = part + (((int64_t)b * a.n_q + t) * a.hkv + g) * nsplit * kPartFloats;
  const float* po = base + 32 + hl * 128 + dim;
  float ov[kCombUnroll];
#pragma unroll
  for (int u = 0; u < kCombUnroll; ++u) {
    const int sp = grp + kCombGroups * u;
    ov[u] = sp < nsplit ? po[(int64_t)sp * kPartFloats] : 0.f;
  }
  float M = -INFINITY;
  for (int sp = tid; sp < nsplit; sp += NT) M = fmaxf(M, base[(int64_t)sp * kPartFloats + hl]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) red[wv] = M;
  __syncthreads();
  M = red[0];
#pragma unroll
  for (int x = 1; x < NW; ++x) M = fmaxf(M, red[x]);
  float L = 0.f;
  for (int sp = tid; sp < nsplit; sp += NT) {
    const float* pp = base + (int64_t)sp * kPartFloats;
    const float ms = pp[hl];
    const float ws = ms == -INFINITY ? 0.f : exp2f(ms - M);
    wgt[sp] = ws;
    L += ws * pp[16 + hl];
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) L += __shfl_xor(L, off);
  __syncthreads();
  if (lane == 0) red[NW + wv] = L;
  __syncthreads();
  L = 0.f;
#pragma unroll
  for (int x = 0; x < NW; ++x) L += red[NW + x];
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < kCombUnroll; ++u) {
    const int sp = grp + kCombGroups * u;
    if (sp < nsplit) acc += wgt[sp] * ov[u];
  }
  for (int sp = grp + kCombGroups * kCombUnroll; sp < nsplit; sp += kCombGroups)
    acc += wgt[sp] * po[(int64_t)sp * kPartFloats];
  if (grp > 0) osum[grp - 1][dim] = acc;
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int x = 0; x < kCombGroups - 1; ++x) acc += osum[x][dim];
    Elt<T>::st((T*)a.out, (((int64_t)b * a.n_q + t) * a.hq + h) * 128 + dim, acc / L);
  }
}

// LDS the bf16 kernel uses: one V chunk and a window of slot ids.
static size_t bf16_lds_need() { return 2 * 32 * 128 * 2 + (size_t)kIdWin * 4; }

// Waves of the prefill bf16 kernel allowed on one CU.  Fewer concurrent waves
// keep the window of the history that the resident waves read at one time
// small enough to be shared in L2; enough remain to keep the gathers in
// flight, two per SIMD (256K-token prefill step, attention: 15 waves per CU
// 45.4 ms, 10 41.0, 9 40.7, 8 39.5, 7 41.7, 6 46.8).  The LDS each wave
// requests enforces the limit.
constexpr int kPrefillWavesPerCu = 8;

// LDS requested per prefill wave: what the kernel uses, or the CU's LDS
// shared by kPrefillWavesPerCu waves if that is more.
static size_t bf16_lds_prefill() {
  static thread_local int dev_cached = -1;
  static thread_local size_t cached = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return bf16_lds_need();
  if (dev == dev_cached) return cached;
  int per_cu = 0;
  size_t bytes = bf16_lds_need();
  if (hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) ==
          hipSuccess &&
      per_cu > 0) {
    const size_t share = ((size_t)per_cu / kPrefillWavesPerCu) & ~(size_t)255;
    if (share > bytes) bytes = share;
  }
  dev_cached = dev;
  cached = bytes;
  return cached;
}

// The period of the prefill kernel's chunk phase: the waves resident on the
// whole device at once, from the occupancy of the current device.  With each
// wave's copies running one chunk ahead, the full occupancy bound aligns
// best (256K-token prefill, attention: 38.5 ms at 1.0 of the bound, 38.8 at
// 0.9, 40.5 at 0.8 and at 1.2); with copies issued only when a chunk was
// computed, 0.9 had (39.2 ms against 39.7 at 1.0).
static int resident_waves() {
  static thread_local int dev_cached = -1, res_cached = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev == dev_cached) return res_cached;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_bf16_kernel<false, 4>, 64,
                                                   bf16_lds_prefill()) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  dev_cached = dev;
  res_cached = per_cu * cus;
  return res_cached;
}

// Tail slots a row can have: its incomplete block, and with a shared
// selection the blocks completed by the step's later tokens as well.
static int max_tail_slots(int r, int n_q, bool shared) {
  const int tail = r - 1 + (shared ? n_q - 1 : 0);
  return (tail + r - 1) / r;
}
// A split of the decode attention is a run of whole chunks (32 / r slots
// each): one chunk while a launch for one new token per sequence stays
// within kDecodeWaves waves, else the fewest chunks (a power of two) that
// keep it there, so that a large batch writes and merges fewer partials.
// The count depends on the batch, the KV heads and the selected blocks
// only: not on the number of new tokens (a token's result does not depend
// on how many tokens share its call) nor on the tail (the shared-selection
// form, with more tail slots, never needs fewer splits than the plain one).
constexpr int64_t kDecodeWaves = 1024;
static int decode_chunks_per_split(int B, int n_q, int hkv, int kB, int r) {
  (void)n_q;
  const int spc = kChunkKeys / r;
  const int64_t rows = (int64_t)B * hkv;
  const int base = (kB + spc - 1) / spc;
  int cps = 1;
  // a split's slots must fit the kernel's slot-id window
  while (2 * cps * spc + spc <= kIdWin && rows * ((base + cps - 1) / cps) > kDecodeWaves) cps *= 2;
  return cps;
}
static int decode_splits(int B, int n_q, int hkv, int kB, int r, bool shared) {
  const int spc = kChunkKeys / r;
  const int slots = spc * decode_chunks_per_split(B, n_q, hkv, kB, r);
  return (kB + max_tail_slots(r, n_q, shared) + slots - 1) / slots;
}

template <bool WIN>
static void launch_bf16(const AttnArgs& a, dim3 grid, size_t lds, hipStream_t st, int nsplit,
                        float* part, int resident) {
  switch (a.r) {
    case 1:
      hipLaunchKernelGGL((attn_bf16_kernel<WIN, 1>), grid, dim3(64), lds, st, a, nsplit, part,
                         resident);
      break;
    case 2:
      hipLaunchKernelGGL((attn_bf16_kernel<WIN, 2>), grid, dim3(64), lds, st, a, nsplit, part,
                         resident);
      break;
    case 8:
      hipLaunchKernelGGL((attn_bf16_kernel<WIN, 8>), grid, dim3(64), lds, st, a, nsplit, part,
                         resident);
      break;
    case 16:
      hipLaunchKernelGGL((attn_bf16_kernel<WIN, 16>), grid, dim3(64), lds, st, a, nsplit, part,
                         resident);
      break;
    default:
      hipLaunchKernelGGL((attn_bf16_kernel<WIN, 4>), grid, dim3(64), lds, st, a, nsplit, part,
                         resident);
  }
}

hipError_t launch_attn_prefill(qsa_dtype dt, const AttnArgs& a, hipStream_t st) {
  const int64_t waves = (int64_t)a.B * a.n_q * a.hkv;
  if (waves == 0) return hipSuccess;
  if (dt == QSA_BF16) {
    // every slot id fits one window
    const int spc = kChunkKeys / a.r;
    if (a.kB + max_tail_slots(a.r, a.n_q, a.shared) + spc <= kIdWin)
      launch_bf16<false>(a, dim3((unsigned)waves), bf16_lds_prefill(), st, 1, nullptr,
                         resident_waves());
    else
      launch_bf16<true>(a, dim3((unsigned)waves), bf16_lds_prefill(), st, 1, nullptr, 0);
  }
  else
    hipLaunchKernelGGL(attn_f32_kernel, dim3((unsigned)waves), dim3(64), 0, st, a, 1,
                       (float*)nullptr);
  return hipGetLastError();
}

size_t attn_decode_workspace(int B, int n_q, int hkv, int kB, int r, bool shared) {
  return (size_t)B * n_q * hkv * decode_splits(B, n_q, hkv, kB, r, shared) * kPartFloats *
         sizeof(float);
}

// ---- fixed scratch for the allocation-free decode entry point -------------
// Each device that runs the library holds one copy of this array until the
// process ends; its address on the current device is looked up once per
// device (hipGetSymbolAddress) and kept.  Host code never passes the array's
// name to a kernel: only the looked-up device address.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t attn_static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_attn_decode(qsa_dtype dt, const AttnArgs& args, void* ws, hipStream_t st) {
  AttnArgs a = args;
  a.split_slots = kChunkKeys / a.r * decode_chunks_per_split(a.B, a.n_q, a.hkv, a.kB, a.r);
  const int nsplit = decode_splits(a.B, a.n_q, a.hkv, a.kB, a.r, a.shared);
  const int64_t waves = (int64_t)a.B * a.n_q * a.hkv * nsplit;
  if (waves == 0) return hipSuccess;
  float* part = (float*)ws;
  if (dt == QSA_BF16)
    launch_bf16<false>(a, dim3((unsigned)waves), bf16_lds_need(), st, nsplit, part, 0);
  else
    hipLaunchKernelGGL(attn_f32_kernel, dim3((unsigned)waves), dim3(64), 0, st, a, nsplit, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one split writes the output itself (no partials to merge)
  return nsplit > 1 ? launch_attn_combine(dt, a, nsplit, part, st) : hipSuccess;
}

hipError_t launch_attn_combine(qsa_dtype dt, const AttnArgs& a, int nsplit, const float* part,
                               hipStream_t st) {
  const dim3 cg((unsigned)((int64_t)a.B * a.n_q * a.hq));
  if (dt == QSA_BF16)
    hipLaunchKernelGGL(attn_combine_kernel<unsigned short>, cg, dim3(128 * kCombGroups),
                       nsplit * sizeof(float), st, a, nsplit, part);
  else
    hipLaunchKernelGGL(attn_combine_kernel<float>, cg, dim3(128 * kCombGroups),
                       nsplit * sizeof(float), st, a, nsplit, part);
  return hipGetLastError();
}

}  // namespace qsa
