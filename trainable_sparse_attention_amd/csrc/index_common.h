// Device helpers shared by the indexer kernels: wave-level synchronisation,
// MFMA fragment traits for the block-score contraction, and the exact,
// order-preserving top-k selection over a candidate list.
#pragma once

#include "qsa_internal.h"

namespace qsa {

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// ReLU-sum over the 4 indexer heads held by one lane of a 16x16 MFMA tile
// (rows 4g..4g+3 are the heads of one query), sign of zero cleared so that
// the float bits order like the values.
__device__ __forceinline__ float relu_sum4(const f32x4& acc) {
  const float s = fmaxf(acc[0], 0.f) + fmaxf(acc[1], 0.f) + fmaxf(acc[2], 0.f) + fmaxf(acc[3], 0.f);
  return __uint_as_float(__float_as_uint(s) & 0x7fffffffu);
}

// q = hi + lo with hi = bf16(q) and lo = bf16(q - hi): the pair carries
// 16 significant bits, so a rotated query keeps float-level accuracy in the
// bf16 contraction (bf16 x bf16 products are exact in the fp32 accumulator).
__device__ __forceinline__ void split_bf16(float v, unsigned short* hi, unsigned short* lo) {
  *hi = f32_to_bf16(v);
  *lo = f32_to_bf16(v - bf16_to_f32(*hi));
}

// Score contraction traits.  A 16x16 output tile holds 4 queries x 4 heads
// (rows) by 16 blocks (columns); lane (hl = lane%16, g = lane/16) receives
// the 4 heads of query g for block hl.
//   bf16: v_mfma_f32_16x16x32_bf16, 4 calls over 128 dims; lane operand of
//         call c = dims 32c + 8g .. 32c + 8g + 7.
//   fp32: v_mfma_f32_16x16x4f32, 32 calls; lane operand of call c = dim
//         32g + c.
// NLO: number of leading 32-dim steps that hold rotated dims (ceil(R/32)),
// the only steps whose bf16 query operand needs a low part.
template <typename T> struct Mma;

template <> struct Mma<unsigned short> {
  static constexpr int kCalls = 4;
  static constexpr bool kSplit = true;  // rotated query dims carry a bf16 low part
  typedef bf16x8 Frag;
  // Fragment of row `row` (16 rows stored [16][ld] in LDS, bf16).
  __device__ __forceinline__ static void load_lds(const unsigned short* base, int ld_elems,
                                                  int row, int g, Frag* f) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      f[c] = __builtin_bit_cast(bf16x8, *(const u16x8*)(base + row * ld_elems + 32 * c + 8 * g));
  }
  __device__ __forceinline__ static void load_glb(const unsigned short* row_ptr, int g, Frag* f) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      f[c] = __builtin_bit_cast(bf16x8, *(const u16x8*)(row_ptr + 32 * c + 8 * g));
  }
  // <a_hi + a_lo, b>: a_lo is non-zero only in the first NLO 32-dim steps
  // (the rotated dims), so only those steps are issued twice.
  template <int NLO>
  __device__ __forceinline__ static f32x4 dot(const Frag* a, const Frag* alo, const Frag* b) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c < NLO) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[c], b[c], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[c], b[c], acc, 0, 0, 0);
    }
    return acc;
  }
};

template <> struct Mma<float> {
  static constexpr int kCalls = 32;
  static constexpr bool kSplit = false;
  typedef float Frag;
  __device__ __forceinline__ static void load_lds(const float* base, int ld_elems, int row, int g,
                                                  Frag* f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const f32x4 v = *(const f32x4*)(base + row * ld_elems + 32 * g + 4 * e);
      f[4 * e] = v[0];
      f[4 * e + 1] = v[1];
      f[4 * e + 2] = v[2];
      f[4 * e + 3] = v[3];
    }
  }
  __device__ __forceinline__ static void load_glb(const float* row_ptr, int g, Frag* f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const f32x4 v = *(const f32x4*)(row_ptr + 32 * g + 4 * e);
      f[4 * e] = v[0];
      f[4 * e + 1] = v[1];
      f[4 * e + 2] = v[2];
      f[4 * e + 3] = v[3];
    }
  }
  template <int NLO>
  __device__ __forceinline__ static f32x4 dot(const Frag* a, const Frag* /*alo*/, const Frag* b) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 32; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[c], b[c], acc, 0, 0, 0);
    return acc;
  }
};

// Wave-wide: among the first c entries of `buf` (64-bit keys: score bits in
// the high word, block id in the low word; entries in ascending block order),
// find the k-th largest score v (k <= c) and how many entries equal to v
// belong to the top k (krem): the top k are every entry with score > v plus
// the first krem entries with score == v (smaller block ids win ties).
// `hist` is 256 words of LDS private to the wave.
__device__ __forceinline__ void wave_radix_kth(const uint64_t* buf, int c, int k, uint32_t* hist,
                                               int lane, uint32_t* v_out, int* krem_out) {
  uint32_t prefix = 0, pmask = 0;
  int krem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[4 * lane + i] = 0;
    wave_sync();
    for (int e = lane; e < c; e += 64) {
      const uint32_t sb = (uint32_t)(buf[e] >> 32);
      if ((sb & pmask) == prefix) atomicAdd(&hist[(sb >> shift) & 255u], 1u);
    }
    wave_sync();
    // lane L owns bins 4L..4L+3; count of entries in bins above lane L's.
    uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
             h3 = hist[4 * lane + 3];
    const uint32_t mine = h0 + h1 + h2 + h3;
    uint32_t incl = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_down(incl, off);
      if (lane + off < 64) incl += y;
    }
    const uint32_t above = incl - mine;
    int digit = -1;
    uint32_t above_digit = 0;
    if (above < (uint32_t)krem && incl >= (uint32_t)krem) {
      uint32_t run = above;
      const uint32_t hh[4] = {h0, h1, h2, h3};
      for (int bb = 3; bb >= 0; --bb) {
        if (run + hh[bb] >= (uint32_t)krem) {
          digit = 4 * lane + bb;
          above_digit = run;
          break;
        }
        run += hh[bb];
      }
    }
    const uint64_t who = __ballot(digit >= 0);
    if (who == 0) {  // only if c < k: keep the search in range
      digit = 0;
      above_digit = 0;
    } else {
      const int src = __ffsll((long long)who) - 1;
      digit = __shfl(digit, src);
      above_digit = __shfl(above_digit, src);
    }
    krem -= (int)above_digit;
    prefix |= ((uint32_t)digit) << shift;
    pmask |= 255u << shift;
    wave_sync();
  }
  *v_out = prefix;
  *krem_out = krem;
}

// Wave-wide, order-preserving: keep the top-k entries (per wave_radix_kth)
// of the first c entries.  mode 0 writes the kept keys back into buf[0..k);
// mode 1 writes their block ids to ids[0..k) and pads ids[k..kB) with -1.
__device__ __forceinline__ void wave_keep_topk(uint64_t* buf, int c, int k, uint32_t v, int krem,
                                               int lane, int mode, int32_t* ids, int kB) {
  const uint64_t lt = lanemask_lt(lane);
  int written = 0, eq_seen = 0;
  for (int base = 0; base < c; base += 64) {
    const int e = base + lane;
    const bool valid = e < c;
    const uint64_t key = valid ? buf[e] : 0ull;
    const uint32_t sb = (uint32_t)(key >> 32);
    const bool gt = valid && sb > v;
    const bool eq = valid && sb == v;
    const uint64_t beq = __ballot(eq);
    const int eq_rank = eq_seen + __popcll(beq & lt);
    const bool keep = gt || (eq && eq_rank < krem);
    const uint64_t bk = __ballot(keep);
    const int pos = written + __popcll(bk & lt);
    if (keep && pos < k) {
      if (mode == 0)
        buf[pos] = key;
      else
        ids[pos] = (int32_t)(uint32_t)key;
    }
    written += __popcll(bk);
    eq_seen += __popcll(beq);
  }
  if (mode == 1)
    for (int e = k + lane; e < kB; e += 64) ids[e] = -1;
}

}  // namespace qsa
