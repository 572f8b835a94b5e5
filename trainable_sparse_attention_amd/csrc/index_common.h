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
// max(x, 0) as one integer max on the bit pattern: negative floats (sign bit
// set, -0 included) are negative as int32 and become +0.
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}
__device__ __forceinline__ float relu_sum4(const f32x4& acc) {
  return relu(acc[0]) + relu(acc[1]) + relu(acc[2]) + relu(acc[3]);  // >= +0
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
  // Four row tiles against one B fragment, the chains interleaved so that
  // consecutive MFMAs are independent.
  template <int NLO, int NA>
  __device__ __forceinline__ static void dot4(const Frag (*a)[4], const Frag (*alo)[NA],
                                              const Frag* b, f32x4* acc) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c < NLO) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[r][c < NLO ? c : 0], b[c], acc[r], 0,
                                                          0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r][c], b[c], acc[r], 0, 0, 0);
    }
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
  template <int NLO, int NA>
  __device__ __forceinline__ static void dot4(const Frag (*a)[32], const Frag (*)[NA],
                                              const Frag* b, f32x4* acc) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 32; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[r] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r][c], b[c], acc[r], 0, 0, 0);
  }
};

typedef float f32x16 __attribute__((ext_vector_type(16)));

// 32x32 score tiles for the many-row indexer.  A tile holds 8 queries x 4
// heads (rows 4q + h) by 32 blocks (columns); lane (n = lane%32, g =
// lane/32) receives, in accumulator elements 4j..4j+3, the 4 heads of query
// 2j + g for block n (j = 0..3).
//   bf16: v_mfma_f32_32x32x16_bf16, 8 k-steps over 128 dims; the lane
//         operand of step c is dims 16c + 8g .. 16c + 8g + 7.  NLO leading
//         steps (the rotated dims) also carry the query's bf16 low part.
//   fp32: v_mfma_f32_32x32x2f32, 64 k-steps; the lane operand of step c is
//         dim 64g + c.
template <typename T> struct Mma32;

typedef unsigned int u32x32 __attribute__((ext_vector_type(32)));
typedef unsigned int u32x16 __attribute__((ext_vector_type(16)));
typedef float f32x64 __attribute__((ext_vector_type(64)));

template <> struct Mma32<unsigned short> {
  static constexpr int kSteps = 8;
  static constexpr bool kSplit = true;
  // one row tile's (or one B tile's) operands for all 8 steps, as a single
  // vector value so that it stays in registers: step c = dwords 4c..4c+3
  typedef u32x32 Tile;
  __device__ __forceinline__ static bf16x8 step(const Tile& t, int c) {
    const u32x4 v = {t[4 * c], t[4 * c + 1], t[4 * c + 2], t[4 * c + 3]};
    return __builtin_bit_cast(bf16x8, v);
  }
  // hi operands of one row held as 128 floats; the lo operands of the NLO
  // rotated steps go to lo[c * 64] (LDS) when write_lo
  template <int NLO>
  __device__ __forceinline__ static Tile a_from_f32(const float* row, int g, u16x8* lo,
                                                    bool write_lo) {
    Tile hi;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const f32x4 v0 = *(const f32x4*)(row + 16 * c + 8 * g);
      const f32x4 v1 = *(const f32x4*)(row + 16 * c + 8 * g + 4);
      u16x8 h, l;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = j < 4 ? v0[j] : v1[j - 4];
        unsigned short h16, l16;
        split_bf16(v, &h16, &l16);
        h[j] = h16;
        l[j] = l16;
      }
      const u32x4 hw = __builtin_bit_cast(u32x4, h);
#pragma unroll
      for (int j = 0; j < 4; ++j) hi[4 * c + j] = hw[j];
      if constexpr (NLO > 0) {
        if (c < NLO && write_lo) lo[(c < NLO ? c : 0) * 64] = l;
      }
    }
    return hi;
  }
  // B operands of block row `row` of an LDS stage whose 16-byte chunks are
  // stored at chunk ^ (row & 15) (conflict-free for 16 consecutive rows).
  __device__ __forceinline__ static Tile load_b(const unsigned short* stage, int row, int g) {
    const unsigned char* rb = (const unsigned char*)stage + row * 256;
    Tile t;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const u32x4 v = *(const u32x4*)(rb + (((2 * c + g) ^ (row & 15)) << 4));
#pragma unroll
      for (int j = 0; j < 4; ++j) t[4 * c + j] = v[j];
    }
    return t;
  }
  // B operands of step c of block row `row` (layout of load_b)
  __device__ __forceinline__ static bf16x8 load_b_step(const unsigned short* stage, int row,
                                                       int g, int c) {
    const unsigned char* rb = (const unsigned char*)stage + row * 256;
    return __builtin_bit_cast(bf16x8, *(const u32x4*)(rb + (((2 * c + g) ^ (row & 15)) << 4)));
  }
  // lo operands of the NLO rotated steps of one row tile, in registers
  typedef u32x16 LoTile;
  template <int NLO>
  __device__ __forceinline__ static void a_from_f32_reg(const float* row, int g, Tile& hi,
                                                        LoTile& lo) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const f32x4 v0 = *(const f32x4*)(row + 16 * c + 8 * g);
      const f32x4 v1 = *(const f32x4*)(row + 16 * c + 8 * g + 4);
      u16x8 h, l;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = j < 4 ? v0[j] : v1[j - 4];
        unsigned short h16, l16;
        split_bf16(v, &h16, &l16);
        h[j] = h16;
        l[j] = l16;
      }
      const u32x4 hw = __builtin_bit_cast(u32x4, h);
      const u32x4 lw = __builtin_bit_cast(u32x4, l);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hi[4 * c + j] = hw[j];
        if (c < NLO && c < 4) lo[4 * (c & 3) + j] = lw[j];
      }
    }
  }
  // one row tile against one B tile
  template <int NLO>
  __device__ __forceinline__ static f32x16 mma1(const Tile& a, const LoTile& lo, const Tile& b) {
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const bf16x8 bc = step(b, c);
      if (c < NLO && c < 4) {
        const u32x4 lv = {lo[4 * (c & 3)], lo[4 * (c & 3) + 1], lo[4 * (c & 3) + 2],
                          lo[4 * (c & 3) + 3]};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, lv), bc, acc, 0,
                                                      0, 0);
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(step(a, c), bc, acc, 0, 0, 0);
    }
    return acc;
  }
  // one row tile against the B operands of block row `row` of an LDS stage,
  // each step's operand read just before its MFMAs
  template <int NLO>
  __device__ __forceinline__ static f32x16 mma1_lds(const Tile& a, const LoTile& lo,
                                                    const unsigned short* stage, int row, int g) {
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const bf16x8 bc = load_b_step(stage, row, g, c);
      if (c < NLO && c < 4) {
        const u32x4 lv = {lo[4 * (c & 3)], lo[4 * (c & 3) + 1], lo[4 * (c & 3) + 2],
                          lo[4 * (c & 3) + 3]};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, lv), bc, acc, 0,
                                                      0, 0);
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(step(a, c), bc, acc, 0, 0, 0);
    }
    return acc;
  }
  // two row tiles against one B tile, the two chains interleaved; the lo
  // part of each rotated step (LDS, lo[(r * NLO + c) * 64 + lane]) goes into
  // the same chain
  template <int NLO>
  __device__ __forceinline__ static void mma2(const Tile& a0, const Tile& a1, const u16x8* lo,
                                              int lane, const Tile& b, f32x16& acc0,
                                              f32x16& acc1) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      acc0[e] = 0.f;
      acc1[e] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const bf16x8 bc = step(b, c);
      if (c < NLO) {
        const int cc = c < NLO ? c : 0;
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, lo[cc * 64 + lane]), bc, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, lo[(NLO + cc) * 64 + lane]), bc, acc1, 0, 0, 0);
      }
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(step(a0, c), bc, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(step(a1, c), bc, acc1, 0, 0, 0);
    }
  }
};

template <> struct Mma32<float> {
  static constexpr int kSteps = 64;
  static constexpr bool kSplit = false;
  typedef f32x64 Tile;
  template <int NLO>
  __device__ __forceinline__ static Tile a_from_f32(const float* row, int g, u16x8*, bool) {
    Tile hi;
#pragma unroll
    for (int c = 0; c < 64; c += 4) {
      const f32x4 v = *(const f32x4*)(row + 64 * g + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) hi[c + j] = v[j];
    }
    return hi;
  }
  __device__ __forceinline__ static Tile load_b(const float* stage, int row, int g) {
    const unsigned char* rb = (const unsigned char*)stage + row * 512;
    Tile t;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const f32x4 v = *(const f32x4*)(rb + (((16 * g + c) ^ (row & 15)) << 4));
#pragma unroll
      for (int j = 0; j < 4; ++j) t[4 * c + j] = v[j];
    }
    return t;
  }
  typedef u32x16 LoTile;
  template <int NLO>
  __device__ __forceinline__ static void a_from_f32_reg(const float* row, int g, Tile& hi,
                                                        LoTile&) {
    hi = a_from_f32<NLO>(row, g, nullptr, false);
  }
  template <int NLO>
  __device__ __forceinline__ static f32x16 mma1(const Tile& a, const LoTile&, const Tile& b) {
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int c = 0; c < 64; ++c) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[c], b[c], acc, 0, 0, 0);
    return acc;
  }
  template <int NLO>
  __device__ __forceinline__ static void mma2(const Tile& a0, const Tile& a1, const u16x8*, int,
                                              const Tile& b, f32x16& acc0, f32x16& acc1) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      acc0[e] = 0.f;
      acc1[e] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < 64; ++c) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a0[c], b[c], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a1[c], b[c], acc1, 0, 0, 0);
    }
  }
};

// Wave-wide: among c candidate scores (bit patterns of non-negative floats,
// read through get(e) for e < c; entries in ascending block order), find the
// k-th largest score v (1 <= k <= c) and how many entries equal to v belong
// to the top k (krem): the top k are every entry with score > v plus the
// first krem entries with score == v (smaller block ids win ties).
// Radix select, 8 bits per pass, starting below the leading bits all entries
// share (so the first digit already spreads the entries over the bins).
// `hist` is 256 words of LDS private to the wave.
// The entries are visited through each(f), which calls f(score bits) for
// every entry the calling lane owns (each entry owned by exactly one lane);
// s0 is any one entry's score.
template <typename Each>
__device__ __forceinline__ void wave_radix_kth_each(Each each, uint32_t s0, int k, uint32_t* hist,
                                                    int lane, uint32_t* v_out, int* krem_out) {
  uint32_t diff = 0;
  each([&](uint32_t sb) { diff |= sb ^ s0; });
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) diff |= __shfl_xor(diff, off);
  int hi = diff ? 31 - __clz(diff) : -1;  // highest bit that differs
  const uint32_t common = hi < 0 ? ~0u : (hi >= 31 ? 0u : ~((2u << hi) - 1u));
  uint32_t prefix = s0 & common, pmask = common;
  int krem = k;
  while (hi >= 0) {
    const int shift = hi >= 7 ? hi - 7 : 0;
    const uint32_t dmask = (2u << (hi - shift)) - 1u;
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[4 * lane + i] = 0;
    wave_sync();
    each([&](uint32_t sb) {
      if ((sb & pmask) == prefix) atomicAdd(&hist[(sb >> shift) & dmask], 1u);
    });
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
    pmask |= dmask << shift;
    hi = shift - 1;
    wave_sync();
  }
  *v_out = prefix;
  *krem_out = krem;
}

// The same over entries e < c read through get(e); lane L owns e = L + 64 j.
template <typename Get>
__device__ __forceinline__ void wave_radix_kth(Get get, int c, int k, uint32_t* hist, int lane,
                                               uint32_t* v_out, int* krem_out) {
  wave_radix_kth_each(
      [&](auto f) {
        for (int e = lane; e < c; e += 64) f(get(e));
      },
      get(0), k, hist, lane, v_out, krem_out);
}

// The same over scores held in registers: lane L holds entry L + 64 j in
// sc[j] (c is wave-uniform), so no pass reads memory for them.
template <int J>
__device__ __forceinline__ void wave_radix_kth_regs(const uint32_t (&sc)[J], int c, int k,
                                                    uint32_t* hist, int lane, uint32_t* v_out,
                                                    int* krem_out) {
  wave_radix_kth_each(
      [&](auto f) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
          if (64 * j >= c) break;
          if (lane + 64 * j < c) f(sc[j]);
        }
      },
      (uint32_t)__shfl((int)sc[0], 0), k, hist, lane, v_out, krem_out);
}

// Wave-wide, order-preserving: keep the top-k entries (per wave_radix_kth)
// of the first c entries of buf (64-bit keys, score bits high, block id low).
// mode 0 writes the kept keys back into buf[0..k); mode 1 writes their block
// ids to ids[0..k) and pads ids[k..kB) with -1.  Reads 4 chunks of 64 keys
// ahead so that global loads overlap.
__device__ __forceinline__ void wave_keep_topk(uint64_t* buf, int c, int k, uint32_t v, int krem,
                                               int lane, int mode, int32_t* ids, int kB) {
  const uint64_t lt = lanemask_lt(lane);
  int written = 0, eq_seen = 0;
  for (int base = 0; base < c; base += 256) {
    uint64_t keys[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = base + 64 * j + lane;
      keys[j] = e < c ? buf[e] : 0ull;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = base + 64 * j + lane;
      const bool valid = e < c;
      const uint32_t sb = (uint32_t)(keys[j] >> 32);
      const bool gt = valid && sb > v;
      const bool eq = valid && sb == v;
      const uint64_t beq = __ballot(eq);
      const int eq_rank = eq_seen + __popcll(beq & lt);
      const bool keep = gt || (eq && eq_rank < krem);
      const uint64_t bk = __ballot(keep);
      const int pos = written + __popcll(bk & lt);
      if (keep && pos < k) {
        if (mode == 0)
          buf[pos] = keys[j];
        else
          ids[pos] = (int32_t)(uint32_t)keys[j];
      }
      written += __popcll(bk);
      eq_seen += __popcll(beq);
    }
  }
  if (mode == 1)
    for (int e = k + lane; e < kB; e += 64) ids[e] = -1;
}

// Copy the score words of c keys into LDS (lsc), 8 loads in flight per lane.
__device__ __forceinline__ void stage_scores(const uint64_t* buf, int c, uint32_t* lsc, int lane) {
  for (int base = 0; base < c; base += 512) {
    uint64_t keys[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = base + 64 * j + lane;
      keys[j] = e < c ? buf[e] : 0ull;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = base + 64 * j + lane;
      if (e < c) lsc[e] = (uint32_t)(keys[j] >> 32);
    }
  }
  wave_sync();
}

}  // namespace qsa
