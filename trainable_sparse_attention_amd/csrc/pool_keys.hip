// Pooled indexer keys: the mean of each block's r keys, then a rotation of the
// leading rope_dims dims at the block's last position (research-hub note,
// "Key ideas", QSA bullet: pooling into micro-blocks, partial RoPE applied
// after the compression).  Optionally the mean is RMS-normalised with a
// learned gain before the rotation (paperglide reader, "Qwen Sparse
// Attention": its toy normalises the pooled keys).
//
// HBM-bound stream: each block reads r * d_idx inputs and writes d_idx
// outputs.  One 64-lane wave per block; lane c covers dims c and c + 64.
// A decode step pools one block per sequence, where the fp64 angle
// reduction, not the bytes, sets the time: it overlaps the key loads.
// Means are taken in float, the rotation in float with cos/sin formed from
// a double angle, and the result is rounded once to the storage type.
#include "qsa_internal.h"

namespace qsa {

__device__ __forceinline__ uint32_t raw_bits(unsigned short x) { return x; }
__device__ __forceinline__ uint32_t raw_bits(float x) { return __float_as_uint(x); }
template <typename T> __device__ __forceinline__ float from_bits(uint32_t x);
template <> __device__ __forceinline__ float from_bits<unsigned short>(uint32_t x) {
  return __uint_as_float(x << 16);
}
template <> __device__ __forceinline__ float from_bits<float>(uint32_t x) {
  return __uint_as_float(x);
}

// NORM: the block mean is RMS-normalised with gain gamma before the
// rotation (m * gamma / sqrt(mean(m^2) + eps)).
template <typename T, bool NORM>
__global__ __launch_bounds__(256) void pool_keys_kernel(const T* __restrict__ k_idx,
                                                        int64_t n_cap, T* __restrict__ kbar,
                                                        int64_t nb_cap, int B, int64_t b0,
                                                        int64_t nblk, int r, int R,
                                                        double log2_theta,
                                                        const float* __restrict__ gamma,
                                                        float eps) {
  __shared__ float mean_s[4][128];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t job = (int64_t)blockIdx.x * 4 + wv;  // (sequence, block) pair
  const bool live = job < (int64_t)B * nblk;
  const int64_t b = live ? job / nblk : 0, j = live ? b0 + job % nblk : 0;
  const int64_t pos = (j + 1) * r - 1;
  const int half = R / 2;
  // the first four keys of the block are loaded, then the rotation factors
  // of this lane's columns c = lane, lane + 64 (those below R) are formed
  // while the loads are in flight
  const T* src = k_idx + ((int64_t)b * n_cap + j * r) * 128;
  // (token min(t, r - 1): every load stays inside the block and none waits
  // on a per-load branch; the sum below takes only tokens t < r)
  uint32_t v[2][4] = {};  // raw bits: converted only after the factors exist
  if (live) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        v[i][t] = raw_bits(src[(int64_t)min(t, r - 1) * 128 + lane + 64 * i]);
  }
  float cs[2] = {1.f, 1.f}, sn[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = lane + 64 * i;
    if (live && c < R) rope_cs(pos, c < half ? c : c - half, R, log2_theta, &cs[i], &sn[i]);
  }
  // the raw values pass through an empty asm that also reads the factors,
  // so the wait for the loads is placed after the factors are formed
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t)
      asm volatile("" : "+v"(v[i][t]) : "v"(cs[0]), "v"(sn[0]), "v"(cs[1]), "v"(sn[1]));
  float mv[2] = {0.f, 0.f};
  if (live) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float s = 0.f;
      for (int t = 0; t < r; ++t)
        s += t < 4 ? from_bits<T>(v[i][t]) : Elt<T>::ld(src, (int64_t)t * 128 + lane + 64 * i);
      mv[i] = s / (float)r;
    }
  }
  if constexpr (NORM) {
    // the wave holds the block's 128 means (two per lane)
    float ss = mv[0] * mv[0] + mv[1] * mv[1];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off);
    const float inv = 1.f / sqrtf(ss / 128.f + eps);
#pragma unroll
    for (int i = 0; i < 2; ++i) mv[i] = mv[i] * inv * gamma[lane + 64 * i];
  }
  if (live) {
#pragma unroll
    for (int i = 0; i < 2; ++i) mean_s[wv][lane + 64 * i] = mv[i];
  }
  __syncthreads();
  if (!live) return;
  T* dst = kbar + ((int64_t)b * nb_cap + j) * 128;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = lane + 64 * i;
    float out;
    if (c < R) {
      const int jj = c < half ? c : c - half;
      const float a = mean_s[wv][jj], bb = mean_s[wv][jj + half];
      out = c < half ? (a * cs[i] - bb * sn[i]) : (a * sn[i] + bb * cs[i]);
    } else {
      out = mean_s[wv][c];
    }
    Elt<T>::st(dst, c, out);
  }
}

hipError_t launch_pool(qsa_dtype dt, const qsa_params& p, const void* k_idx, int64_t n_cap,
                       void* kbar, int64_t nb_cap, int B, int64_t b0, int64_t b1,
                       const float* gamma, float eps, hipStream_t st) {
  const int64_t nblk = b1 - b0;
  const int64_t jobs = (int64_t)B * nblk;
  if (jobs == 0) return hipSuccess;
  const dim3 grid((unsigned)((jobs + 3) / 4)), block(256);
  const double l2t = log2((double)p.rope_theta);
  if (dt == QSA_BF16) {
    if (gamma)
      hipLaunchKernelGGL((pool_keys_kernel<unsigned short, true>), grid, block, 0, st,
                         (const unsigned short*)k_idx, n_cap, (unsigned short*)kbar, nb_cap, B,
                         b0, nblk, p.r, p.rope_dims, l2t, gamma, eps);
    else
      hipLaunchKernelGGL((pool_keys_kernel<unsigned short, false>), grid, block, 0, st,
                         (const unsigned short*)k_idx, n_cap, (unsigned short*)kbar, nb_cap, B,
                         b0, nblk, p.r, p.rope_dims, l2t, gamma, eps);
  } else {
    if (gamma)
      hipLaunchKernelGGL((pool_keys_kernel<float, true>), grid, block, 0, st,
                         (const float*)k_idx, n_cap, (float*)kbar, nb_cap, B, b0, nblk, p.r,
                         p.rope_dims, l2t, gamma, eps);
    else
      hipLaunchKernelGGL((pool_keys_kernel<float, false>), grid, block, 0, st,
                         (const float*)k_idx, n_cap, (float*)kbar, nb_cap, B, b0, nblk, p.r,
                         p.rope_dims, l2t, gamma, eps);
  }
  return hipGetLastError();
}

}  // namespace qsa
