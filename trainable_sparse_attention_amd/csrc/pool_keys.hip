// Pooled indexer keys: block mean over r tokens, then partial RoPE at the
// block's last position (research-hub note, "Key ideas", QSA bullet: keys
// avg-pooled into blocks of r, partial RoPE 64/128 after compression).
//
// HBM-bound stream: each block reads r * d_idx inputs and writes d_idx
// outputs.  One 64-lane wave per block; lane c covers dims c and c + 64.
// Means are taken in float, the rotation in float with cos/sin formed from
// a double angle, and the result is rounded once to the storage type.
#include "qsa_internal.h"

namespace qsa {

template <typename T>
__global__ __launch_bounds__(256) void pool_keys_kernel(const T* __restrict__ k_idx,
                                                        int64_t n_cap, T* __restrict__ kbar,
                                                        int64_t nb_cap, int B, int64_t b0,
                                                        int64_t nblk, int r, int R,
                                                        double log2_theta) {
  __shared__ float mean_s[4][128];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t job = (int64_t)blockIdx.x * 4 + wv;  // (sequence, block) pair
  const bool live = job < (int64_t)B * nblk;
  int64_t b = 0, j = 0;
  if (live) {
    b = job / nblk;
    j = b0 + job % nblk;
    const T* src = k_idx + ((int64_t)b * n_cap + j * r) * 128;
    for (int c = lane; c < 128; c += 64) {
      float s = 0.f;
      for (int t = 0; t < r; ++t) s += Elt<T>::ld(src, (int64_t)t * 128 + c);
      mean_s[wv][c] = s / (float)r;
    }
  }
  __syncthreads();
  if (!live) return;
  const int64_t pos = (j + 1) * r - 1;
  const int half = R / 2;
  T* dst = kbar + ((int64_t)b * nb_cap + j) * 128;
  for (int c = lane; c < 128; c += 64) {
    float out;
    if (c < R) {
      const int jj = c < half ? c : c - half;
      float cs, sn;
      rope_cs(pos, jj, R, log2_theta, &cs, &sn);
      const float a = mean_s[wv][jj], bb = mean_s[wv][jj + half];
      out = c < half ? (a * cs - bb * sn) : (a * sn + bb * cs);
    } else {
      out = mean_s[wv][c];
    }
    Elt<T>::st(dst, c, out);
  }
}

hipError_t launch_pool(qsa_dtype dt, const qsa_params& p, const void* k_idx, int64_t n_cap,
                       void* kbar, int64_t nb_cap, int B, int64_t b0, int64_t b1,
                       hipStream_t st) {
  const int64_t nblk = b1 - b0;
  const int64_t jobs = (int64_t)B * nblk;
  if (jobs == 0) return hipSuccess;
  const dim3 grid((unsigned)((jobs + 3) / 4)), block(256);
  const double l2t = log2((double)p.rope_theta);
  if (dt == QSA_BF16)
    hipLaunchKernelGGL(pool_keys_kernel<unsigned short>, grid, block, 0, st,
                       (const unsigned short*)k_idx, n_cap, (unsigned short*)kbar, nb_cap, B, b0,
                       nblk, p.r, p.rope_dims, l2t);
  else
    hipLaunchKernelGGL(pool_keys_kernel<float>, grid, block, 0, st, (const float*)k_idx, n_cap,
                       (float*)kbar, nb_cap, B, b0, nblk, p.r, p.rope_dims, l2t);
  return hipGetLastError();
}

}  // namespace qsa
