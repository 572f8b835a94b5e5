// Compressed MQA indexer + streaming top-k_B for many query rows (prefill).
// (research-hub note, "Key ideas", QSA bullet: I_ib = sum_h ReLU(<q_i^h,
// kbar_b>), top-k_B = ceil(K/r); paperglide reader, "Qwen Sparse Attention":
// block-causal scores, top-K_B per query.)
//
// Persistent grid, one 512-thread workgroup per CU.  A workgroup owns a tile
// of 128 consecutive query rows (8 waves x 16 rows) and streams the pooled
// keys of every block any of its rows can see, 64 blocks per LDS stage,
// double-buffered.  Each wave holds its 16 rows' rotated queries as MFMA A
// fragments (4 row tiles of 4 queries x 4 heads) and computes 16x16 score
// tiles (4 queries x 16 blocks) with bf16 MFMA and fp32 accumulation; the
// ReLU-sum over heads is lane-local.
//
// Selection never stores the score matrix.  Each row keeps, in workspace, a
// list of candidate (score, block) keys in ascending block order and a
// threshold tau; a score enters the list iff it is >= tau.  When a list
// nears its capacity the owning wave cuts it to the exact top-k_B so far
// (radix select on the score bits; ties go to the smaller block id, which
// comes first in the list) and raises tau just above the k_B-th score.
// After the last stage the same cut, to min(k_B, visible), writes the
// ascending block ids straight into the output row.
#include "index_common.h"

namespace qsa {

namespace {

constexpr int kRows = 128;     // query rows per workgroup
constexpr int kWaves = 8;
constexpr int kStageBlk = 64;  // pooled blocks per LDS stage

template <typename T> struct PrefillLds {
  static constexpr int kRowElems = 128 + 16 / (int)sizeof(T);  // 16-byte pad per block row
  static constexpr int kStageBytes = kStageBlk * kRowElems * (int)sizeof(T);
  static constexpr int kScratchElems = 16 * 128;                // per wave: one row tile
};

}  // namespace

// Wave-wide cut of one candidate list (see wave_radix_kth / wave_keep_topk).
// mode 0: keep the top k in place and return the new threshold (just above
// the k-th score); mode 1: write the ascending ids of the top k to `out`.
__device__ __forceinline__ float cut_list(uint64_t* lb, int c, int k, uint32_t* hist, int lane,
                                       int mode, int32_t* out, int kB) {
  __threadfence();
  uint32_t v;
  int krem;
  wave_radix_kth(lb, c, k, hist, lane, &v, &krem);
  wave_keep_topk(lb, c, k, v, krem, lane, mode, out, kB);
  __threadfence();
  return __uint_as_float(v + 1u);
}

template <typename T, int NLO>
__global__ __launch_bounds__(512, 1) void index_prefill_kernel(IndexArgs a, uint64_t* cand_all,
                                                               int cap, int ntiles, int total,
                                                               int region_a_bytes) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  typedef Mma<T> M;
  typedef PrefillLds<T> LDS;
  const int tid = threadIdx.x;
  const int wv = tid >> 6, lane = tid & 63, hl = lane & 15, gq = lane >> 4;
  const int half = a.R / 2;
  // Region A: prologue (rope table + rotated-query scratch) then the stages.
  float2* table = (float2*)smem;                                         // [128][half]
  float* scratch = (float*)(smem + (size_t)kRows * (half > 0 ? half : 1) * sizeof(float2));
  T* stage0 = (T*)smem;
  T* stage1 = (T*)(smem + LDS::kStageBytes);
  uint32_t* hist = (uint32_t*)(smem + region_a_bytes) + wv * 256;
  // per-wave query state while a list is cut: [16] counts, [16] thresholds
  int* qcnt = (int*)(smem + region_a_bytes + kWaves * 256 * 4) + wv * 32;
  float* qtau = (float*)(qcnt + 16);
  uint64_t* cand_wg = cand_all + (size_t)blockIdx.x * kRows * cap;

  for (int L = blockIdx.x; L < total; L += gridDim.x) {
    const int tile = ntiles - 1 - L / a.B;  // longest rows first
    const int b = L % a.B;
    const int row0 = tile * kRows;
    const int64_t seq_off = a.seq_len ? (int64_t)a.seq_len[b] - a.n_q : a.q_pos0;
    const int last_row = min(row0 + kRows, a.n_q) - 1;
    const int64_t ncol = (seq_off + last_row + 1) / a.r;  // blocks any row of the tile sees

    // ---- prologue: rotated queries -> A fragments --------------------------
    for (int e = tid; e < kRows * half; e += 512) {
      const int p = e / half, j = e % half;
      float c = 1.f, s = 0.f;
      if (row0 + p < a.n_q) rope_cs(seq_off + row0 + p, j, a.R, a.log2_theta, &c, &s);
      table[e] = make_float2(c, s);
    }
    __syncthreads();
    typename M::Frag A[4][M::kCalls];
    typename M::Frag Alo[4][(M::kSplit && NLO > 0) ? NLO : 1];
    int nbq[4];
    {
      float* scr = scratch + wv * LDS::kScratchElems;
      const T* qsrc = (const T*)a.q_idx;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        // rows of this row tile: 4 queries (16 wv + 4 rt + x) x 4 heads, in float
        for (int e = lane; e < 16 * 128; e += 64) {
          const int rr = e >> 7, d = e & 127;
          const int ql = 16 * wv + 4 * rt + (rr >> 2), hh = rr & 3;
          const int t = row0 + ql;
          float val = 0.f;
          if (t < a.n_q) {
            const T* qr = qsrc + (((int64_t)b * a.n_q + t) * 4 + hh) * 128;
            const float x = Elt<T>::ld(qr, d);
            if (d < a.R) {
              const int j = d < half ? d : d - half;
              const float2 cs = table[ql * half + j];
              const float y = Elt<T>::ld(qr, d < half ? d + half : d - half);
              val = d < half ? (x * cs.x - y * cs.y) : (y * cs.y + x * cs.x);
            } else {
              val = x;
            }
          }
          scr[e] = val;
        }
        wave_sync();
        if constexpr (M::kSplit) {
          // bf16 fragment of row hl, call c: dims 32c + 8gq .. +7 (hi and lo)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const f32x4 v0 = *(const f32x4*)(scr + hl * 128 + 32 * c + 8 * gq);
            const f32x4 v1 = *(const f32x4*)(scr + hl * 128 + 32 * c + 8 * gq + 4);
            u16x8 hi, lo;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float v = j < 4 ? v0[j] : v1[j - 4];
              unsigned short h16, l16;
              split_bf16(v, &h16, &l16);
              hi[j] = h16;
              lo[j] = l16;
            }
            A[rt][c] = __builtin_bit_cast(typename M::Frag, hi);
            if constexpr (NLO > 0) {
              if (c < NLO) Alo[rt][c < NLO ? c : 0] = __builtin_bit_cast(typename M::Frag, lo);
            }
          }
        } else {
          M::load_lds((const T*)scr, 128, hl, gq, A[rt]);
        }
        wave_sync();
        const int t = row0 + 16 * wv + 4 * rt + gq;
        nbq[rt] = t < a.n_q ? (int)((seq_off + t + 1) / a.r) : 0;
      }
    }
    __syncthreads();  // region A is reused by the stages from here on

    float tau[4] = {0.f, 0.f, 0.f, 0.f};
    int cnt[4] = {0, 0, 0, 0};
    uint64_t* mybuf = cand_wg + (size_t)(16 * wv) * cap;

    // ---- stream pooled keys ------------------------------------------------
    const T* kb = (const T*)a.kbar + (size_t)b * a.nb_cap * 128;
    const int nst = (int)((ncol + kStageBlk - 1) / kStageBlk);
    constexpr int kVec = 128 * sizeof(T) / 16 / 8;  // 16-byte pieces per thread per block row
    u32x4 pre[kVec];
    auto fetch = [&](int s) {
      const int blk = s * kStageBlk + (tid >> 3);
      const int piece = (tid & 7) * kVec;
      if (blk < ncol) {
        const u32x4* src = (const u32x4*)(kb + (size_t)blk * 128) + piece;
#pragma unroll
        for (int v = 0; v < kVec; ++v) pre[v] = src[v];
      }
    };
    auto store = [&](T* st) {
      u32x4* dst = (u32x4*)(st + (tid >> 3) * LDS::kRowElems) + (tid & 7) * kVec;
#pragma unroll
      for (int v = 0; v < kVec; ++v) dst[v] = pre[v];
    };
    if (nst > 0) {
      fetch(0);
      store(stage0);
    }
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
      T* cur = (s & 1) ? stage1 : stage0;
      T* nxt = (s & 1) ? stage0 : stage1;
      if (s + 1 < nst) fetch(s + 1);
#pragma unroll 1
      for (int ct = 0; ct < kStageBlk / 16; ++ct) {
        const int col0 = s * kStageBlk + ct * 16;
        if (col0 >= ncol) break;
        typename M::Frag Bf[M::kCalls];
        M::load_lds(cur + ct * 16 * LDS::kRowElems, LDS::kRowElems, hl, gq, Bf);
        const int blk = col0 + hl;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const f32x4 acc = M::template dot<NLO>(A[rt], Alo[rt], Bf);
          const float sc = relu_sum4(acc);
          const bool pass = (blk < nbq[rt]) && (sc >= tau[rt]);
          const uint64_t bal = __ballot(pass);
          if (bal) {
            const uint32_t grp = (uint32_t)(bal >> (16 * gq)) & 0xffffu;
            if (pass) {
              const int slot = cnt[rt] + __popc(grp & ((1u << hl) - 1u));
              mybuf[(size_t)(4 * rt + gq) * cap + slot] =
                  ((uint64_t)__float_as_uint(sc) << 32) | (uint32_t)blk;
            }
            cnt[rt] += __popc(grp);
          }
        }
      }
      if (s + 1 < nst) store(nxt);
      // keep every list below capacity for the next stage (<= 64 appends)
      bool full = false;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) full |= cnt[rt] > cap - kStageBlk;
      if (__ballot(full)) {
        if (hl == 0) {
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            qcnt[4 * rt + gq] = cnt[rt];
            qtau[4 * rt + gq] = tau[rt];
          }
        }
        wave_sync();
        for (int q = 0; q < 16; ++q) {
          const int c = qcnt[q];
          if (c > cap - kStageBlk) {
            const float nt = cut_list(mybuf + (size_t)q * cap, c, a.kB, hist, lane, 0, nullptr, 0);
            wave_sync();
            if (lane == 0) {
              qcnt[q] = a.kB;
              qtau[q] = nt;
            }
            wave_sync();
          }
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          cnt[rt] = qcnt[4 * rt + gq];
          tau[rt] = qtau[4 * rt + gq];
        }
        wave_sync();
      }
      __syncthreads();
    }

    // ---- final selection: exact top-min(k_B, visible), ascending ids ------
    if (hl == 0) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        qcnt[4 * rt + gq] = cnt[rt];
        qcnt[16 + 4 * rt + gq] = nbq[rt];  // reuses the threshold slots
      }
    }
    wave_sync();
    for (int q = 0; q < 16; ++q) {
      const int t = row0 + 16 * wv + q;
      if (t >= a.n_q) break;
      const int c = qcnt[q];
      const int k = min(min(a.kB, qcnt[16 + q]), c);
      int32_t* out = a.idx + ((int64_t)b * a.n_q + t) * a.kB;
      if (k == 0) {
        for (int e = lane; e < a.kB; e += 64) out[e] = -1;
      } else {
        cut_list(mybuf + (size_t)q * cap, c, k, hist, lane, 1, out, a.kB);
      }
      if (lane == 0) a.cnt[(int64_t)b * a.n_q + t] = k;
    }
    __syncthreads();
  }
}

static int prefill_cap(int kB) {
  int cap = 2 * kB + 2 * kStageBlk;
  if (cap < 2048) cap = 2048;
  return (cap + 63) & ~63;
}

static int prefill_grid(int B, int n_q, int num_cu) {
  const int ntiles = (n_q + kRows - 1) / kRows;
  const long long total = (long long)ntiles * B;
  return (int)(total < num_cu ? total : num_cu);
}

size_t index_prefill_workspace(int B, int n_q, int num_cu, int kB) {
  return (size_t)prefill_grid(B, n_q, num_cu) * kRows * prefill_cap(kB) * sizeof(uint64_t);
}

template <typename T> static int region_a_bytes(int R) {
  typedef PrefillLds<T> LDS;
  const int half = R / 2 > 0 ? R / 2 : 1;
  const int pro = kRows * half * (int)sizeof(float2) + kWaves * LDS::kScratchElems * 4;
  const int stg = 2 * LDS::kStageBytes;
  const int r = pro > stg ? pro : stg;
  return (r + 15) & ~15;
}

template <typename T, int NLO>
static hipError_t launch_t(const IndexArgs& a, void* ws, int num_cu, hipStream_t st) {
  const int ntiles = (a.n_q + kRows - 1) / kRows;
  const int total = ntiles * a.B;
  const int grid = prefill_grid(a.B, a.n_q, num_cu);
  const int ra = region_a_bytes<T>(a.R);
  const int lds = ra + kWaves * 256 * 4 + kWaves * 32 * 4;
  hipError_t e = hipFuncSetAttribute((const void*)index_prefill_kernel<T, NLO>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((index_prefill_kernel<T, NLO>), dim3(grid), dim3(512), lds, st, a,
                     (uint64_t*)ws, prefill_cap(a.kB), ntiles, total, ra);
  return hipGetLastError();
}

hipError_t launch_index_prefill(qsa_dtype dt, const IndexArgs& a, void* ws, int num_cu,
                                hipStream_t st) {
  if (a.n_q == 0 || a.B == 0) return hipSuccess;
  if (dt != QSA_BF16) return launch_t<float, 0>(a, ws, num_cu, st);
  if (a.R == 0) return launch_t<unsigned short, 0>(a, ws, num_cu, st);
  if (a.R <= 64) return launch_t<unsigned short, 2>(a, ws, num_cu, st);
  return launch_t<unsigned short, 4>(a, ws, num_cu, st);
}

}  // namespace qsa
