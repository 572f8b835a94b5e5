// Compressed MQA indexer + streaming top-k_B for many query rows, in one
// self-contained kernel (research-hub note, "Key ideas", QSA bullet: I_ib =
// sum_h ReLU(<q_i^h, kbar_b>), top-k_B = ceil(K/r); paperglide reader, "Qwen
// Sparse Attention": block-causal scores, top-K_B per query).
//
// It is exact for any input: the prefill pipeline (index_prefill.hip) runs it
// on the query tiles whose sampled threshold failed, and it serves the
// configurations that pipeline does not cover (fp32 inputs, more than 64
// rotated dims).
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
// threshold tau; a score enters the list iff it is >= tau.
//   1. Threshold estimate (rows that see more blocks than the list holds):
//      score a strided sample of m blocks, take the j-th largest sample
//      score, j = ceil(E + 5 sqrt(E) + 2) with E = m k_B / visible, i.e. five
//      standard deviations above the expected number of the row's top-k_B
//      blocks in the sample.  Then tau = that score: about j/m of the
//      blocks pass instead of all of them.
//   2. Stream every visible block against tau.  If a list nears capacity
//      anyway, the owning wave cuts it to the exact top-k_B so far (radix
//      select; ties go to the smaller block id, which comes first) and
//      raises tau just above the k_B-th score.
//   3. A row whose list ends with fewer than min(k_B, visible) entries had
//      tau too high: it is streamed again with tau = 0 (exact streaming).
//   4. The same cut, to min(k_B, visible), writes the ascending block ids.
#include <type_traits>

#include "index_common.h"

namespace qsa {

namespace {

constexpr int kRows = 128;            // query rows per workgroup
constexpr int kWaves = 8;             // two waves per SIMD
constexpr int kRPW = kRows / kWaves;  // rows per wave: two 32x32 row tiles (8 queries x 4 heads)
constexpr int kStageBytes = 32768;    // one LDS stage of pooled keys
constexpr int kCap = 4096;            // candidate list capacity per row (entries)
constexpr int kSampleMin = 1024, kSampleMax = 2048;

template <typename T> struct PrefillLds {
  static constexpr int kRowBytes = 128 * (int)sizeof(T);  // one pooled key
  static constexpr int kBlk = kStageBytes / kRowBytes;    // pooled keys per stage
  static constexpr int kScratchElems = 8 * 128;           // per wave: 8 query-head rows at a time
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

}  // namespace

// Wave-wide cut of one candidate list (see wave_radix_kth / wave_keep_topk).
// mode 0: keep the top k in place; mode 1: write the ascending ids of the top
// k to `out` (padding to kB with -1); mode 2: only find the k-th score.
// When lsc (lcap words of wave-private LDS) is given and the list fits, the
// scores are staged there once and the radix passes read LDS.
// Returns the k-th largest score.
__device__ __forceinline__ float cut_list(uint64_t* lb, int c, int k, uint32_t* hist,
                                       uint32_t* lsc, int lcap, int lane, int mode,
                                       int32_t* out, int kB) {
  // The list was written by this wave: completing its stores suffices (a
  // device-scope fence would write back the L2 of the whole XCD).
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  if (mode == 1 && c == k) {  // everything is kept: copy in order
    for (int e = lane; e < kB; e += 64) out[e] = e < c ? (int32_t)(uint32_t)lb[e] : -1;
    return 0.f;
  }
  uint32_t v;
  int krem;
  if (lsc != nullptr && c <= lcap) {
    stage_scores(lb, c, lsc, lane);
    wave_radix_kth([&](int e) { return lsc[e]; }, c, k, hist, lane, &v, &krem);
  } else {
    wave_radix_kth([&](int e) { return (uint32_t)(lb[e] >> 32); }, c, k, hist, lane, &v, &krem);
  }
  if (mode != 2) wave_keep_topk(lb, c, k, v, krem, lane, mode, out, kB);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  return __uint_as_float(v);
}

// Tiles L in [g0, g0 + count) (L indexes 128-row tiles longest first); when
// `only` is given, only the tiles with only[L - g0] != 0 are processed.
template <typename T, int NLO>
__global__ __launch_bounds__(512, 1) void index_exact_kernel(IndexArgs a, uint64_t* cand_all,
                                                              int ntiles, int g0, int count,
                                                              const uint32_t* only,
                                                              int region_a_bytes) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  typedef Mma32<T> M;
  typedef PrefillLds<T> LDS;
  constexpr int kStageBlk = LDS::kBlk;
  constexpr int kThreads = kWaves * 64;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, col = lane & 31, g = lane >> 5;
  const uint32_t lt32 = (1u << col) - 1u;
  const int half = a.R / 2;
  // Region A: prologue (rope table + rotated-query scratch) then the stages
  // and the staged scores of list cuts.
  float2* table = (float2*)smem;  // [128][half]
  float* scratch = (float*)(smem + (size_t)kRows * (half > 0 ? half : 1) * sizeof(float2));
  T* stage0 = (T*)smem;
  T* stage1 = (T*)(smem + kStageBytes);
  uint32_t* hist = (uint32_t*)(smem + region_a_bytes) + wv * 256;
  // per-wave row state while lists are cut: [8] counts, [8] thresholds
  int* qcnt = (int*)(smem + region_a_bytes + kWaves * 256 * 4) + wv * 2 * kRPW;
  float* qtau = (float*)(qcnt + kRPW);
  int* wg_flag = (int*)(smem + region_a_bytes + kWaves * 256 * 4 + kWaves * 2 * kRPW * 4);
  uint64_t* mybuf = cand_all + ((size_t)blockIdx.x * kRows + kRPW * wv) * kCap;
  uint32_t* lsc = (uint32_t*)smem + wv * (region_a_bytes / 4 / kWaves);
  const int lcap = region_a_bytes / 4 / kWaves;
  constexpr int NL = (M::kSplit && NLO > 0) ? NLO : 1;  // lo steps kept in LDS
  // lo operands of the wave's row tiles: [rt][step][lane]
  u16x8* alo = (u16x8*)(smem + region_a_bytes + kWaves * 256 * 4 + kWaves * 2 * kRPW * 4 + 16) +
               wv * 2 * NL * 64;

  for (int Lg = blockIdx.x; Lg < count; Lg += gridDim.x) {
    if (only != nullptr && only[Lg] == 0) continue;
    const int L = g0 + Lg;
    const int tile = ntiles - 1 - L / a.B;  // longest rows first
    const int b = L % a.B;
    const int row0 = tile * kRows;
    const int64_t seq_off = a.seq_len ? (int64_t)a.seq_len[b] - a.n_q : a.q_pos0;
    const int last_row = min(row0 + kRows, a.n_q) - 1;
    const int ncol = (int)((seq_off + last_row + 1) / a.r);  // blocks any row of the tile sees
    const int nbmin = (int)((seq_off + row0 + 1) / a.r);     // blocks every row sees

    // ---- prologue: rotated queries -> A operands --------------------------
    for (int e = tid; e < kRows * half; e += kThreads) {
      const int p = e / half, j = e % half;
      float c = 1.f, s = 0.f;
      if (row0 + p < a.n_q) rope_cs(seq_off + row0 + p, j, a.R, a.log2_theta, &c, &s);
      table[e] = make_float2(c, s);
    }
    __syncthreads();
    // the wave's two row tiles (wave rows 0-7 and 8-15): rows 4q + h for
    // their queries q < 8; lane row `col`.  The lo operands of the rotated
    // steps live in LDS (alo), the hi operands in registers.
    typename M::Tile A0, A1;
    {
      float* scr = scratch + wv * LDS::kScratchElems;
      const T* qsrc = (const T*)a.q_idx;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int hf = 0; hf < 4; ++hf) {
          // tile rows 8 hf .. 8 hf + 7 (queries 2 hf, 2 hf + 1), in float
          for (int e = lane; e < 8 * 128; e += 64) {
            const int rr = e >> 7, d = e & 127;
            const int m = 8 * hf + rr;
            const int ql = kRPW * wv + 8 * rt + (m >> 2), hh = m & 3;
            const int t = row0 + ql;
            float val = 0.f;
            if (t < a.n_q && hh < a.h) {
              const T* qr = qsrc + (((int64_t)b * a.n_q + t) * a.h + hh) * 128;
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
          // every lane converts the row it would own in this pass; only the
          // lanes whose row it is keep it
          const bool mine = (col >> 3) == hf;
          const typename M::Tile th = M::template a_from_f32<NLO>(
              scr + (col & 7) * 128, g, alo + rt * NL * 64 + lane, mine);
          if (rt == 0)
            A0 = mine ? th : A0;
          else
            A1 = mine ? th : A1;
          wave_sync();
        }
      }
    }
    __syncthreads();  // region A is reused by the stages from here on

    // lane state: the 8 rows it scores, wave row 8 rt + 2 j + g = row index
    // x = 4 rt + j below
    float tau[8];
    int cnt[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      tau[x] = 0.f;
      cnt[x] = 0;
    }
    auto wrow = [&](int x) { return 8 * (x >> 2) + 2 * (x & 3) + g; };
    // visible blocks of wave row w: (nb_base + w) / r, rows beyond n_q see none
    const int nb_base = (int)(seq_off + row0 + kRPW * wv + 1);
    const int wave_rows = min(kRPW, a.n_q - (row0 + kRPW * wv));
    auto nb_of = [&](int w) -> int { return w < wave_rows ? (nb_base + w) / a.r : 0; };
    const int nb_wave_min = wave_rows > 0 ? nb_of(0) : 0;  // every row of the wave sees these
    const T* kb = (const T*)a.kbar + (size_t)b * a.nb_cap * 128;

    auto save_state = [&](bool with_tau) {
      if (col == 0) {
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          qcnt[wrow(x)] = cnt[x];
          if (with_tau) qtau[wrow(x)] = tau[x];
        }
      }
      wave_sync();
    };
    auto load_state = [&]() {
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        cnt[x] = qcnt[wrow(x)];
        tau[x] = qtau[wrow(x)];
      }
      wave_sync();
    };

    // Stream the blocks of a column list through LDS and append every score
    // >= tau of a visible block.  Column u < len holds block u, or, for the
    // sample, block u * nbmin / len.
    auto scan = [&](int len, auto sample_tag) {
      constexpr bool kSample = decltype(sample_tag)::value;
      auto block_of = [&](int u) -> int {
        if constexpr (kSample) return (int)(((int64_t)u * nbmin) / len);
        return u;
      };
      const int nst = (len + kStageBlk - 1) / kStageBlk;
      // Stage s into LDS with direct loads: instruction i of wave wv fills the
      // 1 KB at (kIss wv + i) KB; lane l's 16 bytes land at l * 16 within it,
      // so the lane loads the global chunk that belongs there after the swizzle
      // (chunk c of block row r is stored at chunk c ^ (r & 15)).
      constexpr int kIss = kStageBytes / (kWaves * 64 * 16);
      auto issue = [&](int s, T* st) {
        // lane index re-read here: the addresses are recomputed on the spot
        // instead of being kept (or spilled) across the loop
        int ln = __lane_id();
        asm volatile("" : "+v"(ln));
        const T* kbs = kb;
        asm volatile("" : "+s"(kbs));
#pragma unroll
        for (int i = 0; i < kIss; ++i) {
          const int o = ((wv * kIss + i) * 64 + ln) * 16;  // byte offset in the stage
          const int r = o / LDS::kRowBytes;
          const int pch = (o % LDS::kRowBytes) >> 4;
          const int lch = pch ^ (r & 15);
          const int u = s * kStageBlk + r;
          const int blk = u < len ? block_of(u) : 0;
          const unsigned char* src = (const unsigned char*)(kbs + (size_t)blk * 128) + lch * 16;
          __builtin_amdgcn_global_load_lds(
              (glb_void_t*)src, (lds_void_t*)((unsigned char*)st + (wv * kIss + i) * 1024), 16,
              0, 0);
        }
      };
      if (nst > 0) issue(0, stage0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      for (int s = 0; s < nst; ++s) {
        T* cur = (s & 1) ? stage1 : stage0;
        T* nxt = (s & 1) ? stage0 : stage1;
        if (s + 1 < nst) issue(s + 1, nxt);
#pragma unroll 1
        for (int ct = 0; ct < kStageBlk / 32; ++ct) {
          const int u0 = s * kStageBlk + ct * 32;
          if (u0 >= len) break;
          const typename M::Tile Bt = M::load_b(cur, ct * 32 + col, g);
          f32x16 acc0, acc1;
          M::template mma2<NLO>(A0, A1, alo, lane, Bt, acc0, acc1);
          const int u = u0 + col;
          const int blk = u < len ? block_of(u) : 0x7fffffff;
          float sc[8];
          bool pass[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const f32x16& acc = x < 4 ? acc0 : acc1;
            const int j = x & 3;
            sc[x] = relu(acc[4 * j]) + relu(acc[4 * j + 1]) + relu(acc[4 * j + 2]) +
                    relu(acc[4 * j + 3]);
            pass[x] = sc[x] >= tau[x];
          }
          if (u0 + 32 > nb_wave_min || u0 + 32 > len) {  // causal edge of the tile (uniform)
#pragma unroll
            for (int x = 0; x < 8; ++x) pass[x] = pass[x] && (blk < nb_of(wrow(x)));
          }
          bool any = false;
#pragma unroll
          for (int x = 0; x < 8; ++x) any |= pass[x];
          if (__ballot(any)) {
#pragma unroll
            for (int x = 0; x < 8; ++x) {
              const uint64_t bal = __ballot(pass[x]);
              if (bal) {
                const uint32_t grp = (uint32_t)(bal >> (32 * g));
                if (pass[x]) {
                  const int slot = cnt[x] + __popc(grp & lt32);
                  mybuf[(size_t)wrow(x) * kCap + slot] =
                      ((uint64_t)__float_as_uint(sc[x]) << 32) | (uint32_t)blk;
                }
                cnt[x] += __popc(grp);
              }
            }
          }
        }
        // keep every list below capacity for the next stage (<= kStageBlk appends)
        bool full = false;
#pragma unroll
        for (int x = 0; x < 8; ++x) full |= cnt[x] > kCap - kStageBlk;
        if (__ballot(full)) {
          save_state(true);
          for (int q = 0; q < kRPW; ++q) {
            const int c = qcnt[q];
            if (c > kCap - kStageBlk) {
              const float v = cut_list(mybuf + (size_t)q * kCap, c, a.kB, hist, nullptr, 0, lane,
                                       0, nullptr, 0);
              wave_sync();
              if (lane == 0) {
                qcnt[q] = a.kB;
                qtau[q] = __uint_as_float(__float_as_uint(v) + 1u);  // just above the k_B-th
              }
              wave_sync();
            }
          }
          load_state();
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // stage s+1 has landed
        __syncthreads();
      }
    };

    // ---- 1. threshold estimate from a strided sample -----------------------
    if (ncol > kCap - kStageBlk) {
      int m = nbmin / 16;
      m = m < kSampleMin ? kSampleMin : (m > kSampleMax ? kSampleMax : m);
      if (m > nbmin) m = nbmin;
      scan(m, std::true_type{});
      save_state(false);
      for (int q = 0; q < kRPW; ++q) {
        const int c = qcnt[q];
        const int t = row0 + kRPW * wv + q;
        const float nvis = t < a.n_q ? (float)((seq_off + t + 1) / a.r) : 0.f;
        float thr = 0.f;
        if (c > 0 && nvis > 0.f) {
          const float E = (float)m * (float)a.kB / nvis;
          int j = (int)ceilf(E + 5.f * sqrtf(E) + 2.f);
          if (j > c) j = c;
          thr = cut_list(mybuf + (size_t)q * kCap, c, j, hist, lsc, lcap, lane, 2, nullptr, 0);
        }
        wave_sync();
        if (lane == 0) {
          qtau[q] = thr;
          qcnt[q] = 0;
        }
        wave_sync();
      }
      load_state();
    }

    // ---- 2. stream every visible block against tau ------------------------
    __syncthreads();  // the staged scores of the sample cuts share region A
    scan(ncol, std::false_type{});

    // ---- 3. rows whose threshold was too high: stream again, exact --------
    if (tid == 0) *wg_flag = 0;
    __syncthreads();
    bool failed_any = false;
    int keep[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const bool f = cnt[x] < min(a.kB, nb_of(wrow(x)));
      failed_any |= f;
      keep[x] = cnt[x];
      tau[x] = f ? 0.f : INFINITY;  // rows that succeeded append nothing more
      if (f) cnt[x] = 0;
    }
    if (__ballot(failed_any) && lane == 0) atomicOr(wg_flag, 1);
    __syncthreads();
    if (*wg_flag) {
      scan(ncol, std::false_type{});
#pragma unroll
      for (int x = 0; x < 8; ++x) cnt[x] = (tau[x] == INFINITY) ? keep[x] : cnt[x];
    }

    // ---- 4. final selection: exact top-min(k_B, visible), ascending ids ---
    save_state(false);
    for (int q = 0; q < kRPW; ++q) {
      const int t = row0 + kRPW * wv + q;
      if (t >= a.n_q) break;
      const int c = qcnt[q];
      const int nb = (int)((seq_off + t + 1) / a.r);
      const int k = min(min(a.kB, nb), c);
      int32_t* out = a.idx + ((int64_t)b * a.n_q + t) * a.kB;
      if (k == 0) {
        for (int e = lane; e < a.kB; e += 64) out[e] = -1;
      } else {
        cut_list(mybuf + (size_t)q * kCap, c, k, hist, lsc, lcap, lane, 1, out, a.kB);
      }
      if (lane == 0) a.cnt[(int64_t)b * a.n_q + t] = k;
    }
    __syncthreads();
  }
}

static int exact_grid(int count, int num_cu) { return count < num_cu ? count : num_cu; }

size_t index_exact_workspace(int B, int n_q, int num_cu) {
  const int ntiles = (n_q + kRows - 1) / kRows;
  return (size_t)exact_grid(ntiles * B, num_cu) * kRows * kCap * sizeof(uint64_t);
}

template <typename T> static int region_a_bytes(int R) {
  typedef PrefillLds<T> LDS;
  const int half = R / 2 > 0 ? R / 2 : 1;
  const int pro = kRows * half * (int)sizeof(float2) + kWaves * LDS::kScratchElems * 4;
  const int stg = 2 * kStageBytes;
  const int r = pro > stg ? pro : stg;
  return (r + 15) & ~15;
}

template <typename T, int NLO>
static hipError_t launch_t(const IndexArgs& a, void* ws, int num_cu, int g0, int count,
                           const uint32_t* only, hipStream_t st) {
  const int ntiles = (a.n_q + kRows - 1) / kRows;
  const int grid = exact_grid(count, num_cu);
  const int ra = region_a_bytes<T>(a.R);
  const int nl = (sizeof(T) == 2 && NLO > 0) ? NLO : 1;
  const int lds = ra + kWaves * 256 * 4 + kWaves * 2 * kRPW * 4 + 16 + kWaves * 2 * nl * 64 * 16;
  hipError_t e = hipFuncSetAttribute((const void*)index_exact_kernel<T, NLO>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((index_exact_kernel<T, NLO>), dim3(grid), dim3(kWaves * 64), lds, st, a,
                     (uint64_t*)ws, ntiles, g0, count, only, ra);
  return hipGetLastError();
}

hipError_t launch_index_exact(qsa_dtype dt, const IndexArgs& a, void* ws, int num_cu, int g0,
                              int count, const uint32_t* only, hipStream_t st) {
  if (a.n_q == 0 || a.B == 0 || count <= 0) return hipSuccess;
  // NLO: 16-dim k-steps holding rotated dims, ceil(R / 16)
  if (dt != QSA_BF16) return launch_t<float, 0>(a, ws, num_cu, g0, count, only, st);
  if (a.R == 0) return launch_t<unsigned short, 0>(a, ws, num_cu, g0, count, only, st);
  if (a.R <= 32) return launch_t<unsigned short, 2>(a, ws, num_cu, g0, count, only, st);
  if (a.R <= 64) return launch_t<unsigned short, 4>(a, ws, num_cu, g0, count, only, st);
  return launch_t<unsigned short, 8>(a, ws, num_cu, g0, count, only, st);
}

}  // namespace qsa
