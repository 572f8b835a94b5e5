// Compressed MQA indexer + top-k_B for many query rows (prefill), as a
// pipeline of lean kernels (research-hub note, "Key ideas", QSA bullet:
// I_ib = sum_h ReLU(<q_i^h, kbar_b>), top-k_B = ceil(K/r); paperglide reader,
// "Qwen Sparse Attention": block-causal scores, top-K_B per query).
//
// Query rows go in tiles of 128: 16 waves of 8 rows, the rows of a wave being
// one 32-row MFMA tile (8 queries x 4 heads) whose bf16 hi and lo parts stay
// in registers.  Tiles run longest first, in groups whose candidate lists fit
// the workspace.  Per group:
//   1. scan (sample): tiles whose rows see more blocks than a list holds
//      score a strided sample of m blocks, m = 16 visible / k_B (so that
//      E = m k_B / visible, the expected number of the row's top-k_B blocks
//      in the sample, is about 16).  Each lane keeps its four largest sample
//      scores per row; tau = the j-th largest of those 128 values,
//      j = ceil(E + 5 sqrt(E) + 2): five standard deviations above E, and
//      never above the j-th largest sample score.  Rows that are not
//      sampled get tau = 0.
//   2. scan (main): stream every visible block and append each score >= tau
//      to the row's list, in block order (counting past the list capacity).
//   3. cut (final): a row whose list holds at least min(k_B, visible) entries
//      and did not overflow holds its exact top-k_B (the k-th score is then
//      >= tau, so every block scoring at least as much was appended); the
//      order-preserving radix cut writes the ascending ids.  Any other row
//      flags its tile.
//   4. exact: the flagged tiles are recomputed by the self-contained exact
//      kernel (index_exact.hip).
// Appends are staged in LDS and written out before the next stage's loads
// are issued, so the wait for a stage never waits on fresh stores.
#include "index_common.h"

namespace qsa {

namespace {

constexpr int kTileRows = 128;
constexpr int kScanWaves = 16;             // 8 rows (one 32-row MFMA tile) per wave
constexpr int kStageBytes = 32768;         // one LDS stage: 128 pooled keys (bf16)
constexpr int kStageBlk = 128;
constexpr int kList = 3072;                // candidate list capacity per row
constexpr int kBuf = 384;                  // LDS append buffer per wave (16-byte entries)
constexpr int kGroupTiles = 2048;
constexpr float kSampleE = 16.f;           // expected top-k_B blocks in a sample
constexpr int kKeep = 4;                   // sample scores kept per lane and row
constexpr int kCutWaves = 4;
constexpr int kScanLds = 2 * kStageBytes + kScanWaves * kBuf * 16;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

struct PipeWs {
  uint64_t* list;  // [gt * 128][kList] (score bits << 32 | block id)
  uint32_t* cnt;   // [gt * 128] entries appended (may exceed kList)
  float* tau;      // [gt * 128]
  uint32_t* fail;  // [gt] tile needs the exact kernel
  int gt;
};

struct TileGeo {
  int b, row0;
  int64_t seq_off;
  int ncol;   // blocks the last row of the tile sees
  int nbmin;  // blocks every row of the tile sees
};

__device__ __forceinline__ TileGeo tile_geo(const IndexArgs& a, int L, int ntiles) {
  TileGeo G;
  const int tile = ntiles - 1 - L / a.B;  // longest rows first
  G.b = L % a.B;
  G.row0 = tile * kTileRows;
  G.seq_off = a.seq_len ? (int64_t)a.seq_len[G.b] - a.n_q : a.q_pos0;
  const int last_row = min(G.row0 + kTileRows, a.n_q) - 1;
  G.ncol = (int)((G.seq_off + last_row + 1) / a.r);
  G.nbmin = (int)((G.seq_off + G.row0 + 1) / a.r);
  return G;
}

// The lane id recomputed where it is used (v_mbcnt in a volatile asm block,
// which the compiler cannot merge with an earlier value): the sample pass
// then keeps no lane-derived value live across its register-heavy query
// prologue, whose spill would be reloaded, with a wait on every load in
// flight, inside the block loop.
__device__ __forceinline__ int fresh_lane_id() {
  int ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  return ln;
}

__device__ __forceinline__ int sample_size(int nbmin, int kB) {
  int m = (int)ceilf(kSampleE * (float)nbmin / (float)kB);
  m = m < 64 ? 64 : m;
  return m > nbmin ? nbmin : m;
}

}  // namespace

template <int NLO, bool SAMPLE>
__global__ __launch_bounds__(1024, 1) void index_scan_kernel(IndexArgs a, PipeWs w, int g0,
                                                              int ntiles) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  typedef Mma32<unsigned short> M;
  const int tid = threadIdx.x;
  // the wave index as a scalar, so that what derives from it (row counts,
  // the causal edge, the stage's LDS destination) stays wave-uniform
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 31, g = lane >> 5;
  const int Lg = blockIdx.x;
  const TileGeo G = tile_geo(a, g0 + Lg, ntiles);
  if (SAMPLE) {
    if (tid == 0) w.fail[Lg] = 0;
    if (G.ncol <= kList) {  // every visible block fits the lists: no threshold
      if (tid < kTileRows) w.tau[Lg * kTileRows + tid] = 0.f;
      return;
    }
  }
  const int len = SAMPLE ? sample_size(G.nbmin, a.kB) : G.ncol;
  auto block_of = [&](int u) -> int {
    if constexpr (SAMPLE) return (int)(((int64_t)u * G.nbmin) / len);
    return u;
  };
  unsigned short* stage0 = (unsigned short*)smem;
  unsigned short* stage1 = (unsigned short*)(smem + kStageBytes);
  // staged appends: (list entry, block id, score bits, unused)
  u32x4* bent = (u32x4*)(smem + 2 * kStageBytes) + wv * kBuf;

  // ---- prologue: rotated queries -> the wave's A tile (hi and lo) --------
  const int half = a.R / 2;
  {
    float2* table = (float2*)(smem + 2 * kStageBytes);  // [128][half]
    for (int e = tid; e < kTileRows * half; e += kScanWaves * 64) {
      const int p = e / half, j = e % half;
      float c = 1.f, s = 0.f;
      if (G.row0 + p < a.n_q) rope_cs(G.seq_off + G.row0 + p, j, a.R, a.log2_theta, &c, &s);
      table[e] = make_float2(c, s);
    }
    __syncthreads();
  }
  M::Tile A;
  M::LoTile Alo;
#pragma unroll
  for (int e = 0; e < 32; ++e) A[e] = 0u;
#pragma unroll
  for (int e = 0; e < 16; ++e) Alo[e] = 0u;
  {
    const float2* table = (const float2*)(smem + 2 * kStageBytes);
    float* scr = (float*)smem + wv * 8 * 128;  // 8 A rows in float
    // the wave's queries (8 x 4 heads x 128 bf16) are one contiguous 8 KB
    // run; four queries at a time go to LDS (load j of a lane brings 16
    // bytes of query j, all four in flight together; absent queries read as
    // zeros) for the rotation, which pairs dims across lanes
    // (with h < 4 indexer heads a query is h * 16 uint4; slots h .. 3 are zero)
    const uint4* qw = (const uint4*)a.q_idx + ((int64_t)G.b * a.n_q + G.row0 + 8 * wv) * (16 * a.h);
    uint4* rawq = (uint4*)(smem + 2 * kStageBytes + 32768) + wv * 256;
#pragma unroll 1
    for (int hf = 0; hf < 4; ++hf) {
      if ((hf & 1) == 0) {
        uint4 rq[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int ql = 2 * hf + j;
          rq[j] = (G.row0 + 8 * wv + ql < a.n_q && (lane >> 4) < a.h)
                      ? qw[ql * (16 * a.h) + lane]
                      : uint4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) rawq[j * 64 + lane] = rq[j];
        wave_sync();
      }
      const unsigned short* raw16 = (const unsigned short*)(rawq + (hf & 1) * 128);
      // A rows 8 hf .. 8 hf + 7 = queries 2 hf, 2 hf + 1 (rows 4q + h)
      for (int e = lane; e < 8 * 128; e += 64) {
        const int rr = e >> 7, d = e & 127;
        const int ql = 8 * wv + ((8 * hf + rr) >> 2);
        const unsigned short* qr = raw16 + rr * 128;  // query 2 hf + rr / 4, head rr % 4
        const float x = bf16_to_f32(qr[d]);
        float val = x;
        if (d < a.R) {
          const int j = d < half ? d : d - half;
          const float2 cs = table[ql * half + j];
          const float y = bf16_to_f32(qr[d < half ? d + half : d - half]);
          val = d < half ? (x * cs.x - y * cs.y) : (y * cs.y + x * cs.x);
        }
        scr[e] = val;
      }
      wave_sync();
      // every lane converts the row it would own in this pass; only the
      // lanes whose row it is keep it
      M::Tile th;
      M::LoTile tl;
      M::template a_from_f32_reg<NLO>(scr + (col & 7) * 128, g, th, tl);
      const bool mine = (col >> 3) == hf;
      A = mine ? th : A;
      Alo = mine ? tl : Alo;
      wave_sync();
    }
  }
  __syncthreads();  // the prologue's LDS is reused from here on

  // ---- per-lane row state: rows q = 2j + g of the wave -------------------
  const int rbase = G.row0 + 8 * wv;
  const int wave_rows = min(8, a.n_q - rbase);
  float tau[4];
  float tk[4][kKeep];  // tk[j][0] >= tk[j][1] >= ...: the lane's largest sample scores
  // entries appended to rows 2j (cnt_lo) and 2j + 1 (cnt_hi): wave-uniform
  int cnt_lo[4], cnt_hi[4];
  // list of row q = 2j + g starts at lbase0 + 2j kList; row q sees (nb0 + q) / r
  const uint32_t lbase0 = (uint32_t)(Lg * kTileRows + 8 * wv + g) * (uint32_t)kList;
  const int nb0 = (int)(G.seq_off + rbase + 1);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = 2 * j + g;
    tau[j] = SAMPLE ? 0.f : (q < wave_rows ? w.tau[Lg * kTileRows + 8 * wv + q] : 0.f);
#pragma unroll
    for (int m = 0; m < kKeep; ++m) tk[j][m] = 0.f;
    cnt_lo[j] = cnt_hi[j] = 0;
  }
  // every row of the wave sees blocks below nb_all (0 if some row is absent)
  const int nb_all = wave_rows == 8 ? nb0 / a.r : 0;
  const unsigned short* kb = (const unsigned short*)a.kbar + (size_t)G.b * a.nb_cap * 128;

  int nbuf = 0;
  auto flush = [&]() {
    wave_sync();
    for (int e = lane; e < nbuf; e += 64) {
      const u32x4 x = bent[e];
      w.list[x.x] = ((uint64_t)x.z << 32) | x.y;
    }
    nbuf = 0;
    wave_sync();
  };
  // Stage s into LDS with direct loads: instruction i of wave wv fills the
  // 1 KB at (2 wv + i) KB; lane l's 16 bytes land at l * 16 within it, so the
  // lane loads the chunk that belongs there after the swizzle (chunk c of
  // block row r is stored at chunk c ^ (r & 15)).
  auto issue = [&](int s, unsigned short* st) {
    int ln = __lane_id();
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int o = ((wv * 2 + i) * 64 + ln) * 16;  // byte offset in the stage
      const int r = o >> 8;
      const int lch = ((o & 255) >> 4) ^ (r & 15);
      const int u = s * kStageBlk + r;
      const int blk = u < len ? block_of(u) : 0;
      const unsigned short* src = kb + (size_t)blk * 128 + lch * 8;
      __builtin_amdgcn_global_load_lds((glb_void_t*)src,
                                       (lds_void_t*)(st + (wv * 2 + i) * 512), 16, 0, 0);
    }
  };

  const int nst = (len + kStageBlk - 1) / kStageBlk;
  if (nst > 0) issue(0, stage0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    const unsigned short* cur = (s & 1) ? stage1 : stage0;
    unsigned short* nxt = (s & 1) ? stage0 : stage1;
    if (nbuf > 0) flush();  // stores go out before the next stage's loads
    if (s + 1 < nst) issue(s + 1, nxt);
    if (wave_rows > 0) {
#pragma unroll 1
      for (int ct = 0; ct < kStageBlk / 32; ++ct) {
        const int u0 = s * kStageBlk + ct * 32;
        if (u0 >= len) break;
        if (nbuf > kBuf - 256) flush();  // a column tile appends at most 8 x 32
        const f32x16 acc = M::template mma1_lds<NLO>(A, Alo, cur, ct * 32 + col, g);
        const int u = u0 + col;
        const int blk = u < len ? block_of(u) : 0x7fffffff;
        float sc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sc[j] = relu(acc[4 * j]) + relu(acc[4 * j + 1]) + relu(acc[4 * j + 2]) +
                  relu(acc[4 * j + 3]);
        if constexpr (SAMPLE) {
          const bool in = u0 + (fresh_lane_id() & 31) < len;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float x = in ? sc[j] : 0.f;  // insertion into the sorted kKeep
#pragma unroll
            for (int m = 0; m < kKeep; ++m) {
              const float hi = fmaxf(x, tk[j][m]);
              x = fminf(x, tk[j][m]);
              tk[j][m] = hi;
            }
          }
          continue;
        }
        // bal[j]: the lanes whose score for row 2j + g passes (low half: row
        // 2j, high half: row 2j + 1)
        uint64_t bal[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bal[j] = __ballot(sc[j] >= tau[j]);
        if (u0 + 32 > nb_all || u0 + 32 > len) {  // causal edge of the wave (uniform)
#pragma unroll
          for (int j = 0; j < 4; ++j) bal[j] &= __ballot(blk < (nb0 + 2 * j + g) / a.r);
        }
        if (bal[0] | bal[1] | bal[2] | bal[3]) {
          // a passing lane's rank in the wave (mbcnt) gives its buffer
          // position; minus the passing lanes of the low half when it is in
          // the high half, its place in its row's list.  Past a full list the
          // entry goes to the list's last place: the row's count then exceeds
          // kList and the row fails, whatever the list holds.
          int pos = nbuf;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (bal[j] == 0) continue;
            const uint32_t lo = (uint32_t)bal[j], hi = (uint32_t)(bal[j] >> 32);
            const int n_lo = __popc(lo), n_hi = __popc(hi);
            if (__builtin_amdgcn_inverse_ballot_w64(bal[j])) {
              const uint32_t rank =
                  __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
              const uint32_t slot = (uint32_t)(g ? cnt_hi[j] - n_lo : cnt_lo[j]) + rank;
              bent[pos + rank] =
                  u32x4{lbase0 + (uint32_t)(2 * j * kList) + min(slot, (uint32_t)kList - 1u),
                        (uint32_t)blk, __float_as_uint(sc[j]), 0u};
            }
            cnt_lo[j] += n_lo;
            cnt_hi[j] += n_hi;
            pos += n_lo + n_hi;
          }
          nbuf = pos;
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // stage s + 1 has landed
    __syncthreads();
  }
  if constexpr (SAMPLE) {
    // tau of each row from the 32 kKeep kept sample scores of its lanes
    constexpr int kKept = 32 * kKeep;
    float* tv = (float*)(smem + 2 * kStageBytes) + wv * (8 * kKept + 256);  // [8][kKept], hist
    uint32_t* hist = (uint32_t*)(tv + 8 * kKept);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int m = 0; m < kKeep; ++m) tv[(2 * j + g) * kKept + kKeep * col + m] = tk[j][m];
    wave_sync();
    for (int q = 0; q < wave_rows; ++q) {
      const float nvis = (float)((nb0 + q) / a.r);
      const float E = (float)len * (float)a.kB / nvis;
      const int jj = (int)ceilf(E + 5.f * sqrtf(E) + 2.f);
      float thr = 0.f;
      if (jj <= kKept) {
        uint32_t v;
        int krem;
        const uint32_t* tb = (const uint32_t*)(tv + q * kKept);
        wave_radix_kth([&](int e) { return tb[e]; }, kKept, jj, hist, lane, &v, &krem);
        thr = __uint_as_float(v);
      }
      if (lane == 0) w.tau[Lg * kTileRows + 8 * wv + q] = thr;
      wave_sync();
    }
    return;
  }
  if (nbuf > 0) flush();
  if (col == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (2 * j + g < wave_rows)
        w.cnt[Lg * kTileRows + 8 * wv + 2 * j + g] = (uint32_t)(g ? cnt_hi[j] : cnt_lo[j]);
  }
}

// One wave per row of the group: the exact top-k_B from the candidate list.
__global__ __launch_bounds__(kCutWaves * 64) void index_cut_kernel(IndexArgs a, PipeWs w, int g0,
                                                                    int ntiles, int nrows) {
  __shared__ uint32_t hist[kCutWaves][256];
  // the wave index as a scalar: the row, its count and its list are then
  // wave-uniform
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int slot = blockIdx.x * kCutWaves + wv;
  if (slot >= nrows) return;
  const int Lg = slot / kTileRows;
  const TileGeo G = tile_geo(a, g0 + Lg, ntiles);
  const int t = G.row0 + slot % kTileRows;
  if (t >= a.n_q) return;
  const int nvis = (int)((G.seq_off + t + 1) / a.r);
  const int c = (int)w.cnt[slot];
  uint64_t* list = w.list + (size_t)slot * kList;
  const int k = min(a.kB, nvis);
  int32_t* out = a.idx + ((int64_t)G.b * a.n_q + t) * a.kB;
  if (c < k || c > kList) {
    if (lane == 0) atomicOr(&w.fail[Lg], 1u);
    return;
  }
  if (k == 0) {
    for (int e = lane; e < a.kB; e += 64) out[e] = -1;
  } else if (c == k) {  // everything is kept: copy in order
    for (int e = lane; e < a.kB; e += 64) out[e] = e < c ? (int32_t)(uint32_t)list[e] : -1;
  } else {
    // One read of the list: lane holds entries lane + 64 j in registers, for
    // the radix select (scores) and the order-preserving keep pass.
    constexpr int J = kList / 64;
    uint32_t klo[J], khi[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = lane + 64 * j;
      const uint64_t key = e < c ? list[e] : 0ull;
      klo[j] = (uint32_t)key;
      khi[j] = (uint32_t)(key >> 32);
    }
    uint32_t v;
    int krem;
    wave_radix_kth_regs(khi, c, k, hist[wv], lane, &v, &krem);
    // the top k in block order: every score above v, then the first krem
    // scores equal to v (smaller block ids win ties)
    const uint64_t lt = lanemask_lt(lane);
    int written = 0, eq_seen = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (64 * j >= c) break;
      const int e = lane + 64 * j;
      const bool valid = e < c;
      const bool gt = valid && khi[j] > v;
      const bool eq = valid && khi[j] == v;
      const uint64_t beq = __ballot(eq);
      const int eq_rank = eq_seen + __popcll(beq & lt);
      const bool keep = gt || (eq && eq_rank < krem);
      const uint64_t bk = __ballot(keep);
      const int pos = written + __popcll(bk & lt);
      if (keep && pos < k) out[pos] = (int32_t)klo[j];
      written += __popcll(bk);
      eq_seen += __popcll(beq);
    }
    for (int e = k + lane; e < a.kB; e += 64) out[e] = -1;
  }
  if (lane == 0) a.cnt[(int64_t)G.b * a.n_q + t] = k;
}

// ---- host side ------------------------------------------------------------

static int group_tiles(int total) { return total < kGroupTiles ? total : kGroupTiles; }

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static PipeWs carve(void* ws, int B, int n_q, int num_cu, size_t* total_bytes) {
  const int ntiles = (n_q + kTileRows - 1) / kTileRows;
  PipeWs w;
  w.gt = group_tiles(ntiles * B);
  const size_t rows = (size_t)w.gt * kTileRows;
  size_t lb = rows * kList * sizeof(uint64_t);
  const size_t eb = index_exact_workspace(B, n_q, num_cu);  // shares the list region
  if (eb > lb) lb = eb;
  char* p = (char*)ws;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* q = p ? p + off : nullptr;
    off += align256(bytes);
    return q;
  };
  w.list = (uint64_t*)take(lb);
  w.cnt = (uint32_t*)take(rows * sizeof(uint32_t));
  w.tau = (float*)take(rows * sizeof(float));
  w.fail = (uint32_t*)take((size_t)w.gt * sizeof(uint32_t));
  if (total_bytes) *total_bytes = off;
  return w;
}

// bf16 with at most 64 rotated dims (lo parts in registers), and k_B small
// enough that the lists hold a few times k_B
static bool pipeline_covers(qsa_dtype dt, const IndexArgs& a) {
  return dt == QSA_BF16 && a.R <= 64 && a.kB <= kList / 3;
}

size_t index_prefill_workspace(int B, int n_q, int num_cu, int kB) {
  (void)kB;
  size_t total = 0;
  carve(nullptr, B, n_q, num_cu, &total);
  const size_t ex = index_exact_workspace(B, n_q, num_cu);
  return total > ex ? total : ex;
}

template <int NLO>
static hipError_t run_pipeline(const IndexArgs& a, const PipeWs& w, int num_cu, hipStream_t st) {
  const int ntiles = (a.n_q + kTileRows - 1) / kTileRows;
  const int total = ntiles * a.B;
  hipError_t e;
  if ((e = hipFuncSetAttribute((const void*)index_scan_kernel<0, true>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, kScanLds)) != hipSuccess)
    return e;
  if ((e = hipFuncSetAttribute((const void*)index_scan_kernel<NLO, false>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, kScanLds)) != hipSuccess)
    return e;
  for (int g0 = 0; g0 < total; g0 += w.gt) {
    const int gt = total - g0 < w.gt ? total - g0 : w.gt;
    const int nrows = gt * kTileRows;
    const dim3 cg((unsigned)((nrows + kCutWaves - 1) / kCutWaves));
    // The threshold only has to be a value that at least k_B exact scores
    // reach (the cut checks that, else the row falls back to the exact
    // kernel), so the sample pass scores with the bf16 query alone.
    hipLaunchKernelGGL((index_scan_kernel<0, true>), dim3(gt), dim3(kScanWaves * 64), kScanLds,
                       st, a, w, g0, ntiles);
    hipLaunchKernelGGL((index_scan_kernel<NLO, false>), dim3(gt), dim3(kScanWaves * 64), kScanLds,
                       st, a, w, g0, ntiles);
    hipLaunchKernelGGL(index_cut_kernel, cg, dim3(kCutWaves * 64), 0, st, a, w, g0, ntiles, nrows);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // the lists are dead now: the exact kernel reuses their memory
    if ((e = launch_index_exact(QSA_BF16, a, w.list, num_cu, g0, gt, w.fail, st)) != hipSuccess)
      return e;
  }
  return hipSuccess;
}

hipError_t launch_index_prefill(qsa_dtype dt, const IndexArgs& a, void* ws, int num_cu,
                                hipStream_t st) {
  if (a.n_q == 0 || a.B == 0) return hipSuccess;
  if (!pipeline_covers(dt, a)) {
    const int total = ((a.n_q + kTileRows - 1) / kTileRows) * a.B;
    return launch_index_exact(dt, a, ws, num_cu, 0, total, nullptr, st);
  }
  const PipeWs w = carve(ws, a.B, a.n_q, num_cu, nullptr);
  // NLO: 16-dim k-steps holding rotated dims, ceil(R / 16)
  if (a.R == 0) return run_pipeline<0>(a, w, num_cu, st);
  if (a.R <= 32) return run_pipeline<2>(a, w, num_cu, st);
  return run_pipeline<4>(a, w, num_cu, st);
}

}  // namespace qsa
