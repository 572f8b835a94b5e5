// Compressed MQA indexer + top-k_B for a few new tokens per sequence
// (decode; paperglide reader, "QSA Ablations and Efficiency", Figure 6(d):
// decode with next_n new tokens per sequence).  Decode is bound by streaming
// the pooled key cache once, so the scan is spread over many workgroups and
// the selection works on a short candidate list:
//
//   prep    : one workgroup per (sequence, new token): rotates the indexer
//             queries once (fp32), clears the token's score histogram and
//             candidate counter.
//   scan    : grid (splits, B).  Each workgroup streams a contiguous range of
//             pooled keys (global -> MFMA B operand, two tiles prefetched per
//             wave), writes each score (4 bytes per 256-byte key row) and adds
//             its histogram of the score's top 11 value bits (exponent + 3
//             mantissa bits) into the token's global histogram.
//   collect : grid (slices, B * n_q).  Every workgroup finds the bin holding
//             the k_B-th largest score from the global histogram; when the
//             scores at or above that bin's lower edge fit kCandCap, it
//             writes its slice's share of them, in block order, to the
//             slice's own region of the token's candidate area (no atomics);
//             slice 0 also records the bin and the counts for select.
//   select  : one workgroup per (sequence, new token).  Gathers the slice
//             lists in slice order (= block order) and cuts them to the exact
//             top k_B (score desc, block id asc): the bin fixes the top 12
//             bits, two 10-bit radix passes the rest; writes ascending block
//             ids.  When the list would not fit (e.g. most scores are zero),
//             it selects from all scores instead, refining the histogram
//             until the candidates fit.
#include "index_common.h"

namespace qsa {

namespace {
constexpr int kBins = 2048;         // top 11 value bits of a non-negative float
constexpr int kScanThreads = 256;
constexpr int kSelThreads = 1024;
constexpr int kCandCap = 6016;      // candidates per token (global list and select LDS)
constexpr int kSliceLen = 8192;     // scores per collect workgroup
constexpr int kCollectThreads = 256;
constexpr int kPerThread = kSliceLen / kCollectThreads;  // 32
constexpr int kMaxSlicesFast = 1024;                    // slice table held in select LDS
}  // namespace

struct DecodeWs {
  float* qrot;       // [B*n_q][4][128] rotated indexer queries
  float* scores;     // [B*n_q][ld]
  uint32_t* ghist;   // [B*n_q][kBins]
  uint32_t* meta;    // [B*n_q][4]: bin of the k_B-th score, count above it, count >= its edge
  uint32_t* table;   // [B*n_q][nslice][2] (offset, count) of each slice's list
  uint64_t* cand;    // [B*n_q][nslice][kCandCap] (score bits << 32 | block id)
  int64_t ld;        // score row stride (multiple of 4 floats)
  int nsplit;
  int chunk;         // blocks per scan split (multiple of 64)
  int nslice;
};

static int decode_nsplit(int B, int64_t nb_cap, int* chunk_out) {
  // ~8 workgroups per CU over the whole batch, at least 256 blocks each; a
  // split is 64, 256 or 1024 blocks (1, 4 or 16 tiles of 16 blocks per wave,
  // a compile-time count, so the tile loop is straight-line code)
  int64_t want = (2048 + B - 1) / B;
  int64_t maxs = (nb_cap + 255) / 256;
  if (want > maxs) want = maxs;
  if (want < 1) want = 1;
  int64_t chunk = (nb_cap + want - 1) / want;
  chunk = chunk <= 64 ? 64 : (chunk <= 256 ? 256 : 1024);
  const int64_t ns = (nb_cap + chunk - 1) / chunk;
  *chunk_out = (int)chunk;
  return (int)(ns < 1 ? 1 : ns);
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static DecodeWs carve(void* ws, int B, int n_q, int64_t nb_cap, size_t* total) {
  DecodeWs d;
  d.nsplit = decode_nsplit(B, nb_cap, &d.chunk);
  d.ld = (nb_cap + 3) & ~(int64_t)3;
  d.nslice = (int)((nb_cap + kSliceLen - 1) / kSliceLen);
  if (d.nslice < 1) d.nslice = 1;
  const size_t rows = (size_t)B * n_q;
  char* p = (char*)ws;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* q = p ? p + off : nullptr;
    off += align256(bytes);
    return q;
  };
  d.qrot = (float*)take(rows * 4 * 128 * sizeof(float));
  d.scores = (float*)take(rows * (size_t)d.ld * sizeof(float));
  d.ghist = (uint32_t*)take(rows * kBins * sizeof(uint32_t));
  d.meta = (uint32_t*)take(rows * 4 * sizeof(uint32_t));
  d.table = (uint32_t*)take(rows * (size_t)d.nslice * 2 * sizeof(uint32_t));
  d.cand = (uint64_t*)take(rows * (size_t)d.nslice * kCandCap * sizeof(uint64_t));
  if (total) *total = off;
  return d;
}

size_t index_decode_workspace(int B, int n_q, int64_t nb_cap) {
  size_t total = 0;
  carve(nullptr, B, n_q, nb_cap, &total);
  return total;
}

__device__ __forceinline__ int64_t dec_pos(const IndexArgs& a, int b, int t) {
  return (int64_t)a.seq_len[b] - a.n_q + t;
}
__device__ __forceinline__ int64_t dec_nb(const IndexArgs& a, int b, int t) {
  const int64_t p = dec_pos(a, b, t);
  return p < 0 ? 0 : (p + 1) / a.r;
}

// Rotate the 4 indexer heads of one new token (RoPE at its position on the
// first R dims, rotate-half pairs) and clear its histogram.
template <typename T>
__global__ __launch_bounds__(256) void index_decode_prep(IndexArgs a, DecodeWs w) {
  __shared__ float2 table[64];
  const int tid = threadIdx.x;
  const int row = blockIdx.x, b = row / a.n_q, t = row % a.n_q;
  const int half = a.R / 2;
  const int64_t pos = dec_pos(a, b, t);
  // the query values are loaded first; the angles are formed while they fly
  const T* qr0 = (const T*)a.q_idx + (int64_t)row * a.h * 128;
  float xv[2], yv[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {  // elements tid and tid + 256 of the 4 x 128
    const int e = tid + 256 * k, hh = e >> 7, d = e & 127;
    const T* qr = qr0 + hh * 128;
    // head slots at or above h are zero queries
    xv[k] = hh < a.h ? Elt<T>::ld(qr, d) : 0.f;
    yv[k] = hh < a.h && d < a.R ? Elt<T>::ld(qr, d < half ? d + half : d - half) : 0.f;
  }
  for (int j = tid; j < half; j += 256) {
    float c, s;
    rope_cs(pos < 0 ? 0 : pos, j, a.R, a.log2_theta, &c, &s);
    table[j] = make_float2(c, s);
  }
  uint32_t* h = w.ghist + (int64_t)row * kBins;
  for (int e = tid; e < kBins; e += 256) h[e] = 0;
  __syncthreads();
  float* dst = w.qrot + (int64_t)row * 4 * 128;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int e = tid + 256 * k, d = e & 127;
    float val = xv[k];
    if (d < a.R) {
      const float2 cs = table[d < half ? d : d - half];
      val = d < half ? (xv[k] * cs.x - yv[k] * cs.y) : (yv[k] * cs.y + xv[k] * cs.x);
    }
    dst[e] = val;
  }
}

// TPW: 16-block tiles per wave (the split holds 4 * 16 * TPW blocks).
template <typename T, int NLO, int TPW>
__global__ __launch_bounds__(kScanThreads) void index_decode_scan(IndexArgs a, DecodeWs w) {
  typedef Mma<T> M;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_dec[];
  T* qs = (T*)smem_dec;                                           // [16][128]
  uint32_t* hist = (uint32_t*)(smem_dec + 16 * 128 * sizeof(T));  // [n_q][kBins]
  // the wave index as a scalar: tile positions are wave-uniform
  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63,
            hl = lane & 15, gq = lane >> 4;
  const int split = blockIdx.x, b = blockIdx.y;
  for (int e = tid; e < a.n_q * kBins; e += kScanThreads) hist[e] = 0;
  int64_t nbt[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) nbt[t] = t < a.n_q ? dec_nb(a, b, t) : 0;
  const int64_t nbmax = nbt[a.n_q - 1];
  const int64_t lo = (int64_t)split * w.chunk;
  const int64_t hi = min(lo + (int64_t)w.chunk, nbmax);
  const T* kb = (const T*)a.kbar + (size_t)b * a.nb_cap * 128;
  if (lo >= hi) return;  // the whole workgroup: nothing to scan, nothing to count
  // A operand rows 4t + h hold the rotated queries (zero for absent tokens);
  // bf16 keeps a low part for the rotated dims (see split_bf16)
  float vals[16 * 128 / kScanThreads];
#pragma unroll
  for (int u = 0; u < 16 * 128 / kScanThreads; ++u) {
    const int e = tid + kScanThreads * u;
    const int t = e >> 9;
    vals[u] = t < a.n_q ? w.qrot[((int64_t)b * a.n_q) * 512 + e] : 0.f;
  }
  // Wave wv takes the TPW 16-block tiles lo + 16 (wv + 4 j), j < TPW, in
  // three rotating buffers: the next two tiles are in flight while one is
  // scored.  The first three are issued while the queries are staged (after
  // the query loads, so staging waits on those alone).  The tile loop is
  // unrolled and every load is unconditional: the block index is clamped to
  // the workgroup's last block (hi > lo >= 0), so a tile past `hi` re-reads
  // rows the workgroup already fetched (cache hits) and is never scored, and
  // the compiler's load counts stay exact (a load inside a branch or a loop
  // makes it wait for every load in flight).
  auto load = [&](int64_t c0, typename M::Frag* f) {
    M::load_glb(kb + min(c0 + hl, hi - 1) * 128, gq, f);
  };
  typename M::Frag Bt[3][M::kCalls];
  const int64_t c00 = lo + 16 * wv;
#pragma unroll
  for (int j = 0; j < 3 && j < TPW; ++j) load(c00 + 64 * j, Bt[j]);
#pragma unroll
  for (int u = 0; u < 16 * 128 / kScanThreads; ++u) Elt<T>::st(qs, tid + kScanThreads * u, vals[u]);
  __syncthreads();
  typename M::Frag A[M::kCalls];
  typename M::Frag Alo[M::kSplit ? M::kCalls : 1];
  M::load_lds(qs, 128, hl, gq, A);
  if constexpr (M::kSplit && NLO > 0) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 16 * 128 / kScanThreads; ++u)
      Elt<T>::st(qs, tid + kScanThreads * u, vals[u] - bf16_to_f32(f32_to_bf16(vals[u])));
    __syncthreads();
    M::load_lds(qs, 128, hl, gq, Alo);
  }

  const int tq = gq < a.n_q ? gq : 0;
  const int64_t my_nb = gq < a.n_q ? nbt[gq] : 0;
  float* srow = w.scores + ((int64_t)b * a.n_q + tq) * w.ld;
  uint32_t* my_hist = hist + tq * kBins;
  auto score = [&](int64_t c0, const typename M::Frag* f) {
    const float sc = relu_sum4(M::template dot<NLO>(A, Alo, f));
    const int64_t blk = c0 + hl;
    if (blk < hi && blk < my_nb) {
      srow[blk] = sc;
      atomicAdd(&my_hist[__float_as_uint(sc) >> 20], 1u);
    }
  };
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    score(c00 + 64 * j, Bt[j % 3]);
    if (j + 3 < TPW) load(c00 + 64 * (j + 3), Bt[j % 3]);
  }
  __syncthreads();
  for (int e = tid; e < a.n_q * kBins; e += kScanThreads) {
    const uint32_t v = hist[e];
    if (v) atomicAdd(&w.ghist[(int64_t)b * a.n_q * kBins + e], v);
  }
}

// Block-wide (NT threads): over nbins bins held in LDS (hist), find the bin
// where the count of larger bins stays below k but reaches k with the bin
// itself.  Returns the bin (0 if the total is below k); *above = count of
// entries in larger bins.  red needs 2 * (NT / 64) + 2 words.
template <int NT>
__device__ int block_find_bin(const uint32_t* hist, int nbins, uint32_t k, uint32_t* red,
                              uint32_t* above) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = (nbins + NT - 1) / NT;  // bins per thread (high first)
  // thread tid owns bins [nbins - per*(tid+1), nbins - per*tid): thread 0 the largest
  const int hiB = nbins - per * tid, loB = max(0, hiB - per);
  if (tid == 0) {
    red[2 * NW] = 0;
    red[2 * NW + 1] = 0;
  }
  uint32_t mine = 0;
  for (int x = loB; x < hiB; ++x) mine += hist[x];
  // inclusive scan from thread 0 upward = count in bins >= loB
  uint32_t incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) red[wv] = incl;
  __syncthreads();
  if (tid < 64) {
    uint32_t v = tid < NW ? red[tid] : 0, s = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_up(s, off);
      if (lane >= off) s += y;
    }
    if (tid < NW) red[NW + tid] = s - v;  // exclusive prefix of wave totals
  }
  __syncthreads();
  incl += red[NW + wv];
  const uint32_t excl = incl - mine;
  if (excl < k && incl >= k) {
    uint32_t run = excl;
    for (int x = hiB - 1; x >= loB; --x) {
      if (run + hist[x] >= k) {
        red[2 * NW] = (uint32_t)x;
        red[2 * NW + 1] = run;
        break;
      }
      run += hist[x];
    }
  }
  __syncthreads();
  const int bin = min((int)red[2 * NW], nbins - 1);
  *above = red[2 * NW + 1];
  __syncthreads();
  return bin;
}

__global__ __launch_bounds__(kCollectThreads) void index_decode_collect(IndexArgs a, DecodeWs w) {
  constexpr int NW = kCollectThreads / 64;
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t red[2 * NW + 2];
  __shared__ uint32_t wsum[NW];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int slice = blockIdx.x, row = blockIdx.y;
  const int b = row / a.n_q, t = row % a.n_q;
  const int64_t nb = dec_nb(a, b, t);
  if (nb <= a.kB || slice >= w.nslice) return;
  // thread tid owns scores [s0 + 32 tid, s0 + 32 tid + 32) of this slice;
  // they are fetched first, while the threshold is found
  const int64_t s0 = (int64_t)slice * kSliceLen;
  const int64_t e0 = s0 + (int64_t)kPerThread * tid;
  const float* src = w.scores + (int64_t)row * w.ld;
  uint32_t bits[kPerThread];
#pragma unroll
  for (int j = 0; j < kPerThread; j += 4) {
    const int64_t e = e0 + j;
    if (e + 4 <= nb) {
      const f32x4 v = *(const f32x4*)(src + e);
#pragma unroll
      for (int z = 0; z < 4; ++z) bits[j + z] = __float_as_uint(v[z]);
    } else {
#pragma unroll
      for (int z = 0; z < 4; ++z) bits[j + z] = e + z < nb ? __float_as_uint(src[e + z]) : 0u;
    }
  }
  const uint32_t* gh = w.ghist + (int64_t)row * kBins;
  for (int e = tid; e < kBins; e += kCollectThreads) hist[e] = gh[e];
  __syncthreads();
  uint32_t above;
  const int bin = block_find_bin<kCollectThreads>(hist, kBins, (uint32_t)a.kB, red, &above);
  const uint32_t count = above + hist[bin];
  if (slice == 0 && tid == 0) {
    uint32_t* m = w.meta + (int64_t)row * 4;
    m[0] = (uint32_t)bin;
    m[1] = above;
    m[2] = count;
  }
  if (count > (uint32_t)kCandCap) return;  // select takes the exact route
  const uint32_t thr = (uint32_t)bin << 20;
  uint32_t mask = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (e0 + j < nb && bits[j] >= thr) mask |= 1u << j;
  const uint32_t mine = __popc(mask);
  uint32_t incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int x = 0; x < NW; ++x) {
    before += x < wv ? wsum[x] : 0u;
    total += wsum[x];
  }
  // the slice's share is at most the row's count (<= kCandCap): it has a
  // region of that size of its own
  const uint32_t off = (uint32_t)slice * kCandCap;
  if (tid == 0) {
    uint32_t* te = w.table + ((int64_t)row * w.nslice + slice) * 2;
    te[0] = off;
    te[1] = total;
  }
  uint32_t p = off + before + incl - mine;
  uint64_t* dst = w.cand + (int64_t)row * w.nslice * kCandCap;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (mask >> j & 1u) dst[p++] = ((uint64_t)bits[j] << 32) | (uint32_t)(e0 + j);
}

__global__ __launch_bounds__(kSelThreads) void index_decode_select(IndexArgs a, DecodeWs w) {
  constexpr int NW = kSelThreads / 64;
  __shared__ uint32_t hist[4096];  // histograms; slice table; radix bins of the final cut
  __shared__ uint64_t cand[kCandCap];
  __shared__ uint32_t red[2 * NW + 2];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int row = blockIdx.x, b = row / a.n_q, t = row % a.n_q;
  const int64_t nb = dec_nb(a, b, t);
  int32_t* out = a.idx + (int64_t)row * a.kB;
  if (nb <= a.kB) {
    for (int e = tid; e < a.kB; e += kSelThreads) out[e] = e < nb ? e : -1;
    if (tid == 0) a.cnt[row] = (int)nb;
    return;
  }
  const uint32_t k = (uint32_t)a.kB;
  // bin of the k-th score, entries in larger bins, entries >= its lower edge
  const uint32_t* mrow = w.meta + (int64_t)row * 4;
  const int bin = (int)mrow[0];
  uint32_t above = mrow[1];
  uint32_t count = mrow[2];
  int c;
  // radix cut of the collected list: the first pass resolves the bits below
  // `resolved` (the list's entries all share or exceed `cut_prefix` there)
  uint32_t cut_prefix = 0, cut_mask = 0, cut_krem = k;
  int cut_bits = 8;
  if (count <= (uint32_t)kCandCap && w.nslice <= kMaxSlicesFast) {
    // fast route: the collect kernel left every score >= bin << 20 in
    // per-slice lists; place them in slice order
    __syncthreads();
    uint32_t* spos = hist;               // [nslice] start of each slice in cand
    uint32_t* soff = hist + kMaxSlicesFast;
    const uint32_t* tab = w.table + (int64_t)row * w.nslice * 2;
    const uint32_t mine = tid < w.nslice ? tab[2 * tid + 1] : 0u;
    if (tid < w.nslice) soff[tid] = tab[2 * tid];
    uint32_t incl = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (lane == 63) red[wv] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (int x = 0; x < wv; ++x) before += red[x];
    if (tid < w.nslice) spos[tid] = before + incl - mine;
    __syncthreads();
    c = (int)count;
    const uint64_t* src = w.cand + (int64_t)row * w.nslice * kCandCap;
    const uint32_t lim = (uint32_t)w.nslice * kCandCap - 1;
    for (int pidx = tid; pidx < c; pidx += kSelThreads) {
      // slice holding list position pidx: the last s with spos[s] <= pidx
      int lo_s = 0, hi_s = w.nslice - 1;
      while (lo_s < hi_s) {
        const int mid = (lo_s + hi_s + 1) >> 1;
        if (spos[mid] <= (uint32_t)pidx) lo_s = mid; else hi_s = mid - 1;
      }
      // (empty slices share their start with the next slice, so the last
      // such s is never empty)
      cand[pidx] = src[min(soff[lo_s] + (pidx - spos[lo_s]), lim)];
    }
    __syncthreads();
    // every entry is >= the bin's edge; the `above` ones lie in larger bins
    cut_prefix = (uint32_t)bin << 20;
    cut_mask = 0xFFF00000u;
    cut_krem = k - above;
    cut_bits = 10;
  } else {
    // exact route over all scores: refine the bin while the candidates
    // (>= prefix) do not fit: 12 + 12 + 8 bits
    const float* sc = w.scores + (int64_t)row * w.ld;
    uint32_t prefix = (uint32_t)bin << 20;  // resolved high bits
    int resolved = 12;                       // number of resolved high bits
    while (count > (uint32_t)kCandCap && resolved < 32) {
      const int nbits = resolved == 12 ? 12 : 8;
      const int shift = 32 - resolved - nbits;
      const int nb2 = 1 << nbits;
      for (int e = tid; e < nb2; e += kSelThreads) hist[e] = 0;
      __syncthreads();
      const uint32_t hm = ~0u << (32 - resolved);
      for (int64_t e = tid; e < nb; e += kSelThreads) {
        const uint32_t sb = __float_as_uint(sc[e]);
        if ((sb & hm) == prefix) atomicAdd(&hist[(sb >> shift) & (nb2 - 1)], 1u);
      }
      __syncthreads();
      uint32_t ab2;
      const int b2 = block_find_bin<kSelThreads>(hist, nb2, k - above, red, &ab2);
      above += ab2;
      prefix |= (uint32_t)b2 << shift;
      resolved += nbits;
      count = above + hist[b2];
      __syncthreads();
    }
    // collect, in block order, every score >= prefix; when the value is fully
    // resolved keep only the first (k - above) entries equal to it.
    const bool exact = resolved >= 32;
    const uint32_t need_eq = k - above;
    uint32_t base = 0, eq_base = 0;
    const uint64_t lt = lanemask_lt(lane);
    for (int64_t c0 = 0; c0 < nb; c0 += kSelThreads) {
      const int64_t e = c0 + tid;
      const uint32_t sb = e < nb ? __float_as_uint(sc[e]) : 0u;
      const bool isc = e < nb && sb >= prefix;
      const bool iseq = exact && isc && sb == prefix;
      const uint64_t beq = __ballot(iseq);
      const uint64_t bc = __ballot(isc);
      if (lane == 0) {
        red[wv] = __popcll(bc);
        red[NW + wv] = __popcll(beq);
      }
      __syncthreads();
      uint32_t wofs = 0, wofs_eq = 0, tot = 0, tot_eq = 0;
      for (int x = 0; x < NW; ++x) {
        if (x < wv) {
          wofs += red[x];
          wofs_eq += red[NW + x];
        }
        tot += red[x];
        tot_eq += red[NW + x];
      }
      if (isc) {
        bool keep = true;
        if (iseq) keep = eq_base + wofs_eq + __popcll(beq & lt) < need_eq;
        if (keep) {
          // positions count kept entries only: equal entries beyond need_eq are dropped
          const uint32_t ne_before = (wofs - wofs_eq) + __popcll((bc & ~beq) & lt);
          uint32_t eq_before = wofs_eq + __popcll(beq & lt);
          const uint32_t eq_room = need_eq > eq_base ? need_eq - eq_base : 0;
          if (eq_before > eq_room) eq_before = eq_room;
          const uint32_t p = base + ne_before + eq_before;
          if (p < (uint32_t)kCandCap) cand[p] = ((uint64_t)sb << 32) | (uint32_t)e;
        }
      }
      const uint32_t eq_take =
          exact ? min(tot_eq, need_eq > eq_base ? need_eq - eq_base : 0u) : tot_eq;
      base += (tot - tot_eq) + eq_take;
      eq_base += tot_eq;
      __syncthreads();
    }
    c = (int)min(base, (uint32_t)kCandCap);
  }
  // exact cut of the collected list (ascending block order) by the whole
  // workgroup: radix select of the k-th score, then an ordered compaction
  // (every score above it, and the first equal ones up to k)
  __syncthreads();
  uint32_t prefix = cut_prefix, pmask = cut_mask;
  uint32_t krem = cut_krem;
  const int nbin = 1 << cut_bits;
  for (int shift = 32 - __popc(cut_mask) - cut_bits; shift >= 0; shift -= cut_bits) {
    for (int e = tid; e < nbin; e += kSelThreads) hist[e] = 0;
    __syncthreads();
    for (int e = tid; e < c; e += kSelThreads) {
      const uint32_t sb = (uint32_t)(cand[e] >> 32);
      if ((sb & pmask) == prefix) atomicAdd(&hist[(sb >> shift) & (uint32_t)(nbin - 1)], 1u);
    }
    __syncthreads();
    uint32_t ab;
    const int digit = block_find_bin<kSelThreads>(hist, nbin, krem, red, &ab);
    krem -= ab;
    prefix |= (uint32_t)digit << shift;
    pmask |= (uint32_t)(nbin - 1) << shift;
    __syncthreads();
  }
  const uint32_t v = prefix;  // the k-th largest score; krem equal ones are kept
  const uint64_t lt = lanemask_lt(lane);
  uint32_t written = 0, eq_seen = 0;
  for (int c0 = 0; c0 < c; c0 += kSelThreads) {
    const int e = c0 + tid;
    const uint64_t key = e < c ? cand[e] : 0ull;
    const uint32_t sb = (uint32_t)(key >> 32);
    const bool gt = e < c && sb > v;
    const bool eq = e < c && sb == v;
    const uint64_t beq = __ballot(eq);
    if (lane == 0) red[NW + wv] = __popcll(beq);
    __syncthreads();
    uint32_t eq_before = eq_seen, eq_tot = 0;
    for (int x = 0; x < NW; ++x) {
      eq_before += x < wv ? red[NW + x] : 0u;
      eq_tot += red[NW + x];
    }
    const bool keep = gt || (eq && eq_before + __popcll(beq & lt) < krem);
    const uint64_t bk = __ballot(keep);
    if (lane == 0) red[wv] = __popcll(bk);
    __syncthreads();
    uint32_t k_before = written, k_tot = 0;
    for (int x = 0; x < NW; ++x) {
      k_before += x < wv ? red[x] : 0u;
      k_tot += red[x];
    }
    const uint32_t pos = k_before + __popcll(bk & lt);
    if (keep && pos < k) out[pos] = (int32_t)(uint32_t)key;
    written += k_tot;
    eq_seen += eq_tot;
    __syncthreads();
  }
  if (tid == 0) a.cnt[row] = (int)k;
}

template <int TPW>
static hipError_t launch_scan_tpw(qsa_dtype dt, const IndexArgs& a, const DecodeWs& w, dim3 g1,
                                  size_t lds, hipStream_t st) {
  if (dt != QSA_BF16)
    hipLaunchKernelGGL((index_decode_scan<float, 0, TPW>), g1, dim3(kScanThreads), lds, st, a, w);
  else if (a.R == 0)
    hipLaunchKernelGGL((index_decode_scan<unsigned short, 0, TPW>), g1, dim3(kScanThreads), lds,
                       st, a, w);
  else if (a.R <= 64)
    hipLaunchKernelGGL((index_decode_scan<unsigned short, 2, TPW>), g1, dim3(kScanThreads), lds,
                       st, a, w);
  else
    hipLaunchKernelGGL((index_decode_scan<unsigned short, 4, TPW>), g1, dim3(kScanThreads), lds,
                       st, a, w);
  return hipGetLastError();
}

static hipError_t launch_scan(qsa_dtype dt, const IndexArgs& a, const DecodeWs& w, dim3 g1,
                              size_t lds, hipStream_t st) {
  switch (w.chunk) {
    case 64: return launch_scan_tpw<1>(dt, a, w, g1, lds, st);
    case 256: return launch_scan_tpw<4>(dt, a, w, g1, lds, st);
    default: return launch_scan_tpw<16>(dt, a, w, g1, lds, st);
  }
}

hipError_t launch_index_decode(qsa_dtype dt, const IndexArgs& a, void* ws, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const DecodeWs w = carve(ws, a.B, a.n_q, a.nb_cap, nullptr);
  const unsigned rows = (unsigned)(a.B * a.n_q);
  if (dt == QSA_BF16)
    hipLaunchKernelGGL(index_decode_prep<unsigned short>, dim3(rows), dim3(256), 0, st, a, w);
  else
    hipLaunchKernelGGL(index_decode_prep<float>, dim3(rows), dim3(256), 0, st, a, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g1((unsigned)w.nsplit, (unsigned)a.B);
  const size_t lds_bf = 16 * 128 * 2 + (size_t)a.n_q * kBins * 4;
  const size_t lds_f = 16 * 128 * 4 + (size_t)a.n_q * kBins * 4;
  if ((e = launch_scan(dt, a, w, g1, dt == QSA_BF16 ? lds_bf : lds_f, st)) != hipSuccess) return e;
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(index_decode_collect, dim3((unsigned)w.nslice, rows), dim3(kCollectThreads),
                     0, st, a, w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(index_decode_select, dim3(rows), dim3(kSelThreads), 0, st, a, w);
  return hipGetLastError();
}

}  // namespace qsa
