// Compressed MQA indexer + top-k_B for a few new tokens per sequence
// (decode; paperglide reader, "QSA Ablations and Efficiency", Figure 6(d):
// decode with next_n new tokens per sequence).  Decode is bound by streaming
// the pooled key cache, so the scan is spread over many workgroups:
//
//   scan   : grid (splits, B).  Each workgroup streams a contiguous range of
//            pooled keys once (global -> MFMA B operand), writes each score
//            (4 bytes per 256-byte key row) and a 2048-bin histogram of the
//            score's top bits (exponent + 3 mantissa bits) for its range.
//   select : one workgroup per (sequence, new token).  Sums the split
//            histograms, finds the bin holding the k_B-th largest score,
//            collects every score at or above that bin's lower edge in block
//            order (refining the bin by further histogram passes if too
//            many), then cuts the collected list to the exact top k_B with
//            the same radix rule as the prefill kernel and writes the
//            ascending block ids.
#include "index_common.h"

namespace qsa {

namespace {
constexpr int kBins = 2048;        // top 11 value bits of a non-negative float
constexpr int kScanThreads = 256;
constexpr int kSelThreads = 1024;
constexpr int kSelCap = 4096;      // candidates held in LDS by the select kernel
}  // namespace

struct DecodeWs {
  float* scores;     // [B][n_q][nb_cap]
  uint32_t* hist;    // [B][n_q][nsplit][kBins]
  int nsplit;
  int chunk;         // blocks per split (multiple of 64)
};

static int decode_nsplit(int B, int64_t nb_cap, int* chunk_out) {
  // ~4 workgroups per CU over the whole batch, at least 1024 blocks each.
  int64_t want = (1024 + B - 1) / B;
  int64_t maxs = (nb_cap + 1023) / 1024;
  if (want > maxs) want = maxs;
  if (want < 1) want = 1;
  int64_t chunk = (nb_cap + want - 1) / want;
  chunk = (chunk + 63) & ~(int64_t)63;
  const int64_t ns = (nb_cap + chunk - 1) / chunk;
  *chunk_out = (int)chunk;
  return (int)(ns < 1 ? 1 : ns);
}

size_t index_decode_workspace(int B, int n_q, int64_t nb_cap) {
  int chunk;
  const int ns = decode_nsplit(B, nb_cap, &chunk);
  const size_t sc = (size_t)B * n_q * nb_cap * sizeof(float);
  const size_t hs = (size_t)B * n_q * ns * kBins * sizeof(uint32_t);
  return ((sc + 255) & ~(size_t)255) + hs;
}

static DecodeWs carve(void* ws, int B, int n_q, int64_t nb_cap) {
  DecodeWs d;
  d.nsplit = decode_nsplit(B, nb_cap, &d.chunk);
  d.scores = (float*)ws;
  const size_t sc = (size_t)B * n_q * nb_cap * sizeof(float);
  d.hist = (uint32_t*)((char*)ws + ((sc + 255) & ~(size_t)255));
  return d;
}

template <typename T, int NLO>
__global__ __launch_bounds__(kScanThreads) void index_decode_scan(IndexArgs a, DecodeWs w) {
  typedef Mma<T> M;
  __shared__ uint32_t hist[4][kBins];
  __shared__ __attribute__((aligned(16))) T qrot[16 * 128];
  __shared__ float2 table[4][64];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, hl = lane & 15, gq = lane >> 4;
  const int split = blockIdx.x, b = blockIdx.y;
  const int half = a.R / 2;
  for (int e = tid; e < 4 * kBins; e += kScanThreads) (&hist[0][0])[e] = 0;
  int64_t pos[4];
  int64_t nbt[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    pos[t] = t < a.n_q ? (int64_t)a.seq_len[b] - a.n_q + t : 0;
    nbt[t] = t < a.n_q ? (pos[t] + 1) / a.r : 0;
  }
  for (int e = tid; e < 4 * half; e += kScanThreads) {
    const int t = e / half, j = e % half;
    float c = 1.f, s = 0.f;
    if (t < a.n_q) rope_cs(pos[t], j, a.R, a.log2_theta, &c, &s);
    table[t][j] = make_float2(c, s);
  }
  __syncthreads();
  // rotated query rows 4t + h (t < n_q), rows of absent tokens are zero;
  // bf16 keeps a low part for the rotated dims (see split_bf16)
  const T* qsrc = (const T*)a.q_idx;
  float vals[16 * 128 / kScanThreads];
#pragma unroll
  for (int u = 0; u < 16 * 128 / kScanThreads; ++u) {
    const int e = tid + kScanThreads * u;
    const int rr = e >> 7, d = e & 127, t = rr >> 2, hh = rr & 3;
    float val = 0.f;
    if (t < a.n_q) {
      const T* qr = qsrc + (((int64_t)b * a.n_q + t) * 4 + hh) * 128;
      const float x = Elt<T>::ld(qr, d);
      if (d < a.R) {
        const int j = d < half ? d : d - half;
        const float2 cs = table[t][j];
        const float y = Elt<T>::ld(qr, d < half ? d + half : d - half);
        val = d < half ? (x * cs.x - y * cs.y) : (y * cs.y + x * cs.x);
      } else {
        val = x;
      }
    }
    vals[u] = val;
    Elt<T>::st(qrot, e, val);
  }
  __syncthreads();
  typename M::Frag A[M::kCalls];
  typename M::Frag Alo[M::kSplit ? M::kCalls : 1];
  M::load_lds(qrot, 128, hl, gq, A);
  if constexpr (M::kSplit && NLO > 0) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 16 * 128 / kScanThreads; ++u)
      Elt<T>::st(qrot, tid + kScanThreads * u, vals[u] - bf16_to_f32(f32_to_bf16(vals[u])));
    __syncthreads();
    M::load_lds(qrot, 128, hl, gq, Alo);
  }

  const int64_t nbmax = nbt[a.n_q - 1];
  const int64_t lo = (int64_t)split * w.chunk;
  const int64_t hi = min(lo + (int64_t)w.chunk, nbmax);
  const T* kb = (const T*)a.kbar + (size_t)b * a.nb_cap * 128;
  const int64_t my_nb = gq < a.n_q ? nbt[gq] : 0;
  float* srow = w.scores + ((int64_t)b * a.n_q + (gq < a.n_q ? gq : 0)) * a.nb_cap;
  // waves take 16-block column tiles round robin; two tiles in flight
  for (int64_t c0 = lo + 16 * wv; c0 < hi; c0 += 16 * 4 * 2) {
    typename M::Frag B0[M::kCalls], B1[M::kCalls];
    const int64_t c1 = c0 + 16 * 4;
    const int64_t r0 = min(c0 + hl, nbmax - 1), r1 = min(c1 + hl, nbmax - 1);
    M::load_glb(kb + r0 * 128, gq, B0);
    const bool has1 = c1 < hi;
    if (has1) M::load_glb(kb + r1 * 128, gq, B1);
    {
      const float sc = relu_sum4(M::template dot<NLO>(A, Alo, B0));
      const int64_t blk = c0 + hl;
      if (blk < hi && blk < my_nb) {
        srow[blk] = sc;
        atomicAdd(&hist[gq][__float_as_uint(sc) >> 20], 1u);
      }
    }
    if (has1) {
      const float sc = relu_sum4(M::template dot<NLO>(A, Alo, B1));
      const int64_t blk = c1 + hl;
      if (blk < hi && blk < my_nb) {
        srow[blk] = sc;
        atomicAdd(&hist[gq][__float_as_uint(sc) >> 20], 1u);
      }
    }
  }
  __syncthreads();
  for (int t = 0; t < a.n_q; ++t) {
    uint32_t* dst = w.hist + (((int64_t)b * a.n_q + t) * w.nsplit + split) * kBins;
    for (int e = tid; e < kBins; e += kScanThreads) dst[e] = hist[t][e];
  }
}

// Block-wide: over nbins bins held in LDS (hist), find the bin where the
// count of larger bins stays below k but reaches k with the bin itself.
// Returns the bin; *above = count of entries in larger bins.
__device__ int block_find_bin(const uint32_t* hist, int nbins, uint32_t k, uint32_t* red,
                              uint32_t* above) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = (nbins + kSelThreads - 1) / kSelThreads;  // bins per thread (high first)
  // thread tid owns bins [nbins - per*(tid+1), nbins - per*tid): thread 0 the largest
  const int hiB = nbins - per * tid, loB = max(0, hiB - per);
  if (tid == 0) {
    red[40] = 0;
    red[41] = 0;
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
    uint32_t v = tid < kSelThreads / 64 ? red[tid] : 0, s = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_up(s, off);
      if (lane >= off) s += y;
    }
    if (tid < kSelThreads / 64) red[16 + tid] = s - v;  // exclusive prefix of wave totals
  }
  __syncthreads();
  incl += red[16 + wv];
  const uint32_t excl = incl - mine;
  if (excl < k && incl >= k) {
    uint32_t run = excl;
    for (int x = hiB - 1; x >= loB; --x) {
      if (run + hist[x] >= k) {
        red[40] = (uint32_t)x;
        red[41] = run;
        break;
      }
      run += hist[x];
    }
  }
  __syncthreads();
  const int bin = min((int)red[40], nbins - 1);
  *above = red[41];
  __syncthreads();
  return bin;
}

__global__ __launch_bounds__(kSelThreads) void index_decode_select(IndexArgs a, DecodeWs w) {
  __shared__ uint32_t hist[4096];
  __shared__ uint64_t cand[kSelCap];
  __shared__ uint32_t red[64];
  __shared__ uint32_t whist[4][256];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = blockIdx.x / a.n_q, t = blockIdx.x % a.n_q;
  const int64_t pos = (int64_t)a.seq_len[b] - a.n_q + t;
  const int64_t nb = (pos + 1) / a.r;
  int32_t* out = a.idx + ((int64_t)b * a.n_q + t) * a.kB;
  if (nb <= a.kB) {
    for (int e = tid; e < a.kB; e += kSelThreads) out[e] = e < nb ? e : -1;
    if (tid == 0) a.cnt[(int64_t)b * a.n_q + t] = (int)nb;
    return;
  }
  const uint32_t k = (uint32_t)a.kB;
  const float* sc = w.scores + ((int64_t)b * a.n_q + t) * a.nb_cap;
  // level 1: the scan's histograms (bits 30..20)
  const uint32_t* hs = w.hist + ((int64_t)b * a.n_q + t) * w.nsplit * kBins;
  for (int e = tid; e < kBins; e += kSelThreads) {
    uint32_t s = 0;
    for (int p = 0; p < w.nsplit; ++p) s += hs[(int64_t)p * kBins + e];
    hist[e] = s;
  }
  __syncthreads();
  uint32_t above;
  int bin = block_find_bin(hist, kBins, k, red, &above);
  uint32_t prefix = (uint32_t)bin << 20;  // resolved high bits
  int resolved = 12;                       // number of resolved high bits
  uint32_t count = above + hist[bin];
  // refine while the candidates (>= prefix) do not fit: 12 + 12 + 8 bits
  while (count > (uint32_t)kSelCap && resolved < 32) {
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
    const int b2 = block_find_bin(hist, nb2, k - above, red, &ab2);
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
      red[16 + wv] = __popcll(beq);
    }
    __syncthreads();
    uint32_t wofs = 0, wofs_eq = 0, tot = 0, tot_eq = 0;
    for (int x = 0; x < kSelThreads / 64; ++x) {
      if (x < wv) {
        wofs += red[x];
        wofs_eq += red[16 + x];
      }
      tot += red[x];
      tot_eq += red[16 + x];
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
        if (p < (uint32_t)kSelCap) cand[p] = ((uint64_t)sb << 32) | (uint32_t)e;
      }
    }
    const uint32_t eq_take = exact ? min(tot_eq, need_eq > eq_base ? need_eq - eq_base : 0u) : tot_eq;
    base += (tot - tot_eq) + eq_take;
    eq_base += tot_eq;
    __syncthreads();
  }
  const int c = (int)min(base, (uint32_t)kSelCap);
  // exact cut of the collected list by wave 0 (list is in ascending block order)
  if (wv == 0) {
    uint32_t v;
    int krem;
    wave_radix_kth([&](int e) { return (uint32_t)(cand[e] >> 32); }, c, (int)k, whist[0], lane,
                   &v, &krem);
    wave_keep_topk(cand, c, (int)k, v, krem, lane, 1, out, a.kB);
    if (lane == 0) a.cnt[(int64_t)b * a.n_q + t] = (int)k;
  }
}

hipError_t launch_index_decode(qsa_dtype dt, const IndexArgs& a, void* ws, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const DecodeWs w = carve(ws, a.B, a.n_q, a.nb_cap);
  const dim3 g1((unsigned)w.nsplit, (unsigned)a.B);
  if (dt != QSA_BF16)
    hipLaunchKernelGGL((index_decode_scan<float, 0>), g1, dim3(kScanThreads), 0, st, a, w);
  else if (a.R == 0)
    hipLaunchKernelGGL((index_decode_scan<unsigned short, 0>), g1, dim3(kScanThreads), 0, st, a, w);
  else if (a.R <= 64)
    hipLaunchKernelGGL((index_decode_scan<unsigned short, 2>), g1, dim3(kScanThreads), 0, st, a, w);
  else
    hipLaunchKernelGGL((index_decode_scan<unsigned short, 4>), g1, dim3(kScanThreads), 0, st, a, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(index_decode_select, dim3((unsigned)(a.B * a.n_q)), dim3(kSelThreads), 0, st,
                     a, w);
  return hipGetLastError();
}

}  // namespace qsa
