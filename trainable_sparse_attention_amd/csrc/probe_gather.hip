// Gather-ceiling microbenchmark of the sparse attention's memory traffic.
//
// It reads exactly the K and V bytes the prefill attention gathers (paperglide
// reader, "Qwen Sparse Attention", Figure 3: each query reads the tokens of
// its selected micro-blocks and of its incomplete-block tail), in the same
// launch order (one 64-lane wave per query row and KV head), with the same
// per-wave LDS request (hence the same waves per CU) and the same cyclic
// chunk order, and does nothing with them: no dot products, no softmax.  Its
// time is the memory ceiling of that access pattern on this part, against
// which the attention kernel's own time is placed.
//
// Every slot (one selected block of 4 keys, or the tail) moves 1 KB of K and
// 1 KB of V with one 16-byte-per-lane global->LDS instruction each.  The LDS
// destination is shared by every instruction of the wave (the bytes are
// never read), so the probe can keep `depth` chunks of 8 slots in flight
// without the LDS it would otherwise need.  Slot ids come through scalar
// loads, so no vector-memory wait is spent on them.
#include "qsa_internal.h"

namespace qsa {

namespace {
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef const __attribute__((address_space(4))) i32x8* cids8_t;
constexpr int kProbeSlots = 8;  // slots per chunk, as in the attention
}  // namespace

template <int D>
__global__ __launch_bounds__(64) void probe_gather_kernel(AttnArgs a, int rg, int resident,
                                                          uint32_t* sink) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_probe[];
  const int lane = threadIdx.x;
  // wave -> (sequence, group of rg consecutive rows, KV head)
  const int ngroups = (a.n_q + rg - 1) / rg;
  int64_t w = blockIdx.x;
  const int g = (int)(w % a.hkv);
  w /= a.hkv;
  const int grp = (int)(w % ngroups);
  const int b = (int)(w / ngroups);
  const int t0 = grp * rg, t1 = min(a.n_q, t0 + rg);
  const char* kb = (const char*)a.k + ((int64_t)b * a.hkv + g) * a.n_cap * 256;
  const char* vb = (const char*)a.v + ((int64_t)b * a.hkv + g) * a.n_cap * 256;
  const int tok = lane >> 4;
  const uint64_t lofs = (uint64_t)(lane & 15) * 16;
  auto row_chunks = [&](int t) {
    const int64_t pos = a.q_pos0 + t;
    const int64_t nb = (pos + 1) / a.r;
    const int nslots = a.cnt[(int64_t)b * a.n_q + t] + ((pos + 1 - nb * a.r) > 0 ? 1 : 0);
    return (nslots + kProbeSlots - 1) / kProbeSlots;
  };
  // the group's longest row sets the sweep; a row with fewer chunks visits
  // chunk floor(c * its count / that count) at step c, each chunk once
  int nch = 0;
  for (int t = t0; t < t1; ++t) nch = max(nch, row_chunks(t));
  int ph = 0;
  if (resident > 0 && nch > 0)
    ph = (int)((((int64_t)(b * ngroups + grp) * a.hkv + g) * nch / resident) % nch);
  for (int cc = 0; cc < nch; ++cc) {
    int cw = ph + cc;
    if (cw >= nch) cw -= nch;
    for (int t = t0; t < t1; ++t) {
      const int64_t pos = a.q_pos0 + t;
      const int64_t nb = (pos + 1) / a.r;
      const int ntail = (int)(pos + 1 - nb * a.r);
      const int cnt = a.cnt[(int64_t)b * a.n_q + t];
      const int nslots = cnt + (ntail > 0 ? 1 : 0);
      const int nchr = (nslots + kProbeSlots - 1) / kProbeSlots;
      if (nchr == 0) continue;
      const int c = nchr == nch ? cw : (int)((int64_t)cw * nchr / nch);
      if (nchr != nch && c == (int)((int64_t)(cw == 0 ? nch - 1 : cw - 1) * nchr / nch) &&
          cw != 0)
        continue;  // a shorter row's chunk is visited once
      const int32_t* ids = a.idx + ((int64_t)b * a.n_q + t) * a.kB;
      // the chunk's 8 ids in one scalar load (k_B is a multiple of 8; a
      // chunk starting at k_B holds only the tail, whose id is not read)
      const int u0 = kProbeSlots * c;
      const i32x8 id8 = *(cids8_t)(ids + min(u0, a.kB - kProbeSlots));
#pragma unroll
      for (int i = 0; i < kProbeSlots; ++i) {
        const int u = u0 + i;
        const int64_t blk = u < cnt ? (int64_t)id8[i] : nb;
        const bool ok = u < cnt || (u < nslots && tok < ntail);
        const uint64_t row = ok ? (uint64_t)(blk * a.r + tok) : 0ull;
        __builtin_amdgcn_global_load_lds((glb_void_t*)(kb + row * 256 + lofs),
                                         (lds_void_t*)smem_probe, 16, 0, 0);
        __builtin_amdgcn_global_load_lds((glb_void_t*)(vb + row * 256 + lofs),
                                         (lds_void_t*)(smem_probe + 1024), 16, 0, 0);
      }
      // keep at most `depth` chunks (16 loads each) in flight
      if (D == 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (D == 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      if (D == 3) asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
      if (D == 4) asm volatile("s_waitcnt vmcnt(48)" ::: "memory");
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (lane == 0) sink[blockIdx.x] = *(const uint32_t*)smem_probe;
}

template <int D> static const void* probe_fn() { return (const void*)probe_gather_kernel<D>; }

hipError_t launch_probe_gather(const AttnArgs& a, int waves_per_cu, int depth, int rg,
                               uint32_t* sink, hipStream_t st) {
  const int64_t waves = (int64_t)a.B * ((a.n_q + rg - 1) / rg) * a.hkv;
  if (waves == 0) return hipSuccess;
  int dev = 0, per_cu = 0, cus = 0;
  hipError_t e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                                 dev)) != hipSuccess)
    return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return e;
  size_t lds = 2048;
  if (waves_per_cu > 0) {
    const size_t share = ((size_t)per_cu / waves_per_cu) & ~(size_t)255;
    if (share > lds) lds = share;
  }
  const void* fn = depth <= 1 ? probe_fn<1>() : depth == 2 ? probe_fn<2>()
                 : depth == 3 ? probe_fn<3>() : probe_fn<4>();
  int occ = 0;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, 64, lds)) != hipSuccess)
    return e;
  const int resident = occ * cus * 9 / 10;
  const dim3 grid((unsigned)waves), block(64);
  if (depth <= 1)
    hipLaunchKernelGGL(probe_gather_kernel<1>, grid, block, lds, st, a, rg, resident, sink);
  else if (depth == 2)
    hipLaunchKernelGGL(probe_gather_kernel<2>, grid, block, lds, st, a, rg, resident, sink);
  else if (depth == 3)
    hipLaunchKernelGGL(probe_gather_kernel<3>, grid, block, lds, st, a, rg, resident, sink);
  else
    hipLaunchKernelGGL(probe_gather_kernel<4>, grid, block, lds, st, a, rg, resident, sink);
  return hipGetLastError();
}

}  // namespace qsa
