// Step metadata (page prefix sums + work plan) and the KV-append kernel.
//
// The prefix sum is built once per decode step and reused by every layer, as
// the pages moved it out of the per-layer attention call (AstrAI commit
// 05739629, astrai/inference, bind_tasks bullets).  The plan then cuts the
// step's tiles (request, head group, page) into equal contiguous ranges, one
// per workgroup and one per wave: the pages tuned their split count to the
// number of blocks that saturates bandwidth (commits by ViperEkura,
// compute_num_splits bullets); here every wave gets the same number of pages
// whatever the length mix, and the plan is computed on the device, so the host
// never reads seq_lens.
#include <algorithm>

#include "pkv_internal.h"

namespace pkv {
namespace {

// Threads of a metadata workgroup: one wave up to 64 requests (its barriers
// cost next to nothing), 256 up to 256 requests, else 1024 (fewer passes of
// the block scan over the lengths).  A 16-request step (metadata + decode)
// measured 0.9 us shorter with one wave than with 1024 threads, 0.45 us with
// 256.
constexpr int kMetaThreadsTiny = 64;
constexpr int kMetaThreadsSmall = 256;
constexpr int kMetaThreadsLarge = 1024;

// Inclusive prefix sum over the THREADS threads of the block.  `total`
// receives the block sum.  smem holds THREADS / 64 ints.
template <int THREADS>
__device__ int block_inclusive_scan(int x, int* smem, int* total) {
  constexpr int kMetaWaves = THREADS / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) smem[w] = x;
  __syncthreads();
  if (w == 0) {
    int v = lane < kMetaWaves ? smem[lane] : 0;
#pragma unroll
    for (int off = 1; off < kMetaWaves; off <<= 1) {
      const int y = __shfl_up(v, off, kWave);
      if (lane >= off) v += y;
    }
    if (lane < kMetaWaves) smem[lane] = v;
  }
  __syncthreads();
  const int prefix = w > 0 ? smem[w - 1] : 0;
  *total = smem[kMetaWaves - 1];
  __syncthreads();  // smem is reused by the next scan
  return x + prefix;
}

__device__ __forceinline__ int pages_of(int len, int P) { return len > 0 ? (len + P - 1) / P : 0; }

// Integer arithmetic of the plan, in I = uint32_t when the step has fewer than
// 2^31 tiles (every division a 32-bit one) and uint64_t otherwise.  All
// results are the exact floors the plan defines, whatever I is.
template <typename I>
struct PlanMath {
  I T;         // tiles
  uint32_t W;  // workgroups, 1 <= W <= min(T, 65536)
  I q, r;      // T = q W + r
  __device__ PlanMath(I tiles, uint32_t groups) : T(tiles), W(groups), q(tiles / groups),
                                                  r(tiles % groups) {}
  // First tile of workgroup i (i <= W): floor(i T / W) = i q + floor(i r / W),
  // where i r <= 65536 * 65535 fits 32 bits.
  __device__ I start(uint32_t i) const { return (I)i * q + (I)(i * (uint32_t)r / W); }
  // floor(w len / 8) without forming w len.
  __device__ static I part(I len, int w) {
    return (I)w * (len >> 3) + (I)(((uint32_t)w * (uint32_t)(len & 7)) >> 3);
  }
  // Workgroup that owns tile t: floor(((t + 1) W - 1) / T), the largest i with
  // start(i) <= t.  In 32-bit plans the dividend is below 2^47, so a double
  // division is within one of the floor, and one integer check fixes it.
  __device__ uint32_t owner(I t) const {
    const uint64_t num = ((uint64_t)t + 1) * W - 1;
    if constexpr (sizeof(I) == 4) {
      uint64_t q = (uint64_t)((double)num / (double)T);
      if (q * T > num) --q;
      else if ((q + 1) * T <= num) ++q;
      return (uint32_t)q;
    } else {
      return (uint32_t)(num / T);
    }
  }
};

struct Locator {
  const int32_t* ip;  // page prefix sums (LDS copy or global)
  const int32_t* seq_lens;  // (LDS copy or global)
  int batch, units;
  // (request, head group, page) of tile t < T: the request is the largest b
  // with ip[b] * U <= t (requests without pages have empty ranges).
  template <typename I>
  __device__ WaveRange at(I t, int count) const {
    int lo = 0, hi = batch;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((I)ip[mid] * (I)units <= t) lo = mid;
      else hi = mid - 1;
    }
    const int n = ip[lo + 1] - ip[lo];
    const I rr = t - (I)ip[lo] * (I)units;
    const int u = (int)(rr / (I)n);
    WaveRange w;
    w.b = lo;
    w.u = u;
    w.p = (int)(rr - (I)u * (I)n);
    w.count = count;
    w.ip0 = ip[lo];
    w.pages = n;
    w.len = max(seq_lens[lo], 0);
    w.pad = 0;
    return w;
  }
};

// Phases 2 and 3 of the metadata kernel (see there), in integer type I.  The
// work items -- one per wave of the grid, then two per workgroup record -- are
// dealt to the threads of all metadata workgroups.
template <int THREADS, typename I>
__device__ void build_plan(const MetaArgs& a, const Locator& loc, I T, int W) {
  const int U = a.units;
  const PlanMath<I> pm(T, (uint32_t)max(W, 1));
  const int nw = a.groups * kWavesPerGroup;
  for (int x = blockIdx.x * THREADS + threadIdx.x; x < nw + 2 * a.groups;
       x += gridDim.x * THREADS) {
    if (x < nw) {
      // Phase 2: the range of wave w of group i.  Group i covers
      // [start(i), start(i + 1)); its wave w the w-th of kWavesPerGroup equal
      // parts.
      const int i = x / kWavesPerGroup;
      const int w = x - i * kWavesPerGroup;
      WaveRange r{0, 0, 0, 0, 0, 0, 0, 0};
      if (i < W) {
        const I g0 = pm.start(i), len = pm.start(i + 1) - g0;
        const I t0 = g0 + PlanMath<I>::part(len, w);
        const I t1 = g0 + PlanMath<I>::part(len, w + 1);
        if (t1 > t0) r = loc.at(t0, (int)(t1 - t0));
      }
      a.waves[x] = r;
    } else {
      // Phase 3: half k of the merge record of group i (two threads per
      // group): its first (k = 0) or last (k = 1) segment (b * U + u), and the
      // workgroups that segment's tiles span.  A segment is the first segment
      // of a workgroup exactly when that workgroup's range starts inside it.
      const int i = (x - nw) >> 1, k = (x - nw) & 1;
      int seg = -1, lo = 0, hi = -1, slot = 0;
      const I g0 = i < W ? pm.start(i) : 0;
      const I g1 = i < W ? pm.start(i + 1) : 0;
      if (g1 > g0) {
        const WaveRange e = loc.at(k == 0 ? g0 : g1 - 1, 0);
        const I t0 = (I)e.ip0 * (I)U + (I)e.u * (I)e.pages;
        const I t1 = t0 + (I)(e.pages - 1);
        const uint32_t l = pm.owner(t0);
        seg = e.b * U + e.u;
        lo = (int)l;
        hi = (int)pm.owner(t1);
        slot = pm.start(l) >= t0 ? 0 : 1;
      }
      GroupInfo& gi = a.ginfo[i];
      gi.seg[k] = seg;
      gi.lo[k] = lo;
      gi.hi[k] = hi;
      gi.slot_lo[k] = slot;
    }
  }
}

template <int THREADS>
__global__ void __launch_bounds__(THREADS) metadata_kernel(MetaArgs a) {
  __shared__ int smem[THREADS / kWave];
  __shared__ int s_err;
  __shared__ int s_empty;
  __shared__ int32_t s_ip[kMetaLdsRequests + 1];
  __shared__ int32_t s_len[kMetaLdsRequests];
  const int tid = threadIdx.x;
  const bool in_lds = a.batch <= kMetaLdsRequests;
  int err = 0;
  // Every workgroup builds the prefix sums for its own searches; workgroup 0
  // also writes kv_indptr, the counters and the header.  (With more requests
  // than LDS holds the launch has one workgroup, which searches kv_indptr.)
  const bool lead = blockIdx.x == 0;
  if (tid == 0) {
    s_err = 0;
    s_empty = 0;
    s_ip[0] = 0;
    if (lead) a.kv_indptr[0] = 0;
  }

  // Phase 1: kv_indptr = exclusive prefix sum of page counts.
  int carry = 0, empty = 0;
  for (int base = 0; base < a.batch; base += THREADS) {
    const int b = base + tid;
    int n = 0;
    if (b < a.batch) {
      const int L = a.seq_lens[b];
      if (in_lds) s_len[b] = L;
      if (L < 0) err |= kErrNegativeLength;
      n = pages_of(L, a.page_size);
      empty += n == 0;
    }
    int total;
    const int incl = block_inclusive_scan<THREADS>(n, smem, &total);
    if (b < a.batch) {
      if (lead) a.kv_indptr[b + 1] = carry + incl;
      if (in_lds) s_ip[b + 1] = carry + incl;
    }
    carry += total;
  }
  __syncthreads();

  const int U = a.units;
  const long long T = (long long)carry * U;
  int W = 0;
  if (T > 0) {
    if (a.forced > 0) {
      W = min(a.forced, a.groups);
      if ((long long)W > T) W = (int)T;  // every workgroup gets at least one tile
    } else {
      const long long want = (T + a.min_tiles - 1) / a.min_tiles;
      W = (int)(want < a.groups ? want : a.groups);
    }
  }
  // The searches read the prefix sums from LDS when they fit there (a
  // separate instantiation, so that they compile to LDS loads).
  const bool small = T < 0x80000000LL;
  if (in_lds) {
    const Locator loc{s_ip, s_len, a.batch, U};
    if (small) build_plan<THREADS, uint32_t>(a, loc, (uint32_t)T, W);
    else build_plan<THREADS, uint64_t>(a, loc, (uint64_t)T, W);
  } else {
    const Locator loc{a.kv_indptr, a.seq_lens, a.batch, U};
    if (small) build_plan<THREADS, uint32_t>(a, loc, (uint32_t)T, W);
    else build_plan<THREADS, uint64_t>(a, loc, (uint64_t)T, W);
  }

  if (!lead) return;
  // Phase 4: arrival counters of the cross-workgroup merge.
  for (int sgi = tid; sgi < a.batch * U; sgi += THREADS) a.counters[sgi] = 0;

  if (err) atomicOr(&s_err, err);
  if (empty) atomicAdd(&s_empty, empty);
  __syncthreads();
  if (tid == 0) {
    // The metadata build starts a step: its bits replace the previous step's.
    a.hdr[kHdrError] = s_err;
    a.hdr[kHdrGroups] = W;
    a.hdr[kHdrTiles] = (int)T;
    a.hdr[kHdrUnits] = U;
    a.hdr[kHdrBatch] = a.batch;
    a.hdr[kHdrEmpty] = s_empty;
  }
}

// One thread per 8-channel chunk of (request, KV head, K or V) rows.  A tile is
// page_size / 16 steps of 16 tokens; a K step keeps 8-channel blocks of each
// token together ([D/8][16][8]): one 16-byte store per chunk.  V steps are
// channel-major ([D][16]), so a V row is a column of its step: eight 2-byte
// stores, 16 elements apart.
__global__ void __launch_bounds__(256) append_kernel(AppendArgs a) {
  // 32-bit index arithmetic: the host checks that the grid fits.
  const uint32_t idx = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t lc = a.head_dim == 128 ? 4u : 3u;  // log2 of 8-channel chunks per row
  const int c = (int)(idx & ((1u << lc) - 1));
  const uint32_t rest = idx >> (lc + 1);
  const int which = (int)((idx >> lc) & 1);  // 0 = K, 1 = V
  const int h = (int)(rest % (uint32_t)a.num_kv_heads);
  const int b = (int)(rest / (uint32_t)a.num_kv_heads);
  if (b >= a.batch) return;
  // The length, the prefix sum and the new row are loaded together; only the
  // page id waits for them.  Invalid entries read a clamped index and write
  // nothing.
  const size_t src_off = ((size_t)b * a.num_kv_heads + h) * a.head_dim + (size_t)c * 8;
  const int L = a.seq_lens[b];
  const int ip = a.kv_indptr[b];
  const uint4 w = *reinterpret_cast<const uint4*>((which == 0 ? a.k_new : a.v_new) + src_off);
  const int pos = L - 1;
  const long long slot = (long long)ip + (pos >= 0 ? pos / a.page_size : 0);
  const bool slot_ok = L > 0 && slot >= 0 && slot < a.num_indices;
  const int page = slot_ok ? a.kv_indices[slot] : -1;
  if (!slot_ok || page < 0 || page >= a.num_pages) return;
  const int off = pos % a.page_size;
  // Step off / 16 of the (page, head) tile, then token off % 16 in it.
  const size_t step = ((((size_t)page * a.num_kv_heads + h) * a.page_size) + (off & ~15)) *
                      a.head_dim;
  if (which == 0) {
    *reinterpret_cast<uint4*>(a.k + step + ((size_t)c * 16 + (off & 15)) * 8) = w;
  } else {
    const uint32_t words[4] = {w.x, w.y, w.z, w.w};
    uint16_t* col = a.v + step + (size_t)c * 8 * 16 + (off & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      col[(size_t)(2 * j) * 16] = (uint16_t)(words[j] & 0xffffu);
      col[(size_t)(2 * j + 1) * 16] = (uint16_t)(words[j] >> 16);
    }
  }
}

// Extend append: request b's n_b = qo_indptr[b+1] - qo_indptr[b] new rows go
// to positions seq_len - n_b .. seq_len - 1.  A workgroup covers 16 rows of
// one (request, KV head) with one thread per (row, 8-channel chunk), rows
// fastest, so that the K chunks of one channel block of a step's consecutive
// tokens ([c][t][8]) form one run and their V values of one channel ([c][t])
// another.
__global__ void __launch_bounds__(256) append_rows_kernel(AppendArgs a) {
  const uint32_t nblk = (uint32_t)a.row_blocks;
  const uint32_t bid = blockIdx.x;
  const int blk = (int)(bid % nblk);
  const int h = (int)((bid / nblk) % (uint32_t)a.num_kv_heads);
  const int b = (int)(bid / nblk / (uint32_t)a.num_kv_heads);
  const int i = blk * 16 + (int)(threadIdx.x & 15);  // row of request b
  const int c = (int)(threadIdx.x >> 4);              // 8-channel chunk
  const int r0 = a.qo_indptr[b];
  const int n = a.qo_indptr[b + 1] - r0;
  const int L = a.seq_lens[b];
  const int ip = a.kv_indptr[b];
  if (i >= n || i >= a.max_rows) return;
  const int pos = L - n + i;
  if (pos < 0) return;
  const long long slot = (long long)ip + pos / a.page_size;
  const bool slot_ok = slot >= 0 && slot < a.num_indices;
  const int page = slot_ok ? a.kv_indices[slot] : -1;
  if (page < 0 || page >= a.num_pages) return;
  const size_t src = ((size_t)(r0 + i) * a.num_kv_heads + h) * a.head_dim + (size_t)c * 8;
  const uint4 kw = *reinterpret_cast<const uint4*>(a.k_new + src);
  const uint4 vw = *reinterpret_cast<const uint4*>(a.v_new + src);
  const int off = pos % a.page_size;
  const size_t step = ((((size_t)page * a.num_kv_heads + h) * a.page_size) + (off & ~15)) *
                      a.head_dim;
  *reinterpret_cast<uint4*>(a.k + step + ((size_t)c * 16 + (off & 15)) * 8) = kw;
  const uint32_t words[4] = {vw.x, vw.y, vw.z, vw.w};
  uint16_t* col = a.v + step + (size_t)c * 8 * 16 + (off & 15);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    col[(size_t)(2 * j) * 16] = (uint16_t)(words[j] & 0xffffu);
    col[(size_t)(2 * j + 1) * 16] = (uint16_t)(words[j] >> 16);
  }
}

}  // namespace

hipError_t launch_metadata(const MetaArgs& a, hipStream_t s) {
  // Plan items (one per wave of the decode grid, two per workgroup record)
  // spread over several workgroups when the prefix sums fit in LDS.
  const long long items = (long long)a.groups * (kWavesPerGroup + 2);
  const int threads = a.batch <= kMetaThreadsTiny    ? kMetaThreadsTiny
                      : a.batch <= kMetaThreadsSmall ? kMetaThreadsSmall
                                                     : kMetaThreadsLarge;
  const int parts = a.batch <= kMetaLdsRequests
                        ? (int)std::max(1LL, (items + threads - 1) / threads)
                        : 1;
  if (threads == kMetaThreadsTiny)
    hipLaunchKernelGGL(metadata_kernel<kMetaThreadsTiny>, dim3(parts), dim3(threads), 0, s, a);
  else if (threads == kMetaThreadsSmall)
    hipLaunchKernelGGL(metadata_kernel<kMetaThreadsSmall>, dim3(parts), dim3(threads), 0, s, a);
  else
    hipLaunchKernelGGL(metadata_kernel<kMetaThreadsLarge>, dim3(parts), dim3(threads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  const long long threads = (long long)a.batch * a.num_kv_heads * 2 * (a.head_dim / 8);
  if (threads == 0) return hipSuccess;
  const int blocks = (int)((threads + 255) / 256);
  hipLaunchKernelGGL(append_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv

namespace pkv {

hipError_t launch_append_rows(const AppendArgs& a, hipStream_t s) {
  const long long blocks = (long long)a.batch * a.num_kv_heads * a.row_blocks;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(append_rows_kernel, dim3((uint32_t)blocks), dim3(16 * (a.head_dim / 8)), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace pkv
