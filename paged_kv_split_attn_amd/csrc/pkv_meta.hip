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

#include "pkv_plan.h"

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

// Phases 2 and 3 of the metadata kernel (see there), in integer type I.  The
// work items -- one per wave of the grid, then two per workgroup record -- are
// dealt to the threads of all metadata workgroups.
template <int THREADS, typename I>
__device__ void build_plan(const MetaArgs& a, const Locator& loc, I T, int W) {
  const PlanMath<I> pm(T, (uint32_t)max(W, 1));
  const int nw = a.groups * kWavesPerGroup;
  for (int x = blockIdx.x * THREADS + threadIdx.x; x < nw + 2 * a.groups;
       x += gridDim.x * THREADS) {
    if (x < nw) {
      const int i = x / kWavesPerGroup;
      const int w = x - i * kWavesPerGroup;
      const WaveRange r = plan_wave_range<I>(loc, pm, W, i, w);
      a.waves[x] = r;
      plan_wave_slots<I>(loc, pm, i, w, a.units, r, &a.ginfo[i].slot_seg[2 * w],
                         &a.ginfo[i].slot_seg[2 * w + 1]);
    } else {
      const int i = (x - nw) >> 1, k = (x - nw) & 1;
      plan_group_half<I>(loc, pm, W, a.units, i, k, &a.ginfo[i]);
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
  const int W = plan_groups(T, a.groups, a.min_tiles, a.forced);
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
  // Phase 4: arrival counters of the cross-workgroup merge, all of the
  // descriptor's (every decode leaves them at zero again, so a later step of
  // any batch, planned in its decode launch, finds them cleared).
  for (int sgi = tid; sgi < a.segments; sgi += THREADS) a.counters[sgi] = 0;

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
