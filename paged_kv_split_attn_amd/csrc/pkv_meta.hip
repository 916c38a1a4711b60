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
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kMetaThreads = 1024;
constexpr int kMetaWaves = kMetaThreads / kWave;

// Inclusive prefix sum over the 1024 threads of the block.  `total` receives
// the block sum.  smem holds kMetaWaves ints.
__device__ int block_inclusive_scan(int x, int* smem, int* total) {
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

struct Locator {
  const int32_t* ip;  // page prefix sums (LDS copy or global)
  const int32_t* seq_lens;
  int batch, units;
  // (request, head group, page) of tile t < T: the request is the largest b
  // with ip[b] * U <= t (requests without pages have empty ranges).
  __device__ WaveRange at(long long t, int count) const {
    int lo = 0, hi = batch;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((long long)ip[mid] * units <= t) lo = mid;
      else hi = mid - 1;
    }
    const int n = ip[lo + 1] - ip[lo];
    const long long r = t - (long long)ip[lo] * units;
    const int u = (int)(r / n);
    WaveRange w;
    w.b = lo;
    w.u = u;
    w.p = (int)(r - (long long)u * n);
    w.count = count;
    w.ip0 = ip[lo];
    w.pages = n;
    w.len = max(seq_lens[lo], 0);
    w.pad = 0;
    return w;
  }
};

__global__ void __launch_bounds__(kMetaThreads) metadata_kernel(MetaArgs a) {
  __shared__ int smem[kMetaWaves];
  __shared__ int s_err;
  __shared__ int s_empty;
  __shared__ int32_t s_ip[kMetaLdsRequests + 1];
  const int tid = threadIdx.x;
  const bool in_lds = a.batch <= kMetaLdsRequests;
  int err = 0;
  if (tid == 0) {
    s_err = 0;
    s_empty = 0;
    s_ip[0] = 0;
    a.kv_indptr[0] = 0;
  }

  // Phase 1: kv_indptr = exclusive prefix sum of page counts.
  int carry = 0, empty = 0;
  for (int base = 0; base < a.batch; base += kMetaThreads) {
    const int b = base + tid;
    int n = 0;
    if (b < a.batch) {
      const int L = a.seq_lens[b];
      if (L < 0) err |= kErrNegativeLength;
      n = pages_of(L, a.page_size);
      empty += n == 0;
    }
    int total;
    const int incl = block_inclusive_scan(n, smem, &total);
    if (b < a.batch) {
      a.kv_indptr[b + 1] = carry + incl;
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
  Locator loc{in_lds ? s_ip : a.kv_indptr, a.seq_lens, a.batch, U};

  // Phase 2: every wave's range.  Group i covers [i*T/W, (i+1)*T/W); its wave
  // w covers the w-th of kWavesPerGroup equal parts.
  for (int gw = tid; gw < a.groups * kWavesPerGroup; gw += kMetaThreads) {
    const int i = gw / kWavesPerGroup;
    const int w = gw - i * kWavesPerGroup;
    WaveRange r{0, 0, 0, 0, 0, 0, 0, 0};
    if (i < W) {
      const long long g0 = (long long)i * T / W, g1 = (long long)(i + 1) * T / W;
      const long long len = g1 - g0;
      const long long t0 = g0 + (long long)w * len / kWavesPerGroup;
      const long long t1 = g0 + (long long)(w + 1) * len / kWavesPerGroup;
      if (t1 > t0) r = loc.at(t0, (int)(t1 - t0));
    }
    a.waves[gw] = r;
  }

  // Phase 3: the merge record of every workgroup.  Its first and last segment
  // (b * U + u), and for each the workgroups its tiles span: tile t belongs to
  // workgroup floor(((t + 1) * W - 1) / T).  A segment is the first segment of
  // a workgroup exactly when that workgroup's range starts inside it.
  for (int i = tid; i < a.groups; i += kMetaThreads) {
    GroupInfo gi{{-1, -1}, {0, 0}, {-1, -1}, {0, 0}};
    const long long g0 = i < W ? (long long)i * T / W : 0;
    const long long g1 = i < W ? (long long)(i + 1) * T / W : 0;
    if (g1 > g0) {
      const WaveRange ends[2] = {loc.at(g0, 0), loc.at(g1 - 1, 0)};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const WaveRange& e = ends[k];
        const long long t0 = (long long)e.ip0 * U + (long long)e.u * e.pages;
        const long long t1 = t0 + e.pages - 1;
        const int lo = (int)(((t0 + 1) * W - 1) / T);
        gi.seg[k] = e.b * U + e.u;
        gi.lo[k] = lo;
        gi.hi[k] = (int)(((t1 + 1) * W - 1) / T);
        gi.slot_lo[k] = (long long)lo * T / W >= t0 ? 0 : 1;
      }
    }
    a.ginfo[i] = gi;
  }

  // Phase 4: arrival counters of the cross-workgroup merge.
  for (int sgi = tid; sgi < a.batch * U; sgi += kMetaThreads) a.counters[sgi] = 0;

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

// One thread per 8-channel chunk of (request, KV head, K or V) rows.  A K tile
// keeps 8-channel blocks of each token together ([D/8][P][8]): one 16-byte
// store per chunk.  V tiles are channel-major ([D][P]), so a V row is a column
// of its tile: eight 2-byte stores, page_size apart.
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
  const size_t tile = (((size_t)page * a.num_kv_heads + h) * a.page_size) * a.head_dim;
  const int off = pos % a.page_size;
  if (which == 0) {
    *reinterpret_cast<uint4*>(a.k + tile + ((size_t)c * a.page_size + off) * 8) = w;
  } else {
    const uint32_t words[4] = {w.x, w.y, w.z, w.w};
    uint16_t* col = a.v + tile + (size_t)c * 8 * a.page_size + off;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      col[(size_t)(2 * j) * a.page_size] = (uint16_t)(words[j] & 0xffffu);
      col[(size_t)(2 * j + 1) * a.page_size] = (uint16_t)(words[j] >> 16);
    }
  }
}

}  // namespace

hipError_t launch_metadata(const MetaArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(metadata_kernel, dim3(1), dim3(kMetaThreads), 0, s, a);
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
