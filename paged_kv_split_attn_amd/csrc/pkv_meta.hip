// Step metadata (page prefix sums + split plan) and the KV-append kernel.
//
// The prefix sum is built once per decode step and reused by every layer, as
// the pages moved it out of the per-layer attention call (AstrAI commit
// 05739629, astrai/inference, bind_tasks bullets).  The plan sizes chunks so a
// batch yields about target_items (chunk, KV head) work items: the pages tuned
// their split count to the number of blocks that saturates bandwidth
// (commits by ViperEkura, compute_num_splits bullets); here the count is sized
// for 256 CUs and computed on the device, so the host never reads seq_lens.
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

__global__ void __launch_bounds__(kMetaThreads) metadata_kernel(MetaArgs a) {
  __shared__ int smem[kMetaWaves];
  __shared__ int s_err;
  const int tid = threadIdx.x;
  int err = 0;
  if (tid == 0) s_err = 0;

  // Phase 1: kv_indptr = exclusive prefix sum of page counts.
  int carry = 0;
  if (tid == 0) a.kv_indptr[0] = 0;
  for (int base = 0; base < a.batch; base += kMetaThreads) {
    const int b = base + tid;
    int n = 0;
    if (b < a.batch) {
      const int L = a.seq_lens[b];
      if (L < 0) err |= kErrNegativeLength;
      n = pages_of(L, a.page_size);
    }
    int total;
    const int incl = block_inclusive_scan(n, smem, &total);
    if (b < a.batch) a.kv_indptr[b + 1] = carry + incl;
    carry += total;
  }
  const int N = carry;

  // Phase 2: chunks per request and their prefix sum.
  int chunk = 0;
  if (a.forced <= 0) {
    const long long want = ((long long)a.num_kv_heads * N + a.target_items - 1) / a.target_items;
    chunk = (int)(want > a.min_chunk ? want : a.min_chunk);
  }
  carry = 0;
  if (tid == 0) a.split_indptr[0] = 0;
  for (int base = 0; base < a.batch; base += kMetaThreads) {
    const int b = base + tid;
    int ns = 0;
    if (b < a.batch) {
      const int n = pages_of(a.seq_lens[b], a.page_size);
      if (n > 0) {
        if (a.forced > 0) {
          ns = min(min(a.forced, n), a.max_splits);
        } else {
          ns = min((n + chunk - 1) / chunk, a.max_splits);
        }
      }
    }
    int total;
    const int incl = block_inclusive_scan(ns, smem, &total);
    if (b < a.batch) {
      a.split_indptr[b + 1] = carry + incl;
      // Phase 3: the work list, ordered by request then chunk.
      const int first = carry + incl - ns;
      for (int s = 0; s < ns && first + s < a.max_items; ++s) a.items[first + s] = make_int2(b, s);
    }
    carry += total;
  }

  if (err) atomicOr(&s_err, err);
  __syncthreads();
  if (tid == 0) {
    // The metadata build starts a step: its bits replace the previous step's.
    a.hdr[kHdrError] = s_err;
    a.hdr[kHdrNumItems] = min(carry, a.max_items);
    a.hdr[kHdrChunk] = chunk;
    a.hdr[kHdrTotalPages] = N;
    a.hdr[kHdrBatch] = a.batch;
  }
}

// One thread per 16-byte chunk of (request, KV head, K or V) rows.
__global__ void __launch_bounds__(256) append_kernel(AppendArgs a) {
  const int chunks = a.head_dim / 8;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int c = (int)(idx % chunks);
  long long rest = idx / chunks;
  const int which = (int)(rest & 1);  // 0 = K, 1 = V
  rest >>= 1;
  const int h = (int)(rest % a.num_kv_heads);
  const long long b = rest / a.num_kv_heads;
  if (b >= a.batch) return;
  const int L = a.seq_lens[b];
  if (L <= 0) return;
  const int pos = L - 1;
  const long long slot = (long long)a.kv_indptr[b] + pos / a.page_size;
  if (slot < 0 || slot >= a.num_indices) return;
  const int page = a.kv_indices[slot];
  if (page < 0 || page >= a.num_pages) return;
  const uint16_t* src = which ? a.v_new : a.k_new;
  uint16_t* dst = which ? a.v : a.k;
  const size_t src_off = ((size_t)b * a.num_kv_heads + h) * a.head_dim + (size_t)c * 8;
  const size_t dst_off =
      (((size_t)page * a.num_kv_heads + h) * a.page_size + pos % a.page_size) * a.head_dim +
      (size_t)c * 8;
  *reinterpret_cast<uint4*>(dst + dst_off) = *reinterpret_cast<const uint4*>(src + src_off);
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
