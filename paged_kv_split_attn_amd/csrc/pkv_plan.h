// Device-side planning shared by the metadata kernel and the decode that
// plans its own step: prefix sums of page counts, the split of the step's
// tiles into workgroup and wave ranges, and the workgroups' merge records.
// The plan cuts the step's tiles (request, head group, page) into equal
// contiguous ranges, one per workgroup and one per wave (the pages tuned their
// split count to the number of blocks that saturates bandwidth: commits by
// ViperEkura, compute_num_splits bullets).
#pragma once

#include "pkv_internal.h"

namespace pkv {
namespace {

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
  // floor(w len / kWavesPerGroup) without forming w len.
  __device__ static I part(I len, int w) {
    static_assert((kWavesPerGroup & (kWavesPerGroup - 1)) == 0, "a power-of-two wave count");
    constexpr int kShift = __builtin_ctz(kWavesPerGroup);
    return (I)w * (len >> kShift) +
           (I)(((uint32_t)w * (uint32_t)(len & (kWavesPerGroup - 1))) >> kShift);
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

// The same search when the requests are the lanes of one wave (batch <= 64):
// lane b holds request b's page prefix sum, page count and length, and one
// ballot finds the request (the lanes with prefix * U <= t form a prefix of
// the wave, since the prefix sums do not decrease).
struct WaveLocator {
  int excl;   // this lane's request: pages of the requests before it
  int pages;  // its pages
  int len;    // its length (tokens, may be negative)
  int batch, units;
  template <typename I>
  __device__ WaveRange at(I t, int count) const {
    const int lane = threadIdx.x & (kWave - 1);
    const bool before = lane < batch && (I)excl * (I)units <= t;
    const int b = __popcll(__ballot(before)) - 1;
    const int ip0 = __shfl(excl, b, kWave);
    const int n = __shfl(pages, b, kWave);
    const I rr = t - (I)ip0 * (I)units;
    const int u = (int)(rr / (I)n);
    WaveRange w;
    w.b = b;
    w.u = u;
    w.p = (int)(rr - (I)u * (I)n);
    w.count = count;
    w.ip0 = ip0;
    w.pages = n;
    w.len = max(__shfl(len, b, kWave), 0);
    w.pad = 0;
    return w;
  }
};

// Workgroups of a plan of T tiles: min(groups, ceil(T / min_tiles)), or
// min(forced, groups, T) when forced > 0; 0 when there is no tile.
__device__ __forceinline__ int plan_groups(long long T, int groups, int min_tiles, int forced) {
  if (T <= 0) return 0;
  if (forced > 0) {
    const int W = min(forced, groups);
    return (long long)W > T ? (int)T : W;  // every workgroup gets at least one tile
  }
  // ceil(T / min_tiles), in 32-bit arithmetic when T leaves room for it
  const long long want = T < 0x40000000LL
                             ? (long long)(((uint32_t)T + (uint32_t)min_tiles - 1u) /
                                           (uint32_t)min_tiles)
                             : (T + min_tiles - 1) / min_tiles;
  return (int)(want < groups ? want : groups);
}

// Range of wave w of workgroup i: workgroup i covers [start(i), start(i + 1));
// its wave w the w-th of kWavesPerGroup equal parts.  Empty past the plan.
template <typename I, typename Loc>
__device__ WaveRange plan_wave_range(const Loc& loc, const PlanMath<I>& pm, int W, int i,
                                     int w) {
  WaveRange r{0, 0, 0, 0, 0, 0, 0, 0};
  if (i < W) {
    const I g0 = pm.start(i), len = pm.start(i + 1) - g0;
    const I t0 = g0 + PlanMath<I>::part(len, w);
    const I t1 = g0 + PlanMath<I>::part(len, w + 1);
    if (t1 > t0) r = loc.at(t0, (int)(t1 - t0));
  }
  return r;
}

// The merge slots of wave w of workgroup i, whose range is r: its first piece
// (the part of segment (r.b, r.u) from page r.p on) is partial unless it starts
// at the segment's first page and covers the whole segment; its last piece,
// when the range reaches past the first segment, starts at its segment's
// first page and is partial when it stops before the segment's last page.
// Every piece between is a whole segment.
template <typename I, typename Loc>
__device__ void plan_wave_slots(const Loc& loc, const PlanMath<I>& pm, int i, int w, int U,
                                const WaveRange& r, int32_t* first, int32_t* last) {
  int s0 = -1, s1 = -1;
  if (r.count > 0) {
    const int first_len = min(r.count, r.pages - r.p);
    if (!(r.p == 0 && first_len == r.pages)) s0 = r.b * U + r.u;
    if (r.count > first_len) {
      const I g0 = pm.start(i), len = pm.start(i + 1) - g0;
      const I t1 = g0 + PlanMath<I>::part(len, w + 1);  // end of the wave's range
      const WaveRange e = loc.at(t1 - 1, 0);
      if (e.p + 1 < e.pages) s1 = e.b * U + e.u;
    }
  }
  *first = s0;
  *last = s1;
}

// Half k of the merge record of workgroup i: its first (k = 0) or last (k = 1)
// segment (b * U + u), and the workgroups that segment's tiles span.  A
// segment is the first segment of a workgroup exactly when that workgroup's
// range starts inside it.
template <typename I>
__device__ void plan_group_half(const Locator& loc, const PlanMath<I>& pm, int W, int U, int i,
                                int k, GroupInfo* gi) {
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
  gi->seg[k] = seg;
  gi->lo[k] = lo;
  gi->hi[k] = hi;
  gi->slot_lo[k] = slot;
}

}  // namespace
}  // namespace pkv
