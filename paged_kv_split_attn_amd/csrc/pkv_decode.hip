// Paged split-KV decode attention for gfx950 (MI355X), one kernel per call.
//
// Work decomposition (stream-K style).  The step's tiles, ordered (request,
// head group, page), are cut into equal contiguous ranges: one per workgroup of
// eight waves, one eighth of that per wave.  A head group is HG query heads
// that share one KV head (HG = G for G <= 4), so a tile is one page of one KV
// head, K and V, read once for HG query heads.  Each wave streams its range,
// keeping an online-softmax state that it closes whenever the range leaves a
// (request, head group) segment.  A segment wholly inside a wave is written
// straight to the output; other pieces go to LDS, where the workgroup merges
// the pieces of each segment; a segment that also spans other workgroups leaves
// a normalised partial and its log-sum-exp in the workspace, and the last
// workgroup to arrive merges them in a fixed order.  Split partials merged by
// log-sum-exp follow the pages' decode design (commits by ViperEkura: o_part /
// ml_part partials and their combine kernel); here the merge is fused into the
// same launch and every wave gets the same number of pages.  K and V go
// straight from HBM into registers with 16-byte loads: every element is used by
// exactly one lane, so LDS staging would only add traffic.
//
// Lane layout inside a wave (head_dim D, LPT = D / 16 lanes per token,
// TPR = 64 / LPT tokens per round).  Lane l serves token slot l / LPT of a round
// and holds 16 of the token's D channels: channels [8e, 8e + 8) and
// [D/2 + 8e, D/2 + 8e + 8) with e = l % LPT.  Each half is one 16-byte load, so
// one load instruction of the wave reads TPR half-rows of 128 (D=128) or 64
// (D=64) contiguous bytes.  q.K partial dot products use v_dot2 on bf16 pairs,
// then DPP adds inside the LPT-lane group.  Every lane keeps its own online
// softmax state (running max m, sum l, 16-channel accumulators per head) for
// the tokens of its slot; slots are merged once per piece.
//
// The running max is updated lazily: the accumulators are rescaled only when
// a score exceeds the stored max by more than 2^8 in the exp2 domain, so
// weights stay below 256 and the rescale branch is rarely taken after the
// first round.  Scores are kept in the log2 domain (sm_scale * log2 e folded
// into one multiply) so every exponential is a single v_exp_f32.
#include <math.h>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr float kRescaleSlack = 8.0f;  // log2 of the largest un-rescaled weight
constexpr float kMinusInf = -INFINITY;
constexpr float kFloorMax = -1.0e30f;  // initial running max (finite: exp2 never sees inf - inf)

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// fp32 -> bf16 bits, round to nearest even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// Stores and loads coherent across the XCDs' L2 caches (agent scope), used for
// the partials one workgroup hands to another.  They compile to sc1 accesses:
// no L2 write-back or invalidate is needed around them.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every earlier store of the wave has been acknowledged (for the
// sc1 stores above: is visible at agent scope).  s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// DPP lane moves inside a row of 16 lanes.
enum DppCtrl : int {
  kQuadXor1 = 0xB1,      // quad_perm [1,0,3,2]
  kQuadXor2 = 0x4E,      // quad_perm [2,3,0,1]
  kRowHalfMirror = 0x141,
  kRowRor4 = 0x124,
  kRowRor8 = 0x128,
};

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Sum over the LPT consecutive lanes that share a token (LPT = 4 or 8).
template <int LPT>
__device__ __forceinline__ float token_group_sum(float x) {
  x += dpp_mov<kQuadXor1>(x);
  x += dpp_mov<kQuadXor2>(x);
  if constexpr (LPT == 8) x += dpp_mov<kRowHalfMirror>(x);
  return x;
}

// Value of the lane `OFF` token slots away (a rotation inside the 16-lane row
// for OFF < 16, an xor across rows otherwise).  Any pairing works for the
// all-reduce below as long as every step pairs distinct slots.
template <int OFF>
__device__ __forceinline__ float slot_partner(float x) {
  if constexpr (OFF == 4) return dpp_mov<kRowRor4>(x);
  else if constexpr (OFF == 8) return dpp_mov<kRowRor8>(x);
  else return __shfl_xor(x, OFF, kWave);
}

struct Round {
  uint4 k0, k1, v0, v1;
};

template <int D, int HG>
struct SplitWave {
  static constexpr int LPT = D / 16;
  static constexpr int TPR = kWave / LPT;

  float m[HG], l[HG], acc[HG][16];
  uint32_t qw[HG][8];

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      m[h] = kFloorMax;
      l[h] = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[h][j] = 0.f;
    }
  }

  // One round: TPR tokens, lane slot `tok`; `live` = this lane's token counts.
  __device__ __forceinline__ void consume(const Round& rd, bool live, float scale_log2) {
    float s[HG];
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      float d = 0.f;
      d = dot2_bf16(rd.k0.x, qw[h][0], d);
      d = dot2_bf16(rd.k0.y, qw[h][1], d);
      d = dot2_bf16(rd.k0.z, qw[h][2], d);
      d = dot2_bf16(rd.k0.w, qw[h][3], d);
      d = dot2_bf16(rd.k1.x, qw[h][4], d);
      d = dot2_bf16(rd.k1.y, qw[h][5], d);
      d = dot2_bf16(rd.k1.z, qw[h][6], d);
      d = dot2_bf16(rd.k1.w, qw[h][7], d);
      d = token_group_sum<LPT>(d);
      s[h] = live ? d * scale_log2 : kMinusInf;
    }
    // Slots past the sequence end (or in a skipped page) may hold anything,
    // NaN included: zero them so a zero weight really contributes zero.
    const uint32_t keep = live ? 0xffffffffu : 0u;
    uint4 v0 = rd.v0, v1 = rd.v1;
    v0.x &= keep; v0.y &= keep; v0.z &= keep; v0.w &= keep;
    v1.x &= keep; v1.y &= keep; v1.z &= keep; v1.w &= keep;
    bool grow = false;
#pragma unroll
    for (int h = 0; h < HG; ++h) grow |= s[h] > m[h] + kRescaleSlack;
    if (grow) {
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        const float mn = fmaxf(m[h], s[h]);
        const float alpha = fast_exp2(m[h] - mn);
        l[h] *= alpha;
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[h][j] *= alpha;
        m[h] = mn;
      }
    }
    float vf[16];
    vf[0] = bf16_lo(v0.x); vf[1] = bf16_hi(v0.x); vf[2] = bf16_lo(v0.y); vf[3] = bf16_hi(v0.y);
    vf[4] = bf16_lo(v0.z); vf[5] = bf16_hi(v0.z); vf[6] = bf16_lo(v0.w); vf[7] = bf16_hi(v0.w);
    vf[8] = bf16_lo(v1.x); vf[9] = bf16_hi(v1.x); vf[10] = bf16_lo(v1.y); vf[11] = bf16_hi(v1.y);
    vf[12] = bf16_lo(v1.z); vf[13] = bf16_hi(v1.z); vf[14] = bf16_lo(v1.w); vf[15] = bf16_hi(v1.w);
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      const float p = fast_exp2(s[h] - m[h]);
      l[h] += p;
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[h][j] = fmaf(p, vf[j], acc[h][j]);
    }
  }

  template <int OFF>
  __device__ __forceinline__ void merge_slot_step() {
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      const float mo = slot_partner<OFF>(m[h]);
      const float lo = slot_partner<OFF>(l[h]);
      const float mn = fmaxf(m[h], mo);
      const float ca = fast_exp2(m[h] - mn);
      const float cb = fast_exp2(mo - mn);
      l[h] = l[h] * ca + lo * cb;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float ao = slot_partner<OFF>(acc[h][j]);
        acc[h][j] = acc[h][j] * ca + ao * cb;
      }
      m[h] = mn;
    }
  }

  // All-reduce of the lane-local states over the TPR token slots of the wave.
  __device__ __forceinline__ void merge_slots() {
    if constexpr (LPT <= 4) merge_slot_step<4>();
    merge_slot_step<8>();
    merge_slot_step<16>();
    merge_slot_step<32>();
  }
};


// Online-softmax combine of (m, l, value) triples in the log2 domain.
struct Combine {
  float m = kFloorMax, den = 0.f, num = 0.f;
  __device__ __forceinline__ void add(float mk, float lk, float vk) {
    const float mn = fmaxf(m, mk);
    const float ca = fast_exp2(m - mn);
    const float cb = fast_exp2(mk - mn);
    den = den * ca + lk * cb;
    num = num * ca + vk * cb;
    m = mn;
  }
};

template <int D, int HG>
__global__ void __launch_bounds__(kGroupThreads) decode_kernel(DecodeArgs a) {
  using W = SplitWave<D, HG>;
  constexpr int LPT = W::LPT;
  constexpr int TPR = W::TPR;
  static_assert(HG * D <= kGroupThreads, "one output channel per thread");

  // Pieces that leave a wave unfinished: slot 0 = the wave's first piece,
  // slot 1 = its last piece (every other piece is a whole segment).
  __shared__ float s_acc[kWavesPerGroup][2][HG][D];
  __shared__ float s_m[kWavesPerGroup][2][HG];
  __shared__ float s_l[kWavesPerGroup][2][HG];
  __shared__ int s_seg[kWavesPerGroup][2];
  __shared__ int s_glob[2];   // segments this workgroup left as global partials
  __shared__ int s_merge[2];  // of those, the ones this workgroup merges

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int grp = blockIdx.x;
  const int U = a.units;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int Hq = a.num_q_heads;

  if (grp == 0) {
    // Requests without tokens get zero rows (no tile covers them).
    for (int b = tid; b < a.batch; b += kGroupThreads) {
      if (a.kv_indptr[b + 1] == a.kv_indptr[b]) {
        uint4* row = reinterpret_cast<uint4*>(a.out + (size_t)b * Hq * D);
        for (int i = 0; i < Hq * D / 8; ++i) row[i] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  if (grp >= a.hdr[kHdrGroups]) return;  // uniform over the workgroup
  if (lane == 0) {
    s_seg[w][0] = -1;
    s_seg[w][1] = -1;
  }
  if (tid < 2) s_glob[tid] = -1;

  const WaveRange rng = a.waves[grp * kWavesPerGroup + w];
  const int tok = lane / LPT;
  const int e = lane % LPT;
  const int c0 = e * 8;  // first channel of the lane's low half; high half at D/2 + c0
  const size_t tile = (size_t)a.page_size * D;               // elements per (page, head) tile
  const uint32_t lane_boff = (uint32_t)(tok * D + c0) * 2;  // lane's byte offset inside a round
  const char* kbase = reinterpret_cast<const char*>(a.k);
  const char* vbase = reinterpret_cast<const char*>(a.v);
  const int P = a.page_size;
  const int log2_r = a.log2_rounds;
  int err = 0;

  int b = rng.b, u = rng.u, p = rng.p, left = rng.count, piece = 0;
  W st;
  while (left > 0) {  // one piece = the part of segment (b, u) inside this wave's range
    const int ip0 = a.kv_indptr[b];
    const int n = a.kv_indptr[b + 1] - ip0;
    const int L = a.seq_lens[b];
    const int len = min(left, n - p);
    if (len <= 0) break;  // only reachable with metadata that does not match kv_indptr
    const int hq0 = u * HG;
    const int g = hq0 / G;

    st.init();
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      const uint4* qp = reinterpret_cast<const uint4*>(
          a.q + ((size_t)b * Hq + hq0 + h) * D + c0);
      const uint4 lo = qp[0];
      const uint4 hi = qp[D / 16];
      st.qw[h][0] = lo.x; st.qw[h][1] = lo.y; st.qw[h][2] = lo.z; st.qw[h][3] = lo.w;
      st.qw[h][4] = hi.x; st.qw[h][5] = hi.y; st.qw[h][6] = hi.z; st.qw[h][7] = hi.w;
    }
    const size_t head_off = (size_t)g * tile;

    for (int jb = 0; jb < len; jb += kWave) {
      const int nb = min(kWave, len - jb);
      // One vector load fetches the page ids of the next (up to) 64 pages: lane i
      // holds the id of page p + jb + i, or -1 if it is unusable.
      int vpage = -1;
      {
        const int pos = ip0 + p + jb + lane;
        const bool pos_ok = pos >= 0 && pos < a.num_indices;
        const int pid = a.kv_indices[pos_ok ? pos : 0];
        if (lane < nb) {
          if (!pos_ok) err |= kErrBadIndexPos;
          else if (pid < 0 || pid >= a.num_pages) err |= kErrBadPageId;
          else vpage = pid;
        }
      }
      const int nr = nb << log2_r;  // rounds in this block, >= 1

      // Round rr of the block: page id (uniform), first token, loads.  Rounds
      // past the block re-read its last round (a cache hit) and are never
      // consumed, so the issue sequence has no data-dependent branch.
      auto issue = [&](int rr, Round& rd) {
        const int rc = rr < nr ? rr : nr - 1;
        const int j = rc >> log2_r;
        const int r = rc & ((1 << log2_r) - 1);
        const int pid = __builtin_amdgcn_readlane(vpage, j);
        const size_t off = ((size_t)(pid < 0 ? 0 : pid) * a.num_kv_heads * tile + head_off +
                            (size_t)r * TPR * D) * 2;
        const char* kp = kbase + off + lane_boff;
        const char* vp = vbase + off + lane_boff;
        rd.k0 = *reinterpret_cast<const uint4*>(kp);
        rd.k1 = *reinterpret_cast<const uint4*>(kp + D);
        rd.v0 = *reinterpret_cast<const uint4*>(vp);
        rd.v1 = *reinterpret_cast<const uint4*>(vp + D);
      };
      auto consume = [&](int rr, const Round& rd) {
        const int j = rr >> log2_r;
        const int r = rr & ((1 << log2_r) - 1);
        const int pid = __builtin_amdgcn_readlane(vpage, j);
        const int t0 = (p + jb + j) * P + r * TPR;
        const bool live = pid >= 0 && t0 + tok < L;
        st.consume(rd, live, a.scale_log2);
      };

      // Two stages of two rounds each: while one stage is consumed the other
      // is in flight.
      Round A0, A1, B0, B1;
      issue(0, A0);
      issue(1, A1);
      for (int rr = 0; rr < nr; rr += 4) {
        issue(rr + 2, B0);
        issue(rr + 3, B1);
        consume(rr, A0);
        if (rr + 1 < nr) consume(rr + 1, A1);
        issue(rr + 4, A0);
        issue(rr + 5, A1);
        if (rr + 2 < nr) consume(rr + 2, B0);
        if (rr + 3 < nr) consume(rr + 3, B1);
      }
    }

    st.merge_slots();
    const int seg = b * U + u;
    if (p == 0 && len == n) {
      // The whole segment lies in this wave: write its rows.  Lane slot h < HG
      // writes head h (after the merge every slot holds the totals).
      float o[16];
      float lv = st.l[0];
#pragma unroll
      for (int j = 0; j < 16; ++j) o[j] = st.acc[0][j];
#pragma unroll
      for (int h = 1; h < HG; ++h) {
        if (tok == h) {
          lv = st.l[h];
#pragma unroll
          for (int j = 0; j < 16; ++j) o[j] = st.acc[h][j];
        }
      }
      if (tok < HG) {
        const float inv = lv > 0.f ? 1.0f / lv : 0.f;
        uint16_t* op = a.out + ((size_t)b * Hq + hq0 + tok) * D + c0;
        *reinterpret_cast<uint4*>(op) =
            make_uint4(pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                       pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv));
        *reinterpret_cast<uint4*>(op + D / 2) =
            make_uint4(pack_bf16x2(o[8] * inv, o[9] * inv), pack_bf16x2(o[10] * inv, o[11] * inv),
                       pack_bf16x2(o[12] * inv, o[13] * inv),
                       pack_bf16x2(o[14] * inv, o[15] * inv));
      }
    } else {
      const int slot = piece == 0 ? 0 : 1;
      if (tok == 0) {
#pragma unroll
        for (int h = 0; h < HG; ++h) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            s_acc[w][slot][h][c0 + j] = st.acc[h][j];
            s_acc[w][slot][h][D / 2 + c0 + j] = st.acc[h][8 + j];
          }
          if (e == 0) {
            s_m[w][slot][h] = st.m[h];
            s_l[w][slot][h] = st.l[h];
          }
        }
        if (e == 0) s_seg[w][slot] = seg;
      }
    }
    left -= len;
    ++piece;
    if (left > 0) {
      p = 0;
      if (++u == U) {
        u = 0;
        do { ++b; } while (b < a.batch - 1 && a.kv_indptr[b + 1] == a.kv_indptr[b]);
      }
    }
  }
  if (err) atomicOr(&a.hdr[kHdrError], err);
  __syncthreads();

  // Merge the pieces in LDS segment by segment (a segment's pieces are
  // consecutive in wave order).  Thread t owns channel t % D of head t / D.
  const int2 gsegs = a.group_segs[grp];
  const bool act = tid < HG * D;
  const int h = tid / D;
  const int c = tid - h * D;
  auto emit = [&](int sgm, const Combine& cb) {
    const int eb = sgm / U;
    const int hq = (sgm - eb * U) * HG + h;
    const int2 sg = a.seg_groups[sgm];
    const float val = cb.den > 0.f ? cb.num / cb.den : 0.f;
    if (sg.x == grp && sg.y == grp) {
      if (act) a.out[((size_t)eb * Hq + hq) * D + c] = (uint16_t)bf16_rne(val);
    } else {
      const int slot = sgm == gsegs.x ? 0 : 1;
      const size_t row = (size_t)(2 * grp + slot) * HG + h;
      if (act) {
        store_coherent(&a.opart[row * D + c], val);
        if (c == 0) store_coherent(&a.lse[row], cb.den > 0.f ? cb.m + fast_log2(cb.den) : kMinusInf);
      }
      if (tid == 0) s_glob[slot] = sgm;
    }
  };
  {
    int cur = -1;
    Combine cb;
#pragma unroll 1
    for (int k = 0; k < 2 * kWavesPerGroup; ++k) {
      const int sgm = s_seg[k >> 1][k & 1];
      if (sgm < 0) continue;
      if (sgm != cur) {
        if (cur >= 0) emit(cur, cb);
        cur = sgm;
        cb = Combine();
      }
      if (act) cb.add(s_m[k >> 1][k & 1][h], s_l[k >> 1][k & 1][h], s_acc[k >> 1][k & 1][h][c]);
    }
    if (cur >= 0) emit(cur, cb);
  }

  // Cross-workgroup merge: publish the partials, count arrivals, and let the
  // last workgroup of each segment combine every workgroup's partial in order.
  wait_stores();
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int sgm = s_glob[k];
      s_merge[k] = -1;
      if (sgm >= 0 && !(k == 1 && sgm == s_glob[0])) {
        const int2 sg = a.seg_groups[sgm];
        const int old = __hip_atomic_fetch_add(&a.counters[sgm], 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        if (old == sg.y - sg.x) s_merge[k] = sgm;
      }
    }
  }
  __syncthreads();
#pragma unroll 1
  for (int k = 0; k < 2; ++k) {
    const int sgm = s_merge[k];
    if (sgm < 0) continue;
    const int2 sg = a.seg_groups[sgm];
    Combine cb;
    for (int j = sg.x; j <= sg.y; ++j) {
      const int slot = a.group_segs[j].x == sgm ? 0 : 1;
      const size_t row = (size_t)(2 * j + slot) * HG + h;
      if (act) cb.add(load_coherent(&a.lse[row]), 1.0f, load_coherent(&a.opart[row * D + c]));
    }
    const int eb = sgm / U;
    const int hq = (sgm - eb * U) * HG + h;
    if (act) {
      const float val = cb.den > 0.f ? cb.num / cb.den : 0.f;
      a.out[((size_t)eb * Hq + hq) * D + c] = (uint16_t)bf16_rne(val);
    }
    if (tid == 0) __hip_atomic_store(&a.counters[sgm], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, int hg, int groups, hipStream_t s) {
  switch (hg) {
    case 1: hipLaunchKernelGGL((decode_kernel<D, 1>), dim3(groups), dim3(kGroupThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<D, 2>), dim3(groups), dim3(kGroupThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL((decode_kernel<D, 3>), dim3(groups), dim3(kGroupThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_kernel<D, 4>), dim3(groups), dim3(kGroupThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int head_dim, int hg, int groups, hipStream_t s) {
  if (groups <= 0) return hipSuccess;
  if (head_dim == 128) return launch_d<128>(a, hg, groups, s);
  if (head_dim == 64) return launch_d<64>(a, hg, groups, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv
