// Split-KV paged decode attention for gfx950 (MI355X): split kernel + merge kernel.
//
// Work decomposition.  The step's plan lists (request, chunk) items; every item
// is expanded into Hq / HG workgroups, one per group of HG query heads sharing
// a KV head (HG = G for G <= 4).  A workgroup has four waves.  Wave w of a
// workgroup walks pages p0 + w, p0 + w + 4, ... of the chunk, so the four waves
// stream four different pages at a time, then combine their online-softmax
// states through LDS and write one partial (or, for a one-chunk request, the
// final bf16 row).  The split partials and a separate combine kernel follow the
// pages' decode design (commits by ViperEkura: o_part / ml_part partials, one
// combine kernel); staging is different: K and V go straight from HBM into
// registers with 16-byte loads, since every K/V element is used by exactly one
// lane and LDS staging would only add traffic.
//
// Lane layout inside a wave (head_dim D, LPT = D / 16 lanes per token,
// TPR = 64 / LPT tokens per round).  Lane l serves token slot l / LPT of a round
// and holds 16 of the token's D channels: channels [8e, 8e + 8) and
// [D/2 + 8e, D/2 + 8e + 8) with e = l % LPT.  Each half is one 16-byte load, so
// one load instruction of the wave reads TPR half-rows of 128 (D=128) or 64
// (D=64) contiguous bytes.  q.K partial dot products use v_dot2 on bf16 pairs,
// then DPP adds inside the LPT-lane group.  Every lane keeps its own online
// softmax state (running max m, sum l, 16-channel accumulators per head) for
// the tokens of its slot; slots are merged once, at the end of the chunk.
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

constexpr int kWavesPerGroup = 4;
constexpr int kGroupThreads = kWavesPerGroup * kWave;
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

template <int D, int HG, int RS>
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
  __device__ __forceinline__ void consume(const Round& rd, bool live, bool any_dead,
                                          float scale_log2) {
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
    uint4 v0 = rd.v0, v1 = rd.v1;
    if (any_dead) {
      // Slots past the sequence end (or in a skipped page) may hold anything,
      // NaN included: zero them so a zero weight really contributes zero.
      if (!live) {
        v0 = make_uint4(0, 0, 0, 0);
        v1 = make_uint4(0, 0, 0, 0);
      }
    }
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

template <int D, int HG>
__global__ void __launch_bounds__(kGroupThreads) split_kernel(DecodeArgs a) {
  constexpr int RS = 2;  // rounds per pipeline stage
  using W = SplitWave<D, HG, RS>;
  constexpr int LPT = W::LPT;
  constexpr int TPR = W::TPR;

  __shared__ float s_acc[kWavesPerGroup][HG][D];
  __shared__ float s_m[kWavesPerGroup][HG];
  __shared__ float s_l[kWavesPerGroup][HG];

  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int units = a.num_q_heads / HG;
  const int item = blockIdx.x / units;
  if (item >= a.hdr[kHdrNumItems]) return;  // uniform over the workgroup
  const int hq0 = (blockIdx.x - item * units) * HG;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int g = hq0 / G;
  const int2 bs = a.items[item];
  const int b = bs.x, s = bs.y;
  const int ns = a.split_indptr[b + 1] - a.split_indptr[b];
  const int ip0 = a.kv_indptr[b];
  const int npages = a.kv_indptr[b + 1] - ip0;
  const int L = a.seq_lens[b];
  const int P = a.page_size;
  const int p0 = (int)(((long long)s * npages) / ns);
  const int p1 = (int)(((long long)(s + 1) * npages) / ns);
  const int log2_r = a.log2_rounds;  // rounds per page = P / TPR, a power of two
  const int tok = lane / LPT;
  const int e = lane % LPT;
  const int c0 = e * 8;  // first channel of the lane's low half; high half at D/2 + c0

  W st;
  st.init();
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    const uint4* qp = reinterpret_cast<const uint4*>(
        a.q + ((size_t)b * a.num_q_heads + hq0 + h) * D + c0);
    const uint4 lo = qp[0];
    const uint4 hi = qp[D / 16];
    st.qw[h][0] = lo.x; st.qw[h][1] = lo.y; st.qw[h][2] = lo.z; st.qw[h][3] = lo.w;
    st.qw[h][4] = hi.x; st.qw[h][5] = hi.y; st.qw[h][6] = hi.z; st.qw[h][7] = hi.w;
  }

  // This wave's pages: p0 + w, p0 + w + 4, ...
  const int mine = p1 - p0 > w ? (p1 - p0 - w + kWavesPerGroup - 1) / kWavesPerGroup : 0;
  const int nrounds = mine << log2_r;
  const size_t head_stride = (size_t)P * D;  // elements per (page, head) tile
  const int lane_off = tok * D + c0;         // element offset of the lane inside a round

  int err = 0;
  // Issue the loads of round rr.  Returns the round's first token (request
  // coordinates) and whether its page is usable.
  auto issue = [&](int rr, Round& rd, int& t0, bool& ok) {
    const int j = rr >> log2_r;
    const int r = rr & ((1 << log2_r) - 1);
    const int lp = p0 + w + j * kWavesPerGroup;  // logical page
    t0 = lp * P + r * TPR;
    ok = false;
    rd.k0 = rd.k1 = rd.v0 = rd.v1 = make_uint4(0, 0, 0, 0);
    if (t0 >= L) return;
    const int pos = ip0 + lp;
    if (pos < 0 || pos >= a.num_indices) {
      err |= kErrBadIndexPos;
      return;
    }
    const int page = a.kv_indices[pos];
    if (page < 0 || page >= a.num_pages) {
      err |= kErrBadPageId;
      return;
    }
    ok = true;
    const size_t base = ((size_t)page * a.num_kv_heads + g) * head_stride + (size_t)r * TPR * D;
    const uint4* kp = reinterpret_cast<const uint4*>(a.k + base + lane_off);
    const uint4* vp = reinterpret_cast<const uint4*>(a.v + base + lane_off);
    rd.k0 = kp[0];
    rd.k1 = kp[D / 16];
    rd.v0 = vp[0];
    rd.v1 = vp[D / 16];
  };
  auto consume = [&](const Round& rd, int t0, bool ok) {
    const bool live = ok && (t0 + tok < L);
    const bool any_dead = !ok || (t0 + TPR > L);
    st.consume(rd, live, any_dead, a.scale_log2);
  };

  // Two-stage software pipeline of RS rounds per stage.
  Round A[RS], B[RS];
  int tA[RS], tB[RS];
  bool okA[RS], okB[RS];
  const int nstages = (nrounds + RS - 1) / RS;
  if (nstages > 0) {
#pragma unroll
    for (int i = 0; i < RS; ++i) {
      if (i < nrounds) issue(i, A[i], tA[i], okA[i]);
      else { okA[i] = false; tA[i] = L; }
    }
  }
  for (int sg = 0; sg < nstages; sg += 2) {
    if (sg + 1 < nstages) {
#pragma unroll
      for (int i = 0; i < RS; ++i) {
        const int rr = (sg + 1) * RS + i;
        if (rr < nrounds) issue(rr, B[i], tB[i], okB[i]);
        else { okB[i] = false; tB[i] = L; }
      }
    }
#pragma unroll
    for (int i = 0; i < RS; ++i)
      if (tA[i] < L) consume(A[i], tA[i], okA[i]);
    if (sg + 2 < nstages) {
#pragma unroll
      for (int i = 0; i < RS; ++i) {
        const int rr = (sg + 2) * RS + i;
        if (rr < nrounds) issue(rr, A[i], tA[i], okA[i]);
        else { okA[i] = false; tA[i] = L; }
      }
    }
    if (sg + 1 < nstages) {
#pragma unroll
      for (int i = 0; i < RS; ++i)
        if (tB[i] < L) consume(B[i], tB[i], okB[i]);
    }
  }
  if (err) atomicOr(&a.hdr[kHdrError], err);

  st.merge_slots();

  // Hand the wave's state to LDS: slot 0 lanes hold channels [8e, 8e+8) and
  // [D/2 + 8e, D/2 + 8e + 8) of every head.
  if (tok == 0) {
#pragma unroll
    for (int h = 0; h < HG; ++h) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        s_acc[w][h][c0 + j] = st.acc[h][j];
        s_acc[w][h][D / 2 + c0 + j] = st.acc[h][8 + j];
      }
      if (e == 0) {
        s_m[w][h] = st.m[h];
        s_l[w][h] = st.l[h];
      }
    }
  }
  __syncthreads();

  // Combine the four waves and write: two channels per thread.
  const bool direct = ns == 1;
  for (int idx = threadIdx.x * 2; idx < HG * D; idx += kGroupThreads * 2) {
    const int h = idx / D;
    const int c = idx - h * D;
    float M = s_m[0][h];
#pragma unroll
    for (int v = 1; v < kWavesPerGroup; ++v) M = fmaxf(M, s_m[v][h]);
    float den = 0.f, n0 = 0.f, n1 = 0.f;
#pragma unroll
    for (int v = 0; v < kWavesPerGroup; ++v) {
      const float wt = fast_exp2(s_m[v][h] - M);
      den = fmaf(wt, s_l[v][h], den);
      n0 = fmaf(wt, s_acc[v][h][c], n0);
      n1 = fmaf(wt, s_acc[v][h][c + 1], n1);
    }
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    const int hq = hq0 + h;
    if (direct) {
      uint32_t* op = reinterpret_cast<uint32_t*>(a.out + ((size_t)b * a.num_q_heads + hq) * D + c);
      *op = pack_bf16x2(n0 * inv, n1 * inv);
    } else {
      float2* op = reinterpret_cast<float2*>(a.opart + ((size_t)item * a.num_q_heads + hq) * D + c);
      *op = make_float2(n0 * inv, n1 * inv);
      if (c == 0) a.lse[(size_t)item * a.num_q_heads + hq] = den > 0.f ? M + fast_log2(den) : kMinusInf;
    }
  }
}

// Merge: one workgroup per (request, query head).  Waves take every fourth
// chunk, each thread two channels (D = 128) or one (D = 64); the four waves'
// sums are combined through LDS.
template <int D>
__global__ void __launch_bounds__(kGroupThreads) merge_kernel(DecodeArgs a) {
  constexpr int CPT = D / kWave;  // channels per thread
  __shared__ float s_num[kWavesPerGroup][D];
  __shared__ float s_den[kWavesPerGroup];
  __shared__ float s_max[kWavesPerGroup];

  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int b = blockIdx.x / a.num_q_heads;
  const int hq = blockIdx.x - b * a.num_q_heads;
  if (b >= a.batch) return;
  const int base = a.split_indptr[b];
  int ns = a.split_indptr[b + 1] - base;
  if (ns == 1) return;  // written by the split kernel
  const int nitems = min(a.hdr[kHdrNumItems], a.max_items);
  if (base + ns > nitems) ns = nitems > base ? nitems - base : 0;

  const size_t hstride = (size_t)a.num_q_heads;
  float M = kMinusInf;
  for (int sp = threadIdx.x; sp < ns; sp += kGroupThreads)
    M = fmaxf(M, a.lse[(base + sp) * hstride + hq]);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, kWave));
  if (lane == 0) s_max[w] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));

  float num[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) num[i] = 0.f;
  float den = 0.f;
  if (M > kMinusInf) {
#pragma unroll 4
    for (int sp = w; sp < ns; sp += kWavesPerGroup) {
      const size_t row = (base + sp) * hstride + hq;
      const float wt = fast_exp2(a.lse[row] - M);
      den += wt;
      const float* op = a.opart + row * D + lane * CPT;
      if constexpr (CPT == 2) {
        const float2 o = *reinterpret_cast<const float2*>(op);
        num[0] = fmaf(wt, o.x, num[0]);
        num[1] = fmaf(wt, o.y, num[1]);
      } else {
        num[0] = fmaf(wt, op[0], num[0]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) s_num[w][lane * CPT + i] = num[i];
  if (lane == 0) s_den[w] = den;
  __syncthreads();
  if (w == 0) {
    const float dt = s_den[0] + s_den[1] + s_den[2] + s_den[3];
    const float inv = dt > 0.f ? 1.0f / dt : 0.f;
    float r[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = lane * CPT + i;
      r[i] = (s_num[0][c] + s_num[1][c] + s_num[2][c] + s_num[3][c]) * inv;
    }
    uint16_t* op = a.out + ((size_t)b * a.num_q_heads + hq) * D + lane * CPT;
    if constexpr (CPT == 2) {
      *reinterpret_cast<uint32_t*>(op) = pack_bf16x2(r[0], r[1]);
    } else {
      *op = (uint16_t)bf16_rne(r[0]);
    }
  }
}

template <int D>
hipError_t launch_split_d(const DecodeArgs& a, int hg, int grid, hipStream_t s) {
  switch (hg) {
    case 1: hipLaunchKernelGGL((split_kernel<D, 1>), dim3(grid), dim3(kGroupThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((split_kernel<D, 2>), dim3(grid), dim3(kGroupThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL((split_kernel<D, 3>), dim3(grid), dim3(kGroupThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((split_kernel<D, 4>), dim3(grid), dim3(kGroupThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_split(const DecodeArgs& a, int head_dim, int hg, int max_items, hipStream_t s) {
  const long long grid = (long long)max_items * (a.num_q_heads / hg);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (head_dim == 128) return launch_split_d<128>(a, hg, (int)grid, s);
  if (head_dim == 64) return launch_split_d<64>(a, hg, (int)grid, s);
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const DecodeArgs& a, int head_dim, hipStream_t s) {
  const long long grid = (long long)a.batch * a.num_q_heads;
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)grid), dim3(kGroupThreads), 0, s, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)grid), dim3(kGroupThreads), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
