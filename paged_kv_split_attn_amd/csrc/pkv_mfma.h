// Matrix-core attention step shared by the decode and prefill kernels: the
// operand layouts of one 16-token step of a (page, KV head) tile and the
// online-softmax state of one wave over up to 16 score rows.
//
// Scores S^T[token][row] = K . Q^T come from D/32 v_mfma_f32_16x16x32_bf16 (K
// rows are the A operand, the query rows the B operand).  The result leaves
// lane (g, r) = (l / 16, l % 16) holding row r's scores for tokens 4g .. 4g+3,
// which is the A-operand layout of v_mfma_f32_16x16x16_bf16 for P . V, so the
// softmax weights never move between lanes; V^T is the B operand (4 tokens
// of one channel per lane, one 8-byte load).  The weights enter as bf16 hi +
// lo parts (two MFMAs).  Output: lane (g, r) register i of block nb holds
// O[row 4g+i][channel 16 nb + r].
#pragma once

#include <math.h>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr float kRescaleSlack = 8.0f;  // log2 of the largest un-rescaled weight
constexpr float kMinusInf = -INFINITY;
constexpr float kFloorMax = -1.0e30f;  // initial running max (finite: exp2 never sees inf - inf)

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

// Cross-row exchange with the gfx950 row-swap permutes (VALU, no LDS round
// trip): every lane of a pair (l, l ^ 16) or (l, l ^ 32) receives both values,
// the lower lane's first, so a reduction over the pair gives the same bits in
// both lanes.  Called with the whole wave active.
struct LanePair {
  float lo, hi;
};
__device__ __forceinline__ LanePair pair16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ LanePair pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// Maxima of score values without the compiler's NaN quieting (fmaxf makes it
// canonicalise every input first, which doubles the instruction count of a
// max tree).  A NaN score can only come from NaN q or K data: masked keys are
// set to -inf before any max, so garbage past the sequence end never gets here,
// and the merges combine maxima that are finite or -inf.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  __asm__("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmax2(float a, float b) {
  float r;
  __asm__("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// Max over the four lanes l % 16 + 16 k (the four lane groups).
__device__ __forceinline__ float max_over_groups(float x) {
  const LanePair a = pair16(x);
  const LanePair b = pair32(vmax2(a.lo, a.hi));
  return vmax2(b.lo, b.hi);
}

// Sum over the four lanes l % 16 + 16 k (the four lane groups).
__device__ __forceinline__ float sum_over_groups(float x) {
  const LanePair a = pair16(x);
  const LanePair b = pair32(a.lo + a.hi);
  return b.lo + b.hi;
}

// MFMA operand vectors.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// One step's operands: 16 tokens of one (page, head) tile.
template <int D>
struct Step {
  uint4 k[D / 32];  // K of token r, channels 8*(4kk + g) .. +8 (A of q.K, block kk)
  uint2 v[D / 16];  // V^T: channel 16*nb + r, tokens 4g .. 4g+3 (B of p.V)
  uint32_t keep;    // masked decode: keep bytes of tokens 4g .. 4g+3
};

// ROWS = score rows in use (heads of a head group in decode, query rows in
// prefill); rows >= ROWS carry bias -inf.
template <int D, int ROWS>
struct MfmaWave {
  static constexpr int KB = D / 32;  // q.K MFMAs per step
  static constexpr int VB = D / 16;  // p.V channel blocks
  floatx4_t o[VB];                   // O[row 4g+i][channel 16*nb + r]
  bf16x8_t qb[KB];                   // q^T operand (zero for rows >= ROWS)
  float m, l;                        // row r: running max (log2 domain), partial sum

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int nb = 0; nb < VB; ++nb) o[nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    m = kFloorMax;
    l = 0.f;
  }

  // Consume one step.  `live` = tokens of the step that count (uniform, 0..16);
  // `g` = lane / 16; `bias` = 0 for rows < ROWS, -inf otherwise.
  template <class S>
  __device__ __forceinline__ void step(const S& st, int live, int g, float scale_log2,
                                       float bias, uint32_t keep = 0x01010101u) {
    floatx4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KB; ++kk)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, st.k[kk]),
                                                   qb[kk], sc, 0, 0, 0);
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = fmaf(sc[i], scale_log2, bias);
    uint2 vv[VB];
#pragma unroll
    for (int nb = 0; nb < VB; ++nb) vv[nb] = st.v[nb];
    if (live < 16) {
      // Tokens past the sequence end (or in a skipped page) may hold anything,
      // NaN included: drop their scores and zero their V so that a zero weight
      // contributes exactly zero.
      const int t = 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (t + i >= live) s[i] = kMinusInf;
      const uint32_t m0 = (t + 0 < live ? 0x0000ffffu : 0u) | (t + 1 < live ? 0xffff0000u : 0u);
      const uint32_t m1 = (t + 2 < live ? 0x0000ffffu : 0u) | (t + 3 < live ? 0xffff0000u : 0u);
#pragma unroll
      for (int nb = 0; nb < VB; ++nb) {
        vv[nb].x &= m0;
        vv[nb].y &= m1;
      }
    }
    // Keep mask: byte i of `keep` is zero for a dropped token 4g + i (its V is
    // real data, so a zero weight suffices).
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (((keep >> (8 * i)) & 0xffu) == 0) s[i] = kMinusInf;
    // Step max of row r over its 16 tokens (4 per lane, 4 lanes).
    const float pm = max_over_groups(vmax3(s[0], s[1], vmax2(s[2], s[3])));
    if (__builtin_amdgcn_ballot_w64(pm > m + kRescaleSlack) != 0) {
      const float mn = fmaxf(m, pm);
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
      m = mn;
      if constexpr (ROWS <= 4) {
        // Rows live in lane group 0: lane i holds row i's factor, register i its O.
#pragma unroll
        for (int i = 0; i < ROWS; ++i) {
          const float ai = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), i));
#pragma unroll
          for (int nb = 0; nb < VB; ++nb) o[nb][i] *= ai;
        }
      } else {
        // Register i of lane group g holds row 4g + i, whose factor lane 4g + i has.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ai = __shfl(alpha, 4 * g + i, kWave);
#pragma unroll
          for (int nb = 0; nb < VB; ++nb) o[nb][i] *= ai;
        }
      }
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(s[i] - m);
    l += (p[0] + p[1]) + (p[2] + p[3]);
    // p = hi + lo, both bf16: the product keeps ~16 mantissa bits of p.
    short4_t phi, plo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 h = (__bf16)p[i];
      const float hf = (float)h;
      const __bf16 lo = (__bf16)(p[i] - hf);
      phi[i] = __builtin_bit_cast(short, h);
      plo[i] = __builtin_bit_cast(short, lo);
    }
#pragma unroll
    for (int nb = 0; nb < VB; ++nb) {
      const short4_t vb = __builtin_bit_cast(short4_t, vv[nb]);
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, vb, o[nb], 0, 0, 0);
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, vb, o[nb], 0, 0, 0);
    }
  }
};

}  // namespace
}  // namespace pkv
