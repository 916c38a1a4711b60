// Paged prefill / extend attention for gfx950: ragged query rows per request
// attend to the request's paged KV (prefix + new tokens), causal or not.
//
// The pages' paged prefill takes query rows flattened over the batch with
// per-request offsets, per-request KV lengths and a causal flag with offset 0
// (AstrAI compare v1.3.12..6f09b1d, attention_ops.py, attn_paged_prefill); its
// grid is sized from the longest query length.  Here the grid is (query
// block, head group, request): every wave owns one block of 16 score rows --
// 16 / HG query tokens times the HG query heads of a head group that share one
// KV head -- and streams that KV head's pages up to the block's causal limit,
// with the decode kernel's matrix-core step (pkv_mfma.h).  Query row i of a
// request with n rows and L keys sees keys 0 .. L - n + i when causal (the
// mask aligned to the end of the KV, so n = 1 is decode).  Rows are
// independent: no partials, no merge, no workspace.
#include "pkv_mfma.h"

namespace pkv {
namespace {

template <int D, int HG>
__global__ void __launch_bounds__(kGroupThreads) prefill_kernel(PrefillArgs a) {
  constexpr int QT = 16 / HG;     // query tokens per wave block
  constexpr int ROWS = QT * HG;   // score rows in use (15 for HG = 3)
  constexpr int kStages = 2;      // register ring: steps in flight per wave
  __shared__ __align__(16) float s_out[kWavesPerGroup][16][D];  // per-wave transpose of rows

  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int b = blockIdx.z;
  const int u = blockIdx.y;
  const int tok0 = (blockIdx.x * kWavesPerGroup + w) * QT;  // first query token of the block
  const int q0 = a.qo_indptr[b];
  const int n = a.qo_indptr[b + 1] - q0;
  if (tok0 >= n) return;  // uniform per wave; the kernel has no workgroup barrier
  const int L = max(a.seq_lens[b], 0);
  const int ip0 = a.kv_indptr[b];
  const int Hq = a.num_q_heads;
  const int G = Hq / a.num_kv_heads;
  const int hq0 = u * HG;
  const int g = hq0 / G;  // KV head of the head group

  const int g4 = lane >> 4;
  const int r16 = lane & 15;
  // Row r16 = (token tok0 + r16 / HG, head r16 % HG).
  const int rt = tok0 + r16 / HG;
  const bool rvalid = r16 < ROWS && rt < n;
  const int lim = a.causal ? L - n + rt : L - 1;  // last key row r16 sees
  const float bias = rvalid ? 0.f : kMinusInf;
  const int last_tok = min(tok0 + QT, n) - 1;
  const int kv_end = a.causal ? max(0, min(L, L - n + last_tok + 1)) : L;  // keys the block reads

  MfmaWave<D, 16> st;
  st.init();
  {
    // q^T operand: lane (g4, r16) supplies row r16, channels 8*(4kk + g4) .. +8.
    const uint4* qp = reinterpret_cast<const uint4*>(
        a.q + ((size_t)(q0 + (rvalid ? rt : 0)) * Hq + hq0 + r16 % HG) * D + g4 * 8);
#pragma unroll
    for (int kk = 0; kk < MfmaWave<D, 16>::KB; ++kk) {
      const uint4 w4 = rvalid ? qp[4 * kk] : make_uint4(0, 0, 0, 0);
      st.qb[kk] = __builtin_bit_cast(bf16x8_t, w4);
    }
  }

  const int P = a.page_size;
  const int log2_s = a.log2_steps;
  const size_t tile_b = (size_t)P * D * 2;
  const size_t head_b = (size_t)g * tile_b;
  const uint32_t k_boff = (uint32_t)(g4 * P + r16) * 16;
  const uint32_t v_boff = (uint32_t)(r16 * P + 4 * g4) * 2;
  const char* kbase = reinterpret_cast<const char*>(a.k);
  const char* vbase = reinterpret_cast<const char*>(a.v);
  const int pages = (kv_end + P - 1) / P;

  for (int jb = 0; jb < pages; jb += kWave) {
    const int nb = min(kWave, pages - jb);
    // Page ids of the next (up to) 64 pages, one per lane; -1 if unusable.
    int vpage = -1;
    {
      const int pos = ip0 + jb + lane;
      const bool ok = lane < nb && pos >= 0 && pos < a.num_indices;
      const int pid = ok ? a.kv_indices[pos] : -1;
      if (pid >= 0 && pid < a.num_pages) vpage = pid;
    }
    const int ns = nb << log2_s;
    auto issue = [&](int j, Step<D>& sd) {
      const int jc = j < ns ? j : ns - 1;
      const int pg = jc >> log2_s;
      const int sub = jc & ((1 << log2_s) - 1);
      const int pid = __builtin_amdgcn_readlane(vpage, pg);
      const size_t base = (size_t)(pid < 0 ? 0 : pid) * a.num_kv_heads * tile_b + head_b;
      const char* kp = kbase + base + (size_t)sub * 16 * 16 + k_boff;
      const char* vp = vbase + base + (size_t)sub * 16 * 2 + v_boff;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        sd.k[kk] = *reinterpret_cast<const uint4*>(kp + (size_t)kk * 4 * P * 16);
#pragma unroll
      for (int vb = 0; vb < D / 16; ++vb)
        sd.v[vb] = *reinterpret_cast<const uint2*>(vp + (size_t)vb * 16 * P * 2);
    };
    auto consume = [&](int j, const Step<D>& sd) {
      const int pg = j >> log2_s;
      const int sub = j & ((1 << log2_s) - 1);
      const int pid = __builtin_amdgcn_readlane(vpage, pg);
      const int t0 = (jb + pg) * P + sub * 16;
      const int live = pid < 0 ? 0 : min(16, max(0, kv_end - t0));
      // Causal: key t0 + 4 g4 + i is visible to row r16 iff it is <= lim.
      const int k0 = t0 + 4 * g4;
      const uint32_t keep = (k0 + 0 <= lim ? 0x1u : 0u) | (k0 + 1 <= lim ? 0x100u : 0u) |
                            (k0 + 2 <= lim ? 0x10000u : 0u) | (k0 + 3 <= lim ? 0x1000000u : 0u);
      st.step(sd, live, g4, a.scale_log2, bias, keep);
    };
    Step<D> ring[kStages];
#pragma unroll
    for (int i = 0; i < kStages - 1; ++i) issue(i, ring[i]);
    for (int j = 0; j < ns; j += kStages) {
#pragma unroll
      for (int i = 0; i < kStages; ++i) {
        issue(j + i + kStages - 1, ring[(i + kStages - 1) % kStages]);
        if (j + i < ns) consume(j + i, ring[i]);
      }
    }
  }

  // Normalise: the four lanes of row r hold its partial sums; register i of
  // lane group g holds row 4g + i.  Rows go through LDS so that every lane
  // writes 8 channels (16 bytes) of one row.
  float lt = st.l + __shfl_xor(st.l, 16, kWave);
  lt += __shfl_xor(lt, 32, kWave);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float li = __shfl(lt, 4 * g4 + i, kWave);
    const float inv = li > 0.f ? 1.0f / li : 0.f;
#pragma unroll
    for (int vb = 0; vb < MfmaWave<D, 16>::VB; ++vb)
      s_out[w][4 * g4 + i][16 * vb + r16] = st.o[vb][i] * inv;
  }
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's LDS writes land first
  constexpr int kChunks = ROWS * (D / 8);
#pragma unroll
  for (int c = lane; c < kChunks; c += kWave) {
    const int rr = c / (D / 8);
    const int c8 = (c - rr * (D / 8)) * 8;
    const int tok = tok0 + rr / HG;
    if (tok < n) {
      const float4 x0 = *reinterpret_cast<const float4*>(&s_out[w][rr][c8]);
      const float4 x1 = *reinterpret_cast<const float4*>(&s_out[w][rr][c8 + 4]);
      *reinterpret_cast<uint4*>(a.out + ((size_t)(q0 + tok) * Hq + hq0 + rr % HG) * D + c8) =
          make_uint4(pack_bf16x2(x0.x, x0.y), pack_bf16x2(x0.z, x0.w), pack_bf16x2(x1.x, x1.y),
                     pack_bf16x2(x1.z, x1.w));
    }
  }
}

template <int D>
hipError_t launch_p(const PrefillArgs& a, int hg, dim3 grid, hipStream_t s) {
  const dim3 block(kGroupThreads);
  switch (hg) {
    case 1: hipLaunchKernelGGL((prefill_kernel<D, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<D, 2>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((prefill_kernel<D, 3>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<D, 4>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int hg, int max_q_len,
                          hipStream_t s) {
  const int qt = 16 / hg;
  const int per_group = qt * kWavesPerGroup;  // query tokens one workgroup covers
  const dim3 grid((max_q_len + per_group - 1) / per_group, a.num_q_heads / hg, a.batch);
  if (grid.x == 0 || grid.z == 0) return hipSuccess;
  if (head_dim == 128) return launch_p<128>(a, hg, grid, s);
  if (head_dim == 64) return launch_p<64>(a, hg, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv
