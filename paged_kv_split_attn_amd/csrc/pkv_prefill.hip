// Paged prefill / extend attention for gfx950: ragged query rows per request
// attend to the request's paged KV (prefix + new tokens), causal or not.
// The eight waves of a workgroup share one KV head: each 64-token chunk of its
// K and V is fetched once into LDS (double buffered) and read by all of them.
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
  constexpr int kCh = 4;          // 16-token steps per LDS chunk
  constexpr int kPieces = D * 16 * 2 / 16;  // 16-byte pieces of one step's K (same for V)
  static_assert(2 * kPieces * kCh % kGroupThreads == 0 && kPieces % kWave == 0,
                "whole, wave-uniform loads per thread");
  constexpr int kLoads = 2 * kPieces * kCh / kGroupThreads;  // per thread and chunk
  // Two chunks (double buffer) of K as [step][D/8][16][8] and V as
  // [step][D][16] (the layouts of a 16-token tile); after the last chunk the
  // same bytes hold the per-wave output rows [wave][16][D] in fp32.
  constexpr int kKBytes = kCh * D * 16 * 2;
  constexpr int kBufBytes = 2 * kKBytes;  // K + V of one chunk
  constexpr int kOutBytes = kWavesPerGroup * 16 * D * 4;
  __shared__ __align__(16) char smem[2 * kBufBytes > kOutBytes ? 2 * kBufBytes : kOutBytes];
  auto k_at = [&](int buf, int st, int cb, int t) {  // 16 bytes: K channels 8cb.. of token t
    return smem + buf * kBufBytes + ((st * (D / 8) + cb) * 16 + t) * 16;
  };
  auto v_at = [&](int buf, int st, int ch, int t) {  // V channel ch from token t on
    return smem + buf * kBufBytes + kKBytes + ((st * D + ch) * 16 + t) * 2;
  };
  float* s_out = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int b = blockIdx.z;
  const int u = blockIdx.y;
  const int wg_tok0 = blockIdx.x * kWavesPerGroup * QT;  // first query token of the workgroup
  const int tok0 = wg_tok0 + w * QT;                      // first query token of this wave
  const int q0 = a.qo_indptr[b];
  const int n = a.qo_indptr[b + 1] - q0;
  if (wg_tok0 >= n) return;  // uniform over the workgroup
  const int L = max(a.seq_lens[b], 0);
  const int ip0 = a.kv_indptr[b];
  const int Hq = a.num_q_heads;
  const int G = Hq / a.num_kv_heads;
  const int hq0 = u * HG;
  const int g = hq0 / G;  // KV head of the head group
  const bool active = tok0 < n;  // this wave has query rows

  const int g4 = lane >> 4;
  const int r16 = lane & 15;
  // Row r16 = (token tok0 + r16 / HG, head r16 % HG).
  const int rt = tok0 + r16 / HG;
  const bool rvalid = r16 < ROWS && rt < n;
  const int lim = a.causal ? L - n + rt : L - 1;  // last key row r16 sees
  const float bias = rvalid ? 0.f : kMinusInf;
  // Keys this wave reads, and keys the workgroup reads (its last wave's limit).
  auto block_end = [&](int t0) {
    const int last = min(t0 + QT, n) - 1;
    return a.causal ? max(0, min(L, L - n + last + 1)) : L;
  };
  const int kv_end = active ? block_end(tok0) : 0;
  const int wg_end = block_end(min(wg_tok0 + (kWavesPerGroup - 1) * QT, n - 1));

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
  const char* kbase = reinterpret_cast<const char*>(a.k);
  const char* vbase = reinterpret_cast<const char*>(a.v);
  const int steps = (wg_end + 15) / 16;
  const int chunks = (steps + kCh - 1) / kCh;

  // Page of a step, -1 for an index outside kv_indices or the pool (its
  // tokens are skipped).  Wave-uniform.
  auto page_of = [&](int step) {
    const int pos = ip0 + (step >> log2_s);
    int pid = pos >= 0 && pos < a.num_indices ? a.kv_indices[pos] : -1;
    if (pid >= a.num_pages) pid = -1;
    return __builtin_amdgcn_readfirstlane(pid);
  };
  // Global -> registers: the workgroup's threads fetch 16-byte pieces
  // tid, tid + 512, ... of a chunk, step by step, K pieces before V pieces.
  // Piece y of a step's K is (channel block y / 16, token y % 16); piece y of
  // its V is (channel y / 2, tokens 8 (y % 2) .. +7).  A wave's 64 pieces lie in
  // one step and one operand, so page lookup and K/V choice are wave-uniform.
  uint4 stage[kLoads];
  auto piece = [&](int i, int& st, int& y, bool& is_v) {
    const int xw = w * kWave + i * kGroupThreads;  // the wave's first piece
    st = xw / (2 * kPieces);
    const int yw = xw - st * 2 * kPieces;
    is_v = yw >= kPieces;
    y = yw - (is_v ? kPieces : 0) + lane;
  };
  auto fetch = [&](int c) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      int st, y;
      bool is_v;
      piece(i, st, y, is_v);
      const int step = c * kCh + st;
      const int pid = step < steps ? page_of(step) : -1;
      if (pid < 0) {
        stage[i] = make_uint4(0, 0, 0, 0);
        continue;
      }
      const int sub = step & ((1 << log2_s) - 1);
      const char* tile = (is_v ? vbase : kbase) + (size_t)pid * a.num_kv_heads * tile_b + head_b;
      const int off = is_v ? ((y >> 1) * P + sub * 16 + 8 * (y & 1)) * 2
                           : ((y >> 4) * P + sub * 16 + (y & 15)) * 16;
      stage[i] = *reinterpret_cast<const uint4*>(tile + off);
    }
  };
  auto publish = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      int st, y;
      bool is_v;
      piece(i, st, y, is_v);
      char* dst = is_v ? v_at(buf, st, y >> 1, 8 * (y & 1)) : k_at(buf, st, y >> 4, y & 15);
      *reinterpret_cast<uint4*>(dst) = stage[i];
    }
  };

  if (chunks > 0) {
    fetch(0);
    publish(0);
  }
  __syncthreads();
  for (int c = 0; c < chunks; ++c) {
    const int buf = c & 1;
    if (c + 1 < chunks) fetch(c + 1);  // in flight while this chunk is consumed
#pragma unroll
    for (int s = 0; s < kCh; ++s) {
      const int t0 = (c * kCh + s) * 16;
      if (t0 < kv_end) {  // uniform per wave
        Step<D> sd;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
          sd.k[kk] = *reinterpret_cast<const uint4*>(k_at(buf, s, 4 * kk + g4, r16));
#pragma unroll
        for (int vb = 0; vb < D / 16; ++vb)
          sd.v[vb] = *reinterpret_cast<const uint2*>(v_at(buf, s, 16 * vb + r16, 4 * g4));
        const int live = page_of(c * kCh + s) < 0 ? 0 : min(16, kv_end - t0);
        const int k0 = t0 + 4 * g4;
        const uint32_t keep = (k0 + 0 <= lim ? 0x1u : 0u) | (k0 + 1 <= lim ? 0x100u : 0u) |
                              (k0 + 2 <= lim ? 0x10000u : 0u) | (k0 + 3 <= lim ? 0x1000000u : 0u);
        st.step(sd, live, g4, a.scale_log2, bias, keep);
      }
    }
    // The other buffer held chunk c - 1, which every wave finished before the
    // barrier that closed the previous iteration.
    if (c + 1 < chunks) publish(buf ^ 1);
    __syncthreads();
  }
  // Every wave has passed the barrier after the last chunk: the K/V buffers
  // are free for the output rows.
  if (!active) return;

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
      s_out[(w * 16 + 4 * g4 + i) * D + 16 * vb + r16] = st.o[vb][i] * inv;
  }
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's LDS writes land first
  constexpr int kChunks = ROWS * (D / 8);
#pragma unroll
  for (int c = lane; c < kChunks; c += kWave) {
    const int rr = c / (D / 8);
    const int c8 = (c - rr * (D / 8)) * 8;
    const int tok = tok0 + rr / HG;
    if (tok < n) {
      const float4 x0 = *reinterpret_cast<const float4*>(&s_out[(w * 16 + rr) * D + c8]);
      const float4 x1 = *reinterpret_cast<const float4*>(&s_out[(w * 16 + rr) * D + c8 + 4]);
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
