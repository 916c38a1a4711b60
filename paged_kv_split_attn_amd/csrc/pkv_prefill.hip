// Paged prefill / extend attention for gfx950: ragged query rows per request
// attend to the request's paged KV (prefix + new tokens), causal or not.
// The waves of a workgroup share one KV head: each chunk of its K and V (32
// keys) is fetched once into LDS (double buffered) and read by all of them.
//
// The pages' paged prefill takes query rows flattened over the batch with
// per-request offsets, per-request KV lengths and a causal flag with offset 0
// (AstrAI compare v1.3.12..6f09b1d, attention_ops.py, attn_paged_prefill); its
// grid is sized from the longest query length.  Here the grid is (query
// block, head group, request): every wave owns one block of 16 score rows --
// 16 / HG query tokens times the HG query heads of a head group that share one
// KV head -- and streams that KV head's pages up to the block's causal limit,
// 32 keys per matrix-core step.  Query row i of a
// request with n rows and L keys sees keys 0 .. L - n + i when causal (the
// mask aligned to the end of the KV, so n = 1 is decode).  Rows are
// independent: no partials, no merge, no workspace.
#include "pkv_mfma.h"

namespace pkv {
namespace {

// Bits 4h + j (h, j < 2, 4) of the keys 16h + j <= d of a lane group's eight.
__device__ __forceinline__ uint32_t keys_upto(int d) {
  auto four = [](int x) { return x < 0 ? 0u : x >= 3 ? 15u : (2u << x) - 1u; };
  return four(d) | (four(d - 16) << 4);
}

// One wave's online softmax over NT tiles of 16 score rows, 32 keys per step;
// the tiles share every K and V operand the wave reads.  Scores of the
// step's two 16-key halves come from v_mfma_f32_16x16x32_bf16 as in the decode
// step (K rows the A operand, q^T the B operand), leaving lane (g, r) row r's
// scores of keys 4g .. 4g+3 of each half.  P . V then takes one
// v_mfma_f32_16x16x32_bf16 per tile, 16 channels and part of P, whose
// reduction index runs over the eight keys lane group g holds (4g .. 4g+3 of
// half 0, then of half 1): the weights never move between lanes, and the
// double-rate instruction does twice the work of the 16-key one in the same
// time.  P enters rounded to bf16 (a weight is at most 2^8: a row is rescaled
// once a score passes its running max by kRescaleSlack in the log2 domain;
// splitting P into bf16 high and low parts cost a third more matrix-core
// time), and the row sums are those of the rounded
// weights (numerator and denominator use the same weights), accumulated in
// fp32 by four v_dot2c_f32_bf16 against a pair of ones per step.
// Output: lane (g, r) register i of block vb of tile t holds O[row 4g+i of
// t][channel 16 vb + r].
//
// The running max m is kept in the scaled log2 domain; the step compares the
// raw scores with thr = (m + kRescaleSlack) / scale, so that the common step
// (no rescale) needs only each lane's own maximum: the row maximum over the
// four lane groups is formed only when some lane is over its threshold, and
// the scale goes into the exponent's fma.  This needs scale > 0: the kernel
// folds a negative scale's sign into q and raises its magnitude to at least
// FLT_MIN (so a zero scale gives equal weights to the visible keys, and a
// masked key's -inf times the scale stays -inf).
template <int D, int NT>
struct Wave32 {
  static constexpr int KB = D / 32;  // q.K MFMAs per half and tile
  static constexpr int VB = D / 16;  // p.V channel blocks
  floatx4_t o[NT][VB];
  bf16x8_t qb[NT][KB];  // q^T operands
  float m[NT];          // row r of tile t: running max (scaled, log2 domain)
  float thr[NT];        // row r of tile t: (m + kRescaleSlack) / scale
  float l[NT];          // row r of tile t: this lane's part of its weight sum

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) o[t][vb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
      l[t] = 0.f;
      m[t] = kFloorMax;
      thr[t] = kMinusInf;  // the first step with any live key sets m
    }
  }

  // k[h][kk]: K of token r of half h, channels 8 (4kk + g) .. +8.
  // load_v(vv) fills vv[vb] with channel 16 vb + r, keys 4g .. 4g+3 of half 0
  // then of half 1; it is called after the score MFMAs, which need only K.
  // keep[t]: bit 4h + j set when key 16h + 4g + j counts for this lane's row
  // of tile t.  vlive: keys from this one on hold no data; pages_ok (uniform):
  // bits 4h .. 4h+3 set when half h has a page; the V of keys outside both is
  // zeroed.  masked (uniform) false: every key of the step counts for every
  // row of the wave, and keep, vlive and pages_ok are not read (most steps of
  // a causal block lie below its diagonal, and the per-key selects are a
  // fifth of a step's vector work).
  template <class LoadV>
  __device__ __forceinline__ void step(const uint4 (&k)[2][KB], LoadV&& load_v,
                                       const uint32_t (&keep)[NT], int vlive, uint32_t pages_ok,
                                       bool masked, int g, float scale, float inv_scale) {
    floatx4_t sc[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t) sc[t][0] = sc[t][1] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    // The matrix-core runs of a step (scores here, P.V below) are issued at a
    // raised wave priority, so that a wave that reaches them goes ahead of the
    // other waves of its SIMD, which are in their vector (softmax) phase: the
    // waves of a workgroup move in step between the per-chunk barriers, and
    // without this their matrix and vector phases line up instead of
    // overlapping (95 -> 91 us on the 4 x 1024 causal batch).
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < KB; ++kk)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          sc[t][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, k[h][kk]), qb[t][kk], sc[t][h], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    float s[NT][8];  // raw scores q . k
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[t][i] = sc[t][0][i];
        s[t][4 + i] = sc[t][1][i];
      }
    }
    if (masked) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (((keep[t] >> i) & 1u) == 0) s[t][i] = kMinusInf;
    }
    uint4 vv[VB];
    load_v(vv);
    if (masked && (vlive < 32 || pages_ok != 0xffu)) {
      // Keys past the sequence end, and keys of a piece without a page, may
      // hold anything, NaN included: a zero weight times their V must give
      // exactly zero.
      const uint32_t lv = keys_upto(vlive - 1 - 4 * g) & pages_ok;
      uint32_t msk[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        msk[j] = ((lv >> (2 * j)) & 1u ? 0x0000ffffu : 0u) | ((lv >> (2 * j + 1)) & 1u ? 0xffff0000u : 0u);
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        vv[vb].x &= msk[0];
        vv[vb].y &= msk[1];
        vv[vb].z &= msk[2];
        vv[vb].w &= msk[3];
      }
    }
    bf16x8_t pb[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float lm = vmax3(vmax3(s[t][0], s[t][1], s[t][2]), vmax3(s[t][3], s[t][4], s[t][5]),
                             vmax2(s[t][6], s[t][7]));
      if (__builtin_amdgcn_ballot_w64(lm > thr[t]) != 0) {
        // Some row's maximum is over its threshold: form every row's maximum.
        const float pm = max_over_groups(lm) * scale;
        const float mn = fmaxf(m[t], pm);
        const float alpha = fast_exp2(m[t] - mn);
        m[t] = mn;
        thr[t] = (mn + kRescaleSlack) * inv_scale;
        l[t] *= alpha;
        // Register i of lane group g holds row 4g + i, whose factor lane 4g + i has.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ai = __shfl(alpha, 4 * g + i, kWave);
#pragma unroll
          for (int vb = 0; vb < VB; ++vb) o[t][vb][i] *= ai;
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[t][i] = (__bf16)fast_exp2(fmaf(s[t][i], scale, -m[t]));
      const uint4 pw = __builtin_bit_cast(uint4, pb[t]);
      const bf16x2_t one2 = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
      l[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw.x), one2, l[t], false);
      l[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw.y), one2, l[t], false);
      l[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw.z), one2, l[t], false);
      l[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw.w), one2, l[t], false);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      const bf16x8_t vt = __builtin_bit_cast(bf16x8_t, vv[vb]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        o[t][vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb[t], vt, o[t][vb], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }
};

// Two workgroups per CU (four waves per SIMD) need at most 128 VGPRs: the
// attribute holds the compiler to that (a couple of spilled registers at
// D = 128); with one workgroup per CU the kernel measured 11% slower.
template <int D, int HG>
__global__ void __launch_bounds__(kPrefillWaves * kWave) __attribute__((amdgpu_waves_per_eu(4)))
prefill_kernel(PrefillArgs a) {
  constexpr int QT = 16 / HG;     // query tokens per row tile
  constexpr int ROWS = QT * HG;   // score rows in use per tile (15 for HG = 3)
  constexpr int NT = kPrefillTiles;  // row tiles per wave
  constexpr int kThreads = kPrefillWaves * kWave;
  constexpr int kSteps = kPrefillSteps;  // 32-key steps per LDS chunk
  constexpr int kHalves = 2 * kSteps;  // 16-key pieces per chunk (one page each at P = 16)
  constexpr int kPieces = D * 16 * 2 / 16;  // 16-byte pieces of 16 keys' K (same for V)
  static_assert(2 * kPieces * kHalves % kThreads == 0 && kPieces % kWave == 0,
                "whole, wave-uniform loads per thread");
  constexpr int kLoads = 2 * kPieces * kHalves / kThreads;  // per thread and chunk
  // Two chunks (double buffer) of K as [16 keys][D/8][16 keys][8 channels]
  // and V as [32 keys][D/16][4][16 channels][2][4 keys]: the operand of lane
  // (g, r) -- K channel block 4kk + g of key r, V keys 4g .. 4g+3 of both
  // halves of channel 16 vb + r -- is 16 contiguous bytes, and the 16 lanes of
  // a lane group read one contiguous run (no bank conflicts).  After the last
  // chunk the same bytes hold the per-wave output rows [wave][16][D] in fp32.
  constexpr int kKBytes = kHalves * D * 16 * 2;
  constexpr int kBufBytes = 2 * kKBytes;  // K + V of one chunk
  constexpr int kOutBytes = kPrefillWaves * 16 * D * 4;
  __shared__ __align__(16) char smem[2 * kBufBytes > kOutBytes ? 2 * kBufBytes : kOutBytes];
  auto k_at = [&](int buf, int hf, int cb, int t) {  // 16 bytes: K channels 8cb.. of key t
    return smem + buf * kBufBytes + ((hf * (D / 8) + cb) * 16 + t) * 16;
  };
  auto v_at = [&](int buf, int st, int ch, int g, int hf) {  // 8 bytes: keys 4g.. of half hf
    return smem + buf * kBufBytes + kKBytes +
           ((((st * (D / 16) + (ch >> 4)) * 4 + g) * 16 + (ch & 15)) * 2 + hf) * 8;
  };
  float* s_out = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  // Tile order.  Workgroups go to the XCDs round robin by linear id, and on
  // each XCD in that order.  The order below gives each XCD whole runs of
  // query blocks of a few (request, head group) pairs, so that their K/V
  // chunks stay in that XCD's L2, and hands out the XCD's blocks longest
  // causal range first across all of its pairs (longest-processing-time
  // order: with the pairs taken one after another, the short blocks of the
  // first pairs ran early and the long blocks of the last pairs formed a tail
  // that left CUs idle).
  int b, u, bx;
  {
    const uint32_t gx = gridDim.x, gy = gridDim.y;
    const uint32_t n_wg = gx * gy * gridDim.z;  // below 2^31 (checked on the host)
    uint32_t t = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
    const uint32_t full = n_wg & ~(uint32_t)(kXcds - 1);
    if (t < full) {
      const uint32_t per = full / kXcds;  // workgroups of one XCD
      const uint32_t x = t % kXcds, j = t / kXcds;  // XCD, place in its order
      if (per % gx == 0) {
        const uint32_t pairs = per / gx;  // whole (request, head group) runs
        t = x * per + (j % pairs) * gx + j / pairs;
      } else {
        t = x * per + j;
      }
    }
    bx = (int)(gx - 1 - t % gx);
    u = (int)((t / gx) % gy);
    b = (int)(t / (gx * gy));
  }
  const int wg_tok0 = bx * kPrefillWaves * NT * QT;  // first query token of the workgroup
  const int tok0 = wg_tok0 + w * NT * QT;              // first query token of this wave
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
  // Row r16 of tile t = (token tok0 + t QT + r16 / HG, head r16 % HG).
  // Rows without a query token read the request's first row of q (so that
  // every lane loads, with no masked branch around the loads): their weights
  // are computed and never stored, and rows do not mix.
  int rt[NT], lim[NT];
  bool rvalid[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    rt[t] = tok0 + t * QT + r16 / HG;
    rvalid[t] = r16 < ROWS && rt[t] < n;
    lim[t] = a.causal ? L - n + rt[t] : L - 1;  // last key the row sees
  }
  // The step wants a positive scale: a negative one's sign goes into q (an
  // exact bf16 sign flip, below), and its magnitude is at least FLT_MIN.
  const float scale = fmaxf(fabsf(a.scale_log2), 1.17549435e-38f);
  const float inv_scale = 1.0f / scale;
  // Keys this wave reads, and keys the workgroup reads (its last wave's limit).
  auto block_end = [&](int t0) {
    const int last = min(t0 + NT * QT, n) - 1;
    return a.causal ? max(0, min(L, L - n + last + 1)) : L;
  };
  const int kv_end = active ? block_end(tok0) : 0;
  // The last key every row of the wave sees (its first token has the
  // smallest causal limit).
  const int lim_min = min(a.causal ? L - n + tok0 : L - 1, kv_end - 1);
  const int wg_end = block_end(min(wg_tok0 + (kPrefillWaves - 1) * NT * QT, n - 1));

  Wave32<D, NT> st;
  st.init();
  {
    // q^T operands: lane (g4, r16) supplies row r16 of each tile, channels
    // 8*(4kk + g4) .. +8.
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint4* qp = reinterpret_cast<const uint4*>(
          a.q + ((size_t)(q0 + (rvalid[t] ? rt[t] : 0)) * Hq + hq0 + r16 % HG) * D + g4 * 8);
#pragma unroll
      for (int kk = 0; kk < Wave32<D, NT>::KB; ++kk) {
        st.qb[t][kk] = __builtin_bit_cast(bf16x8_t, qp[4 * kk]);
      }
    }
    // Wait for q here: left to the first matrix-core step, the wait would sit
    // inside the KV loop and drain the next chunk's loads with it every step.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    if (a.scale_log2 < 0.f) {  // uniform; after the wait, so the q loads go out together
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int kk = 0; kk < Wave32<D, NT>::KB; ++kk) {
          uint4 w4 = __builtin_bit_cast(uint4, st.qb[t][kk]);
          w4.x ^= 0x80008000u;
          w4.y ^= 0x80008000u;
          w4.z ^= 0x80008000u;
          w4.w ^= 0x80008000u;
          st.qb[t][kk] = __builtin_bit_cast(bf16x8_t, w4);
        }
    }
  }

  const int P = a.page_size;
  const int log2_s = a.log2_steps;
  const size_t tile_b = (size_t)P * D * 2;
  const size_t head_b = (size_t)g * tile_b;
  const char* kbase = reinterpret_cast<const char*>(a.k);
  const char* vbase = reinterpret_cast<const char*>(a.v);
  const int halves = (wg_end + 15) / 16;  // 16-key pieces the workgroup reads
  const int chunks = (halves + kHalves - 1) / kHalves;

  // Page ids are read 64 at a time, one per lane, and taken out with a
  // uniform readlane (a vector load of a uniform address would need a wait
  // that also drains the K/V loads in flight).  Page of a 16-key piece: -1 for
  // an index outside kv_indices or the pool (its keys are skipped).
  int vblk = -1, vpage = -1;
  auto page_of = [&](int hf) {
    const int pg = hf >> log2_s;
    if ((pg >> 6) != vblk) {  // uniform; once per 64 pages
      vblk = pg >> 6;
      const int pos = ip0 + (vblk << 6) + lane;
      vpage = pos >= 0 && pos < a.num_indices ? a.kv_indices[pos] : -1;
      if (vpage >= a.num_pages) vpage = -1;
    }
    return __builtin_amdgcn_readlane(vpage, pg & 63);
  };
  // Global -> registers: the workgroup's threads fetch 16-byte pieces
  // tid, tid + 512, ... of a chunk, 16 keys at a time, K pieces before V
  // pieces.  Piece y of 16 keys' K is (channel block y / 16, key y % 16);
  // piece y of their V is (channel y / 2, keys 8 (y % 2) .. +7).  A wave's 64
  // pieces lie in one 16-key piece and one operand, so page lookup and K/V
  // choice are wave-uniform.  A piece whose page does not exist is not
  // loaded: its registers keep older data, which the step masks (its keys'
  // weights are zero and their V is zeroed), so no register is cleared per
  // chunk.
  uint4 stage[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) stage[i] = make_uint4(0, 0, 0, 0);
  int pids[kHalves];    // pages of the 16-key pieces of the chunk being fetched
  uint32_t pages_next;  // bit hf: piece hf of that chunk has a page (uniform)
  auto piece = [&](int i, int& hf, int& y, bool& is_v) {
    const int xw = w * kWave + i * kThreads;  // the wave's first piece
    if constexpr ((2 * kPieces) % kThreads == 0) {
      // The workgroup's pieces i cover whole 16-key pieces: hf is known here.
      hf = i * kThreads / (2 * kPieces);
    } else {
      hf = xw / (2 * kPieces);
    }
    const int yw = xw - hf * 2 * kPieces;
    is_v = yw >= kPieces;
    y = yw - (is_v ? kPieces : 0) + lane;
  };
  auto fetch = [&](int c) {
    uint32_t ok = 0;
#pragma unroll
    for (int hf = 0; hf < kHalves; ++hf) {
      pids[hf] = c * kHalves + hf < halves ? page_of(c * kHalves + hf) : -1;
      ok |= pids[hf] >= 0 ? 1u << hf : 0u;
    }
    pages_next = __builtin_amdgcn_readfirstlane(ok);
    // Nothing is in flight here (the last chunk's loads were published), but
    // the compiler cannot tell: without this wait it puts one between the
    // chunk's loads (a load may skip a piece, so their registers keep older
    // values) and the second load leaves only when the first has returned.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      int hf, y;
      bool is_v;
      piece(i, hf, y, is_v);
      const int pid = pids[hf];
      if (pid < 0) continue;
      const int sub = (c * kHalves + hf) & ((1 << log2_s) - 1);
      const char* tile = (is_v ? vbase : kbase) + (size_t)pid * a.num_kv_heads * tile_b + head_b;
      // Step sub of the tile: V [D][16], K [D/8][16][8].
      const int off = sub * 16 * D * 2 + (is_v ? ((y >> 1) * 16 + 8 * (y & 1)) * 2
                                               : ((y >> 4) * 16 + (y & 15)) * 16);
      stage[i] = *reinterpret_cast<const uint4*>(tile + off);
    }
  };
  auto publish = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      int hf, y;
      bool is_v;
      piece(i, hf, y, is_v);
      if (is_v) {  // keys 8h .. 8h+7 of one channel: two 4-key pieces
        const int ch = y >> 1, h = y & 1;
        *reinterpret_cast<uint2*>(v_at(buf, hf >> 1, ch, 2 * h, hf & 1)) =
            make_uint2(stage[i].x, stage[i].y);
        *reinterpret_cast<uint2*>(v_at(buf, hf >> 1, ch, 2 * h + 1, hf & 1)) =
            make_uint2(stage[i].z, stage[i].w);
      } else {
        *reinterpret_cast<uint4*>(k_at(buf, hf, y >> 4, y & 15)) = stage[i];
      }
    }
  };

  if (chunks > 0) {
    fetch(0);
    publish(0);
  }
  __syncthreads();
  for (int c = 0; c < chunks; ++c) {
    const int buf = c & 1;
    const uint32_t pages_live = pages_next;
    if (c + 1 < chunks) fetch(c + 1);  // in flight while this chunk is consumed
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int t0 = (c * kSteps + s) * 32;
      if (t0 < kv_end) {  // uniform per wave
        uint4 kop[2][Wave32<D, NT>::KB];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int kk = 0; kk < Wave32<D, NT>::KB; ++kk)
            kop[h][kk] = *reinterpret_cast<const uint4*>(k_at(buf, 2 * s + h, 4 * kk + g4, r16));
        auto load_v = [&](uint4 (&vv)[Wave32<D, NT>::VB]) {
#pragma unroll
          for (int vb = 0; vb < Wave32<D, NT>::VB; ++vb)
            vv[vb] = *reinterpret_cast<const uint4*>(v_at(buf, s, 16 * vb + r16, g4, 0));
        };
        // Key t0 + 16h + 4 g4 + j counts for a row when it is at most
        // min(lim, kv_end - 1) and its page exists; when that holds for all 32
        // keys and every row of the wave (uniform), no key is masked.
        const uint32_t pages_ok = ((pages_live >> (2 * s)) & 1u ? 0x0fu : 0u) |
                                  ((pages_live >> (2 * s + 1)) & 1u ? 0xf0u : 0u);
        const bool masked = !(pages_ok == 0xffu && t0 + 31 <= lim_min);
        const int vlive = min(32, kv_end - t0);
        uint32_t keep[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) keep[t] = 0xffu;
        if (masked) {
#pragma unroll
          for (int t = 0; t < NT; ++t)
            keep[t] = keys_upto(min(lim[t], kv_end - 1) - t0 - 4 * g4) & pages_ok;
        }
        st.step(kop, load_v, keep, vlive, pages_ok, masked, g4, scale, inv_scale);
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

  // Normalise, one tile at a time: the four lanes of row r hold its partial
  // sums; register i of lane group g holds row 4g + i.  Rows go through LDS
  // so that every lane writes 8 channels (16 bytes) of one row.
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float lt = sum_over_groups(st.l[t]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float li = __shfl(lt, 4 * g4 + i, kWave);
      const float inv = li > 0.f ? 1.0f / li : 0.f;
#pragma unroll
      for (int vb = 0; vb < Wave32<D, NT>::VB; ++vb)
        s_out[(w * 16 + 4 * g4 + i) * D + 16 * vb + r16] = st.o[t][vb][i] * inv;
    }
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's LDS writes land first
    constexpr int kChunks = ROWS * (D / 8);
    const int tt0 = tok0 + t * QT;  // first token of the tile
#pragma unroll
    for (int c = lane; c < kChunks; c += kWave) {
      const int rr = c / (D / 8);
      const int c8 = (c - rr * (D / 8)) * 8;
      const int tok = tt0 + rr / HG;
      if (tok < n) {
        const float4 x0 = *reinterpret_cast<const float4*>(&s_out[(w * 16 + rr) * D + c8]);
        const float4 x1 = *reinterpret_cast<const float4*>(&s_out[(w * 16 + rr) * D + c8 + 4]);
        *reinterpret_cast<uint4*>(a.out + ((size_t)(q0 + tok) * Hq + hq0 + rr % HG) * D + c8) =
            make_uint4(pack_bf16x2(x0.x, x0.y), pack_bf16x2(x0.z, x0.w), pack_bf16x2(x1.x, x1.y),
                       pack_bf16x2(x1.z, x1.w));
      }
    }
    // The next tile's rows reuse the wave's LDS rows: the reads above come
    // first (LDS operations of a wave complete in order).
  }
}

template <int D>
hipError_t launch_p(const PrefillArgs& a, int hg, dim3 grid, hipStream_t s) {
  const dim3 block(kPrefillWaves * kWave);
  switch (hg) {
    case 1: hipLaunchKernelGGL((prefill_kernel<D, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<D, 2>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((prefill_kernel<D, 3>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<D, 4>), grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL((prefill_kernel<D, 5>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((prefill_kernel<D, 6>), grid, block, 0, s, a); break;
    case 7: hipLaunchKernelGGL((prefill_kernel<D, 7>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int hg, int max_q_len,
                          hipStream_t s) {
  const int qt = 16 / hg;
  const int per_group = qt * kPrefillTiles * kPrefillWaves;  // query tokens one workgroup covers
  const dim3 grid((max_q_len + per_group - 1) / per_group, a.num_q_heads / hg, a.batch);
  if (grid.x == 0 || grid.z == 0) return hipSuccess;
  if ((long long)grid.x * grid.y * grid.z > INT32_MAX) return hipErrorInvalidConfiguration;
  if (head_dim == 128) return launch_p<128>(a, hg, grid, s);
  if (head_dim == 64) return launch_p<64>(a, hg, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv
