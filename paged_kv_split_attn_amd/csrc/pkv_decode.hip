// Paged split-KV decode attention for gfx950 (MI355X), one kernel per call.
//
// Work decomposition (stream-K style).  The step's tiles, ordered (request,
// head group, page), are cut into equal contiguous ranges: one per workgroup of
// eight waves (one workgroup per CU, two waves per SIMD), an eighth of that per
// wave.  Each wave keeps two steps of loads in flight; two waves per SIMD hide
// each other's tail of a step better than one wave with a deeper register ring
// (which measured slower at every depth).  A head group is HG query heads
// that share one KV head (the largest of 16, 12, 8, 7, .., 1 that divides G), so
// a tile is one page of one KV head, K and V, read once for HG query heads.  Each wave streams its range,
// keeping an online-softmax state that it closes whenever the range leaves a
// (request, head group) segment.  A segment wholly inside a wave is written
// straight to the output; other pieces go to LDS, where the workgroup merges
// the pieces of each segment; a segment that also spans other workgroups leaves
// a normalised partial and its log-sum-exp in the workspace, and the last
// workgroup to arrive merges them in a fixed order.  Split partials merged by
// log-sum-exp follow the pages' decode design (commits by ViperEkura: o_part /
// ml_part partials and their combine kernel); here the merge is fused into the
// same launch and every wave gets the same number of pages.
//
// Arithmetic on the matrix cores.  A wave consumes 16 tokens of one tile per
// step.  Scores S^T[token][head] = K . q^T come from D/32
// v_mfma_f32_16x16x32_bf16 (K rows are the A operand, q the B operand; query
// heads beyond HG are zero columns).  Each 16-token step of a K tile is stored
// [D/8][16][8], so the A operand of one MFMA (channels 32kk .. 32kk+31 of 16
// tokens) is one contiguous kilobyte: lane (g, r) reads channel block 4kk + g
// of token r.  The result leaves lane (g, r) = (l / 16, l % 16) holding the
// scores of head r for tokens 4g .. 4g+3, which is exactly the A-operand layout
// of v_mfma_f32_16x16x16_bf16 for P . V, so the softmax weights never move
// between lanes.  Each V step is stored channel-major ([D][16]), so the B
// operand (4 tokens of one channel per lane) is one 8-byte load, and one load
// instruction reads 512 contiguous bytes at every page size.  The weights
// enter the product as bf16 hi + lo parts (two MFMAs), keeping the p.V sum
// accurate to about 2^-16 relative, while the softmax sums stay in fp32.  K and
// V go straight from HBM into registers: every element is used once.
//
// Online softmax.  The running max of each head is shared by the four lanes
// that hold its scores (a two-step cross-lane max per step) and updated lazily:
// accumulators are rescaled only when a step's max exceeds the stored one by
// more than 2^8 in the exp2 domain, so weights stay below 256 and the rescale
// branch (wave-uniform) is rarely taken.  Scores are kept in the log2 domain
// (sm_scale * log2 e folded into one multiply-add) so every exponential is a
// single v_exp_f32.
//
// Variants (template KIND): the plain decode; the KV append fused into the
// decode; a per-token keep mask; and token-major K/V ([slot][Hkv][D] rows, the
// contiguous layout or a page-size-1 token table), where the plan's pages are
// 16-token blocks and V^T operands are gathered element by element.

#include "pkv_mfma.h"
#include "pkv_plan.h"

namespace pkv {
namespace {


// Wait until every earlier store of the wave has been acknowledged (for the
// device-coherent partial stores of the epilogue: is visible to every XCD).
// s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// A pointer that every lane holds the same value of, moved to scalar
// registers (readfirstlane works on 32 bits: both halves are read).
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Pointers the epilogue needs, parked in LDS at the start so that they do
// not hold scalar registers through the streaming loop.
struct EpiloguePtrs {
  int32_t* hdr;
  int32_t* counters;
  float* lse;
  float* opart;
};


// Kernel variants: plain decode, KV append fused into the decode, decode with
// a per-token keep mask, decode over token-major K/V.
enum Kind : int { kPlain = 0, kAppend = 1, kMasked = 2, kTokens = 3 };


typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));
typedef unsigned u2v __attribute__((ext_vector_type(2)));

// Online-softmax combine of (m, l, values) in the log2 domain, four channels
// that share m and l.
struct Combine4 {
  float m = kFloorMax, den = 0.f;
  f4 num = {0.f, 0.f, 0.f, 0.f};
  __device__ __forceinline__ void add(float mk, float lk, f4 vk) {
    const float mn = vmax2(m, mk);
    const float ca = fast_exp2(m - mn);
    const float cb = fast_exp2(mk - mn);
    den = den * ca + lk * cb;
    num = num * ca + vk * cb;
    m = mn;
  }
};

// Buffer resource word 3 for raw (untyped) buffer accesses on gfx950, and the
// cache-policy bit that makes a buffer access coherent at device scope (sc1):
// the partials one workgroup hands to another on a different XCD.  Buffer
// accesses outside the resource's size read 0 and write nothing.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kCoherent = 16;

// The in-workgroup merge slots: slot 2w + j is wave w's first (j = 0) or last
// (j = 1) piece when that piece leaves its segment unfinished.
constexpr int kSlots = 2 * kWavesPerGroup;
static_assert(kSlots <= 32, "slot masks of 32 bits");

// Where each slot's segment goes, as lane masks over the slots: valid slots,
// slots that end their segment, segments written to the output here, and
// segments left as the workgroup's first / last partial.  Slot k's segment
// (-1: none) is on lane k.  Vector work, one slot per lane: the scalar unit is
// shared by the waves of a compute unit, and all of them build the same table.
struct SlotTable {
  uint32_t validm, endm, localm, kind1m, glob0m;
  int sk;
};

__device__ __forceinline__ SlotTable make_slot_table(int sk_l, int lane, int grp,
                                                     const GroupInfo& g) {
  // Segments do not decrease along the valid slots, so slot k ends its
  // segment exactly when the smallest valid segment after it differs.
  int after = __shfl_down(sk_l < 0 ? 0x7fffffff : sk_l, 1, kWave);  // every lane shuffles
  after = lane + 1 < kSlots ? after : 0x7fffffff;
#pragma unroll
  for (int off = 1; off < kSlots; off <<= 1) {
    const int y = __shfl_down(after, off, kWave);
    if (lane + off < kSlots) after = min(after, y);
  }
  const int slot_l = sk_l == g.seg[0] ? 0 : (sk_l == g.seg[1] ? 1 : -1);
  const bool local_l = slot_l < 0 || (slot_l == 0 ? (g.lo[0] == grp && g.hi[0] == grp)
                                                  : (g.lo[1] == grp && g.hi[1] == grp));
  const bool valid_l = lane < kSlots && sk_l >= 0;
  SlotTable t;
  t.validm = (uint32_t)__ballot(valid_l);
  t.endm = (uint32_t)__ballot(valid_l && after != sk_l);
  t.localm = (uint32_t)__ballot(valid_l && local_l);
  t.kind1m = (uint32_t)__ballot(valid_l && !local_l && slot_l == 1);
  t.glob0m = (uint32_t)__ballot(valid_l && !local_l && slot_l == 0);
  t.sk = sk_l;
  return t;
}

template <int D, int HG, int KIND, bool PLAN>
__global__ void __launch_bounds__(kGroupThreads) decode_kernel(DecodeArgs a) {
  constexpr bool APPEND = KIND == kAppend;
  constexpr bool MASKED = KIND == kMasked;
  constexpr bool TOKENS = KIND == kTokens;  // token-major K/V, 16-token blocks as pages
  constexpr int kStages = 2;  // register ring: steps in flight per wave

  // Pieces that leave a wave unfinished: slot 0 = the wave's first piece,
  // slot 1 = its last piece (every other piece is a whole segment).  Slot 1
  // also serves as the wave's transpose of a whole segment's finished rows:
  // whole segments come before the last piece, and a partial piece after the
  // first is the last (its range ends inside it), so the rows are written out
  // before slot 1 takes the last piece.  (Sixteen-head groups fit in LDS only
  // with the transpose kept there.)
  __shared__ __align__(16) float s_acc[kWavesPerGroup][2][HG][D];
  // Max and sum of slot k = 2 w + (0 | 1) of head h at [h][k]: a head's 16
  // slots are four 16-byte reads.
  __shared__ __align__(16) float s_m[HG][kSlots];
  __shared__ __align__(16) float s_l[HG][kSlots];
  __shared__ int s_seg[PLAN ? kWavesPerGroup : 1][2];  // planning launch: the slot segments
  __shared__ int s_merge[2];  // of those, the ones this workgroup merges
  __shared__ GroupInfo s_gi;  // the workgroup's merge record, for the epilogue
  __shared__ EpiloguePtrs s_ptr;
  __shared__ uint32_t s_vn[APPEND ? kWavesPerGroup : 1][kWave];  // appended V row, per wave
  // The step's page prefix sums and lengths, when this launch plans the step.
  __shared__ int32_t s_pip[PLAN ? kPlanLdsRequests + 1 : 1];
  __shared__ int32_t s_plen[PLAN ? kPlanLdsRequests : 1];
  __shared__ int s_scan[kWavesPerGroup];
  __shared__ int s_pcount[2];  // requests without pages, error bits

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int grp = blockIdx.x;
  const int U = a.units;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int Hq = a.num_q_heads;

  int ngroups, nempty;
  WaveRange rng;
  GroupInfo gi0;
  int slot_seg_l = -1;  // two-call path: segment of merge slot `lane` (lanes below kSlots)
  long long ptiles = 0;  // planning launch: tiles of the plan
  int perr_bits = 0;     // and its error bits
  if constexpr (PLAN) {
    // The step's plan, computed here from the lengths with the arithmetic of
    // the metadata kernel: prefix sums of page counts, the tile count, the
    // workgroup count and each wave's range (this workgroup's merge record is
    // only needed at the end, and is made there).  The launch reads its plan
    // from registers and LDS only; what it stores for the step's later calls
    // goes out at the end.
    int carry = 0;
    if (a.batch <= kWave) {
      // Every wave plans on its own, the requests on its lanes: no barrier.
      const int Lb = lane < a.batch ? a.seq_lens[lane] : 0;
      const int nb = pages_of(Lb, a.page_size);
      int incl = nb;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += y;
      }
      carry = __shfl(incl, kWave - 1, kWave);
      if (lane < a.batch) {
        s_plen[lane] = Lb;
        s_pip[lane + 1] = incl;
      }
      if (lane == 0) s_pip[0] = 0;  // every wave writes the same values
      nempty = (int)__popcll(__ballot(lane < a.batch && nb == 0));
      perr_bits = __ballot(lane < a.batch && Lb < 0) ? (int)kErrNegativeLength : 0;
      const long long T = (long long)carry * U;
      ngroups = plan_groups(T, a.groups, a.min_tiles, a.forced);
      ptiles = T;
      const WaveLocator loc{incl - nb, nb, Lb, a.batch, U};
      if (T < 0x80000000LL) {
        const PlanMath<uint32_t> pm((uint32_t)T, (uint32_t)max(ngroups, 1));
        rng = plan_wave_range<uint32_t>(loc, pm, ngroups, grp, w);
      } else {
        const PlanMath<uint64_t> pm((uint64_t)T, (uint32_t)max(ngroups, 1));
        rng = plan_wave_range<uint64_t>(loc, pm, ngroups, grp, w);
      }
    } else {
      // A block-wide scan over the requests, the prefix sums in LDS.
      if (tid == 0) {
        s_pip[0] = 0;
        s_pcount[0] = 0;
        s_pcount[1] = 0;
      }
      __syncthreads();
      int empty = 0, perr = 0;
      for (int base = 0; base < a.batch; base += kGroupThreads) {  // uniform trip count
        const int b = base + tid;
        int n = 0;
        if (b < a.batch) {
          const int L = a.seq_lens[b];
          s_plen[b] = L;
          if (L < 0) perr |= kErrNegativeLength;
          n = pages_of(L, a.page_size);
          empty += n == 0;
        }
        int total;
        const int incl = block_inclusive_scan<kGroupThreads>(n, s_scan, &total);
        if (b < a.batch) s_pip[b + 1] = carry + incl;
        carry += total;
      }
      if (empty) atomicAdd(&s_pcount[0], empty);
      if (perr) atomicOr(&s_pcount[1], perr);
      __syncthreads();
      const long long T = (long long)carry * U;
      ngroups = plan_groups(T, a.groups, a.min_tiles, a.forced);
      ptiles = T;
      nempty = s_pcount[0];
      perr_bits = s_pcount[1];
      const Locator loc{s_pip, s_plen, a.batch, U};
      if (T < 0x80000000LL) {
        const PlanMath<uint32_t> pm((uint32_t)T, (uint32_t)max(ngroups, 1));
        rng = plan_wave_range<uint32_t>(loc, pm, ngroups, grp, w);
      } else {
        const PlanMath<uint64_t> pm((uint64_t)T, (uint32_t)max(ngroups, 1));
        rng = plan_wave_range<uint64_t>(loc, pm, ngroups, grp, w);
      }
    }
    gi0 = GroupInfo{{-1, -1}, {0, 0}, {0, 0}, {0, 0}};  // made at the end
  } else {
    // The plan size, this wave's range and the workgroup's merge record are
    // fetched together (the test reads all three, so no load waits for
    // another): the first K/V loads wait on them, and the merges at the end
    // need nothing else from the plan.
    ngroups = a.hdr[kHdrGroups];
    nempty = a.hdr[kHdrEmpty];
    // The plan must be the one built for this call's batch and head grouping:
    // a plan of a larger batch would send waves to requests past the caller's
    // arrays.  On a mismatch nothing is read or written but the error word.
    const bool plan_ok = a.hdr[kHdrBatch] == a.batch && a.hdr[kHdrUnits] == a.units;
    rng = a.waves[grp * kWavesPerGroup + w];
    gi0 = a.ginfo[grp];
    // The slot segments, one per lane, for the merge at the end: one vector
    // load that nothing waits for before then (held in scalar registers
    // through the stream they crowd the stream's own registers).
    slot_seg_l = a.ginfo[grp].slot_seg[lane & (kSlots - 1)];
    if (!plan_ok) {  // uniform over the grid
      if (grp == 0 && tid == 0) atomicOr(&a.hdr[kHdrError], (int)kErrPlanMismatch);
      return;
    }
  }
  // Page prefix sum and length of request i, from LDS when this launch planned.
  auto indptr_at = [&](int i) -> int {
    if constexpr (PLAN) return s_pip[i];
    else return a.kv_indptr[i];
  };
  auto len_at = [&](int i) -> int {
    if constexpr (PLAN) return s_plen[i];
    else return a.seq_lens[i];
  };
  // Requests without tokens get zero rows (no tile covers them); workgroup 0
  // writes them, after its stream, or at once when the plan has no tile at all.
  auto zero_empty_rows = [&]() {
    if (nempty > 0 && w == 0) {
      for (int eb = lane; eb < a.batch; eb += kWave) {
        if (indptr_at(eb + 1) == indptr_at(eb)) {
          uint4* row = reinterpret_cast<uint4*>(a.out + (size_t)eb * Hq * D);
          for (int i = 0; i < Hq * D / 8; ++i) row[i] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  // Planning launch: this workgroup's merge record, made by wave 0 (lanes 0
  // and 1, one half each) from the prefix sums in LDS, which that wave wrote
  // itself or saw complete at a barrier.
  auto make_group_info = [&]() {
    if constexpr (PLAN) {
      if (w == 0 && lane < 2) {
        const Locator loc{s_pip, s_plen, a.batch, U};
        if (ptiles < 0x80000000LL) {
          const PlanMath<uint32_t> pm((uint32_t)ptiles, (uint32_t)max(ngroups, 1));
          plan_group_half<uint32_t>(loc, pm, ngroups, U, grp, lane, &s_gi);
        } else {
          const PlanMath<uint64_t> pm((uint64_t)ptiles, (uint32_t)max(ngroups, 1));
          plan_group_half<uint64_t>(loc, pm, ngroups, U, grp, lane, &s_gi);
        }
      }
    }
  };
  // The plan this launch made, stored for the step's later calls (nothing in
  // this launch reads it back): each wave its range, wave 0 the merge record
  // (after make_group_info) and, in workgroup 0, kv_indptr and the header.
  // Stores count with loads in a wave's vector-memory counter, so they go out
  // after the wave's last load: issued before the K/V stream, every wait for a
  // K/V step would also wait for them to be acknowledged.
  auto store_plan = [&](bool streamed) {
    if constexpr (PLAN) {
      if (lane == 0) a.plan_waves[grp * kWavesPerGroup + w] = rng;
      if (w == 0) {
        // Words 0..7 from s_gi, then the slot segments this workgroup's
        // waves recorded (none when it had no range).
        constexpr int kHead = 8, kWords = (int)(sizeof(GroupInfo) / 4);
        static_assert(kHead + 2 * kWavesPerGroup == kWords, "merge record layout");
        if (lane < kWords) {
          const int v = lane < kHead ? reinterpret_cast<const int*>(&s_gi)[lane]
                                     : (streamed ? reinterpret_cast<const int*>(s_seg)[lane - kHead]
                                                 : -1);
          reinterpret_cast<int*>(&a.plan_ginfo[grp])[lane] = v;
        }
        if (grp == 0) {
          for (int b = lane; b <= a.batch; b += kWave) a.plan_indptr[b] = s_pip[b];
          if (lane == 0) {
            a.hdr[kHdrGroups] = ngroups;
            a.hdr[kHdrTiles] = (int)ptiles;
            a.hdr[kHdrUnits] = U;
            a.hdr[kHdrBatch] = a.batch;
            a.hdr[kHdrEmpty] = nempty;
            // Other workgroups may already have latched decode errors: OR, never store.
            if (perr_bits) atomicOr(&a.hdr[kHdrError], perr_bits);
          }
        }
      }
    }
  };
  if ((grp >= ngroups) | (rng.count < 0) | (gi0.seg[0] < -1)) {  // uniform over the workgroup
    if (grp == 0) zero_empty_rows();
    make_group_info();
    store_plan(false);
    return;
  }
  if (tid == 0) {  // parked in LDS until the epilogue
    if constexpr (!PLAN) s_gi = gi0;
    s_ptr = EpiloguePtrs{a.hdr, a.counters, a.lse, a.opart};
  }
  if constexpr (PLAN) {
    if (lane == 0) {
      s_seg[w][0] = -1;
      s_seg[w][1] = -1;
    }
  }

  const int g4 = lane >> 4;   // lane group: tokens 4*g4 .. 4*g4+3 of a step
  const int r16 = lane & 15;  // head of the scores / channel of the outputs
  // Channel of output column r16 of P.V block vb: 16 vb + r16, or for
  // token-major K/V (whose V is read as contiguous channels per token)
  // (D / 16) r16 + vb.
  auto out_ch = [&](int vb) { return TOKENS ? (D / 16) * r16 + vb : 16 * vb + r16; };
  const float bias = r16 < HG ? 0.f : kMinusInf;
  const int P = a.page_size;
  const int log2_s = a.log2_steps;  // steps of 16 tokens per page
  const size_t tile_b = (size_t)P * D * 2;  // bytes of one (page, head) tile
  // A tile is P / 16 steps of 16 tokens, each laid out K [D/8][16][8] and
  // V [D][16], kStepBytes apiece.
  constexpr size_t kStepBytes = (size_t)16 * D * 2;
  // Lane byte offsets inside a step: K block g4, token r16; V^T channel r16, tokens 4*g4.
  const uint32_t k_boff = (uint32_t)(g4 * 16 + r16) * 16;
  const uint32_t v_boff = (uint32_t)(r16 * 16 + 4 * g4) * 2;
  const char* kbase = reinterpret_cast<const char*>(a.k);
  const char* vbase = reinterpret_cast<const char*>(a.v);
  const size_t slot_b = (size_t)a.num_kv_heads * D * 2;  // bytes of one token slot (TOKENS)
  // Fused KV append (k_new / v_new given): the step that holds token seq_len - 1
  // takes that token's K and V from k_new / v_new instead of the pool, and the
  // wave of the KV head's first head group writes them into the pool.
  constexpr bool fuse_append = APPEND;
  // Keep mask of the masked variant: bytes [batch][mask_stride] behind a
  // bounds-checked buffer resource (reads past the end return 0).
  const __amdgpu_buffer_rsrc_t mask_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(MASKED ? a.mask : reinterpret_cast<const uint8_t*>(a.q)), 0,
      MASKED ? a.mask_stride * a.batch : 0, kBufferWord3);
  int err = 0;

  int b = rng.b, u = rng.u, p = rng.p, left = rng.count, piece = 0;
  int ip0 = rng.ip0, n = rng.pages, L = rng.len;  // request b (reloaded when b changes)
  MfmaWave<D, HG> st;
  // Fused append: the appended token's rows (K one 8-channel chunk per lane,
  // V two channels per lane), fetched when a piece reaches a request's last
  // page, and the pool slot they still have to be written to (page -1: none).
  // The pool write waits until the wave's loads are all issued: a store counts
  // with loads in the wave's vector-memory counter, so one issued mid-stream
  // would hold up every later wait for a K/V step until it is acknowledged.
  uint4 knew4 = make_uint4(0, 0, 0, 0);
  uint32_t vnew2 = 0;
  int pend_page = -1, pend_head = 0, pend_sub = 0, pend_tok = 0;
  auto flush_token = [&]() {
    if constexpr (APPEND) {
      if (pend_page >= 0) {
        const size_t off = (size_t)pend_page * a.num_kv_heads * tile_b +
                           (size_t)pend_head * tile_b + (size_t)pend_sub * kStepBytes;
        if (lane < D / 8)  // K chunk `lane` of the token: [D/8][16][8] step layout
          *reinterpret_cast<uint4*>(const_cast<char*>(kbase) + off +
                                    ((size_t)lane * 16 + pend_tok) * 16) = knew4;
        uint16_t* vcol = reinterpret_cast<uint16_t*>(const_cast<char*>(vbase) + off);
        if (lane < D / 2) {  // V channels 2 lane, 2 lane + 1: [D][16] step layout
          vcol[(size_t)(2 * lane) * 16 + pend_tok] = (uint16_t)(vnew2 & 0xffffu);
          vcol[(size_t)(2 * lane + 1) * 16 + pend_tok] = (uint16_t)(vnew2 >> 16);
        }
        pend_page = -1;
      }
    }
  };
  while (left > 0) {  // one piece = the part of segment (b, u) inside this wave's range
    const int len = min(left, n - p);
    if (len <= 0) break;  // only reachable with metadata that does not match kv_indptr
    const int hq0 = u * HG;
    const int g = hq0 / G;

    st.init();
    {
      // q^T operand: lane (g4, r16) supplies head r16, channels 8*(4kk + g4) .. +8.
      const uint4* qp = reinterpret_cast<const uint4*>(
          a.q + ((size_t)b * Hq + hq0 + (r16 < HG ? r16 : 0)) * D + g4 * 8);
#pragma unroll
      for (int kk = 0; kk < MfmaWave<D, HG>::KB; ++kk) {
        const uint4 w4 = r16 < HG ? qp[4 * kk] : make_uint4(0, 0, 0, 0);
        st.qb[kk] = __builtin_bit_cast(bf16x8_t, w4);
      }
    }
    const size_t head_b = (size_t)g * tile_b;
    // Rows of the appended token (only formed when there is one to append).
    const size_t new_off = fuse_append ? ((size_t)b * a.num_kv_heads + g) * D : 0;
    const char* knew_row = reinterpret_cast<const char*>(fuse_append ? a.k_new + new_off : a.k);
    const uint16_t* vnew_row = fuse_append ? a.v_new + new_off : a.v;
    const bool writer = hq0 % G == 0;  // first head group of KV head g
    const int mask_row = MASKED ? b * a.mask_stride : 0;  // byte offset of request b's keep row
    // Rows of the appended token, fetched when this piece reaches the
    // request's last page (a write still pending from an earlier request goes
    // out first: it needs these registers).
    if constexpr (APPEND) {
      if (p + len == n) {
        flush_token();
        if (lane < D / 2) vnew2 = reinterpret_cast<const uint32_t*>(vnew_row)[lane];
        if (lane < D / 8) knew4 = reinterpret_cast<const uint4*>(knew_row)[lane];
      }
    }

    // Token-major K/V: blocks of 16 steps, register r of lane i holding the
    // slot of token 16 (p + jb) + 64 r + i of the block (the K row of lanes
    // r16 = i % 16 in step 4 r + i / 16, and the V row of the lanes whose four
    // tokens include it, both fetched by a lane shuffle), or -1 past the
    // sequence or for an unusable slot.  The register ring starts again at
    // every block, behind the block's slot-id loads, so blocks are long.
    constexpr int kTokRegs = 4;
    constexpr int kBlock = TOKENS ? 4 * kTokRegs : kWave;
    for (int jb = 0; jb < len; jb += kBlock) {
      const int nb = min(kBlock, len - jb);
      int vpage = -1;
      int vslot[TOKENS ? kTokRegs : 1];
      if constexpr (TOKENS) {
#pragma unroll
        for (int r = 0; r < kTokRegs; ++r) {
          vslot[r] = -1;
          const int tk = (p + jb) * 16 + 64 * r + lane;
          if (64 * r + lane < nb * 16 && tk < L) {
            if (tk >= a.table_stride) {
              err |= kErrBadIndexPos;
            } else {
              const int pos = b * a.table_stride + tk;  // below 2^31 (checked on the host)
              const int slot = a.slot_table ? a.slot_table[pos] : pos;
              if (slot < 0 || slot >= a.num_slots) err |= kErrBadPageId;
              else vslot[r] = slot;
            }
          }
        }
      } else {
        // One vector load fetches the page ids of the next (up to) 64 pages:
        // lane i holds the id of page p + jb + i, or -1 if it is unusable.
        const int pos = ip0 + p + jb + lane;
        const bool pos_ok = pos >= 0 && pos < a.num_indices;
        const int pid = pos_ok ? a.kv_indices[pos] : -1;
        if (lane < nb) {
          if (!pos_ok) err |= kErrBadIndexPos;
          else if (pid < 0 || pid >= a.num_pages) err |= kErrBadPageId;
          else vpage = pid;
        }
      }
      const int ns = TOKENS ? nb : nb << log2_s;  // steps in this block, >= 1

      // Step j of the block: page id (uniform) and loads.  Steps past the block
      // re-read its last step (a cache hit) and are never consumed, so the
      // issue sequence has no data-dependent branch.
      // Token of step j that was appended in this call (0..15), or -1.
      auto fresh_token = [&](int j) {
        const int t0 = (p + jb + (j >> log2_s)) * P + (j & ((1 << log2_s) - 1)) * 16;
        const int tok = L - 1 - t0;
        return fuse_append && j < ns && tok >= 0 && tok < 16 ? tok : -1;
      };
      auto issue_tokens = [&](int j, Step<D>& sd) {
        const int jc = j < ns ? j : ns - 1;
        const char* khead = kbase + (size_t)g * D * 2;
        const char* vhead = vbase + (size_t)g * D * 2;
        // The slot register of step jc (uniform choice), and its first lane.
        const int reg = jc >> 2;
        int vs = vslot[0];
#pragma unroll
        for (int r = 1; r < kTokRegs; ++r) vs = reg == r ? vslot[r] : vs;
        const int l0 = 16 * (jc & 3);
        // K: lane (g4, r16) reads channels 8 (4kk + g4) .. +8 of token r16.
        const int sk = __shfl(vs, l0 + r16, kWave);
        const char* kq = khead + (size_t)(sk < 0 ? 0 : sk) * slot_b + g4 * 16;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) sd.k[kk] = *reinterpret_cast<const uint4*>(kq + kk * 64);
        // V: lane (g4, r16) reads channels VB r16 .. VB r16 + VB - 1 of each of
        // tokens 4 g4 .. 4 g4 + 3 (one 2 VB-byte load per token; sd.v holds
        // token i's channels in its entries VB/4 i ..); consume() turns them
        // into the V^T operand with column r of block vb = channel VB r + vb.
        // An unusable slot reads slot 0 and gets keep byte 0 (its V is zeroed
        // in consume()).
        constexpr int VB = D / 16;
        int sv[4];
        uint32_t keep = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[i] = __shfl(vs, l0 + 4 * g4 + i, kWave);
          keep |= (sv[i] >= 0 ? 1u : 0u) << (8 * i);
          const char* vq = vhead + (size_t)(sv[i] < 0 ? 0 : sv[i]) * slot_b + r16 * (2 * VB);
          if constexpr (VB == 8) {
            const uint4 x = *reinterpret_cast<const uint4*>(vq);
            sd.v[2 * i] = make_uint2(x.x, x.y);
            sd.v[2 * i + 1] = make_uint2(x.z, x.w);
          } else {
            sd.v[i] = *reinterpret_cast<const uint2*>(vq);
          }
        }
        sd.keep = keep;
      };
      // Token-major V, as loaded, into the V^T operand: block vb takes half
      // vb % 2 of dword vb / 2 of each token's channels.
      auto transpose_tokens_v = [&](Step<D>& sd) {
        constexpr int VB = D / 16;
        constexpr int PER = VB / 2;  // dwords of one token's channels
        uint32_t wv[4][PER];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < PER; ++j) {
            const uint2 u = sd.v[i * PER / 2 + j / 2];
            wv[i][j] = (j & 1) ? u.y : u.x;
          }
        if (__builtin_amdgcn_ballot_w64(sd.keep != 0x01010101u) != 0) {
          // Some lane has a token without a usable slot (past the sequence
          // end, or a bad slot id): zero its V so that its zero weight gives
          // exactly zero.
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool ok = ((sd.keep >> (8 * i)) & 0xffu) != 0;
#pragma unroll
            for (int j = 0; j < PER; ++j) wv[i][j] = ok ? wv[i][j] : 0u;
          }
        }
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
          const int j = vb >> 1;
          if (vb & 1) {
            sd.v[vb] = make_uint2((wv[0][j] >> 16) | (wv[1][j] & 0xffff0000u),
                                  (wv[2][j] >> 16) | (wv[3][j] & 0xffff0000u));
          } else {
            sd.v[vb] = make_uint2((wv[0][j] & 0xffffu) | (wv[1][j] << 16),
                                  (wv[2][j] & 0xffffu) | (wv[3][j] << 16));
          }
        }
      };
      auto issue = [&](int j, Step<D>& sd) {
        if constexpr (TOKENS) {
          issue_tokens(j, sd);
          return;
        }
        const int jc = j < ns ? j : ns - 1;
        const int pg = jc >> log2_s;
        const int sub = jc & ((1 << log2_s) - 1);
        const int pid = __builtin_amdgcn_readlane(vpage, pg);
        const size_t base = (size_t)(pid < 0 ? 0 : pid) * a.num_kv_heads * tile_b + head_b;
        const char* kp = kbase + base + (size_t)sub * kStepBytes + k_boff;
        const char* vp = vbase + base + (size_t)sub * kStepBytes + v_boff;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
          sd.k[kk] = *reinterpret_cast<const uint4*>(kp + (size_t)kk * 4 * 16 * 16);
#pragma unroll
        for (int vb = 0; vb < D / 16; ++vb)
          sd.v[vb] = *reinterpret_cast<const uint2*>(vp + (size_t)vb * 16 * 16 * 2);
        if constexpr (MASKED) {
          // Keep bytes of this lane's four tokens; a row shorter than the
          // request reads 0 (dropped) past the end of the mask buffer.
          const int t0 = (p + jb + pg) * P + sub * 16 + 4 * g4;
          sd.keep = __builtin_amdgcn_raw_buffer_load_b32(mask_rs, mask_row + t0, 0, 0);
        }
      };
      auto consume = [&](int j, Step<D>& sd) {
        if constexpr (TOKENS) {
          const int t0 = (p + jb + j) * 16;
          transpose_tokens_v(sd);
          st.step(sd, min(16, max(0, L - t0)), g4, a.scale_log2, bias, sd.keep);
          return;
        }
        const int pg = j >> log2_s;
        const int sub = j & ((1 << log2_s) - 1);
        const int pid = __builtin_amdgcn_readlane(vpage, pg);
        const int t0 = (p + jb + pg) * P + sub * 16;
        const int live = pid < 0 ? 0 : min(16, max(0, L - t0));
        const int tok = fresh_token(j);
        if constexpr (MASKED) {
          st.step(sd, live, g4, a.scale_log2, bias, sd.keep);
          return;
        }
        if (!APPEND || tok < 0) {
          st.step(sd, live, g4, a.scale_log2, bias);
          return;
        }
        // The appended token replaces what the pool slot held (in place: the
        // ring slot is reloaded after this step).  K: the lanes of token tok
        // take chunk 4 kk + g4 of the row from the lane that fetched it.  V:
        // the lanes whose four tokens include it take their channel's value,
        // passed between lanes through this wave's LDS row.  The KV head's
        // first head group also marks the token for its pool write.
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
          const int src = 4 * kk + g4;
          uint4 x;
          x.x = (uint32_t)__shfl((int)knew4.x, src, kWave);
          x.y = (uint32_t)__shfl((int)knew4.y, src, kWave);
          x.z = (uint32_t)__shfl((int)knew4.z, src, kWave);
          x.w = (uint32_t)__shfl((int)knew4.w, src, kWave);
          if (r16 == tok) sd.k[kk] = x;
        }
        if (lane < D / 2) s_vn[w][lane] = vnew2;
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const uint16_t* vrow = reinterpret_cast<const uint16_t*>(&s_vn[w][0]);
        uint16_t vn[D / 16];
#pragma unroll
        for (int vb = 0; vb < D / 16; ++vb) vn[vb] = vrow[16 * vb + r16];
        const bool vlane = g4 == (tok >> 2);
        const int shift = (tok & 1) * 16;
        const uint32_t keep = ~(0xffffu << shift);
#pragma unroll
        for (int vb = 0; vb < D / 16; ++vb) {
          const uint32_t nv = (uint32_t)vn[vb] << shift;
          if (vlane) {
            if (tok & 2) sd.v[vb].y = (sd.v[vb].y & keep) | nv;
            else sd.v[vb].x = (sd.v[vb].x & keep) | nv;
          }
        }
        if (writer && pid >= 0) {
          pend_page = pid;
          pend_head = g;
          pend_sub = sub;
          pend_tok = tok;
        }
        st.step(sd, live, g4, a.scale_log2, bias);
      };

      // A ring of kStages steps: while one is consumed, kStages - 1 are in flight.
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

    // Close the piece: total sum of each head over its four lanes; lane (0, i)
    // then holds head i's max and sum, and lanes 0..15 hold its output rows.
    const float lt = sum_over_groups(st.l);
    const int seg = b * U + u;
    if (p == 0 && len == n) {
      // The whole segment lies in this wave: normalise its rows, transpose
      // them through LDS and write 8 channels (16 bytes) per lane.
#pragma unroll
      for (int i = 0; i < HG; ++i) {
        const float li = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lt), i));
        const float inv = li > 0.f ? 1.0f / li : 0.f;
        if (g4 == (i >> 2)) {  // head i: register i % 4 of lane group i / 4
#pragma unroll
          for (int vb = 0; vb < MfmaWave<D, HG>::VB; ++vb)
            s_acc[w][1][i][out_ch(vb)] = st.o[vb][i & 3] * inv;
        }
      }
      __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's LDS writes land first
#pragma unroll
      for (int e8 = 0; e8 < HG * (D / 8); e8 += kWave) {  // one pass when HG * D <= 512
        if (e8 + lane < HG * (D / 8)) {
          const int i = (e8 + lane) / (D / 8);
          const int c8 = (e8 + lane - i * (D / 8)) * 8;
          const float4 x0 = *reinterpret_cast<const float4*>(&s_acc[w][1][i][c8]);
          const float4 x1 = *reinterpret_cast<const float4*>(&s_acc[w][1][i][c8 + 4]);
          *reinterpret_cast<uint4*>(a.out + ((size_t)b * Hq + hq0 + i) * D + c8) =
              make_uint4(pack_bf16x2(x0.x, x0.y), pack_bf16x2(x0.z, x0.w),
                         pack_bf16x2(x1.x, x1.y), pack_bf16x2(x1.z, x1.w));
        }
      }
      __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before slot 1 is reused
    } else {
      const int slot = piece == 0 ? 0 : 1;
#pragma unroll
      for (int i = 0; i < HG; ++i) {
        if (g4 == (i >> 2)) {
#pragma unroll
          for (int vb = 0; vb < MfmaWave<D, HG>::VB; ++vb)
            s_acc[w][slot][i][out_ch(vb)] = st.o[vb][i & 3];
        }
        if (lane == i) {
          s_m[i][2 * w + slot] = st.m;
          s_l[i][2 * w + slot] = lt;
        }
      }
      if constexpr (PLAN) {
        if (lane == 0) s_seg[w][slot] = seg;
      }
    }
    left -= len;
    ++piece;
    if (left > 0) {
      p = 0;
      if (++u == U) {
        u = 0;
        do { ++b; } while (b < a.batch - 1 && indptr_at(b + 1) == indptr_at(b));
        ip0 = indptr_at(b);
        n = indptr_at(b + 1) - ip0;
        L = max(len_at(b), 0);
      }
    }
  }
  flush_token();
  if (grp == 0) zero_empty_rows();
  make_group_info();
  constexpr int NS = kSlots;
  SlotTable tab;
  if constexpr (!PLAN) {
    // The slot segments come with the plan: the table is built here, while
    // the workgroup's other waves may still stream.
    tab = make_slot_table(lane < NS ? slot_seg_l : -1, lane, grp, gi0);
  }
  __syncthreads();  // also publishes s_gi, s_seg and s_ptr
  const GroupInfo gi = s_gi;
  if constexpr (PLAN)
    tab = make_slot_table(lane < NS ? reinterpret_cast<const int*>(s_seg)[lane] : -1, lane, grp,
                          gi);
  float* const lse_p = uniform_ptr(s_ptr.lse);
  float* const opart_p = uniform_ptr(s_ptr.opart);
  int32_t* const counters_p = uniform_ptr(s_ptr.counters);
  if (err) atomicOr(&uniform_ptr(s_ptr.hdr)[kHdrError], err);
  // Fields of the record by a run-time slot index, as selects (an indexed
  // access would move the record to scratch memory).
  auto lo_of = [&](int k) { return k == 0 ? gi.lo[0] : gi.lo[1]; };
  auto hi_of = [&](int k) { return k == 0 ? gi.hi[0] : gi.hi[1]; };

  // Epilogue.  Outputs are handled as groups of four channels: thread t < kVec
  // owns channels 4 (t % (D / 4)) .. +3 of head t / (D / 4) of a segment.
  constexpr int kVec = HG * D / 4;
  constexpr int kVecPass = kWavesPerGroup * 16;  // output groups one merge pass covers
  constexpr int kVecPasses = (kVec + kVecPass - 1) / kVecPass;
  static_assert(kGroupThreads % 128 == 0, "thread quarters of 128");
  // Buffer resources of the partials (built where used: they occupy scalar
  // registers).
  auto lse_rsrc = [&]() {
    return __builtin_amdgcn_make_buffer_rsrc(lse_p, 0, (int)(sizeof(float) * 2 * HG * gridDim.x),
                                             kBufferWord3);
  };
  auto opart_rsrc = [&]() {
    return __builtin_amdgcn_make_buffer_rsrc(
        opart_p, 0, (int)(sizeof(float) * 2 * HG * D * gridDim.x), kBufferWord3);
  };

  // Merge the pieces in LDS segment by segment (a segment's pieces are the
  // valid slots between two changes of segment, in wave order).  A segment
  // inside this workgroup is written to the output; the first and the last
  // segment, if they reach other workgroups, leave a normalised partial and its
  // log-sum-exp.  Where each slot's segment goes is the same for every thread
  // (the slot table); each thread then folds the slots of its output element
  // in order with a running max, as the pieces themselves did.
  const uint32_t validm = tab.validm, endm = tab.endm, localm = tab.localm;
  const uint32_t kind1m = tab.kind1m, glob0m = tab.glob0m, glob1m = tab.kind1m;
  int segs[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) segs[k] = __builtin_amdgcn_readlane(tab.sk, k);
  // segments this workgroup leaves as partials (first, last)
  const int g0s = __builtin_amdgcn_readlane(tab.sk, glob0m ? __builtin_ctz(glob0m) : 0);
  const int g1s = __builtin_amdgcn_readlane(tab.sk, glob1m ? __builtin_ctz(glob1m) : 0);
  const int glob[2] = {glob0m ? g0s : -1, glob1m ? g1s : -1};
  // Thread t < HG * D / kCh folds channels c .. c + kCh - 1 of head h: four
  // channels for eight-head groups, else two (256 threads either way at
  // D = 128; measured: two for four heads, four for eight).
  constexpr int kCh = HG * D >= 1024 ? 4 : 2;
  static_assert(HG * D / kCh <= kGroupThreads, "one pass over the outputs");
  using ChVec = float __attribute__((ext_vector_type(kCh)));
  if (tid < HG * D / kCh) {
    const int e = kCh * tid;
    const int h = e / D;
    const int c = e - h * D;
    const __amdgpu_buffer_rsrc_t lse_rs = lse_rsrc(), opart_rs = opart_rsrc();
    // Every slot's max, sum and values are loaded up front (independent LDS
    // reads); slots without a segment are skipped.
    float mv[NS], lv[NS];
    ChVec xv[NS];
#pragma unroll
    for (int k4 = 0; k4 < NS; k4 += 4) {
      const float4 m4 = *reinterpret_cast<const float4*>(&s_m[h][k4]);
      const float4 l4 = *reinterpret_cast<const float4*>(&s_l[h][k4]);
      mv[k4] = m4.x, mv[k4 + 1] = m4.y, mv[k4 + 2] = m4.z, mv[k4 + 3] = m4.w;
      lv[k4] = l4.x, lv[k4 + 1] = l4.y, lv[k4 + 2] = l4.z, lv[k4 + 3] = l4.w;
    }
#pragma unroll
    for (int k = 0; k < NS; ++k)
      xv[k] = *reinterpret_cast<const ChVec*>(&s_acc[k >> 1][k & 1][h][c]);
    float M = kFloorMax, L = 0.f;
    ChVec acc = {};
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      if (!((validm >> k) & 1u)) continue;
      const float mn = vmax2(M, mv[k]);
      const float ca = fast_exp2(M - mn);
      const float cb = fast_exp2(mv[k] - mn);
      L = L * ca + lv[k] * cb;
#pragma unroll
      for (int j = 0; j < kCh; ++j) acc[j] = acc[j] * ca + xv[k][j] * cb;
      M = mn;
      if (!((endm >> k) & 1u)) continue;
      const bool live = L > 0.f;
      const float inv = live ? __builtin_amdgcn_rcpf(L) : 0.f;
      const int sk = segs[k];
      if ((localm >> k) & 1u) {
        const int eb = sk / U;
        const int row0 = eb * Hq + (sk - eb * U) * HG;
        uint32_t* dst = reinterpret_cast<uint32_t*>(a.out + (size_t)(row0 + h) * D + c);
        if constexpr (kCh == 4)
          *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(acc[0] * inv, acc[1] * inv),
                                                      pack_bf16x2(acc[2] * inv, acc[3] * inv));
        else
          *dst = pack_bf16x2(acc[0] * inv, acc[1] * inv);
      } else {
        const int row = (2 * grp + (int)((kind1m >> k) & 1u)) * HG + h;
        const int off = (row * D + c) * 4;
        if constexpr (kCh == 4)
          __builtin_amdgcn_raw_buffer_store_b128(
              u4v{__float_as_uint(acc[0] * inv), __float_as_uint(acc[1] * inv),
                  __float_as_uint(acc[2] * inv), __float_as_uint(acc[3] * inv)},
              opart_rs, off, 0, kCoherent);
        else
          __builtin_amdgcn_raw_buffer_store_b64(
              u2v{__float_as_uint(acc[0] * inv), __float_as_uint(acc[1] * inv)}, opart_rs, off, 0,
              kCoherent);
        if (c == 0)
          __builtin_amdgcn_raw_buffer_store_b32(
              __float_as_uint(live ? M + fast_log2(L) : kMinusInf), lse_rs, row * 4, 0, kCoherent);
      }
      M = kFloorMax;
      L = 0.f;
      acc = ChVec{};
    }
  }

  // Cross-workgroup merge: publish the partials, count arrivals, and let the
  // last workgroup of each segment combine every workgroup's partial in order.
  // Lanes 0 and 1 arrive for the first and the last segment at the same time.
  store_plan(true);
  wait_stores();
  __syncthreads();
  if (tid < 2) {
    const int k = tid;
    const int sgm = k == 0 ? glob[0] : glob[1];
    int merge = -1;
    if (sgm >= 0 && !(k == 1 && sgm == glob[0])) {
      // The last arrival of a call brings the counter to a multiple of the
      // contributor count n (the metadata build zeroes it).  That workgroup
      // takes n off again at once (no result needed), so the counter is back
      // at zero by the end of the call without a store at the end of the merge.
      const int n = hi_of(k) - lo_of(k) + 1;
      const int old = __hip_atomic_fetch_add(&counters_p[sgm], 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      if ((old + 1) % n == 0) {
        merge = sgm;
        __hip_atomic_fetch_add(&counters_p[sgm], -n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    s_merge[k] = merge;
  }
  __syncthreads();
  const int msg[2] = {s_merge[0], s_merge[1]};
  if (msg[0] < 0 && msg[1] < 0) return;  // uniform over the workgroup

  // Merge every segment this workgroup arrived last for.  Wave w merges output
  // groups 16 w .. 16 w + 15; the four 16-lane quarters of the wave take the
  // segment's workgroups in turn (quarter q: contributors q, q + 4, ...).  Every
  // load of a round is issued before any is used; a quarter issues loads only
  // for contributors that exist (the loads bypass the caches, so a repeated
  // load would cost a memory round trip of its own).  The quarters' results
  // are then combined across lanes (quarter pairs 0+1 and 2+3, then the two
  // pairs, lower first), so the result depends only on the plan and no
  // barrier is needed.
  constexpr int kQuarters = 4;
  // Output groups per lane: one pass covers 128 groups (a single pass when
  // HG * D <= 512); with more, one lane takes several groups and the loads of
  // all of them go out together (one round trip, not one per pass), with
  // proportionally fewer contributors per quarter and round.
  constexpr int NO = kVecPasses;
  constexpr int kPer = 8 / NO;  // contributors per quarter and segment in one round
  static_assert(kPer >= 1, "output groups per lane");
  const int q = lane >> 4;
  // Segment k's contributors are workgroups lo[k] .. hi[k] (none if not merged
  // here).  Workgroup j > lo holds the segment as its first segment (slot 0);
  // the first workgroup holds it in the slot the plan recorded.
  const int lo[2] = {msg[0] >= 0 ? gi.lo[0] : 0, msg[1] >= 0 ? gi.lo[1] : 0};
  const int hi[2] = {msg[0] >= 0 ? gi.hi[0] : -1, msg[1] >= 0 ? gi.hi[1] : -1};
  const int slot0[2] = {gi.slot_lo[0], gi.slot_lo[1]};
  const __amdgpu_buffer_rsrc_t lse_rs = lse_rsrc(), opart_rs = opart_rsrc();
  const int span = max(hi[0] - lo[0], hi[1] - lo[1]) + 1;
  const int rounds = (span + kQuarters * kPer - 1) / (kQuarters * kPer);
  int h[NO], c[NO];
  bool tact[NO];
#pragma unroll
  for (int og = 0; og < NO; ++og) {
    const int t = og * kVecPass + w * 16 + (lane & 15);
    tact[og] = t < kVec;
    h[og] = tact[og] ? t / (D / 4) : 0;
    c[og] = tact[og] ? (t - h[og] * (D / 4)) * 4 : 0;
  }
  Combine4 mc[2][NO];
#pragma unroll 1
  for (int rd = 0; rd < rounds; ++rd) {
    float ls[2][NO][kPer];
    f4 ov[2][NO][kPer];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int j = lo[k] + (rd * kPer + i) * kQuarters + q;
#pragma unroll
        for (int og = 0; og < NO; ++og) {
          ls[k][og][i] = kFloorMax;
          ov[k][og][i] = f4{0.f, 0.f, 0.f, 0.f};
        }
        if (j <= hi[k]) {  // uniform over a quarter
#pragma unroll
          for (int og = 0; og < NO; ++og) {
            const int row = (2 * j + (j == lo[k] ? slot0[k] : 0)) * HG + h[og];
            ls[k][og][i] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(lse_rs, row * 4, 0, kCoherent));
            ov[k][og][i] = __builtin_bit_cast(
                f4, __builtin_amdgcn_raw_buffer_load_b128(opart_rs, (row * D + c[og]) * 4, 0,
                                                          kCoherent));
          }
        }
      }
    }
    // This round's contributors: max first, then one exponential each.
#pragma unroll
    for (int k = 0; k < 2; ++k) {
#pragma unroll
      for (int og = 0; og < NO; ++og) {
        float mr = kFloorMax;
#pragma unroll
        for (int i = 0; i < kPer; ++i)
          if (lo[k] + (rd * kPer + i) * kQuarters + q <= hi[k]) mr = vmax2(mr, ls[k][og][i]);
        float den = 0.f;
        f4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          if (lo[k] + (rd * kPer + i) * kQuarters + q <= hi[k]) {
            const float wi = fast_exp2(ls[k][og][i] - mr);
            den += wi;
            num += ov[k][og][i] * wi;
          }
        }
        mc[k][og].add(mr, den, num);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (msg[k] < 0) continue;
#pragma unroll
    for (int og = 0; og < NO; ++og) {
      Combine4 x = mc[k][og];
#pragma unroll
      for (int off = 16; off <= 32; off <<= 1) {
        // Both lanes of the pair get (lower, upper) and add the upper to the lower.
        auto pr = [&](float v) { return off == 16 ? pair16(v) : pair32(v); };
        const LanePair m = pr(x.m), den = pr(x.den), nx = pr(x.num.x), ny = pr(x.num.y),
                       nz = pr(x.num.z), nw = pr(x.num.w);
        Combine4 r;
        r.m = m.lo;
        r.den = den.lo;
        r.num = f4{nx.lo, ny.lo, nz.lo, nw.lo};
        r.add(m.hi, den.hi, f4{nx.hi, ny.hi, nz.hi, nw.hi});
        x = r;
      }
      if (q == 0 && tact[og]) {
        const int eb = msg[k] / U;
        const int hq = (msg[k] - eb * U) * HG + h[og];
        const float inv = x.den > 0.f ? 1.0f / x.den : 0.f;
        const f4 val = x.num * inv;
        *reinterpret_cast<uint2*>(a.out + ((size_t)eb * Hq + hq) * D + c[og]) =
            make_uint2(pack_bf16x2(val.x, val.y), pack_bf16x2(val.z, val.w));
      }
    }
  }
}

template <int D, int KIND, bool PLAN>
hipError_t launch_d(const DecodeArgs& a, int hg, int groups, hipStream_t s) {
  const dim3 grid(groups), block(kGroupThreads);
  switch (hg) {
    case 1: hipLaunchKernelGGL((decode_kernel<D, 1, KIND, PLAN>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<D, 2, KIND, PLAN>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((decode_kernel<D, 3, KIND, PLAN>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_kernel<D, 4, KIND, PLAN>), grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL((decode_kernel<D, 5, KIND, PLAN>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((decode_kernel<D, 6, KIND, PLAN>), grid, block, 0, s, a); break;
    case 7: hipLaunchKernelGGL((decode_kernel<D, 7, KIND, PLAN>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_kernel<D, 8, KIND, PLAN>), grid, block, 0, s, a); break;
    case 12: hipLaunchKernelGGL((decode_kernel<D, 12, KIND, PLAN>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((decode_kernel<D, 16, KIND, PLAN>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_head_dim(const DecodeArgs& a, int hg, int groups, hipStream_t s) {
  if (a.token_major) return launch_d<D, kTokens, false>(a, hg, groups, s);
  if (a.k_new != nullptr) {
    return a.plan ? launch_d<D, kAppend, true>(a, hg, groups, s)
                  : launch_d<D, kAppend, false>(a, hg, groups, s);
  }
  if (a.mask != nullptr) return launch_d<D, kMasked, false>(a, hg, groups, s);
  return a.plan ? launch_d<D, kPlain, true>(a, hg, groups, s)
                : launch_d<D, kPlain, false>(a, hg, groups, s);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int head_dim, int hg, int groups, hipStream_t s) {
  if (groups <= 0) return hipSuccess;
  // Planning launches cover plain and fused-append decodes of at most
  // kPlanLdsRequests requests (the host checks).
  if (a.plan && (a.token_major || a.mask != nullptr || a.batch > kPlanLdsRequests))
    return hipErrorInvalidValue;
  if (head_dim == 128) return launch_head_dim<128>(a, hg, groups, s);
  if (head_dim == 64) return launch_head_dim<64>(a, hg, groups, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv
