// Internal definitions shared by the libpkv translation units: workspace
// layout, kernel argument blocks and launchers.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

constexpr int kWave = 64;
constexpr int kWavesPerGroup = PKV_WAVES_PER_WORKGROUP;  // waves of one decode workgroup (two per SIMD)
constexpr int kGroupThreads = kWavesPerGroup * kWave;  // 512
constexpr int kXcds = 8;  // accelerator dies of the chip, each with its own L2
constexpr int kPrefillTiles = 1;  // 16-row tiles per prefill wave (2 measured slower: fewer, longer workgroups)
constexpr int kPrefillWaves = 8;  // waves of a prefill workgroup (they share each K/V chunk)
constexpr int kPrefillSteps = 1;  // 32-key steps per prefill K/V chunk (two measured slower)
constexpr int kDefaultMinTiles = 16;  // fewer tiles per workgroup measured slower on small batches
constexpr int kMaxBatch = 65536;
constexpr int kMaxGroups = 65536;
constexpr int kMetaLdsRequests = 8192;  // kv_indptr entries the metadata kernel keeps in LDS
// Largest batch a decode that plans its own step handles in one launch (its
// prefix sums and lengths live in LDS next to the decode's own buffers).
constexpr int kPlanLdsRequests = 1024;

// Header words at the start of the workspace (int32).
enum HeaderWord : int {
  kHdrGroups = 0,      // workgroups the plan uses (W)
  kHdrTiles = 1,       // tiles T = pages * head groups
  kHdrUnits = 2,       // head groups per request (U)
  kHdrBatch = 3,       // batch of the last pkv_build_metadata
  kHdrError = 4,       // error bits latched since the last metadata build
  kHdrEmpty = 5,       // requests without tokens (their output rows are zeroed)
  kHdrWords = 64
};

enum ErrorBit : int {
  kErrNegativeLength = 1,
  kErrBadPageId = 2,
  kErrBadIndexPos = 4,
  kErrPlanMismatch = 8,  // a decode got a plan built for another batch or head grouping
};

// Range of one wave: tiles of request b, head group u, pages p, p+1, ... and
// on into the following (request, head group) segments, `count` tiles in all.
// The rest describes request b, so the wave can start loading at once.
struct alignas(16) WaveRange {
  int32_t b, u, p, count;
  int32_t ip0;    // kv_indptr[b]
  int32_t pages;  // pages of request b
  int32_t len;    // tokens of request b
  int32_t pad;
};

// What a workgroup needs for its merges, prepared by the metadata kernel so
// the decode reads it in one load at its start.  A segment is one (request,
// head group); only the first and the last segment of a workgroup's tile range
// can extend into other workgroups.
struct alignas(16) GroupInfo {
  int32_t seg[2];      // first and last segment of the range (-1: no range)
  int32_t lo[2];       // first workgroup whose range touches seg[k]
  int32_t hi[2];       // last workgroup whose range touches seg[k]
  int32_t slot_lo[2];  // partial slot (0 = first segment, 1 = last) seg[k] has in workgroup lo[k]
  // Segment of each wave's partial first (slot 2w) and last (slot 2w + 1)
  // piece, -1 when that piece is a whole segment or absent: the table the
  // in-workgroup merge works from, known from the plan before any K/V is read.
  int32_t slot_seg[2 * kWavesPerGroup];
};

// Byte offsets of the workspace sections; every section is 256-byte aligned.
struct WsLayout {
  int32_t groups;    // decode grid size (workgroups)
  int32_t segments;  // max_batch * U
  size_t hdr, waves, ginfo, counters, lse, opart, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Query heads one decode head group covers: the largest size the decode is
// built for (1 .. 8, 12, 16) that divides G (G >= 1) -- the whole GQA group
// up to eight heads.  One 16-row matrix-core tile holds up to sixteen.  The
// rest of a larger group goes to sibling head groups that read the same K/V
// tiles again, so the largest divisor means the fewest passes over each KV
// head.
inline int heads_per_group(int G) {
  constexpr int kBuilt[] = {16, 12, 8, 7, 6, 5, 4, 3, 2};
  for (int h : kBuilt)
    if (G % h == 0) return h;
  return 1;
}
// Query heads of one prefill row tile (16 rows hold 16 / HG tokens x HG
// heads): the whole group up to seven heads, else four when four divide G
// (every row of the tile used), else the largest size up to seven that does.
inline int prefill_heads_per_group(int G) {
  if (G <= 7) return G;
  if (G % 4 == 0) return 4;
  for (int h = 7; h > 1; --h)
    if (G % h == 0) return h;
  return 1;
}

// Returns false for an invalid descriptor; `groups` is the resolved grid size.
bool ws_layout(const pkv_desc& d, int groups, WsLayout* out);

struct MetaArgs {
  const int32_t* seq_lens;
  int32_t* kv_indptr;
  int32_t* hdr;
  WaveRange* waves;    // [groups * kWavesPerGroup]
  GroupInfo* ginfo;    // [groups]
  int32_t* counters;   // [segments]: arrivals for the cross-workgroup merge
  int32_t batch, page_size, units, groups, min_tiles, forced;
  int32_t segments;    // counters of the descriptor (max_batch * units), all cleared
};

struct AppendArgs {
  uint16_t* k;
  uint16_t* v;
  const uint16_t* k_new;     // [batch][Hkv][D], or [rows][Hkv][D] with qo_indptr
  const uint16_t* v_new;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* seq_lens;
  int32_t num_indices, num_pages, page_size, num_kv_heads, head_dim, batch;
  // Several new tokens per request (extend): rows qo_indptr[b] .. qo_indptr[b+1]
  // of k_new / v_new, at most max_rows per request, in blocks of 16 rows.
  const int32_t* qo_indptr;
  int32_t max_rows, row_blocks;
};

struct DecodeArgs {
  uint16_t* k;              // written only by a fused append
  uint16_t* v;
  const uint16_t* k_new;    // [batch][Hkv][D] token to append, or null (no append)
  const uint16_t* v_new;
  const uint8_t* mask;      // [batch][mask_stride] keep bytes, or null (no mask)
  int32_t mask_stride;
  const uint16_t* q;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* seq_lens;
  int32_t* hdr;
  const WaveRange* waves;
  const GroupInfo* ginfo;
  int32_t* counters;
  float* lse;     // [2 * groups][HG], log2-domain log-sum-exp of workgroup partials
  float* opart;   // [2 * groups][HG][D], normalised workgroup partials
  uint16_t* out;  // [batch][Hq][D] bf16
  int32_t num_indices, num_pages, num_q_heads, num_kv_heads, page_size, batch;
  int32_t units;        // head groups per request
  int32_t log2_steps;   // log2(page_size / 16): steps of 16 tokens per page
  float scale_log2;     // sm_scale * log2(e)
  // Token-major K/V (k, v are [num_slots][Hkv][D]; the plan's pages are
  // 16-token blocks): slot of token t of request b = slot_table[b * stride + t],
  // or b * stride + t without a table.
  int32_t token_major;
  const int32_t* slot_table;
  int32_t table_stride;
  int32_t num_slots;
  // Planning inside the launch (plan != 0, batch <= kPlanLdsRequests): every
  // workgroup computes the step's plan from seq_lens in LDS, uses it at once
  // and writes its own part of it (waves, ginfo; workgroup 0 also kv_indptr
  // and the header) for the calls that follow in the step.
  int32_t plan;
  int32_t groups, min_tiles, forced;
  int32_t* plan_indptr;
  WaveRange* plan_waves;
  GroupInfo* plan_ginfo;
};

struct PrefillArgs {
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* q;          // [total_q][Hq][D] bf16
  const int32_t* qo_indptr;   // [batch + 1] query-row offsets
  const int32_t* kv_indptr;   // [batch + 1] page prefix sums
  const int32_t* kv_indices;
  const int32_t* seq_lens;    // KV tokens per request (new tokens included)
  uint16_t* out;              // [total_q][Hq][D] bf16
  int32_t num_indices, num_pages, num_q_heads, num_kv_heads, page_size, batch;
  int32_t causal;
  int32_t log2_steps;
  float scale_log2;
};

hipError_t launch_metadata(const MetaArgs& a, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_append_rows(const AppendArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int head_dim, int heads_per_group, int groups,
                         hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int heads_per_group, int max_q_len,
                          hipStream_t s);

}  // namespace pkv
