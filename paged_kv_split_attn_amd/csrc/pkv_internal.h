// Internal definitions shared by the libpkv translation units: workspace
// layout, kernel argument blocks and launchers.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

constexpr int kWave = 64;
constexpr int kDefaultTargetItems = 2048;
constexpr int kDefaultMinChunkPages = 4;
constexpr int kMaxSplitsLimit = 4096;

// Header words at the start of the workspace (int32).
enum HeaderWord : int {
  kHdrNumItems = 0,    // (request, chunk) items planned this step
  kHdrChunk = 1,       // planned chunk length in pages (0 when splits are forced)
  kHdrTotalPages = 2,  // pages over the batch
  kHdrBatch = 3,       // batch of the last pkv_build_metadata
  kHdrError = 4,       // error bits latched by kernels since the last metadata build
  kHdrWords = 64
};

enum ErrorBit : int {
  kErrNegativeLength = 1,
  kErrBadPageId = 2,
  kErrBadIndexPos = 4,
};

// Byte offsets of the workspace sections; every section is 256-byte aligned.
struct WsLayout {
  int32_t max_items;  // (request, chunk) items the partial buffers hold
  size_t hdr, split_indptr, items, lse, opart, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Returns false for an invalid descriptor.
bool ws_layout(const pkv_desc& d, WsLayout* out);

// Resolved per-descriptor tuning values.
inline int target_items(const pkv_desc& d) {
  return d.target_items > 0 ? d.target_items : kDefaultTargetItems;
}
inline int min_chunk(const pkv_desc& d) {
  return d.min_chunk_pages > 0 ? d.min_chunk_pages : kDefaultMinChunkPages;
}

// Query heads one wave of the split kernel handles (the rest of a GQA group
// goes to sibling waves that read the same K/V tiles).
inline int heads_per_wave(int G) { return G <= 4 ? G : 4; }

struct MetaArgs {
  const int32_t* seq_lens;
  int32_t* kv_indptr;
  int32_t* hdr;
  int32_t* split_indptr;
  int2* items;
  int32_t batch, page_size, num_kv_heads, max_splits, target_items, min_chunk, forced, max_items;
};

struct AppendArgs {
  uint16_t* k;
  uint16_t* v;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* seq_lens;
  int32_t num_indices, num_pages, page_size, num_kv_heads, head_dim, batch;
};

struct DecodeArgs {
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* q;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* seq_lens;
  int32_t* hdr;
  const int32_t* split_indptr;
  const int2* items;
  float* lse;    // [max_items][Hq], log2-domain log-sum-exp of each chunk
  float* opart;  // [max_items][Hq][D], normalised chunk outputs
  uint16_t* out; // [batch][Hq][D] bf16
  int32_t num_indices, num_pages, num_q_heads, num_kv_heads, page_size, batch;
  int32_t max_items;    // capacity of the partial buffers, in (request, chunk) items
  int32_t log2_rounds;  // log2(page_size / tokens per round); tokens per round = 1024 / head_dim
  float scale_log2;     // sm_scale * log2(e)
};

hipError_t launch_metadata(const MetaArgs& a, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_split(const DecodeArgs& a, int head_dim, int heads_per_wave, int max_items,
                        hipStream_t s);
hipError_t launch_merge(const DecodeArgs& a, int head_dim, hipStream_t s);

}  // namespace pkv
