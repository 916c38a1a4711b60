// C ABI of libpkv: host-side argument checks, workspace layout and launches.
// Nothing here allocates device memory, synchronises or reads device memory,
// except pkv_debug_validate, which is documented as syncing.
#include <string.h>

#include <atomic>
#include <vector>

#include "pkv_internal.h"

namespace pkv {

bool ws_layout(const pkv_desc& d, int groups, WsLayout* out) {
  if (d.max_batch < 1 || d.max_batch > kMaxBatch || d.num_q_heads < 1 || d.num_kv_heads < 1 ||
      d.head_dim < 1 || d.page_size < 1 || d.num_workgroups < 0 ||
      d.num_workgroups > kMaxGroups || d.min_tiles_per_group < 0 || d.reserved != 0 ||
      d.num_q_heads % d.num_kv_heads != 0 || groups < 1 || groups > kMaxGroups)
    return false;
  const int hg = heads_per_group(d.num_q_heads / d.num_kv_heads);
  if (d.num_q_heads % hg != 0) return false;
  WsLayout L;
  L.groups = groups;
  L.segments = d.max_batch * (d.num_q_heads / hg);
  size_t off = 0;
  L.hdr = off;
  off = align256(off + sizeof(int32_t) * kHdrWords);
  L.waves = off;
  off = align256(off + sizeof(WaveRange) * (size_t)groups * kWavesPerGroup);
  L.ginfo = off;
  off = align256(off + sizeof(GroupInfo) * (size_t)groups);
  L.counters = off;
  off = align256(off + sizeof(int32_t) * (size_t)L.segments);
  L.lse = off;
  off = align256(off + sizeof(float) * (size_t)2 * groups * hg);
  L.opart = off;
  off = align256(off + sizeof(float) * (size_t)2 * groups * hg * d.head_dim);
  L.total = off;
  *out = L;
  return true;
}

namespace {

// Shapes the kernels are compiled for.
bool supported(int head_dim, int page_size, int G) {
  if (head_dim != 64 && head_dim != 128) return false;
  // A wave consumes 16 tokens of one page per step.
  if (page_size < 16 || (page_size & (page_size - 1)) != 0) return false;
  if (G < 1) return false;
  return true;
}

int log2i(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

// Decode grid size: the descriptor's, or one workgroup per compute unit.
int resolve_groups(const pkv_desc& d) {
  if (d.num_workgroups > 0) return d.num_workgroups;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus;
}

int check_desc(const pkv_desc* d, WsLayout* L) {
  if (!d) return PKV_ERR_INVALID_ARG;
  if (d->num_kv_heads > 0 && d->num_q_heads > 0 && d->num_q_heads % d->num_kv_heads == 0 &&
      !supported(d->head_dim, d->page_size, d->num_q_heads / d->num_kv_heads))
    return PKV_ERR_UNSUPPORTED;
  if (!ws_layout(*d, resolve_groups(*d), L)) return PKV_ERR_INVALID_ARG;
  return PKV_OK;
}

int check_pool(const pkv_pool* p, const pkv_desc* d) {
  if (!p || !p->k || !p->v || p->num_pages < 1) return PKV_ERR_INVALID_ARG;
  if (d && (p->page_size != d->page_size || p->num_kv_heads != d->num_kv_heads ||
            p->head_dim != d->head_dim))
    return PKV_ERR_INVALID_ARG;
  return PKV_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH; }

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" {

const char* pkv_status_str(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape (head_dim, page_size or group size)";
    case PKV_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PKV_ERR_CAPACITY: return "batch above the descriptor's capacity";
    case PKV_ERR_LAUNCH: return "kernel launch failed";
    case PKV_ERR_DEVICE_DATA: return "invalid device metadata";
    case PKV_ERR_SCRATCH_TOO_SMALL:
      return "the descriptor needs more workspace than the library's static scratch holds";
    default: return "unknown status";
  }
}

int32_t pkv_version(void) { return (2 << 16) | 6; }

size_t pkv_workspace_bytes(const pkv_desc* desc) {
  WsLayout L;
  if (check_desc(desc, &L) != PKV_OK) return 0;
  return L.total;
}

int pkv_build_metadata(const pkv_desc* desc, const int32_t* seq_lens, int32_t batch,
                       int32_t forced_groups, int32_t* kv_indptr, void* workspace,
                       size_t workspace_bytes, void* stream) {
  WsLayout L;
  int st = check_desc(desc, &L);
  if (st != PKV_OK) return st;
  if (!seq_lens || !kv_indptr || !workspace || batch < 0 || forced_groups < 0)
    return PKV_ERR_INVALID_ARG;
  if (batch > desc->max_batch) return PKV_ERR_CAPACITY;
  if (workspace_bytes < L.total) return PKV_ERR_WORKSPACE_TOO_SMALL;
  MetaArgs a;
  a.seq_lens = seq_lens;
  a.kv_indptr = kv_indptr;
  a.hdr = at<int32_t>(workspace, L.hdr);
  a.waves = at<WaveRange>(workspace, L.waves);
  a.ginfo = at<GroupInfo>(workspace, L.ginfo);
  a.counters = at<int32_t>(workspace, L.counters);
  a.batch = batch;
  a.page_size = desc->page_size;
  a.units = desc->num_q_heads / heads_per_group(desc->num_q_heads / desc->num_kv_heads);
  a.groups = L.groups;
  a.min_tiles = desc->min_tiles_per_group > 0 ? desc->min_tiles_per_group : kDefaultMinTiles;
  a.forced = forced_groups;
  a.segments = L.segments;
  return launch_status(launch_metadata(a, static_cast<hipStream_t>(stream)));
}

int pkv_append_kv(const pkv_pool* pool, const void* k_new, const void* v_new,
                  const int32_t* kv_indptr, const int32_t* kv_indices, int32_t num_indices,
                  const int32_t* seq_lens, int32_t batch, void* stream) {
  int st = check_pool(pool, nullptr);
  if (st != PKV_OK) return st;
  if (!k_new || !v_new || !kv_indptr || (num_indices > 0 && !kv_indices) || !seq_lens || batch < 0 ||
      num_indices < 0 || pool->page_size < 1 || pool->num_kv_heads < 1)
    return PKV_ERR_INVALID_ARG;
  if (pool->head_dim != 64 && pool->head_dim != 128) return PKV_ERR_UNSUPPORTED;
  // One thread per 8 channels of every K and V row; the kernel indexes in 32 bits.
  if ((long long)batch * pool->num_kv_heads * 2 * (pool->head_dim / 8) > 0x7fffffffLL)
    return PKV_ERR_INVALID_ARG;
  AppendArgs a{};
  a.k = static_cast<uint16_t*>(pool->k);
  a.v = static_cast<uint16_t*>(pool->v);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.kv_indptr = kv_indptr;
  a.kv_indices = kv_indices;
  a.seq_lens = seq_lens;
  a.num_indices = num_indices;
  a.num_pages = pool->num_pages;
  a.page_size = pool->page_size;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.batch = batch;
  return launch_status(launch_append(a, static_cast<hipStream_t>(stream)));
}

int pkv_append_kv_ragged(const pkv_pool* pool, const void* k_new, const void* v_new,
                         const int32_t* qo_indptr, const int32_t* kv_indptr,
                         const int32_t* kv_indices, int32_t num_indices, const int32_t* seq_lens,
                         int32_t batch, int32_t max_new_rows, void* stream) {
  int st = check_pool(pool, nullptr);
  if (st != PKV_OK) return st;
  if (!k_new || !v_new || !qo_indptr || !kv_indptr || (num_indices > 0 && !kv_indices) ||
      !seq_lens || batch < 0 || num_indices < 0 || max_new_rows < 0 || pool->page_size < 1 ||
      pool->num_kv_heads < 1)
    return PKV_ERR_INVALID_ARG;
  if (pool->head_dim != 64 && pool->head_dim != 128) return PKV_ERR_UNSUPPORTED;
  const int row_blocks = (max_new_rows + 15) / 16;
  // One workgroup per 16 rows of a (request, KV head); the grid is one dimension.
  if ((long long)batch * pool->num_kv_heads * row_blocks > 0x7fffffffLL) return PKV_ERR_CAPACITY;
  AppendArgs a{};
  a.k = static_cast<uint16_t*>(pool->k);
  a.v = static_cast<uint16_t*>(pool->v);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.kv_indptr = kv_indptr;
  a.kv_indices = kv_indices;
  a.seq_lens = seq_lens;
  a.num_indices = num_indices;
  a.num_pages = pool->num_pages;
  a.page_size = pool->page_size;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.batch = batch;
  a.qo_indptr = qo_indptr;
  a.max_rows = max_new_rows;
  a.row_blocks = row_blocks;
  return launch_status(launch_append_rows(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Checks of pkv_decode / pkv_decode_append / pkv_decode_masked /
// pkv_decode_plan and the launch arguments they share (the plan fields are
// left off).
int prepare_decode(const pkv_pool* pool, const pkv_desc* desc, const void* q, const void* k_new,
                   const void* v_new, const uint8_t* mask, int32_t mask_stride,
                   const int32_t* kv_indptr, const int32_t* kv_indices, int32_t num_indices,
                   const int32_t* seq_lens, int32_t batch, float sm_scale, void* workspace,
                   size_t workspace_bytes, void* out, WsLayout* Lp, int* hg_out, DecodeArgs* dp) {
  WsLayout& L = *Lp;
  int st = check_desc(desc, &L);
  if (st != PKV_OK) return st;
  st = check_pool(pool, desc);
  if (st != PKV_OK) return st;
  if (!q || !kv_indptr || (num_indices > 0 && !kv_indices) || !seq_lens || !workspace || !out ||
      batch < 0 ||
      num_indices < 0 || !(sm_scale == sm_scale) || (k_new == nullptr) != (v_new == nullptr))
    return PKV_ERR_INVALID_ARG;
  if (batch > desc->max_batch) return PKV_ERR_CAPACITY;
  if (workspace_bytes < L.total) return PKV_ERR_WORKSPACE_TOO_SMALL;
  if (mask && (mask_stride < 0 || mask_stride % 4 != 0 ||
               (long long)mask_stride * batch > 0x7fffffffLL))
    return PKV_ERR_INVALID_ARG;
  DecodeArgs d{};
  d.mask = mask;
  d.mask_stride = mask ? mask_stride : 0;
  d.k = static_cast<uint16_t*>(pool->k);
  d.v = static_cast<uint16_t*>(pool->v);
  d.k_new = static_cast<const uint16_t*>(k_new);
  d.v_new = static_cast<const uint16_t*>(v_new);
  d.q = static_cast<const uint16_t*>(q);
  d.kv_indptr = kv_indptr;
  d.kv_indices = kv_indices;
  d.seq_lens = seq_lens;
  d.hdr = at<int32_t>(workspace, L.hdr);
  d.waves = at<WaveRange>(workspace, L.waves);
  d.ginfo = at<GroupInfo>(workspace, L.ginfo);
  d.counters = at<int32_t>(workspace, L.counters);
  d.lse = at<float>(workspace, L.lse);
  d.opart = at<float>(workspace, L.opart);
  d.out = static_cast<uint16_t*>(out);
  d.num_indices = num_indices;
  d.num_pages = pool->num_pages;
  d.num_q_heads = desc->num_q_heads;
  d.num_kv_heads = desc->num_kv_heads;
  d.page_size = desc->page_size;
  d.batch = batch;
  const int hg = heads_per_group(desc->num_q_heads / desc->num_kv_heads);
  d.units = desc->num_q_heads / hg;
  d.log2_steps = log2i(desc->page_size / 16);
  d.scale_log2 = sm_scale * 1.4426950408889634f;
  d.token_major = 0;
  d.slot_table = nullptr;
  d.table_stride = 0;
  d.num_slots = 0;
  d.plan = 0;
  *hg_out = hg;
  *dp = d;
  return PKV_OK;
}

// pkv_decode and pkv_decode_append: the same launch, with or without the
// token to append.
int decode_impl(const pkv_pool* pool, const pkv_desc* desc, const void* q, const void* k_new,
                const void* v_new, const uint8_t* mask, int32_t mask_stride,
                const int32_t* kv_indptr, const int32_t* kv_indices, int32_t num_indices,
                const int32_t* seq_lens, int32_t batch, float sm_scale, void* workspace,
                size_t workspace_bytes, void* out, void* stream) {
  WsLayout L;
  DecodeArgs d;
  int hg = 0;
  const int st = prepare_decode(pool, desc, q, k_new, v_new, mask, mask_stride, kv_indptr,
                                kv_indices, num_indices, seq_lens, batch, sm_scale, workspace,
                                workspace_bytes, out, &L, &hg, &d);
  if (st != PKV_OK) return st;
  if (batch == 0) return PKV_OK;
  return launch_status(
      launch_decode(d, desc->head_dim, hg, L.groups, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int pkv_decode(const pkv_pool* pool, const pkv_desc* desc, const void* q,
               const int32_t* kv_indptr, const int32_t* kv_indices, int32_t num_indices,
               const int32_t* seq_lens, int32_t batch, float sm_scale, void* workspace,
               size_t workspace_bytes, void* out, void* stream) {
  return decode_impl(pool, desc, q, nullptr, nullptr, nullptr, 0, kv_indptr, kv_indices,
                     num_indices, seq_lens, batch, sm_scale, workspace, workspace_bytes, out,
                     stream);
}

int pkv_decode_masked(const pkv_pool* pool, const pkv_desc* desc, const void* q,
                      const uint8_t* mask, int32_t mask_stride, const int32_t* kv_indptr,
                      const int32_t* kv_indices, int32_t num_indices, const int32_t* seq_lens,
                      int32_t batch, float sm_scale, void* workspace, size_t workspace_bytes,
                      void* out, void* stream) {
  if (!mask) return PKV_ERR_INVALID_ARG;
  return decode_impl(pool, desc, q, nullptr, nullptr, mask, mask_stride, kv_indptr, kv_indices,
                     num_indices, seq_lens, batch, sm_scale, workspace, workspace_bytes, out,
                     stream);
}

int pkv_decode_append(const pkv_pool* pool, const pkv_desc* desc, const void* q,
                      const void* k_new, const void* v_new, const int32_t* kv_indptr,
                      const int32_t* kv_indices, int32_t num_indices, const int32_t* seq_lens,
                      int32_t batch, float sm_scale, void* workspace, size_t workspace_bytes,
                      void* out, void* stream) {
  if (!k_new || !v_new) return PKV_ERR_INVALID_ARG;
  return decode_impl(pool, desc, q, k_new, v_new, nullptr, 0, kv_indptr, kv_indices, num_indices,
                     seq_lens, batch, sm_scale, workspace, workspace_bytes, out, stream);
}

int pkv_decode_plan(const pkv_pool* pool, const pkv_desc* desc, const void* q,
                    const void* k_new, const void* v_new, const int32_t* seq_lens, int32_t batch,
                    int32_t forced_groups, int32_t* kv_indptr, const int32_t* kv_indices,
                    int32_t num_indices, float sm_scale, void* workspace, size_t workspace_bytes,
                    void* out, void* stream) {
  WsLayout L;
  DecodeArgs d;
  int hg = 0;
  if (forced_groups < 0) return PKV_ERR_INVALID_ARG;
  int st = prepare_decode(pool, desc, q, k_new, v_new, nullptr, 0, kv_indptr, kv_indices,
                          num_indices, seq_lens, batch, sm_scale, workspace, workspace_bytes, out,
                          &L, &hg, &d);
  if (st != PKV_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (batch == 0 || batch > kPlanLdsRequests) {
    // No request, or more than the planning launch keeps in LDS: the metadata
    // kernel plans, then the decode runs on its plan (the same results).
    st = pkv_build_metadata(desc, seq_lens, batch, forced_groups, kv_indptr, workspace,
                            workspace_bytes, stream);
    if (st != PKV_OK || batch == 0) return st;
    return launch_status(launch_decode(d, desc->head_dim, hg, L.groups, s));
  }
  d.plan = 1;
  d.groups = L.groups;
  d.min_tiles = desc->min_tiles_per_group > 0 ? desc->min_tiles_per_group : kDefaultMinTiles;
  d.forced = forced_groups;
  d.plan_indptr = kv_indptr;
  d.plan_waves = at<WaveRange>(workspace, L.waves);
  d.plan_ginfo = at<GroupInfo>(workspace, L.ginfo);
  return launch_status(launch_decode(d, desc->head_dim, hg, L.groups, s));
}

int pkv_decode_tokens(const pkv_desc* desc, const void* k_cache, const void* v_cache,
                      int32_t num_slots, const int32_t* slot_table, int32_t table_stride,
                      const void* q, const int32_t* kv_indptr, const int32_t* seq_lens,
                      int32_t batch, float sm_scale, void* workspace, size_t workspace_bytes,
                      void* out, void* stream) {
  WsLayout L;
  int st = check_desc(desc, &L);
  if (st != PKV_OK) return st;
  if (desc->page_size != 16) return PKV_ERR_INVALID_ARG;
  if (!k_cache || !v_cache || !q || !kv_indptr || !seq_lens || !workspace || !out || batch < 0 ||
      num_slots < 1 || table_stride < 0 || !(sm_scale == sm_scale))
    return PKV_ERR_INVALID_ARG;
  if (batch > desc->max_batch) return PKV_ERR_CAPACITY;
  if ((long long)batch * table_stride > INT32_MAX) return PKV_ERR_CAPACITY;
  if (!slot_table && (long long)batch * table_stride > num_slots) return PKV_ERR_INVALID_ARG;
  if (workspace_bytes < L.total) return PKV_ERR_WORKSPACE_TOO_SMALL;
  if (batch == 0) return PKV_OK;
  DecodeArgs d{};
  d.k = static_cast<uint16_t*>(const_cast<void*>(k_cache));  // read only: no append here
  d.v = static_cast<uint16_t*>(const_cast<void*>(v_cache));
  d.q = static_cast<const uint16_t*>(q);
  d.kv_indptr = kv_indptr;
  d.seq_lens = seq_lens;
  d.hdr = at<int32_t>(workspace, L.hdr);
  d.waves = at<WaveRange>(workspace, L.waves);
  d.ginfo = at<GroupInfo>(workspace, L.ginfo);
  d.counters = at<int32_t>(workspace, L.counters);
  d.lse = at<float>(workspace, L.lse);
  d.opart = at<float>(workspace, L.opart);
  d.out = static_cast<uint16_t*>(out);
  d.num_q_heads = desc->num_q_heads;
  d.num_kv_heads = desc->num_kv_heads;
  d.page_size = 16;
  d.batch = batch;
  const int hg = heads_per_group(desc->num_q_heads / desc->num_kv_heads);
  d.units = desc->num_q_heads / hg;
  d.log2_steps = 0;
  d.scale_log2 = sm_scale * 1.4426950408889634f;
  d.token_major = 1;
  d.slot_table = slot_table;
  d.table_stride = table_stride;
  d.num_slots = num_slots;
  return launch_status(
      launch_decode(d, desc->head_dim, hg, L.groups, static_cast<hipStream_t>(stream)));
}

int pkv_prefill(const pkv_pool* pool, const pkv_desc* desc, const void* q,
                const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                int32_t num_indices, const int32_t* seq_lens, int32_t batch, int32_t max_q_len,
                int32_t causal, float sm_scale, void* out, void* stream) {
  WsLayout L;
  int st = check_desc(desc, &L);
  if (st != PKV_OK) return st;
  st = check_pool(pool, desc);
  if (st != PKV_OK) return st;
  if (!q || !qo_indptr || !kv_indptr || (num_indices > 0 && !kv_indices) || !seq_lens || !out ||
      batch < 0 || num_indices < 0 || max_q_len < 0 || !(sm_scale == sm_scale))
    return PKV_ERR_INVALID_ARG;
  if (batch > desc->max_batch || batch > 65535) return PKV_ERR_CAPACITY;
  if (batch == 0 || max_q_len == 0) return PKV_OK;
  const int hg = prefill_heads_per_group(desc->num_q_heads / desc->num_kv_heads);
  const long long per_group = 16 / hg * kPrefillTiles * kPrefillWaves;  // query tokens of one workgroup
  if ((max_q_len + per_group - 1) / per_group * (desc->num_q_heads / hg) * batch > INT32_MAX)
    return PKV_ERR_CAPACITY;
  PrefillArgs a;
  a.k = static_cast<const uint16_t*>(pool->k);
  a.v = static_cast<const uint16_t*>(pool->v);
  a.q = static_cast<const uint16_t*>(q);
  a.qo_indptr = qo_indptr;
  a.kv_indptr = kv_indptr;
  a.kv_indices = kv_indices;
  a.seq_lens = seq_lens;
  a.out = static_cast<uint16_t*>(out);
  a.num_indices = num_indices;
  a.num_pages = pool->num_pages;
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = desc->num_kv_heads;
  a.page_size = desc->page_size;
  a.batch = batch;
  a.causal = causal != 0;
  a.log2_steps = log2i(desc->page_size / 16);
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  return launch_status(launch_prefill(a, desc->head_dim, hg, max_q_len,
                                      static_cast<hipStream_t>(stream)));
}

int pkv_debug_validate(const pkv_desc* desc, const int32_t* seq_lens, const int32_t* kv_indptr,
                       const int32_t* kv_indices, int32_t num_indices, int32_t num_pages,
                       int32_t batch, void* workspace, size_t workspace_bytes,
                       int32_t* groups_out, int32_t* waves_out, void* stream) {
  WsLayout L;
  int st = check_desc(desc, &L);
  if (st != PKV_OK) return st;
  if (!seq_lens || !kv_indptr || !workspace || batch < 0 || num_indices < 0 ||
      (num_indices > 0 && !kv_indices))
    return PKV_ERR_INVALID_ARG;
  if (batch > desc->max_batch) return PKV_ERR_CAPACITY;
  if (workspace_bytes < L.total) return PKV_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<int32_t> sl(batch), ip(batch + 1), hdr(kHdrWords), idx(num_indices);
  bool ok = hipMemcpyAsync(sl.data(), seq_lens, sizeof(int32_t) * batch, hipMemcpyDeviceToHost,
                           s) == hipSuccess;
  ok &= hipMemcpyAsync(ip.data(), kv_indptr, sizeof(int32_t) * (batch + 1),
                       hipMemcpyDeviceToHost, s) == hipSuccess;
  ok &= hipMemcpyAsync(hdr.data(), at<int32_t>(workspace, L.hdr), sizeof(int32_t) * kHdrWords,
                       hipMemcpyDeviceToHost, s) == hipSuccess;
  if (num_indices > 0)
    ok &= hipMemcpyAsync(idx.data(), kv_indices, sizeof(int32_t) * num_indices,
                         hipMemcpyDeviceToHost, s) == hipSuccess;
  std::vector<WaveRange> waves(waves_out ? (size_t)L.groups * kWavesPerGroup : 0);
  if (waves_out)
    ok &= hipMemcpyAsync(waves.data(), at<WaveRange>(workspace, L.waves),
                         sizeof(WaveRange) * waves.size(), hipMemcpyDeviceToHost, s) == hipSuccess;
  ok &= hipStreamSynchronize(s) == hipSuccess;
  if (!ok) return PKV_ERR_LAUNCH;

  bool bad = hdr[kHdrError] != 0;
  // The plan in the workspace must be this batch's, for this descriptor.
  const int units = desc->num_q_heads / heads_per_group(desc->num_q_heads / desc->num_kv_heads);
  if (hdr[kHdrBatch] != batch || hdr[kHdrUnits] != units) bad = true;
  long long acc = 0;
  if (ip[0] != 0) bad = true;
  for (int b = 0; b < batch; ++b) {
    const int L0 = sl[b] > 0 ? sl[b] : 0;
    acc += (L0 + desc->page_size - 1) / desc->page_size;
    if (ip[b + 1] != acc) bad = true;
  }
  if (acc > num_indices) bad = true;
  const long long used = acc < num_indices ? acc : num_indices;
  for (long long i = 0; i < used; ++i)
    if (idx[i] < 0 || idx[i] >= num_pages) bad = true;
  if (groups_out) *groups_out = hdr[kHdrGroups];
  for (size_t i = 0; i < waves.size(); ++i) {
    waves_out[4 * i + 0] = waves[i].b;
    waves_out[4 * i + 1] = waves[i].u;
    waves_out[4 * i + 2] = waves[i].p;
    waves_out[4 * i + 3] = waves[i].count;
  }
  if (hdr[kHdrError] != 0) {
    const int32_t zero = 0;
    if (hipMemcpyAsync(at<int32_t>(workspace, L.hdr) + kHdrError, &zero, sizeof(zero),
                       hipMemcpyHostToDevice, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return PKV_ERR_LAUNCH;
  }
  return bad ? PKV_ERR_DEVICE_DATA : PKV_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Decode without a caller workspace, for callers that cannot allocate (code
// under graph capture, tight serving loops, harnesses that forbid it).  The
// plan, partials and counters live in `scratch`, a file-scope device array of
// PKV_SCRATCH_BYTES that every GPU the library runs on holds until the process
// ends.  In host code the array's name is only a stand-in for its symbol: its
// device address is looked up once per device with hipGetSymbolAddress and
// that address, never the name, is what the kernels receive.

static __device__ __align__(256) unsigned char scratch[PKV_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of this device's copy of `scratch` (looked up on the first
// call made with that device current).  Returns PKV_OK or an error status.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PKV_ERR_LAUNCH;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PKV_ERR_LAUNCH;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return PKV_OK;
}

}  // namespace

extern "C" int pkv_decode_scratch(const pkv_pool* pool, const pkv_desc* desc, const void* q,
                                  const int32_t* seq_lens, const int32_t* kv_indices,
                                  int32_t num_indices, int32_t batch, float sm_scale,
                                  int32_t* kv_indptr, void* out, void* stream) {
  WsLayout L;
  int st = check_desc(desc, &L);
  if (st != PKV_OK) return st;
  st = check_pool(pool, desc);
  if (st != PKV_OK) return st;
  if (!q || !seq_lens || (num_indices > 0 && !kv_indices) || !kv_indptr || !out || batch < 0 ||
      num_indices < 0 || !(sm_scale == sm_scale))
    return PKV_ERR_INVALID_ARG;
  if (batch > desc->max_batch) return PKV_ERR_CAPACITY;
  if (L.total > (size_t)PKV_SCRATCH_BYTES) return PKV_ERR_SCRATCH_TOO_SMALL;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != PKV_OK) return st;
  st = pkv_build_metadata(desc, seq_lens, batch, 0, kv_indptr, ws, L.total, stream);
  if (st != PKV_OK) return st;
  return pkv_decode(pool, desc, q, kv_indptr, kv_indices, num_indices, seq_lens, batch, sm_scale,
                    ws, L.total, out, stream);
}
