// C ABI of libpkv: host-side argument checks, workspace layout and launches.
// Nothing here allocates device memory, synchronises or reads device memory,
// except pkv_debug_validate, which is documented as syncing.
#include <string.h>

#include <vector>

#include "pkv_internal.h"

namespace pkv {

bool ws_layout(const pkv_desc& d, WsLayout* out) {
  if (d.max_batch < 1 || d.num_q_heads < 1 || d.num_kv_heads < 1 || d.head_dim < 1 ||
      d.page_size < 1 || d.max_splits < 1 || d.max_splits > kMaxSplitsLimit ||
      d.target_items < 0 || d.min_chunk_pages < 0 || d.num_q_heads % d.num_kv_heads != 0)
    return false;
  const long long per_planner = (target_items(d) + d.num_kv_heads - 1) / d.num_kv_heads +
                                (long long)d.max_batch;
  const long long all_split = (long long)d.max_batch * d.max_splits;
  const long long max_items = per_planner < all_split ? per_planner : all_split;
  if (max_items > 0x7fffffffLL) return false;
  WsLayout L;
  L.max_items = (int32_t)max_items;
  size_t off = 0;
  L.hdr = off;
  off = align256(off + sizeof(int32_t) * kHdrWords);
  L.split_indptr = off;
  off = align256(off + sizeof(int32_t) * ((size_t)d.max_batch + 1));
  L.items = off;
  off = align256(off + sizeof(int2) * (size_t)max_items);
  L.lse = off;
  off = align256(off + sizeof(float) * (size_t)max_items * d.num_q_heads);
  L.opart = off;
  off = align256(off + sizeof(float) * (size_t)max_items * d.num_q_heads * d.head_dim);
  L.total = off;
  *out = L;
  return true;
}

namespace {

// Shapes the kernels are compiled for.
bool supported(int head_dim, int page_size, int G) {
  if (head_dim != 64 && head_dim != 128) return false;
  const int tpr = 1024 / head_dim;  // tokens per round of one wave
  if (page_size < tpr || page_size % tpr != 0) return false;
  const int r = page_size / tpr;
  if ((r & (r - 1)) != 0) return false;  // rounds per page must be a power of two
  if (G < 1 || (G > 4 && G % 4 != 0)) return false;
  return true;
}

int log2i(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

int check_desc(const pkv_desc* d, WsLayout* L) {
  if (!d) return PKV_ERR_INVALID_ARG;
  if (!ws_layout(*d, L)) return PKV_ERR_INVALID_ARG;
  if (!supported(d->head_dim, d->page_size, d->num_q_heads / d->num_kv_heads))
    return PKV_ERR_UNSUPPORTED;
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

struct Ws {
  int32_t* hdr;
  int32_t* split_indptr;
  int2* items;
  float* lse;
  float* opart;
};

Ws ws_ptrs(void* base, const WsLayout& L) {
  char* c = static_cast<char*>(base);
  return Ws{reinterpret_cast<int32_t*>(c + L.hdr), reinterpret_cast<int32_t*>(c + L.split_indptr),
            reinterpret_cast<int2*>(c + L.items), reinterpret_cast<float*>(c + L.lse),
            reinterpret_cast<float*>(c + L.opart)};
}

int prepare_decode(const pkv_pool* pool, const pkv_desc* desc, const void* q,
                   const int32_t* kv_indptr, const int32_t* kv_indices, int32_t num_indices,
                   const int32_t* seq_lens, int32_t batch, float sm_scale, void* workspace,
                   size_t workspace_bytes, void* out, DecodeArgs* a, WsLayout* L) {
  int st = check_desc(desc, L);
  if (st != PKV_OK) return st;
  st = check_pool(pool, desc);
  if (st != PKV_OK) return st;
  if (!q || !kv_indptr || !kv_indices || !seq_lens || !workspace || !out || batch < 0 ||
      num_indices < 0 || !(sm_scale == sm_scale))
    return PKV_ERR_INVALID_ARG;
  if (batch > desc->max_batch) return PKV_ERR_CAPACITY;
  if (workspace_bytes < L->total) return PKV_ERR_WORKSPACE_TOO_SMALL;
  const Ws w = ws_ptrs(workspace, *L);
  DecodeArgs& d = *a;
  d.k = static_cast<const uint16_t*>(pool->k);
  d.v = static_cast<const uint16_t*>(pool->v);
  d.q = static_cast<const uint16_t*>(q);
  d.kv_indptr = kv_indptr;
  d.kv_indices = kv_indices;
  d.seq_lens = seq_lens;
  d.hdr = w.hdr;
  d.split_indptr = w.split_indptr;
  d.items = w.items;
  d.lse = w.lse;
  d.opart = w.opart;
  d.out = static_cast<uint16_t*>(out);
  d.num_indices = num_indices;
  d.num_pages = pool->num_pages;
  d.num_q_heads = desc->num_q_heads;
  d.num_kv_heads = desc->num_kv_heads;
  d.page_size = desc->page_size;
  d.batch = batch;
  d.max_items = L->max_items;
  d.log2_rounds = log2i(desc->page_size / (1024 / desc->head_dim));
  d.scale_log2 = sm_scale * 1.4426950408889634f;
  return PKV_OK;
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
    case PKV_ERR_CAPACITY: return "batch or split count above the descriptor's capacity";
    case PKV_ERR_LAUNCH: return "kernel launch failed";
    case PKV_ERR_DEVICE_DATA: return "invalid device metadata";
    default: return "unknown status";
  }
}

int32_t pkv_version(void) { return (1 << 16) | 0; }

size_t pkv_workspace_bytes(const pkv_desc* desc) {
  WsLayout L;
  if (!desc || !ws_layout(*desc, &L)) return 0;
  return L.total;
}

int pkv_build_metadata(const pkv_desc* desc, const int32_t* seq_lens, int32_t batch,
                       int32_t forced_splits, int32_t* kv_indptr, void* workspace,
                       size_t workspace_bytes, void* stream) {
  WsLayout L;
  int st = check_desc(desc, &L);
  if (st != PKV_OK) return st;
  if (!seq_lens || !kv_indptr || !workspace || batch < 0 || forced_splits < 0)
    return PKV_ERR_INVALID_ARG;
  if (batch > desc->max_batch) return PKV_ERR_CAPACITY;
  if (workspace_bytes < L.total) return PKV_ERR_WORKSPACE_TOO_SMALL;
  if (forced_splits > 0) {
    const long long f = forced_splits < desc->max_splits ? forced_splits : desc->max_splits;
    if ((long long)batch * f > L.max_items) return PKV_ERR_CAPACITY;
  }
  const Ws w = ws_ptrs(workspace, L);
  MetaArgs a;
  a.seq_lens = seq_lens;
  a.kv_indptr = kv_indptr;
  a.hdr = w.hdr;
  a.split_indptr = w.split_indptr;
  a.items = w.items;
  a.batch = batch;
  a.page_size = desc->page_size;
  a.num_kv_heads = desc->num_kv_heads;
  a.max_splits = desc->max_splits;
  a.target_items = target_items(*desc);
  a.min_chunk = min_chunk(*desc);
  a.forced = forced_splits;
  a.max_items = L.max_items;
  return launch_status(launch_metadata(a, static_cast<hipStream_t>(stream)));
}

int pkv_append_kv(const pkv_pool* pool, const void* k_new, const void* v_new,
                  const int32_t* kv_indptr, const int32_t* kv_indices, int32_t num_indices,
                  const int32_t* seq_lens, int32_t batch, void* stream) {
  int st = check_pool(pool, nullptr);
  if (st != PKV_OK) return st;
  if (!k_new || !v_new || !kv_indptr || !kv_indices || !seq_lens || batch < 0 ||
      num_indices < 0 || pool->page_size < 1 || pool->num_kv_heads < 1)
    return PKV_ERR_INVALID_ARG;
  if (pool->head_dim < 8 || pool->head_dim % 8 != 0) return PKV_ERR_UNSUPPORTED;
  AppendArgs a;
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

int pkv_decode_partials(const pkv_pool* pool, const pkv_desc* desc, const void* q,
                        const int32_t* kv_indptr, const int32_t* kv_indices,
                        int32_t num_indices, const int32_t* seq_lens, int32_t batch,
                        float sm_scale, void* workspace, size_t workspace_bytes, void* out,
                        void* stream) {
  DecodeArgs a;
  WsLayout L;
  int st = prepare_decode(pool, desc, q, kv_indptr, kv_indices, num_indices, seq_lens, batch,
                          sm_scale, workspace, workspace_bytes, out, &a, &L);
  if (st != PKV_OK) return st;
  if (batch == 0) return PKV_OK;
  const int hg = heads_per_wave(desc->num_q_heads / desc->num_kv_heads);
  return launch_status(
      launch_split(a, desc->head_dim, hg, L.max_items, static_cast<hipStream_t>(stream)));
}

int pkv_decode_merge(const pkv_desc* desc, int32_t batch, void* workspace, size_t workspace_bytes,
                     void* out, void* stream) {
  WsLayout L;
  int st = check_desc(desc, &L);
  if (st != PKV_OK) return st;
  if (!workspace || !out || batch < 0) return PKV_ERR_INVALID_ARG;
  if (batch > desc->max_batch) return PKV_ERR_CAPACITY;
  if (workspace_bytes < L.total) return PKV_ERR_WORKSPACE_TOO_SMALL;
  if (batch == 0) return PKV_OK;
  const Ws w = ws_ptrs(workspace, L);
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.hdr = w.hdr;
  a.split_indptr = w.split_indptr;
  a.items = w.items;
  a.lse = w.lse;
  a.opart = w.opart;
  a.out = static_cast<uint16_t*>(out);
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = desc->num_kv_heads;
  a.page_size = desc->page_size;
  a.batch = batch;
  a.max_items = L.max_items;
  return launch_status(launch_merge(a, desc->head_dim, static_cast<hipStream_t>(stream)));
}

int pkv_decode(const pkv_pool* pool, const pkv_desc* desc, const void* q,
               const int32_t* kv_indptr, const int32_t* kv_indices, int32_t num_indices,
               const int32_t* seq_lens, int32_t batch, float sm_scale, void* workspace,
               size_t workspace_bytes, void* out, void* stream) {
  int st = pkv_decode_partials(pool, desc, q, kv_indptr, kv_indices, num_indices, seq_lens, batch,
                               sm_scale, workspace, workspace_bytes, out, stream);
  if (st != PKV_OK) return st;
  return pkv_decode_merge(desc, batch, workspace, workspace_bytes, out, stream);
}

int pkv_debug_validate(const pkv_desc* desc, const int32_t* seq_lens, const int32_t* kv_indptr,
                       const int32_t* kv_indices, int32_t num_indices, int32_t num_pages,
                       int32_t batch, void* workspace, size_t workspace_bytes,
                       int32_t* nsplit_out, int32_t* chunk_out, int32_t* items_out,
                       void* stream) {
  WsLayout L;
  int st = check_desc(desc, &L);
  if (st != PKV_OK) return st;
  if (!seq_lens || !kv_indptr || !workspace || batch < 0 || num_indices < 0 ||
      (num_indices > 0 && !kv_indices))
    return PKV_ERR_INVALID_ARG;
  if (batch > desc->max_batch) return PKV_ERR_CAPACITY;
  if (workspace_bytes < L.total) return PKV_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Ws w = ws_ptrs(workspace, L);
  std::vector<int32_t> sl(batch), ip(batch + 1), hdr(kHdrWords), sp(batch + 1),
      idx(num_indices);
  bool ok = hipMemcpyAsync(sl.data(), seq_lens, sizeof(int32_t) * batch, hipMemcpyDeviceToHost,
                           s) == hipSuccess;
  ok &= hipMemcpyAsync(ip.data(), kv_indptr, sizeof(int32_t) * (batch + 1),
                       hipMemcpyDeviceToHost, s) == hipSuccess;
  ok &= hipMemcpyAsync(hdr.data(), w.hdr, sizeof(int32_t) * kHdrWords, hipMemcpyDeviceToHost,
                       s) == hipSuccess;
  ok &= hipMemcpyAsync(sp.data(), w.split_indptr, sizeof(int32_t) * (batch + 1),
                       hipMemcpyDeviceToHost, s) == hipSuccess;
  if (num_indices > 0)
    ok &= hipMemcpyAsync(idx.data(), kv_indices, sizeof(int32_t) * num_indices,
                         hipMemcpyDeviceToHost, s) == hipSuccess;
  ok &= hipStreamSynchronize(s) == hipSuccess;
  if (!ok) return PKV_ERR_LAUNCH;

  bool bad = hdr[kHdrError] != 0;
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
  if (nsplit_out)
    for (int b = 0; b < batch; ++b) nsplit_out[b] = sp[b + 1] - sp[b];
  if (chunk_out) *chunk_out = hdr[kHdrChunk];
  if (items_out) *items_out = hdr[kHdrNumItems];
  if (hdr[kHdrError] != 0) {
    const int32_t zero = 0;
    if (hipMemcpyAsync(w.hdr + kHdrError, &zero, sizeof(zero), hipMemcpyHostToDevice, s) !=
            hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return PKV_ERR_LAUNCH;
  }
  return bad ? PKV_ERR_DEVICE_DATA : PKV_OK;
}

}  // extern "C"
