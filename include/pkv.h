/*
 * pkv.h - C ABI of the paged-KV split-KV decode attention library (libpkv.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * What it computes.  At every decode step each request contributes one query
 * token with Hq query heads that share Hkv key/value heads (grouped-query
 * attention, G = Hq / Hkv query heads per KV head).  Query head hq attends over
 * the request's cached tokens through KV head hq / G:
 *
 *     out[b, hq, :] = softmax_t( sm_scale * q[b, hq, :] . K_t[hq / G, :] ) V_t[hq / G, :]
 *
 * for t = 0 .. seq_lens[b] - 1.  (Sources, the AstrAI project pages: the
 * paged decode wrapper's docstring, AstrAI compare v1.3.12..6f09b1d,
 * astrai/extension/attention_ops.py, attn_paged_decode; the reference
 * semantics of TorchNativeBackend.fwd_decode in
 * astrai/extension/attention_backend.py on the same page.)  The decode query is
 * the newest position, so a causal mask removes nothing.
 *
 * Paged KV pool.  K and V of one layer live in fixed-size pages of a pool shared
 * by all requests.  This library lays a pool out page-major, then head-major,
 * and stores each (page, KV head) tile as page_size / 16 steps of 16 tokens,
 * each step in the order the matrix-core loads read it:
 *
 *     K : bf16 [num_pages][Hkv][page_size / 16][head_dim / 8][16][8]
 *     V : bf16 [num_pages][Hkv][page_size / 16][head_dim][16]
 *
 * K(t, c) of a tile sits at [t / 16][c / 8][t % 16][c % 8] and V(t, c) at
 * [t / 16][c][t % 16].  One tile is one contiguous run of bytes, one 16-token
 * step of it (4 KiB of K and 4 KiB of V at head_dim 128) another, at every page
 * size, and every load instruction of the decode reads whole contiguous blocks
 * (1 KiB of K, 512 B of V).  (The pages' pool is token-major, [slot][Hkv][D]
 * per layer: the same bytes per token, ordered differently inside a page; the
 * library's append calls write new tokens into this layout.)  Token t of request b
 * lives in page
 * kv_indices[kv_indptr[b] + t / page_size] at offset t % page_size (the pages'
 * PagePool addressing: page index pos // page_size, offset pos % page_size,
 * astrai/inference/core/cache.py on the compare page).  kv_indptr counts
 * pages: kv_indptr[0] = 0, kv_indptr[b + 1] = kv_indptr[b] + ceil(seq_lens[b] /
 * page_size); it is built once per step and reused by every layer (AstrAI
 * commit 05739629, astrai/inference: the bind_tasks bullet on the prefix sum).
 *
 * Split KV.  The work of a call is the list of tiles (request b, group of query
 * heads u, page p) in that order: every tile is one page of one KV head read
 * for one group of query heads.  The list is cut into equal contiguous ranges,
 * one per workgroup, and each workgroup's range again into one range per wave,
 * so every wave streams the same number of pages whatever the mix of sequence
 * lengths.  A range may cover a request's pages only in part: each part leaves
 * an online-softmax partial (normalised output and log-sum-exp); parts of the
 * same (request, head group) are merged with log-sum-exp weights, first inside
 * the workgroup through LDS, then across workgroups by the last workgroup to
 * finish its part (commits by ViperEkura on the author-search page: split
 * partials o_part / ml_part, one combine kernel, the split count retuned so
 * the grid fills the chip).  Everything runs in one kernel launch.
 *
 * Conventions for every entry point.
 *  - Pointers documented "device" are device memory owned by the caller; the
 *    library keeps no pointer after a call returns, holds no global state and
 *    allocates nothing (no hipMalloc / hipFree in any entry point).
 *  - "stream" is a hipStream_t passed as void* (NULL = the default stream).
 *    Launch entry points enqueue work on it and return without synchronising;
 *    nothing on the launch path reads device memory from the host, so a
 *    sequence of launches can be captured into a hipGraph.
 *  - Every entry point returns a pkv_status.  Only host-checkable conditions
 *    are reported (null pointers, shapes, capacities, workspace size, launch
 *    failure).  The contents of device arrays are not validated on the launch
 *    path: out-of-range page ids are skipped by the kernels (never read or
 *    written) and latched in a device error word that pkv_debug_validate
 *    reports.
 *  - bf16 values are IEEE binary32 upper halves; fp32 -> bf16 rounds to
 *    nearest, ties to even.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Waves (64 lanes each) in one decode workgroup: two per SIMD of a compute
 * unit.  The plan splits every workgroup's tile range into this many parts. */
#define PKV_WAVES_PER_WORKGROUP 8

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,          /* null pointer, negative size, inconsistent shapes */
  PKV_ERR_UNSUPPORTED = 2,          /* head_dim / page_size not compiled in */
  PKV_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes below pkv_workspace_bytes(desc) */
  PKV_ERR_CAPACITY = 4,             /* batch or forced split count above the descriptor's capacity */
  PKV_ERR_LAUNCH = 5,               /* the HIP runtime rejected a kernel launch */
  PKV_ERR_DEVICE_DATA = 6,          /* pkv_debug_validate found bad device metadata */
  PKV_ERR_SCRATCH_TOO_SMALL = 7     /* pkv_decode_scratch: the descriptor's workspace exceeds
                                       PKV_SCRATCH_BYTES */
} pkv_status;

/* Static description of one message of pkv_status (never NULL).  Errors are
 * status codes, not exceptions: the pages' kernel wrappers raise a runtime
 * error when a kernel is missing and a value error for an input they do not
 * support (AstrAI compare v1.3.12..6f09b1d, attention_ops.py, _check_available;
 * attention_backend.py, FlashAttnBackend.fwd_prefill); here the Python
 * binding turns every status other than PKV_OK into an exception. */
const char* pkv_status_str(int status);

/* Library ABI version: (major << 16) | minor. */
int32_t pkv_version(void);

/* One layer's paged K/V pool (device memory owned by the caller), contiguous:
 * k: bf16 [num_pages][num_kv_heads][page_size / 16][head_dim / 8][16][8]
 * v: bf16 [num_pages][num_kv_heads][page_size / 16][head_dim][16] */
typedef struct pkv_pool {
  int32_t num_pages;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  void* k;
  void* v;
} pkv_pool;

/* Fixed capacities and shapes.  They fix the launch grid, so one captured
 * hipGraph per batch size replays for any seq_lens within capacity (a grid
 * that followed the step's longest sequence made graph replay unstable on the
 * pages, which fixed it by sizing the split grid from the context capacity;
 * commits by ViperEkura, PagedKV::host_kv_len bullet).
 *
 *  max_batch            requests per call (1 .. 65536)
 *  num_q_heads          Hq; num_kv_heads must divide it, and the group size
 *                       G = Hq / Hkv may be any size; the decode reads each
 *                       K/V tile once per head group of H heads, H the
 *                       largest of 1 .. 8, 12 and 16 that divides G (all of
 *                       G up to 8; a prime G above 8 reads each tile G times)
 *  num_kv_heads         Hkv
 *  head_dim             D, 64 or 128
 *  page_size            P, a power of two >= 16
 *  num_workgroups       workgroups of the decode grid (0 = one per compute unit
 *                       of the device current at the call; 1 .. 65536)
 *  min_tiles_per_group  fewest tiles a workgroup is given; small batches use
 *                       fewer workgroups (0 = default 16)
 */
typedef struct pkv_desc {
  int32_t max_batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t num_workgroups;
  int32_t min_tiles_per_group;
  int32_t reserved; /* must be 0 */
} pkv_desc;

/* Bytes of workspace a descriptor needs (split plan, partial outputs and
 * log-sum-exp values, error word), or 0 if the descriptor is invalid.  The
 * caller allocates it once (any device allocation, 256-byte aligned) and passes
 * it to every pkv_build_metadata / pkv_decode call of that descriptor: the
 * pages moved the split partials into a workspace the executor allocates once,
 * so the decode loop allocates nothing and every kernel address is stable for
 * graph capture (AstrAI commit 05739629, astrai/inference: the
 * InferenceWorkspace bullets on decode_o_part / decode_ml_part and zero
 * allocation in the decode hot loop).  Its
 * contents need no initialisation: pkv_build_metadata writes everything the
 * decode reads.  The decode calls of a step reuse the plan and overwrite the
 * partials and arrival counters, so calls that share a workspace must run one
 * after another (in one stream, or ordered by events); concurrent calls need
 * one workspace each. */
size_t pkv_workspace_bytes(const pkv_desc* desc);

/* Step metadata, once per decode step (before the per-layer calls).
 *
 * From seq_lens (device int32 [batch]: tokens each request attends to this
 * step, the token appended this step included) it writes
 *   kv_indptr   device int32 [batch + 1], page prefix sums as defined above,
 * and the work plan into the workspace.  Plan, with U = num_q_heads / H query
 * head groups per request (H the largest of 1 .. 8, 12 and 16 that divides G) and
 * T = kv_indptr[batch] * U
 * tiles:
 *   groups   W = min(num_workgroups, max(1, ceil(T / min_tiles_per_group))),
 *            or min(forced_groups, num_workgroups, T) when forced_groups > 0;
 *   group i  covers tiles [floor(i*T/W), floor((i+1)*T/W));
 *   wave w   of a group covers the w-th of PKV_WAVES_PER_WORKGROUP equal
 *            sub-ranges of the group's range.
 * Negative seq_lens count as 0 and latch the device error word.
 * Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_CAPACITY
 * (batch > max_batch), PKV_ERR_WORKSPACE_TOO_SMALL, PKV_ERR_LAUNCH. */
int pkv_build_metadata(const pkv_desc* desc, const int32_t* seq_lens, int32_t batch,
                       int32_t forced_groups, int32_t* kv_indptr, void* workspace,
                       size_t workspace_bytes, void* stream);

/* KV append (once per layer, after pkv_build_metadata): writes this step's
 * token of every request into the pool; on the pages this is an indexed store
 * into the layer's K and V buffers at out_cache_loc before the attention call
 * (attention_backend.py, CudaBackend.fwd_decode).  The token goes to position seq_lens[b] - 1:
 *   K[kv_indices[kv_indptr[b] + pos / P]][h][pos % P][:] = k_new[b][h][:], same for V.
 *  k_new, v_new   device bf16 [batch][num_kv_heads][head_dim]
 *  kv_indptr      device int32 [batch + 1] (from pkv_build_metadata)
 *  kv_indices     device int32 [num_indices], physical page ids (may be NULL
 *                 when num_indices is 0)
 *  seq_lens       device int32 [batch], post-append lengths; <= 0 writes nothing
 * Two requests must not target the same slot (the writes would race).
 * Page ids outside [0, num_pages) or index positions outside [0, num_indices)
 * are skipped.
 * Errors: PKV_ERR_INVALID_ARG (null pointer, negative size, or more than
 * 2^31 - 1 row chunks), PKV_ERR_UNSUPPORTED (head_dim other than 64 or 128),
 * PKV_ERR_LAUNCH. */
int pkv_append_kv(const pkv_pool* pool, const void* k_new, const void* v_new,
                  const int32_t* kv_indptr, const int32_t* kv_indices, int32_t num_indices,
                  const int32_t* seq_lens, int32_t batch, void* stream);

/* KV append of several new tokens per request (extend / chunked prefill),
 * one launch: request b's n_b = qo_indptr[b+1] - qo_indptr[b] new tokens are
 * its newest, positions seq_lens[b] - n_b .. seq_lens[b] - 1, and row
 * qo_indptr[b] + i of k_new / v_new goes to position seq_lens[b] - n_b + i:
 *   K[kv_indices[kv_indptr[b] + pos / P]][h][pos % P][:] = k_new[qo_indptr[b] + i][h][:]
 * in the pool's tile layout, same for V.  On the pages the extend step stores
 * every new token this way before the paged prefill (attention_backend.py,
 * CudaBackend.fwd_prefill; cache.py, the KVCache docstring: out_cache_loc
 * [batch, new_seq_len]; both on the compare page).
 *  k_new, v_new   device bf16 [rows][num_kv_heads][head_dim], rows = qo_indptr[batch]
 *  qo_indptr      device int32 [batch + 1], non-decreasing, qo_indptr[0] = 0
 *                 (the same array pkv_prefill takes)
 *  kv_indptr      device int32 [batch + 1] (from pkv_build_metadata)
 *  kv_indices     device int32 [num_indices] (may be NULL when num_indices is 0)
 *  seq_lens       device int32 [batch], lengths with the new tokens included
 *  max_new_rows   host int: an upper bound of every n_b; it sizes the grid
 *                 (rows beyond it are not written)
 * Rows whose position would be negative (n_b > seq_lens[b]), page ids outside
 * [0, num_pages) and index positions outside [0, num_indices) are skipped.
 * Two rows must not target the same slot.  No allocation; capturable.
 * Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED (head_dim other than 64 or
 * 128), PKV_ERR_CAPACITY (batch * num_kv_heads * ceil(max_new_rows / 16) of
 * 2^31 or more), PKV_ERR_LAUNCH. */
int pkv_append_kv_ragged(const pkv_pool* pool, const void* k_new, const void* v_new,
                         const int32_t* qo_indptr, const int32_t* kv_indptr,
                         const int32_t* kv_indices, int32_t num_indices, const int32_t* seq_lens,
                         int32_t batch, int32_t max_new_rows, void* stream);

/* Decode attention for one layer (one kernel launch).
 *  q            device bf16 [batch][num_q_heads][head_dim], contiguous
 *  kv_indptr    device int32 [batch + 1] written by pkv_build_metadata this step
 *  kv_indices   device int32 [num_indices] (may be NULL when num_indices is 0)
 *  seq_lens     device int32 [batch], the same array pkv_build_metadata read
 *  sm_scale     softmax scale (usually 1 / sqrt(head_dim)); any value but NaN,
 *               zero and negative included (zero gives equal weights)
 *  workspace    the workspace pkv_build_metadata wrote this step
 *  out          device bf16 [batch][num_q_heads][head_dim]; a request with
 *               seq_len 0 gets a zero row
 * Accumulation is fp32 (scores, online softmax, partials, merges).  For a fixed
 * plan the result is deterministic: partials are merged in a fixed order
 * whichever workgroup merges them.  Calls that share a workspace must be
 * ordered (same stream): the cross-workgroup merge uses counters in it. */
int pkv_decode(const pkv_pool* pool, const pkv_desc* desc, const void* q,
               const int32_t* kv_indptr, const int32_t* kv_indices, int32_t num_indices,
               const int32_t* seq_lens, int32_t batch, float sm_scale, void* workspace,
               size_t workspace_bytes, void* out, void* stream);

/* KV append and decode attention of one layer in one kernel launch: the same
 * result, pool contents included, as pkv_append_kv(pool, k_new, v_new, ...)
 * followed by pkv_decode(...) with the same arguments, without the separate
 * append launch.  On the pages the per-layer step is exactly this pair: the
 * new token's K and V are stored into the layer's buffers, then attention runs
 * over the cache that includes them (attention_backend.py, CudaBackend.
 * fwd_decode, on the compare page).  The wave that reads the page holding
 * token seq_lens[b] - 1 takes that token from k_new / v_new and writes it into
 * the pool.
 *  k_new, v_new   device bf16 [batch][num_kv_heads][head_dim], both non-NULL
 * Every other argument, the layouts and the errors are those of pkv_decode and
 * pkv_append_kv (PKV_ERR_INVALID_ARG for a NULL k_new or v_new). */
int pkv_decode_append(const pkv_pool* pool, const pkv_desc* desc, const void* q,
                      const void* k_new, const void* v_new, const int32_t* kv_indptr,
                      const int32_t* kv_indices, int32_t num_indices, const int32_t* seq_lens,
                      int32_t batch, float sm_scale, void* workspace, size_t workspace_bytes,
                      void* out, void* stream);

/* Step metadata and the first layer's decode in one launch: the same results
 * (kv_indptr, the plan in the workspace, the pool and out) as
 *   pkv_build_metadata(desc, seq_lens, batch, forced_groups, kv_indptr, ws)
 * followed by pkv_decode_append(..., k_new, v_new, ...), or by pkv_decode(...)
 * when k_new and v_new are both NULL.  The pages build the step's page prefix
 * sums once and reuse them in every layer (AstrAI commit 05739629,
 * astrai/inference, bind_tasks bullets); here each workgroup of the first
 * layer's launch computes the plan from seq_lens in its own LDS, starts its
 * tiles at once and writes its part of the plan for the step's later layers,
 * which call pkv_decode / pkv_decode_append with the same kv_indptr and
 * workspace.  Deterministic: bitwise the result of the two-call sequence.
 *  seq_lens       device int32 [batch], read by this launch only
 *  kv_indptr      device int32 [batch + 1], written (as pkv_build_metadata)
 *  forced_groups  as for pkv_build_metadata
 * Every other argument is as for pkv_decode_append.  Differences from the
 * two-call sequence: the workspace error word is not cleared, new error bits
 * are ORed into it (pkv_debug_validate reads and clears it); and the merge's
 * arrival counters must be zero when the launch starts, which holds for a
 * workspace that has been through pkv_build_metadata once, since every decode
 * leaves them at zero (a workspace that never has must be zero-filled).  For
 * batch 0 or batch above 1024 the call runs the metadata kernel and then the
 * decode, two launches.
 * Errors: those of pkv_build_metadata and pkv_decode_append. */
int pkv_decode_plan(const pkv_pool* pool, const pkv_desc* desc, const void* q,
                    const void* k_new, const void* v_new, const int32_t* seq_lens, int32_t batch,
                    int32_t forced_groups, int32_t* kv_indptr, const int32_t* kv_indices,
                    int32_t num_indices, float sm_scale, void* workspace, size_t workspace_bytes,
                    void* out, void* stream);

/* Decode attention with a per-token keep mask (one launch): the optional 2-D
 * bool mask [batch, max_seq_len], True = keep, of the pages' paged decode
 * wrapper (attention_ops.py, attn_paged_decode docstring, on the compare page).
 * Token t of request b attends iff t < seq_lens[b] and mask[b * mask_stride + t]
 * is nonzero; a request that keeps no token gets a zero row.
 *  mask          device uint8 [batch][mask_stride]; row b must hold at least
 *                seq_lens[b] entries (entries past seq_lens[b] are ignored;
 *                reads past batch * mask_stride bytes return 0)
 *  mask_stride   bytes between rows, a multiple of 4, with
 *                batch * mask_stride < 2^31
 * Every other argument is as for pkv_decode.  Errors: those of pkv_decode, and
 * PKV_ERR_INVALID_ARG for a NULL mask or a bad stride. */
int pkv_decode_masked(const pkv_pool* pool, const pkv_desc* desc, const void* q,
                      const uint8_t* mask, int32_t mask_stride, const int32_t* kv_indptr,
                      const int32_t* kv_indices, int32_t num_indices, const int32_t* seq_lens,
                      int32_t batch, float sm_scale, void* workspace, size_t workspace_bytes,
                      void* out, void* stream);

/* Decode attention over token-major K/V (one launch): one [num_kv_heads]
 * [head_dim] row per token slot instead of pages.  Covers the token-level mode
 * in which the request-to-token table is the page table with page size 1
 * (commits by ViperEkura, the bullet on the CUDA backend's decode) and, with no
 * table, the contiguous K/V of the non-paged decode wrapper, laid out [batch,
 * seq_len, kv_heads, head_dim] (attention_ops.py, attn_decode and the BLHD
 * layout, on the compare page), here with per-request lengths.
 *  desc         as for pkv_decode, with page_size 16: the plan cuts each request
 *               into 16-token blocks
 *  k_cache, v_cache  device bf16 [num_slots][num_kv_heads][head_dim]
 *  num_slots    slots in the caches, >= 1
 *  slot_table   device int32 [batch][table_stride]: slot of token t of request
 *               b at slot_table[b * table_stride + t] (entries at t >=
 *               seq_lens[b] are not read), or NULL: slot b * table_stride + t,
 *               which needs batch * table_stride <= num_slots
 *  table_stride tokens per table row (request row of the contiguous layout);
 *               batch * table_stride < 2^31
 *  kv_indptr    device int32 [batch + 1] from pkv_build_metadata(desc, seq_lens)
 *               (the plan of the same call)
 * q, seq_lens, batch, sm_scale, the workspace and out are as for pkv_decode.
 * A token at t >= table_stride or with a slot outside [0, num_slots) is
 * dropped and sets a bit in the workspace error word.  Errors: those of
 * pkv_decode; PKV_ERR_INVALID_ARG for page_size other than 16, NULL caches or a
 * contiguous layout larger than the caches; PKV_ERR_CAPACITY for
 * batch * table_stride >= 2^31. */
int pkv_decode_tokens(const pkv_desc* desc, const void* k_cache, const void* v_cache,
                      int32_t num_slots, const int32_t* slot_table, int32_t table_stride,
                      const void* q, const int32_t* kv_indptr, const int32_t* seq_lens,
                      int32_t batch, float sm_scale, void* workspace, size_t workspace_bytes,
                      void* out, void* stream);

/* Paged prefill / extend attention of one layer (one launch, no workspace).
 * Request b has n_b = qo_indptr[b+1] - qo_indptr[b] query rows (its newest
 * tokens) and attends to its L_b = seq_lens[b] cached tokens, the new ones
 * included, through the same page table as the decode.  With causal != 0,
 * query row i (0-based) sees keys 0 .. L_b - n_b + i (the mask aligned to the
 * end of the KV: the pages' causal offset 0, attention_ops.py,
 * attn_paged_prefill, on the compare page); otherwise every row sees all L_b
 * keys.  A row that sees no key gets zeros.
 *  q            device bf16 [total_q][num_q_heads][head_dim], rows of request b
 *               at qo_indptr[b] ..
 *  qo_indptr    device int32 [batch + 1], non-decreasing, qo_indptr[0] = 0
 *  kv_indptr    device int32 [batch + 1] from pkv_build_metadata(seq_lens)
 *  kv_indices   device int32 [num_indices] (may be NULL when num_indices is 0)
 *  seq_lens     device int32 [batch] KV lengths
 *  max_q_len    host int: an upper bound of every n_b; it sizes the grid
 *               (rows beyond it are not computed)
 *  out          device bf16 [total_q][num_q_heads][head_dim]
 * The descriptor gives the shapes (num_workgroups and min_tiles_per_group are
 * not used).  Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED,
 * PKV_ERR_CAPACITY (batch above max_batch or 65535, or a grid of 2^31 or
 * more workgroups: ceil(max_q_len / (8 * 16 / hg)) * (num_q_heads / hg) *
 * batch, hg = query heads per workgroup row block, min(G, 4)), PKV_ERR_LAUNCH. */
int pkv_prefill(const pkv_pool* pool, const pkv_desc* desc, const void* q,
                const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                int32_t num_indices, const int32_t* seq_lens, int32_t batch, int32_t max_q_len,
                int32_t causal, float sm_scale, void* out, void* stream);

/* Debug only (synchronises the stream; not capturable).  Checks device
 * metadata and copies the plan to host memory.  The launch entry points do not
 * read device data from the host (the pages keep host reads out of the decode
 * step: KVCache carries the longest length as a host integer so that decode
 * needs no device synchronisation, cache.py, the KVCache docstring on the
 * compare page), so the checks they cannot make live here.
 *  groups_out   host int32 or NULL: workgroups the plan uses (W above)
 *  waves_out    host int32 [num_workgroups * PKV_WAVES_PER_WORKGROUP * 4] or
 *               NULL: for every wave of
 *               the grid, {request, head group, first page, tiles} of its range
 *               (tiles = 0 for an idle wave)
 * Returns PKV_ERR_DEVICE_DATA if kv_indptr is not the page prefix sum of
 * seq_lens, any listed page id is outside [0, num_pages), kv_indptr[batch]
 * exceeds num_indices, the plan in the workspace was built for another batch
 * size or head grouping, or a kernel latched the device error word (which it
 * then clears).  A decode given a workspace whose plan was built for another
 * batch or head grouping writes no output and latches that word. */
int pkv_debug_validate(const pkv_desc* desc, const int32_t* seq_lens, const int32_t* kv_indptr,
                       const int32_t* kv_indices, int32_t num_indices, int32_t num_pages,
                       int32_t batch, void* workspace, size_t workspace_bytes,
                       int32_t* groups_out, int32_t* waves_out, void* stream);

/* Decode without a caller workspace, for callers that cannot allocate device
 * memory: code under hipGraph capture, tight serving loops, harnesses that
 * forbid allocation.  The same result as pkv_build_metadata(desc, seq_lens,
 * batch, 0, kv_indptr, ws, ...) followed by pkv_decode(..., ws, ...) (two
 * launches), with ws a static device array of PKV_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends.  Every call on
 * a GPU shares that GPU's array and rewrites all of it that it reads, so calls
 * that overlap on one GPU (other streams, other host threads) race; calls in
 * one stream are safe.  Nothing is allocated (no hipMalloc / hipFree); the
 * first call with a device current looks up that device's array address.
 *  kv_indptr    device int32 [batch + 1], written (the step's page prefix sums)
 * Every other argument is as for pkv_build_metadata and pkv_decode.  Errors:
 * those of pkv_build_metadata and pkv_decode, and PKV_ERR_SCRATCH_TOO_SMALL when
 * pkv_workspace_bytes(desc) exceeds PKV_SCRATCH_BYTES. */
#define PKV_SCRATCH_BYTES 8388608 /* 8 MiB */
int pkv_decode_scratch(const pkv_pool* pool, const pkv_desc* desc, const void* q,
                       const int32_t* seq_lens, const int32_t* kv_indices, int32_t num_indices,
                       int32_t batch, float sm_scale, int32_t* kv_indptr, void* out, void* stream);

/* Diagnostic, not part of the attention path: one launch that reads `bytes`
 * of device memory at src (16-byte aligned, a multiple of 16) with the decode
 * kernel's load shape on MI355X -- PKV_READ_CEILING_GROUPS workgroups (one
 * per compute unit) of PKV_WAVES_PER_WORKGROUP waves, 16-byte loads, eight in
 * flight per wave --
 * and writes one xor-fold per lane to sink, so that timing it gives the
 * achievable read rate of a launch of that size on this machine.
 *  sink        device uint32 [sink_words], sink_words >= PKV_READ_CEILING_GROUPS
 *              * 64 * PKV_WAVES_PER_WORKGROUP
 * Errors: PKV_ERR_INVALID_ARG (NULL, misaligned size, small sink), PKV_ERR_LAUNCH. */
#define PKV_READ_CEILING_GROUPS 256
int pkv_debug_read_ceiling(const void* src, size_t bytes, uint32_t* sink, size_t sink_words,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
