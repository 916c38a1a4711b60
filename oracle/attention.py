"""fp64 CPU oracle for paged-KV split-KV decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module.  The HIP library never
calls it, and it shares no code with the HIP library: it decodes bf16, walks
the page table, computes prefix sums, plans splits and merges partials with
its own plain numpy code.

What it computes (sources are the AstrAI pages; citations name the page and
the hunk or bullet, as the pages have no section numbers):

* Decode attention: one query token per request attends over that request's
  cached tokens with grouped-query heads.  The semantics are those of the
  reference backend that gathers K/V through the token table, zeroes padding,
  repeats KV heads and calls SDPA (AstrAI compare v1.3.12..6f09b1d,
  astrai/extension/attention_backend.py, TorchNativeBackend.fwd_decode), and
  of the paged kernel's wrapper (same page, astrai/extension/attention_ops.py,
  attn_paged_decode docstring: q [batch, n_heads, head_dim], per-request
  lengths from kv_indptr).  The decode query is the newest position, so the
  causal mask removes nothing (commits by ViperEkura: the bullet that makes the
  CUDA decode backend always causal).
* Paged addressing: token t of request b lives in page
  kv_indices[kv_indptr[b] + t // P] at offset t % P (same page,
  astrai/inference/core/cache.py, PagePool._extend_slot: page index is
  pos // page_size, slot offset is pos % page_size).  kv_indptr is a prefix
  sum over requests, built once per step (AstrAI commit 05739629,
  astrai/inference: the bind_tasks bullet on the kv_indptr prefix sum).  Here
  it counts pages, not tokens.
* Split KV and merge: a request's KV range is cut into chunks whose partial
  outputs and (max, sum) statistics are merged by one combine kernel
  (commits by ViperEkura: split-partial tensors o_part / ml_part, the shared
  combine kernel, the compute_num_splits retune).  Each partial is stored as the
  chunk's normalised output and its log-sum-exp; the merge weights each chunk
  by exp(lse_s - max lse).
* KV append: the token written this step goes to position seq_len - 1
  (cache.py, bind_tasks: write_pos = seq_lens - 1); an extend step's n new
  tokens go to positions seq_len - n .. seq_len - 1 (append_kv_rows).
* Keep mask (decode_masked): token t of request b attends iff t < seq_len and
  the mask keeps it (the paged decode wrapper's optional 2-D bool mask).
* Prefill / extend (prefill): n new query rows per request over its L keys,
  the causal mask aligned to the end of the keys (causal offset 0).
* Token-major K/V (decode_tokens): one [Hkv, D] row per token slot, found
  through a request-to-token table (page size 1) or at b * stride + t in the
  contiguous [batch, seq, kv_heads, head_dim] layout of the non-paged decode.

Readings taken where the pages are silent:
kv_indptr in pages; KV head of query head hq is hq // G; seq_len includes
the token appended this step; empty chunks have lse = -inf and weight 0; a
request with seq_len 0 gets a zero output row; chunks are contiguous runs of
pages; the work plan below (equal contiguous ranges of (request, head group,
page) tiles) is this library's own (the pages give only its goal: enough
blocks to fill the chip).

Parity status: every function here is pinned by tests that do not re-type its
formulas (brute force, closed forms, invariants, a library special case,
NaN poisoning and planted mistakes); none is "parity unpinned".
"""

from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

__all__ = [
    "bf16_to_f64",
    "page_counts",
    "kv_indptr",
    "kv_head_of",
    "gather_request",
    "softmax_attend",
    "decode",
    "decode_masked",
    "decode_tokens",
    "prefill",
    "chunk_partial",
    "merge_partials",
    "even_page_ranges",
    "head_groups",
    "tile_of",
    "plan_stream",
    "decode_split",
    "decode_pieces",
    "append_kv",
    "append_kv_rows",
]


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) to float64, exactly (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    f32 = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def page_counts(seq_lens, P: int) -> np.ndarray:
    """Pages that hold each request's tokens: ceil(L / P)."""
    L = np.asarray(seq_lens, dtype=np.int64)
    return (L + (P - 1)) // P


def kv_indptr(seq_lens, P: int) -> np.ndarray:
    """kv_indptr[0] = 0, kv_indptr[b + 1] = kv_indptr[b] + ceil(L_b / P)."""
    n = page_counts(seq_lens, P)
    out = np.zeros(n.size + 1, dtype=np.int64)
    out[1:] = np.cumsum(n)
    return out


def kv_head_of(hq: int, G: int) -> int:
    """KV head shared by query head hq under grouped-query attention (G = Hq / Hkv)."""
    return hq // G


def gather_request(pool_bits, indptr, indices, b: int, L: int, P: int) -> np.ndarray:
    """Dense float64 [L, Hkv, D] copy of request b's first L tokens from a paged pool."""
    pool = np.asarray(pool_bits)
    Hkv, D = pool.shape[1], pool.shape[3]
    out = np.empty((L, Hkv, D), dtype=np.float64)
    base = int(indptr[b])
    for t in range(L):
        page = int(indices[base + t // P])
        out[t] = bf16_to_f64(pool[page, :, t % P, :])
    return out


def softmax_attend(qv: np.ndarray, Kd: np.ndarray, Vd: np.ndarray, sm_scale: float) -> np.ndarray:
    """softmax(sm_scale * q K^T) V for one query row; Kd, Vd are [L, D] float64."""
    if Kd.shape[0] == 0:
        return np.zeros(Vd.shape[1], dtype=np.float64)
    x = sm_scale * (Kd @ qv)
    m = np.max(x)
    e = np.exp(x - m)
    return (e @ Vd) / np.sum(e)


def decode(q_bits, k_pool, v_pool, indptr, indices, seq_lens, sm_scale: float, P: int) -> np.ndarray:
    """Unsplit decode attention for every request and query head -> float64 [B, Hq, D]."""
    q = bf16_to_f64(q_bits)
    B, Hq, D = q.shape
    Hkv = np.asarray(k_pool).shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        Kd = gather_request(k_pool, indptr, indices, b, L, P)
        Vd = gather_request(v_pool, indptr, indices, b, L, P)
        for hq in range(Hq):
            h = kv_head_of(hq, G)
            out[b, hq] = softmax_attend(q[b, hq], Kd[:, h, :], Vd[:, h, :], sm_scale)
    return out


def decode_masked(q_bits, k_pool, v_pool, indptr, indices, seq_lens, sm_scale: float, P: int,
                  mask) -> np.ndarray:
    """Decode attention with a per-token keep mask -> float64 [B, Hq, D].

    ``mask`` is bool [B, S] with S at least every seq_len; True keeps the token
    (the optional 2-D mask [batch, max_seq_len], True = keep, of the paged
    decode wrapper: AstrAI compare v1.3.12..6f09b1d, attention_ops.py,
    attn_paged_decode docstring).  Token t of request b attends iff t < seq_len
    and mask[b, t]; mask entries past seq_len are ignored.  A request that keeps
    no token gets a zero row, as an empty request does.
    """
    q = bf16_to_f64(q_bits)
    B, Hq, D = q.shape
    Hkv = np.asarray(k_pool).shape[1]
    G = Hq // Hkv
    keep_all = np.asarray(mask, dtype=bool)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        keep = keep_all[b, :L]
        Kd = gather_request(k_pool, indptr, indices, b, L, P)[keep]
        Vd = gather_request(v_pool, indptr, indices, b, L, P)[keep]
        for hq in range(Hq):
            h = kv_head_of(hq, G)
            out[b, hq] = softmax_attend(q[b, hq], Kd[:, h, :], Vd[:, h, :], sm_scale)
    return out


def decode_tokens(q_bits, k_cache, v_cache, seq_lens, sm_scale: float, slot_table=None,
                  stride: int = 0) -> np.ndarray:
    """Decode attention over token-major K/V -> float64 [B, Hq, D].

    ``k_cache`` / ``v_cache`` hold one row [Hkv, D] per token slot.  Token t of
    request b is slot ``slot_table[b, t]``: the token-level mode in which the
    request-to-token table serves as the page table with page size 1 (commits
    by ViperEkura: the bullet on the CUDA backend's decode).  Without a table it
    is slot b * stride + t: the contiguous K/V of the non-paged decode wrapper,
    laid out [batch, seq_len, kv_heads, head_dim] (AstrAI compare
    v1.3.12..6f09b1d, attention_ops.py: attn_decode and the BLHD TensorLayout),
    here with a per-request length.  That wrapper's causal flag puts the
    causal offset at the last key, so every key of a decode query counts.
    """
    q = bf16_to_f64(q_bits)
    B, Hq, D = q.shape
    k_all = np.asarray(k_cache)
    Hkv = k_all.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if slot_table is None:
            slots = b * int(stride) + np.arange(L)
        else:
            slots = np.asarray(slot_table)[b, :L].astype(np.int64)
        Kd = bf16_to_f64(k_all[slots])
        Vd = bf16_to_f64(np.asarray(v_cache)[slots])
        for hq in range(Hq):
            h = kv_head_of(hq, G)
            out[b, hq] = softmax_attend(q[b, hq], Kd[:, h, :], Vd[:, h, :], sm_scale)
    return out


def prefill(q_rows, k_pool, v_pool, kv_indptr, kv_indices, seq_lens, qo_indptr, sm_scale: float,
            P: int, causal: bool) -> np.ndarray:
    """Paged prefill / extend attention -> float64 [total_q, Hq, D].

    Request b has qo_indptr[b+1] - qo_indptr[b] = n query rows and attends to
    its L = seq_lens[b] cached tokens (the new tokens included), read through
    the page table as in decode.  The pages' paged prefill wrapper takes
    flattened query rows with per-request offsets, per-request KV lengths and
    a causal flag with offset 0 (AstrAI compare v1.3.12..6f09b1d,
    attention_ops.py, attn_paged_prefill).  Reading of offset 0: the causal
    mask is aligned to the end of the KV, so query row i (0-based) is the
    token at position L - n + i and sees keys 0 .. L - n + i; with n = 1 this
    is decode.  Without the causal flag every row sees all L keys.  A row that
    sees no key gets zeros.
    """
    q = bf16_to_f64(q_rows)
    total, Hq, D = q.shape
    Hkv = np.asarray(k_pool).shape[1]
    G = Hq // Hkv
    out = np.zeros((total, Hq, D), dtype=np.float64)
    for b in range(len(qo_indptr) - 1):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        n, L = q1 - q0, max(int(seq_lens[b]), 0)
        Kd = gather_request(k_pool, kv_indptr, kv_indices, b, L, P)
        Vd = gather_request(v_pool, kv_indptr, kv_indices, b, L, P)
        for i in range(n):
            vis = min(L, max(0, L - n + i + 1)) if causal else L
            for hq in range(Hq):
                h = kv_head_of(hq, G)
                out[q0 + i, hq] = softmax_attend(q[q0 + i, hq], Kd[:vis, h, :], Vd[:vis, h, :],
                                                 sm_scale)
    return out


def chunk_partial(qv, Kd, Vd, sm_scale: float) -> Tuple[np.ndarray, float]:
    """One chunk's normalised partial output and its natural-log log-sum-exp.

    An empty chunk returns (zeros, -inf).
    """
    if Kd.shape[0] == 0:
        return np.zeros(Vd.shape[1], dtype=np.float64), -math.inf
    x = sm_scale * (Kd @ qv)
    m = float(np.max(x))
    e = np.exp(x - m)
    s = float(np.sum(e))
    return (e @ Vd) / s, m + math.log(s)


def merge_partials(parts: Sequence[Tuple[np.ndarray, float]]) -> np.ndarray:
    """Log-sum-exp combine of chunk partials: sum_s w_s o_s / sum_s w_s, w_s = exp(lse_s - max lse)."""
    lses = [lse for _, lse in parts]
    M = max(lses)
    D = parts[0][0].shape[0]
    if M == -math.inf:
        return np.zeros(D, dtype=np.float64)
    num = np.zeros(D, dtype=np.float64)
    den = 0.0
    for o, lse in parts:
        if lse == -math.inf:
            continue
        w = math.exp(lse - M)
        num += w * o
        den += w
    return num / den


def even_page_ranges(n_pages: int, nsplit: int) -> List[Tuple[int, int]]:
    """Cut pages [0, n_pages) into nsplit contiguous runs as evenly as possible.

    Run s is [floor(s * n / k), floor((s + 1) * n / k)).
    """
    return [((s * n_pages) // nsplit, ((s + 1) * n_pages) // nsplit) for s in range(nsplit)]


def head_groups(Hq: int, Hkv: int) -> Tuple[int, int]:
    """(HG, U): query heads per head group and head groups per request.

    A head group is query heads of one KV head: the largest number of them
    in 1 .. 8, 12 or 16 that divides G (all of them up to eight); a KV head
    with more query heads than that gets several head groups.  (The grouping is the decode plan's, not the pages': it only
    orders the plan's tiles.)
    """
    G = Hq // Hkv
    HG = max(h for h in (1, 2, 3, 4, 5, 6, 7, 8, 12, 16) if G % h == 0)
    return HG, Hq // HG


def tile_of(indptr, units: int, t: int) -> Tuple[int, int, int]:
    """(request, head group, page) of tile t in the order request, head group, page."""
    starts = np.asarray(indptr, dtype=np.int64) * units
    b = int(np.searchsorted(starts, t, side="right")) - 1
    n = int(indptr[b + 1] - indptr[b])
    r = t - int(starts[b])
    return b, r // n, r % n


def plan_stream(seq_lens, P: int, units: int, groups: int, min_tiles: int,
                forced: int = 0, waves_per_group: int = 8) -> dict:
    """This library's work plan (not from the pages, which give only its goal).

    T = pages * units tiles; W = min(groups, ceil(T / min_tiles)) workgroups
    (min(forced, groups, T) if forced > 0, 0 if T = 0); workgroup i covers tiles
    [floor(i*T/W), floor((i+1)*T/W)) and its wave w the w-th of waves_per_group
    equal parts of that range.  Returns W and, for every wave of the grid,
    (request, head group, first page, tiles), zeros for an idle wave.
    """
    ip = kv_indptr(seq_lens, P)
    T = int(ip[-1]) * units
    if T == 0:
        W = 0
    elif forced > 0:
        W = min(forced, groups, T)
    else:
        W = min(groups, -(-T // min_tiles))
    waves = np.zeros((groups * waves_per_group, 4), dtype=np.int64)
    for i in range(W):
        g0, g1 = i * T // W, (i + 1) * T // W
        for w in range(waves_per_group):
            t0 = g0 + w * (g1 - g0) // waves_per_group
            t1 = g0 + (w + 1) * (g1 - g0) // waves_per_group
            if t1 > t0:
                waves[i * waves_per_group + w] = (*tile_of(ip, units, t0), t1 - t0)
    return {"kv_indptr": ip, "tiles": T, "groups": W, "waves": waves}


def decode_split(q_bits, k_pool, v_pool, indptr, indices, seq_lens, sm_scale: float,
                 P: int, nsplit) -> np.ndarray:
    """Split-then-merge decode with nsplit[b] page-contiguous chunks for request b."""
    q = bf16_to_f64(q_bits)
    B, Hq, D = q.shape
    Hkv = np.asarray(k_pool).shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        ns = int(nsplit[b])
        if L == 0 or ns == 0:
            continue
        Kd = gather_request(k_pool, indptr, indices, b, L, P)
        Vd = gather_request(v_pool, indptr, indices, b, L, P)
        n_pages = -(-L // P)
        ranges = even_page_ranges(n_pages, ns)
        for hq in range(Hq):
            h = kv_head_of(hq, G)
            parts = []
            for p0, p1 in ranges:
                t0, t1 = p0 * P, min(L, p1 * P)
                parts.append(chunk_partial(q[b, hq], Kd[t0:t1, h, :], Vd[t0:t1, h, :], sm_scale))
            out[b, hq] = merge_partials(parts)
    return out


def append_kv(k_pool, v_pool, k_new, v_new, indptr, indices, seq_lens, P: int):
    """Write this step's token of every request into the pool (returns new copies).

    The token goes to position seq_len - 1; requests with seq_len 0 write nothing.
    """
    k = np.array(k_pool, copy=True)
    v = np.array(v_pool, copy=True)
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        pos = L - 1
        page = int(indices[int(indptr[b]) + pos // P])
        k[page, :, pos % P, :] = k_new[b]
        v[page, :, pos % P, :] = v_new[b]
    return k, v


def append_kv_rows(k_pool, v_pool, k_rows, v_rows, qo_indptr, indptr, indices, seq_lens, P: int):
    """Write every request's new tokens into the pool (returns new copies).

    Request b brings n_b = qo_indptr[b+1] - qo_indptr[b] new tokens, rows
    qo_indptr[b] .. qo_indptr[b+1] - 1 of k_rows / v_rows ([rows, Hkv, D]);
    they are its newest tokens, positions seq_len - n_b .. seq_len - 1.  This
    is the extend step's store of every new token before the paged prefill
    (AstrAI compare v1.3.12..6f09b1d, attention_backend.py, CudaBackend.
    fwd_prefill: k_buffer[layer_id, out_cache_loc] = k; cache.py, the KVCache
    docstring: out_cache_loc [batch, new_seq_len], and bind_tasks, which takes
    the write slots of positions start_pos .. seq_len - 1).  A row whose
    position would fall before the request's first token writes nothing.
    """
    k = np.array(k_pool, copy=True)
    v = np.array(v_pool, copy=True)
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        r0, r1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        n = r1 - r0
        for i in range(n):
            pos = L - n + i
            if pos < 0:
                continue
            page = int(indices[int(indptr[b]) + pos // P])
            k[page, :, pos % P, :] = k_rows[r0 + i]
            v[page, :, pos % P, :] = v_rows[r0 + i]
    return k, v


def decode_pieces(q_bits, k_pool, v_pool, indptr, indices, seq_lens, sm_scale: float, P: int,
                  pieces) -> np.ndarray:
    """Split-then-merge decode over arbitrary pieces.

    pieces: iterable of (request b, head group u, first page p0, pages n) with
    the head groups of head_groups(); each (b, u) must be covered exactly once.
    Every piece yields a partial per query head of its group; each (b, u) merges
    its partials in the order given.
    """
    q = bf16_to_f64(q_bits)
    B, Hq, D = q.shape
    Hkv = np.asarray(k_pool).shape[1]
    G = Hq // Hkv
    HG, _ = head_groups(Hq, Hkv)
    parts = {}
    dense = {}
    for b, u, p0, n in pieces:
        b, u, p0, n = int(b), int(u), int(p0), int(n)
        L = int(seq_lens[b])
        if b not in dense:
            dense[b] = (gather_request(k_pool, indptr, indices, b, L, P),
                        gather_request(v_pool, indptr, indices, b, L, P))
        Kd, Vd = dense[b]
        t0, t1 = p0 * P, min(L, (p0 + n) * P)
        for hq in range(u * HG, (u + 1) * HG):
            h = kv_head_of(hq, G)
            parts.setdefault((b, hq), []).append(
                chunk_partial(q[b, hq], Kd[t0:t1, h, :], Vd[t0:t1, h, :], sm_scale))
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for (b, hq), pl in parts.items():
        out[b, hq] = merge_partials(pl)
    return out

