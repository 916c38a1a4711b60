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
  (cache.py, bind_tasks: write_pos = seq_lens - 1).

Readings taken where the pages are silent:
kv_indptr in pages; KV head of query head hq is hq // G; seq_len includes
the token appended this step; empty chunks have lse = -inf and weight 0; a
request with seq_len 0 gets a zero output row; chunks are contiguous runs of
pages split as evenly as possible; the split planner rule below is this
library's own (the pages give only its goal: enough blocks to fill the chip).

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
    "chunk_partial",
    "merge_partials",
    "even_page_ranges",
    "plan_splits",
    "decode_split",
    "append_kv",
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


def plan_splits(seq_lens, P: int, Hkv: int, max_splits: int, target_items: int,
                min_chunk: int, forced: int = 0) -> dict:
    """This library's split plan (not from the pages, which give only its goal).

    chunk  = max(min_chunk, ceil(Hkv * N / target_items)) pages, N = total pages;
    nsplit = min(max_splits, ceil(n_b / chunk)) for a request of n_b >= 1 pages,
             0 for an empty request;
    forced > 0 overrides: nsplit = min(forced, n_b, max_splits).
    Split s of request b covers even_page_ranges(n_b, nsplit_b)[s].
    """
    n = page_counts(seq_lens, P)
    N = int(n.sum())
    chunk = max(int(min_chunk), -(-Hkv * N // int(target_items))) if N > 0 else int(min_chunk)
    nsplit = np.zeros(n.size, dtype=np.int64)
    for b, nb in enumerate(n):
        nb = int(nb)
        if nb == 0:
            continue
        if forced > 0:
            nsplit[b] = min(forced, nb, max_splits)
        else:
            nsplit[b] = min(max_splits, -(-nb // chunk))
    split_indptr = np.zeros(n.size + 1, dtype=np.int64)
    split_indptr[1:] = np.cumsum(nsplit)
    return {"chunk": chunk, "total_pages": N, "nsplit": nsplit,
            "split_indptr": split_indptr, "num_items": int(split_indptr[-1])}


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
