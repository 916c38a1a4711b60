"""Seeded synthetic inputs for paged-KV split-KV decode attention.

This module is shared by the fp64 oracle's tests and by the HIP path's tests
and benchmark.  It holds data generation only: random draws, bf16 encoding,
page placement in a pool and NaN poisoning.  It computes no part of the
attention method (no prefix sums, no scores, no softmax, no split plan).

The workloads follow the five decode batches the project studies (one query
token per request, grouped-query heads, page_size 16).  The pages describe the
K/V pool as a flat token pool addressed through a request-to-token table
(AstrAI compare v1.3.12..6f09b1d, astrai/inference/core/cache.py, PagePool
and KVStorage); here the pool is page-granular and head-major:

    K, V : bf16 bits, uint16 [num_pages][Hkv][page_size][D]

A request's pages are listed in logical order in ``page_lists[b]``; the flat
``kv_indices`` array is their concatenation in request order.

Draw order (one numpy PCG64 generator per batch): sequence lengths, page
permutation (and prefix sharing), q, K pool, V pool, then k_new / v_new.
All values are float32 standard normal draws rounded to bf16 by
round-to-nearest-even.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

BF16_QNAN = np.uint16(0x7FC0)

__all__ = [
    "BF16_QNAN",
    "DecodeBatch",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "normal_bf16",
    "make_batch",
    "make_prefill",
    "config",
    "CONFIG_NAMES",
    "permute_pool",
    "identity_layout",
    "to_device",
    "v_pool_channel_major",
    "v_pool_token_major",
    "k_pool_blocked",
    "k_pool_token_major",
    "TokenBatch",
    "make_tokens",
    "tokens_from_pages",
    "tokens_to_device",
]


def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even.

    NaN maps to the canonical quiet NaN 0x7FC0.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    r[np.isnan(x)] = BF16_QNAN
    return r


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit pattern (uint16) -> float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    """Draw float32 N(0,1) * scale and round it to bf16 bits."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x = x * np.float32(scale)
    return f32_to_bf16_bits(x)


@dataclass
class DecodeBatch:
    """One decode step's inputs for one layer.

    ``seq_lens[b]`` is the number of tokens request ``b`` attends to.  For a
    batch with ``append=True`` the last of those tokens is the one written this
    step (``k_new``/``v_new``); before the append its slot holds poison (or
    noise) like any other unwritten slot.
    """

    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    P: int
    num_pages: int
    seq_lens: np.ndarray  # int32 [B]
    page_lists: List[np.ndarray]  # int32 physical page ids per request, logical order
    q: np.ndarray  # uint16 [B, Hq, D]
    k_pool: np.ndarray  # uint16 [num_pages, Hkv, P, D]
    v_pool: np.ndarray  # uint16 [num_pages, Hkv, P, D]
    sm_scale: float
    append: bool = False
    k_new: Optional[np.ndarray] = None  # uint16 [B, Hkv, D]
    v_new: Optional[np.ndarray] = None  # uint16 [B, Hkv, D]
    forced_splits: Tuple[int, ...] = ()
    poisoned: bool = False
    shared_pages: int = 0  # pages referenced by more than one request
    notes: dict = field(default_factory=dict)
    # Prefill batches: query rows of every request, flattened, and their offsets.
    q_rows: Optional[np.ndarray] = None  # uint16 [total_q, Hq, D]
    qo_indptr: Optional[np.ndarray] = None  # int32 [B + 1]
    # Extend batches whose new tokens are not in the pool yet: their K/V rows,
    # one per query row, and the pool slots of those tokens hold poison.
    k_rows: Optional[np.ndarray] = None  # uint16 [total_q, Hkv, D]
    v_rows: Optional[np.ndarray] = None  # uint16 [total_q, Hkv, D]

    @property
    def kv_indices(self) -> np.ndarray:
        if not self.page_lists:
            return np.zeros(0, np.int32)
        return np.concatenate(self.page_lists).astype(np.int32)

    @property
    def kv_tokens(self) -> int:
        """Tokens attended summed over the batch (logical, shared pages counted per request)."""
        return int(np.sum(self.seq_lens, dtype=np.int64))

    @property
    def unique_pages(self) -> int:
        if not self.page_lists:
            return 0
        return int(np.unique(self.kv_indices).size)


def _pages_for(length: int, P: int) -> int:
    # Allocator bookkeeping: how many pages must be reserved to hold `length` tokens.
    return -(-int(length) // P)


def _fill_pools(rng, num_pages, Hkv, P, D):
    k = normal_bf16(rng, (num_pages, Hkv, P, D))
    v = normal_bf16(rng, (num_pages, Hkv, P, D))
    return k, v


def _poison(batch: DecodeBatch) -> None:
    """Write bf16 NaN into every pool slot that no request has written.

    Written slots: tokens [0, seq_len) of each request, except the append slot
    (the last token) of an append batch, which the append op writes.
    """
    P = batch.P
    written = np.zeros((batch.num_pages, P), dtype=bool)
    for b in range(batch.B):
        filled = int(batch.seq_lens[b]) - (1 if batch.append else 0)
        if batch.k_rows is not None:  # the new tokens of an extend batch come later
            filled = int(batch.seq_lens[b]) - int(batch.qo_indptr[b + 1] - batch.qo_indptr[b])
        pages = batch.page_lists[b]
        for j, page in enumerate(pages):
            ntok = min(P, filled - j * P)
            if ntok > 0:
                written[page, :ntok] = True
    mask = ~written  # [num_pages, P]
    kp = batch.k_pool.reshape(batch.num_pages, batch.Hkv, P, batch.D)
    vp = batch.v_pool.reshape(batch.num_pages, batch.Hkv, P, batch.D)
    sel = np.broadcast_to(mask[:, None, :, None], kp.shape)
    kp[sel] = BF16_QNAN
    vp[sel] = BF16_QNAN
    batch.poisoned = True


def make_batch(
    *,
    name: str,
    seed: int,
    B: int,
    Hq: int,
    Hkv: int,
    D: int,
    P: int,
    lengths,
    num_pages: Optional[int] = None,
    pool_slack: float = 0.10,
    q_scale: float = 1.0,
    append: bool = False,
    poison: bool = True,
    forced_splits: Tuple[int, ...] = (),
    rng: Optional[np.random.Generator] = None,
) -> DecodeBatch:
    """Generic batch with private pages at random places in a shuffled pool.

    ``lengths`` is either an int array of per-request token counts or a
    callable ``rng -> array`` (so that length draws come first from the
    generator).  ``num_pages`` defaults to ``ceil((1 + pool_slack) * pages)``.
    """
    if rng is None:
        rng = np.random.default_rng(np.random.PCG64(seed))
    seq = lengths(rng) if callable(lengths) else lengths
    seq = np.asarray(seq, dtype=np.int64).reshape(B)
    npages = [_pages_for(L, P) for L in seq]
    total = int(sum(npages))
    if num_pages is None:
        num_pages = max(1, math.ceil((1.0 + pool_slack) * total))
    if num_pages < total:
        raise ValueError("pool too small for the batch")
    perm = rng.permutation(num_pages).astype(np.int32)
    page_lists, cur = [], 0
    for n in npages:
        page_lists.append(perm[cur : cur + n].copy())
        cur += n
    q = normal_bf16(rng, (B, Hq, D), q_scale)
    k_pool, v_pool = _fill_pools(rng, num_pages, Hkv, P, D)
    k_new = v_new = None
    if append:
        k_new = normal_bf16(rng, (B, Hkv, D))
        v_new = normal_bf16(rng, (B, Hkv, D))
    batch = DecodeBatch(
        name=name, seed=seed, B=B, Hq=Hq, Hkv=Hkv, D=D, P=P, num_pages=num_pages,
        seq_lens=seq.astype(np.int32), page_lists=page_lists, q=q,
        k_pool=k_pool, v_pool=v_pool, sm_scale=1.0 / math.sqrt(D),
        append=append, k_new=k_new, v_new=v_new, forced_splits=forced_splits,
    )
    if poison:
        _poison(batch)
    return batch


def make_prefill(*, name: str, seed: int, Hq: int, Hkv: int, D: int, P: int, q_lens,
                 prefix_lens, poison: bool = True, q_scale: float = 1.0,
                 new_rows: bool = False) -> DecodeBatch:
    """Prefill / extend batch: request b has prefix_lens[b] cached tokens and
    q_lens[b] new ones (seq_len = prefix + q_len); its q_lens[b] query rows are
    stored flattened in ``q_rows`` with offsets ``qo_indptr``.  By default the
    new tokens' K/V are already in the pool.  With ``new_rows`` they are drawn
    as ``k_rows`` / ``v_rows`` (one row per query row) for an append to write,
    and their pool slots hold poison like any unwritten slot.  Draw order: pool
    layout and contents as in make_batch, the query rows, then k_rows and
    v_rows."""
    rng = np.random.default_rng(np.random.PCG64(seed))
    ql = np.asarray(q_lens, dtype=np.int64)
    pl = np.asarray(prefix_lens, dtype=np.int64)
    batch = make_batch(name=name, seed=seed, B=ql.size, Hq=Hq, Hkv=Hkv, D=D, P=P,
                       lengths=pl + ql, poison=False, rng=rng)
    offsets = np.zeros(ql.size + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(ql)
    batch.qo_indptr = offsets
    batch.q_rows = normal_bf16(rng, (int(offsets[-1]), Hq, D), q_scale)
    if new_rows:
        batch.k_rows = normal_bf16(rng, (int(offsets[-1]), Hkv, D))
        batch.v_rows = normal_bf16(rng, (int(offsets[-1]), Hkv, D))
    if poison:
        _poison(batch)
    return batch


def _config1(poison: bool, seed: int) -> DecodeBatch:
    # Tiny: one request of 37 tokens (pages of 16, 16, 5) at permuted places in
    # a 64-page pool; checked with 1 and with 3 KV splits.
    return make_batch(
        name="tiny", seed=seed, B=1, Hq=8, Hkv=2, D=64, P=16,
        lengths=np.array([37]), num_pages=64, poison=poison, forced_splits=(1, 3),
    )


def _config2(poison: bool, seed: int) -> DecodeBatch:
    # 1B-GQA-like layer: 4 requests of 512 tokens in a shuffled 4096-page pool.
    return make_batch(
        name="gqa1b_b4_l512", seed=seed, B=4, Hq=32, Hkv=8, D=64, P=16,
        lengths=np.full(4, 512), num_pages=4096, poison=poison,
    )


def _config3(poison: bool, seed: int) -> DecodeBatch:
    # Ragged: 16 requests, lengths uniform in [1, 4096], pool = used pages + 10%.
    return make_batch(
        name="ragged_b16_4k", seed=seed, B=16, Hq=32, Hkv=8, D=128, P=16,
        lengths=lambda r: r.integers(1, 4097, size=16), poison=poison,
    )


def _config4(poison: bool, seed: int) -> DecodeBatch:
    # Long context: one request of 32768 tokens over 2048 shuffled pages,
    # q scaled by 2 to sharpen the softmax.
    return make_batch(
        name="long_b1_32k", seed=seed, B=1, Hq=32, Hkv=8, D=128, P=16,
        lengths=np.array([32768]), num_pages=2048, q_scale=2.0, poison=poison,
    )


def _config5(poison: bool, seed: int) -> DecodeBatch:
    """Mixed batch of 64 with page-aligned shared prefixes and one append.

    Cached lengths L_i are log-uniform in [16, 16384]; attention runs over
    L_i + 1 tokens (the appended one included).  Requests 8g..8g+7 alias their
    first s_i = min(64, L_i // 16) logical pages to the group's shared pages;
    only full pages are shared, so the appended token lands in a private page.
    """
    B, Hq, Hkv, D, P = 64, 32, 8, 128, 16
    rng = np.random.default_rng(np.random.PCG64(seed))
    u = rng.uniform(math.log(16.0), math.log(16384.0), size=B)
    cached = np.clip(np.floor(np.exp(u)), 16, 16384).astype(np.int64)
    seq = cached + 1
    share = np.minimum(64, cached // P)
    groups = B // 8
    group_shared = [int(share[8 * g : 8 * g + 8].max()) for g in range(groups)]
    private = [_pages_for(seq[i], P) - int(share[i]) for i in range(B)]
    unique = sum(group_shared) + sum(private)
    num_pages = math.ceil(1.10 * unique)
    perm = rng.permutation(num_pages).astype(np.int32)
    cur = 0
    shared_sets = []
    for g in range(groups):
        shared_sets.append(perm[cur : cur + group_shared[g]])
        cur += group_shared[g]
    page_lists = []
    for i in range(B):
        own = perm[cur : cur + private[i]]
        cur += private[i]
        page_lists.append(np.concatenate([shared_sets[i // 8][: share[i]], own]).astype(np.int32))
    q = normal_bf16(rng, (B, Hq, D))
    k_pool, v_pool = _fill_pools(rng, num_pages, Hkv, P, D)
    k_new = normal_bf16(rng, (B, Hkv, D))
    v_new = normal_bf16(rng, (B, Hkv, D))
    batch = DecodeBatch(
        name="mixed_b64_shared", seed=seed, B=B, Hq=Hq, Hkv=Hkv, D=D, P=P,
        num_pages=num_pages, seq_lens=seq.astype(np.int32), page_lists=page_lists,
        q=q, k_pool=k_pool, v_pool=v_pool, sm_scale=1.0 / math.sqrt(D),
        append=True, k_new=k_new, v_new=v_new, shared_pages=sum(group_shared),
    )
    if poison:
        _poison(batch)
    return batch


_CONFIGS = {1: _config1, 2: _config2, 3: _config3, 4: _config4, 5: _config5}
CONFIG_NAMES = {
    1: "tiny",
    2: "gqa1b_b4_l512",
    3: "ragged_b16_4k",
    4: "long_b1_32k",
    5: "mixed_b64_shared",
}


def config(i: int, poison: bool = True, seed: Optional[int] = None) -> DecodeBatch:
    """Preset workload ``i`` in 1..5 (default seed = i)."""
    return _CONFIGS[i](poison, i if seed is None else seed)


def permute_pool(batch: DecodeBatch, seed: int) -> DecodeBatch:
    """Relabel physical pages by a random permutation pi.

    Page p of the old pool becomes page pi[p] of the new one and every page
    list is mapped through pi; the logical content of each request is unchanged.
    """
    rng = np.random.default_rng(np.random.PCG64(seed))
    pi = rng.permutation(batch.num_pages).astype(np.int32)
    k = np.empty_like(batch.k_pool)
    v = np.empty_like(batch.v_pool)
    k[pi] = batch.k_pool
    v[pi] = batch.v_pool
    out = DecodeBatch(**{**batch.__dict__})
    out.k_pool, out.v_pool = k, v
    out.page_lists = [pi[pl] for pl in batch.page_lists]
    return out


def identity_layout(batch: DecodeBatch) -> DecodeBatch:
    """Same logical content with request b's pages stored consecutively, in order.

    Request b's logical page j becomes physical page (sum of earlier requests'
    page counts) + j; the pool holds exactly the used pages.
    """
    counts = [len(pl) for pl in batch.page_lists]
    total = int(sum(counts))
    k = np.empty((total,) + batch.k_pool.shape[1:], np.uint16)
    v = np.empty_like(k)
    lists, cur = [], 0
    for pl in batch.page_lists:
        n = len(pl)
        k[cur : cur + n] = batch.k_pool[pl]
        v[cur : cur + n] = batch.v_pool[pl]
        lists.append(np.arange(cur, cur + n, dtype=np.int32))
        cur += n
    out = DecodeBatch(**{**batch.__dict__})
    out.k_pool, out.v_pool, out.page_lists, out.num_pages = k, v, lists, total
    return out


def v_pool_channel_major(v_pool: np.ndarray) -> np.ndarray:
    """[pages][Hkv][P][D] -> [pages][Hkv][P/16][D][16]: the device layout of V
    tiles (each 16-token step of a page channel-major)."""
    n, h, p, d = v_pool.shape
    return np.ascontiguousarray(v_pool.reshape(n, h, p // 16, 16, d).transpose(0, 1, 2, 4, 3))


def v_pool_token_major(v_dev: np.ndarray) -> np.ndarray:
    """Inverse of v_pool_channel_major."""
    n, h, s, d, t = v_dev.shape
    return np.ascontiguousarray(v_dev.transpose(0, 1, 2, 4, 3).reshape(n, h, s * t, d))


def k_pool_blocked(k_pool: np.ndarray) -> np.ndarray:
    """[pages][Hkv][P][D] -> [pages][Hkv][P/16][D/8][16][8]: the device layout
    of K tiles (each 16-token step of a page in 8-channel blocks)."""
    n, h, p, d = k_pool.shape
    return np.ascontiguousarray(
        k_pool.reshape(n, h, p // 16, 16, d // 8, 8).transpose(0, 1, 2, 4, 3, 5))


def k_pool_token_major(k_dev: np.ndarray) -> np.ndarray:
    """Inverse of k_pool_blocked."""
    n, h, s, d8, t, e = k_dev.shape
    return np.ascontiguousarray(k_dev.transpose(0, 1, 2, 4, 3, 5).reshape(n, h, s * t, d8 * e))


def to_device(batch: DecodeBatch, device="cuda:0") -> dict:
    """Copy a batch's arrays to device tensors (bf16 bits as int16, indices as int32).

    Returns a dict with q, k_pool, v_pool, seq_lens, kv_indices and, for an
    append batch, k_new and v_new.  The batch keeps K and V token-major; the
    device copies use the library's tile layouts (inside each (page, head) tile,
    P / 16 steps of K [D/8][16][8] and V [D][16]).  Data movement only.
    """
    import torch

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)

    d = {
        "q": bits(batch.q),
        "k_pool": bits(k_pool_blocked(batch.k_pool)),
        "v_pool": bits(v_pool_channel_major(batch.v_pool)),
        "seq_lens": torch.from_numpy(batch.seq_lens.astype(np.int32)).to(device),
        "kv_indices": torch.from_numpy(batch.kv_indices.astype(np.int32)).to(device),
    }
    if batch.append:
        d["k_new"] = bits(batch.k_new)
        d["v_new"] = bits(batch.v_new)
    if batch.q_rows is not None:
        d["q_rows"] = bits(batch.q_rows)
        d["qo_indptr"] = torch.from_numpy(batch.qo_indptr.astype(np.int32)).to(device)
    if batch.k_rows is not None:
        d["k_rows"] = bits(batch.k_rows)
        d["v_rows"] = bits(batch.v_rows)
    return d


# ------------------------------------------------------------ token-major K/V

@dataclass
class TokenBatch:
    """Decode inputs over token-major K/V: one row [Hkv][D] per token slot.

    Token t of request b is slot ``slot_table[b, t]`` (the token-level mode:
    a request-to-token table used as a page table with page size 1) or, when
    ``slot_table`` is None, slot ``b * stride + t`` (the contiguous layout
    [batch, seq, kv_heads, head_dim], flattened over batch and seq).  Table
    entries at t >= seq_lens[b] are -1 and are not read.
    """

    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    seq_lens: np.ndarray  # int32 [B]
    stride: int  # table row length / tokens per request row of the contiguous layout
    slot_table: Optional[np.ndarray]  # int32 [B, stride] or None (contiguous)
    num_slots: int
    q: np.ndarray  # uint16 [B, Hq, D]
    k_cache: np.ndarray  # uint16 [num_slots, Hkv, D]
    v_cache: np.ndarray  # uint16 [num_slots, Hkv, D]
    sm_scale: float
    poisoned: bool = False


def make_tokens(*, name: str, seed: int, B: int, Hq: int, Hkv: int, D: int, lengths,
                table: bool = True, stride: Optional[int] = None, slot_slack: float = 0.10,
                poison: bool = True) -> TokenBatch:
    """Token-major batch.  With ``table`` the tokens of all requests sit at
    random slots of a shuffled cache of ceil((1 + slot_slack) * tokens) slots;
    without it the cache is the contiguous [B, stride, Hkv, D] array.  Unwritten
    slots hold bf16 NaN when ``poison``.  Draw order: lengths, slot permutation
    (table mode), q, K cache, V cache."""
    rng = np.random.default_rng(np.random.PCG64(seed))
    seq = lengths(rng) if callable(lengths) else lengths
    seq = np.asarray(seq, dtype=np.int64).reshape(B)
    S = int(stride) if stride is not None else max(1, int(seq.max(initial=0)))
    if int(seq.max(initial=0)) > S:
        raise ValueError("stride below the longest request")
    total = int(seq.sum())
    slot_table = None
    written = None
    if table:
        num_slots = max(1, math.ceil((1.0 + slot_slack) * total))
        perm = rng.permutation(num_slots).astype(np.int32)
        slot_table = np.full((B, S), -1, dtype=np.int32)
        cur = 0
        for b in range(B):
            L = int(seq[b])
            slot_table[b, :L] = perm[cur : cur + L]
            cur += L
        written = np.zeros(num_slots, dtype=bool)
        written[perm[:total]] = True
    else:
        num_slots = B * S
        written = np.zeros((B, S), dtype=bool)
        for b in range(B):
            written[b, : int(seq[b])] = True
        written = written.reshape(-1)
    q = normal_bf16(rng, (B, Hq, D))
    k = normal_bf16(rng, (num_slots, Hkv, D))
    v = normal_bf16(rng, (num_slots, Hkv, D))
    if poison:
        k[~written] = BF16_QNAN
        v[~written] = BF16_QNAN
    return TokenBatch(name=name, seed=seed, B=B, Hq=Hq, Hkv=Hkv, D=D,
                      seq_lens=seq.astype(np.int32), stride=S, slot_table=slot_table,
                      num_slots=num_slots, q=q, k_cache=k, v_cache=v,
                      sm_scale=1.0 / math.sqrt(D), poisoned=poison)


def tokens_from_pages(batch: DecodeBatch) -> TokenBatch:
    """The same K/V as a paged batch, stored token-major: slot p * P + o holds
    offset o of page p, and the table lists each request's token slots."""
    P = batch.P
    k = np.ascontiguousarray(np.swapaxes(batch.k_pool, 1, 2)).reshape(-1, batch.Hkv, batch.D)
    v = np.ascontiguousarray(np.swapaxes(batch.v_pool, 1, 2)).reshape(-1, batch.Hkv, batch.D)
    S = max(1, int(np.max(batch.seq_lens, initial=0)))
    table = np.full((batch.B, S), -1, dtype=np.int32)
    for b in range(batch.B):
        L = int(batch.seq_lens[b])
        t = np.arange(L)
        table[b, :L] = batch.page_lists[b][t // P] * P + t % P
    return TokenBatch(name=batch.name + "_tokens", seed=batch.seed, B=batch.B, Hq=batch.Hq,
                      Hkv=batch.Hkv, D=batch.D, seq_lens=batch.seq_lens.copy(), stride=S,
                      slot_table=table, num_slots=k.shape[0], q=batch.q, k_cache=k,
                      v_cache=v, sm_scale=batch.sm_scale, poisoned=batch.poisoned)


def tokens_to_device(tb: TokenBatch, device="cuda:0") -> dict:
    """Device copies of a token batch (bf16 bits as int16; the slot table, if
    any, as int32).  Data movement only."""
    import torch

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)

    d = {
        "q": bits(tb.q),
        "k_cache": bits(tb.k_cache),
        "v_cache": bits(tb.v_cache),
        "seq_lens": torch.from_numpy(tb.seq_lens.astype(np.int32)).to(device),
        "slot_table": None,
    }
    if tb.slot_table is not None:
        d["slot_table"] = torch.from_numpy(np.ascontiguousarray(tb.slot_table, np.int32)).to(device)
    return d
