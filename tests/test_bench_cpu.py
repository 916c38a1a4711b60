"""Host-side byte counts of bench.py (no GPU)."""

from types import SimpleNamespace

import numpy as np

import bench


def _batch(page_lists, seq_lens, P=16, Hkv=8, D=128):
    return SimpleNamespace(page_lists=[np.asarray(p, np.int32) for p in page_lists],
                           seq_lens=np.asarray(seq_lens, np.int32), P=P, Hkv=Hkv, D=D)


def test_unique_bytes_equal_logical_without_sharing():
    b = _batch([[4, 9, 2], [7], [0, 1]], [40, 16, 17])
    assert bench.unique_kv_bytes(b) == (40 + 16 + 17) * 8 * 128 * 4


def test_unique_bytes_count_a_shared_prefix_once():
    # Requests 0..2 share the two full pages 10 and 11 (32 tokens) and then
    # own private pages; request 3 shares nothing.  Unique tokens: the shared
    # 32 once, plus every request's tokens past its shared prefix.
    lists = [[10, 11, 20], [10, 11, 21, 22], [10, 30], [40]]
    lens = [35, 60, 20, 9]
    shared = [2, 2, 1, 0]
    unique_tokens = 32 + sum(L - 16 * s for L, s in zip(lens, shared))
    b = _batch(lists, lens)
    assert bench.unique_kv_bytes(b) == unique_tokens * 8 * 128 * 4
    assert bench.unique_kv_bytes(b) < sum(lens) * 8 * 128 * 4
