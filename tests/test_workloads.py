"""Checks of the seeded input generator (data only; no attention arithmetic)."""

import math

import numpy as np
import pytest
import torch

import workloads as W


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-39).astype(np.float32),  # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 1.0, 3.0e38, -3.0e38], np.float32),
        # exact ties: mantissa low half 0x8000 with even and odd kept bit
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x3F80FFFF], np.uint32).view(np.float32),
    ])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = W.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    assert W.f32_to_bf16_bits(np.array([np.nan], np.float32))[0] == W.BF16_QNAN


def test_deterministic():
    a, b = W.config(1), W.config(1)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k_pool, b.k_pool, equal_nan=True)
    assert [list(p) for p in a.page_lists] == [list(p) for p in b.page_lists]


def _check_private_layout(batch):
    idx = batch.kv_indices
    assert len(np.unique(idx)) == len(idx), "private pages must not repeat"
    assert idx.min() >= 0 and idx.max() < batch.num_pages
    for b, pl in enumerate(batch.page_lists):
        L = int(batch.seq_lens[b])
        assert (len(pl) - 1) * batch.P < L <= len(pl) * batch.P


@pytest.mark.parametrize("i", [1, 2, 3, 4])
def test_private_configs(i):
    batch = W.config(i)
    _check_private_layout(batch)
    exp = {1: (1, 8, 2, 64), 2: (4, 32, 8, 64), 3: (16, 32, 8, 128), 4: (1, 32, 8, 128)}[i]
    assert (batch.B, batch.Hq, batch.Hkv, batch.D, batch.P) == exp + (16,)
    assert batch.q.shape == (batch.B, batch.Hq, batch.D)
    assert batch.k_pool.shape == (batch.num_pages, batch.Hkv, batch.P, batch.D)
    assert batch.sm_scale == 1.0 / math.sqrt(batch.D)
    if i == 1:
        assert list(batch.seq_lens) == [37] and batch.num_pages == 64
        assert batch.forced_splits == (1, 3)
    if i == 2:
        assert list(batch.seq_lens) == [512] * 4 and batch.num_pages == 4096
    if i == 3:
        n = sum(len(p) for p in batch.page_lists)
        assert batch.num_pages == math.ceil(1.1 * n)
        assert batch.seq_lens.min() >= 1 and batch.seq_lens.max() <= 4096
    if i == 4:
        assert list(batch.seq_lens) == [32768] and batch.num_pages == 2048


def test_config5_shared_prefix_and_append():
    batch = W.config(5)
    assert batch.B == 64 and batch.append
    cached = batch.seq_lens.astype(np.int64) - 1
    assert cached.min() >= 16 and cached.max() <= 16384
    owners = {}
    for b, pl in enumerate(batch.page_lists):
        for j, p in enumerate(pl):
            owners.setdefault(int(p), set()).add((b, j))
    for p, uses in owners.items():
        if len(uses) > 1:
            groups = {b // 8 for b, _ in uses}
            js = {j for _, j in uses}
            assert len(groups) == 1 and len(js) == 1, "a shared page is one logical page of one group"
            for b, j in uses:
                assert (j + 1) * batch.P <= cached[b], "only full pages are shared"
    for b, pl in enumerate(batch.page_lists):
        last = int(pl[int(cached[b]) // batch.P])
        assert len(owners[last]) == 1, "the appended token lands in a private page"
    assert batch.shared_pages > 0


def test_poison_marks_exactly_unwritten_slots():
    batch = W.config(1)
    nan_slots = np.isnan(W.bf16_bits_to_f32(batch.k_pool[:, 0, :, 0]))
    pl = batch.page_lists[0]
    assert not nan_slots[pl[0]].any() and not nan_slots[pl[1]].any()
    assert not nan_slots[pl[2], :5].any() and nan_slots[pl[2], 5:].all()
    free = np.setdiff1d(np.arange(batch.num_pages), pl)
    assert nan_slots[free].all()


def test_permute_and_identity_keep_content():
    batch = W.config(1)
    for other in (W.permute_pool(batch, 3), W.identity_layout(batch)):
        for b in range(batch.B):
            a = batch.k_pool[batch.page_lists[b]]
            c = other.k_pool[other.page_lists[b]]
            assert np.array_equal(a.view(np.uint16), c.view(np.uint16))
