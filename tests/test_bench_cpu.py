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


def test_cpu_baseline_units_reassemble_the_oracle_decode():
    # The CPU baseline splits a decode call into per-request units of the
    # oracle; put back together they are the oracle's whole-batch answer.
    import oracle
    import workloads as W

    batch = W.make_batch(name="units", seed=17, B=3, Hq=8, Hkv=2, D=16, P=4,
                         lengths=np.array([9, 0, 14]))
    units, unit = bench.oracle_units(batch)
    assert units == [0, 2]
    got = np.zeros((batch.B, batch.Hq, batch.D))
    for b in units:
        got[b] = unit(b)[0]
    ip = oracle.kv_indptr(batch.seq_lens, batch.P)
    ref = oracle.decode(batch.q, batch.k_pool, batch.v_pool, ip, batch.kv_indices,
                        batch.seq_lens, batch.sm_scale, batch.P)
    assert np.array_equal(got, ref)


def test_cpu_baseline_reports_cores_and_model():
    import workloads as W

    batch = W.make_batch(name="units", seed=18, B=2, Hq=8, Hkv=2, D=16, P=4,
                         lengths=np.array([5, 7]), poison=False)
    r = bench.cpu_baseline(batch, 0.2)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["cpu"]
    assert r["value"] > 0 and "median of" in r["sample"]


def test_cpu_baseline_worker_processes():
    # the worker-process form on the tiny preset: workers rebuild the batch
    import workloads as W

    r = bench.cpu_baseline(W.config(1, poison=False), 0.1, cfg=1)
    assert r["cores"] == 1 and "worker processes" in r["sample"] and r["value"] > 0
