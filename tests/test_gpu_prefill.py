"""Parity of the HIP paged prefill / extend kernel with the fp64 oracle.

Query rows of ragged lengths attend to each request's paged KV (prefix plus the
new tokens), with and without the causal mask, for G = 1 .. 8, 10 and 12, head dims
64 and 128 and pages of 16, 32 and 64 tokens.  The metadata comes from
pkv_build_metadata, as in a serving step.  Outputs start as NaN, so a row the
kernel skips shows up.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_split_attn_amd as pkv
import workloads as W
from gpu_util import compare, say

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_g4": dict(Hq=8, Hkv=2, D=64, P=16, q_lens=[3, 1, 17, 40], prefix_lens=[5, 0, 30, 100]),
    "g1_d128": dict(Hq=4, Hkv=4, D=128, P=16, q_lens=[16, 33, 7], prefix_lens=[0, 64, 200]),
    "g2_p32": dict(Hq=8, Hkv=4, D=128, P=32, q_lens=[9, 40], prefix_lens=[31, 0]),
    "g3": dict(Hq=24, Hkv=8, D=64, P=16, q_lens=[11, 6], prefix_lens=[4, 20]),
    "g8_p64": dict(Hq=32, Hkv=4, D=128, P=64, q_lens=[50, 3], prefix_lens=[77, 128]),
    "square_512": dict(Hq=32, Hkv=8, D=128, P=16, q_lens=[512, 300], prefix_lens=[0, 0]),
    # row tiles of 3 tokens x 5 heads, 2 x 6 and 2 x 7 (15, 12 and 14 of 16 rows)
    "g5": dict(Hq=10, Hkv=2, D=128, P=16, q_lens=[20, 1, 33], prefix_lens=[7, 40, 0]),
    "g6_d64": dict(Hq=24, Hkv=4, D=64, P=32, q_lens=[9, 50], prefix_lens=[100, 3]),
    "g7": dict(Hq=14, Hkv=2, D=128, P=16, q_lens=[17, 64], prefix_lens=[0, 31]),
    # two row-tile head groups of five per KV head; three of four at G = 12
    "g10": dict(Hq=20, Hkv=2, D=128, P=16, q_lens=[25, 6], prefix_lens=[12, 70]),
    "g12": dict(Hq=24, Hkv=2, D=64, P=16, q_lens=[11, 40], prefix_lens=[33, 0]),
}


def run_prefill(batch, causal, max_q_len=None, seq_lens=None, edit=None, pools_out=None):
    """Metadata + (for a batch with new K/V rows) pkv_append_kv_ragged + prefill."""
    dev = "cuda:0"
    t = W.to_device(batch, dev)
    if edit is not None:  # change the device inputs (e.g. corrupt a page id)
        edit(t)
    if seq_lens is not None:  # attend to fewer keys than the pool holds
        t["seq_lens"] = torch.from_numpy(np.asarray(seq_lens, np.int32)).to(dev)
    desc = pkv.Desc(max_batch=batch.B, num_q_heads=batch.Hq, num_kv_heads=batch.Hkv,
                    head_dim=batch.D, page_size=batch.P)
    ws = torch.empty(pkv.pkv_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    kv_indptr = torch.empty(batch.B + 1, dtype=torch.int32, device=dev)
    pkv.pkv_build_metadata(desc, t["seq_lens"], 0, kv_indptr, ws)
    out = torch.full(tuple(batch.q_rows.shape), 0x7FC0, dtype=torch.int16, device=dev)
    q_lens = np.diff(batch.qo_indptr)
    if batch.k_rows is not None:  # the new tokens reach the pool through the library
        pkv.pkv_append_kv_ragged(pkv.Pool(t["k_pool"], t["v_pool"]), t["k_rows"], t["v_rows"],
                                 t["qo_indptr"], kv_indptr, t["kv_indices"], t["seq_lens"],
                                 int(q_lens.max()))
    pkv.pkv_prefill(pkv.Pool(t["k_pool"], t["v_pool"]), desc, t["q_rows"], t["qo_indptr"],
                    kv_indptr, t["kv_indices"], t["seq_lens"],
                    int(q_lens.max()) if max_q_len is None else max_q_len, causal,
                    batch.sm_scale, out)
    torch.cuda.synchronize()
    if pools_out is not None:
        pools_out.append((W.k_pool_token_major(t["k_pool"].cpu().numpy().view(np.uint16)),
                          W.v_pool_token_major(t["v_pool"].cpu().numpy().view(np.uint16))))
    return out.cpu().numpy().view(np.uint16)


def oracle_pools(batch):
    """The pool after the batch's new K/V rows are written (unchanged without them)."""
    if batch.k_rows is None:
        return batch.k_pool, batch.v_pool
    ip = oracle.kv_indptr(batch.seq_lens, batch.P)
    return oracle.append_kv_rows(batch.k_pool, batch.v_pool, batch.k_rows, batch.v_rows,
                                 batch.qo_indptr, ip, batch.kv_indices, batch.seq_lens, batch.P)


def oracle_prefill(batch, causal):
    ip = oracle.kv_indptr(batch.seq_lens, batch.P)
    k, v = oracle_pools(batch)
    return oracle.prefill(batch.q_rows, k, v, ip, batch.kv_indices,
                          batch.seq_lens, batch.qo_indptr, batch.sm_scale, batch.P, causal)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("case", list(CASES))
def test_prefill_parity(case, causal):
    say(f"prefill {case} causal={causal}")
    batch = W.make_prefill(name=case, seed=sum(map(ord, case)), **CASES[case])
    got = run_prefill(batch, causal)
    compare(got, oracle_prefill(batch, causal), f"prefill {case} causal={causal}")


@pytest.mark.parametrize("scale", [-1.0 / np.sqrt(128.0), 0.0, 1.0],
                         ids=["negative", "zero", "large"])
def test_prefill_scale_sign_and_size(scale):
    # The kernel compares raw scores against a threshold divided by a positive
    # scale: a negative scale's sign goes into q, a zero scale gives equal
    # weights to the visible keys, and a large one (scores with a standard
    # deviation of about 16 log2 units) makes many steps raise the running max.
    # V is scaled by 1/4 (exact in bf16): a sharp softmax puts outputs near
    # single V values, and at |o| ~ 3 the bf16 rounding of the output alone is
    # 7.8e-3, which with the bf16 weights' rounding exceeds the 1e-2 bar at
    # scale 1 for any kernel that rounds them (1.4e-2 measured).
    say(f"prefill sm_scale={scale}")
    batch = W.make_prefill(name="scale", seed=9, Hq=8, Hkv=2, D=128, P=16, q_lens=[40, 7, 1],
                           prefix_lens=[30, 100, 0])
    v_quarter = W.f32_to_bf16_bits(W.bf16_bits_to_f32(batch.v_pool) * np.float32(0.25))
    batch = dataclasses.replace(batch, sm_scale=scale, v_pool=v_quarter)
    for causal in (True, False):
        got = run_prefill(batch, causal)
        compare(got, oracle_prefill(batch, causal), f"sm_scale={scale} causal={causal}")


def test_prefill_single_rows_match_decode_semantics():
    # one new token per request: the causal prefill is the decode of that token
    say("prefill one row per request")
    batch = W.make_prefill(name="one", seed=5, Hq=32, Hkv=8, D=128, P=16, q_lens=[1, 1, 1, 1],
                           prefix_lens=[0, 15, 16, 4000])
    got = run_prefill(batch, True)
    ip = oracle.kv_indptr(batch.seq_lens, batch.P)
    dec = oracle.decode(batch.q_rows, batch.k_pool, batch.v_pool, ip, batch.kv_indices,
                        batch.seq_lens, batch.sm_scale, batch.P)
    compare(got, dec, "prefill q_len 1 vs decode oracle")


def test_prefill_ragged_extend_batch():
    # Many requests of a serving step's extend phase: ragged new-token counts
    # (zero included) over ragged cached prefixes, G = 4, D = 128.  The new
    # tokens' K/V start outside the pool (their slots hold NaN) and are written
    # by pkv_append_kv_ragged before the prefill, as in a serving step.
    rng = np.random.default_rng(np.random.PCG64(61))
    q_lens = rng.integers(0, 41, size=24)
    q_lens[[3, 17]] = 0
    prefix = rng.integers(0, 301, size=24)
    say(f"prefill ragged extend: {int(q_lens.sum())} rows, {int((q_lens + prefix).sum())} keys")
    batch = W.make_prefill(name="extend24", seed=61, Hq=32, Hkv=8, D=128, P=16,
                           q_lens=q_lens, prefix_lens=prefix, new_rows=True)
    k_ref, v_ref = oracle_pools(batch)
    for causal in (True, False):
        pools = []
        got = run_prefill(batch, causal, pools_out=pools)
        assert np.array_equal(pools[0][0], k_ref) and np.array_equal(pools[0][1], v_ref)
        compare(got, oracle_prefill(batch, causal), f"ragged extend causal={causal}")


APPEND_ROWS_CASES = [  # (D, P, new rows per request, prefix per request)
    (128, 16, [0, 1, 15, 16, 17, 300], [5, 0, 16, 1, 31, 40]),
    (64, 16, [300, 17, 1, 0], [0, 3, 64, 9]),
    (128, 32, [1, 15, 16, 17, 300, 0], [31, 0, 1, 63, 7, 12]),
    (64, 64, [17, 300, 0, 16, 1, 15], [64, 1, 5, 0, 127, 200]),
    (128, 64, [300, 1], [70, 0]),
]


@pytest.mark.parametrize("D,P,q_lens,prefix", APPEND_ROWS_CASES,
                         ids=[f"d{c[0]}_p{c[1]}" for c in APPEND_ROWS_CASES])
def test_append_rows_bit_exact(D, P, q_lens, prefix):
    # pkv_append_kv_ragged writes every new row into the tile layout at
    # positions seq_len - n .. seq_len - 1: pool bytes equal the oracle's.
    say(f"append rows D={D} P={P} n={q_lens}")
    batch = W.make_prefill(name=f"rows_d{D}_p{P}", seed=D + P + sum(q_lens), Hq=8, Hkv=2, D=D,
                           P=P, q_lens=q_lens, prefix_lens=prefix, new_rows=True)
    dev = "cuda:0"
    t = W.to_device(batch, dev)
    kv_indptr = torch.from_numpy(oracle.kv_indptr(batch.seq_lens, P).astype(np.int32)).to(dev)
    pool = pkv.Pool(t["k_pool"], t["v_pool"])
    pkv.pkv_append_kv_ragged(pool, t["k_rows"], t["v_rows"], t["qo_indptr"], kv_indptr,
                             t["kv_indices"], t["seq_lens"], max(q_lens))
    torch.cuda.synchronize()
    k_ref, v_ref = oracle_pools(batch)
    k = W.k_pool_token_major(t["k_pool"].cpu().numpy().view(np.uint16))
    v = W.v_pool_token_major(t["v_pool"].cpu().numpy().view(np.uint16))
    assert np.array_equal(k, k_ref)
    assert np.array_equal(v, v_ref)
    # a bound below the longest request writes exactly its first rows
    t2 = W.to_device(batch, dev)
    cut = 16
    pkv.pkv_append_kv_ragged(pkv.Pool(t2["k_pool"], t2["v_pool"]), t2["k_rows"], t2["v_rows"],
                             t2["qo_indptr"], kv_indptr, t2["kv_indices"], t2["seq_lens"], cut)
    torch.cuda.synchronize()
    qo = batch.qo_indptr
    keep_rows = np.concatenate([np.arange(qo[b], qo[b] + min(cut, qo[b + 1] - qo[b]))
                                for b in range(batch.B)]).astype(np.int64)
    # expected: rows past the bound keep their pool contents
    k_exp, v_exp = batch.k_pool.copy(), batch.v_pool.copy()
    kr, vr = batch.k_rows.copy(), batch.v_rows.copy()
    drop = np.setdiff1d(np.arange(int(qo[-1])), keep_rows)
    ip_h = oracle.kv_indptr(batch.seq_lens, P)
    k_all, v_all = oracle.append_kv_rows(k_exp, v_exp, kr, vr, qo, ip_h, batch.kv_indices,
                                         batch.seq_lens, P)
    for r in drop:  # restore the slots of the rows the bound leaves out
        b = int(np.searchsorted(qo, r, side="right") - 1)
        n = int(qo[b + 1] - qo[b])
        pos = int(batch.seq_lens[b]) - n + int(r - qo[b])
        page = int(batch.page_lists[b][pos // P])
        k_all[page, :, pos % P] = batch.k_pool[page, :, pos % P]
        v_all[page, :, pos % P] = batch.v_pool[page, :, pos % P]
    assert np.array_equal(W.k_pool_token_major(t2["k_pool"].cpu().numpy().view(np.uint16)), k_all)
    assert np.array_equal(W.v_pool_token_major(t2["v_pool"].cpu().numpy().view(np.uint16)), v_all)


def test_prefill_rows_without_keys_are_zero():
    # Fewer keys than query rows (seq_len below q_len): with the causal mask
    # aligned to the end of the keys, the first rows see none and are zero.
    batch = W.make_prefill(name="nokeys", seed=62, Hq=8, Hkv=2, D=64, P=16, q_lens=[40],
                           prefix_lens=[0])
    short = np.array([25], np.int32)
    got = run_prefill(batch, True, seq_lens=short)
    ip = oracle.kv_indptr(short, batch.P)
    ref = oracle.prefill(batch.q_rows, batch.k_pool, batch.v_pool, ip, batch.kv_indices, short,
                         batch.qo_indptr, batch.sm_scale, batch.P, True)
    assert np.array_equal(got[:15], np.zeros_like(got[:15]))
    compare(got, ref, "rows without keys")


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_prefill_bad_page_id_drops_its_keys(causal):
    # Request 1's second page id points one past the pool.  The kernel skips
    # that page's 16 keys; they lie below every row's causal limit, so the
    # result is the attention over the request without that page (positions
    # after it shift down by a page in the reduced problem and every limit
    # with them).  The other requests are untouched.
    say(f"prefill bad page id causal={causal}")
    batch = W.make_prefill(name="badpage", seed=63, Hq=32, Hkv=8, D=128, P=16,
                           q_lens=[5, 20, 7], prefix_lens=[40, 64, 30])
    pos = len(batch.page_lists[0]) + 1

    def corrupt(t):
        t["kv_indices"][pos] = batch.num_pages
    got = run_prefill(batch, causal, edit=corrupt)
    ref = oracle_prefill(batch, causal)
    qo = batch.qo_indptr
    for b in (0, 2):
        compare(got[qo[b]:qo[b + 1]], ref[qo[b]:qo[b + 1]], f"untouched request {b}")
    pages = np.delete(batch.page_lists[1], 1).astype(np.int32)
    L = np.array([int(batch.seq_lens[1]) - batch.P], np.int32)
    q1 = batch.q_rows[qo[1]:qo[2]]
    ref1 = oracle.prefill(q1, batch.k_pool, batch.v_pool, oracle.kv_indptr(L, batch.P), pages, L,
                          np.array([0, len(q1)], np.int32), batch.sm_scale, batch.P, causal)
    compare(got[qo[1]:qo[2]], ref1, "request 1 without its skipped page")


def test_prefill_bench_batch_sampled_rows():
    # The benchmark's prefill batch and launch (4 requests x 1024 new tokens,
    # no prefix, causal, Hq 32, Hkv 8, D 128, max_q_len 1024), checked on
    # sampled query rows (every head of each), which the oracle computes one
    # by one: first and last rows of each request plus random ones.
    say("prefill benchmark batch, sampled rows")
    batch = W.make_prefill(name="prefill_b4_q1024", seed=7, Hq=32, Hkv=8, D=128, P=16,
                           q_lens=[1024] * 4, prefix_lens=[0] * 4, poison=False)
    got = run_prefill(batch, True, max_q_len=1024)
    ip = oracle.kv_indptr(batch.seq_lens, batch.P)
    rng = np.random.default_rng(np.random.PCG64(71))
    rows = sorted(set(rng.integers(0, 4096, size=40).tolist())
                  | {0, 1, 1023, 1024, 2047, 3071, 3072, 4095})
    q = oracle.bf16_to_f64(batch.q_rows)
    G = batch.Hq // batch.Hkv
    kv = {}
    ref = np.zeros((len(rows), batch.Hq, batch.D))
    for j, r in enumerate(rows):
        b, i = divmod(r, 1024)
        if b not in kv:
            L = int(batch.seq_lens[b])
            kv[b] = (oracle.gather_request(batch.k_pool, ip, batch.kv_indices, b, L, batch.P),
                     oracle.gather_request(batch.v_pool, ip, batch.kv_indices, b, L, batch.P))
        Kd, Vd = kv[b]
        for hq in range(batch.Hq):
            h = oracle.kv_head_of(hq, G)
            ref[j, hq] = oracle.softmax_attend(q[r, hq], Kd[:i + 1, h, :], Vd[:i + 1, h, :],
                                               batch.sm_scale)
    compare(got[rows], ref, f"benchmark prefill batch, {len(rows)} sampled rows")


def test_prefill_graph_replay_matches_eager():
    # One prefill launch captured in a hipGraph and replayed with new query
    # rows written in place between replays (the caller's buffers stay put):
    # every replay is bitwise the eager launch on the same inputs, and both
    # match the oracle.
    say("prefill graph replay")
    batch = W.make_prefill(name="graph_pf", seed=64, Hq=32, Hkv=8, D=128, P=16,
                           q_lens=[40, 7, 64], prefix_lens=[100, 0, 33])
    dev = "cuda:0"
    t = W.to_device(batch, dev)
    desc = pkv.Desc(max_batch=batch.B, num_q_heads=batch.Hq, num_kv_heads=batch.Hkv,
                    head_dim=batch.D, page_size=batch.P)
    ws = torch.empty(pkv.pkv_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    kv_indptr = torch.empty(batch.B + 1, dtype=torch.int32, device=dev)
    pkv.pkv_build_metadata(desc, t["seq_lens"], 0, kv_indptr, ws)
    out = torch.full(tuple(batch.q_rows.shape), 0x7FC0, dtype=torch.int16, device=dev)
    pool = pkv.Pool(t["k_pool"], t["v_pool"])

    def launch():
        pkv.pkv_prefill(pool, desc, t["q_rows"], t["qo_indptr"], kv_indptr, t["kv_indices"],
                        t["seq_lens"], 64, True, batch.sm_scale, out)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        launch()  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    rng = np.random.default_rng(np.random.PCG64(65))
    for rep in range(3):
        batch.q_rows = W.normal_bf16(rng, batch.q_rows.shape)
        t["q_rows"].copy_(torch.from_numpy(batch.q_rows.view(np.int16)))
        out.fill_(0x7FC0)
        g.replay()
        torch.cuda.synchronize()
        replay_bits = out.cpu().numpy().view(np.uint16).copy()
        out.fill_(0x7FC0)
        launch()
        torch.cuda.synchronize()
        eager = out.cpu().numpy().view(np.uint16).copy()
        assert np.array_equal(replay_bits, eager), f"replay {rep} differs from eager"
        compare(eager, oracle_prefill(batch, True), f"graph replay {rep}")
