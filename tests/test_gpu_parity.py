"""Parity of the HIP path (through the C ABI) with the fp64 oracle on the GPU.

Integer work (kv_indptr, split plan, KV append) must be bit-exact; decode
outputs must be within max |err| 1e-2 and mean |err| 1e-3 of the oracle with
bf16 inputs/outputs and fp32 accumulation.  Pools carry NaN in every unwritten
slot and the workspace starts as all-ones bytes (NaN as fp32), so any stray
read or unwritten partial shows up as NaN.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_split_attn_amd as pkv
import workloads as W
from gpu_util import GpuRun, compare, make_desc, oracle_out, oracle_plan, say

pytestmark = pytest.mark.gpu

_BATCHES = {}
_REFS = {}


def cfg(i):
    if i not in _BATCHES:
        _BATCHES[i] = W.config(i)
    return _BATCHES[i]


def ref(i):
    if i not in _REFS:
        _REFS[i] = oracle_out(cfg(i))
    return _REFS[i]


# ------------------------------------------------------------------ metadata

def _random_lengths_batch(seed, B, with_zeros):
    rng = np.random.default_rng(seed)
    L = rng.integers(0 if with_zeros else 1, 5000, size=B)
    return W.make_batch(name=f"lens{seed}", seed=seed, B=B, Hq=8, Hkv=2, D=64, P=16,
                        lengths=L, poison=False)


# Plans away from four query heads per KV head and pages of 16 tokens:
# (Hq, Hkv, P) -> head groups of the largest of 1 .. 8 and 12 that divides G:
# all of G up to eight (G = 1, 3, 6, 7, 8), twelve (G = 12), sixteen (G = 16),
# five (G = 20: four groups per KV head) or one (G = 11, a prime).
PLAN_SHAPES = {
    "g8": (64, 8, 16), "g3": (24, 8, 16), "g12": (48, 4, 16), "g1": (8, 8, 16),
    "g16": (128, 8, 16), "g20": (40, 2, 16), "g6": (48, 8, 16), "g7": (28, 4, 16),
    "g11": (22, 2, 16), "g4_p32": (32, 8, 32), "g4_p64": (32, 8, 64), "g8_p64": (64, 8, 64),
}


def _shape_lengths_batch(case):
    Hq, Hkv, P = PLAN_SHAPES[case]
    rng = np.random.default_rng(sum(map(ord, case)))
    L = rng.integers(0, 3000, size=29)
    return W.make_batch(name=f"plan_{case}", seed=int(rng.integers(1 << 30)), B=29, Hq=Hq,
                        Hkv=Hkv, D=64, P=P, lengths=L, poison=False)


@pytest.mark.parametrize("case", ["c1", "c2", "c3", "c4", "c5", "rand0", "rand1", "rand_big"]
                         + list(PLAN_SHAPES))
@pytest.mark.parametrize("grid,forced", [(0, 0), (0, 3), (1000, 0)])
def test_metadata_bit_exact(case, grid, forced):
    say(f"metadata case={case} grid={grid} forced={forced}")
    if case in PLAN_SHAPES:
        batch = _shape_lengths_batch(case)
    elif case.startswith("c"):
        batch = cfg(int(case[1]))
    elif case == "rand_big":
        batch = _random_lengths_batch(77, 1500, True)  # more requests than one block scans at once
    else:
        batch = _random_lengths_batch(int(case[-1]) + 10, 37, case == "rand0")
    desc = make_desc(batch, num_workgroups=grid)
    run = GpuRun(batch, desc)
    run.metadata(forced)
    torch.cuda.synchronize()
    ip = run.kv_indptr.cpu().numpy()
    assert np.array_equal(ip, oracle.kv_indptr(batch.seq_lens, batch.P))
    info = run.validate()
    assert info["status"] == pkv.PKV_OK
    plan = oracle_plan(batch, desc, forced)
    assert info["groups"] == plan["groups"]
    assert np.array_equal(np.array(info["waves"]), plan["waves"])


def _merge_records_brute_force(batch, desc, plan):
    """Every workgroup's merge record, worked out tile by tile from the plan.

    Words: first / last segment of the workgroup's tiles (b * U + u), the
    first and last workgroup each of them touches, whether that segment is
    the first (0) or last (1) partial slot of the workgroup where it starts,
    then per wave the segment of its first and of its last piece when that
    piece does not cover its whole segment (-1 otherwise or when absent).
    """
    _, U = oracle.head_groups(batch.Hq, batch.Hkv)
    ip = np.asarray(plan["kv_indptr"], dtype=np.int64)
    T, Wn = int(plan["tiles"]), int(plan["groups"])
    nw = pkv.WAVES_PER_GROUP
    starts = ip * U
    t = np.arange(T, dtype=np.int64)
    b = np.searchsorted(starts, t, side="right") - 1
    n = ip[b + 1] - ip[b]
    seg = b * U + (t - starts[b]) // n  # segment of every tile
    pages = n                            # tiles of that segment
    g = [i * T // Wn for i in range(Wn + 1)] if Wn else [0]
    owner = np.zeros(T, dtype=np.int64)
    for i in range(Wn):
        owner[g[i]:g[i + 1]] = i
    first_tile = {}
    for x in range(T - 1, -1, -1):
        first_tile[int(seg[x])] = x
    recs = np.zeros((desc.groups(), 8 + 2 * nw), dtype=np.int64)
    for i in range(desc.groups()):
        rec = [-1, -1, 0, 0, -1, -1, 0, 0] + [-1] * (2 * nw)
        if i < Wn and g[i + 1] > g[i]:
            for k, x in enumerate((g[i], g[i + 1] - 1)):
                s_ = int(seg[x])
                t0 = first_tile[s_]
                t1 = t0 + int(pages[x]) - 1
                rec[k], rec[2 + k], rec[4 + k] = s_, int(owner[t0]), int(owner[t1])
                rec[6 + k] = 0 if g[int(owner[t0])] >= t0 else 1
            for w in range(nw):
                a0 = g[i] + w * (g[i + 1] - g[i]) // nw
                a1 = g[i] + (w + 1) * (g[i + 1] - g[i]) // nw
                if a1 <= a0:
                    continue
                pieces = []  # (segment, tiles) runs of the wave's range
                for x in range(a0, a1):
                    if pieces and pieces[-1][0] == int(seg[x]):
                        pieces[-1][1] += 1
                    else:
                        pieces.append([int(seg[x]), 1])
                sp = int(pages[a0])
                if pieces[0][1] < sp:
                    rec[8 + 2 * w] = pieces[0][0]
                if len(pieces) > 1 and pieces[-1][1] < int(pages[a1 - 1]):
                    rec[8 + 2 * w + 1] = pieces[-1][0]
        recs[i] = rec
    return recs


@pytest.mark.parametrize("case", ["c1", "c3", "c5", "rand0", "g8", "g12", "g4_p64"])
@pytest.mark.parametrize("grid,forced", [(0, 0), (0, 3), (1000, 0)])
def test_merge_records_match_brute_force(case, grid, forced):
    say(f"merge records case={case} grid={grid} forced={forced}")
    if case in PLAN_SHAPES:
        batch = _shape_lengths_batch(case)
    elif case.startswith("c"):
        batch = cfg(int(case[1]))
    else:
        batch = _random_lengths_batch(10, 37, True)
    desc = make_desc(batch, num_workgroups=grid)
    run = GpuRun(batch, desc)
    run.metadata(forced)
    torch.cuda.synchronize()
    groups = desc.groups()
    waves_end = 256 + (32 * groups * pkv.WAVES_PER_GROUP + 255) // 256 * 256
    words = 8 + 2 * pkv.WAVES_PER_GROUP
    got = run.ws[waves_end:waves_end + 4 * words * groups].view(torch.int32).view(groups, words)
    want = _merge_records_brute_force(batch, desc, oracle_plan(batch, desc, forced))
    bad = np.argwhere(got.cpu().numpy() != want)
    assert bad.size == 0, f"{len(bad)} words differ, first at (workgroup, word) {tuple(bad[0])}"


# -------------------------------------------------------------------- append

@pytest.mark.parametrize("which", ["small", "c5"])
def test_append_bit_exact(which):
    say(f"append {which}")
    if which == "c5":
        batch = cfg(5)
    else:
        batch = W.make_batch(name="app", seed=41, B=9, Hq=8, Hkv=2, D=128, P=16,
                             lengths=np.array([1, 15, 16, 17, 33, 64, 100, 2, 48]), append=True)
    run = GpuRun(batch, make_desc(batch))
    run.metadata()
    run.append()
    torch.cuda.synchronize()
    ip = oracle.kv_indptr(batch.seq_lens, batch.P)
    k_ref, v_ref = oracle.append_kv(batch.k_pool, batch.v_pool, batch.k_new, batch.v_new, ip,
                                    batch.kv_indices, batch.seq_lens, batch.P)
    k = W.k_pool_token_major(run.t["k_pool"].cpu().numpy().view(np.uint16))
    v = W.v_pool_token_major(run.t["v_pool"].cpu().numpy().view(np.uint16))
    assert np.array_equal(k, k_ref)
    assert np.array_equal(v, v_ref)


# ------------------------------------------------------ fused append + decode

FUSED_CASES = {  # name: (Hq, Hkv, D, P, lengths)
    "g4_p16": (8, 2, 64, 16, [1, 15, 16, 17, 40, 33]),
    "g8_p64": (32, 4, 128, 64, [100, 64, 65, 1, 300, 128]),
    "g1_p32": (8, 8, 128, 32, [31, 32, 33, 2, 257]),
    # one head group of twelve per KV head
    "g12_p16": (48, 4, 128, 16, [1, 16, 17, 250, 47]),
    # four head groups of five per KV head: only the first writes the token
    "g20_p16": (40, 2, 128, 16, [1, 16, 17, 250, 47]),
    # one head group of seven per KV head
    "g7_p16": (28, 4, 128, 16, [1, 16, 17, 250, 47]),
    # two head groups of five per KV head
    "g10_p32": (20, 2, 64, 32, [2, 31, 32, 33, 400]),
    # one head group of sixteen per KV head
    "g16_p32": (64, 4, 64, 32, [33, 1, 96, 500, 31]),
    # two head groups of sixteen per KV head
    "g32_p16": (64, 2, 128, 16, [1, 16, 17, 250, 47]),
}


@pytest.mark.parametrize("case", ["c5"] + list(FUSED_CASES))
@pytest.mark.parametrize("forced", [0, 3])
def test_fused_append_decode_matches_separate(case, forced):
    # pkv_decode_append must leave the pool and the output exactly as
    # pkv_append_kv followed by pkv_decode does, and match the oracle.
    say(f"fused append+decode {case} forced={forced}")
    if case == "c5":
        batch = cfg(5)
    else:
        Hq, Hkv, D, P, lens = FUSED_CASES[case]
        batch = W.make_batch(name=case, seed=Hq + 7 * D + P, B=len(lens), Hq=Hq, Hkv=Hkv, D=D,
                             P=P, lengths=np.array(lens), append=True)
    desc = make_desc(batch, min_tiles=1)
    sep = GpuRun(batch, desc)
    sep_bits = sep.step(forced).copy()
    fus = GpuRun(batch, desc)
    fus.metadata(forced)
    pkv.pkv_decode_append(fus.pool, desc, fus.t["q"], fus.t["k_new"], fus.t["v_new"],
                          fus.kv_indptr, fus.t["kv_indices"], fus.t["seq_lens"], batch.sm_scale,
                          fus.ws, fus.out)
    torch.cuda.synchronize()
    assert torch.equal(fus.t["k_pool"], sep.t["k_pool"]), "K pool differs"
    assert torch.equal(fus.t["v_pool"], sep.t["v_pool"]), "V pool differs"
    fus_bits = fus.out_bits()
    assert np.array_equal(fus_bits, sep_bits), "fused output differs from append + decode"
    compare(fus_bits, ref(5) if case == "c5" else oracle_out(batch), f"fused {case}")


# ---------------------------------------------------------------- keep mask

def _masked_run(batch, desc, mask_np, forced=0):
    """metadata (+ append) + masked decode on the GPU; the oracle's answer."""
    run = GpuRun(batch, desc)
    run.metadata(forced)
    k, v = batch.k_pool, batch.v_pool
    ip = oracle.kv_indptr(batch.seq_lens, batch.P)
    if batch.append:
        run.append()
        k, v = oracle.append_kv(k, v, batch.k_new, batch.v_new, ip, batch.kv_indices,
                                batch.seq_lens, batch.P)
    mask = torch.from_numpy(mask_np.astype(np.uint8)).to("cuda:0")
    pkv.pkv_decode_masked(run.pool, desc, run.t["q"], mask, run.kv_indptr, run.t["kv_indices"],
                          run.t["seq_lens"], batch.sm_scale, run.ws, run.out)
    torch.cuda.synchronize()
    expect = oracle.decode_masked(batch.q, k, v, ip, batch.kv_indices, batch.seq_lens,
                                  batch.sm_scale, batch.P, mask_np)
    return run.out_bits(), expect


MASK_CASES = [  # (workload, keep density, forced workgroups)
    ("c1", 0.5, 3), ("c2", 0.5, 0), ("c3", 0.5, 0), ("c3", 0.02, 0), ("c4", 0.9, 0),
    ("c5", 0.7, 0), ("g8_p64", 0.3, 2), ("g1_p32", 0.6, 0),
]


@pytest.mark.parametrize("case,density,forced", MASK_CASES,
                         ids=[f"{c}-keep{d}-groups{f or 'plan'}" for c, d, f in MASK_CASES])
def test_masked_decode(case, density, forced):
    say(f"masked decode {case} keep={density} forced={forced}")
    if case.startswith("c"):
        batch = cfg(int(case[1]))
    else:
        Hq, Hkv, D, P, lens = FUSED_CASES[case]
        batch = W.make_batch(name=case, seed=Hq + 11 * D + P, B=len(lens), Hq=Hq, Hkv=Hkv, D=D,
                             P=P, lengths=np.array(lens))
    S = -(-int(batch.seq_lens.max()) // 4) * 4 + 4
    rng = np.random.default_rng(int(density * 1000) + batch.B)
    mask = rng.random((batch.B, S)) < density
    mask[0, :] = False  # one request keeps nothing: zero row
    got, expect = _masked_run(batch, make_desc(batch, min_tiles=1), mask, forced)
    assert not W.bf16_bits_to_f32(got[0]).any()
    compare(got, expect, f"masked {case} keep={density}")


def test_all_true_mask_is_plain_decode():
    # the masked kernel keeping every token does the plain kernel's arithmetic
    batch = cfg(3)
    say("all-true mask cfg3")
    desc = make_desc(batch)
    plain = GpuRun(batch, desc).step().copy()
    S = -(-int(batch.seq_lens.max()) // 4) * 4
    got, _ = _masked_run(batch, desc, np.ones((batch.B, S), bool))
    assert np.array_equal(got, plain)


# -------------------------------------------------------------------- decode

DECODE_CASES = [  # (workload, grid size (0 = one per CU), forced workgroups (0 = planner))
    (1, 0, 1), (1, 0, 3), (1, 0, 0),
    (2, 0, 0), (2, 0, 1), (2, 1024, 1024),
    (3, 0, 0), (3, 0, 1), (3, 0, 7), (3, 2048, 0),
    (4, 0, 0), (4, 0, 1), (4, 4096, 0),
    (5, 0, 0), (5, 64, 0),
]


@pytest.mark.parametrize("i,grid,forced", DECODE_CASES,
                         ids=[f"cfg{i}-grid{g or 'cu'}-groups{f or 'plan'}" for i, g, f in DECODE_CASES])
def test_decode_parity(i, grid, forced):
    batch = cfg(i)
    say(f"decode cfg{i} ({batch.name}) grid={grid} forced={forced}")
    desc = make_desc(batch, num_workgroups=grid)
    run = GpuRun(batch, desc)
    got = run.step(forced)
    info = run.validate()
    assert info["status"] == pkv.PKV_OK
    assert info["groups"] == oracle_plan(batch, desc, forced)["groups"]
    compare(got, ref(i), f"cfg{i} grid={grid or 'cu'} groups={info['groups']}")


def test_repeated_decodes_reuse_one_plan():
    # several layers per step: one metadata build, many decodes (merge counters reset themselves)
    batch = cfg(3)
    say("repeated decodes cfg3")
    run = GpuRun(batch, make_desc(batch, num_workgroups=512))
    first = run.step()
    for _ in range(3):
        run.decode()
        torch.cuda.synchronize()
        assert np.array_equal(run.out_bits(), first)
    compare(first, ref(3), "cfg3 repeated")


@pytest.mark.parametrize("Hq,Hkv,D,P", [
    (8, 8, 128, 16),   # G = 1
    (16, 8, 128, 16),  # G = 2
    (24, 8, 64, 16),   # G = 3
    (64, 8, 128, 16),  # G = 8: one head group of eight per KV head
    (48, 4, 128, 16),  # G = 12: one head group of twelve per KV head
    (40, 2, 128, 16),  # G = 20: four head groups of five per KV head
    (40, 8, 128, 16),  # G = 5: one head group of five
    (48, 8, 64, 16),   # G = 6: one head group of six
    (28, 4, 128, 16),  # G = 7: one head group of seven
    (36, 4, 64, 16),   # G = 9: three head groups of three per KV head
    (22, 2, 128, 16),  # G = 11: eleven head groups of one per KV head
    (128, 8, 64, 16),  # G = 16: one head group of sixteen
    (64, 2, 128, 16),  # G = 32: two head groups of sixteen per KV head
    (96, 8, 128, 32),  # G = 12 with pages of 32
    (32, 4, 64, 32),   # two rounds per page at D = 64
    (8, 2, 128, 32),   # four rounds per page at D = 128
    (8, 2, 128, 64),   # eight rounds per page
])
def test_decode_shapes(Hq, Hkv, D, P):
    say(f"shapes Hq={Hq} Hkv={Hkv} D={D} P={P}")
    batch = W.make_batch(name="shape", seed=Hq * 131 + D + P, B=5, Hq=Hq, Hkv=Hkv, D=D, P=P,
                         lengths=np.array([1, P - 1, P + 1, 5 * P + 3, 700]))
    expect = oracle_out(batch)
    for grid, forced in ((0, 0), (0, 2), (300, 300)):
        desc = make_desc(batch, num_workgroups=grid, min_tiles=1)
        got = GpuRun(batch, desc).step(forced)
        compare(got, expect, f"Hq={Hq} Hkv={Hkv} D={D} P={P} forced={forced}")


@pytest.mark.parametrize("scale", [-1.0 / np.sqrt(128.0), 0.0], ids=["negative", "zero"])
def test_decode_scale_sign_and_zero(scale):
    # Any scale but NaN is accepted: a negative one reverses which keys weigh
    # most, and zero gives every live token of a request the same weight.
    say(f"decode sm_scale={scale}")
    batch = dataclasses.replace(
        W.make_batch(name="scale", seed=77, B=5, Hq=32, Hkv=8, D=128, P=16,
                     lengths=np.array([1, 15, 17, 83, 700])), sm_scale=scale)
    expect = oracle_out(batch)
    for grid, forced in ((0, 0), (300, 300)):
        desc = make_desc(batch, num_workgroups=grid, min_tiles=1)
        got = GpuRun(batch, desc).step(forced)
        compare(got, expect, f"sm_scale={scale} forced={forced}")


def test_seq_len_one_is_exact():
    say("seq_len one")
    batch = W.make_batch(name="len1", seed=5, B=6, Hq=32, Hkv=8, D=128, P=16,
                         lengths=np.ones(6, np.int64), num_pages=40)
    got = GpuRun(batch, make_desc(batch)).step()
    G = batch.Hq // batch.Hkv
    for b in range(batch.B):
        page = batch.page_lists[b][0]
        for hq in range(batch.Hq):
            assert np.array_equal(got[b, hq], batch.v_pool[page, hq // G, 0])


def test_zero_length_requests_give_zero_rows():
    say("zero lengths")
    batch = W.make_batch(name="zeros", seed=6, B=5, Hq=32, Hkv=8, D=128, P=16,
                         lengths=np.array([0, 100, 0, 1, 17]))
    got = GpuRun(batch, make_desc(batch, min_tiles=1)).step()
    assert not got[0].any() and not got[2].any()
    compare(got, oracle_out(batch), "zero-length mix")


def test_all_requests_empty():
    # no tile at all: the plan uses no workgroup and every output row is zero
    say("all empty")
    batch = W.make_batch(name="allzero", seed=8, B=6, Hq=8, Hkv=2, D=64, P=16,
                         lengths=np.zeros(6, dtype=np.int64), num_pages=8)
    run = GpuRun(batch, make_desc(batch))
    got = run.step()
    info = run.validate()
    assert info["status"] == pkv.PKV_OK and info["groups"] == 0
    assert not got.any()


def test_batch_beyond_metadata_lds():
    # more requests than the metadata kernel keeps in LDS (8192): the prefix sums
    # are then searched in global memory
    say("batch of 10000")
    rng = np.random.default_rng(123)
    lens = rng.integers(0, 40, size=10000)
    batch = W.make_batch(name="big_b", seed=124, B=10000, Hq=8, Hkv=2, D=64, P=16, lengths=lens,
                         poison=False)
    desc = make_desc(batch)
    run = GpuRun(batch, desc)
    got = run.step()
    ip = run.kv_indptr.cpu().numpy()
    assert np.array_equal(ip, oracle.kv_indptr(batch.seq_lens, batch.P))
    info = run.validate()
    assert info["status"] == pkv.PKV_OK
    plan = oracle_plan(batch, desc)
    assert info["groups"] == plan["groups"]
    assert np.array_equal(np.array(info["waves"]), plan["waves"])
    compare(got, oracle_out(batch), "B=10000")


def test_deterministic_and_page_permutation_invariant():
    say("determinism / permutation cfg3")
    batch = cfg(3)
    desc = make_desc(batch)
    a = GpuRun(batch, desc).step()
    b = GpuRun(batch, desc).step()
    assert np.array_equal(a, b)
    c = GpuRun(W.permute_pool(batch, seed=1234), desc).step()
    assert np.array_equal(a, c)


def test_bad_page_id_is_skipped_and_reported():
    say("bad page id")
    batch = W.make_batch(name="bad", seed=8, B=3, Hq=8, Hkv=2, D=64, P=16,
                         lengths=np.array([40, 50, 60]), poison=False)
    run = GpuRun(batch, make_desc(batch))
    # request 1's second page id points one past the pool: the kernels must skip it
    pos = len(batch.page_lists[0]) + 1
    run.t["kv_indices"][pos] = batch.num_pages
    got = run.step()
    info = run.validate()
    assert info["status"] == pkv.PKV_ERR_DEVICE_DATA
    assert run.validate()["status"] == pkv.PKV_ERR_DEVICE_DATA  # page id still bad
    expect = oracle_out(batch)
    compare(got[[0, 2]], expect[[0, 2]], "untouched requests")


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
def test_graph_capture_replay_matches_eager(fused):
    say(f"graph replay fused={fused}")
    batch = W.make_batch(name="graph", seed=9, B=8, Hq=32, Hkv=8, D=128, P=16,
                         lengths=np.array([3000, 1, 700, 2048, 16, 4096, 999, 64]), append=True)
    desc = make_desc(batch)
    run = GpuRun(batch, desc)
    full = batch.seq_lens.copy()
    rng = np.random.default_rng(10)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run.step()  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.metadata()
        if fused:
            run.decode_append()
        else:
            run.append()
            run.decode()
    hk, hv = batch.k_pool.copy(), batch.v_pool.copy()
    for rep in range(4):
        lens = np.maximum(1, (full * rng.uniform(0.2, 1.0, size=batch.B)).astype(np.int32))
        lists = [pl[: -(-int(L) // batch.P)] for pl, L in zip(batch.page_lists, lens)]
        idx = np.concatenate(lists).astype(np.int32)
        # the caller re-lays out kv_indices for the new lengths, in place
        run.t["kv_indices"][: idx.size].copy_(torch.from_numpy(idx))
        run.t["seq_lens"].copy_(torch.from_numpy(lens))
        g.replay()
        torch.cuda.synchronize()
        replay_bits = run.out_bits().copy()
        eager = run.step()
        assert np.array_equal(replay_bits, eager), f"replay {rep} differs from eager"
        # both the replay and the eager step wrote k_new/v_new at position lens-1
        ip = oracle.kv_indptr(lens, batch.P)
        hk, hv = oracle.append_kv(hk, hv, batch.k_new, batch.v_new, ip, idx, lens, batch.P)
        expect = oracle.decode(batch.q, hk, hv, ip, idx, lens, batch.sm_scale, batch.P)
        compare(eager, expect, f"replay {rep}")


def test_gqa8_ragged_lengths_full_size():
    # Eight query heads per KV head (Hq 64, Hkv 8): head groups of eight, so
    # every output pass of the workgroup merge and of the cross-workgroup merge
    # runs twice; the ragged batch's lengths give merges across many workgroups.
    say("G = 8 on the ragged lengths")
    lens = cfg(3).seq_lens.copy()
    batch = W.make_batch(name="g8_ragged", seed=31, B=16, Hq=64, Hkv=8, D=128, P=16,
                         lengths=lens)
    got = GpuRun(batch, make_desc(batch)).step()
    compare(got, oracle_out(batch), "G=8 ragged lengths")


def test_two_streams_with_separate_workspaces():
    # The library keeps no state of its own: two steps issued on two streams,
    # each with its own workspace, metadata and output, may run concurrently
    # and give bitwise the results each gives alone.
    say("two streams, separate workspaces")
    a = W.make_batch(name="s1", seed=41, B=8, Hq=32, Hkv=8, D=128, P=16,
                     lengths=np.array([3000, 17, 900, 4096, 1, 640, 2048, 333]))
    b = W.make_batch(name="s2", seed=42, B=5, Hq=8, Hkv=2, D=64, P=32,
                     lengths=np.array([700, 64, 65, 1500, 9]))
    ra, rb = GpuRun(a, make_desc(a)), GpuRun(b, make_desc(b))
    alone_a, alone_b = ra.step().copy(), rb.step().copy()
    for run in (ra, rb):
        run.out.fill_(0x7FC0)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        with torch.cuda.stream(sa):
            ra.metadata()
            ra.decode()
        with torch.cuda.stream(sb):
            rb.metadata()
            rb.decode()
    torch.cuda.synchronize()
    assert np.array_equal(ra.out_bits(), alone_a)
    assert np.array_equal(rb.out_bits(), alone_b)
    compare(alone_a, oracle_out(a), "stream 1")
    compare(alone_b, oracle_out(b), "stream 2")


def test_plan_of_another_batch_is_refused():
    # A decode whose workspace holds the plan of a different batch must not
    # follow it (its ranges may name requests past this call's arrays): the
    # kernel writes nothing and latches the error word, which validate reports.
    say("plan mismatch")
    batch = W.make_batch(name="mismatch", seed=12, B=6, Hq=32, Hkv=8, D=128, P=16,
                         lengths=np.array([900, 17, 3000, 1, 64, 2500]))
    run = GpuRun(batch, make_desc(batch))
    run.metadata()
    short = batch.B - 1
    out = torch.full((short, batch.Hq, batch.D), 0x7FC0, dtype=torch.int16, device="cuda:0")
    pkv.pkv_decode(run.pool, run.desc, run.t["q"][:short], run.kv_indptr[: short + 1],
                   run.t["kv_indices"], run.t["seq_lens"][:short], batch.sm_scale, run.ws, out)
    torch.cuda.synchronize()
    assert (out == 0x7FC0).all(), "the decode wrote output under a plan of another batch"
    assert run.validate()["status"] == pkv.PKV_ERR_DEVICE_DATA
    # validate cleared the error word; a new plan for this batch decodes normally
    got = run.step()
    assert run.validate()["status"] == pkv.PKV_OK
    compare(got, oracle_out(batch), "after mismatch")
