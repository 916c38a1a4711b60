"""Parity of the token-major decode (pkv_decode_tokens) with the fp64 oracle.

K/V hold one [Hkv][D] row per token slot, found through a request-to-token
table (page size 1) or at b * stride + t in the contiguous [batch, seq,
kv_heads, head_dim] layout.  Unwritten slots hold NaN, outputs start as NaN,
and the workspace starts as NaN bits, so a skipped row, a stray read or a
missing merge shows up.  The plan comes from pkv_build_metadata with a
page_size-16 descriptor, as the entry point requires.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_split_attn_amd as pkv
import workloads as W
from gpu_util import compare, say

pytestmark = pytest.mark.gpu

CASES = {
    "table_g4_d64": dict(B=5, Hq=8, Hkv=2, D=64, lengths=[1, 37, 0, 200, 16], table=True),
    "table_g4_d128": dict(B=4, Hq=32, Hkv=8, D=128, lengths=[513, 2, 1000, 64], table=True),
    "table_g1": dict(B=3, Hq=4, Hkv=4, D=128, lengths=[17, 300, 5], table=True),
    "table_g3": dict(B=3, Hq=24, Hkv=8, D=64, lengths=[40, 1, 129], table=True),
    "table_g8": dict(B=2, Hq=32, Hkv=4, D=128, lengths=[250, 31], table=True),
    "table_g7": dict(B=3, Hq=28, Hkv=4, D=128, lengths=[90, 1, 333], table=True),
    "contig_d128": dict(B=4, Hq=32, Hkv=8, D=128, lengths=[100, 1, 700, 0], table=False,
                        stride=704),
    "contig_d64": dict(B=3, Hq=8, Hkv=2, D=64, lengths=[33, 64, 5], table=False, stride=64),
}


def run_tokens(tb, forced=0, num_workgroups=0, table_override=None):
    dev = "cuda:0"
    t = W.tokens_to_device(tb, dev)
    desc = pkv.Desc(max_batch=tb.B, num_q_heads=tb.Hq, num_kv_heads=tb.Hkv, head_dim=tb.D,
                    page_size=16, num_workgroups=num_workgroups)
    ws = torch.empty(pkv.pkv_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    ws.fill_(0xFF)
    kv_indptr = torch.full((tb.B + 1,), -7, dtype=torch.int32, device=dev)
    pkv.pkv_build_metadata(desc, t["seq_lens"], forced, kv_indptr, ws)
    out = torch.full((tb.B, tb.Hq, tb.D), 0x7FC0, dtype=torch.int16, device=dev)
    table = t["slot_table"] if table_override is None else table_override
    pkv.pkv_decode_tokens(desc, t["k_cache"], t["v_cache"], table, tb.stride, t["q"], kv_indptr,
                          t["seq_lens"], tb.sm_scale, ws, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


def oracle_tokens(tb, table=None):
    return oracle.decode_tokens(tb.q, tb.k_cache, tb.v_cache, tb.seq_lens, tb.sm_scale,
                                tb.slot_table if table is None else table, tb.stride)


@pytest.mark.parametrize("grid", ["plan", "forced3", "forced1"])
@pytest.mark.parametrize("case", list(CASES))
def test_tokens_parity(case, grid):
    say(f"tokens {case} grid={grid}")
    kw = dict(CASES[case])
    B, lengths = kw.pop("B"), np.array(kw.pop("lengths"))
    tb = W.make_tokens(name=case, seed=sum(map(ord, case)), B=B, lengths=lengths, **kw)
    forced = {"plan": 0, "forced3": 3, "forced1": 1}[grid]
    got = run_tokens(tb, forced=forced)
    compare(got, oracle_tokens(tb), f"{case} {grid}")


def test_tokens_from_pages_full_ragged():
    # The ragged 16-request batch (25,284 tokens, Hq 32, Hkv 8, D 128) stored
    # token-major through its page table: the token path at full size.
    batch = W.config(3)
    tb = W.tokens_from_pages(batch)
    say(f"tokens from pages: {tb.num_slots} slots, {int(tb.seq_lens.sum())} tokens")
    got = run_tokens(tb)
    compare(got, oracle_tokens(tb), "ragged_b16_4k tokens")


def test_tokens_contiguous_long():
    # One 32,768-token request in the contiguous layout: split across the chip.
    tb = W.make_tokens(name="contig_long", seed=77, B=1, Hq=32, Hkv=8, D=128,
                       lengths=np.array([32768]), table=False)
    got = run_tokens(tb)
    compare(got, oracle_tokens(tb), "contig 32k")


def test_tokens_all_empty():
    tb = W.make_tokens(name="empty", seed=5, B=3, Hq=8, Hkv=2, D=64, lengths=np.zeros(3, int))
    got = run_tokens(tb)
    assert np.array_equal(got, np.zeros_like(got))


def test_tokens_unusable_slots_are_dropped():
    # Slots -1 and num_slots inside the sequence: those tokens are skipped, as
    # if they were not in the request.
    tb = W.make_tokens(name="bad", seed=9, B=2, Hq=8, Hkv=2, D=64, lengths=np.array([50, 20]))
    table = tb.slot_table.copy()
    table[0, 3] = -1
    table[0, 40] = tb.num_slots
    table[1, 19] = -5
    got = run_tokens(tb, table_override=torch.from_numpy(table).to("cuda:0"))
    kept = np.full_like(table, -1)
    lens = np.zeros(2, np.int32)
    for b in range(2):
        row = [s for s in table[b, : int(tb.seq_lens[b])] if 0 <= s < tb.num_slots]
        kept[b, : len(row)] = row
        lens[b] = len(row)
    ref = oracle.decode_tokens(tb.q, tb.k_cache, tb.v_cache, lens, tb.sm_scale, kept, tb.stride)
    compare(got, ref, "unusable slots")


def test_tokens_match_paged_decode_bitwise():
    # Same K/V through the page table (paged kernel) and through the token
    # table (token kernel): same plan shape, same arithmetic order per step.
    batch = W.config(2)
    from gpu_util import GpuRun, make_desc
    run = GpuRun(batch, make_desc(batch))
    paged = run.step()
    tok = run_tokens(W.tokens_from_pages(batch))
    assert np.array_equal(paged, tok)


def test_read_ceiling_probe_reads_every_word_once():
    # The diagnostic read kernel: the xor of all its per-lane folds equals the
    # xor of every 32-bit word of the buffer (each word read exactly once).
    g = torch.Generator().manual_seed(5)
    n_words = (3 << 20) + 4 * 37  # not a multiple of the per-wave span
    host = torch.randint(-(1 << 31), (1 << 31) - 1, (n_words,), dtype=torch.int64,
                         generator=g).to(torch.int32)
    src = host.to("cuda:0")
    sink = torch.full((pkv.READ_CEILING_GROUPS * 64 * pkv.WAVES_PER_GROUP,), 7, dtype=torch.int32,
                      device="cuda:0")
    pkv.pkv_debug_read_ceiling(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want
