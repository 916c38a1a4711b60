"""K/V pools larger than 4 GiB: every page, slot and row offset past the 4 GiB
mark needs 64-bit address arithmetic in the kernels.  A small seeded batch is
placed in the top pages (or slots) of a pool of about 4.6 GiB per K and per V,
the rest of the pool left zero; the results must match the oracle on the small
batch, whose page ids are the big pool's ids mapped back."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_split_attn_amd as pkv
import workloads as W
from gpu_util import compare, make_desc, oracle_out, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
# Hkv 8, D 128, P 16: 32 KiB of K (and of V) per page, 2 KiB per token slot.
BIG_PAGES = 150_000
BIG_SLOTS = 2_400_000
FOUR_GIB = 4 << 30


def _big_like(small, rows):
    return torch.zeros((rows,) + tuple(small.shape[1:]), dtype=small.dtype, device=DEV)


def _spread(n, rows, stride):
    """Small row i -> big row rows - 1 - stride i (all of them at the top)."""
    return rows - 1 - stride * np.arange(n, dtype=np.int64)


def test_decode_append_and_prefill_past_4gib():
    say("pool past 4 GiB: decode + append, prefill")
    batch = W.make_batch(name="big", seed=91, B=3, Hq=32, Hkv=8, D=128, P=16,
                         lengths=np.array([100, 700, 33]), append=True)
    t = W.to_device(batch, DEV)
    page_bytes = t["k_pool"][0].numel() * 2
    ids = _spread(t["k_pool"].shape[0], BIG_PAGES, 7)
    assert int(ids.min()) * page_bytes > FOUR_GIB
    kb, vb = _big_like(t["k_pool"], BIG_PAGES), _big_like(t["v_pool"], BIG_PAGES)
    idx = torch.from_numpy(ids).to(DEV)
    kb[idx] = t["k_pool"]
    vb[idx] = t["v_pool"]
    kv_big = idx[t["kv_indices"].long()].to(torch.int32)
    pool = pkv.Pool(kb, vb)

    desc = make_desc(batch)
    ws = torch.empty(pkv.pkv_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    ip = torch.empty(batch.B + 1, dtype=torch.int32, device=DEV)
    out = torch.full((batch.B, batch.Hq, batch.D), 0x7FC0, dtype=torch.int16, device=DEV)
    pkv.pkv_build_metadata(desc, t["seq_lens"], 0, ip, ws)
    pkv.pkv_decode_append(pool, desc, t["q"], t["k_new"], t["v_new"], ip, kv_big, t["seq_lens"],
                          batch.sm_scale, ws, out)
    torch.cuda.synchronize()
    compare(out.cpu().numpy().view(np.uint16), oracle_out(batch), "decode + append past 4 GiB")
    # The appended tokens landed in the big pool's pages, bit for bit.
    ref_ip = oracle.kv_indptr(batch.seq_lens, batch.P)
    k_ref, v_ref = oracle.append_kv(batch.k_pool, batch.v_pool, batch.k_new, batch.v_new, ref_ip,
                                    batch.kv_indices, batch.seq_lens, batch.P)
    assert np.array_equal(kb[idx].cpu().numpy().view(np.uint16), W.k_pool_blocked(k_ref))
    assert np.array_equal(vb[idx].cpu().numpy().view(np.uint16), W.v_pool_channel_major(v_ref))

    # Prefill over the same big pool (new pages of its own, written the same way).
    pb = W.make_prefill(name="bigp", seed=92, Hq=32, Hkv=8, D=128, P=16, q_lens=[40, 3],
                        prefix_lens=[60, 500])
    tp = W.to_device(pb, DEV)
    ids_p = _spread(tp["k_pool"].shape[0], BIG_PAGES, 5)
    idx_p = torch.from_numpy(ids_p).to(DEV)
    kb.zero_()
    vb.zero_()
    kb[idx_p] = tp["k_pool"]
    vb[idx_p] = tp["v_pool"]
    kv_big_p = idx_p[tp["kv_indices"].long()].to(torch.int32)
    pdesc = make_desc(pb)
    pws = torch.empty(pkv.pkv_workspace_bytes(pdesc), dtype=torch.uint8, device=DEV)
    pip = torch.empty(pb.B + 1, dtype=torch.int32, device=DEV)
    pkv.pkv_build_metadata(pdesc, tp["seq_lens"], 0, pip, pws)
    pout = torch.full(tuple(pb.q_rows.shape), 0x7FC0, dtype=torch.int16, device=DEV)
    q_lens = np.diff(pb.qo_indptr)
    pkv.pkv_prefill(pool, pdesc, tp["q_rows"], tp["qo_indptr"], pip, kv_big_p, tp["seq_lens"],
                    int(q_lens.max()), True, pb.sm_scale, pout)
    torch.cuda.synchronize()
    ref = oracle.prefill(pb.q_rows, pb.k_pool, pb.v_pool, oracle.kv_indptr(pb.seq_lens, pb.P),
                         pb.kv_indices, pb.seq_lens, pb.qo_indptr, pb.sm_scale, pb.P, True)
    compare(pout.cpu().numpy().view(np.uint16), ref, "prefill past 4 GiB")
    del kb, vb
    torch.cuda.empty_cache()


def test_token_major_past_4gib():
    say("token-major cache past 4 GiB")
    tb = W.make_tokens(name="bigt", seed=93, B=3, Hq=32, Hkv=8, D=128,
                       lengths=np.array([90, 1, 333]), table=True)
    t = W.tokens_to_device(tb, DEV)
    slot_bytes = t["k_cache"][0].numel() * 2
    ids = _spread(t["k_cache"].shape[0], BIG_SLOTS, 3)
    assert int(ids.min()) * slot_bytes > FOUR_GIB
    kc, vc = _big_like(t["k_cache"], BIG_SLOTS), _big_like(t["v_cache"], BIG_SLOTS)
    idx = torch.from_numpy(ids).to(DEV)
    kc[idx] = t["k_cache"]
    vc[idx] = t["v_cache"]
    table = t["slot_table"].long()
    big_table = torch.where(table >= 0, idx[table.clamp(min=0)], table).to(torch.int32)
    desc = pkv.Desc(max_batch=tb.B, num_q_heads=tb.Hq, num_kv_heads=tb.Hkv, head_dim=tb.D,
                    page_size=16)
    ws = torch.empty(pkv.pkv_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    ip = torch.empty(tb.B + 1, dtype=torch.int32, device=DEV)
    pkv.pkv_build_metadata(desc, t["seq_lens"], 0, ip, ws)
    out = torch.full((tb.B, tb.Hq, tb.D), 0x7FC0, dtype=torch.int16, device=DEV)
    pkv.pkv_decode_tokens(desc, kc, vc, big_table, tb.stride, t["q"], ip, t["seq_lens"],
                          tb.sm_scale, ws, out)
    torch.cuda.synchronize()
    ref = oracle.decode_tokens(tb.q, tb.k_cache, tb.v_cache, tb.seq_lens, tb.sm_scale,
                               tb.slot_table, tb.stride)
    compare(out.cpu().numpy().view(np.uint16), ref, "token-major past 4 GiB")
    del kc, vc
    torch.cuda.empty_cache()
