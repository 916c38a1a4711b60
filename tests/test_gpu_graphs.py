"""The whole-step hipGraph harness (paged_kv_split_attn_amd.step_graphs).

One graph per power-of-two batch size; a live batch is padded into its bucket
with zero-length requests before each replay.  Replays must be bitwise equal
to the same step issued eagerly (padded) and to the unpadded step, write the
same pools, and match the fp64 oracle layer by layer.  The lengths and page
tables change between replays.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_split_attn_amd as pkv
from paged_kv_split_attn_amd.step_graphs import StepGraphs
import workloads as W
from gpu_util import compare, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _universe(seed, n, Hq, Hkv, D, P, max_len):
    """n requests at their largest lengths: the pages a live batch may use."""
    rng = np.random.default_rng(seed)
    caps = rng.integers(1, max_len + 1, size=n)
    return W.make_batch(name=f"universe{seed}", seed=seed, B=n, Hq=Hq, Hkv=Hkv, D=D, P=P,
                        lengths=caps, append=True)


def _live(uni, n, rng):
    """The first n requests at random lengths within their capacity."""
    lens = np.array([int(rng.integers(1, int(uni.seq_lens[b]) + 1)) for b in range(n)], np.int32)
    lists = [uni.page_lists[b][: -(-int(L) // uni.P)] for b, L in enumerate(lens)]
    idx = np.concatenate(lists).astype(np.int32)
    return lens, idx


def _bits(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def _host_pool(pool):
    return (W.k_pool_token_major(pool.k.cpu().numpy().view(np.uint16)),
            W.v_pool_token_major(pool.v.cpu().numpy().view(np.uint16)))


@pytest.mark.parametrize("n", [1, 3, 9, 16])
def test_bucket_replay_matches_eager_unpadded_and_oracle(n):
    say(f"step graph bucket replay n={n}")
    layers = 2
    uni = _universe(71, 16, 32, 8, 128, 16, 1200)
    dev = W.to_device(uni, DEV)
    pools = [pkv.Pool(dev["k_pool"].clone(), dev["v_pool"].clone()) for _ in range(layers)]
    tmpl = pkv.Desc(max_batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16)
    sg = StepGraphs(tmpl, pools, uni.sm_scale, max_batch=16, max_pages=len(uni.kv_indices))
    sg.capture()
    rng = np.random.default_rng(100 + n)
    for rep in range(3):  # lengths and page tables change between replays
        lens, idx = _live(uni, n, rng)
        q = W.normal_bf16(rng, (layers, n, 32, 128))
        kn = W.normal_bf16(rng, (layers, n, 8, 128))
        vn = W.normal_bf16(rng, (layers, n, 8, 128))
        snap = [(p.k.clone(), p.v.clone()) for p in pools]
        host_before = [_host_pool(p) for p in pools]
        bk = sg.load(torch.from_numpy(lens).to(DEV), torch.from_numpy(idx).to(DEV), _bits(q),
                     _bits(kn), _bits(vn))
        assert bk.B == sg.bucket_for(n)
        sg.replay(bk)
        torch.cuda.synchronize()
        got = bk.out.cpu().numpy().view(np.uint16).copy()
        after = [(p.k.clone(), p.v.clone()) for p in pools]
        assert not got[:, n:].any(), "padded requests must get zero rows"
        # the same padded step issued eagerly, from the same pools
        for p, (k, v) in zip(pools, snap):
            p.k.copy_(k)
            p.v.copy_(v)
        sg.eager(bk)
        torch.cuda.synchronize()
        assert np.array_equal(bk.out.cpu().numpy().view(np.uint16), got), f"rep {rep}: eager"
        for p, (k, v) in zip(pools, after):
            assert torch.equal(p.k, k) and torch.equal(p.v, v), f"rep {rep}: pools differ"
        # the unpadded step (a descriptor of exactly n requests)
        for p, (k, v) in zip(pools, snap):
            p.k.copy_(k)
            p.v.copy_(v)
        desc = pkv.Desc(max_batch=n, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16)
        ws = torch.zeros(pkv.pkv_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
        ip = torch.zeros(n + 1, dtype=torch.int32, device=DEV)
        sl, ix = torch.from_numpy(lens).to(DEV), torch.from_numpy(idx).to(DEV)
        pkv.pkv_build_metadata(desc, sl, 0, ip, ws)
        for layer, p in enumerate(pools):
            out = torch.empty((n, 32, 128), dtype=torch.int16, device=DEV)
            pkv.pkv_decode_append(p, desc, _bits(q[layer]), _bits(kn[layer]), _bits(vn[layer]),
                                  ip, ix, sl, uni.sm_scale, ws, out)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy().view(np.uint16), got[layer, :n]), \
                f"rep {rep} layer {layer}: padded replay differs from the unpadded step"
        # the oracle, layer by layer
        ipn = oracle.kv_indptr(lens, uni.P)
        for layer in range(layers):
            k_h, v_h = oracle.append_kv(*host_before[layer], kn[layer], vn[layer], ipn, idx, lens,
                                        uni.P)
            ref = oracle.decode(q[layer], k_h, v_h, ipn, idx, lens, uni.sm_scale, uni.P)
            compare(got[layer, :n], ref, f"n={n} rep={rep} layer={layer}")
        for p, (k, v) in zip(pools, after):  # keep the replay's pools for the next round
            p.k.copy_(k)
            p.v.copy_(v)


def test_24_layer_step_graph_against_oracle():
    # A model-like step: one metadata build and 24 layers of fused append +
    # decode, each layer its own pool and inputs, replayed from one graph and
    # checked against the oracle on every layer.
    say("24-layer step graph")
    layers, n = 24, 4
    uni = _universe(72, n, 8, 2, 64, 16, 400)
    dev = W.to_device(uni, DEV)
    pools = [pkv.Pool(dev["k_pool"].clone(), dev["v_pool"].clone()) for _ in range(layers)]
    tmpl = pkv.Desc(max_batch=n, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=16)
    sg = StepGraphs(tmpl, pools, uni.sm_scale, max_batch=n, max_pages=len(uni.kv_indices))
    sg.capture()
    rng = np.random.default_rng(7)
    lens, idx = _live(uni, n, rng)
    q = W.normal_bf16(rng, (layers, n, 8, 64))
    kn = W.normal_bf16(rng, (layers, n, 2, 64))
    vn = W.normal_bf16(rng, (layers, n, 2, 64))
    host_before = [_host_pool(p) for p in pools]
    bk = sg.load(torch.from_numpy(lens).to(DEV), torch.from_numpy(idx).to(DEV), _bits(q), _bits(kn),
                 _bits(vn))
    sg.replay(bk)
    torch.cuda.synchronize()
    got = bk.out.cpu().numpy().view(np.uint16)
    ipn = oracle.kv_indptr(lens, uni.P)
    for layer in range(layers):
        k_h, v_h = oracle.append_kv(*host_before[layer], kn[layer], vn[layer], ipn, idx, lens,
                                    uni.P)
        ref = oracle.decode(q[layer], k_h, v_h, ipn, idx, lens, uni.sm_scale, uni.P)
        compare(got[layer, :n], ref, f"layer {layer}")
