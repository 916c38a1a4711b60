"""The decode that plans its own step (pkv_decode_plan).

One launch must leave everything exactly as pkv_build_metadata followed by
pkv_decode_append (or pkv_decode) does: the output, the pool, kv_indptr and
the plan in the workspace (header, wave ranges, merge records), so that the
step's later layers run on it unchanged.  The workspace of the planning
launch starts as all-ones bytes with one metadata build of a one-request
batch before it: that build must clear every arrival counter of the
descriptor, since the planning launch cannot.
"""

import numpy as np
import pytest
import torch

import paged_kv_split_attn_amd as pkv
import workloads as W
from gpu_util import GpuRun, compare, make_desc, oracle_out, say

pytestmark = pytest.mark.gpu

CASES = {  # name: (Hq, Hkv, D, P, lengths)
    "g4_p16": (8, 2, 64, 16, [1, 15, 16, 17, 40, 33]),
    "g4_p16_zeros": (32, 8, 128, 16, [0, 700, 0, 1, 2049, 0, 16]),
    "g8_p64": (32, 4, 128, 64, [100, 64, 65, 1, 300, 128]),
    "g1_p32": (8, 8, 128, 32, [31, 32, 33, 2, 257]),
    "g12_p16": (48, 4, 128, 16, [1, 16, 17, 250, 47]),
    "g20_p16": (40, 2, 128, 16, [1, 16, 17, 250, 47]),
    "g6_p16": (48, 8, 64, 16, [1, 16, 17, 250, 47]),
    "g10_p32": (20, 2, 128, 32, [2, 31, 32, 33, 400]),
    "g16_p32": (64, 4, 64, 32, [33, 1, 96, 500, 31]),
    "g2_p16": (8, 4, 64, 16, [5000, 3, 77]),
}


def _batch(case):
    if case.startswith("c"):
        batch = W.config(int(case[1]))
        if not batch.append:  # give every request a token to append
            rng = np.random.default_rng(500 + int(case[1]))
            batch.k_new = W.normal_bf16(rng, (batch.B, batch.Hkv, batch.D))
            batch.v_new = W.normal_bf16(rng, (batch.B, batch.Hkv, batch.D))
            batch.append = True
        return batch
    Hq, Hkv, D, P, lens = CASES[case]
    return W.make_batch(name=case, seed=Hq + 3 * D + P + len(lens), B=len(lens), Hq=Hq, Hkv=Hkv,
                        D=D, P=P, lengths=np.array(lens), append=True)


def _many_requests(B, seed):
    rng = np.random.default_rng(seed)
    return W.make_batch(name=f"many{B}", seed=seed, B=B, Hq=8, Hkv=2, D=64, P=16,
                        lengths=rng.integers(0, 120, size=B), append=True)


def _plan_bytes(ws, groups):
    """Header words but the error word, the wave ranges and the merge records."""
    b = ws.cpu().numpy()
    hdr = b[:256].view(np.int32)
    waves = 32 * groups * pkv.WAVES_PER_GROUP
    waves_end = 256 + (waves + 255) // 256 * 256
    ginfo_end = waves_end + (32 + 8 * pkv.WAVES_PER_GROUP) * groups
    return np.concatenate([hdr[[0, 1, 2, 3, 5]].view(np.uint8), b[256:256 + waves],
                           b[waves_end:ginfo_end]])


def _two_call(batch, desc, forced, append):
    run = GpuRun(batch, desc)
    run.metadata(forced)
    if append:
        run.decode_append()
    else:
        run.decode()
    torch.cuda.synchronize()
    return run


def _planned(batch, desc, forced, append):
    run = GpuRun(batch, desc)  # all-ones workspace
    # one metadata build of a one-request batch: clears every arrival counter
    pkv.pkv_build_metadata(desc, run.t["seq_lens"][:1], 0, run.kv_indptr[:2], run.ws)
    pkv.pkv_decode_plan(run.pool, desc, run.t["q"], run.t["k_new"] if append else None,
                        run.t["v_new"] if append else None, run.t["seq_lens"], forced,
                        run.kv_indptr, run.t["kv_indices"], batch.sm_scale, run.ws, run.out)
    torch.cuda.synchronize()
    return run


def _check_same(a, b, desc, label):
    assert np.array_equal(a.out_bits(), b.out_bits()), f"{label}: output differs"
    assert torch.equal(a.t["k_pool"], b.t["k_pool"]), f"{label}: K pool differs"
    assert torch.equal(a.t["v_pool"], b.t["v_pool"]), f"{label}: V pool differs"
    assert torch.equal(a.kv_indptr, b.kv_indptr), f"{label}: kv_indptr differs"
    assert np.array_equal(_plan_bytes(a.ws, desc.groups()), _plan_bytes(b.ws, desc.groups())), \
        f"{label}: plan differs"


@pytest.mark.parametrize("case", ["c3", "c5"] + list(CASES))
@pytest.mark.parametrize("forced", [0, 1, 3])
@pytest.mark.parametrize("append", [True, False], ids=["append", "plain"])
def test_planned_decode_equals_metadata_then_decode(case, forced, append):
    say(f"planned decode {case} forced={forced} append={append}")
    batch = _batch(case)
    desc = make_desc(batch, min_tiles=1 if case in CASES else 0)
    a = _two_call(batch, desc, forced, append)
    b = _planned(batch, desc, forced, append)
    _check_same(a, b, desc, case)
    assert b.validate()["status"] == pkv.PKV_OK
    if append:
        compare(b.out_bits(), oracle_out(batch), f"planned {case} forced={forced}")


def test_later_layers_run_on_the_written_plan():
    # Layer 0 plans; layers 1 and 2 (their own pools and queries) reuse the
    # plan and kv_indptr it wrote, and match the two-call step bitwise.
    say("later layers on the written plan")
    batch = _batch("c3")
    desc = make_desc(batch)
    a = _two_call(batch, desc, 0, True)
    b = _planned(batch, desc, 0, True)
    _check_same(a, b, desc, "layer 0")
    rng = np.random.default_rng(5)
    for layer in (1, 2):
        q = torch.from_numpy(W.normal_bf16(rng, (batch.B, batch.Hq, batch.D)).view(np.int16)).cuda()
        for run in (a, b):
            pkv.pkv_decode(run.pool, desc, q, run.kv_indptr, run.t["kv_indices"],
                           run.t["seq_lens"], batch.sm_scale, run.ws, run.out)
        torch.cuda.synchronize()
        assert np.array_equal(a.out_bits(), b.out_bits()), f"layer {layer} differs"


@pytest.mark.parametrize("B", [1024, 1100])
def test_largest_planned_batch_and_two_launch_fallback(B):
    # 1024 requests: the largest batch planned in LDS; above it the call runs
    # the metadata kernel first.  Both must equal the two-call step.
    say(f"planned decode B={B}")
    batch = _many_requests(B, 90 + B)
    desc = make_desc(batch)
    for forced in (0, 5):
        a = _two_call(batch, desc, forced, True)
        b = _planned(batch, desc, forced, True)
        _check_same(a, b, desc, f"B={B} forced={forced}")
    compare(b.out_bits(), oracle_out(batch), f"B={B}")


def test_negative_length_latches_error_and_keeps_other_rows():
    say("planned decode with a negative length")
    batch = _batch("g4_p16")
    desc = make_desc(batch, min_tiles=1)
    run = GpuRun(batch, desc)
    pkv.pkv_build_metadata(desc, run.t["seq_lens"], 0, run.kv_indptr, run.ws)
    torch.cuda.synchronize()
    assert run.validate()["status"] == pkv.PKV_OK  # also clears the error word
    lens = run.t["seq_lens"].clone()
    lens[2] = -5
    pkv.pkv_decode_plan(run.pool, desc, run.t["q"], run.t["k_new"], run.t["v_new"], lens, 0,
                        run.kv_indptr, run.t["kv_indices"], batch.sm_scale, run.ws, run.out)
    torch.cuda.synchronize()
    info = pkv.pkv_debug_validate(desc, lens, run.kv_indptr, run.t["kv_indices"],
                                  batch.num_pages, run.ws)
    assert info["status"] == pkv.PKV_ERR_DEVICE_DATA
    got = run.out_bits()
    assert not got[2].any(), "a negative length must give a zero row"
    # the other rows: the same as a step where that request is empty
    ref_lens = lens.clone()
    ref_lens[2] = 0
    ref = GpuRun(batch, desc)
    pkv.pkv_build_metadata(desc, ref_lens, 0, ref.kv_indptr, ref.ws)
    pkv.pkv_decode_append(ref.pool, desc, ref.t["q"], ref.t["k_new"], ref.t["v_new"],
                          ref.kv_indptr, ref.t["kv_indices"], ref_lens, batch.sm_scale, ref.ws,
                          ref.out)
    torch.cuda.synchronize()
    assert np.array_equal(got, ref.out_bits())
    assert torch.equal(run.t["k_pool"], ref.t["k_pool"]) and torch.equal(run.t["v_pool"],
                                                                         ref.t["v_pool"])
