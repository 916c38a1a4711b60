"""pkv_decode_scratch, the decode that takes no workspace (its plan, partials
and counters live in the library's static device scratch), against the
two-call path with a caller workspace: bitwise the same kv_indptr and output,
within the parity bar of the oracle, on two calls in a row, the second with a
smaller batch and shorter lengths (so stale scratch contents would show)."""

import numpy as np
import pytest
import torch

import paged_kv_split_attn_amd as pkv
import workloads as W
from gpu_util import GpuRun, compare, make_desc, oracle_out, say

pytestmark = pytest.mark.gpu


def _scratch_call(run, desc):
    ip = torch.full_like(run.kv_indptr, -7)
    out = torch.full_like(run.out, 0x7FC0)
    pkv.pkv_decode_scratch(run.pool, desc, run.t["q"], run.t["seq_lens"], run.t["kv_indices"],
                           run.batch.sm_scale, ip, out)
    torch.cuda.synchronize()
    return ip.cpu().numpy(), out.cpu().numpy().view(np.uint16)


def test_scratch_decode_matches_workspace_decode_twice():
    big = W.make_batch(name="scratch_big", seed=91, B=12, Hq=32, Hkv=8, D=128, P=16,
                       lengths=np.array([4096, 17, 900, 1, 2500, 64, 3000, 333, 16, 1200, 2047, 5]))
    small = W.make_batch(name="scratch_small", seed=92, B=5, Hq=32, Hkv=8, D=128, P=16,
                         lengths=np.array([40, 1, 700, 16, 129]))
    desc = make_desc(big)  # one descriptor (capacity 12) serves both calls
    for batch in (big, small):
        say(f"scratch decode {batch.name} B={batch.B}")
        run = GpuRun(batch, desc)
        ref = run.step().copy()  # pkv_build_metadata + pkv_decode with a caller workspace
        ref_ip = run.kv_indptr.cpu().numpy()
        ip, got = _scratch_call(run, desc)
        assert np.array_equal(ip, ref_ip)
        assert np.array_equal(got, ref), "scratch decode differs from the workspace decode"
        compare(got, oracle_out(batch), f"scratch {batch.name}")


def test_scratch_too_small_is_refused():
    batch = W.make_batch(name="scratch_refuse", seed=93, B=2, Hq=8, Hkv=2, D=64, P=16,
                         lengths=np.array([10, 20]))
    desc = make_desc(batch, num_workgroups=65536)
    assert pkv.pkv_workspace_bytes(desc) > pkv.SCRATCH_BYTES
    run = GpuRun(batch, make_desc(batch))
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_decode_scratch(run.pool, desc, run.t["q"], run.t["seq_lens"], run.t["kv_indices"],
                               batch.sm_scale, run.kv_indptr, run.out)
    assert e.value.status == pkv.PKV_ERR_SCRATCH_TOO_SMALL
