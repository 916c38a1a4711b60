"""Helpers for the GPU tests: run the HIP path through the C ABI on a batch and
compute the oracle's answer for the same seeded inputs."""

import sys

import numpy as np
import torch

import oracle
import paged_kv_split_attn_amd as pkv
import workloads as W

# Parity bar for bf16 inputs/outputs with fp32 accumulation, against the fp64 oracle.
MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_desc(batch, num_workgroups=0, min_tiles=0, max_batch=None):
    return pkv.Desc(max_batch=max_batch or batch.B, num_q_heads=batch.Hq,
                    num_kv_heads=batch.Hkv, head_dim=batch.D, page_size=batch.P,
                    num_workgroups=num_workgroups, min_tiles_per_group=min_tiles)


def oracle_plan(batch, desc, forced=0):
    _, U = oracle.head_groups(batch.Hq, batch.Hkv)
    return oracle.plan_stream(batch.seq_lens, batch.P, U, desc.groups(),
                              desc.min_tiles_per_group or 16, forced,
                              waves_per_group=pkv.WAVES_PER_GROUP)


class GpuRun:
    """Device copies of a batch plus the step buffers; runs metadata, append, decode."""

    def __init__(self, batch, desc, device="cuda:0", poison_workspace=True):
        self.batch, self.desc = batch, desc
        self.t = W.to_device(batch, device)
        self.pool = pkv.Pool(self.t["k_pool"], self.t["v_pool"])
        self.ws = torch.empty(pkv.pkv_workspace_bytes(desc), dtype=torch.uint8, device=device)
        if poison_workspace:
            self.ws.fill_(0xFF)  # every fp32 partial reads as NaN until written
        self.kv_indptr = torch.full((batch.B + 1,), -7, dtype=torch.int32, device=device)
        self.out = torch.full((batch.B, batch.Hq, batch.D), 0x7FC0, dtype=torch.int16,
                              device=device)

    def metadata(self, forced=0):
        pkv.pkv_build_metadata(self.desc, self.t["seq_lens"], forced, self.kv_indptr, self.ws)

    def append(self):
        pkv.pkv_append_kv(self.pool, self.t["k_new"], self.t["v_new"], self.kv_indptr,
                          self.t["kv_indices"], self.t["seq_lens"])

    def decode(self):
        pkv.pkv_decode(self.pool, self.desc, self.t["q"], self.kv_indptr, self.t["kv_indices"],
                       self.t["seq_lens"], self.batch.sm_scale, self.ws, self.out)

    def decode_append(self):
        pkv.pkv_decode_append(self.pool, self.desc, self.t["q"], self.t["k_new"], self.t["v_new"],
                              self.kv_indptr, self.t["kv_indices"], self.t["seq_lens"],
                              self.batch.sm_scale, self.ws, self.out)

    def step(self, forced=0):
        self.metadata(forced)
        if self.batch.append:
            self.append()
        self.decode()
        torch.cuda.synchronize()
        return self.out_bits()

    def out_bits(self):
        return self.out.cpu().numpy().view(np.uint16)

    def validate(self):
        return pkv.pkv_debug_validate(self.desc, self.t["seq_lens"], self.kv_indptr,
                                      self.t["kv_indices"], self.batch.num_pages, self.ws)


def oracle_out(batch):
    ip = oracle.kv_indptr(batch.seq_lens, batch.P)
    k, v = batch.k_pool, batch.v_pool
    if batch.append:
        k, v = oracle.append_kv(k, v, batch.k_new, batch.v_new, ip, batch.kv_indices,
                                batch.seq_lens, batch.P)
    return oracle.decode(batch.q, k, v, ip, batch.kv_indices, batch.seq_lens, batch.sm_scale,
                         batch.P)


def compare(got_bits, ref, label=""):
    got = W.bf16_bits_to_f32(got_bits).astype(np.float64)
    assert not np.isnan(got).any(), f"{label}: NaN in output"
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    say(f"  {label}: max_abs={mx:.3e} mean_abs={mean:.3e} max|o|={np.abs(ref).max():.3f}")
    assert mx <= MAX_ABS, f"{label}: max abs error {mx} > {MAX_ABS}"
    assert mean <= MEAN_ABS, f"{label}: mean abs error {mean} > {MEAN_ABS}"
    return mx, mean
