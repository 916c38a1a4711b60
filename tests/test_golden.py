"""The oracle still reproduces its stored output for the tiny seeded batch."""

import os

import numpy as np

import oracle
import workloads

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_tiny():
    rows, indptr = [], None
    with open(os.path.join(HERE, "tiny_decode_out.txt")) as f:
        for line in f:
            if line.startswith("# kv_indptr"):
                indptr = [int(x) for x in line.split()[2:]]
            elif not line.startswith("#"):
                rows.append([float(x) for x in line.split()])
    return np.array(indptr), np.array(rows).reshape(1, 8, 64)


def test_tiny_golden():
    indptr, ref = load_tiny()
    b = workloads.config(1)
    ip = oracle.kv_indptr(b.seq_lens, b.P)
    assert list(ip) == list(indptr) == [0, 3]
    out = oracle.decode(b.q, b.k_pool, b.v_pool, ip, b.kv_indices, b.seq_lens, b.sm_scale, b.P)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-15)
