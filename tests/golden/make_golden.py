"""Write the stored expected values under tests/golden/ (calls only the oracle).

The pages print no worked numeric example for paged decode attention, so the
only stored values are the fp64 oracle's own outputs for the tiny seeded batch
(one request of 37 tokens over pages of 16, 16 and 5 tokens, 8 query heads on
2 KV heads, head_dim 64).  They guard the oracle against accidental change;
the oracle itself is pinned by tests/test_oracle_pins.py.

Run from the repository root:  python tests/golden/make_golden.py
"""

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def tiny_expected():
    b = workloads.config(1)
    ip = oracle.kv_indptr(b.seq_lens, b.P)
    out = oracle.decode(b.q, b.k_pool, b.v_pool, ip, b.kv_indices, b.seq_lens, b.sm_scale, b.P)
    return ip, out


def main():
    ip, out = tiny_expected()
    path = os.path.join(HERE, "tiny_decode_out.txt")
    with open(path, "w") as f:
        f.write("# fp64 oracle output for the tiny seeded batch (seed 1): B=1 Hq=8 Hkv=2 D=64\n")
        f.write("# P=16 seq_len=37; written by tests/golden/make_golden.py (oracle only)\n")
        f.write("# kv_indptr " + " ".join(str(int(x)) for x in ip) + "\n")
        for row in out.reshape(-1, out.shape[-1]):
            f.write(" ".join(repr(float(v)) for v in row) + "\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
