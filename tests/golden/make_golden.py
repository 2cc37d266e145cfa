"""Write tests/golden/c1_oracle_sample.txt.

Calls only the seeded input generator and the fp64 oracle: the fixture
records a digest of the single-head T=64 workload's input bits and a sample
of the oracle's outputs on it, so a later run (or another machine) can check
that the generator and the oracle still agree with what was committed.
Run:  python tests/golden/make_golden.py
"""
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from gated_delta_amd import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c1_oracle_sample.txt")
O_IDX = [(0, 0, 0), (1, 0, 5), (17, 0, 64), (31, 0, 127), (63, 0, 99), (63, 0, 0)]
S_IDX = [(0, 0, 0, 0), (0, 0, 3, 100), (0, 0, 64, 64), (0, 0, 127, 1), (0, 0, 77, 127)]


def input_digest(p) -> str:
    h = hashlib.sha256()
    for name in ("q", "k", "v", "a", "b"):
        h.update(np.ascontiguousarray(getattr(p, name), dtype=np.float32).tobytes())
    return h.hexdigest()


def main():
    p = synth.config1()
    o, S = oracle.prefill(p.q, p.k, p.v, p.a, p.b)
    with open(OUT, "w") as f:
        f.write("# single-head T=64 d=128 fp32 workload (seeded generator), fp64 oracle\n")
        f.write("# written by tests/golden/make_golden.py (generator + oracle only)\n")
        f.write(f"inputs_sha256 {input_digest(p)}\n")
        for idx in O_IDX:
            f.write("o {} {} {} {!r}\n".format(*idx, float(o[idx])))
        for idx in S_IDX:
            f.write("S {} {} {} {} {!r}\n".format(*idx, float(S[idx])))


if __name__ == "__main__":
    main()
