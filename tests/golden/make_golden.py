"""Writes the oracle's results on the tiny fp32 decode workload (B=2, T=1,
H_k=2, H_v=4, K=V=32, slots [2, 0]) to ``tiny_fp32_b2.txt``.

The pages print no worked example or output values (the fused gating +
delta-rule kernel of vLLM PR #35777 and sglang PR #18271 is described only
by its inputs, tiling and timings), so this fixture is an oracle regression
record, not an external pin: it calls only ``oracle`` and the seeded input
generator.  Regenerate with ``python tests/golden/make_golden.py`` and name
the reason in the commit message.
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from linear_attention_recurrent_gating_amd import workloads as W  # noqa: E402

PATH = os.path.join(HERE, "tiny_fp32_b2.txt")


def compute():
    inp = W.make_host_inputs(W.TINY_F32)
    pool = W.make_pool_host(W.TINY_F32)
    out, _ = oracle.run_inputs(inp, pool)
    return inp, out, pool


def main():
    inp, out, pool = compute()
    lines = ["# oracle regression record: tiny fp32 decode (seed 0), written by make_golden.py",
             "# out[N=2, H_v=4, V=32], then for slots 2 and 0 the final state of v-head 1,",
             "# rows 0..3 [4, V=32], and the sum of the slot's whole final state",
             "# values are %.17g"]
    lines.append("out " + " ".join("%.17g" % x for x in out.ravel()))
    for s in inp.state_idx:
        lines.append(f"slot{s}_h1_rows0to3 " + " ".join("%.9g" % x for x in pool[s, 1, :4].ravel()))
        lines.append(f"slot{s}_sum %.17g" % float(pool[s].astype(np.float64).sum()))
    with open(PATH, "w") as f:
        f.write("\n".join(lines) + "\n")


def load():
    rec = {}
    with open(PATH) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            rec[key] = np.array([float(x) for x in vals])
    return rec


if __name__ == "__main__":
    main()
