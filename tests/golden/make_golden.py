"""Writes tests/golden/tiny_oracle.txt from the oracle alone (no GPU code).

Run from the repository root:  python tests/golden/make_golden.py
The fixture freezes the oracle's output on the tiny workload (2 heads x 64,
16 queries, 128 cached keys, one Euler step of size 1), so that any later
change to the oracle's arithmetic shows up as a diff of this file."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workload  # noqa: E402


def compute():
    wl = workload.get("tiny")
    ui = workload.make_inputs(wl)
    s = ui.sessions[0]
    sh = s.shape
    res = oracle.denoise_unit(s.ring_k, s.ring_v, sh.len_before, sh.head_before, None, None,
                              s.q, s.k_u, s.v_u, s.eps, list(sh.h), ui.w_o)
    dz = res["z"] - s.eps
    return res["Os"][0], dz


def main():
    O, dz = compute()
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.txt")
    with open(path, "w") as f:
        f.write("# Oracle output on the tiny workload (seed 0), written by make_golden.py.\n")
        f.write("# O[row][head][0:8] for rows 0, 15 and heads 0, 1; dz = z_final - eps, row 0 and 15, cols 0:8\n")
        for r in (0, 15):
            for h in (0, 1):
                f.write(f"O_{r}_{h} = " + " ".join(f"{x:.17g}" for x in O[r, h, :8]) + "\n")
        for r in (0, 15):
            f.write(f"dz_{r} = " + " ".join(f"{x:.17g}" for x in dz[r, :8]) + "\n")
        f.write(f"O_norm = {np.linalg.norm(O):.17g}\n")
        f.write(f"dz_norm = {np.linalg.norm(dz):.17g}\n")


if __name__ == "__main__":
    main()
