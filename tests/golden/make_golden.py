"""Write the golden codebooks with the oracle.

    python tests/golden/make_golden.py

Inputs come from ``synth`` (N(0,1) samples, PCG64 seed 0); values come from
``oracle.kmeans_codebook`` only.  The workloads name 20 Lloyd iterations on
65536 4-vectors (2-bit) and 262144 8-vectors (1-bit), 256 codes.
"""

import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402
from tests.golden import codebook_path  # noqa: E402


def main():
    for m, n in ((4, 65536), (8, 262144)):
        t0 = time.time()
        X = synth.codebook_samples(m, n, seed=0)
        C, hist = oracle.kmeans_codebook(X, 256, 20, return_history=True)
        with open(codebook_path(m), "w") as f:
            f.write(f"# NSNQuant codebook, m={m}, 256 codes: Lloyd k-means, 20 iterations,\n")
            f.write(f"# on {n} N(0,1) {m}-vectors (synth.codebook_samples(m={m}, n={n}, seed=0)),\n")
            f.write("# first-K init, lowest-index ties, entries rounded to fp16.\n")
            f.write("# Written by: python tests/golden/make_golden.py  (oracle only)\n")
            f.write(f"# per-dim training distortion before/after: {hist[0]:.6f} -> {hist[-1]:.6f}\n")
            for row in C.astype(np.float64):
                f.write(" ".join(repr(float(v)) for v in row) + "\n")
        print(f"m={m}: {time.time() - t0:.1f}s, distortion {hist[-1]:.6f}")


if __name__ == "__main__":
    main()
