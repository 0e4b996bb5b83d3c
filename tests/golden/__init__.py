"""Stored expected values for the tests.

Every file here is either a value printed on the pages (none exist for this
method: the pages give no worked example) or is written by
``tests/golden/make_golden.py``, which calls only ``oracle/`` on inputs from
``synth``.  Each file's header names the command that wrote it.
"""

import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def codebook_path(m):
    return os.path.join(HERE, f"codebook_m{m}.txt")


def load_codebook(m):
    """float32 (256, m) codebook from its text file."""
    rows = []
    with open(codebook_path(m)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([float(t) for t in line.split()])
    return np.asarray(rows, dtype=np.float32)
