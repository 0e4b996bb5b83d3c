"""Plain CPU oracle for the NSNQuant KV-cache quantization path.

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously-correct
definition that the HIP library is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import it.  The product library (``kv_cache_calibration_amd``) never
imports, calls or links anything here, and nothing here imports the
product library: the two share no code, tables or constants.

Everything is numpy float64.  Values are rounded to fp16 only where the
method stores them (codes' metadata), with IEEE round-to-nearest-even as
``numpy.astype(float16)`` does.

Sources (the pages this follows):
  * "NSNQuant: A Double Normalization Approach for Calibration-Free Low-Bit
    Vector Quantization of KV Cache", technical summary on gist.science
    (Spanish and German editions, identical content): Methodology §1 NSN,
    §2 Hadamard transform, §3 vector quantization and codebook (codebook
    construction, scale adjustment, double quantization), §4 implementation
    details (residuals, attention computation, efficiency).
  * The authors' repository README (DHdroid/NSNQuant): Overview, Codebook
    tuning.
  * News summary on marsel.app: "How NSNQuant Works".

Pinning status per function (what fixes it other than itself) is listed in
each module header; ``scale_adjust`` is the one step whose *formula* is a
reading of a sentence rather than a printed definition, and its parity
with the authors' system is unpinned (only its stated property is).
"""

from .nsn import (  # noqa: F401
    hadamard_matrix,
    rotate,
    rht,
    rht_inverse,
    normalize_tokens,
    shift_channels,
    nsn,
    nearest_codeword,
    scale_adjust,
    quantize,
    dequantize,
    sq_dist_exact,
)
from .codebook import kmeans_codebook, round_to_fp16  # noqa: F401
from .tune import cosine_loss, cosine_tune  # noqa: F401
from .attention import (  # noqa: F401
    apply_rope,
    attend,
    decode_attention,
    decode_attention_rope,
    decode_attention_rotated,
)
from .dq import (  # noqa: F401
    codebook_4bit,
    dq_decode_group,
    dq_encode_group,
    dq_pack,
    dq_unpack,
    record_bytes,
)
