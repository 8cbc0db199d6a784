"""CPU oracle for ROCmFP2 matrix-vector and matrix products.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
statement of what the GPU library computes.  Only the test suite, the smoke
check in ``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py``
may import it.  It shares no code with the HIP library (``bit_gemv_amd``) and
never imports it; the HIP library never imports this package.

Everything here follows the page "ROCmFP2 codebook research report"
(llm.ciru.ai, 2026-07-13), cited by its section headings:

* "01 · Storage" -- the 10-byte block: eight code bytes, two scale bytes.
* "02 · Quantization" -- the four-level codebook, the 2.5 midpoint rule,
  the UE4M3 scale byte and the per-half scale search.
* "03 · Runtime" -- int8 activations, int32 half sums, the rescale
  d_a * (d0*S0 + d1*S1), and the multi-column expand-once reuse.

Pins (what each function is checked against, besides itself) live in
``tests/test_oracle_*.py``.  Functions whose result no printed value fixes are
pinned by brute force, exact rational arithmetic, or invariants; there is no
"parity unpinned" function in this package.
"""
from .rfp2 import (  # noqa: F401
    CODEBOOK, UE4M3_MAX_BYTE, ue4m3_decode, ue4m3_table, select_code,
    pack_block, unpack_block, pack_matrix, unpack_matrix,
    start_byte, quantize_half, quantize_weights, dequantize_weights,
    quantize_acts, dequantize_acts, decoded_int8, half_sums,
    ref_gemv, ref_gemm, ref_moe_gemv, ref_moe_batch, sort_by_expert, abs_product_sums,
    row_bytes, matrix_bytes,
)
