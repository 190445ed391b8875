"""CPU oracle for the MegaMoE expert layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and it shares no code
with the kernels.  Every function cites the passage of the pages it follows.
"""
from .codecs import (E2M1_MAX, E4M3_MAX, bf16_bits_rne, bf16_bits_to_f32, e2m1_decode_table,
                     e2m1_unpack_decode, e4m3_decode, e4m3_decode_table, e4m3_encode_rne,
                     ue8m0_code_for_amax, ue8m0_decode)
from .moe import (RECIPE_FP8_B128, RECIPE_MXFP4W_B32, RECIPE_MXFP8_B32, Problem, block_scaled_gemm, expert_rows,
                  flops, forward, requant, route, swiglu_weighted)
