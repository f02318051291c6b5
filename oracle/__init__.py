"""CPU oracle for 1-bit QJL KV-cache compression (fp64, numpy).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the tests under tests/, the smoke check in
__graft_entry__.py and the cpu_baseline leg of bench.py may import or call anything in this package.
The library (bit_kv_cache_qjl_amd and its HIP kernels) never imports it, and it never imports the
library: the two share no code; only the seeded input generators (seeded_inputs) serve both.

Pinned by tests/test_oracle_pins.py and tests/test_oracle_statistics.py against what the pages and
the mathematics fix: the pages' worked examples (tests/golden/), closed forms, invariants, special
cases and Monte-Carlo unbiasedness.  Every function is pinned; none is "parity unpinned".
"""
from .qjl import (SQRT_HALF_PI, attend, decode_attention, dequantize_value_vectors, estimator_scores,
                  exact_attention, fp16, jl_project, outlier_mask, pack_bits, pack_codes, project_query,
                  quantize_key_vectors, quantize_keys, quantize_value_vectors, quantize_values,
                  rotate_sign_scores, select_outliers, softmax, two_sided_estimate, two_sided_scores,
                  uniform_quantize, unpack_bits, unpack_codes)

__all__ = ["SQRT_HALF_PI", "attend", "decode_attention", "dequantize_value_vectors", "estimator_scores",
           "exact_attention", "fp16", "jl_project", "outlier_mask", "pack_bits", "pack_codes",
           "project_query", "quantize_key_vectors", "quantize_keys", "quantize_value_vectors",
           "quantize_values", "rotate_sign_scores", "select_outliers", "softmax", "two_sided_estimate",
           "two_sided_scores", "uniform_quantize", "unpack_bits", "unpack_codes"]
