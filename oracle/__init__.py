"""CPU oracle for 1-bit QJL KV-cache compression (fp64, numpy).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the tests under tests/, the smoke check in
__graft_entry__.py and the cpu_baseline leg of bench.py may import or call anything in this package.
The library (bit_kv_cache_qjl_amd and its HIP kernels) never imports it, and it never imports the
library: the two share no code; only the seeded input generators (seeded_inputs) serve both.

Pinned by tests/test_oracle_pins.py and tests/test_oracle_statistics.py against what the pages and
the mathematics fix: the pages' worked examples (tests/golden/), closed forms, invariants, special
cases and Monte-Carlo unbiasedness.  What pins each function:
  * uniform_quantize: the uniform 2-bit worked example of "Why Compressing the KV Cache Is Hard";
  * quantize_value_vectors, dequantize_value_vectors, quantize_values, pack_codes / unpack_codes: the
    2- and 3-bit token-wise examples of "2 numbers out of 128 destroy the entire KV cache", extreme
    values at codes 0 and L, brute-force nearest level, the half-step error bound, constant vectors,
    the bit layout by example;
  * jl_project, quantize_key_vectors, quantize_keys, pack_bits / unpack_bits, outlier_mask: S = I
    reproduces the sign vector of "Your Brain Already Runs on 1-Bit Keys", the norm closed form with
    fp16 rounding, scale and negation invariants, the orientation of S, the d = 8 brute force;
  * project_query, estimator_scores: Monte-Carlo unbiasedness with the exact variance, the outlier
    split as two independent sketches, antisymmetry, q = k, the one-dimensional closed form, the
    1/sqrt(m) error decay, the d = 8 brute force;
  * softmax, attend: the pages' softmax vectors, the two-score logistic form, equal scores, a
    dominant score, token permutation;
  * decode_attention: the d = 8 brute force over the whole decode, the estimator switch, and the
    batch / KV-head routing (several sequences, KV heads and query heads per KV head, one outlier set
    per KV head: constant values, outlier-only keys and per-head scores);
  * exact_attention: the page's 16.203 dot product and its [0.65, 0.35] weights, one key, equal
    scores, and the softmax definition written out as loops;
  * select_outliers: the pages' outlier examples, closed forms, ties, invariances;
  * two_sided_scores, two_sided_estimate, rotate_sign_scores: parallel and antiparallel closed forms,
    the identity projection on the page vectors, Monte-Carlo expectation 1 - 2 theta / pi, R = I and
    row permutations of R.
No function is "parity unpinned".
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
