"""Plant plausible mistakes in copies of the oracle source and check that the
pins catch every one.

Each mutant is a text substitution in a temporary copy of ``oracle/oracle.c``
(a dropped term, a wrong sign, a wrong index or stride, a missing scale, a
wrong rounding), compiled with gcc on the CPU.  The pin tests of
``test_oracle_attention`` / ``test_oracle_fp8`` are then run against the mutant
library; at least one must fail.  The committed oracle is never modified.
"""
import os
import shutil

import pytest

import oracle
from tests import test_oracle_attention as ta
from tests import test_oracle_fp8 as tf

ATTN_PINS = [
    lambda: ta.test_bruteforce_tiny(2, 2, 3, 5, 4),
    lambda: ta.test_bruteforce_tiny(1, 3, 7, 2, 8),
    lambda: ta.test_matches_torch_sdpa_f64(1, 2, 65, 33, 128),
    ta.test_two_key_closed_form,
    ta.test_single_key_returns_its_value,
    ta.test_constant_v_returns_v,
    ta.test_zero_query_uniform_weights,
    ta.test_rows_of_softmax_sum_to_one,
    ta.test_key_shift_changes_only_lse,
    ta.test_row_subset_equals_full,
]
MERGE_PINS = [
    lambda: ta.test_merge_of_split_partials_equals_full([0, 40, 100]),
    ta.test_merge_identities,
    ta.test_merge_weights_against_closed_form,
]
FP8_PINS = [
    tf.test_decode_spec_points,
    tf.test_decode_table_matches_torch,
    tf.test_encode_roundtrip_and_order,
    tf.test_encode_ties_to_even_and_saturation,
    tf.test_encode_matches_torch_cast,
    tf.test_quantiser_closed_forms,
    tf.test_quantiser_matches_torch_cast,
    tf.test_quantiser_blocks_are_independent_and_zero_block,
]
DEQUANT_PINS = [
    tf.test_dequant_inverts_within_bound,
    tf.test_dequant_closed_form,
]

# (name, original text, mutated text, pins expected to catch it)
MUTANTS = [
    ("lse_drops_max", "*lse_out = m + log(l);", "*lse_out = log(l);", ATTN_PINS),
    ("exp_sign", "double p = exp(s[j] - m);", "double p = exp(m - s[j]);", ATTN_PINS),
    ("no_normalise", "orow[c] /= l;", "orow[c] /= 1.0;", ATTN_PINS),
    ("no_scale", "s[j] = scale * acc;", "s[j] = acc;", ATTN_PINS),
    ("key_channel_reversed", "acc += qrow[c] * kj[c];", "acc += qrow[c] * kj[d - 1 - c];",
     ATTN_PINS),
    ("head_stride_dropped", "const double* kh = k + ((long)b * Skv * H + h) * d;",
     "const double* kh = k + ((long)b * Skv * H) * d;", ATTN_PINS),
    ("value_from_key", "const double* vh = v + ((long)b * Skv * H + h) * d;",
     "const double* vh = k + ((long)b * Skv * H + h) * d;", ATTN_PINS),
    ("merge_weight_sign", "double w = exp(lse_parts[c * l_part_stride + lidx] - M);",
     "double w = exp(M - lse_parts[c * l_part_stride + lidx]);", MERGE_PINS),
    ("merge_lse_drops_max", "lse[lidx] = M + log(L);", "lse[lidx] = log(L);", MERGE_PINS),
    ("merge_no_normalise", "orow[e] /= L;", "orow[e] /= 1.0;", MERGE_PINS),
    ("e4m3_bias_8", "mag = ldexp(1.0 + (double)m / 8.0, e - 7);",
     "mag = ldexp(1.0 + (double)m / 8.0, e - 8);", FP8_PINS),
    ("e4m3_truncate", "double mant = rint((2.0 * fr - 1.0) * 8.0);",
     "double mant = floor((2.0 * fr - 1.0) * 8.0);", FP8_PINS),
    ("e4m3_subnormal_trunc", "double q = rint(ldexp(a, 9));", "double q = floor(ldexp(a, 9));",
     FP8_PINS),
    ("quant_inverse_scale", "inv = 448.0f / famax;", "inv = 440.0f / famax;", FP8_PINS),
    ("quant_block_len", "int s1 = s0 + ORACLE_FP8_BLOCK < S ? s0 + ORACLE_FP8_BLOCK : S;",
     "int s1 = s0 + 64 < S ? s0 + 64 : S;", FP8_PINS),
    # the dequantiser defines the reference of every fp8 kernel-error test
    ("dequant_block_index",
     "double sc = (double)scale[((long)b * H + h) * nblk + s / ORACLE_FP8_BLOCK];",
     "double sc = (double)scale[((long)b * H + h) * nblk];", DEQUANT_PINS),
    ("dequant_head_stride",
     "double sc = (double)scale[((long)b * H + h) * nblk + s / ORACLE_FP8_BLOCK];",
     "double sc = (double)scale[((long)b * H) * nblk + s / ORACLE_FP8_BLOCK];", DEQUANT_PINS),
    ("dequant_batch_stride",
     "double sc = (double)scale[((long)b * H + h) * nblk + s / ORACLE_FP8_BLOCK];",
     "double sc = (double)scale[((long)h) * nblk + s / ORACLE_FP8_BLOCK];", DEQUANT_PINS),
    ("dequant_no_scale", "x[t * d + c] = oracle_e4m3_decode(q[t * d + c]) * sc;",
     "x[t * d + c] = oracle_e4m3_decode(q[t * d + c]);", DEQUANT_PINS),
]


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


@pytest.mark.parametrize("name,orig,mut,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, orig, mut, pins, mutant_dir):
    src = open(oracle._SRC).read()
    assert src.count(orig) == 1, f"mutation site for {name} not unique/present"
    d = mutant_dir / name
    d.mkdir()
    shutil.copy(os.path.join(os.path.dirname(oracle._SRC), "oracle.h"), d / "oracle.h")
    (d / "oracle.c").write_text(src.replace(orig, mut))
    so = oracle.build(force=True, src=str(d / "oracle.c"), out=str(d / "liboracle_mut.so"))
    lib = oracle.load_library(so)
    caught = []
    try:
        oracle.use_library(lib)
        for pin in pins:
            try:
                pin()
            except AssertionError:
                caught.append(pin)
    finally:
        oracle.use_library(None)
    assert caught, f"no pin caught mutant {name}"
