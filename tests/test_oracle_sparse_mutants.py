"""The sparse-layer oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/sparse_oracle.c (the softmax scale
dropped, the own block's causal bound off by one, the own block among the
candidates, the lowest scores selected, ties to the higher block, key means taken
from the queries, the query mean of one row, the gate's sign, decode's own block or
candidates cut short), builds it in a temporary directory, routes the oracle's
sparse calls to it and checks that at least one pin of ``test_oracle_sparse_pins``
fails.  CPU only.
"""
import os
import shutil
import subprocess

import pytest

import oracle
import test_oracle_sparse_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "sparse_oracle.c")

MUTANTS = {
    "scale_dropped": ("logit[i] = a * scale;", "logit[i] = a;"),
    "own_block_strict": ("for (int u = r0; u <= t; ++u) keys[n++] = u;",
                         "for (int u = r0; u < t; ++u) keys[n++] = u;"),
    "own_block_is_a_candidate": ("const int ncand = i < nkb ? i : nkb;",
                                 "const int ncand = i + 1 <= nkb ? i + 1 : nkb;"),
    "lowest_scores_selected": ("if (!taken[j] && (best < 0 || score[j] > score[best])) best = j;",
                               "if (!taken[j] && (best < 0 || score[j] < score[best])) best = j;"),
    "ties_to_higher_block": ("if (!taken[j] && (best < 0 || score[j] > score[best])) best = j;",
                             "if (!taken[j] && (best < 0 || score[j] >= score[best])) best = j;"),
    "key_means_from_queries": ("mean_rows(k, row0, rs, j * blk, j * blk + blk, D, kmean + (size_t)j * D);",
                               "mean_rows(q, row0, rs, j * blk, j * blk + blk, D, kmean + (size_t)j * D);"),
    "query_mean_of_first_row": ("mean_rows(q, row0, rs, r0, r1, D, qmean);",
                                "mean_rows(q, row0, rs, r0, r0 + 1, D, qmean);"),
    "gate_sign": ("o[d] = sigmoid((double)g[d]) * o[d] / den;", "o[d] = sigmoid(-(double)g[d]) * o[d] / den;"),
    "decode_own_block_start": ("for (int u = own * blk; u <= t; ++u) keys[nk++] = u;",
                               "for (int u = own * blk + 1; u <= t; ++u) keys[nk++] = u;"),
    "decode_candidates_one_short": ("const int ncand = own;", "const int ncand = own > 0 ? own - 1 : 0;"),
}

PIN_CALLS = [
    (pins.test_dense_fallback_is_causal_softmax_attention, (1, 70, 2, 16, 16, 4)),
    (pins.test_dense_fallback_is_causal_softmax_attention, (2, 33, 1, 8, 8, 4)),
    (pins.test_attention_over_its_selection_is_masked_softmax, (200, 16, 3)),
    (pins.test_planted_blocks_are_selected, ()),
    (pins.test_decode_step_is_the_last_row_of_a_prefill, ()),
    (pins.test_decode_matches_masked_attention_at_ragged_lengths, ()),
    (pins.test_identical_keys_average_the_values_and_zero_gate_halves, ()),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found once"
    mutant = tmp_path / "sparse_mutant.c"
    mutant.write_text(src.replace(old, new, 1))
    lib = tmp_path / "libsparsemutant.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(mutant),
                           "-o", str(lib), "-lm"])
    caught = None
    with oracle.use_sparse_library(str(lib)):
        for fn, args in PIN_CALLS:
            try:
                fn(*args)
            except (AssertionError, FloatingPointError):
                caught = fn.__name__
                break
    assert caught is not None, f"no pin caught the planted mistake {name}"
