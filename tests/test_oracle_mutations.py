"""The oracle pins must reject plausible mistakes.

Each case compiles a copy of the oracle source with one planted error (a dropped
rope term, a sign flip, a missing scale, a wrong causal boundary, a transposed
statistics layout, ...) and checks that the finite-difference, dense-reduction
or closed-form pins of test_oracle_pins.py fail on it.  Mistakes are planted
only in CPU copies of the oracle; the real source is never touched.
"""

import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "sfag_oracle.c")

MUTATIONS = {
    "rope_dropped": ("dot(qrh, kr + key_row * pb->Dr, pb->Dr)", "0.0 * dot(qrh, kr + key_row * pb->Dr, pb->Dr)"),
    "ds_sign": ("p * (dp - Dt[h])", "p * (Dt[h] - dp)"),
    "ds_sign_dkv": ("p * (dp - dot(doh, oh, pb->D))", "p * (dot(doh, oh, pb->D) - dp)"),
    "dq_unscaled": ("const double c = pb->scale * ds;                        /* stage 3",
                    "const double c = ds;                        /* stage 3"),
    "causal_top_left": ("j > r->i + r->lkv - r->lq", "j > r->i"),
    "dv_uses_ds": ("dva[d] += p * doh[d]", "dva[d] += ds * doh[d]"),
    "prob_times_sum": ("exp(z - m) / l : 0.0", "exp(z - m) * l : 0.0"),
    "dp_uses_key": ("dot(doh, v + key_row * pb->D, pb->D);  /* stage 1", "dot(doh, k + key_row * pb->D, pb->D);  /* stage 1"),
    "stats_row_major": ("r.stat = r.b * pb->N1 * pb->S1 + r.i;\n    r.hstride = pb->S1;",
                        "r.stat = (r.b * pb->S1 + r.i) * pb->N1;\n    r.hstride = 1;"),
    "flashsoftmaxgrad_wrong_operand": ("Dt[h] = dot(dout + (g * pb->N1 + h) * pb->D, out + (g * pb->N1 + h) * pb->D, pb->D);",
                                       "Dt[h] = dot(dout + (g * pb->N1 + h) * pb->D, dout + (g * pb->N1 + h) * pb->D, pb->D);"),
    "dk_transposed_operand": ("dka[d] += c * qh[d];", "dka[d] += c * doh[d];"),
    "tnd_key_offset_zero": ("r.kbase = ckv;", "r.kbase = 0;"),
    "block_index_as_start": ("const int64_t j = jb * bs + s % bs;", "const int64_t j = jb + s % bs;"),
    "block_causal_on_start": ("if (pb->sparse_mode == 3 && j > r->i + r->lkv - r->lq) return -1;",
                              "if (pb->sparse_mode == 3 && jb * bs > r->i + r->lkv - r->lq) return -1;"),
    "block_uncut_by_length": ("if (j >= r->lkv) return -1;", "if (jb * bs >= r->lkv) return -1;"),
}


def _pins_pass() -> bool:
    """Run a representative set of pins; True when all of them pass."""
    checks = [
        lambda: pins.test_finite_differences_all_gradients(0),
        lambda: pins.test_finite_differences_all_gradients(3),
        lambda: pins.test_dense_reduction_matches_torch_autograd(0),
        lambda: pins.test_dense_reduction_matches_torch_autograd(4),
        pins.test_column_sums,
        pins.test_two_valid_slots_closed_form,
        lambda: pins.test_every_block_selected_matches_dense_autograd(0),
        lambda: pins.test_every_block_selected_matches_dense_autograd(1),
        lambda: pins.test_every_block_selected_matches_dense_autograd(3),
    ]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


def test_unmutated_oracle_passes_the_selected_pins():
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert old in src, f"mutation anchor for {name} not found in the oracle source"
    bad = src.replace(old, new)
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "m.c")
        so = os.path.join(d, "libm.so")
        open(c, "w").write(bad)
        subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-std=c99", "-I", os.path.dirname(SRC),
                        "-o", so, c, "-lm"], check=True)
        prev = oracle.swap_library(so)
        try:
            assert not _pins_pass(), f"pins did not catch mutation {name}"
        finally:
            oracle._lib = prev
