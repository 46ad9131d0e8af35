"""The pins must catch plausible mistakes in the oracle.

Each mutant is conv_oracle.c with one plausible slip planted by text
substitution (on the CPU, in a temporary directory).  The pin suite
(test_oracle.py) runs against the mutant's library in a child process and
must fail.  A mutant the pins let through would mean a hole in the pins.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "conv_oracle.c")

MUTANTS = {
    "drop_last_s_tap": ("s < pb->S; ++s", "s < pb->S - 1; ++s"),
    "drop_first_channel": ("int64_t c = 0; c < pb->C", "int64_t c = 1; c < pb->C"),
    "flipped_filter_rows": ("* pb->R + r) * pb->S + s]", "* pb->R + (pb->R - 1 - r)) * pb->S + s]"),
    "flipped_filter_cols": ("* pb->S + s]", "* pb->S + (pb->S - 1 - s)]"),
    "pad_sign": ("r - pb->pad_top", "r + pb->pad_top"),
    "left_pad_for_top": ("r - pb->pad_top", "r - pb->pad_left"),
    "stride_swapped": ("p * pb->u + r", "p * pb->v + r"),
    "c_r_swapped_in_filter": ("((k * pb->C + c) * pb->R + r)", "((k * pb->C + r % pb->C) * pb->R + c % pb->R)"),
    "ceil_output_width": ("*Q = wspan / pb->v + 1;", "*Q = (wspan + pb->v - 1) / pb->v + 1;"),
    "bottom_pad_ignored": ("pb->H + pb->pad_top + pb->pad_bottom - pb->R", "pb->H + pb->pad_top - pb->R"),
    "beta_dropped": ("val += beta * y_old[o];", "val += 0.0 * y_old[o];"),
    "alpha_dropped": ("double val = alpha * acc;\n                    if (beta", "double val = acc;\n                    if (beta"),
    "bound_without_abs": ("bound += fabs(prod);", "bound += prod;"),
    "no_zero_padding_right": ("w < 0 || w >= pb->W", "w < 0 || w > pb->W"),
}

# slips in the data-gradient code, caught by test_oracle_dgrad.py
MUTANTS_DGRAD = {
    "dgrad_pad_sign": ("hh = h + pb->pad_top - r", "hh = h - pb->pad_top + r"),
    "dgrad_left_pad_sign": ("ww = w + pb->pad_left - s", "ww = w + pb->pad_left + s"),
    "dgrad_stride_swapped": ("hh % pb->u != 0", "hh % pb->v != 0"),
    "dgrad_last_row_dropped": ("hh / pb->u >= P", "hh / pb->u >= P - 1"),
    "dgrad_divisibility_ignored": ("ww < 0 || ww % pb->v != 0 || ww / pb->v >= Q", "ww < 0 || ww / pb->v >= Q"),
    "dgrad_filter_flipped": ("double fv = f[((k * pb->C + c) * pb->R + r) * pb->S + s];\n                double prod = dv",
                             "double fv = f[((k * pb->C + c) * pb->R + (pb->R - 1 - r)) * pb->S + s];\n                double prod = dv"),
    "dgrad_dy_p_q_swapped": ("p * sdy[2] + q * sdy[3]", "q * sdy[2] + p * sdy[3]"),
    "dgrad_first_filter_dropped": ("for (int64_t k = 0; k < pb->K; ++k) {\n        for (int64_t r = 0; r < pb->R; ++r) {\n            int64_t hh",
                                   "for (int64_t k = 1; k < pb->K; ++k) {\n        for (int64_t r = 0; r < pb->R; ++r) {\n            int64_t hh"),
    "dgrad_beta_dropped": ("val += beta * dx_old[o];", "val += 0.0 * dx_old[o];"),
}

# slips in the filter-gradient code, caught by test_oracle_wgrad.py
MUTANTS_WGRAD = {
    "wgrad_pad_sign": ("n, c, p * pb->u + r - pb->pad_top, q * pb->v", "n, c, p * pb->u + r + pb->pad_top, q * pb->v"),
    "wgrad_tap_flipped": ("q * pb->v + s - pb->pad_left);\n                double dv", "q * pb->v - s - pb->pad_left);\n                double dv"),
    "wgrad_strides_swapped": ("n, c, p * pb->u + r - pb->pad_top, q * pb->v", "n, c, p * pb->v + r - pb->pad_top, q * pb->u"),
    "wgrad_first_image_dropped": ("for (int64_t n = 0; n < pb->N; ++n) {\n        for (int64_t p = 0; p < P; ++p) {",
                                  "for (int64_t n = 1; n < pb->N; ++n) {\n        for (int64_t p = 0; p < P; ++p) {"),
    "wgrad_r_s_swapped_in_output": ("int64_t o = ((k * C + c) * R + r) * S + s;", "int64_t o = ((k * C + c) * S + s) * R + r;"),
    "wgrad_beta_dropped": ("val += beta * dw_old[o];", "val += 0.0 * dw_old[o];"),
    "wgrad_last_column_dropped": ("for (int64_t q = 0; q < Q; ++q) {\n                double xv", "for (int64_t q = 0; q < Q - 1; ++q) {\n                double xv"),
}

# slips in the pooling code, caught by test_oracle_pool.py
MUTANTS_POOL = {
    "pool_padding_wins_max": ("if (inside == 0 || v > best) best = v;", "if (v > best) best = v;"),
    "pool_include_divides_by_inside": ("if (mode == 1) return sum / (double)(pb->R * pb->S);",
                                       "if (mode == 1) return sum / (double)(inside ? inside : 1);"),
    "pool_exclude_divides_by_window": ("return inside ? sum / (double)inside : 0.0;",
                                       "return inside ? sum / (double)(pb->R * pb->S) : 0.0;"),
    "pool_pad_sign": ("int64_t h = p * pb->u + r - pb->pad_top;\n            int64_t w = q * pb->v + s - pb->pad_left;\n            if (h < 0",
                      "int64_t h = p * pb->u + r + pb->pad_top;\n            int64_t w = q * pb->v + s - pb->pad_left;\n            if (h < 0"),
    "pool_strides_swapped": ("int64_t h = p * pb->u + r - pb->pad_top;\n            int64_t w = q * pb->v + s - pb->pad_left;\n            if (h < 0",
                             "int64_t h = p * pb->v + r - pb->pad_top;\n            int64_t w = q * pb->u + s - pb->pad_left;\n            if (h < 0"),
    "pool_last_window_col_dropped": ("for (int64_t s = 0; s < pb->S; ++s) {\n            int64_t h = p * pb->u",
                                     "for (int64_t s = 0; s < pb->S - 1; ++s) {\n            int64_t h = p * pb->u"),
}

# slips in the batch-reduce GEMM, caught by test_oracle_brgemm.py
MUTANTS_BRGEMM = {
    "brgemm_last_batch_dropped": ("for (int64_t i = 0; i < batch; ++i) {", "for (int64_t i = 0; i < batch - 1; ++i) {"),
    "brgemm_b_strides_swapped": ("b[i * sb_i + k * sb_k + n * sb_n]", "b[i * sb_i + k * sb_n + n * sb_k]"),
    "brgemm_a_batch_stride_ignored": ("a[i * sa_i + m * sa_m + k * sa_k]", "a[m * sa_m + k * sa_k]"),
    "brgemm_beta_dropped": ("if (beta != 0.0) val += beta * c_old[m * N + n];", "if (beta != 0.0) val += 0.0 * c_old[m * N + n];"),
}


def _build_and_run(name, old, new, tmp, pins="test_oracle.py"):
    with open(SRC) as fh:
        text = fh.read()
    assert text.count(old) >= 1, "mutant %s no longer applies to the source" % name
    text = text.replace(old, new)
    src = os.path.join(tmp, name + ".c")
    lib = os.path.join(tmp, name + ".so")
    with open(src, "w") as fh:
        fh.write(text)
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-std=c11", "-o", lib, src, "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    proc = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", pins)],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, proc.returncode


def test_every_mutant_is_caught():
    jobs = [(n, o, w, "test_oracle.py") for n, (o, w) in MUTANTS.items()]
    jobs += [(n, o, w, "test_oracle_dgrad.py") for n, (o, w) in MUTANTS_DGRAD.items()]
    jobs += [(n, o, w, "test_oracle_wgrad.py") for n, (o, w) in MUTANTS_WGRAD.items()]
    jobs += [(n, o, w, "test_oracle_pool.py") for n, (o, w) in MUTANTS_POOL.items()]
    jobs += [(n, o, w, "test_oracle_brgemm.py") for n, (o, w) in MUTANTS_BRGEMM.items()]
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=4) as pool:
            results = list(pool.map(lambda j: _build_and_run(j[0], j[1], j[2], tmp, j[3]), jobs))
    survivors = [name for name, rc in results if rc == 0]
    assert not survivors, "pins let these oracle mutants through: %s" % survivors
