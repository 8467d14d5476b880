"""The pins must catch plausible mistakes in the oracle.

Each case copies gconv_oracle.c, plants one mistake (a wrong sign, a dropped
term, a transposed index, a missing group offset, ...), compiles the copy
with gcc, swaps it in for the real library and runs a battery of the pins
from test_oracle_pins.py. The battery must fail for every mutant and pass
for the unmodified oracle. Everything here runs on the CPU.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins
from cases import random_descs

# (name, text in gconv_oracle.c, replacement, which occurrence)
MUTANTS = [
    ("fwd_pad_sign", "const int64_t h = ho * d->stride_h - d->pad_h + i * d->dil_h;",
     "const int64_t h = ho * d->stride_h + d->pad_h + i * d->dil_h;", 0),
    ("fwd_no_group_offset", "x[((n * d->C + g * Cg + c) * d->H + h) * d->W + w];",
     "x[((n * d->C + c) * d->H + h) * d->W + w];", 0),
    ("fwd_kernel_transposed", "wt[((k * Cg + c) * d->kh + i) * d->kw + j]",
     "wt[((k * Cg + c) * d->kw + j) * d->kh + i]", 0),
    ("fwd_group_from_Cg", "const int64_t g = k / Kg;", "const int64_t g = k / Cg;", 0),
    ("fwd_bias_dropped", "s += bias[k];", "s += 0.0;", 0),
    ("fwd_dilation_ignored_w", "const int64_t w = wo * d->stride_w - d->pad_w + j * d->dil_w;",
     "const int64_t w = wo * d->stride_w - d->pad_w + j;", 0),
    ("fwd_abs_signed", "a += fabs(p);", "a += p;", 0),
    ("bwd_data_no_stride_check",
     "if (th % d->stride_h != 0 || tw % d->stride_w != 0) continue;", "", 0),
    ("bwd_data_flipped", "const int64_t th = h + d->pad_h - i * d->dil_h;",
     "const int64_t th = h + d->pad_h - (d->kh - 1 - i) * d->dil_h;", 0),
    ("bwd_data_wrong_group", "for (int64_t k = g * Kg; k < (g + 1) * Kg; ++k)",
     "for (int64_t k = 0; k < Kg; ++k)", 0),
    ("bwd_data_wo_bound", "if (ho >= Ho || wo >= Wo) continue;",
     "if (ho >= Ho || wo > Wo) continue;", 0),
    ("bwd_filter_first_image_only", "for (int64_t n = 0; n < d->N; ++n)",
     "for (int64_t n = 0; n < 1; ++n)", 0),
    ("bwd_filter_no_group_offset", "x[((n * d->C + g * Cg + c) * d->H + h) * d->W + w];",
     "x[((n * d->C + c) * d->H + h) * d->W + w];", 1),
    ("bwd_filter_pad_sign", "const int64_t h = ho * d->stride_h - d->pad_h + i * d->dil_h;",
     "const int64_t h = ho * d->stride_h + d->pad_h + i * d->dil_h;", 1),
    # the per-element magnitude A_e of each op (the scale of every tolerance bound)
    ("fwd_abs_bias_dropped", "a += fabs(bias[k]);", "a += 0.0;", 0),
    ("bwd_data_abs_scaled", "a += fabs(p);", "a += 4.0 * fabs(p);", 1),
    ("bwd_filter_abs_scaled", "a += fabs(p);", "a += 4.0 * fabs(p);", 2),
    ("bwd_filter_abs_signed", "a += fabs(p);", "a += p;", 2),
    ("bwd_bias_abs_scaled", "a += fabs(v);", "a += 4.0 * fabs(v);", 0),
    ("bwd_bias_abs_signed", "a += fabs(v);", "a += v;", 0),
    ("bwd_bias_drops_column", "const double v = dy[((n * d->K + k) * Ho + ho) * Wo + wo];",
     "const double v = wo ? dy[((n * d->K + k) * Ho + ho) * Wo + wo] : 0.0;", 0),
    ("extent_ceil", "return num / s + 1;", "return (num + s - 1) / s + 1;", 0),
    ("extent_off_by_one", "int64_t num = in + p0 + p1 - d * (k - 1) - 1;",
     "int64_t num = in + p0 + p1 - d * (k - 1);", 0),
    ("extent_end_pad_ignored", "int64_t num = in + p0 + p1 - d * (k - 1) - 1;",
     "int64_t num = in + 2 * p0 - d * (k - 1) - 1;", 0),
    ("extent_end_pads_swapped", "d->pad_h, d->pad_h_end, d->dil_h);",
     "d->pad_h, d->pad_w_end, d->dil_h);", 0),
]


def _battery():
    """Run a compact set of pins; return the names of those that fail."""
    failed = []

    def run(name, fn):
        try:
            fn()
        except (AssertionError, oracle.OracleError):
            failed.append(name)

    def vs_torch():
        for d in random_descs(42, 10):
            ok = pins.check_against_torch(d, 43)
            assert all(ok.values()), ok

    def closed_forms():
        rng = np.random.default_rng(3)
        x, w = np.ones((3, 8, 4, 3)), np.ones((5, 8, 4, 3))
        y, _ = oracle.fwd(x, w, np.ones(5))
        assert np.all(y == 8 * 4 * 3 + 1)
        dy = rng.standard_normal((2, 6, 5, 4))
        db, _ = oracle.bwd_bias(dy)
        np.testing.assert_allclose(db, dy.sum(axis=(0, 2, 3)), rtol=1e-12)

    run("vs_torch", vs_torch)
    run("golden_shapes", pins.test_golden_shapes)
    run("output_dims_more", pins.test_golden_output_dims_more)
    run("group_narrowing", pins.test_group_narrowing_equals_per_group_convs)
    run("adjoint", pins.test_adjoint_identities)
    run("bias", pins.test_bias_closed_forms)
    run("abs_sum", pins.test_abs_sum_is_sum_of_abs_products)
    run("abs_sums_vs_torch", lambda: pins.test_abs_sums_match_torch(0))
    run("closed_forms", closed_forms)
    run("asym_explicit_pad", lambda: pins.test_asymmetric_padding_equals_explicit_zero_pad(0))
    return failed


def _build_mutant(tmpdir, name, old, new, occurrence):
    src = open(oracle._SRC).read()
    pos = -1
    for _ in range(occurrence + 1):
        pos = src.index(old, pos + 1)       # ValueError if the target text moved
    mutated = src[:pos] + new + src[pos + len(old):]
    c_path = os.path.join(tmpdir, name + ".c")
    so_path = os.path.join(tmpdir, "lib" + name + ".so")
    with open(c_path, "w") as f:
        f.write(mutated)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", so_path,
                    c_path, "-lm"], check=True)
    return oracle.bind(ctypes.CDLL(so_path))


@pytest.fixture
def swap_lib():
    saved = oracle._load()
    yield
    oracle._lib = saved


def test_battery_passes_on_real_oracle(swap_lib):
    assert _battery() == []


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_battery_catches_mutant(tmp_path, swap_lib, name, old, new, occ):
    oracle._lib = _build_mutant(str(tmp_path), name, old, new, occ)
    failed = _battery()
    assert failed, "mutant %s survived every pin" % name
