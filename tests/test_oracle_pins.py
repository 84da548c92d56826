"""The fp64 oracle against facts other than itself (CPU only).

Also plants mistakes in copies of the oracle's C source (on the CPU) and shows
that every one of them trips at least one pin.
"""

import json
import os
import shutil

import numpy as np
import pytest
import torch

import pins

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(oracle_mod, check):
    check(oracle_mod.default())


# Mistakes a plausible slip in the oracle could make: a dropped term, a wrong
# sign, a wrong index or statistic, a wrong normalisation, the wrong operand.
MUTANTS = {
    "drop_mean_dyhat": (
        "rs * (dyh - mean_dyhat - xh * mean_dyhat_xhat)",
        "rs * (dyh - xh * mean_dyhat_xhat)"),
    "sign_of_xhat_term": (
        "rs * (dyh - mean_dyhat - xh * mean_dyhat_xhat)",
        "rs * (dyh - mean_dyhat + xh * mean_dyhat_xhat)"),
    "missing_rstd_factor": (
        "dx[r * N + j] = rs * (dyh - mean_dyhat - xh * mean_dyhat_xhat);",
        "dx[r * N + j] = (dyh - mean_dyhat - xh * mean_dyhat_xhat);"),
    "rms_keeps_mean_dyhat": (
        "(kind == ORACLE_LAYERNORM) ? sum_dyhat / (double)N : 0.0",
        "sum_dyhat / (double)N"),
    "dgamma_uses_raw_x": (
        "dgamma[j] += dy[r * N + j] * xh;",
        "dgamma[j] += dy[r * N + j] * x[r * N + j];"),
    "dbeta_reversed_index": (
        "dbeta[j] += dy[r * N + j];",
        "dbeta[j] += dy[r * N + (N - 1 - j)];"),
    "wgrad_wrong_row_stat": (
        "        double rs = rstd[r];\n        for (long j = 0; j < N; ++j) {\n            double xh = (x[r * N + j] - mu) * rs;\n            dgamma",
        "        double rs = rstd[0];\n        for (long j = 0; j < N; ++j) {\n            double xh = (x[r * N + j] - mu) * rs;\n            dgamma"),
    "unbiased_variance": (
        "v = v / (double)N;", "v = v / (double)(N - 1 > 0 ? N - 1 : 1);"),
    "mean2_over_n_minus_1": (
        "double mean_dyhat_xhat = sum_dyhat_xhat / (double)N;",
        "double mean_dyhat_xhat = sum_dyhat_xhat / (double)(N + 1);"),
    "dyhat_without_gamma": (
        "            double dyh = dyr[j] * gamma[j];\n            dx",
        "            double dyh = dyr[j];\n            dx"),
    "rms_eps_dropped": (
        "rstd[r] = 1.0 / sqrt(q / (double)N + eps);",
        "rstd[r] = 1.0 / sqrt(q / (double)N);"),
    "y_drops_beta": (
        "double b = beta ? beta[j] : 0.0;", "double b = 0.0;"),
    "y_gamma_reversed": (
        "y[r * N + j] = gamma[j] * xh + b;", "y[r * N + j] = gamma[N - 1 - j] * xh + b;"),
    "gamma_transposed_in_sum": (
        "            double dyh = dyr[j] * gamma[j];\n            sum_dyhat += dyh;",
        "            double dyh = dyr[j] * gamma[N - 1 - j];\n            sum_dyhat += dyh;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(oracle_mod, tmp_path, name):
    old, new = MUTANTS[name]
    with open(oracle_mod.SOURCE) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle_mod.compile_library(str(mutated), str(tmp_path / "libmutant.so"))
    mutant = oracle_mod.Oracle(lib)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check(mutant)
        except AssertionError as e:
            caught.append(f"{check.__name__}: {e}")
    assert caught, f"planted mistake {name} passed every pin"


def test_generator_is_seeded_and_distributed():
    from rmsnorm_backward_amd import workloads as W
    w = W.scaled(W.RMS_BF16_262144x768, M=512)
    a, b = W.make_inputs(w), W.make_inputs(w)
    for k in ("x", "dy", "gamma", "outliers"):
        assert torch.equal(a[k], b[k])
    assert a["x"].dtype == torch.bfloat16 and "rstd" not in a and "mean" not in a
    cols = a["outliers"]
    assert cols.numel() == 8                       # 1% of 768 features
    big = a["x"][:, cols].float().abs().mean()
    rest = a["x"].float().abs().mean()
    assert big > 20 * rest
    g = a["gamma"].float()
    assert g.min() >= 0.5 and g.max() <= 1.5
    assert abs(a["dy"].float().std().item() - 1e-2) < 1e-3
    w4 = W.scaled(W.LN_BF16_65536x8192, M=256, N=512)
    x4 = W.make_inputs(w4)["x"].float()
    mu = x4.mean(1)
    sd = x4.std(1)
    assert mu.min() > -2.5 and mu.max() < 2.5 and mu.std() > 0.8
    assert sd.min() > 0.3 and sd.max() < 4.5


def test_pages_worked_numbers_pin_byte_accounting():
    """Byte counts printed in the worked example pin the benchmark's accounting."""
    from rmsnorm_backward_amd import workloads as W
    here = os.path.join(os.path.dirname(__file__), "golden", "worked_numbers.json")
    with open(here) as f:
        wn = json.load(f)
    w = W.HEADLINE
    assert (w.M, w.N, w.io_bytes) == (wn["rows"], wn["features"], wn["io_bytes"])
    read_xdy = 2 * w.M * w.N * w.io_bytes
    write_dx = w.M * w.N * w.io_bytes
    assert read_xdy == wn["dx_pass_read_x_dy"]["exact"]
    assert write_dx == wn["dx_pass_write_dx"]["exact"]
    assert round(read_xdy / 1e9, 2) == 0.27 and round(write_dx / 1e9, 2) == 0.13
    assert 256 * w.N * 4 == wn["workspace_256_groups"]["exact"]
    # algorithmic bytes = x + dy + dx + gamma + rstd + dgamma (fp32)
    assert w.algorithmic_bytes() == read_xdy + write_dx + w.N * 2 + w.M * 4 + w.N * 4
    # the pages' time model: ~0.4 GB at 3.35 TB/s is about 120 us
    t = (read_xdy + write_dx) / 3.35e12 * 1e6
    assert 115 < t < 125


def test_oracle_rejects_bad_shapes(oracle_mod):
    o = oracle_mod.default()
    with pytest.raises(ValueError):
        o.bwd_dx("layernorm", np.zeros((2, 3)), np.zeros((2, 3)), np.zeros(3), None, np.ones(2))
    with pytest.raises(ValueError):
        o.bwd_dx("rmsnorm", np.zeros((2, 3)), np.zeros((2, 4)), np.zeros(3), None, np.ones(2))
    with pytest.raises(ValueError):
        o.fwd_stats("groupnorm", np.zeros((2, 3)), 0.0)
