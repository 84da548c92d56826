"""Checks that pin the fp64 oracle to facts other than itself.

Each ``check_*`` function takes an ``oracle.Oracle`` instance and raises
``AssertionError`` when the oracle disagrees with a fact fixed by the pages or
by the mathematics:

* hand-derived closed forms (``tests/golden/hand_derived_cases.json``);
* central finite differences of L = sum(dy * y) through a forward pass;
* an explicit Jacobian of the forward, derived by hand, applied as a mat-vec;
* torch CPU float64 autograd of ``F.layer_norm`` / ``F.rms_norm``;
* closed forms and invariants: dbeta is the column sum of dy, dgamma does not
  depend on gamma, LayerNorm dx sums to zero over a row, the exact eps
  residual of sum_j dx_j * xhat_j, N = 1 and M = 1 special cases,
  linearity in dy.

``tests/test_oracle_pins.py`` runs them on the real oracle and on copies of
its C source with a planted mistake, each of which must trip at least one.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _eval_expr(s: str) -> float:
    """Evaluate a fixture expression: numbers, + - * / ( ) and sqrt()."""
    allowed = set("0123456789.+-*/() sqrt")
    if not set(s) <= allowed:
        raise ValueError(f"bad fixture expression {s!r}")
    return float(eval(s, {"__builtins__": {}}, {"sqrt": math.sqrt}))  # noqa: S307


def load_hand_cases():
    with open(os.path.join(GOLDEN, "hand_derived_cases.json")) as f:
        data = json.load(f)
    cases = []
    for c in data["cases"]:
        d = dict(c)
        d["x"] = np.array(c["x"], dtype=np.float64)
        d["dy"] = np.array(c["dy"], dtype=np.float64)
        d["gamma"] = np.array(c["gamma"], dtype=np.float64)
        for key in ("dx",):
            d[key] = np.array([[_eval_expr(v) for v in row] for row in c[key]])
        for key in ("dgamma", "dbeta", "rstd", "mean"):
            if key in c:
                d[key] = np.array([_eval_expr(v) for v in c[key]])
        cases.append(d)
    return cases


def _close(a, b, rtol, atol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    if not np.all(err <= lim):
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError(f"{what}: got {a[i]!r} want {b[i]!r} at {i}")


def _rand_problem(rng, kind, M, N, spread=1.0):
    x = rng.standard_normal((M, N)) * spread + (0.7 if kind == "layernorm" else 0.0)
    dy = rng.standard_normal((M, N))
    gamma = rng.uniform(0.5, 1.5, N)
    beta = rng.uniform(-0.5, 0.5, N)
    return x, dy, gamma, beta


# --------------------------------------------------------------------------
def check_hand_cases(orc):
    """Closed forms derived by hand (tests/golden/hand_derived_cases.json)."""
    for c in load_hand_cases():
        kind = c["kind"]
        mean, rstd = orc.fwd_stats(kind, c["x"], c["eps"])
        _close(rstd, c["rstd"], 1e-14, 1e-15, c["name"] + " rstd")
        if kind == "layernorm":
            _close(mean, c["mean"], 1e-14, 1e-15, c["name"] + " mean")
        dx, dg, db = orc.bwd(kind, c["x"], c["dy"], c["gamma"], mean, rstd)
        _close(dx, c["dx"], 1e-13, 1e-14, c["name"] + " dx")
        _close(dg, c["dgamma"], 1e-13, 1e-14, c["name"] + " dgamma")
        _close(db, c["dbeta"], 1e-13, 1e-14, c["name"] + " dbeta")


def check_finite_differences(orc, seed=11):
    """Central differences of L = sum(dy * y(x, gamma, beta)) (stats recomputed
    by the forward) agree with the analytic dx, dgamma, dbeta."""
    rng = np.random.default_rng(seed)
    h = 1e-6
    for kind in ("layernorm", "rmsnorm"):
        for (M, N, eps) in ((3, 7, 1e-5), (2, 16, 0.3), (4, 5, 0.0)):
            x, dy, gamma, beta = _rand_problem(rng, kind, M, N)

            def loss(xx, gg, bb):
                y, _, _ = orc.fwd(kind, xx, gg, bb, eps)
                return float(np.sum(dy * y))

            mean, rstd = orc.fwd_stats(kind, x, eps)
            dx, dg, db = orc.bwd(kind, x, dy, gamma, mean, rstd)
            fdx = np.empty_like(x)
            for i in range(M):
                for j in range(N):
                    xp = x.copy(); xp[i, j] += h
                    xm = x.copy(); xm[i, j] -= h
                    fdx[i, j] = (loss(xp, gamma, beta) - loss(xm, gamma, beta)) / (2 * h)
            fdg = np.empty(N)
            fdb = np.empty(N)
            for j in range(N):
                gp = gamma.copy(); gp[j] += h
                gm = gamma.copy(); gm[j] -= h
                fdg[j] = (loss(x, gp, beta) - loss(x, gm, beta)) / (2 * h)
                bp = beta.copy(); bp[j] += h
                bm = beta.copy(); bm[j] -= h
                fdb[j] = (loss(x, gamma, bp) - loss(x, gamma, bm)) / (2 * h)
            scale = max(1.0, float(np.max(np.abs(dx))))
            _close(dx, fdx, 1e-6, 1e-6 * scale, f"{kind} {M}x{N} eps={eps} FD dx")
            _close(dg, fdg, 1e-6, 1e-6, f"{kind} {M}x{N} FD dgamma")
            _close(db, fdb, 1e-6, 1e-6, f"{kind} {M}x{N} FD dbeta")


def check_jacobian(orc, seed=12):
    """dx = J^T dy with the hand-derived Jacobian of one row:
    dy_i/dx_j = gamma_i * rstd * (delta_ij - 1/N - xhat_i*xhat_j/N) (LayerNorm),
    RMSNorm without the 1/N term."""
    rng = np.random.default_rng(seed)
    for kind in ("layernorm", "rmsnorm"):
        for (M, N, eps) in ((3, 6, 1e-5), (2, 9, 0.5)):
            x, dy, gamma, _ = _rand_problem(rng, kind, M, N)
            mean, rstd = orc.fwd_stats(kind, x, eps)
            dx = orc.bwd_dx(kind, x, dy, gamma, mean, rstd)
            for r in range(M):
                mu = mean[r] if kind == "layernorm" else 0.0
                xh = (x[r] - mu) * rstd[r]
                J = np.eye(N) - np.outer(xh, xh) / N
                if kind == "layernorm":
                    J -= 1.0 / N
                J = (gamma[:, None] * rstd[r]) * J      # J[i, j] = dy_i/dx_j
                want = J.T @ dy[r]
                _close(dx[r], want, 1e-12, 1e-13, f"{kind} jacobian row {r}")


def check_torch_autograd(orc, seed=13):
    """torch CPU float64 autograd of F.layer_norm / F.rms_norm, and their
    forward outputs."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(seed)
    for kind in ("layernorm", "rmsnorm"):
        for (M, N, eps) in ((5, 33, 1e-5), (3, 128, 1e-6), (1, 1, 1e-5), (2, 2, 0.1)):
            x, dy, gamma, beta = _rand_problem(rng, kind, M, N, spread=2.0)
            tx = torch.tensor(x, requires_grad=True)
            tg = torch.tensor(gamma, requires_grad=True)
            tb = torch.tensor(beta, requires_grad=True)
            if kind == "layernorm":
                y = F.layer_norm(tx, (N,), tg, tb, eps)
            else:
                y = F.rms_norm(tx, (N,), tg, eps) + tb
            y.backward(torch.tensor(dy))
            mean, rstd = orc.fwd_stats(kind, x, eps)
            dx, dg, db = orc.bwd(kind, x, dy, gamma, mean, rstd)
            _close(dx, tx.grad.numpy(), 1e-10, 1e-12, f"{kind} {M}x{N} torch dx")
            _close(dg, tg.grad.numpy(), 1e-10, 1e-12, f"{kind} {M}x{N} torch dgamma")
            _close(db, tb.grad.numpy(), 1e-12, 1e-12, f"{kind} {M}x{N} torch dbeta")
            # the forward output matches torch's forward (with beta, and without)
            oy, _, _ = orc.fwd(kind, x, gamma, beta, eps)
            _close(oy, y.detach().numpy(), 1e-12, 1e-13, f"{kind} {M}x{N} torch y")
            with torch.no_grad():
                if kind == "layernorm":
                    y0 = F.layer_norm(torch.tensor(x), (N,), torch.tensor(gamma), None, eps)
                else:
                    y0 = F.rms_norm(torch.tensor(x), (N,), torch.tensor(gamma), eps)
            oy0, _, _ = orc.fwd(kind, x, gamma, None, eps)
            _close(oy0, y0.numpy(), 1e-12, 1e-13, f"{kind} {M}x{N} torch y (no beta)")
            # the forward statistics the oracle saves match torch's
            xt = torch.tensor(x)
            if kind == "layernorm":
                var, mu = torch.var_mean(xt, dim=1, unbiased=False)
                _close(mean, mu.numpy(), 1e-13, 1e-14, "torch mean")
                _close(rstd, torch.rsqrt(var + eps).numpy(), 1e-12, 0, "torch rstd")
            else:
                _close(rstd, torch.rsqrt(xt.square().mean(1) + eps).numpy(), 1e-12, 0,
                       "torch rms rstd")


def check_invariants(orc, seed=14):
    """Closed forms and invariants that hold for any input."""
    rng = np.random.default_rng(seed)
    for kind in ("layernorm", "rmsnorm"):
        M, N = 6, 40
        for eps in (0.0, 1e-5, 0.7):
            x, dy, gamma, _ = _rand_problem(rng, kind, M, N)
            mean, rstd = orc.fwd_stats(kind, x, eps)
            dx, dg, db = orc.bwd(kind, x, dy, gamma, mean, rstd)
            mu = mean[:, None] if kind == "layernorm" else 0.0
            xh = (x - mu) * rstd[:, None]
            # dbeta is the column sum of dy
            _close(db, np.sum(dy, axis=0), 1e-13, 1e-13, "dbeta = column sum of dy")
            # LayerNorm: every row of dx sums to zero
            if kind == "layernorm":
                _close(dx.sum(1), np.zeros(M), 0, 1e-12, "LN sum_j dx = 0")
            # sum_j dx_j xhat_j = N * m2 * eps * rstd^3, m2 = mean_j(dy*gamma*xhat)
            m2 = np.mean(dy * gamma * xh, axis=1)
            want = N * m2 * eps * rstd ** 3
            _close((dx * xh).sum(1), want, 1e-9, 1e-12, f"{kind} eps={eps} sum dx*xhat")
            # dgamma does not depend on gamma
            dg2 = orc.bwd_wgrad(kind, x, dy, mean, rstd)[0]
            dx3, dg3, _ = orc.bwd(kind, x, dy, gamma * 3.0 + 1.0, mean, rstd)
            _close(dg3, dg2, 0, 0, "dgamma independent of gamma")
            _close(dg, dg2, 0, 0, "bwd and bwd_wgrad agree")
            # linearity in dy
            dxa, dga, dba = orc.bwd(kind, x, 2.5 * dy, gamma, mean, rstd)
            _close(dxa, 2.5 * dx, 1e-13, 1e-14, "dx linear in dy")
            _close(dga, 2.5 * dg, 1e-13, 1e-14, "dgamma linear in dy")
            # M = 1 rows: dgamma = dy * xhat of that row
            for r in (0, M - 1):
                sub = (slice(r, r + 1),)
                d1 = orc.bwd_wgrad(kind, x[sub], dy[sub],
                                   None if mean is None else mean[sub], rstd[sub])[0]
                _close(d1, dy[r] * xh[r], 1e-15, 1e-15, "M=1 dgamma = dy*xhat")
            # dyhat constant within each row => LayerNorm dx = 0
            if kind == "layernorm":
                dyc = np.repeat(rng.standard_normal((M, 1)), N, axis=1) / gamma[None, :]
                _close(orc.bwd_dx(kind, x, dyc, gamma, mean, rstd), np.zeros((M, N)),
                       0, 1e-12, "constant dyhat => dx = 0")
            # eps = 0 RMSNorm: dx orthogonal to x
            if kind == "rmsnorm" and eps == 0.0:
                _close((dx * x).sum(1), np.zeros(M), 0, 1e-11, "RMS eps=0 dx . x = 0")
        # N = 1: LayerNorm dx = 0 and dgamma = 0; RMSNorm dx = eps*rstd^3*dyhat
        x1, dy1, g1, _ = _rand_problem(rng, kind, 5, 1)
        eps = 0.25
        mean1, rstd1 = orc.fwd_stats(kind, x1, eps)
        dx1, dg1, _ = orc.bwd(kind, x1, dy1, g1, mean1, rstd1)
        if kind == "layernorm":
            _close(dx1, np.zeros_like(dx1), 0, 0, "LN N=1 dx = 0")
            _close(dg1, np.zeros_like(dg1), 0, 0, "LN N=1 dgamma = 0")
        else:
            want = eps * rstd1[:, None] ** 3 * dy1 * g1[None, :]
            _close(dx1, want, 1e-12, 1e-15, "RMS N=1 dx")


def check_empty(orc):
    """M = 0: dgamma and dbeta are the empty sum."""
    for kind in ("layernorm", "rmsnorm"):
        x = np.zeros((0, 5))
        mean = np.zeros(0) if kind == "layernorm" else None
        dg, db = orc.bwd_wgrad(kind, x, x, mean, np.zeros(0))
        _close(dg, np.zeros(5), 0, 0, "M=0 dgamma")
        _close(db, np.zeros(5), 0, 0, "M=0 dbeta")


ALL_CHECKS = [check_hand_cases, check_finite_differences, check_jacobian,
              check_torch_autograd, check_invariants, check_empty]
