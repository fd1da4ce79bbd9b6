"""Planted mistakes in the CPU oracle must be caught by its pins.

Each case compiles a copy of oracle/sla_oracle.c with one plausible mistake
(a dropped term, a wrong sign, a wrong or transposed index) into a temporary
directory and runs the pins of that part of the oracle (tests/test_oracle_pins.py,
or tests/test_oracle_bicgstab.py for BiCGStab) against it in a subprocess.  CPU
only; nothing here touches a GPU or the HIP library.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sla_oracle.c")

PINS = "test_oracle_pins.py"
BICG = "test_oracle_bicgstab.py"
MUTANTS = {
    "gradient sign": ("gvals[k] = sign * t;", "gvals[k] = -sign * t;"),
    "gradient orientation": ("double t = u[i] * v[col[k]];", "double t = u[col[k]] * v[i];"),
    "spmv column index": ("double t = val[k] * x[col[k]];\n            s = s + t;",
                          "double t = val[k] * x[col[k] > 0 ? col[k] - 1 : 0];\n            s = s + t;"),
    "beta inverted": ("double beta = rho1 / rho;", "double beta = rho / rho1;"),
    "residual sign": ("r[i] = r[i] - t;", "r[i] = r[i] + t;"),
    "beta term dropped": ("p[i] = r[i] + t;", "p[i] = r[i];"),
    "alpha perturbed": ("double alpha = rho / sigma;", "double alpha = rho / sigma * 1.0000001;"),
    "transpose permutation": ("perm[dst] = k;", "perm[dst] = k ^ 1;"),
    "threshold not relative": ("double thr = rtol * bnorm;", "double thr = rtol;"),
    "adjoint ignores transpose": ("if (symmetric) {", "if (1) {"),
    "transposed spmv is forward": ("y[col[k]] = y[col[k]] + t;", "y[i] = y[i] + val[k] * x[col[k]];"),
    "dot drops the product remainders": ("c = c + (q + r);", "c = c + q;"),
    "dot is a plain sequential sum": ("return s + c;", "return s;"),
    "pcg without the preconditioner": ("            z[i] = r[i] / d[i];", "            z[i] = r[i];"),
    "pcg beta from <r,r>": ("double rho1 = orc_dot(n, r, z);", "double rho1 = orc_dot(n, r, r);"),
    "pcg direction from r": ("            p[i] = z[i] + t;", "            p[i] = r[i] + t;"),
    # BiCGStab: caught by tests/test_oracle_bicgstab.py
    "bicgstab beta without alpha/omega": ("double beta = (rho1 / rho) * (alpha / omega);",
                                          "double beta = rho1 / rho;", BICG),
    "bicgstab direction drops omega v": ("double d = p[i] - tv;", "double d = p[i];", BICG),
    "bicgstab x update drops omega s": ("x[i] = x1 + ts_;", "x[i] = x1;", BICG),
    "bicgstab residual sign": ("r[i] = s[i] - tt_;", "r[i] = s[i] + tt_;", BICG),
    "bicgstab omega from <s,s>": ("omega = ts / tt;", "omega = ts / ss;", BICG),
    "bicgstab shadow residual follows r": ("double rv = orc_dot(n, rh, v);", "double rv = orc_dot(n, r, v);",
                                           BICG),
    "bicgstab half-way stop skips x": ("                x[i] = x[i] + tp;", "                x[i] = x[i];",
                                       BICG),
    "bicgstab adjoint without transpose": ("    if (symmetric) {", "    if (symmetric || method == 2) {",
                                           BICG),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(SRC).read()
    a, b, pins = (MUTANTS[name] + (PINS,))[:3]
    assert a in src, "mutation anchor vanished from the oracle source"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(a, b, 1))
    so = tmp_path / "mut.so"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-shared", "-fPIC", str(mut),
                           "-o", str(so), "-lm"])
    env = dict(os.environ, SLA_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", pins)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "pins missed the planted mistake: " + name


# The Lanczos eigensolver is Python (oracle/eigsh.py): mutated copies are loaded by
# tests/test_oracle_eigsh.py through SLA_ORACLE_EIGSH.
EIGSH = os.path.join(ROOT, "oracle", "eigsh.py")
EIGSH_MUTANTS = {
    # (a wrong sign in the three-term step is not a mistake in effect: the full
    # reorthogonalization that follows removes any multiple of v_j and v_{j-1})
    "lanczos alpha from v_0": ("a = dot(V[j], w)", "a = dot(V[0], w)"),
    "lanczos without reorthogonalization": ("for _ in range(2):", "for _ in range(0):"),
    "lanczos residual from the first component": ("res = b * np.abs(S[m - 1, idx])", "res = b * np.abs(S[0, idx])"),
    "ritz vectors from a shifted basis": ("U = S[:, idx].T @ V[:m]", "U = S[:, idx].T @ V[1:m + 1]"),
    "largest taken in ascending order": ("order = np.arange(m - 1, -1, -1) if which", "order = np.arange(m) if which"),
    "sign convention dropped": ("if dot(U[i], v) < 0.0:", "if False:"),
    "gradient weights of the first eigenvalue": ("float(g_evals[m])", "float(g_evals[0])"),
    "gradient of the first eigenvector only": ("pattern_outer(A, evecs[m], evecs[m], sign=1.0)",
                                               "pattern_outer(A, evecs[0], evecs[0], sign=1.0)"),
    "restart coupling from the first component": ("H[i, l_keep] = H[l_keep, i] = b * S[m - 1, c]",
                                                  "H[i, l_keep] = H[l_keep, i] = b * S[0, c]"),
    "restart keeps the wrong end": ("kept = order[:l_keep]", "kept = order[::-1][:l_keep]"),
    "restart drops the next Lanczos vector": ("V[l_keep] = nxt", "V[l_keep] = 0.0 * nxt"),
}


@pytest.mark.parametrize("name", sorted(EIGSH_MUTANTS))
def test_eigsh_pins_catch_planted_mistake(name, tmp_path):
    src = open(EIGSH).read()
    a, b = EIGSH_MUTANTS[name]
    assert a in src, "mutation anchor vanished from the oracle source"
    mut = tmp_path / "eigsh_mut.py"
    mut.write_text(src.replace(a, b, 1))
    env = dict(os.environ, SLA_ORACLE_EIGSH=str(mut), OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_eigsh.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "pins missed the planted mistake: " + name


# The LOBPCG eigensolver (oracle/lobpcg.py), loaded by tests/test_oracle_lobpcg.py
# through SLA_ORACLE_LOBPCG.  (Leaving out the projection of W against X is not a
# mistake in effect: the residuals of Ritz pairs are orthogonal to the Ritz space
# already.)
LOBPCG = os.path.join(ROOT, "oracle", "lobpcg.py")
LOBPCG_MUTANTS = {
    "residual with the wrong sign": ("R = AX - X * theta", "R = AX + X * theta"),
    "AX not rotated with the Ritz vectors": ("X, AX = S @ Y, AS @ Y", "X, AX = S @ Y, AS[:, :k]"),
    "largest taken from the smallest end": (
        "idx = np.arange(len(w) - 1, len(w) - 1 - k, -1) if which == \"largest\" else np.arange(k)",
        "idx = np.arange(k)"),
    "cholesky factor not transposed": ("Rinv = np.linalg.inv(L.T)", "Rinv = np.linalg.inv(L)"),
    "ritz values from the diagonal of H": ("theta, Y = _wanted(S.T @ AS, k, which)",
                                           "theta, Y = np.diag(S.T @ AS)[:k].copy(), np.eye(S.shape[1])[:, :k]"),
    "sign convention dropped": ("if U[r] @ X0[r] < 0.0:", "if False:"),
    "stop test on the absolute residual": ("active = res > tol * np.abs(theta)", "active = res > tol"),
    "preconditioner ignored": ("W = R[:, active] * tinv[:, None] if jacobi else R[:, active]",
                               "W = R[:, active]"),
    "conjugate direction from the X part": ("P, AP = S[:, k:] @ Y[k:, :], AS[:, k:] @ Y[k:, :]",
                                            "P, AP = S[:, :k] @ Y[:k, :], AS[:, :k] @ Y[:k, :]"),
}


@pytest.mark.parametrize("name", sorted(LOBPCG_MUTANTS))
def test_lobpcg_pins_catch_planted_mistake(name, tmp_path):
    src = open(LOBPCG).read()
    a, b = LOBPCG_MUTANTS[name]
    assert a in src, "mutation anchor vanished from the oracle source"
    mut = tmp_path / "lobpcg_mut.py"
    mut.write_text(src.replace(a, b, 1))
    env = dict(os.environ, SLA_ORACLE_LOBPCG=str(mut), OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_lobpcg.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "pins missed the planted mistake: " + name
