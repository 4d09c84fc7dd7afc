"""The oracle's pins must fail on plausible mistakes.

Each case plants one mistake (a dropped term, a wrong sign, index, operand or
rounding rule) in a temporary copy of the oracle and runs the pin tests against
that copy; every mutant must be caught.  The oracle file itself is untouched.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kronq_oracle.py")

MUTANTS = [
    ("gram normalization", "return (A.T @ A) / A.shape[0]", "return (A.T @ A) / (A.shape[0] - 1)"),
    ("butterfly sign", "y[..., 1, :] = a - b", "y[..., 1, :] = b - a"),
    ("rotation normalization", "return fwht(Y).reshape(rows, d) / np.sqrt(block)",
     "return fwht(Y).reshape(rows, d) / block"),
    ("rescale exponent", "s[pos] = d[pos] ** alpha", "s[pos] = d[pos] ** (2 * alpha)"),
    ("H_G rescale direction", "HGs = np.asarray(HG, dtype=np.float64) / s[:, None] / s[None, :]",
     "HGs = np.asarray(HG, dtype=np.float64) * s[:, None] * s[None, :]"),
    ("W rescale direction", "Ws = W * s[:, None]", "Ws = W / s[:, None]"),
    ("act-order tie order", 'return np.argsort(-d, kind="stable").astype(np.int64)',
     'return np.argsort(d, kind="stable")[::-1].astype(np.int64)'),
    ("damping scale", "return H + lam * np.mean(np.diag(H)) * np.eye(H.shape[0])",
     "return H + lam * np.eye(H.shape[0])"),
    ("factor of H instead of H^-1", "R = np.linalg.cholesky(Hinv).T", "R = np.linalg.cholesky(H).T"),
    ("range without zero", "xmin = np.minimum(V.min(axis=1), 0.0)\n    xmax = np.maximum(V.max(axis=1), 0.0)\n    deg = xmin == xmax\n    xmin = np.where(deg, -1.0, xmin)\n    xmax = np.where(deg, 1.0, xmax)\n    scale",
     "xmin = V.min(axis=1)\n    xmax = V.max(axis=1)\n    deg = xmin == xmax\n    xmin = np.where(deg, -1.0, xmin)\n    xmax = np.where(deg, 1.0, xmax)\n    scale"),
    ("zero point floor", "zero = np.rint(-xmin / scale)\n    return scale, zero",
     "zero = np.floor(-xmin / scale)\n    return scale, zero"),
    ("error scaling", "e = (Wt[:, j] - wq) / R[j, j]", "e = (Wt[:, j] - wq) * R[j, j]"),
    ("update sign", "Wt[:, j + 1:] -= np.outer(e, R[j, j + 1:])", "Wt[:, j + 1:] += np.outer(e, R[j, j + 1:])"),
    ("transposed factor", "Wt[:, j + 1:] -= np.outer(e, R[j, j + 1:])", "Wt[:, j + 1:] -= np.outer(e, R[j + 1:, j])"),
    ("group params from uncompensated W", "scale, zero = quant_params(Wt[:, j:j + group], bits)",
     "scale, zero = quant_params(W[:, perm][:, j:j + group], bits)"),
    ("round half up", "q = np.clip(np.rint(t), 0, maxq)\n        if decide_codes",
     "q = np.clip(np.floor(t + 0.5), 0, maxq)\n        if decide_codes"),
    ("dropped trace term", "trg = float(np.sum(np.diag(np.asarray(HGp, dtype=np.float64))))",
     "trg = float(np.sum(np.diag(np.asarray(HGp, dtype=np.float64))[1:]))"),
    ("ascending allocation", "order = sorted(range(L), key=lambda i: (-float(scores[i]), i))",
     "order = sorted(range(L), key=lambda i: (float(scores[i]), i))"),
    ("budget boundary", "while bits[i] < bmax and used + n_params[i] <= budget_bits:",
     "while bits[i] < bmax and used + n_params[i] < budget_bits:"),
    ("wrong un-permutation", "codes=codes[:, inv]", "codes=codes[:, perm]"),
    ("pack big-endian in a byte", "<< (bits * (j % per))", "<< (bits * (per - 1 - j % per))"),
    ("dequant group by natural column",
     "pos = np.arange(n) if perm is None else np.argsort(np.asarray(perm, dtype=np.int64))",
     "pos = np.arange(n)"),
    ("dequant zero sign", "return scales[:, g] * (q - zeros[:, g])", "return scales[:, g] * (q + zeros[:, g])"),
    ("unrotate output signs misaligned", "A = A * np.asarray(out_signs, dtype=np.float64)[:, None]",
     "A = A * np.asarray(out_signs, dtype=np.float64)[::-1][:, None]"),
    ("unrotate rescale direction", "return B / np.asarray(sg, dtype=np.float64)[:, None]",
     "return B * np.asarray(sg, dtype=np.float64)[:, None]"),
    ("decode input transform normalization", "          / np.sqrt(in_block))", "          / in_block)"),
    ("pass-wise stops after one pass", "                changed = True\n    return bits",
     "                changed = False\n    return bits"),
    ("marginal gain with eps ~ 2^-b/2", "return math.ldexp(float(score), -2 * b) / float(n)",
     "return math.ldexp(float(score), -b) / float(n)"),
    ("marginal gain ignores the cost", "return math.ldexp(float(score), -2 * b) / float(n)",
     "return math.ldexp(float(score), -2 * b)"),
    ("type score by the largest member", "        total[int(t)] += float(s)",
     "        total[int(t)] = max(total[int(t)], float(s))"),
    ("CV with the sample deviation", "return float(np.std(col) / np.mean(col)), float(np.std(row) / np.mean(row))",
     "return float(np.std(col, ddof=1) / np.mean(col)), float(np.std(row, ddof=1) / np.mean(row))"),
    ("CV columns and rows swapped", "    col = np.sqrt(np.sum(W * W, axis=0))\n    row = np.sqrt(np.sum(W * W, axis=1))",
     "    col = np.sqrt(np.sum(W * W, axis=1))\n    row = np.sqrt(np.sum(W * W, axis=0))"),
    ("su_only keeps the input side", "return biip(W, HX, HG, np.ones(n), 1, out_signs, out_block, alpha)",
     "return biip(W, HX, HG, in_signs, in_block, out_signs, out_block, alpha)"),
    ("sv_only keeps the rescale", "return biip(W, HX, HG, in_signs, in_block, np.ones(m), 1, 0.0)",
     "return biip(W, HX, HG, in_signs, in_block, np.ones(m), 1, alpha)"),
    ("act-order reordering transposed", "Hp = np.asarray(HXp, dtype=np.float64)[np.ix_(perm, perm)]",
     "Hp = np.asarray(HXp, dtype=np.float64)[np.ix_(np.argsort(perm), np.argsort(perm))]"),
    ("zero pre-round snapped to a half-integer", "    return -xmin / ((xmax - xmin) / maxq)",
     "    return np.floor(-xmin / ((xmax - xmin) / maxq)) + 0.5"),
    ("GPTAQ mask with the diagonal", "return alpha * (np.triu(K, 1) @ R)", "return alpha * (np.triu(K, 0) @ R)"),
    ("GPTAQ factor not transposed", "K = C @ R.T\n    return alpha", "K = C @ R\n    return alpha"),
    ("GPTAQ drift term sign",
     "Wt[:, j + 1:] -= np.outer(e, R[j, j + 1:]) - np.outer(W0[:, j], P[j, j + 1:])",
     "Wt[:, j + 1:] -= np.outer(e, R[j, j + 1:]) + np.outer(W0[:, j], P[j, j + 1:])"),
    ("GPTAQ drift term on compensated weights",
     "Wt[:, j + 1:] -= np.outer(e, R[j, j + 1:]) - np.outer(W0[:, j], P[j, j + 1:])",
     "Wt[:, j + 1:] -= np.outer(e, R[j, j + 1:]) - np.outer(Wt[:, j], P[j, j + 1:])"),
    ("drift cross product transposed", "    return (dX.T @ X) / X.shape[0]", "    return (X.T @ dX) / X.shape[0]"),
    ("S_X on H_X multiplies", "HXs = np.asarray(HX, dtype=np.float64) / sx[:, None] / sx[None, :]",
     "HXs = np.asarray(HX, dtype=np.float64) * sx[:, None] * sx[None, :]"),
    ("S_X on W divides", "biip(W * sx[None, :], None", "biip(W / sx[None, :], None"),
    ("S_X exponent sign", "s[pos] = d[pos] ** alpha_x", "s[pos] = d[pos] ** (-alpha_x)"),
    ("S_X from the rotated H_X", "        sx = input_rescale(HX, alpha_x)",
     "        sx = input_rescale(rotate_cols(rotate_rows(HX, in_block, in_signs), in_block, in_signs), alpha_x)"),
    ("unrotate S_X direction", "/ np.asarray(sx, dtype=np.float64)[None, :]",
     "* np.asarray(sx, dtype=np.float64)[None, :]"),
    ("mu without the 1/sqrt(d)", "    return float(np.max(np.abs(Q)))",
     "    return float(np.max(np.abs(Q)) * math.sqrt(Q.shape[0]))"),
    ("mu of the least coherent eigenvector", "    return float(np.max(np.abs(Q)))",
     "    return float(np.min(np.max(np.abs(Q), axis=0)))"),
    ("type ties to the higher id", "ranked = sorted(range(n_types), key=lambda t: (-total[t], t))",
     "ranked = sorted(range(n_types), key=lambda t: (-total[t], -t))"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation anchor not found: " + name
    (tmp_path / "mutant_oracle.py").write_text(text.replace(old, new, 1))
    env = dict(os.environ)
    env["PYTHONPATH"] = str(tmp_path) + os.pathsep + env.get("PYTHONPATH", "")
    env["KRONQ_ORACLE_UNDER_TEST"] = "mutant_oracle"
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, "pins did not catch the planted mistake: " + name
