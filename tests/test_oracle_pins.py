"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test ties one oracle function to something other than itself: a closed
form, an identity stated on the pages (Kronecker objective, Proposition 1's
H_G cancellation, Theorem 1's rotation invariance, the trace of a Kronecker
product), brute force on tiny inputs, or a hand-worked value stored under
tests/golden/ with its derivation.
"""
import importlib
import itertools
import json
import os

import math

import numpy as np
import pytest

# the mutation test points this at a planted-mistake copy of the oracle
O = importlib.import_module(os.environ.get("KRONQ_ORACLE_UNDER_TEST", "oracle.kronq_oracle"))

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def rand_spd(rng, d, cond=10.0):
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    ev = np.geomspace(1.0, cond, d)
    return (Q * ev) @ Q.T


# ---------------------------------------------------------------- Gram


def test_gram_brute_force_integer():
    rng = np.random.default_rng(0)
    A = rng.integers(-3, 4, size=(7, 3)).astype(float)
    H = O.gram(A)
    for i in range(3):
        for j in range(3):
            s = 0.0
            for t in range(7):
                s += A[t][i] * A[t][j]
            assert H[i, j] == s / 7


def test_gram_closed_form_hadamard_rows():
    # rows of a Hadamard matrix are orthogonal: X^T X = N I exactly
    X = O.hadamard_matrix(16)
    np.testing.assert_array_equal(O.gram(X), np.eye(16))


def test_gram_symmetric_psd():
    rng = np.random.default_rng(1)
    H = O.gram(rng.standard_normal((50, 9)))
    np.testing.assert_array_equal(H, H.T)
    assert np.linalg.eigvalsh(H).min() > -1e-12


# ------------------------------------------------- Kronecker objective


def test_kronecker_identity():
    # vec(dW)^T (H_X (x) H_G) vec(dW) = tr(H_G dW H_X dW^T)
    rng = np.random.default_rng(2)
    for m, n in [(2, 3), (3, 5), (4, 4)]:
        dW = rng.standard_normal((m, n))
        HX, HG = rand_spd(rng, n), rand_spd(rng, m)
        a = O.proxy_loss(dW, HX, HG)
        b = O.proxy_loss_kron(dW, HX, HG)
        assert abs(a - b) <= 1e-12 * abs(b)


def test_objective_identity_factors_is_frobenius():
    rng = np.random.default_rng(3)
    dW = rng.standard_normal((3, 4))
    assert O.proxy_loss(dW, np.eye(4), np.eye(3)) == pytest.approx(np.sum(dW * dW), rel=1e-14)


# ------------------------------------------------------------ Hadamard


def test_hadamard_printed_and_sylvester():
    np.testing.assert_array_equal(O.hadamard_matrix(4), np.array(gold("hadamard_sylvester_4.json")["H4"]))
    np.testing.assert_array_equal(O.hadamard_matrix(1), [[1.0]])
    for k in [2, 4, 8, 32]:
        H = O.hadamard_matrix(k)
        h = O.hadamard_matrix(k // 2)
        np.testing.assert_array_equal(H, np.block([[h, h], [h, -h]]))
        np.testing.assert_array_equal(H @ H.T, k * np.eye(k))


def test_fwht_matches_matrix_and_special_vectors():
    rng = np.random.default_rng(4)
    for k in [1, 2, 8, 64, 256]:
        x = rng.standard_normal((3, k))
        np.testing.assert_allclose(O.fwht(x), x @ O.hadamard_matrix(k), rtol=0, atol=1e-12 * k)
        # delta -> first row of H (all ones); constant -> k * delta
        d = np.zeros(k); d[0] = 1.0
        np.testing.assert_array_equal(O.fwht(d), np.ones(k))
        c = np.ones(k)
        e = np.zeros(k); e[0] = k
        np.testing.assert_array_equal(O.fwht(c), e)
        # round trip: H H = k I
        np.testing.assert_allclose(O.fwht(O.fwht(x)) / k, x, rtol=0, atol=1e-12 * k)


def test_rotation_orthogonal_and_matches_explicit():
    rng = np.random.default_rng(5)
    for d, b in [(16, 16), (12, 4), (24, 8), (43 * 4, 4)]:
        s = rng.choice([-1.0, 1.0], size=d)
        T = O.rotation_matrix(d, b, s)
        np.testing.assert_allclose(T @ T.T, np.eye(d), atol=1e-13)
        M = rng.standard_normal((5, d))
        np.testing.assert_allclose(O.rotate_rows(M, b, s), M @ T.T, atol=1e-12)
        np.testing.assert_allclose(O.rotate_cols(M.T, b, s), T @ M.T, atol=1e-12)
        # block-diagonal: mixing stays inside each block
        assert np.all(T[:b, b:] == 0)


def test_rotation_spreads_a_spike():
    # W = c e_i e_j^T: every entry of U W V^T inside the (i-block, j-block)
    # has magnitude c / sqrt(k_out k_in): maximal incoherence of a spike
    m, n, ko, ki = 8, 16, 8, 4
    W = np.zeros((m, n)); W[3, 5] = 2.0
    rng = np.random.default_rng(6)
    so, si = rng.choice([-1.0, 1.0], m), rng.choice([-1.0, 1.0], n)
    Wp, _, _, _ = O.biip(W, None, np.eye(m), si, ki, so, ko, 0.0)
    blk = np.abs(Wp[:, 4:8])
    np.testing.assert_allclose(blk, np.full_like(blk, 2.0 / np.sqrt(ko * ki)), atol=1e-14)
    assert np.count_nonzero(np.abs(Wp) > 1e-15) == ko * ki


# ---------------------------------------------------------------- BiIP


def _biip_case(seed, m=8, n=12, ki=4, ko=8, alpha=0.25):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((m, n))
    HX = rand_spd(rng, n, 50.0)
    HG = rand_spd(rng, m, 1e3)
    si, so = rng.choice([-1.0, 1.0], n), rng.choice([-1.0, 1.0], m)
    return W, HX, HG, si, ki, so, ko, alpha


def test_biip_explicit_matrices():
    W, HX, HG, si, ki, so, ko, a = _biip_case(7)
    Wp, HXp, HGp, s = O.biip(W, HX, HG, si, ki, so, ko, a)
    U = O.rotation_matrix(W.shape[0], ko, so)
    V = O.rotation_matrix(W.shape[1], ki, si)
    S = np.diag(np.diag(HG) ** a)
    np.testing.assert_allclose(Wp, U @ S @ W @ V.T, atol=1e-12)
    np.testing.assert_allclose(HXp, V @ HX @ V.T, atol=1e-10)
    Si = np.linalg.inv(S)
    np.testing.assert_allclose(HGp, U @ Si @ HG @ Si @ U.T, atol=1e-10)


def test_biip_objective_invariance_theorem1():
    # Theorem 1 (rotation invariance), extended to the S_G rescale: the
    # objective of any perturbation is the same before and after BiIP
    W, HX, HG, si, ki, so, ko, a = _biip_case(8)
    rng = np.random.default_rng(9)
    dW = rng.standard_normal(W.shape)
    dWp, HXp, HGp, _ = O.biip(dW, HX, HG, si, ki, so, ko, a)
    assert O.proxy_loss(dWp, HXp, HGp) == pytest.approx(O.proxy_loss(dW, HX, HG), rel=1e-11)


def test_biip_trace_closed_forms():
    W, HX, HG, si, ki, so, ko, a = _biip_case(10)
    _, HXp, HGp, s = O.biip(W, HX, HG, si, ki, so, ko, a)
    assert np.trace(HXp) == pytest.approx(np.trace(HX), rel=1e-13)
    assert np.trace(HGp) == pytest.approx(np.sum(np.diag(HG) ** (1 - 2 * a)), rel=1e-13)
    np.testing.assert_allclose(s, np.diag(HG) ** a, rtol=1e-15)
    # alpha = 0: no rescale, H_G trace preserved
    _, _, HGp0, s0 = O.biip(W, HX, HG, si, ki, so, ko, 0.0)
    np.testing.assert_array_equal(s0, np.ones_like(s0))
    assert np.trace(HGp0) == pytest.approx(np.trace(HG), rel=1e-13)


def test_biip_zero_diagonal_rescale_is_one():
    HG = np.diag([4.0, 0.0, 9.0])
    np.testing.assert_allclose(O.output_rescale(HG, 0.5), [2.0, 1.0, 3.0])


# ---------------------------------------------- act-order, damping, R


def test_act_order_ties_stable():
    H = np.diag([1.0, 3.0, 3.0, 2.0])
    np.testing.assert_array_equal(O.act_order_perm(H), [1, 2, 3, 0])


def test_prepare_hessian_explicit_permutation_matrix():
    # Algorithm 2's damping (H + lambda mean(diag H) I) and the act-order
    # reordering, checked against an explicit permutation matrix P with
    # P[j, perm[j]] = 1 (row j of Hd is original column perm[j]):
    # Hd = P (H + lambda mean(diag) I) P^T.  The diagonal 1, 4, 2, 3 gives
    # perm = [1, 3, 2, 0], which is not its own inverse ([3, 0, 2, 1]), so a
    # transposed reordering is caught.
    rng = np.random.default_rng(21)
    n = 4
    A = rng.standard_normal((n, n)) * 0.1
    H = A @ A.T + np.diag([1.0, 4.0, 2.0, 3.0])
    perm, Hd = O.prepare_hessian(H, 0.05, True)
    np.testing.assert_array_equal(perm, [1, 3, 2, 0])
    P = np.zeros((n, n))
    P[np.arange(n), perm] = 1.0
    lam_mu = 0.05 * np.trace(H) / n
    np.testing.assert_allclose(Hd, P @ (H + lam_mu * np.eye(n)) @ P.T, rtol=0, atol=1e-15)
    # processing-order diagonal is descending; the damped matrix factors
    assert np.all(np.diff(np.diag(Hd)) <= 0)
    R, info = O.chol_inv_upper(Hd)
    assert info == -1
    np.testing.assert_allclose(R.T @ R @ Hd, np.eye(n), atol=1e-12)
    # without act-order the reordering is the identity
    perm0, Hd0 = O.prepare_hessian(H, 0.05, False)
    np.testing.assert_array_equal(perm0, np.arange(n))
    np.testing.assert_allclose(Hd0, H + lam_mu * np.eye(n), rtol=0, atol=1e-15)


def test_damping_hand_value():
    H = np.array([[2.0, 1.0], [1.0, 4.0]])
    np.testing.assert_array_equal(O.damp(H, 0.5), [[3.5, 1.0], [1.0, 5.5]])


def test_chol_inv_worked_example():
    g = gold("chol_inv_2x2.json")
    R, info = O.chol_inv_upper(np.array(g["H"]))
    assert info == -1
    np.testing.assert_allclose(R, g["R"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(R, [[np.sqrt(3 / 8), -1 / np.sqrt(6)], [0, 1 / np.sqrt(3)]], rtol=1e-14)
    np.testing.assert_allclose(1.0 / np.diag(R) ** 2, g["schur_D"], rtol=1e-14)


def test_chol_inv_schur_diagonal_and_inverse():
    # 1/R_jj^2 is the Schur complement of the trailing block at j (the D of
    # H = U D U^T, U unit upper): the tr(D_X) terms of Table 9
    rng = np.random.default_rng(11)
    H = rand_spd(rng, 6, 100.0)
    R, info = O.chol_inv_upper(H)
    assert info == -1
    assert np.allclose(np.tril(R, -1), 0) and np.all(np.diag(R) > 0)
    np.testing.assert_allclose(R.T @ R @ H, np.eye(6), atol=1e-10)
    for j in range(6):
        a = H[j, j]
        if j + 1 < 6:
            b = H[j, j + 1:]
            C = H[j + 1:, j + 1:]
            a = a - b @ np.linalg.solve(C, b)
        assert 1.0 / R[j, j] ** 2 == pytest.approx(a, rel=1e-10)


def test_chol_inv_not_pd_reports_pivot():
    assert O.chol_inv_upper(np.array([[1.0, 2.0], [2.0, 1.0]]))[1] == 1
    assert O.chol_inv_upper(np.array([[-1.0, 0.0], [0.0, 1.0]]))[1] == 0
    assert O.chol_inv_upper(np.array([[1.0, 0.0, 0.0], [0.0, 1.0, 1.0], [0.0, 1.0, 1.0]]))[1] == 2


# ----------------------------------------------------------- quantizer


def test_quant_params_hand_values():
    s, z = O.quant_params(np.array([[-1.0, 0.0, 2.0]]), 2)
    assert (s[0], z[0]) == (1.0, 1.0)
    q, d, t = O.rtn(np.array([[-1.0, 0.0, 2.0]]), s, z, 2)
    np.testing.assert_array_equal(q, [[0, 1, 3]])
    np.testing.assert_array_equal(d, [[-1, 0, 2]])
    # all-positive group: the range is widened to include 0
    s, z = O.quant_params(np.array([[1.0, 2.0, 3.0]]), 2)
    assert (s[0], z[0]) == (1.0, 0.0)
    # degenerate range -> [-1, 1]; zero = round-half-even(1.5) = 2
    s, z = O.quant_params(np.array([[0.0, 0.0]]), 2)
    assert s[0] == pytest.approx(2 / 3) and z[0] == 2.0
    # round half to even on codes: t = 0.5 -> 0, 2.5 -> 2
    q, _, _ = O.rtn(np.array([[0.5, 2.5]]), np.array([1.0]), np.array([0.0]), 2)
    np.testing.assert_array_equal(q, [[0, 2]])
    # clamp to [0, 2^b - 1]
    q, _, _ = O.rtn(np.array([[-3.0, 9.0]]), np.array([1.0]), np.array([0.0]), 2)
    np.testing.assert_array_equal(q, [[0, 3]])


def test_zero_pre_round_hand_values():
    # -xmin / scale before rounding, the value whose distance to a half-integer
    # decides whether two zero points may differ by a rounding tie
    cases = [
        (np.array([[-1.0, 0.0, 2.0]]), 2, 1.0),          # scale 1, -min 1
        (np.array([[-0.3, 1.0]]), 2, 0.3 / (1.3 / 3)),    # 0.6923..., not a half-integer
        (np.array([[-0.5, 0.5]]), 1, 0.5),                # an exact tie
        (np.array([[1.0, 2.0, 3.0]]), 2, 0.0),            # range widened to 0
        (np.array([[0.0, 0.0]]), 2, 1.5),                 # degenerate -> [-1, 1], scale 2/3
        (np.array([[-2.0, -1.0]]), 3, 7.0),               # all negative: max widened to 0
    ]
    for V, bits, want in cases:
        assert O.zero_pre_round(V, bits)[0] == pytest.approx(want, rel=1e-15, abs=1e-15)


def test_zero_pre_round_is_zero_before_rint():
    # equals -min(0, min v) / scale with quant_params' scale, and rounds
    # half-to-even to quant_params' zero point
    rng = np.random.default_rng(22)
    for bits in (1, 2, 3, 4, 8):
        V = rng.standard_normal((50, 7)) + rng.uniform(-1, 1, (50, 1))
        zt = O.zero_pre_round(V, bits)
        scale, zero = O.quant_params(V, bits)
        np.testing.assert_allclose(zt, -np.minimum(V.min(axis=1), 0.0) / scale, rtol=1e-15)
        np.testing.assert_array_equal(np.rint(zt), zero)
        assert np.all((zt >= 0) & (zt <= (2 ** bits - 1) * (1 + 1e-12)))


# --------------------------------------------------------- GPTQ loop


def test_gptq_hand_worked_obs():
    g = gold("obs_1x2.json")
    R, _ = O.chol_inv_upper(np.array(g["H"]))
    out = O.gptq(np.array(g["W"]), R, [0, 1], g["bits"], -1)
    np.testing.assert_array_equal(out["codes"], g["codes"])
    np.testing.assert_allclose(out["What"], g["What"], atol=1e-15)
    np.testing.assert_allclose(out["pre"], g["pre_round"], rtol=1e-14)


@pytest.mark.parametrize("group", [-1, 4])
def test_gptq_identity_hessian_is_rtn(group):
    rng = np.random.default_rng(12)
    W = rng.standard_normal((6, 8))
    out = O.gptq(W, np.eye(8), np.arange(8), 3, group)
    if group <= 0:
        s, z = O.quant_params(W, 3)
        q, d, _ = O.rtn(W, s, z, 3)
    else:
        qs, ds = [], []
        for c in range(0, 8, group):
            s, z = O.quant_params(W[:, c:c + group], 3)
            q_, d_, _ = O.rtn(W[:, c:c + group], s, z, 3)
            qs.append(q_); ds.append(d_)
        q, d = np.hstack(qs), np.hstack(ds)
    np.testing.assert_array_equal(out["codes"], q)
    np.testing.assert_allclose(out["What"], d, atol=1e-15)


def test_gptq_ties_round_half_even_and_natural_order_outputs():
    # R = I: no compensation, so the loop is RTN.  t = 2.5 must round to 2
    # (half to even); with a processing order that is not an involution the
    # returned codes must still be in natural column order
    W = np.array([[-1.0, 2.0, 1.5, 0.25], [0.3, -0.6, 0.9, 0.0]])
    perm = np.array([2, 0, 3, 1])
    out = O.gptq(W, np.eye(4), perm, 2, -1)
    s, z = O.quant_params(W, 2)
    q, d, t = O.rtn(W, s, z, 2)
    assert t[0, 2] == 2.5 and q[0, 2] == 2
    np.testing.assert_array_equal(out["codes"], q)
    np.testing.assert_allclose(out["What"], d, atol=1e-15)
    np.testing.assert_allclose(out["pre"], t, atol=1e-15)


def _obs_full_kronecker(W, HX, HG, bits):
    """Sequential OBS with the explicit (mn x mn) Hessian H_X (x) H_G: each step
    fixes the m entries of one column jointly and moves the still-free
    coordinates by -Hinv[:, S] Hinv[S, S]^-1 (w_S - q_S); the inverse over the
    free set is refreshed by a Schur complement.  Per-channel grid."""
    m, n = W.shape
    maxq = 2 ** bits - 1
    scale, zero = O.quant_params(W, bits)
    w = W.reshape(-1, order="F").copy()          # vec, column stacking
    Hinv = np.linalg.inv(np.kron(HX, HG))
    free = list(range(m * n))
    codes = np.zeros((m, n))
    for j in range(n):
        S = [j * m + i for i in range(m)]
        q = np.clip(np.rint(w[S] / scale + zero), 0, maxq)
        codes[:, j] = q
        wq = scale * (q - zero)
        pos = [free.index(s) for s in S]
        A = Hinv[:, pos]
        delta = -A @ np.linalg.solve(Hinv[np.ix_(pos, pos)], w[S] - wq)
        w[free] += delta
        w[S] = wq
        keep = [p for p in range(len(free)) if p not in pos]
        Hinv = Hinv[np.ix_(keep, keep)] - Hinv[np.ix_(keep, pos)] @ np.linalg.solve(
            Hinv[np.ix_(pos, pos)], Hinv[np.ix_(pos, keep)])
        free = [free[p] for p in keep]
    return codes, w.reshape((m, n), order="F")


@pytest.mark.parametrize("seed", [13, 14, 15])
def test_hg_cancels_proposition1_brute_force(seed):
    # Proposition 1: with the full Kronecker Hessian the column update does not
    # depend on H_G, so the H_X-only loop gives the same codes and weights
    rng = np.random.default_rng(seed)
    m, n, bits = 3, 5, 2
    W = rng.standard_normal((m, n))
    HX = rand_spd(rng, n, 30.0)
    HG = rand_spd(rng, m, 1e3)
    codes_k, w_k = _obs_full_kronecker(W, HX, HG, bits)
    R, _ = O.chol_inv_upper(HX)
    out = O.gptq(W, R, np.arange(n), bits, -1)
    np.testing.assert_array_equal(out["codes"], codes_k)
    np.testing.assert_allclose(out["What"], w_k, atol=1e-12)


def test_gptq_ldl_identity_and_bound():
    # Delta W = E R (processing order), hence for any H_G:
    # tr(H_G dW H dW^T) = sum_j e_j^T H_G e_j  (H = (R^T R)^-1); with no clamp
    # the H_G = I loss is at most 1/4 sum_j sum_r scale_r^2 / R_jj^2 (Table 9's
    # GPTQ-LDLQ form with tr(D))
    rng = np.random.default_rng(16)
    m, n, bits = 5, 16, 4
    W = rng.standard_normal((m, n)) * 0.1
    H = O.damp(O.gram(rng.standard_normal((64, n)) * rng.uniform(0.2, 3.0, n)), 0.01)
    perm = O.act_order_perm(H)
    Hp = H[np.ix_(perm, perm)]
    R, _ = O.chol_inv_upper(Hp)
    out = O.gptq(W, R, perm, bits, -1)
    dW = (W - out["What"])[:, perm]
    np.testing.assert_allclose(dW, out["E"] @ R, atol=1e-12)
    HG = rand_spd(rng, m, 100.0)
    lhs = O.proxy_loss(dW, Hp, HG)
    rhs = float(np.sum(out["E"] * (HG @ out["E"])))
    assert lhs == pytest.approx(rhs, rel=1e-9)
    pre = out["pre"]
    if np.all((pre >= -0.5) & (pre <= 2 ** bits - 0.5)):
        bound = 0.25 * np.sum(out["scales"][:, 0] ** 2) * np.sum(1.0 / np.diag(R) ** 2)
        assert O.proxy_loss(dW, Hp, np.eye(m)) <= bound * (1 + 1e-12)


def test_gptq_exhaustive_2x4_two_bits():
    # exhaustive search over all 4^8 grid codes bounds the compensated loss
    rng = np.random.default_rng(17)
    m, n, bits = 2, 4, 2
    W = rng.standard_normal((m, n))
    HX = O.damp(rand_spd(rng, n, 20.0), 0.01)
    HG = rand_spd(rng, m, 10.0)
    R, _ = O.chol_inv_upper(HX)
    out = O.gptq(W, R, np.arange(n), bits, -1)
    scale, zero = O.quant_params(W, bits)
    best = np.inf
    for cs in itertools.product(range(4), repeat=m * n):
        q = np.array(cs, dtype=float).reshape(m, n)
        best = min(best, O.proxy_loss(W - scale[:, None] * (q - zero[:, None]), HX, HG))
    loss_gptq = O.proxy_loss(W - out["What"], HX, HG)
    _, d_rtn, _ = O.rtn(W, scale, zero, bits)
    assert best <= loss_gptq + 1e-12
    assert best <= O.proxy_loss(W - d_rtn, HX, HG) + 1e-12
    # the codes GPTQ returns are on the grid
    np.testing.assert_allclose(out["What"], scale[:, None] * (out["codes"] - zero[:, None]), atol=1e-15)


def test_gptq_group_params_from_compensated_values():
    # Group parameters are taken when the group's first column is reached, from
    # the values as compensated so far.  One row, 1 bit, group 2, R = I except
    # R[0, 2] = 0.5; by hand: group 0 [0.3, 1.0] -> scale 1, zero 0; column 0
    # rounds to 0 with error e = 0.3, moving w2 by -0.15 to 0.25; group 1 is then
    # [0.25, 0.2] -> scale 0.25 (the uncompensated values would give 0.4);
    # column 3: t = 0.8 -> code 1.
    W = np.array([[0.3, 1.0, 0.4, 0.2]])
    R = np.eye(4)
    R[0, 2] = 0.5
    out = O.gptq(W, R, np.arange(4), 1, 2)
    np.testing.assert_array_equal(out["codes"], [[0, 1, 1, 1]])
    np.testing.assert_allclose(out["scales"], [[1.0, 0.25]], rtol=1e-15)
    np.testing.assert_allclose(out["zeros"], [[0.0, 0.0]])
    np.testing.assert_allclose(out["What"], [[0.0, 1.0, 0.25, 0.25]], rtol=1e-15)
    np.testing.assert_allclose(out["pre"][0, 3], 0.8, rtol=1e-14)


# -------------------------------------------------- sensitivity, bits


def test_sensitivity_trace_of_kronecker():
    rng = np.random.default_rng(18)
    HX, HG = rand_spd(rng, 5), rand_spd(rng, 3)
    trx, trg, s = O.sensitivity(HX, HG)
    assert s == pytest.approx(np.trace(np.kron(HX, HG)), rel=1e-13)
    assert trx == pytest.approx(np.trace(HX), rel=1e-15)


def test_allocation_worked_example():
    g = gold("allocation_llama3_8b_block.json")
    bits = O.allocate_bits(g["scores"], g["n_params"], g["bmin"], g["bmax"], g["budget_bits"])
    assert bits == g["bits"]
    n = np.array(g["n_params"])
    assert int(np.sum(n * np.array(bits))) == g["budget_bits"]


def test_allocation_invariants():
    rng = np.random.default_rng(19)
    for _ in range(50):
        L = int(rng.integers(1, 9))
        n = rng.integers(1, 1000, size=L)
        sc = rng.random(L)
        budget = int(rng.integers(2 * n.sum(), 4 * n.sum() + 1))
        b = np.array(O.allocate_bits(sc, n, 2, 4, budget))
        assert np.all((b >= 2) & (b <= 4))
        assert int(np.sum(b * n)) <= budget
        # maximality: no single +1 still fits
        used = int(np.sum(b * n))
        for i in range(L):
            assert b[i] == 4 or used + n[i] > budget
        # the most sensitive sublayer is raised as far as the budget allows
        top = int(np.argmax(sc))
        assert b[top] == min(4, 2 + (budget - 2 * int(n.sum())) // int(n[top]))
    with pytest.raises(ValueError):
        O.allocate_bits([1.0, 2.0], [10, 10], 2, 4, 39)


# ---------------------------------------------------------------- deploy codec


def test_pack_hand_values():
    # 2-bit: codes 1, 2, 3, 0 -> 0b00_11_10_01; 4-bit: 0xA, 0x3 -> 0x3A; a
    # 5-column 2-bit row takes two bytes, the second holding code 4 alone
    assert O.pack_codes(np.array([[1, 2, 3, 0]]), 2).tolist() == [[0x39]]
    assert O.pack_codes(np.array([[0xA, 0x3]]), 4).tolist() == [[0x3A]]
    assert O.pack_codes(np.array([[0, 0, 0, 0, 3]]), 2).tolist() == [[0, 3]]
    np.testing.assert_array_equal(O.unpack_codes(np.array([[0x39]], dtype=np.uint8), 2, 4), [[1, 2, 3, 0]])


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_roundtrip_brute_force(bits):
    rng = np.random.default_rng(bits)
    q = rng.integers(0, 2 ** bits, (5, 37))
    p = O.pack_codes(q, bits)
    assert p.shape == (5, (37 * bits + 7) // 8)
    np.testing.assert_array_equal(O.unpack_codes(p, bits, 37), q)
    # every byte value decodes to the codes whose bits it holds
    for b in range(256):
        got = O.unpack_codes(np.array([[b]], dtype=np.uint8), bits, 8 // bits)[0]
        assert sum(int(c) << (bits * i) for i, c in enumerate(got)) == b


@pytest.mark.parametrize("seed,ki,ko", [(3, 4, 8), (4, 2, 2), (5, 1, 1)])
def test_unrotate_inverts_biip_and_matches_explicit(seed, ki, ko):
    W, HX, HG, si, _, so, _, a = _biip_case(seed, ki=ki, ko=ko)
    Wp, _, _, s = O.biip(W, HX, HG, si, ki, so, ko, a)
    np.testing.assert_allclose(O.unrotate(Wp, si, ki, so, ko, s), W, atol=1e-12)
    U = O.rotation_matrix(W.shape[0], ko, so)
    V = O.rotation_matrix(W.shape[1], ki, si)
    M = np.random.default_rng(seed + 100).standard_normal(W.shape)
    np.testing.assert_allclose(O.unrotate(M, si, ki, so, ko, s), np.diag(1 / s) @ U.T @ M @ V,
                               atol=1e-12)


@pytest.mark.parametrize("group,act", [(0, False), (0, True), (4, False), (4, True)])
def test_dequant_reproduces_column_loop_outputs(group, act):
    rng = np.random.default_rng(11)
    m, n = 6, 12
    W = rng.standard_normal((m, n))
    H = rand_spd(rng, n, 30.0)
    perm, Hd = O.prepare_hessian(H, 0.01, act)
    R, _ = O.chol_inv_upper(Hd)
    out = O.gptq(W, R, perm, 3, group)
    Wq = O.dequant(out["codes"], out["scales"], out["zeros"], group, perm)
    np.testing.assert_array_equal(Wq, out["What"])


def test_decode_matvec_equals_dense_product():
    rng = np.random.default_rng(21)
    m, n, ki, ko, g = 16, 24, 8, 4, 8
    q = rng.integers(0, 4, (m, n))
    scales = rng.uniform(0.5, 2.0, (m, n // g))
    zeros = rng.integers(0, 4, (m, n // g)).astype(np.float64)
    si, so = rng.choice([-1.0, 1.0], n), rng.choice([-1.0, 1.0], m)
    s = rng.uniform(0.5, 2.0, m)
    x = rng.standard_normal(n)
    y = O.decode_matvec(O.pack_codes(q, 2), 2, n, scales, zeros, g, si, ki, so, ko, s, x)
    U = O.rotation_matrix(m, ko, so)
    V = O.rotation_matrix(n, ki, si)
    Wd = np.zeros((m, n))
    for i in range(m):
        for c in range(n):
            Wd[i, c] = scales[i, c // g] * (q[i, c] - zeros[i, c // g])
    np.testing.assert_allclose(y, np.diag(1 / s) @ U.T @ Wd @ V @ x, atol=1e-11)
    # one code per byte (3-bit weights) takes the codes as they are
    y8 = O.decode_matvec(q, 8, n, scales, zeros, g, si, ki, so, ko, s, x)
    np.testing.assert_allclose(y8, y, atol=1e-12)


def test_decode_recovers_the_quantized_layer():
    # end to end: BiIP, the column loop and the decode give back W x up to
    # the quantization error, and exactly the un-rotated dequantized weight
    rng = np.random.default_rng(5)
    m, n, N = 8, 16, 64
    W = rng.standard_normal((m, n)) * 0.02
    X, G = rng.standard_normal((N, n)), rng.standard_normal((N, m))
    si, so = rng.choice([-1.0, 1.0], n), rng.choice([-1.0, 1.0], m)
    out = O.quantize_sublayer(W, X, G, si, 8, so, 4, 0.25, 0.01, 4, 8, False)
    x = rng.standard_normal(n)
    y = O.decode_matvec(O.pack_codes(out["codes"], 4), 4, n, out["scales"], out["zeros"], 8,
                        si, 8, so, 4, out["sg"], x, out["perm"])
    Wback = O.unrotate(out["What"], si, 8, so, 4, out["sg"])
    np.testing.assert_allclose(y, Wback @ x, atol=1e-12)
    assert np.linalg.norm(Wback - W) < 0.2 * np.linalg.norm(W)


# ---------------------------------------------------------------- allocation variants


def test_passwise_closed_forms():
    # equal sizes: after whole passes every sublayer has the same width, whatever the scores
    sc = [0.3, 5.0, 1.0, 2.0]
    n = [7, 7, 7, 7]
    assert O.allocate_bits_passwise(sc, n, 2, 4, 3 * 28) == [3, 3, 3, 3]
    assert O.allocate_bits_passwise(sc, n, 2, 4, 4 * 28) == [4, 4, 4, 4]   # needs a second pass
    # one bit short of the second pass: the two most sensitive get their 4th bit... only one fits
    assert O.allocate_bits_passwise(sc, n, 2, 4, 3 * 28 + 7) == [3, 4, 3, 3]


def test_passwise_hand_example():
    # scores (3, 1, 2), sizes (10, 10, 20), budget 2*40 + 35: pass one raises 0 (90) and 2 (110);
    # sublayer 1 no longer fits (120), and neither does anything in pass two
    assert O.allocate_bits_passwise([3, 1, 2], [10, 10, 20], 2, 4, 115) == [3, 2, 3]
    # the greedy rule raises the top sublayer to the cap first
    assert O.allocate_bits([3, 1, 2], [10, 10, 20], 2, 4, 115) == [4, 3, 2]


def _loss(scores, bits):
    # expected loss up to a constant: sum_i s_i eps(b_i)^2 with eps(b) = 2^-b
    return sum(float(s) * 4.0 ** (-b) for s, b in zip(scores, bits))


def test_marginal_hand_example_and_ties():
    # gains per bit at 2 bits: 4/16 vs 1/16 -> sublayer 0; at 3 bits 4/64 = 1/16 ties
    # with sublayer 1 at 2 bits -> the lower index, sublayer 0, again
    assert O.allocate_bits_marginal([4, 1], [1, 1], 2, 4, 6) == [4, 2]
    assert O.allocate_bits_marginal([4, 1], [1, 1], 2, 4, 7) == [4, 3]
    # cost matters: s 4^-b / n equal for (1, n=1) and (4, n=4) -> lower index first;
    # then sublayer 1 (4/16/4) beats sublayer 0 at 3 bits (1/64) when it fits ...
    assert O.allocate_bits_marginal([1, 4], [1, 4], 2, 4, 2 * 5 + 1) == [3, 2]
    assert O.allocate_bits_marginal([1, 4], [1, 4], 2, 4, 2 * 5 + 5) == [3, 3]
    # ... and the smaller upgrade is taken when the better one no longer fits
    assert O.allocate_bits_marginal([1, 4], [1, 4], 2, 4, 2 * 5 + 4) == [4, 2]


def test_marginal_is_optimal_by_brute_force():
    # with equal costs and diminishing returns the greedy choice is optimal:
    # no allocation within the budget has a lower expected loss
    import itertools
    rng = np.random.default_rng(29)
    for _ in range(40):
        L = int(rng.integers(1, 5))
        sc = list(rng.random(L) * 10 ** rng.uniform(-2, 2, L))
        n = [3] * L
        budget = int(rng.integers(2 * 3 * L, 4 * 3 * L + 1))
        got = O.allocate_bits_marginal(sc, n, 2, 4, budget)
        assert sum(b * 3 for b in got) <= budget
        best = min(_loss(sc, c) for c in itertools.product(range(2, 5), repeat=L)
                   if sum(b * 3 for b in c) <= budget)
        assert _loss(sc, got) <= best * (1 + 1e-12)


def test_types_hand_example():
    # two layers x three types; type sums: t0 = 1 + 1 = 2, t1 = 5 + 0 = 5, t2 = 2 + 2.5 = 4.5.
    # Ranked by sum: t1, t2, t0 (by the largest single score: t1, t2, t0 too, but
    # t2 beats t1 by max of its layer-2 score below)
    sc = [1.0, 5.0, 2.0, 1.0, 0.0, 2.5]
    ty = [0, 1, 2, 0, 1, 2]
    assert O.allocate_types(sc, ty, 3, 2, 1) == [2, 3, 2, 2, 3, 2]
    assert O.allocate_types(sc, ty, 3, 2, 2) == [2, 3, 3, 2, 3, 3]
    assert O.allocate_types(sc, ty, 3, 2, 0) == [2] * 6
    assert O.allocate_types(sc, ty, 3, 2, 3) == [3] * 6
    # summing, not the largest member: t1 = 3 + 3 = 6 beats t0 = 5 + 0 = 5
    assert O.allocate_types([5.0, 3.0, 0.0, 3.0], [0, 1, 0, 1], 2, 2, 1) == [2, 3, 2, 3]
    # ties between types go to the lower type id
    assert O.allocate_types([1.0, 1.0], [1, 0], 2, 3, 1) == [3, 4]


def test_types_one_sublayer_per_type_is_score_order():
    rng = np.random.default_rng(31)
    sc = list(rng.random(7))
    for N in range(8):
        bits = O.allocate_types(sc, list(range(7)), 7, 2, N)
        top = set(sorted(range(7), key=lambda i: -sc[i])[:N])
        assert bits == [3 if i in top else 2 for i in range(7)]


# ---------------------------------------------------------------- BiIP variants and diagnostics


def _cv_by_definition(v):
    k = len(v)
    mu = sum(v) / k
    return math.sqrt(sum((x - mu) ** 2 for x in v) / k) / mu


def test_weight_cv_by_definition_and_closed_forms():
    rng = np.random.default_rng(53)
    W = rng.standard_normal((5, 7)) * rng.uniform(0.1, 3, 7)
    cols = [math.sqrt(sum(W[i, j] ** 2 for i in range(5))) for j in range(7)]
    rows = [math.sqrt(sum(W[i, j] ** 2 for j in range(7))) for i in range(5)]
    cin, cout = O.weight_cv(W)
    assert abs(cin - _cv_by_definition(cols)) <= 1e-12
    assert abs(cout - _cv_by_definition(rows)) <= 1e-12
    # equal column norms -> CV_in = 0; two column norms a, b, half each -> |a - b| / (a + b)
    H = O.hadamard_matrix(8)
    assert abs(O.weight_cv(H)[0]) <= 1e-15 and abs(O.weight_cv(H)[1]) <= 1e-15
    A = np.ones((4, 6))
    A[:, :3] *= 3.0
    assert abs(O.weight_cv(A)[0] - (3 - 1) / (3 + 1)) <= 1e-15
    # scale invariance
    np.testing.assert_allclose(O.weight_cv(7.5 * W), O.weight_cv(W), rtol=1e-13)


def test_weight_cv_rotation_invariances():
    # an input-side rotation keeps every row norm (CV_out exactly), an
    # output-side rotation every column norm (CV_in exactly)
    rng = np.random.default_rng(59)
    W = rng.standard_normal((16, 32)) * rng.uniform(0.1, 5, 32)[None, :] * rng.uniform(0.1, 5, 16)[:, None]
    V = O.rotation_matrix(32, 8, rng.choice([-1.0, 1.0], 32))
    U = O.rotation_matrix(16, 16, rng.choice([-1.0, 1.0], 16))
    cin, cout = O.weight_cv(W)
    assert abs(O.weight_cv(W @ V.T)[1] - cout) <= 1e-12
    assert abs(O.weight_cv(U @ W)[0] - cin) <= 1e-12
    # and the rotations do change the other one on this matrix
    assert abs(O.weight_cv(W @ V.T)[0] - cin) > 1e-3
    assert abs(O.weight_cv(U @ W)[1] - cout) > 1e-3


def test_biip_modes_against_explicit_matrices():
    rng = np.random.default_rng(61)
    m, n, ko, ki, alpha = 8, 12, 4, 4, 0.25
    W = rng.standard_normal((m, n))
    A = rng.standard_normal((3 * n, n))
    B = rng.standard_normal((3 * m, m)) * rng.uniform(0.1, 4, m)
    HX, HG = A.T @ A, B.T @ B
    si, so = rng.choice([-1.0, 1.0], n), rng.choice([-1.0, 1.0], m)
    U = O.rotation_matrix(m, ko, so)
    V = O.rotation_matrix(n, ki, si)
    S = np.diag(np.diag(HG) ** alpha)
    Si = np.linalg.inv(S)
    want = {
        "full": (U @ S @ W @ V.T, V @ HX @ V.T, U @ Si @ HG @ Si @ U.T),
        "no_rescale": (U @ W @ V.T, V @ HX @ V.T, U @ HG @ U.T),
        "su_only": (U @ S @ W, HX, U @ Si @ HG @ Si @ U.T),
        "sv_only": (W @ V.T, V @ HX @ V.T, HG),
    }
    for mode in O.INCOH_MODES:
        Wp, HXp, HGp, s = O.biip_mode(W, HX, HG, si, ki, so, ko, alpha, mode)
        for got, exp in zip((Wp, HXp, HGp), want[mode]):
            np.testing.assert_allclose(got, exp, rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        O.biip_mode(W, HX, HG, si, ki, so, ko, alpha, "both")


# ------------------------------------------------ GPTAQ asymmetric correction


def test_drift_cross_brute_force_and_closed_forms():
    rng = np.random.default_rng(31)
    N, n = 40, 6
    X = rng.integers(-3, 4, (N, n)).astype(float)
    Xfp = X + rng.integers(-1, 2, (N, n)).astype(float)
    C = O.drift_cross(X, Xfp)
    ref = np.zeros((n, n))
    for i in range(n):
        for k in range(n):
            ref[i, k] = sum((Xfp[t, i] - X[t, i]) * X[t, k] for t in range(N)) / N
    np.testing.assert_allclose(C, ref, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(O.drift_cross(X, X), np.zeros((n, n)))
    np.testing.assert_allclose(O.drift_cross(X, 2 * X), O.gram(X), rtol=1e-15, atol=1e-15)


def test_gptaq_correction_structure():
    # P = alpha ((C R^T) (.) M) R, M strictly upper: P_jk = alpha sum_{j<i<=k}
    # (C R^T)_ji R_ik, zero on and below the diagonal
    rng = np.random.default_rng(32)
    n = 6
    C = rng.standard_normal((n, n))
    R, _ = O.chol_inv_upper(rand_spd(rng, n, 30.0))
    P = O.gptaq_correction(C, R, 0.7)
    K = C @ R.T
    ref = np.zeros((n, n))
    for j in range(n):
        for k in range(n):
            ref[j, k] = 0.7 * sum(K[j, i] * R[i, k] for i in range(j + 1, k + 1))
    np.testing.assert_allclose(P, ref, rtol=1e-13, atol=1e-14)
    assert not np.any(np.tril(P))


def _asym_sequential_obs(W, Hd, HG, C, alpha, bits, group):
    """Sequential OBS on the explicit Kronecker asymmetric objective
    vec(dW)^T (Hd (x) HG) vec(dW) + 2 alpha <dW, HG W_<k C>, where W_<k keeps
    the full-precision columns before k (the drift committed so far): at each
    column k (and at each group start, for the group's grid) the free columns
    take the optimum of that objective given the quantized earlier columns;
    column k is then rounded on its grid.  Returns codes and the pre-round
    values (m x n, natural order = processing order here)."""
    m, n = W.shape
    A = np.kron(Hd, HG)                      # vec index = column * m + row
    maxq = 2 ** bits - 1
    Q = np.zeros((m, n))
    codes = np.zeros((m, n))
    pre = np.zeros((m, n))
    if group <= 0:
        scale, zero = O.quant_params(W, bits)

    def cond_opt(k):
        # optimum of the free columns >= k given columns < k fixed at Q
        dW = np.zeros((m, n))
        dW[:, :k] = W[:, :k] - Q[:, :k]
        Wk = np.zeros((m, n))
        Wk[:, :k] = W[:, :k]
        g = alpha * (HG @ Wk @ C)
        S = [c * m + r for c in range(k) for r in range(m)]
        F = [c * m + r for c in range(k, n) for r in range(m)]
        x = dW.reshape(-1, order="F")
        gv = g.reshape(-1, order="F")
        rhs = -(A[np.ix_(F, S)] @ x[S] if S else 0) - gv[F]
        x[F] = np.linalg.solve(A[np.ix_(F, F)], rhs)
        return W - x.reshape((m, n), order="F")

    for k in range(n):
        Wc = cond_opt(k)
        if group > 0 and k % group == 0:
            scale, zero = O.quant_params(Wc[:, k:k + group], bits)
        t = Wc[:, k] / scale + zero
        q = np.clip(np.rint(t), 0, maxq)
        Q[:, k] = scale * (q - zero)
        codes[:, k], pre[:, k] = q, t
    return codes, pre


@pytest.mark.parametrize("seed,group,act", [(33, -1, False), (34, -1, True), (35, 2, False),
                                            (36, 3, True)])
def test_gptaq_loop_is_sequential_obs_of_the_asymmetric_objective(seed, group, act):
    # the reading of the cut-off column update, pinned by brute force: the loop
    # with P equals the sequential optimum of the explicit Kronecker objective
    # with the drift term (H_G still cancels); groups take their grid from
    # those optima at the group's first column
    rng = np.random.default_rng(seed)
    m, N, n, bits, alpha = 3, 64, 6, 2, 0.6
    X = rng.standard_normal((N, n)) * rng.uniform(0.3, 2.0, n)
    Xfp = X + 0.3 * rng.standard_normal((N, n))
    W = rng.standard_normal((m, n))
    HG = rand_spd(rng, m, 1e3)
    perm, Hd = O.prepare_hessian(O.gram(X), 0.01, act)
    C = O.drift_cross(X, Xfp)[np.ix_(perm, perm)]
    R, _ = O.chol_inv_upper(Hd)
    out = O.gptaq(W, R, perm, bits, group, O.gptaq_correction(C, R, alpha))
    codes_b, pre_b = _asym_sequential_obs(W[:, perm], Hd, HG, C, alpha, bits, group)
    np.testing.assert_array_equal(out["codes"][:, perm], codes_b)
    np.testing.assert_allclose(out["pre"][:, perm], pre_b, rtol=1e-9, atol=1e-9)
    # the drift term matters here: the plain loop decides differently
    plain = O.gptq(W, R, perm, bits, group)
    assert np.max(np.abs(plain["pre"] - out["pre"])) > 1e-3


def test_gptaq_without_drift_is_gptq():
    rng = np.random.default_rng(37)
    m, n = 5, 12
    W = rng.standard_normal((m, n))
    X = rng.standard_normal((50, n))
    perm, Hd = O.prepare_hessian(O.gram(X), 0.01, True)
    R, _ = O.chol_inv_upper(Hd)
    for P in (O.gptaq_correction(O.drift_cross(X, X)[np.ix_(perm, perm)], R, 0.5),
              O.gptaq_correction(rng.standard_normal((n, n)), R, 0.0)):
        a = O.gptaq(W, R, perm, 3, 4, P)
        b = O.gptq(W, R, perm, 3, 4)
        for k in ("codes", "What", "pre", "E", "scales", "zeros"):
            np.testing.assert_array_equal(a[k], b[k])


def test_drift_term_rotation_invariance():
    # Theorem 1's transformed drift matrix (dXX^T)' = V dXX^T V^T keeps the
    # objective's drift term tr(H_G dW C^T W^T) under W' = U S W V^T,
    # H_G' = U S^-1 H_G S^-1 U^T (and dW' = U S dW V^T)
    rng = np.random.default_rng(38)
    m, n, N = 8, 16, 40
    W = rng.standard_normal((m, n))
    dW = 0.1 * rng.standard_normal((m, n))
    X = rng.standard_normal((N, n))
    C = O.drift_cross(X, X + 0.2 * rng.standard_normal((N, n)))
    HG = O.gram(rng.standard_normal((N, m)) * rng.uniform(0.2, 3.0, m))
    si, so = np.sign(rng.standard_normal(n)), np.sign(rng.standard_normal(m))
    V = O.rotation_matrix(n, 8, si)
    U = O.rotation_matrix(m, 4, so)
    s = O.output_rescale(HG, 0.25)
    S = np.diag(s)
    Wp, dWp = U @ S @ W @ V.T, U @ S @ dW @ V.T
    HGp = U @ np.linalg.inv(S) @ HG @ np.linalg.inv(S) @ U.T
    Cp = V @ C @ V.T
    lhs = np.trace(HGp @ dWp @ Cp.T @ Wp.T)
    rhs = np.trace(HG @ dW @ C.T @ W.T)
    assert lhs == pytest.approx(rhs, rel=1e-10)


# ------------------------------------------------ input-side rescale S_X


def _sx_case(seed, m=8, n=16, ki=8, ko=4):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((m, n))
    d = np.exp(rng.standard_normal(n))          # input channels of very different scales
    HX = rand_spd(rng, n, 20.0) * d[:, None] * d[None, :]
    HG = rand_spd(rng, m, 1e3)
    si, so = rng.choice([-1.0, 1.0], n), rng.choice([-1.0, 1.0], m)
    return W, HX, HG, si, ki, so, ko


def test_input_rescale_hand_values():
    HX = np.diag([4.0, 0.0, 9.0, -1.0])
    np.testing.assert_allclose(O.input_rescale(HX, 0.5), [2.0, 1.0, 3.0, 1.0])
    np.testing.assert_allclose(O.input_rescale(np.diag([16.0, 81.0]), 0.25), [2.0, 3.0])
    np.testing.assert_array_equal(O.input_rescale(np.diag([16.0, 81.0]), 0.0), [1.0, 1.0])


def test_biip_sx_explicit_matrices():
    W, HX, HG, si, ki, so, ko = _sx_case(40)
    Wp, HXp, HGp, sg, sx = O.biip_sx(W, HX, HG, si, ki, so, ko, 0.25, 0.25)
    U = O.rotation_matrix(W.shape[0], ko, so)
    V = O.rotation_matrix(W.shape[1], ki, si)
    SG = np.diag(np.diag(HG) ** 0.25)
    SX = np.diag(np.diag(HX) ** 0.25)
    np.testing.assert_allclose(Wp, U @ SG @ W @ SX @ V.T, atol=1e-12)
    np.testing.assert_allclose(HXp, V @ np.linalg.inv(SX) @ HX @ np.linalg.inv(SX) @ V.T, atol=1e-10)
    np.testing.assert_allclose(HGp, U @ np.linalg.inv(SG) @ HG @ np.linalg.inv(SG) @ U.T, atol=1e-10)
    np.testing.assert_allclose(sx, np.diag(SX), rtol=1e-15)


@pytest.mark.parametrize("ax", [0.25, 0.5, -0.3])
def test_biip_sx_objective_invariance(ax):
    # Theorem 1's invariance of tr(H_G dW H_X dW^T), with both rescales
    W, HX, HG, si, ki, so, ko = _sx_case(41)
    dW = np.random.default_rng(42).standard_normal(W.shape)
    _, HXp, HGp, sg, sx = O.biip_sx(W, HX, HG, si, ki, so, ko, 0.25, ax)
    dWp, _, _, _, _ = O.biip_sx(dW, None, HG, si, ki, so, ko, 0.25, ax, sx=sx)
    assert O.proxy_loss(dWp, HXp, HGp) == pytest.approx(O.proxy_loss(dW, HX, HG), rel=1e-11)


def test_biip_sx_trace_closed_forms():
    W, HX, HG, si, ki, so, ko = _sx_case(43)
    for ax in (0.25, 0.5):
        _, HXp, _, _, _ = O.biip_sx(W, HX, HG, si, ki, so, ko, 0.25, ax)
        assert np.trace(HXp) == pytest.approx(np.sum(np.diag(HX) ** (1 - 2 * ax)), rel=1e-13)
    # alpha_x = 1/2 and no rotation: H_X' is the correlation matrix (unit diagonal)
    n = W.shape[1]
    _, HXc, _, _, sx = O.biip_sx(W, HX, HG, np.ones(n), 1, so, ko, 0.25, 0.5)
    np.testing.assert_allclose(np.diag(HXc), np.ones(n), rtol=1e-14)
    np.testing.assert_allclose(HXc, HX / np.sqrt(np.outer(np.diag(HX), np.diag(HX))), rtol=1e-13)
    # the rescale comes from H_X before its rotation: W's columns grow by diag(H_X)^1/2
    Wc, _, _, _, _ = O.biip_sx(W, HX, None, np.ones(n), 1, np.ones(W.shape[0]), 1, 0.0, 0.5)
    np.testing.assert_allclose(Wc, W * np.sqrt(np.diag(HX))[None, :], rtol=1e-14)


def test_biip_sx_alpha_zero_is_biip():
    W, HX, HG, si, ki, so, ko = _sx_case(44)
    a = O.biip(W, HX, HG, si, ki, so, ko, 0.25)
    b = O.biip_sx(W, HX, HG, si, ki, so, ko, 0.25, 0.0)
    for x, y in zip(a, b[:4]):
        np.testing.assert_allclose(x, y, rtol=0, atol=0)
    np.testing.assert_array_equal(b[4], np.ones(W.shape[1]))


@pytest.mark.parametrize("seed,ki,ko", [(45, 8, 4), (46, 1, 1), (47, 16, 8)])
def test_unrotate_sx_inverts_biip_sx(seed, ki, ko):
    W, HX, HG, si, _, so, _ = _sx_case(seed, ki=ki, ko=ko)
    Wp, _, _, sg, sx = O.biip_sx(W, HX, HG, si, ki, so, ko, 0.25, 0.25)
    np.testing.assert_allclose(O.unrotate_sx(Wp, si, ki, so, ko, sg, sx), W, atol=1e-12)
    U = O.rotation_matrix(W.shape[0], ko, so)
    V = O.rotation_matrix(W.shape[1], ki, si)
    M = np.random.default_rng(seed).standard_normal(W.shape)
    np.testing.assert_allclose(O.unrotate_sx(M, si, ki, so, ko, sg, sx),
                               np.diag(1 / sg) @ U.T @ M @ V @ np.diag(1 / sx), atol=1e-12)


def test_biip_sx_drift_matrix_keeps_the_drift_term():
    # the drift cross product transforms as H_X does (C' = V S_X^-1 C S_X^-1 V^T),
    # which keeps the asymmetric objective's drift term tr(H_G dW C^T W^T)
    rng = np.random.default_rng(48)
    W, HX, HG, si, ki, so, ko = _sx_case(48)
    m, n = W.shape
    X = rng.standard_normal((40, n))
    C = O.drift_cross(X, X + 0.2 * rng.standard_normal((40, n)))
    dW = 0.1 * rng.standard_normal((m, n))
    Wp, _, HGp, sg, sx = O.biip_sx(W, HX, HG, si, ki, so, ko, 0.25, 0.25)
    dWp = O.biip_sx(dW, None, HG, si, ki, so, ko, 0.25, 0.0, sx=sx)[0]
    Cp = O.biip_sx(np.zeros((n, n)), C, None, si, ki, si, ki, 0.0, 0.0, sx=sx)[1]
    lhs = np.trace(HGp @ dWp @ Cp.T @ Wp.T)
    rhs = np.trace(HG @ dW @ C.T @ W.T)
    assert lhs == pytest.approx(rhs, rel=1e-10)


# ------------------------------------------------------ mu-incoherence


def test_mu_closed_forms():
    # eigenvectors along the axes: mu / sqrt(d) = 1
    assert O.mu_incoherence(np.diag([3.0, 1.0, 2.0, 5.0])) == pytest.approx(1.0, abs=1e-15)
    # a distinct spectrum rotated by a block Hadamard of order b: every
    # eigenvector is a column of T^T, whose entries are +-1/sqrt(b)
    rng = np.random.default_rng(50)
    for d, b in ((16, 16), (32, 8), (64, 64)):
        T = O.rotation_matrix(d, b, rng.choice([-1.0, 1.0], d))
        H = T @ np.diag(np.linspace(1.0, 2.0, d)) @ T.T
        assert O.mu_incoherence(H) == pytest.approx(1 / math.sqrt(b), rel=1e-12)
    # 2 x 2: the eigenvectors make the angle theta = atan2(2c, a - b) / 2
    for a, b, c in ((2.0, 1.0, 0.3), (1.0, 4.0, -2.0), (1.0, 1.0 + 1e-3, 5.0)):
        th = 0.5 * math.atan2(2 * c, a - b)
        want = max(abs(math.cos(th)), abs(math.sin(th)))
        assert O.mu_incoherence(np.array([[a, c], [c, b]])) == pytest.approx(want, rel=1e-13)
    # block diagonal: the value is the largest over all eigenvectors -- one
    # coordinate left alone (1) beside a Hadamard-rotated block of 4 (1/2)
    T = O.rotation_matrix(4, 4, np.array([1.0, -1.0, 1.0, 1.0]))
    H = np.zeros((5, 5))
    H[:4, :4] = T @ np.diag([1.0, 2.0, 3.0, 4.0]) @ T.T
    H[4, 4] = 2.5
    assert O.mu_incoherence(H) == pytest.approx(1.0, rel=1e-13)
    assert O.mu_incoherence(H[:4, :4]) == pytest.approx(0.5, rel=1e-13)


def test_mu_invariances():
    rng = np.random.default_rng(51)
    d = 24
    H = rand_spd(rng, d, 100.0)
    H[:, 3] *= 5.0
    H[3, :] *= 5.0
    mu = O.mu_incoherence(H)
    p = rng.permutation(d)
    s = rng.choice([-1.0, 1.0], d)
    assert O.mu_incoherence(H[np.ix_(p, p)]) == pytest.approx(mu, rel=1e-10)
    assert O.mu_incoherence(H * s[:, None] * s[None, :]) == pytest.approx(mu, rel=1e-10)
    assert O.mu_incoherence(7.5 * H) == pytest.approx(mu, rel=1e-10)
    assert O.mu_incoherence(H + 3.0 * np.eye(d)) == pytest.approx(mu, rel=1e-9)
    assert 1 / math.sqrt(d) <= mu <= 1.0
