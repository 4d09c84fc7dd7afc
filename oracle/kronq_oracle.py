"""CPU oracle of the KronQ per-sublayer quantization path (float64, numpy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module:
only the tests, the smoke check of the package entry point and the benchmark's
CPU-baseline leg use it.  It shares no code with the GPU library.

Sources (cited by page and section; the pages are web renderings of the KronQ
paper, arXiv 2607.07964, "KronQ: LLM Quantization via Kronecker-Factored
Hessian", Lee, Li, Yin, Panda, COLM 2026):
  [summary]  hyper.ai paper summary, section "Method".
  [review]   Pith review page (pith.science, S4FLMGRF): referee summary, and the
             appendix fragments it reproduces -- proof of Proposition 1 (A.1),
             proof of Theorem 1 (A.2), Table 9, Algorithms 1 and 2.
  [readme]   GitHub README of the KronQ repository, "Reproduce from scratch"
             (flags --w_asym, --w_groupsize, --act_order, --alpha).
Where the pages leave a step open the plainest reading is taken; every such
reading is listed in the design notes of the repository and flagged below with
"Reading:".

Notation: W is m x n (rows = output channels, columns = input channels);
X is N x n activations, G is N x m output gradients; all float64 here.
Every function is pinned by a CPU test against closed forms, brute force or
hand-worked values (tests/test_oracle_pins.py); none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------
# Step 1: Kronecker factors.  [summary] Method: the per-sample gradient of a
# linear layer is g x^T, and under the K-FAC independence assumption the
# empirical-Fisher Hessian factorizes as H ~ H_X (x) H_G with H_X = E[x x^T],
# H_G = E[g g^T].  Reading: the expectation is the mean over the N token rows.
# --------------------------------------------------------------------------


def gram(A: np.ndarray) -> np.ndarray:
    """H = A^T A / N for A of shape (N, d): the second moment of the rows."""
    A = np.asarray(A, dtype=np.float64)
    return (A.T @ A) / A.shape[0]


def proxy_loss(dW: np.ndarray, HX: np.ndarray, HG: np.ndarray) -> float:
    """Kronecker-factored layer objective tr(H_G dW H_X dW^T).

    [summary] Method (the K-FAC quantization objective, equation not rendered);
    [review] proof of Theorem 1 writes the first term in exactly this trace form.
    """
    dW = np.asarray(dW, dtype=np.float64)
    return float(np.trace(HG @ dW @ HX @ dW.T))


def proxy_loss_kron(dW: np.ndarray, HX: np.ndarray, HG: np.ndarray) -> float:
    """The same objective written with the explicit Kronecker Hessian:
    vec(dW)^T (H_X (x) H_G) vec(dW), vec stacking columns.  Tiny inputs only."""
    v = np.asarray(dW, dtype=np.float64).reshape(-1, order="F")
    return float(v @ np.kron(HX, HG) @ v)


# --------------------------------------------------------------------------
# Step 2: bidirectional incoherence processing (BiIP).  [summary] Method and
# [review] Eq. 11-12 / proof of Theorem 1: an output-side diagonal rescale S_G
# (novel) next to the input-side one, then orthogonal transforms
# W' = U W V^T, H_G' = U H_G U^T, H_X' = V H_X V^T with U, V randomized
# Hadamard transforms (machinery after QuIP#, [readme]).
# Readings: S_G = diag(H_G)^alpha applied as W <- S_G W, H_G <- S_G^-1 H_G S_G^-1
# (the direction that leaves the objective unchanged); S_X = I; a randomized
# Hadamard transform on a dimension d = b*k is (I_b (x) H_k) D / sqrt(k) with
# H_k the Sylvester matrix and D = diag(signs); the signs are inputs.
# --------------------------------------------------------------------------


def hadamard_matrix(k: int) -> np.ndarray:
    """Sylvester Hadamard matrix, H[a, b] = (-1)^popcount(a & b)."""
    if k < 1 or (k & (k - 1)):
        raise ValueError("Hadamard order must be a power of two")
    a = np.arange(k)
    bits = np.bitwise_and.outer(a, a)
    pop = np.zeros_like(bits)
    while bits.any():
        pop += bits & 1
        bits >>= 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalized Walsh-Hadamard transform along the last axis (textbook
    in-place butterflies: for each h = 1, 2, 4, ..., pairs (i, i + h) become
    (a + b, a - b)).  Equals x @ hadamard_matrix(k)."""
    y = np.array(x, dtype=np.float64, copy=True)
    k = y.shape[-1]
    if k & (k - 1):
        raise ValueError("length must be a power of two")
    h = 1
    while h < k:
        y = y.reshape(y.shape[:-1] + (k // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (k,))
        h *= 2
    return y


def rotate_rows(M: np.ndarray, block: int, signs: np.ndarray) -> np.ndarray:
    """M T^T where T = (I (x) H_block) diag(signs) / sqrt(block) acts on the
    column index of M (each row r becomes T M[r, :])."""
    M = np.asarray(M, dtype=np.float64)
    rows, d = M.shape
    if d % block:
        raise ValueError("block must divide the dimension")
    Y = (M * np.asarray(signs, dtype=np.float64)[None, :]).reshape(rows, d // block, block)
    return fwht(Y).reshape(rows, d) / np.sqrt(block)


def rotate_cols(M: np.ndarray, block: int, signs: np.ndarray) -> np.ndarray:
    """T M with T as in rotate_rows acting on the row index of M."""
    return rotate_rows(np.asarray(M, dtype=np.float64).T, block, signs).T


def rotation_matrix(d: int, block: int, signs: np.ndarray) -> np.ndarray:
    """Explicit T = (I (x) H_block) diag(signs) / sqrt(block); small d only."""
    T = np.kron(np.eye(d // block), hadamard_matrix(block)) / np.sqrt(block)
    return T * np.asarray(signs, dtype=np.float64)[None, :]


def output_rescale(HG: np.ndarray, alpha: float) -> np.ndarray:
    """s_g = diag(H_G)^alpha; a non-positive diagonal entry gives 1."""
    d = np.diag(np.asarray(HG, dtype=np.float64)).copy()
    s = np.ones_like(d)
    pos = d > 0
    s[pos] = d[pos] ** alpha
    return s


def biip(W, HX, HG, in_signs, in_block, out_signs, out_block, alpha):
    """Returns (W', H_X', H_G', s_g):
       W'   = U S_G W V^T
       H_X' = V H_X V^T
       H_G' = U S_G^-1 H_G S_G^-1 U^T
    with U = (I (x) H_out_block) D_out / sqrt(out_block) and V likewise on the
    input side.  HX or HG may be None (then returned as None)."""
    W = np.asarray(W, dtype=np.float64)
    s = output_rescale(HG, alpha) if HG is not None else np.ones(W.shape[0])
    Ws = W * s[:, None]
    Wp = rotate_cols(rotate_rows(Ws, in_block, in_signs), out_block, out_signs)
    HXp = None
    if HX is not None:
        HXp = rotate_cols(rotate_rows(HX, in_block, in_signs), in_block, in_signs)
    HGp = None
    if HG is not None:
        HGs = np.asarray(HG, dtype=np.float64) / s[:, None] / s[None, :]
        HGp = rotate_cols(rotate_rows(HGs, out_block, out_signs), out_block, out_signs)
    return Wp, HXp, HGp, s


# --------------------------------------------------------------------------
# Step 3: act-order, damping and the Cholesky factor of the inverse.
# [review] Algorithm 2 (its damping step, then its inverse-Cholesky step): the
# damped H_X is H_X + lambda mean(diag(H_X)) I, and the loop takes the inverse
# Cholesky factor of it.  [readme] --act_order.
# Readings: the act-order key is diag(H_X') (post-BiIP, undamped), sorted in
# descending order, ties to the lower index; "InverseCholesky" is the upper
# triangular R with positive diagonal and R^T R = H^-1 (the factor the
# column loop's compensation uses).
# --------------------------------------------------------------------------


def act_order_perm(HX: np.ndarray) -> np.ndarray:
    """perm[j] = original column processed j-th: stable descending sort of diag."""
    d = np.diag(np.asarray(HX, dtype=np.float64))
    return np.argsort(-d, kind="stable").astype(np.int64)


def damp(H: np.ndarray, lam: float) -> np.ndarray:
    """H + lam * mean(diag(H)) * I."""
    H = np.asarray(H, dtype=np.float64)
    return H + lam * np.mean(np.diag(H)) * np.eye(H.shape[0])


def chol_inv_upper(H: np.ndarray):
    """Returns (R, info): R upper triangular with positive diagonal and
    R^T R = H^-1; info = -1 on success, else the first index whose pivot of the
    Cholesky factorization of H is not positive (R is then None)."""
    H = np.asarray(H, dtype=np.float64)
    try:
        np.linalg.cholesky(H)
    except np.linalg.LinAlgError:
        # locate the first non-positive pivot by the textbook column loop
        n = H.shape[0]
        L = np.zeros_like(H)
        for j in range(n):
            piv = H[j, j] - L[j, :j] @ L[j, :j]
            if not piv > 0:
                return None, j
            L[j, j] = np.sqrt(piv)
            L[j + 1:, j] = (H[j + 1:, j] - L[j + 1:, :j] @ L[j, :j]) / L[j, j]
        return None, n - 1
    Hinv = np.linalg.inv(H)
    Hinv = 0.5 * (Hinv + Hinv.T)
    R = np.linalg.cholesky(Hinv).T
    return R, -1


def prepare_hessian(HXp: np.ndarray, lam: float, act_order: bool):
    """Act-order permutation (or identity) and the damped, permuted H."""
    n = HXp.shape[0]
    perm = act_order_perm(HXp) if act_order else np.arange(n, dtype=np.int64)
    Hp = np.asarray(HXp, dtype=np.float64)[np.ix_(perm, perm)]
    return perm, damp(Hp, lam)


# --------------------------------------------------------------------------
# Step 4: column-wise OBS quantize-and-compensate using H_X alone.
# [summary] Method and [review] Proposition 1: after quantizing column p the
# compensation is the scaled quantization error times rows of the inverse
# Cholesky factor; H_G cancels, so the solver is GPTQ/GPTAQ's.  [review]
# Algorithm 2: lazy batches of B columns (an exact reordering of the same
# updates, so this oracle runs the plain column-sequential loop).  GPTAQ's
# asymmetric term is zero here because no drifted input stream exists.
# Quantizer ([readme] --w_asym, --w_groupsize; [review] "plain uniform
# per-channel grid"): asymmetric uniform min/max grid.  Readings: the range
# includes 0; a degenerate range becomes [-1, 1]; scale = (max-min)/(2^b-1);
# zero = round(-min/scale); codes round half to even and clamp to [0, 2^b-1];
# per-channel parameters come from the whole initial row, group parameters from
# the current compensated values of the group when its first column is reached;
# groups follow processing order.
# --------------------------------------------------------------------------


def quant_params(V: np.ndarray, bits: int):
    """Per-row (scale, zero) of the asymmetric grid for the rows of V (m x c)."""
    V = np.asarray(V, dtype=np.float64)
    maxq = 2 ** bits - 1
    xmin = np.minimum(V.min(axis=1), 0.0)
    xmax = np.maximum(V.max(axis=1), 0.0)
    deg = xmin == xmax
    xmin = np.where(deg, -1.0, xmin)
    xmax = np.where(deg, 1.0, xmax)
    scale = (xmax - xmin) / maxq
    zero = np.rint(-xmin / scale)
    return scale, zero


def zero_pre_round(V: np.ndarray, bits: int):
    """-min/scale of quant_params before rounding (for tie checks)."""
    V = np.asarray(V, dtype=np.float64)
    maxq = 2 ** bits - 1
    xmin = np.minimum(V.min(axis=1), 0.0)
    xmax = np.maximum(V.max(axis=1), 0.0)
    deg = xmin == xmax
    xmin = np.where(deg, -1.0, xmin)
    xmax = np.where(deg, 1.0, xmax)
    return -xmin / ((xmax - xmin) / maxq)


def rtn(V: np.ndarray, scale: np.ndarray, zero: np.ndarray, bits: int):
    """Round-to-nearest on the grid: returns (codes, dequantized, pre-round t)."""
    t = np.asarray(V, dtype=np.float64) / scale[:, None] + zero[:, None]
    q = np.clip(np.rint(t), 0, 2 ** bits - 1)
    return q, scale[:, None] * (q - zero[:, None]), t


def gptq(W: np.ndarray, R: np.ndarray, perm, bits: int, group: int, decide_codes=None,
         decide_params=None):
    """Column-sequential OBS loop.

    W      : m x n weights in natural column order (BiIP domain).
    R      : n x n upper factor in processing order (R^T R = H^-1 of the
             damped, permuted H).
    perm   : processing order (perm[j] = natural column of step j).
    group  : <= 0 per-channel; else group size in processing order.
    decide_codes  : optional hook (j, t, q) -> q; the tests use it to compare a
                    second implementation whose rounding ties may differ (it
                    receives step j's pre-round values t and this oracle's q).
    decide_params : optional hook (g, scale, zero, zt) -> (scale, zero) for the
                    parameters of group g (zt = -min/scale before rounding).
    Returns dict(codes (m x n natural, int), scales, zeros (m x ngroups), What
    (m x n natural), pre (m x n natural), E (m x n processing order)).
    """
    W = np.asarray(W, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    m, n = W.shape
    perm = np.asarray(perm, dtype=np.int64)
    maxq = 2 ** bits - 1
    Wt = W[:, perm].copy()
    ng = 1 if group <= 0 else (n + group - 1) // group
    scales = np.zeros((m, ng))
    zeros = np.zeros((m, ng))
    codes = np.zeros((m, n))
    What = np.zeros((m, n))
    pre = np.zeros((m, n))
    E = np.zeros((m, n))
    if group <= 0:
        scale, zero = quant_params(Wt, bits)
        if decide_params is not None:
            scale, zero = decide_params(0, scale, zero, zero_pre_round(Wt, bits))
        scales[:, 0], zeros[:, 0] = scale, zero
    for j in range(n):
        if group > 0 and j % group == 0:
            scale, zero = quant_params(Wt[:, j:j + group], bits)
            if decide_params is not None:
                scale, zero = decide_params(j // group, scale, zero,
                                            zero_pre_round(Wt[:, j:j + group], bits))
            scales[:, j // group], zeros[:, j // group] = scale, zero
        t = Wt[:, j] / scale + zero
        q = np.clip(np.rint(t), 0, maxq)
        if decide_codes is not None:
            q = decide_codes(j, t, q)
        wq = scale * (q - zero)
        e = (Wt[:, j] - wq) / R[j, j]
        Wt[:, j + 1:] -= np.outer(e, R[j, j + 1:])
        codes[:, j], What[:, j], pre[:, j], E[:, j] = q, wq, t, e
    inv = np.empty(n, dtype=np.int64)
    inv[perm] = np.arange(n)
    return dict(codes=codes[:, inv], scales=scales, zeros=zeros, What=What[:, inv],
                pre=pre[:, inv], E=E)


# --------------------------------------------------------------------------
# GPTAQ asymmetric correction.  [summary] Method: building on GPTAQ, the
# objective also corrects for input drift (asymmetric calibration): the
# quantized layer sees the inputs X of the partly quantized model while its
# target is the full-precision layer on the full-precision inputs X_fp;
# [review] Algorithm 2 takes dXX^T with the Hessian factor, forms
# P = alpha (dXX^T L) (.) M_U L^T after the inverse Cholesky step (M_U an
# upper-triangular mask) and uses P in the column loop, whose update is cut
# off on the pages; [review] proof of Theorem 1: (dXX^T)' = V dXX^T V^T.
# Readings (derived, pinned by brute force in the tests):
#  * objective, per output row w (H_G cancels as in Proposition 1):
#      || X w^ - X_fp w ||^2 / N = d^T H_X d + 2 d^T C^T w + const,
#    with d = w - w^, dX = X_fp - X and C = dX^T X / N (row form of the
#    pages' dXX^T, normalized like H_X = X^T X / N); alpha scales the drift
#    term (alpha = 1 is the full asymmetric objective, 0 is GPTQ);
#  * the loop is the sequential OBS where column j's drift term is committed
#    once column j is quantized: each column is rounded at the optimum of the
#    objective given the quantized earlier columns and the drift of the
#    earlier columns.  In the coordinates e = R^-T d that objective separates,
#    and the value at which column k is rounded works out to
#      w~_k = w_k - sum_{i<k} eps_i R_ik + sum_{j<k} w_j P_jk,
#    eps_i = (w~_i - q_i) / R_ii (the scaled quantization error), with
#      P = alpha ((C R^T) (.) M) R,  M_ji = 1 for j < i (strictly upper),
#    i.e. L = R^T is the pages' lower inverse Cholesky factor (L L^T = H^-1);
#    after column j is quantized every later column k moves by
#    -eps_j R_jk + w_j P_jk, with w_j the full-precision weight;
#  * C, like H_X, is rotated by the input side of BiIP and reordered by the
#    act-order permutation; P is formed in processing order.
# --------------------------------------------------------------------------


def drift_cross(X, Xfp) -> np.ndarray:
    """C = (X_fp - X)^T X / N for the N token rows of X (inputs of the partly
    quantized model) and X_fp (inputs of the full-precision model)."""
    X = np.asarray(X, dtype=np.float64)
    dX = np.asarray(Xfp, dtype=np.float64) - X
    return (dX.T @ X) / X.shape[0]


def gptaq_correction(C, R, alpha: float) -> np.ndarray:
    """P = alpha ((C R^T) (.) M) R with M strictly upper triangular; C and R
    in processing order (R^T R = Hd^-1)."""
    C = np.asarray(C, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    K = C @ R.T
    return alpha * (np.triu(K, 1) @ R)


def gptaq(W, R, perm, bits: int, group: int, P, decide_codes=None, decide_params=None):
    """The column loop with the asymmetric correction: as gptq(), and after
    column j is quantized every later column k (processing order) also moves
    by + w_j P[j, k], w_j the full-precision weights of column j.  P = 0 is
    gptq().  Returns gptq()'s dict."""
    W = np.asarray(W, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    P = np.asarray(P, dtype=np.float64)
    m, n = W.shape
    perm = np.asarray(perm, dtype=np.int64)
    maxq = 2 ** bits - 1
    W0 = W[:, perm]
    Wt = W0.copy()
    ng = 1 if group <= 0 else (n + group - 1) // group
    scales = np.zeros((m, ng))
    zeros = np.zeros((m, ng))
    codes = np.zeros((m, n))
    What = np.zeros((m, n))
    pre = np.zeros((m, n))
    E = np.zeros((m, n))
    if group <= 0:
        scale, zero = quant_params(W0, bits)
        if decide_params is not None:
            scale, zero = decide_params(0, scale, zero, zero_pre_round(W0, bits))
        scales[:, 0], zeros[:, 0] = scale, zero
    for j in range(n):
        if group > 0 and j % group == 0:
            scale, zero = quant_params(Wt[:, j:j + group], bits)
            if decide_params is not None:
                scale, zero = decide_params(j // group, scale, zero,
                                            zero_pre_round(Wt[:, j:j + group], bits))
            scales[:, j // group], zeros[:, j // group] = scale, zero
        t = Wt[:, j] / scale + zero
        q = np.clip(np.rint(t), 0, maxq)
        if decide_codes is not None:
            q = decide_codes(j, t, q)
        wq = scale * (q - zero)
        e = (Wt[:, j] - wq) / R[j, j]
        Wt[:, j + 1:] -= np.outer(e, R[j, j + 1:]) - np.outer(W0[:, j], P[j, j + 1:])
        codes[:, j], What[:, j], pre[:, j], E[:, j] = q, wq, t, e
    inv = np.empty(n, dtype=np.int64)
    inv[perm] = np.arange(n)
    return dict(codes=codes[:, inv], scales=scales, zeros=zeros, What=What[:, inv],
                pre=pre[:, inv], E=E)


# --------------------------------------------------------------------------
# Step 5: sensitivity and bit allocation.  [summary] Method: the expected loss
# of a sublayer scales with eps^2 tr(H); with H ~ H_X (x) H_G the score is
# s = tr(H_G) tr(H_X), computed after BiIP; higher bit-widths go to larger s.
# [readme] --inter_layer_mp: upgrade the top sensitive sublayer types by +1 bit.
# Readings: traces of the post-BiIP, undamped factors; allocation is greedy
# from bmin, visiting sublayers in descending score (ties to the lower index),
# raising each by one bit at a time while it is below bmax and the parameter-
# weighted bit total stays within the budget.
# --------------------------------------------------------------------------


def sensitivity(HXp: np.ndarray, HGp: np.ndarray):
    trx = float(np.sum(np.diag(np.asarray(HXp, dtype=np.float64))))
    trg = float(np.sum(np.diag(np.asarray(HGp, dtype=np.float64))))
    return trx, trg, trx * trg


def allocate_bits(scores, n_params, bmin: int, bmax: int, budget_bits: int):
    """Greedy allocation; returns the list of bits (raises ValueError when the
    budget cannot hold every sublayer at bmin)."""
    L = len(scores)
    n_params = [int(x) for x in n_params]
    used = bmin * sum(n_params)
    if budget_bits < used or bmin > bmax:
        raise ValueError("budget below the minimum allocation")
    bits = [bmin] * L
    order = sorted(range(L), key=lambda i: (-float(scores[i]), i))
    for i in order:
        while bits[i] < bmax and used + n_params[i] <= budget_bits:
            bits[i] += 1
            used += n_params[i]
    return bits


# --------------------------------------------------------------------------
# Whole sublayer, end to end (float64 throughout).
# --------------------------------------------------------------------------


def quantize_sublayer(W, X, G, in_signs, in_block, out_signs, out_block, alpha, lam, bits,
                      group, act_order):
    HX = gram(X)
    HG = gram(G)
    Wp, HXp, HGp, s = biip(W, HX, HG, in_signs, in_block, out_signs, out_block, alpha)
    trs = sensitivity(HXp, HGp)
    perm, H = prepare_hessian(HXp, lam, act_order)
    R, info = chol_inv_upper(H)
    if R is None:
        raise np.linalg.LinAlgError("damped H not positive definite at pivot %d" % info)
    out = gptq(Wp, R, perm, bits, group)
    out.update(HX=HX, HG=HG, Wp=Wp, HXp=HXp, HGp=HGp, sg=s, traces=trs, perm=perm, R=R, H=H)
    return out


# --------------------------------------------------------------------------
# Deploy codec.  [readme] the quantized weights are stored packed int4 / int2
# and a fused dequant + BiIP matvec unpacks them on the fly for single-token
# decode; 3-bit weights are not bit-packed.  [review] Theorem 1: W' = U W V^T
# with U, V orthogonal, and [summary] Method: the output-side rescale S_G is
# applied before the transforms, so the original-domain weight is
# S_G^-1 U^T W' V.
# Readings: codes are packed little-endian within a byte (code j of a row at
# bit offset bits * (j mod (8 / bits)) of byte j / (8 / bits)), rows padded to
# whole bytes; a group index follows the processing order as in the column
# loop (natural column c belongs to group pos(c) / group, pos = perm^-1).
# --------------------------------------------------------------------------


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """m x n codes (0 .. 2^bits - 1) -> m x ceil(n * bits / 8) bytes."""
    q = np.asarray(codes, dtype=np.int64)
    m, n = q.shape
    per = 8 // bits
    nb = (n + per - 1) // per
    out = np.zeros((m, nb), dtype=np.int64)
    for j in range(n):
        out[:, j // per] |= (q[:, j] & ((1 << bits) - 1)) << (bits * (j % per))
    return out.astype(np.uint8)


def unpack_codes(packed: np.ndarray, bits: int, n: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.int64)
    per = 8 // bits
    q = np.zeros((p.shape[0], n), dtype=np.int64)
    for j in range(n):
        q[:, j] = (p[:, j // per] >> (bits * (j % per))) & ((1 << bits) - 1)
    return q


def dequant(codes, scales, zeros, group: int, perm=None) -> np.ndarray:
    """W'[i][c] = scale[i][g] (q[i][c] - zero[i][g]) with g the group of
    natural column c (0 per-channel; pos(c) // group otherwise)."""
    q = np.asarray(codes, dtype=np.float64)
    m, n = q.shape
    scales = np.asarray(scales, dtype=np.float64).reshape(m, -1)
    zeros = np.asarray(zeros, dtype=np.float64).reshape(m, -1)
    if group <= 0:
        g = np.zeros(n, dtype=np.int64)
    else:
        pos = np.arange(n) if perm is None else np.argsort(np.asarray(perm, dtype=np.int64))
        g = pos // group
    return scales[:, g] * (q - zeros[:, g])


def unrotate(Wp, in_signs, in_block, out_signs, out_block, sg) -> np.ndarray:
    """S_G^-1 U^T W' V: the inverse of the weight side of biip()."""
    Wp = np.asarray(Wp, dtype=np.float64)
    # U^T M: the transpose of T acts on the row index: undo the Hadamard, then the signs
    A = fwht(Wp.T.reshape(Wp.shape[1], -1, out_block)).reshape(Wp.shape[1], -1).T / np.sqrt(out_block)
    A = A * np.asarray(out_signs, dtype=np.float64)[:, None]
    # M V: V acts on the column index from the right, V = (I (x) H) D / sqrt(k)
    B = fwht(A.reshape(A.shape[0], -1, in_block)).reshape(A.shape) / np.sqrt(in_block)
    B = B * np.asarray(in_signs, dtype=np.float64)[None, :]
    return B / np.asarray(sg, dtype=np.float64)[:, None]


def decode_matvec(packed, bits, n, scales, zeros, group, in_signs, in_block, out_signs,
                  out_block, sg, x, perm=None) -> np.ndarray:
    """y = S_G^-1 U^T W' V x for the packed quantized W', in the order the
    deploy path computes it: x' = V x, y' = W' x', y = S_G^-1 U^T y'."""
    x = np.asarray(x, dtype=np.float64)
    xp = (fwht((x * np.asarray(in_signs, dtype=np.float64)).reshape(-1, in_block)).reshape(-1)
          / np.sqrt(in_block))
    codes = unpack_codes(packed, bits, n) if bits in (2, 4) else np.asarray(packed, dtype=np.int64)
    yp = dequant(codes, scales, zeros, group, perm) @ xp
    y = fwht(yp.reshape(-1, out_block)).reshape(-1) / np.sqrt(out_block)
    return y * np.asarray(out_signs, dtype=np.float64) / np.asarray(sg, dtype=np.float64)


# --------------------------------------------------------------------------
# Allocation variants.  [summary] Method: under the second-order
# approximation a sublayer's expected loss is proportional to eps^2 tr(H), with
# tr(H) = tr(H_X) tr(H_G) = s; higher bit-widths go to larger s.  [readme]
# --inter_layer_mp N: upgrade the top-N sensitive sublayer *types* by +1 bit.
# Readings:
#  * pass-wise: visit the sublayers in score order (ties: lower index) and give
#    each +1 bit when it is below bmax and fits the budget; repeat whole passes
#    until a pass changes nothing.
#  * marginal: eps(b) of a uniform grid halves with every bit, so eps^2 ~ 4^-b
#    and one more bit lowers sublayer i's loss by s_i (4^-b - 4^-(b+1)), at a
#    cost of n_i bits.  Repeatedly take, among the upgrades that fit, the one
#    with the largest loss reduction per bit, s_i 4^-b / n_i (the common factor
#    3/4 dropped; ties: lower index), until none fits.
#  * types: a type's score is the sum of its sublayers' scores; the N types
#    with the largest sums (ties: lower type id) get base + 1 bits, the others
#    base bits.
# --------------------------------------------------------------------------


def _alloc_start(scores, n_params, bmin, bmax, budget_bits):
    n_params = [int(x) for x in n_params]
    used = bmin * sum(n_params)
    if budget_bits < used or bmin > bmax:
        raise ValueError("budget below the minimum allocation")
    return n_params, used, [bmin] * len(scores)


def allocate_bits_passwise(scores, n_params, bmin: int, bmax: int, budget_bits: int):
    n_params, used, bits = _alloc_start(scores, n_params, bmin, bmax, budget_bits)
    order = sorted(range(len(scores)), key=lambda i: (-float(scores[i]), i))
    changed = True
    while changed:
        changed = False
        for i in order:
            if bits[i] < bmax and used + n_params[i] <= budget_bits:
                bits[i] += 1
                used += n_params[i]
                changed = True
    return bits


def marginal_gain_per_bit(score: float, b: int, n: int) -> float:
    """s 4^-b / n: the loss reduction per bit of raising a sublayer from b bits
    (up to the constant 3/4), formed as ldexp then one division."""
    return math.ldexp(float(score), -2 * b) / float(n)


def allocate_bits_marginal(scores, n_params, bmin: int, bmax: int, budget_bits: int):
    n_params, used, bits = _alloc_start(scores, n_params, bmin, bmax, budget_bits)
    while True:
        best = -1
        for i in range(len(scores)):
            if bits[i] >= bmax or used + n_params[i] > budget_bits:
                continue
            if best < 0 or (marginal_gain_per_bit(scores[i], bits[i], n_params[i]) >
                            marginal_gain_per_bit(scores[best], bits[best], n_params[best])):
                best = i
        if best < 0:
            return bits
        bits[best] += 1
        used += n_params[best]


def allocate_types(scores, type_of, n_types: int, base_bits: int, n_upgrade: int):
    """Per-sublayer bits: base + 1 for the sublayers of the n_upgrade types
    with the largest summed scores, base for the rest."""
    total = [0.0] * n_types
    for s, t in zip(scores, type_of):
        total[int(t)] += float(s)
    ranked = sorted(range(n_types), key=lambda t: (-total[t], t))
    up = set(ranked[:n_upgrade])
    return [base_bits + (1 if int(t) in up else 0) for t in type_of]


# --------------------------------------------------------------------------
# BiIP variants and diagnostics.  [readme] --incoh_mode {full, no_rescale,
# su_only, sv_only} (component ablation); [review] Figure 2: CV_in and CV_out
# are the coefficients of variation of the column and row norms of W, and
# incoherence on the input side alone leaves CV_out nearly unchanged while
# BiIP lowers both.
# Readings: full = S_G, U and V; no_rescale = U and V without S_G (alpha 0);
# su_only = the output side alone (S_G and U, V = I); sv_only = the input side
# alone (V, with U = I and no S_G).  An identity side is block 1 with all-one
# signs.  CV = population standard deviation / mean.
# --------------------------------------------------------------------------

INCOH_MODES = ("full", "no_rescale", "su_only", "sv_only")


def biip_mode(W, HX, HG, in_signs, in_block, out_signs, out_block, alpha, mode: str):
    m, n = np.asarray(W).shape
    if mode == "full":
        return biip(W, HX, HG, in_signs, in_block, out_signs, out_block, alpha)
    if mode == "no_rescale":
        return biip(W, HX, HG, in_signs, in_block, out_signs, out_block, 0.0)
    if mode == "su_only":
        return biip(W, HX, HG, np.ones(n), 1, out_signs, out_block, alpha)
    if mode == "sv_only":
        return biip(W, HX, HG, in_signs, in_block, np.ones(m), 1, 0.0)
    raise ValueError("unknown incoherence mode %r" % (mode,))


def weight_cv(W):
    """(CV_in, CV_out) of the column norms and the row norms of W."""
    W = np.asarray(W, dtype=np.float64)
    col = np.sqrt(np.sum(W * W, axis=0))
    row = np.sqrt(np.sum(W * W, axis=1))
    return float(np.std(col) / np.mean(col)), float(np.std(row) / np.mean(row))


# --------------------------------------------------------------------------
# Input-side rescale S_X.  [summary] Method: BiIP extends the input-side
# diagonal rescaling to both directions (the output-side S_G being the new
# part) before the orthogonal transforms; [review] Algorithm 1 returns S_X
# beside S_G, U and V; [review] proof of Theorem 1: the proxy loss
# tr(H_G dW H_X dW^T) is unchanged by the transforms.
# Reading: S_X has the form of S_G on the other side, s_x = diag(H_X)^alpha_x
# (a non-positive diagonal entry gives 1), taken from H_X before any
# transform; W is scaled column-wise by s_x and H_X by s_x^-1 on both sides,
# which leaves the proxy loss of a correspondingly transformed dW unchanged:
#   W'   = U S_G W S_X V^T
#   H_X' = V S_X^-1 H_X S_X^-1 V^T
#   H_G' = U S_G^-1 H_G S_G^-1 U^T
# --------------------------------------------------------------------------

def input_rescale(HX: np.ndarray, alpha_x: float) -> np.ndarray:
    """s_x = diag(H_X)^alpha_x; a non-positive diagonal entry gives 1."""
    d = np.diag(np.asarray(HX, dtype=np.float64)).copy()
    s = np.ones_like(d)
    pos = d > 0
    s[pos] = d[pos] ** alpha_x
    return s


def biip_sx(W, HX, HG, in_signs, in_block, out_signs, out_block, alpha, alpha_x, sx=None):
    """Returns (W', H_X', H_G', s_g, s_x) as above.  s_x is input_rescale(HX,
    alpha_x) unless given (then HX may be None, or any n x n matrix that is to
    be transformed the way H_X is, such as the drift cross product)."""
    W = np.asarray(W, dtype=np.float64)
    if sx is None:
        sx = input_rescale(HX, alpha_x)
    sx = np.asarray(sx, dtype=np.float64)
    Wp, _, HGp, sg = biip(W * sx[None, :], None, HG, in_signs, in_block, out_signs, out_block, alpha)
    HXp = None
    if HX is not None:
        HXs = np.asarray(HX, dtype=np.float64) / sx[:, None] / sx[None, :]
        HXp = rotate_cols(rotate_rows(HXs, in_block, in_signs), in_block, in_signs)
    return Wp, HXp, HGp, sg, sx


def unrotate_sx(Wp, in_signs, in_block, out_signs, out_block, sg, sx) -> np.ndarray:
    """S_G^-1 U^T W' V S_X^-1: the inverse of the weight side of biip_sx()."""
    return unrotate(Wp, in_signs, in_block, out_signs, out_block, sg) / np.asarray(sx, dtype=np.float64)[None, :]


# --------------------------------------------------------------------------
# mu-incoherence.  [summary] Method and [review] Figure 2(a): the incoherence
# of a proxy Hessian is reported as mu(H)/sqrt(d); it is near 1 when an
# eigenvector lies along a coordinate axis and small once the transforms have
# spread every eigenvector over all coordinates.
# Reading: the textbook definition of a mu-incoherent symmetric matrix
# H = Q Lambda Q^T (Q orthogonal) is max_ij |Q_ij| <= mu / sqrt(d), so
# mu(H)/sqrt(d) = max_ij |Q_ij| over the eigenvector matrix.  Where eigenvalues
# repeat, Q (and so the value) is not unique; the checks then compare the
# eigen-decomposition's validity instead.
# --------------------------------------------------------------------------

def mu_incoherence(H: np.ndarray) -> float:
    """max_ij |Q_ij| for the eigenvectors Q of the symmetric H (numpy eigh)."""
    _, Q = np.linalg.eigh(np.asarray(H, dtype=np.float64))
    return float(np.max(np.abs(Q)))
