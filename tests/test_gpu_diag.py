"""Parity of the incoherence modes (identity sides) and of the CV_in / CV_out
weight diagnostic with the oracle on the same inputs.

Tolerances: the modes are the BiIP transform (fp32 butterflies): <= 1e-5
relative Frobenius, as the full mode.  CV: norms from fp32 squares (relative
error ~1e-6), statistics in fp64: |CV - CV_oracle| <= 1e-6 + 1e-5 * CV.
"""
import numpy as np
import pytest
import torch

import post_quantization_02_amd as kq
import synth
from oracle import kronq_oracle as O
from gpu_helpers import DEV, host, rel_fro, say, spd_from_gram, to_dev_f32

pytestmark = pytest.mark.gpu


def _case(m, n, seed):
    W = synth.matrix(synth.NORMAL, seed, m, n, p1=0.02, dtype="f32")
    HX = spd_from_gram(seed + 1, n).astype(np.float32)
    G = synth.matrix(synth.GRAD_LOGNORMAL, seed + 2, 4 * m, m, p1=2.0, dtype="f64")
    HG = O.gram(G).astype(np.float32)
    return W, HX, HG, synth.signs(seed + 3, n), synth.signs(seed + 4, m)


@pytest.mark.parametrize("mode", ["full", "no_rescale", "su_only", "sv_only"])
@pytest.mark.parametrize("m,n,ko,ki", [(384, 352, 128, 32), (256, 4096, 256, 4096), (96, 100, 32, 4)])
def test_biip_modes(mode, m, n, ko, ki):
    say("biip mode", mode, m, n, ko, ki)
    W, HX, HG, si, so = _case(m, n, 71)
    Wd, HXd, HGd = to_dev_f32(W), to_dev_f32(HX), to_dev_f32(HG)
    sg = kq.kronq_biip_rotate_mode(Wd, HXd, HGd, to_dev_f32(si), ki, to_dev_f32(so), ko, 0.25, mode)
    Wp, HXp, HGp, s = O.biip_mode(W.astype(np.float64), HX.astype(np.float64), HG.astype(np.float64),
                                  si, ki, so, ko, 0.25, mode)
    e = (rel_fro(host(Wd), Wp), rel_fro(host(HXd), HXp), rel_fro(host(HGd), HGp), rel_fro(host(sg), s))
    say("  rel fro W %.2e HX %.2e HG %.2e sg %.2e" % e)
    assert max(e[:3]) <= 1e-5 and e[3] <= 1e-6
    if mode == "sv_only":      # untouched factor: bit for bit
        assert np.array_equal(host(HGd), HG)
    if mode == "su_only":
        assert np.array_equal(host(HXd), HX)


def test_identity_sides_in_unrotate_and_decode():
    say("identity sides: un-rotation and decode")
    m, n, bits = 128, 256, 4
    Wp = synth.matrix(synth.NORMAL, 81, m, n, p1=0.05, dtype="f32")
    so = synth.signs(82, m)
    sg = np.exp(synth.matrix(synth.NORMAL, 83, 1, m, p1=0.5, dtype="f64")[0]).astype(np.float32)
    Wd = to_dev_f32(Wp)
    kq.kronq_biip_unrotate(Wd, None, 1, to_dev_f32(so), 32, to_dev_f32(sg))
    want = O.unrotate(Wp.astype(np.float64), np.ones(n), 1, so, 32, sg.astype(np.float64))
    assert rel_fro(host(Wd), want) <= 1e-5
    # decode with the input side the identity and the output side the identity
    v = synth.matrix(synth.INT, 84, m, n, p1=64.0, dtype="f64")
    codes = np.mod(v, 16).astype(np.uint8)
    scales = (np.exp(synth.matrix(synth.NORMAL, 85, m, 1, p1=0.3, dtype="f64")) * 1e-3).astype(np.float32)
    zeros = np.full((m, 1), 7.0, dtype=np.float32)
    x = synth.matrix(synth.ACT_T4, 86, 1, n, dtype="f32")[0]
    packed = O.pack_codes(codes, bits)
    stored = torch.from_numpy(np.ascontiguousarray(packed)).to(DEV)
    for (si_, ki), (so_, ko) in [((None, 1), (so, 32)), ((synth.signs(87, n), 64), (None, 1))]:
        y = kq.kronq_decode_matvec(stored, n, bits, 0, to_dev_f32(scales), to_dev_f32(zeros),
                                   None if si_ is None else to_dev_f32(si_), ki,
                                   None if so_ is None else to_dev_f32(so_), ko, to_dev_f32(sg),
                                   to_dev_f32(x))
        want = O.decode_matvec(packed, bits, n, scales.astype(np.float64), zeros.astype(np.float64), 0,
                               np.ones(n) if si_ is None else si_, ki,
                               np.ones(m) if so_ is None else so_, ko, sg.astype(np.float64), x)
        e = rel_fro(host(y), want)
        say("  decode ki %d ko %d rel fro %.2e" % (ki, ko, e))
        assert e <= 1e-5


def _check_cv(got, want):
    for g, w in zip(got, want):
        assert abs(g - w) <= 1e-6 + 1e-5 * abs(w), (got, want)


@pytest.mark.parametrize("m,n,ld", [(4096, 4096, 4096), (37, 1001, 1001), (5000, 3, 3), (1, 5, 8),
                                    (200, 2048, 2056), (4096, 11008, 11008)])
def test_weight_cv(m, n, ld):
    say("weight cv", m, n, ld)
    W = synth.matrix(synth.NORMAL, 91, m, n, p1=0.02, dtype="f64")
    # outlier rows and columns, as in a real projection
    W[:, :: max(1, n // 7)] *= 6.0
    W[:: max(1, m // 5), :] *= 3.0
    W = W.astype(np.float32)
    buf = np.zeros((m, ld), dtype=np.float32)
    buf[:, :n] = W
    Wd = to_dev_f32(buf)[:, :n]
    cn = torch.empty(n, dtype=torch.float32, device=DEV)
    rn = torch.empty(m, dtype=torch.float32, device=DEV)
    out = kq.kronq_weight_cv(Wd, col_norms=cn, row_norms=rn)
    got = host(out)
    want = O.weight_cv(W.astype(np.float64))
    say("  cv in %.6f out %.6f (oracle %.6f %.6f)" % (got[0], got[1], want[0], want[1]))
    _check_cv(got, want)
    W64 = W.astype(np.float64)
    assert rel_fro(host(cn), np.sqrt((W64 ** 2).sum(0))) <= 1e-6
    assert rel_fro(host(rn), np.sqrt((W64 ** 2).sum(1))) <= 1e-6


def test_cv_out_unchanged_by_input_side_incoherence():
    """sv_only rotates rows by an orthogonal V: every row norm, and CV_out, stays."""
    say("CV_out under sv_only")
    m, n = 512, 1024
    W, HX, HG, si, so = _case(m, n, 95)
    W[:, ::37] *= 8.0
    Wd = to_dev_f32(W)
    before = host(kq.kronq_weight_cv(Wd)).copy()
    kq.kronq_biip_rotate_mode(Wd, None, to_dev_f32(HG), to_dev_f32(si), 256, to_dev_f32(so), 512,
                              0.25, "sv_only")
    after = host(kq.kronq_weight_cv(Wd))
    say("  CV_in %.4f -> %.4f, CV_out %.4f -> %.4f" % (before[0], after[0], before[1], after[1]))
    assert abs(after[1] - before[1]) <= 1e-5 * before[1]
    assert after[0] < 0.5 * before[0]     # the outlier columns are spread
