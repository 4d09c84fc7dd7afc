"""Parity of the input-side rescale S_X (kronq_biip_rotate_sx and
kronq_biip_unrotate_sx) with the oracle on the same fp32 inputs.

Tolerances as for BiIP: the transforms are fp32 butterflies (<= 1e-5 relative
Frobenius); s_x is one fp32 power of an fp32 diagonal entry (<= 1e-6).
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


def _f64(*a):
    return [None if x is None else np.asarray(x, dtype=np.float64) for x in a]


@pytest.mark.parametrize("m,n,ko,ki,ax", [
    (384, 352, 128, 32, 0.25),     # several blocks both sides
    (256, 4096, 256, 4096, 0.25),  # wide input block (two passes on the row side)
    (128, 1376, 128, 32, 0.5),     # 43 input blocks; alpha_x 1/2 (unit-diagonal H_X before V)
    (96, 64, 32, 1, 0.25),         # identity input side: the rescale alone on that side
    (24, 6, 8, 2, 0.25),           # width not a multiple of 4: scalar kernels
])
def test_biip_sx_small(m, n, ko, ki, ax):
    say("biip with S_X", m, n, ko, ki, ax)
    W, HX, HG, si, so = _case(m, n, 91)
    if ki == 1:
        si = np.ones(n, dtype=np.float32)
    Wd, HXd, HGd = to_dev_f32(W), to_dev_f32(HX), to_dev_f32(HG)
    sg, sx = kq.kronq_biip_rotate_sx(Wd, HXd, HGd, None if ki == 1 else to_dev_f32(si), ki,
                                     to_dev_f32(so), ko, 0.25, ax)
    Wp, HXp, HGp, s, t = O.biip_sx(*_f64(W, HX, HG), si, ki, so, ko, 0.25, ax)
    e = (rel_fro(host(Wd), Wp), rel_fro(host(HXd), HXp), rel_fro(host(HGd), HGp),
         rel_fro(host(sg), s), rel_fro(host(sx), t))
    say("  rel fro W %.2e HX %.2e HG %.2e sg %.2e sx %.2e" % e)
    assert max(e[:3]) <= 1e-5 and max(e[3:]) <= 1e-6
    if ax == 0.5 and ki == 1:
        np.testing.assert_allclose(np.diag(host(HXd)), 1.0, rtol=1e-6)


def test_biip_sx_alpha_zero_is_biip_bit_for_bit():
    say("S_X with alpha_x = 0 equals kronq_biip_rotate")
    m, n = 256, 512
    W, HX, HG, si, so = _case(m, n, 92)
    a = [to_dev_f32(x) for x in (W, HX, HG)]
    b = [to_dev_f32(x) for x in (W, HX, HG)]
    kq.kronq_biip_rotate(*a, to_dev_f32(si), 128, to_dev_f32(so), 64, 0.25)
    _, sx = kq.kronq_biip_rotate_sx(*b, to_dev_f32(si), 128, to_dev_f32(so), 64, 0.25, 0.0)
    for x, y in zip(a, b):
        assert np.array_equal(host(x), host(y))
    assert np.array_equal(host(sx), np.ones(n, dtype=np.float32))


def test_biip_sx_given_shared_input_and_drift_matrix():
    """A second sublayer on the same input reuses s_x (sx_given, HX already
    transformed); the drift cross product is transformed as H_X with W and
    H_G absent."""
    say("S_X given: shared input, drift matrix")
    m, n = 128, 384
    W, HX, HG, si, so = _case(m, n, 93)
    W2 = synth.matrix(synth.NORMAL, 94, 2 * m, n, p1=0.02, dtype="f32")
    HG2 = O.gram(synth.matrix(synth.GRAD_LOGNORMAL, 95, 8 * m, 2 * m, p1=2.0, dtype="f64")).astype(np.float32)
    so2 = synth.signs(96, 2 * m)
    X = synth.matrix(synth.ACT_T4, 97, 512, n, dtype="f64")
    C = O.drift_cross(X, X + 0.05 * synth.matrix(synth.NORMAL, 98, 512, n, dtype="f64")).astype(np.float32)
    HXd, sid = to_dev_f32(HX), to_dev_f32(si)
    _, sx = kq.kronq_biip_rotate_sx(to_dev_f32(W), HXd, to_dev_f32(HG), sid, 64, to_dev_f32(so), 128,
                                    0.25, 0.25)
    W2d, HG2d = to_dev_f32(W2), to_dev_f32(HG2)
    kq.kronq_biip_rotate_sx(W2d, None, HG2d, sid, 64, to_dev_f32(so2), 64, 0.25, 0.0, sx=sx, sx_given=True)
    Cd = to_dev_f32(C)
    kq.kronq_biip_rotate_sx(None, Cd, None, sid, 64, None, 1, 0.0, 0.0, sx=sx, sx_given=True, m=1)
    t = host(sx).astype(np.float64)
    Wp2, _, HGp2, _, _ = O.biip_sx(*_f64(W2, None, HG2), si, 64, so2, 64, 0.25, 0.0, sx=t)
    _, Cp, _, _, _ = O.biip_sx(np.zeros((1, n)), C.astype(np.float64), None, si, 64, np.ones(1), 1,
                               0.0, 0.0, sx=t)
    _, HXp, _, _, t0 = O.biip_sx(*_f64(W, HX, HG), si, 64, so, 128, 0.25, 0.25)
    e = (rel_fro(host(W2d), Wp2), rel_fro(host(HG2d), HGp2), rel_fro(host(Cd), Cp),
         rel_fro(host(HXd), HXp), rel_fro(t, t0))
    say("  rel fro W2 %.2e HG2 %.2e C %.2e HX %.2e sx %.2e" % e)
    assert max(e[:4]) <= 1e-5 and e[4] <= 1e-6


@pytest.mark.parametrize("m,n,ko,ki", [(256, 384, 128, 64), (64, 96, 1, 1), (128, 4096, 64, 4096)])
def test_unrotate_sx(m, n, ko, ki):
    say("unrotate with S_X", m, n, ko, ki)
    W, HX, HG, si, so = _case(m, n, 99)
    if ki == 1:
        si = np.ones(n, dtype=np.float32)
    if ko == 1:
        so = np.ones(m, dtype=np.float32)
    sid = None if ki == 1 else to_dev_f32(si)
    sod = None if ko == 1 else to_dev_f32(so)
    Wd = to_dev_f32(W)
    sg, sx = kq.kronq_biip_rotate_sx(Wd, to_dev_f32(HX), to_dev_f32(HG), sid, ki, sod, ko, 0.25, 0.25)
    kq.kronq_biip_unrotate_sx(Wd, sid, ki, sod, ko, sg, sx)
    e0 = rel_fro(host(Wd), W)
    M = synth.matrix(synth.NORMAL, 100, m, n, p1=0.05, dtype="f32")
    Md = to_dev_f32(M)
    kq.kronq_biip_unrotate_sx(Md, sid, ki, sod, ko, sg, sx)
    want = O.unrotate_sx(M.astype(np.float64), si, ki, so, ko, host(sg).astype(np.float64),
                         host(sx).astype(np.float64))
    e1 = rel_fro(host(Md), want)
    say("  round trip %.2e, inverse vs oracle %.2e" % (e0, e1))
    assert e0 <= 1e-5 and e1 <= 1e-5


def test_decode_with_input_rescale():
    """The deploy decode of a layer rescaled on the input side: the input-side
    factor D_in / s_x in the signs slot gives y = S_G^-1 U^T W'^ V S_X^-1 x, the
    dense product of the un-rotated quantized layer."""
    say("decode with S_X")
    m, n, bits, ki, ko = 128, 256, 4, 64, 32
    v = synth.matrix(synth.INT, 101, m, n, p1=64.0, dtype="f64")
    codes = np.mod(v, 16).astype(np.uint8)
    scales = (np.exp(synth.matrix(synth.NORMAL, 102, m, 1, p1=0.3, dtype="f64")) * 1e-3).astype(np.float32)
    zeros = np.full((m, 1), 7.0, dtype=np.float32)
    si, so = synth.signs(103, n), synth.signs(104, m)
    sg = np.exp(synth.matrix(synth.NORMAL, 105, 1, m, p1=0.5, dtype="f64")[0]).astype(np.float32)
    sx = np.exp(synth.matrix(synth.NORMAL, 106, 1, n, p1=0.5, dtype="f64")[0]).astype(np.float32)
    x = synth.matrix(synth.ACT_T4, 107, 1, n, dtype="f32")[0]
    packed = O.pack_codes(codes, bits)
    fac = (si / sx).astype(np.float32)
    y = kq.kronq_decode_matvec(torch.from_numpy(np.ascontiguousarray(packed)).to(DEV), n, bits, 0,
                               to_dev_f32(scales), to_dev_f32(zeros), to_dev_f32(fac), ki,
                               to_dev_f32(so), ko, to_dev_f32(sg), to_dev_f32(x))
    Wq = O.dequant(codes.astype(np.int64), scales.astype(np.float64), zeros.astype(np.float64), 0)
    dense = O.unrotate_sx(Wq, si, ki, so, ko, sg.astype(np.float64), sx.astype(np.float64))
    e = rel_fro(host(y), dense @ x.astype(np.float64))
    say("  rel fro %.2e" % e)
    assert e <= 1e-5
