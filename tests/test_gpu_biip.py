"""Parity of kronq_biip_rotate (S_G rescale + randomized block Hadamard on
both sides of W, H_X and H_G) with the oracle on the same fp32 inputs."""
import numpy as np
import pytest
import torch

import post_quantization_02_amd as kq
import synth
from synth import workloads as WL
from oracle import kronq_oracle as O
from gpu_helpers import DEV, host, rel_fro, say, spd_from_gram, to_dev_f32

pytestmark = pytest.mark.gpu


def _case(m, n, seed):
    W = synth.matrix(synth.NORMAL, seed, m, n, p1=0.02, dtype="f32")
    HX = spd_from_gram(seed + 1, n).astype(np.float32)
    G = synth.matrix(synth.GRAD_LOGNORMAL, seed + 2, 4 * m, m, p1=2.0, dtype="f64")
    HG = O.gram(G).astype(np.float32)
    si = synth.signs(seed + 3, n)
    so = synth.signs(seed + 4, m)
    return W, HX, HG, si, so


@pytest.mark.parametrize("m,n,ko,ki,alpha", [
    (384, 352, 128, 32, 0.25),      # several blocks both sides
    (256, 256, 256, 256, 0.25),     # one full block per side
    (64, 4096, 64, 4096, 0.25),     # wide input block (two passes on the row side)
    (512, 96, 8, 32, 0.5),          # small blocks
    (128, 1376, 128, 32, 0.25),     # 43 blocks on the input side
    (96, 64, 1, 2, 0.25),           # block 1 (no mixing) on the output side
    (24, 6, 8, 2, 0.25),            # width not a multiple of 4: every matrix on the scalar kernels
    (16, 16, 16, 16, 0.25),         # three tiles in all: most persistent workgroups have none
])
def test_biip_small(m, n, ko, ki, alpha):
    say("biip", m, n, ko, ki, alpha)
    W, HX, HG, si, so = _case(m, n, 21)
    Wd, HXd, HGd = to_dev_f32(W), to_dev_f32(HX), to_dev_f32(HG)
    sg = torch.empty(m, dtype=torch.float32, device=DEV)
    kq.kronq_biip_rotate(Wd, HXd, HGd, to_dev_f32(si), ki, to_dev_f32(so), ko, alpha, sg)
    Wp, HXp, HGp, s = O.biip(W.astype(np.float64), HX.astype(np.float64), HG.astype(np.float64),
                             si, ki, so, ko, alpha)
    e = (rel_fro(host(Wd), Wp), rel_fro(host(HXd), HXp), rel_fro(host(HGd), HGp), rel_fro(host(sg), s))
    say("  rel fro W %.2e HX %.2e HG %.2e sg %.2e" % e)
    assert max(e[:3]) <= 1e-5 and e[3] <= 1e-6


def test_biip_optional_factors():
    say("biip HX=None, HG=None with alpha=0")
    m, n = 128, 256
    W, HX, HG, si, so = _case(m, n, 31)
    Wd = to_dev_f32(W)
    kq.kronq_biip_rotate(Wd, None, None, to_dev_f32(si), 64, to_dev_f32(so), 32, 0.0)
    Wp, _, _, _ = O.biip(W.astype(np.float64), None, None, si, 64, so, 32, 0.0)
    assert rel_fro(host(Wd), Wp) <= 1e-5


def test_biip_leading_dimension():
    say("biip ldw > n")
    m, n = 128, 256
    W, HX, HG, si, so = _case(m, n, 41)
    big = np.zeros((m, n + 64), dtype=np.float32)
    big[:, :n] = W
    bd = to_dev_f32(big)
    kq.kronq_biip_rotate(bd[:, :n], None, to_dev_f32(HG), to_dev_f32(si), 128, to_dev_f32(so), 64, 0.25)
    out = host(bd)
    Wp, _, _, _ = O.biip(W.astype(np.float64), None, HG.astype(np.float64), si, 128, so, 64, 0.25)
    assert rel_fro(out[:, :n], Wp) <= 1e-5
    assert np.all(out[:, n:] == 0)


def test_biip_full_size_llama2_7b_q_proj():
    w = WL.C2
    say("biip full size", w.name)
    m = n = 4096
    W = w.w_f32("q_proj")
    HX = spd_from_gram(51, n, N=8192).astype(np.float32)
    G = synth.matrix(synth.GRAD_LOGNORMAL, 52, 8192, m, p1=2.0, dtype="f64")
    HG = O.gram(G).astype(np.float32)
    si, so = w.in_signs("x"), w.out_signs("q_proj")
    Wd, HXd, HGd = to_dev_f32(W), to_dev_f32(HX), to_dev_f32(HG)
    kq.kronq_biip_rotate(Wd, HXd, HGd, to_dev_f32(si), 4096, to_dev_f32(so), 4096, 0.25)
    Wp, HXp, HGp, _ = O.biip(W.astype(np.float64), HX.astype(np.float64), HG.astype(np.float64),
                             si, 4096, so, 4096, 0.25)
    e = (rel_fro(host(Wd), Wp), rel_fro(host(HXd), HXp), rel_fro(host(HGd), HGp))
    say("  rel fro W %.2e HX %.2e HG %.2e" % e)
    assert max(e) <= 1e-5


def test_biip_per_matrix_passes_wide_strips():
    """Above the merged passes' tile limit every matrix runs its own two
    launches, and pass 2 takes 2^15-element tiles where a 2^14 tile would leave
    strips under 128 bytes: here W (8192 x 4096, row block 8192: strips of 32
    bytes become 64), H_X (4096^2: 64 -> 128 bytes) and H_G (8192^2: 16 -> 32
    bytes).  Element by element against the oracle."""
    m, n = 8192, 4096
    say("biip per-matrix passes, wide pass-2 strips", m, n)
    W, HX, HG, si, so = _case(m, n, 61)
    Wd, HXd, HGd = to_dev_f32(W), to_dev_f32(HX), to_dev_f32(HG)
    kq.kronq_biip_rotate(Wd, HXd, HGd, to_dev_f32(si), 4096, to_dev_f32(so), 8192, 0.25)
    Wp, HXp, HGp, _ = O.biip(W.astype(np.float64), HX.astype(np.float64), HG.astype(np.float64),
                             si, 4096, so, 8192, 0.25)
    e = (rel_fro(host(Wd), Wp), rel_fro(host(HXd), HXp), rel_fro(host(HGd), HGp))
    say("  rel fro W %.2e HX %.2e HG %.2e" % e)
    assert max(e) <= 1e-5
    # the same call with W in a buffer of a padded leading dimension (still
    # the per-matrix passes): the padding is left untouched and every result
    # equals the dense call's bit for bit
    buf = torch.full((m, n + 64), 7.0, dtype=torch.float32, device=DEV)
    Wv = buf[:, :n]
    Wv.copy_(to_dev_f32(W))
    HXv, HGv = to_dev_f32(HX), to_dev_f32(HG)
    kq.kronq_biip_rotate(Wv, HXv, HGv, to_dev_f32(si), 4096, to_dev_f32(so), 8192, 0.25)
    assert torch.equal(Wv, Wd) and torch.equal(HXv, HXd) and torch.equal(HGv, HGd)
    assert bool((buf[:, n:] == 7.0).all())
