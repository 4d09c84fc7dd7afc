"""Workload definitions: shapes, distributions and quantizer settings of the five
synthetic configurations, plus scaled-down variants for fast parity tests.

Stand-ins (no real data is available): the calibration set of the pages is 128
WikiText-2 sequences of 2048 tokens, i.e. N = 262144 token rows; X rows are
heavy-tailed activations with a few outlier input channels, G rows are output
gradients whose channel scales are log-normal (the pages show diag(H_G) varying
by orders of magnitude across output channels).  This module only names the
recipe; the numbers come from ``synth`` (its C generator).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

import synth


@dataclass(frozen=True)
class InputSpec:
    name: str
    n: int               # channels (columns of X)
    kind: int            # synth.ACT_NORMAL or synth.ACT_T4
    n_outliers: int
    factor: float


@dataclass(frozen=True)
class Sublayer:
    name: str
    m: int               # output channels (rows of W)
    n: int               # input channels (columns of W)
    x: str               # InputSpec name
    in_block: int        # Hadamard block on the input side (n = in_block * k)
    out_block: int       # Hadamard block on the output side
    bits: int            # 0: decided by the bit allocation
    group: int           # <= 0: per-channel
    act_order: bool = False


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    N: int                               # calibration tokens
    dtype: str                           # "f32" or "bf16" storage of X, G, W
    inputs: tuple
    sublayers: tuple
    alpha: float = 0.25
    lam: float = 0.01
    block: int = 128
    avg_bits: float | None = None        # budget of the bit allocation, if any
    grad_sigma: float = 2.0
    w_std: float = 0.02
    drift: float = 0.05                  # relative size of the full-precision inputs' drift
    description: str = ""

    # ---- seeds: one per tensor, derived from the workload seed ----
    def input_index(self, xname: str) -> int:
        return [s.name for s in self.inputs].index(xname)

    def sub_index(self, sname: str) -> int:
        return [s.name for s in self.sublayers].index(sname)

    def x_seed(self, xname): return self.seed * 1000 + 10 + self.input_index(xname)
    def g_seed(self, sname): return self.seed * 1000 + 100 + self.sub_index(sname)
    def w_seed(self, sname): return self.seed * 1000 + 200 + self.sub_index(sname)
    def in_sign_seed(self, xname): return self.seed * 1000 + 300 + self.input_index(xname)
    def out_sign_seed(self, sname): return self.seed * 1000 + 400 + self.sub_index(sname)

    def input(self, xname) -> InputSpec:
        return self.inputs[self.input_index(xname)]

    def sub(self, sname) -> Sublayer:
        return self.sublayers[self.sub_index(sname)]

    # ---- generation (host, numpy) ----
    def outliers(self, xname):
        spec = self.input(xname)
        return synth.outlier_channels(self.x_seed(xname), spec.n, spec.n_outliers)

    def gen_x(self, xname, r0=0, nr=None, c0=0, nc=None, dtype=None, out=None):
        spec = self.input(xname)
        return synth.matrix(spec.kind, self.x_seed(xname), self.N, spec.n, r0=r0, nr=nr, c0=c0,
                            nc=nc, outliers=self.outliers(xname), out_factor=spec.factor,
                            dtype=dtype or self.dtype, out=out)

    def gen_g(self, sname, r0=0, nr=None, c0=0, nc=None, dtype=None, out=None):
        s = self.sub(sname)
        return synth.matrix(synth.GRAD_LOGNORMAL, self.g_seed(sname), self.N, s.m, r0=r0, nr=nr,
                            c0=c0, nc=nc, p1=self.grad_sigma, dtype=dtype or self.dtype, out=out)

    def gen_xfp(self, xname, r0=0, nr=None, c0=0, nc=None, dtype=None, out=None):
        """Inputs of the full-precision model next to gen_x's (the inputs of a
        partly quantized model): the same activations plus a drift of relative
        size `drift` per channel, each rounded on its own."""
        spec = self.input(xname)
        return synth.matrix(synth.ACT_T4_DRIFT, self.x_seed(xname), self.N, spec.n, r0=r0, nr=nr,
                            c0=c0, nc=nc, p1=self.drift, outliers=self.outliers(xname),
                            out_factor=spec.factor, dtype=dtype or self.dtype, out=out)

    # ---- generation in device memory (large inputs; torch tensors) ----
    def gen_x_dev(self, xname, device="cuda:0"):
        spec = self.input(xname)
        return synth.matrix_dev(spec.kind, self.x_seed(xname), self.N, spec.n,
                                outliers=self.outliers(xname), out_factor=spec.factor,
                                dtype=self.dtype, device=device)

    def gen_xfp_dev(self, xname, device="cuda:0"):
        spec = self.input(xname)
        return synth.matrix_dev(synth.ACT_T4_DRIFT, self.x_seed(xname), self.N, spec.n, p1=self.drift,
                                outliers=self.outliers(xname), out_factor=spec.factor,
                                dtype=self.dtype, device=device)

    def gen_g_dev(self, sname, device="cuda:0"):
        s = self.sub(sname)
        return synth.matrix_dev(synth.GRAD_LOGNORMAL, self.g_seed(sname), self.N, s.m,
                                p1=self.grad_sigma, dtype=self.dtype, device=device)

    def gen_w(self, sname, dtype=None, r0=0, nr=None, c0=0, nc=None):
        s = self.sub(sname)
        return synth.matrix(synth.NORMAL, self.w_seed(sname), s.m, s.n, r0=r0, nr=nr, c0=c0, nc=nc,
                            p1=self.w_std, dtype=dtype or self.dtype)

    def w_f32(self, sname) -> np.ndarray:
        """W as float32 (bf16 storage widened exactly)."""
        w = self.gen_w(sname)
        return synth.bf16_to_f32(w) if self.dtype == "bf16" else w.astype(np.float32)

    def in_signs(self, xname):
        return synth.signs(self.in_sign_seed(xname), self.input(xname).n)

    def out_signs(self, sname):
        return synth.signs(self.out_sign_seed(sname), self.sub(sname).m)

    def n_params(self):
        return [s.m * s.n for s in self.sublayers]


def _ceil_pct(n):
    return int(math.ceil(0.01 * n - 1e-9))


def _t4(name, n):
    return InputSpec(name, n, synth.ACT_T4, _ceil_pct(n), 50.0)


C1 = Workload(
    "tiny_linear_256", 1, 2048, "f32",
    (InputSpec("x", 256, synth.ACT_NORMAL, 4, 20.0),),
    (Sublayer("linear", 256, 256, "x", 256, 256, 4, -1),),
    description="tiny single linear layer, fp32: W 256x256, X/G 2048x256, W4 per-channel")

C2 = Workload(
    "llama2_7b_q_proj", 2, 262144, "bf16",
    (_t4("x", 4096),),
    (Sublayer("q_proj", 4096, 4096, "x", 4096, 4096, 2, 128),),
    description="Llama-2-7B q_proj shape: W 4096x4096, X/G 262144x4096 bf16, W2 g128")

C3 = Workload(
    "llama2_7b_down_proj", 3, 262144, "bf16",
    (_t4("x", 11008),),
    (Sublayer("down_proj", 4096, 11008, "x", 256, 4096, 3, -1, True),),
    description="Llama-2-7B down_proj: W 4096x11008, in block-Hadamard 43x256, W3 per-channel, "
                "act-order")

C4 = Workload(
    "llama3_8b_block", 4, 262144, "bf16",
    (_t4("attn_in", 4096), _t4("o_in", 4096), _t4("mlp_in", 4096), _t4("down_in", 14336)),
    (Sublayer("q_proj", 4096, 4096, "attn_in", 4096, 4096, 0, 128),
     Sublayer("k_proj", 1024, 4096, "attn_in", 4096, 1024, 0, 128),
     Sublayer("v_proj", 1024, 4096, "attn_in", 4096, 1024, 0, 128),
     Sublayer("o_proj", 4096, 4096, "o_in", 4096, 4096, 0, 128),
     Sublayer("gate_proj", 14336, 4096, "mlp_in", 4096, 2048, 0, 128),
     Sublayer("up_proj", 14336, 4096, "mlp_in", 4096, 2048, 0, 128),
     Sublayer("down_proj", 4096, 14336, "down_in", 2048, 4096, 0, 128)),
    avg_bits=3.0,
    description="Llama-3-8B decoder block, 7 sublayers, bits {2,3,4} allocated to a 3.0 average")

C5 = Workload(
    "llama3_70b_mlp", 5, 262144, "bf16",
    (_t4("gate_in", 8192), _t4("down_in", 28672)),
    (Sublayer("gate_proj", 28672, 8192, "gate_in", 8192, 4096, 2, 128),
     Sublayer("down_proj", 8192, 28672, "down_in", 4096, 8192, 2, 128)),
    description="Llama-3-70B MLP: gate 28672x8192, down 8192x28672, W2 g128")

ALL = (C1, C2, C3, C4, C5)
BY_NAME = {w.name: w for w in ALL}


def scaled(w: Workload, *, N: int, div: int, name: str | None = None) -> Workload:
    """Same recipe with every channel count divided by `div` (blocks too, floor 16)
    and N tokens: the small parity cases that the oracle finishes in seconds."""
    ins = tuple(InputSpec(s.name, s.n // div, s.kind, max(1, _ceil_pct(s.n // div)), s.factor)
                for s in w.inputs)
    subs = tuple(Sublayer(s.name, s.m // div, s.n // div, s.x, max(16, s.in_block // div),
                          max(16, s.out_block // div), s.bits, s.group, s.act_order)
                 for s in w.sublayers)
    return Workload(name or (w.name + "_div%d" % div), w.seed, N, w.dtype, ins, subs, w.alpha,
                    w.lam, w.block, w.avg_bits, w.grad_sigma, w.w_std, w.drift, w.description)
