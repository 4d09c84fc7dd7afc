"""Shared helpers of the GPU parity tests (test infrastructure)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth
from oracle import kronq_oracle as O

DEV = "cuda:0"


def say(*a):
    """Name the case before each GPU step (flushed) so a failing run says where."""
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)


def to_dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def rel_fro(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def spd_from_gram(rng_seed: int, n: int, N: int = None, outliers: int = 3) -> np.ndarray:
    """A realistic H_X: Gram of synthetic heavy-tailed rows (fp64)."""
    N = N or 4 * n
    x = synth.matrix(synth.ACT_T4, rng_seed, N, n, outliers=np.arange(outliers) * 7 % n,
                     out_factor=20.0, dtype="f64")
    return O.gram(x)


class TeacherForcing:
    """Compare GPU codes/params with the oracle's loop on the same inputs.

    A code may differ only by one step and only when the oracle's pre-round
    value lies within `tie` grid units of the rounding boundary between the two
    codes; then the oracle adopts the GPU code (counted as a tie mismatch) so
    that both continue from the same state.  Any other difference is a hard
    mismatch.  Zero points follow the same rule on -min/scale."""

    def __init__(self, codes_gpu, scales_gpu, zeros_gpu, perm, tie=1e-5, rows=None):
        self.codes = np.asarray(codes_gpu, dtype=np.float64)   # natural order, rows subset
        self.scales = np.asarray(scales_gpu, dtype=np.float64)
        self.zeros = np.asarray(zeros_gpu, dtype=np.float64)
        self.perm = np.asarray(perm)
        self.tie = tie
        self.ties = 0
        self.hard = 0
        self.scale_err = 0.0
        self.hard_where = []

    def codes_hook(self, j, t, q):
        g = self.codes[:, self.perm[j]]
        diff = g != q
        if not diff.any():
            return q
        lo = np.minimum(g, q)
        near = (np.abs(g - q) == 1) & (np.abs(t - (lo + 0.5)) <= self.tie)
        self.ties += int(np.sum(diff & near))
        bad = diff & ~near
        if bad.any():
            self.hard += int(np.sum(bad))
            if len(self.hard_where) < 5:
                r = int(np.argmax(bad))
                self.hard_where.append((j, r, float(t[r]), float(q[r]), float(g[r])))
        return np.where(diff & near, g, q)

    def params_hook(self, gidx, scale, zero, zt):
        gs, gz = self.scales[:, gidx], self.zeros[:, gidx]
        self.scale_err = max(self.scale_err, float(np.max(np.abs(gs - scale) / np.abs(scale))))
        diff = gz != zero
        if diff.any():
            lo = np.minimum(gz, zero)
            near = (np.abs(gz - zero) == 1) & (np.abs(zt - (lo + 0.5)) <= self.tie)
            self.ties += int(np.sum(diff & near))
            self.hard += int(np.sum(diff & ~near))
            zero = np.where(diff & near, gz, zero)
        return scale, zero
