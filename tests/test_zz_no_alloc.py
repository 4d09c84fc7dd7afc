"""The decode entry point that allocates nothing (kronq_decode_matvec_noalloc,
for callers under graph capture or in serving loops): on two calls in a row,
the second smaller, it returns what kronq_decode_matvec returns with a
caller workspace, bit for bit (the same kernels over the same inputs; that
entry point is itself held to the oracle by the codec tests), and the oracle's
decode within the codec tolerance; a captured graph of it replays the eager
result."""
import numpy as np
import pytest
import torch

import post_quantization_02_amd as kq
import synth
from oracle import kronq_oracle as O
from gpu_helpers import DEV, host, rel_fro, say, to_dev_f32

pytestmark = pytest.mark.gpu


def _case(seed, m, n, bits, group, ki, ko):
    ng = n // group
    codes = np.mod(synth.matrix(synth.INT, seed, m, n, p1=float(4 << bits), dtype="f64"),
                   1 << bits).astype(np.uint8)
    packed = O.pack_codes(codes, bits)
    ldp = (packed.shape[1] + 15) // 16 * 16
    buf = np.zeros((m, ldp), dtype=np.uint8)
    buf[:, :packed.shape[1]] = packed
    scales = (np.abs(synth.matrix(synth.NORMAL, seed + 1, m, ng, p1=1e-2, dtype="f32")) + 1e-3)
    zeros = np.mod(synth.matrix(synth.INT, seed + 2, m, ng, p1=64.0, dtype="f64"),
                   1 << bits).astype(np.float32)
    si, so = synth.signs(seed + 3, n), synth.signs(seed + 4, m)
    sg = np.exp(synth.matrix(synth.NORMAL, seed + 5, 1, m, p1=0.3, dtype="f64")[0]).astype(np.float32)
    x = synth.matrix(synth.NORMAL, seed + 6, 1, n, p1=1.0, dtype="f32")[0]
    want = O.decode_matvec(packed, bits, n, scales, zeros, group, si, ki, so, ko, sg, x)
    dev = dict(codes=torch.from_numpy(buf).to(DEV), scales=to_dev_f32(scales), zeros=to_dev_f32(zeros),
               si=to_dev_f32(si), so=to_dev_f32(so), sg=to_dev_f32(sg), x=to_dev_f32(x))
    return dev, want


def _both(d, n, bits, group, ki, ko):
    m = d["codes"].shape[0]
    y_ws = kq.kronq_decode_matvec(d["codes"], n, bits, group, d["scales"], d["zeros"], d["si"], ki,
                                  d["so"], ko, d["sg"], d["x"])
    y_na = torch.full((m,), float("nan"), dtype=torch.float32, device=DEV)
    kq.kronq_decode_matvec_noalloc(d["codes"], n, bits, group, d["scales"], d["zeros"], d["si"], ki,
                                   d["so"], ko, d["sg"], d["x"], y_na)
    return host(y_ws), host(y_na)


def test_noalloc_matches_the_workspace_entry_point_twice():
    lib = kq.load()
    assert lib.kronq_decode_noalloc_max_bytes() == 4 << 20
    cases = [(4096, 4096, 4, 128, 4096, 4096),      # Llama-2-7B q_proj, 4 bits g128
             (1024, 2048, 2, 64, 2048, 1024)]       # then a smaller layer, 2 bits g64
    for k, (m, n, bits, group, ki, ko) in enumerate(cases):
        say("noalloc decode call", k + 1, m, n, bits, group)
        assert lib.kronq_decode_ws(m, n, bits) <= lib.kronq_decode_noalloc_max_bytes()
        d, want = _case(900 + k, m, n, bits, group, ki, ko)
        y_ws, y_na = _both(d, n, bits, group, ki, ko)
        np.testing.assert_array_equal(y_na, y_ws)
        e = rel_fro(y_na, want)
        say("  rel fro vs oracle %.2e" % e)
        assert e <= 1e-5
        assert np.max(np.abs(y_na - want)) <= 1e-4 * np.max(np.abs(want))


def _stored(seed, m, n, bits, group, perm=False):
    """Random stored codes (any byte is a valid pack of 2- or 4-bit codes; one
    code a byte below 2^bits otherwise), grids, signs, S_G, x and an optional
    column permutation, on the device."""
    row = kq.kronq_packed_row_bytes(n, bits)
    ldp = (row + 15) // 16 * 16
    top = 256 if bits in (2, 4) else 1 << bits
    raw = np.mod(synth.matrix(synth.INT, seed, m, ldp, p1=1024.0, dtype="f64"), top).astype(np.uint8)
    raw[:, row:] = 0
    ng = 1 if group <= 0 else n // group
    d = dict(codes=torch.from_numpy(raw).to(DEV),
             scales=to_dev_f32(np.abs(synth.matrix(synth.NORMAL, seed + 1, m, ng, p1=1e-2, dtype="f32")) + 1e-3),
             zeros=to_dev_f32(np.mod(synth.matrix(synth.INT, seed + 2, m, ng, p1=64.0, dtype="f64"),
                                     1 << bits).astype(np.float32)),
             si=to_dev_f32(synth.signs(seed + 3, n)), so=to_dev_f32(synth.signs(seed + 4, m)),
             sg=to_dev_f32(np.exp(synth.matrix(synth.NORMAL, seed + 5, 1, m, p1=0.3, dtype="f64")[0])
                           .astype(np.float32)),
             x=to_dev_f32(synth.matrix(synth.ACT_T4, seed + 6, 1, n, dtype="f32")[0]), perm=None)
    if perm:
        keys = synth.matrix(synth.NORMAL, seed + 7, 1, n, dtype="f64")[0]
        d["perm"] = torch.from_numpy(np.argsort(-keys, kind="stable").astype(np.int32)).to(DEV)
    return d


@pytest.mark.parametrize("m,n,bits,group,ko,ki,extra", [
    (4096, 4096, 4, 0, 4096, 4096, ""),       # one grid per row, 32 rows a workgroup
    (4096, 11008, 3, 0, 4096, 256, ""),       # one code a byte, 43 input blocks
    (14336, 4096, 4, 128, 2048, 4096, ""),    # last output tile half full
    (11008, 4096, 2, 64, 256, 4096, ""),      # last output tile 2816 rows
    (8192, 1024, 4, 128, 8192, 1024, ""),     # output tile of 8192 rows (past the registers)
    (40000, 1024, 4, 128, 64, 1024, ""),      # ten output tiles
    (100, 200, 4, 0, 4, 8, ""),               # 8 rows a workgroup, ragged rows
    (33, 1000, 2, 0, 1, 8, "no_out_signs"),   # block 1 and no signs on the output side
    (7, 192, 8, 64, 1, 64, "no_sg"),          # one output tile of 8 rows, no S_G
    (1, 64, 4, 64, 1, 64, ""),                # tile of one row: output stage launched apart
    (4096, 11008, 4, 128, 4096, 256, "perm"), # codes in processing order
])
def test_noalloc_matches_the_workspace_entry_point_across_shapes(m, n, bits, group, ko, ki, extra):
    """Bit for bit the workspace entry point's result over the decode's shape
    cases: grid sizes, ragged last tiles, tiles wider than the registers hold,
    NULL output signs or S_G, and the case whose output stage is not fused."""
    say("noalloc decode", m, n, bits, group, ko, ki, extra)
    d = _stored(950 + m % 97 + bits, m, n, bits, group, perm=extra == "perm")
    so = None if extra == "no_out_signs" else d["so"]
    sg = None if extra == "no_sg" else d["sg"]
    args = (d["codes"], n, bits, group, d["scales"], d["zeros"], d["si"], ki, so, ko, sg, d["x"])
    y_ws = kq.kronq_decode_matvec(*args, perm=d["perm"])
    for rep in range(2):
        y_na = torch.full((m,), float("nan"), dtype=torch.float32, device=DEV)
        kq.kronq_decode_matvec_noalloc(*args, y_na, perm=d["perm"])
        np.testing.assert_array_equal(host(y_na), host(y_ws))


def test_noalloc_too_large_is_enomem():
    # 8-bit codes keep 1024 columns a slice: 8 slices x 140000 rows of partial
    # sums exceed the 4 MiB buffer; rejected before anything is launched
    say("noalloc decode ENOMEM")
    m, n, bits = 140000, 8192, 8
    assert kq.load().kronq_decode_ws(m, n, bits) > kq.load().kronq_decode_noalloc_max_bytes()
    codes = torch.empty((m, n), dtype=torch.uint8, device=DEV)
    f = torch.empty(m, dtype=torch.float32, device=DEV)
    s = torch.ones(n, dtype=torch.float32, device=DEV)
    with pytest.raises(kq.KronqError) as e:
        kq.kronq_decode_matvec_noalloc(codes, n, bits, -1, f, f, s, n, f, 1, None, s, f)
    assert e.value.status == kq.KRONQ_ENOMEM


def test_noalloc_graph_replay():
    say("noalloc decode in a HIP graph")
    m, n, bits, group, ki, ko = 2048, 4096, 4, 128, 4096, 2048
    d, _ = _case(930, m, n, bits, group, ki, ko)
    y = torch.empty(m, dtype=torch.float32, device=DEV)

    def call():
        kq.kronq_decode_matvec_noalloc(d["codes"], n, bits, group, d["scales"], d["zeros"], d["si"], ki,
                                       d["so"], ko, d["sg"], d["x"], y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                                   # first call outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        d["x"].copy_(to_dev_f32(synth.matrix(synth.NORMAL, 940 + rep, 1, n, p1=1.0, dtype="f32")[0]))
        g.replay()
        torch.cuda.synchronize()
        got = host(y).copy()
        ref = kq.kronq_decode_matvec(d["codes"], n, bits, group, d["scales"], d["zeros"], d["si"], ki,
                                     d["so"], ko, d["sg"], d["x"])
        np.testing.assert_array_equal(got, host(ref))
