"""Benchmark of the KronQ per-sublayer quantization path on one MI355X.

One step = the whole hot path for every sublayer of the workload, inputs
resident in HBM; per sublayer:
  H_X = X^T X / N, H_G = G^T G / N            (kronq_gram x 2, bf16 matrix cores)
  BiIP: S_G rescale + Hadamard both sides      (kronq_biip_rotate)
  sensitivity tr(H_X') tr(H_G')                (kronq_sensitivity)
  damping + inverse Cholesky factor            (kronq_chol_inv, synchronizes)
  column-wise OBS quantize-and-compensate      (kronq_gptq_quantize)
Workload: the Llama-3-70B MLP -- gate_proj W 28672 x 8192 (X 262144 x 8192,
G 262144 x 28672) and down_proj W 8192 x 28672 (X 262144 x 28672, G 262144 x
8192), bf16 calibration rows (128 sequences x 2048 tokens), 2-bit asymmetric
groups of 128, block-Hadamard 7 x 4096 on the 28672-wide sides and 8192 on the
others, alpha 0.25, damping 1% of the mean diagonal, fp32 Cholesky of the
28672 x 28672 H_X.  Synthetic inputs (heavy-tailed activations with outlier
channels, log-normal gradient channel scales) generated in device memory stand
in for the calibration set.  The Llama-2-7B q_proj workload (4096 x 4096) is
timed the same way as a secondary object of the line.

Prints one JSON line.  `value` is the mean wall time of one sublayer
quantization (seconds, lower is better): the wall time of a step divided by the
number of sublayers.  Per-stage times come from HIP events recorded on the
stream the kernels run on; `roofline` is for the Gram kernel launch at
d = 28672 (the dominant kernel).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6
PEAK_FP32_TFLOPS = 157.3
PEAK_FP64_TFLOPS = 78.6
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the Llama-2-7B q_proj secondary object (and the weight CV figures)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the batch-1 decode measurement of the deploy codec")
    ap.add_argument("--decode-only", action="store_true",
                    help="run only the decode measurement (prints its own JSON line)")
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--configs", action="store_true",
                    help="only time every sublayer of the other workloads (tiny linear, Llama-2-7B "
                         "down_proj, Llama-3-8B block, Llama-3-70B MLP; prints its own JSON line)")
    ap.add_argument("--config-steps", type=int, default=2, help="timed steps per sublayer (--configs)")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0,
                    help="approximate CPU seconds for the oracle baseline sample")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "gram_bf16_llama3_70b_mlp_traffic.json"))
    ap.add_argument("--copy-probe", type=int, metavar="BYTES", default=0,
                    help="only run a plain device copy of BYTES five times (calibrates the HBM byte "
                         "counters) and exit")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                             "COPY_WRITE_CSV"),
                    help="only turn four rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE and "
                         "WRITE_SIZE of this benchmark, then of --copy-probe) into the traffic file "
                         "(--traffic-json) and exit")
    ap.add_argument("--library-gram", metavar="D[,D...]", default="",
                    help="only time kronq_gram against the vendor GEMM (torch.mm, hipBLASLt) on the "
                         "same bf16 262144 x D operand, for each D, and exit")
    ap.add_argument("--copy-bytes", type=int, default=256 * 1024 * 1024,
                    help="BYTES the copy-probe runs used (for --summarize-traffic)")
    return ap.parse_args()


GRAM_SRC = os.path.join(ROOT, "post_quantization_02_amd", "csrc", "gram.hip")
GRAM_MAIN = "gram_bf16_lds"          # gram_bf16_lds_kernel and its persistent one-split variant


def gram_source_hash():
    import hashlib
    with open(GRAM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def copy_probe(nbytes):
    """Plain device-to-device copy of a known size, five times."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "copies": 5}), flush=True)


def library_gram(dims, reps=3):
    """kronq_gram beside the vendor GEMM on one bf16 operand A (262144 x d):
    kronq_gram forms the unique triangle of A^T A (N d (d + 1) flops), torch.mm
    the full product of a transposed copy with A (2 N d^2 flops).  Both rates
    are useful flops per second, so equal rates mean equal efficiency."""
    import torch
    import post_quantization_02_amd as kq
    dev = torch.device("cuda:0")
    kq.load()
    N = 262144
    rows = []
    for d in dims:
        log("library gram d", d)
        g = torch.Generator(device=dev)
        g.manual_seed(d)
        A = torch.randn((N, d), device=dev, dtype=torch.bfloat16, generator=g)
        At = A.t().contiguous()
        H = torch.empty((d, d), dtype=torch.float32, device=dev)
        ws = torch.empty(kq.load().kronq_gram_ws(N, d, kq.KRONQ_BF16), dtype=torch.uint8, device=dev)

        def timed(fn):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        ms_k = timed(lambda: kq.kronq_gram(A, H, ws=ws))
        ms_l = timed(lambda: torch.mm(At, A))
        fk, fl = float(N) * d * (d + 1), 2.0 * N * d * d
        rows.append({"d": d, "N": N, "kronq_gram_ms": ms_k, "kronq_gram_tflops": fk / ms_k / 1e9,
                     "kronq_gram_frac": fk / ms_k / 1e9 / PEAK_BF16_TFLOPS, "torch_mm_ms": ms_l,
                     "torch_mm_tflops": fl / ms_l / 1e9,
                     "torch_mm_frac": fl / ms_l / 1e9 / PEAK_BF16_TFLOPS})
        log("  kronq_gram %.2f ms (%.0f TF/s)  torch.mm %.2f ms (%.0f TF/s)" %
            (ms_k, rows[-1]["kronq_gram_tflops"], ms_l, rows[-1]["torch_mm_tflops"]))
        del A, At, H, ws
        torch.cuda.empty_cache()
    print(json.dumps({"library_gram": rows, "reps": reps, "dtype": "bf16",
                      "data": "synthetic N(0,1) (seeded torch generator)"}), flush=True)


def _pmc_groups(path, kernel_pred, counter):
    """{(kernel, grid size): [per-dispatch counter sums]} for the matching kernels."""
    import csv
    per_dispatch = {}
    key_of = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and kernel_pred(r["Kernel_Name"]):
                key = r["Dispatch_Id"]
                per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
                name = r["Kernel_Name"].replace("(anonymous namespace)", "anon").split("(")[0].split("::")[-1]
                key_of[key] = (name, int(r.get("Grid_Size", 0) or 0))
    out = {}
    for k, v in per_dispatch.items():
        out.setdefault(key_of[k], []).append(v)
    return out


def _pmc_mean(path, kernel_pred, counter):
    vals = [v for vs in _pmc_groups(path, kernel_pred, counter).values() for v in vs]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def summarize_traffic(args):
    """HBM bytes per launch of the roofline kernel (the Gram at d = 28672 of the
    Llama-3-70B MLP step: the launches with the largest grid) from FETCH_SIZE /
    WRITE_SIZE (KiB per dispatch), each scaled so that the same counter over a
    plain copy of known size reads that size."""
    f_csv, w_csv, cf_csv, cw_csv = args.summarize_traffic
    copy = lambda k: "copyBuffer" in k
    cf, _ = _pmc_mean(cf_csv, copy, "FETCH_SIZE")
    cw, _ = _pmc_mean(cw_csv, copy, "WRITE_SIZE")
    kib = args.copy_bytes / 1024.0
    f_scale, w_scale = kib / cf, kib / cw
    out = {"counters": {}, "copy_probe": {"bytes": args.copy_bytes, "fetch_kib": cf, "write_kib": cw,
                                          "fetch_scale": f_scale, "write_scale": w_scale}}
    pred = lambda name: GRAM_MAIN in name
    fg = _pmc_groups(f_csv, pred, "FETCH_SIZE")
    wg = _pmc_groups(w_csv, pred, "WRITE_SIZE")
    for key in sorted(set(fg) & set(wg)):
        fk = sum(fg[key]) / len(fg[key])
        wk = sum(wg[key]) / len(wg[key])
        out["counters"]["%s grid %d" % key] = {
            "fetch_kib": fk, "write_kib": wk, "dispatches": len(fg[key]),
            "hbm_bytes_per_dispatch": (fk * f_scale + wk * w_scale) * 1024.0}
    # d = 28672: the launches that read the 14 GiB inputs fetch the most
    big = max(set(fg) & set(wg), key=lambda k: sum(fg[k]) / len(fg[k]))
    out["roofline_launch"] = "%s grid %d" % big
    out["bytes_per_launch"] = out["counters"]["%s grid %d" % big]["hbm_bytes_per_dispatch"]
    out["unit"] = "bytes per launch of the Gram at d = 28672 (scaled counters)"
    out["gram_source_sha256"] = gram_source_hash()
    run = "python3 -u bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-decode --no-secondary"
    probe = "python3 -u bench.py --copy-probe %d" % args.copy_bytes
    out["commands"] = {
        "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/fetch -o bench -- " + run,
        "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/write -o bench -- " + run,
        "copy_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/cfetch -o copy -- " + probe,
        "copy_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/cwrite -o copy -- " + probe,
        "summary": "python3 bench.py --summarize-traffic <dir>/fetch/bench_counter_collection.csv "
                   "<dir>/write/bench_counter_collection.csv <dir>/cfetch/copy_counter_collection.csv "
                   "<dir>/cwrite/copy_counter_collection.csv --traffic-json <out>",
    }
    with open(args.traffic_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s):
    """The oracle (numpy float64, as it stands) on a bounded sample of every
    sublayer of workload `w`, extrapolated to the whole step and reported per
    sublayer (the mean, like `value`):
      Gram: a token prefix of X and of G on their first 4096 columns (the Gram
            is linear in N and quadratic in d),
      BiIP: the two-sided rotation of a row slice of W (rows are independent on
            the input side; the output side is timed on a column slice), scaled
            by element count, then by (mn + n^2 + m^2) / (mn) for H_X and H_G,
      damping + inverse Cholesky: at n_s = min(n, 2048), scaled by (n / n_s)^3,
      column loop: a row sample (rows are independent), all columns."""
    import synth
    from oracle import kronq_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    N = w.N
    t0 = time.perf_counter()
    Np = 128
    stages = {"gram_x_g": 0.0, "biip": 0.0, "sensitivity": 0.0, "chol_inv": 0.0, "gptq": 0.0}
    notes = []
    for s in w.sublayers:
        m, n = s.m, s.n
        # Gram: Np tokens and the first ds columns (cost N d^2)
        dx, dg = min(n, 4096), min(m, 4096)
        xs = synth.bf16_to_f64(w.gen_x(s.x, r0=0, nr=Np, c0=0, nc=dx))
        gs = synth.bf16_to_f64(w.gen_g(s.name, r0=0, nr=Np, c0=0, nc=dg))
        t_g0 = time.perf_counter()
        HXs = O.gram(xs)
        t_x = (time.perf_counter() - t_g0) * (N / Np) * (n / dx) ** 2
        t_g0 = time.perf_counter()
        HGs = O.gram(gs)
        t_gg = (time.perf_counter() - t_g0) * (N / Np) * (m / dg) ** 2
        stages["gram_x_g"] += t_x + t_gg
        # BiIP: input side on a slice of rows, output side on a slice of columns
        rs = min(m, 512)
        cs = min(n, 512)
        Wr = synth.bf16_to_f64(w.gen_w(s.name, r0=0, nr=rs))
        Wc = synth.bf16_to_f64(w.gen_w(s.name, c0=0, nc=cs))
        t_b0 = time.perf_counter()
        O.rotate_rows(Wr, s.in_block, w.in_signs(s.x))
        t_in = (time.perf_counter() - t_b0) * (m / rs)
        t_b0 = time.perf_counter()
        O.rotate_cols(Wc, s.out_block, w.out_signs(s.name))
        t_out = (time.perf_counter() - t_b0) * (n / cs)
        stages["biip"] += (t_in + t_out) * (m * n + n * n + m * m) / (m * n)
        t_s0 = time.perf_counter()
        O.sensitivity(HXs, HGs)
        stages["sensitivity"] += time.perf_counter() - t_s0
        ns = min(dx, 2048)
        Hs = HXs[:ns, :ns] + np.eye(ns)
        t_c0 = time.perf_counter()
        perm, H = O.prepare_hessian(Hs, w.lam, s.act_order)
        Rs, _ = O.chol_inv_upper(H)
        stages["chol_inv"] += (time.perf_counter() - t_c0) * (n / ns) ** 3
        # column loop: two rows against an n x n upper factor
        rows = 2
        R = np.triu(np.full((n, n), 0.5 / np.sqrt(n))) + np.eye(n)
        t_q0 = time.perf_counter()
        O.gptq(Wr[:rows], R, np.arange(n), s.bits, s.group)
        stages["gptq"] += (time.perf_counter() - t_q0) * (m / rows)
        notes.append("%s %dx%d: Gram on the first %d of %d tokens and the first %d / %d columns "
                     "(x N/%d x (d/d_s)^2), W rotated on %d rows and %d columns, inverse Cholesky at "
                     "n=%d (x(n/%d)^3), column loop on %d rows (x%d)"
                     % (s.name, m, n, Np, N, dx, dg, Np, rs, cs, ns, ns, rows, m // rows))
        del Wr, Wc, R
    total = sum(stages.values())
    wall = time.perf_counter() - t0
    L = len(w.sublayers)
    return {
        "value": total / L, "unit": "s", "cores": int(cores), "kind": "oracle",
        "cpu_model": _cpu_model(),
        "sample": "%s, per sublayer (mean of %d): %s; float64 numpy, extrapolated; %.1f s of host time"
                  % (w.name, L, "; ".join(notes), wall),
        "stages_s_per_step": stages,
    }


# Batch-1 decode through every linear sublayer of a Llama-2-7B decoder stack
# (32 layers x q/k/v/o 4096x4096, gate/up 11008x4096, down 4096x11008) with
# 4-bit codes in groups of 128: one token = 224 kronq_decode_matvec calls,
# captured once in a HIP graph and replayed.  Hadamard blocks 4096 on 4096-wide
# sides, 256 on 11008-wide sides (43 blocks).
DECODE_SUBLAYERS = (("q_proj", 4096, 4096), ("k_proj", 4096, 4096), ("v_proj", 4096, 4096),
                    ("o_proj", 4096, 4096), ("gate_proj", 11008, 4096), ("up_proj", 11008, 4096),
                    ("down_proj", 4096, 11008))
# The same weights with the sublayers that read one input stacked row-wise
# (q/k/v: 12288 x 4096; gate/up: 22016 x 4096).  They share V and x'; the
# output transform of the stack is block-diagonal in the sublayers' own
# transforms because every output block lies inside one sublayer.
DECODE_STACKED = (("qkv_proj", 12288, 4096), ("o_proj", 4096, 4096),
                  ("gate_up_proj", 22016, 4096), ("down_proj", 4096, 11008))


def decode_leg(steps, warmup, n_layers=32, bits=4, group=128, sublayers=DECODE_SUBLAYERS,
               name="llama2_7b_linear_stack", noalloc=False):
    """noalloc: each call through kronq_decode_matvec_noalloc (the library's own
    partial-sum buffer) instead of kronq_decode_matvec with a caller workspace."""
    import torch
    import post_quantization_02_amd as kq
    dev = torch.device("cuda:0")
    lib = kq.load()
    gen = torch.Generator(device=dev)
    gen.manual_seed(20260)
    # Hadamard block of each side: 4096 on 4096-wide sides and on the q/k/v
    # stack (three 4096 blocks), 256 on 11008-wide sides and the gate/up stack
    blocks = {4096: 4096, 11008: 256, 12288: 4096, 22016: 256}
    blk = blocks.__getitem__

    def signs(d):
        return (torch.randint(0, 2, (d,), generator=gen, device=dev).float() * 2 - 1)

    dims = sorted({d for _, m, n in sublayers for d in (m, n)})
    sgn_in = {d: signs(d) for d in dims}
    sgn_out = {d: signs(d) for d in dims}
    sg = {d: torch.rand(d, generator=gen, device=dev) + 0.5 for d in dims}
    xs = {d: torch.randn(d, generator=gen, device=dev) for d in dims}
    ys = {d: torch.empty(d, device=dev) for d in dims}
    layers = []
    alg_bytes = 0
    for _ in range(n_layers):
        for _sub, m, n in sublayers:
            row = lib.kronq_packed_row_bytes(n, bits)
            ldp = (row + 15) // 16 * 16
            codes = torch.randint(0, 256, (m, ldp), dtype=torch.uint8, generator=gen, device=dev)
            ng = n // group
            scales = torch.rand((m, ng), generator=gen, device=dev) * 1e-2 + 1e-3
            zeros = torch.randint(0, 1 << bits, (m, ng), generator=gen, device=dev).float()
            layers.append((codes, m, n, scales, zeros))
            # codes, grids, x, y, signs both sides, S_G
            alg_bytes += m * row + 8 * m * ng + 4 * n + 4 * m + 4 * (n + m) + 4 * m
    ws = torch.empty(max(lib.kronq_decode_ws(m, n, bits) for _, m, n in sublayers),
                     dtype=torch.uint8, device=dev)

    def token():
        for codes, m, n, scales, zeros in layers:
            if noalloc:
                kq.kronq_decode_matvec_noalloc(codes, n, bits, group, scales, zeros, sgn_in[n], blk(n),
                                               sgn_out[m], blk(m), sg[m], xs[n], ys[m])
            else:
                kq.kronq_decode_matvec(codes, n, bits, group, scales, zeros, sgn_in[n], blk(n),
                                       sgn_out[m], blk(m), sg[m], xs[n], y=ys[m], ws=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        token()                        # eager warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        token()
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # the same token issued eagerly (one host call per sublayer)
    t0 = time.perf_counter()
    for _ in range(3):
        token()
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / 3
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    return {"workload": "%s_w%dg%d_batch1" % (name, bits, group),
            "sublayers": len(layers), "calls_per_token": len(layers),
            "entry_point": "kronq_decode_matvec_noalloc" if noalloc else "kronq_decode_matvec",
            "kernels_per_call": 2, "bits": bits, "group": group,
            "algorithmic_bytes_per_token": alg_bytes, "ms_per_token_graph": ms,
            "tokens_per_s": 1e3 / ms, "ms_per_token_eager": eager_ms,
            "gbs": gbs, "frac_hbm_peak": gbs / PEAK_HBM_GBS, "steps": steps, "warmup": warmup,
            "data": "synthetic codes, grids, signs and x (seeded torch generator)"}


CONFIG_LEG_WORKLOADS = ("tiny_linear_256", "llama2_7b_down_proj", "llama3_8b_block", "llama3_70b_mlp")


def configs_leg(steps, warmup, names=CONFIG_LEG_WORKLOADS):
    """Per-sublayer quantize wall time of the other workloads, on inputs generated
    in device memory; reported apart from the headline value.  A sublayer's path
    is both Grams, BiIP, sensitivity, the damped inverse Cholesky factor and the
    column loop.  Where bits are allocated (the Llama-3-8B block) the method needs
    every sublayer's score first: each sublayer is rotated, scored and factored,
    the block's bits are allocated, then each column loop runs.  Sublayers that
    share an input (q/k/v, gate/up) share its X Gram, the rotation of H_X and the
    damped inverse factor, computed once per input; a sublayer's time carries an
    equal share of them."""
    import torch
    import post_quantization_02_amd as kq
    from synth import workloads as WL

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def timed(fn, nev):
        """warmup + steps repetitions of fn(ev); mean ms between consecutive events"""
        for _ in range(warmup):
            fn(None)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
        for k in range(steps):
            fn(evs[k])
        torch.cuda.synchronize()
        return [float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(steps)]))
                for i in range(nev - 1)]

    out = []
    for wname in names:
        w = WL.BY_NAME[wname]
        log("configs leg:", wname)
        N = w.N
        held = {}
        rows = []
        # consecutive sublayers that read the same input form a group
        groups = []
        for s in w.sublayers:
            if groups and groups[-1][0].x == s.x:
                groups[-1].append(s)
            else:
                groups.append([s])
        for grp in groups:
            s0 = grp[0]
            k = len(grp)
            n = s0.n
            log("  shared input %s: Gram, input-side rotation, factor (%d sublayers)" % (s0.x, k))
            Xd = w.gen_x_dev(s0.x)
            si = torch.from_numpy(w.in_signs(s0.x)).to(dev)
            HX = torch.empty((n, n), dtype=torch.float32, device=dev)
            HXs = torch.empty_like(HX)
            R = torch.empty((n, n), dtype=torch.float32, device=dev)
            perm = torch.empty(n, dtype=torch.int32, device=dev)

            def phase_x(ev):
                # the input's H_X, its rotation V H_X V^T (shared input-side
                # signs, no rescale on this side) and the damped inverse factor;
                # the copy kept for the sublayers' traces is not timed
                if ev is not None:
                    ev[0].record(stream)
                kq.kronq_gram(Xd, HX)
                if ev is not None:
                    ev[1].record(stream)
                kq.kronq_biip_rotate_sx(None, HX, None, si, s0.in_block, None, 1, 0.0, 0.0, m=1)
                if ev is not None:
                    ev[2].record(stream)
                HXs.copy_(HX)
                if ev is not None:
                    ev[3].record(stream)
                kq.kronq_chol_inv(HX, w.lam, s0.act_order, perm=perm, R=R)
                if ev is not None:
                    ev[4].record(stream)

            tx = timed(phase_x, 5)
            shared = {"gram_x": tx[0], "rot_hx": tx[1], "chol_inv": tx[3]}
            del Xd, HX
            torch.cuda.empty_cache()
            for s in grp:
                log("  rotate, score:", s.name, s.m, "x", s.n)
                Gd = w.gen_g_dev(s.name)
                W0 = torch.from_numpy(w.w_f32(s.name)).to(dev)
                so = torch.from_numpy(w.out_signs(s.name)).to(dev)
                m = s.m
                HG = torch.empty((m, m), dtype=torch.float32, device=dev)
                Wk = torch.empty_like(W0)
                sg = torch.empty(m, dtype=torch.float32, device=dev)
                tr = torch.empty(3, dtype=torch.float64, device=dev)

                def phase_a(ev):
                    if ev is not None:
                        ev[0].record(stream)
                    kq.kronq_gram(Gd, HG)
                    if ev is not None:
                        ev[1].record(stream)
                    Wk.copy_(W0)
                    if ev is not None:
                        ev[2].record(stream)
                    kq.kronq_biip_rotate(Wk, None, HG, si, s.in_block, so, s.out_block, w.alpha, sg)
                    if ev is not None:
                        ev[3].record(stream)
                    kq.kronq_sensitivity(HXs, HG, out=tr)
                    if ev is not None:
                        ev[4].record(stream)

                ta = timed(phase_a, 5)
                held[s.name] = (Wk, R, perm)
                biip_ms = ta[2] + shared["rot_hx"] / k
                rows.append({"sublayer": s.name, "m": m, "n": n, "in_block": s.in_block,
                             "out_block": s.out_block, "group": s.group, "act_order": s.act_order,
                             "score": float(tr[2].item()), "input_shared_by": k,
                             "stage_ms": {"gram_x": shared["gram_x"] / k, "gram_g": ta[0], "w_restore": ta[1],
                                          "biip": biip_ms, "sensitivity": ta[3],
                                          "chol_inv": shared["chol_inv"] / k},
                             "shared_input_ms": shared,
                             "gram_x_tflops": N * n * (n + 1) / (shared["gram_x"] * 1e-3) / 1e12,
                             "gram_g_tflops": N * m * (m + 1) / (ta[0] * 1e-3) / 1e12,
                             "fwht_gbs": 16.0 * (m * n + m * m) / (ta[2] * 1e-3) / 1e9})
                del Gd, HG, sg, tr, W0
                torch.cuda.empty_cache()
            del HXs
            torch.cuda.empty_cache()
        nparams = w.n_params()
        if any(s.bits <= 0 for s in w.sublayers):
            budget = int(round(w.avg_bits * sum(nparams)))
            t0 = time.perf_counter()
            bits = kq.kronq_allocate_bits([r["score"] for r in rows], nparams, 2, 4, budget)
            alloc_ms = (time.perf_counter() - t0) * 1e3
        else:
            bits = [s.bits for s in w.sublayers]
            alloc_ms = 0.0
        for s, r, b in zip(w.sublayers, rows, bits):
            log("  column loop:", s.name, "bits", b)
            Wk, R, perm = held.pop(s.name)
            res = kq.kronq_gptq_quantize(Wk, R, perm, b, s.group)

            def phase_b(ev):
                if ev is not None:
                    ev[0].record(stream)
                kq.kronq_gptq_quantize(Wk, R, perm, b, s.group, What=res["What"], codes=res["codes"],
                                       scales=res["scales"], zeros=res["zeros"])
                if ev is not None:
                    ev[1].record(stream)

            r["bits"] = b
            r["stage_ms"]["gptq"] = timed(phase_b, 2)[0]
            st = r["stage_ms"]
            r["ms"] = sum(v for k, v in st.items() if k != "w_restore") + alloc_ms / len(rows)
            del Wk, R, perm, res
            torch.cuda.empty_cache()
        out.append({"workload": w.name, "N": N, "x_dtype": w.dtype, "alpha": w.alpha, "damp": w.lam,
                    "allocation_ms": alloc_ms, "sublayers": rows,
                    "total_ms": sum(r["ms"] for r in rows)})
    return out


class SublayerPath:
    """Device buffers and one pass of the path for one sublayer (inputs resident)."""

    NAMES = ("gram_x", "gram_g", "biip", "sensitivity", "chol_inv", "gptq")

    def __init__(self, w, s, Xd, Gd, W0, dev):
        import torch
        import post_quantization_02_amd as kq
        self.kq, self.w, self.s = kq, w, s
        m, n, N = s.m, s.n, w.N
        self.Xd, self.Gd, self.W0 = Xd, Gd, W0
        self.si = torch.from_numpy(w.in_signs(s.x)).to(dev)
        self.so = torch.from_numpy(w.out_signs(s.name)).to(dev)
        f32 = torch.float32
        self.HX = torch.empty((n, n), dtype=f32, device=dev)
        self.HG = torch.empty((m, m), dtype=f32, device=dev)
        self.sg = torch.empty(m, dtype=f32, device=dev)
        self.tr = torch.empty(3, dtype=torch.float64, device=dev)
        self.R = torch.empty((n, n), dtype=f32, device=dev)
        self.perm = torch.empty(n, dtype=torch.int32, device=dev)
        self.What = torch.empty((m, n), dtype=f32, device=dev)
        self.codes = torch.empty((m, n), dtype=torch.uint8, device=dev)
        ng = 1 if s.group <= 0 else n // s.group
        self.scales = torch.empty((m, ng), dtype=f32, device=dev)
        self.zeros = torch.empty((m, ng), dtype=f32, device=dev)
        lib = kq.load()
        u8 = torch.uint8
        self.ws_gx = torch.empty(max(1, lib.kronq_gram_ws(N, n, kq.KRONQ_BF16)), dtype=u8, device=dev)
        self.ws_gg = torch.empty(max(1, lib.kronq_gram_ws(N, m, kq.KRONQ_BF16)), dtype=u8, device=dev)
        self.ws_b = torch.empty(max(1, lib.kronq_biip_ws(m, n)), dtype=u8, device=dev)
        self.ws_c = torch.empty(max(1, lib.kronq_chol_inv_ws(n)), dtype=u8, device=dev)
        self.ws_q = torch.empty(max(1, lib.kronq_gptq_ws(m, n)), dtype=u8, device=dev)

    def step(self, Wk, stream, ev=None):
        """One pass; Wk (rotated in place) holds the step's own copy of W.
        ev: 7 events, recorded between the stages."""
        kq, w, s = self.kq, self.w, self.s

        def mark(i):
            if ev is not None:
                ev[i].record(stream)

        mark(0)
        kq.kronq_gram(self.Xd, self.HX, ws=self.ws_gx)
        mark(1)
        kq.kronq_gram(self.Gd, self.HG, ws=self.ws_gg)
        mark(2)
        kq.kronq_biip_rotate(Wk, self.HX, self.HG, self.si, s.in_block, self.so, s.out_block, w.alpha,
                             self.sg, ws=self.ws_b)
        mark(3)
        kq.kronq_sensitivity(self.HX, self.HG, out=self.tr)
        mark(4)
        kq.kronq_chol_inv(self.HX, w.lam, s.act_order, perm=self.perm, R=self.R, ws=self.ws_c)
        mark(5)
        kq.kronq_gptq_quantize(Wk, self.R, self.perm, s.bits, s.group, What=self.What, ws=self.ws_q,
                               codes=self.codes, scales=self.scales, zeros=self.zeros)
        mark(6)


def run_workload(w, steps, warmup, dev):
    """Time `steps` passes of the path over every sublayer of `w` (after
    `warmup` untimed passes).  Returns (per-step wall ms, per-sublayer event
    times, input generation seconds, the SublayerPath objects)."""
    import torch
    import synth
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    paths = []
    xs = {}
    for s in w.sublayers:
        log("  inputs", w.name, s.name, s.m, "x", s.n)
        if s.x not in xs:
            xs[s.x] = w.gen_x_dev(s.x)
        Gd = w.gen_g_dev(s.name)
        W0 = torch.from_numpy(w.w_f32(s.name)).to(dev)
        paths.append(SublayerPath(w, s, xs[s.x], Gd, W0, dev))
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t0
    log("  warmup", warmup)
    for _ in range(warmup):
        for p in paths:
            Wk = p.W0.clone()
            p.step(Wk, stream)
            del Wk
    # the rotation works in place: every timed step gets its own copy of each W,
    # resident before the timed region like X and G
    Wts = [[p.W0.clone() for p in paths] for _ in range(steps)]
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in paths] for _ in range(steps)]
    torch.cuda.synchronize()
    log("  timing", steps, "steps")
    t0 = time.perf_counter()
    for k in range(steps):
        for j, p in enumerate(paths):
            p.step(Wts[k][j], stream, evs[k][j])
        log("    step", k + 1, "done")
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    per_sub = []
    for j, p in enumerate(paths):
        st = {nm: float(np.mean([evs[k][j][i].elapsed_time(evs[k][j][i + 1]) for k in range(steps)]))
              for i, nm in enumerate(SublayerPath.NAMES)}
        per_sub.append(st)
    for j, p in enumerate(paths):
        p.Wk_last = Wts[-1][j]
    return wall_ms, per_sub, t_gen, paths


def incoherence_leg(w, path, dev):
    """mu(H)/sqrt(d) of H_G and H_X before and after BiIP (the incoherence
    diagnostic), with the time of one call at d = 4096."""
    import torch
    kq = path.kq
    s = w.sublayers[0]
    HG0 = kq.kronq_gram(path.Gd)
    HX0 = kq.kronq_gram(path.Xd)
    W = path.W0.clone()
    HG1, HX1 = HG0.clone(), HX0.clone()
    kq.kronq_biip_rotate(W, HX1, HG1, path.si, s.in_block, path.so, s.out_block, w.alpha)
    lib = kq.load()
    ws = torch.empty(lib.kronq_incoherence_ws(max(s.m, s.n)), dtype=torch.uint8, device=dev)
    res = {}
    for name, H in (("hg_before", HG0), ("hg_after_biip", HG1), ("hx_before", HX0), ("hx_after_biip", HX1)):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        try:
            r = kq.kronq_incoherence(H, ws=ws)
        except kq.KronqError as e:   # reported, not fatal: a diagnostic leg
            res[name] = {"error": str(e)}
            continue
        res[name] = {"mu_over_sqrt_d": r["mu"], "sweeps": r["sweeps"],
                     "ms": (time.perf_counter() - t0) * 1e3}
    return {"workload": w.name, "d": [s.m, s.n], "tol": 1e-13, **res}


def gptaq_leg(w, path, dev, steps=5):
    """The asymmetric correction on the Llama-2-7B q_proj shape: the drift term
    (X_fp - X)^T X / N from a drifted input stream, its input-side rotation, P,
    and the column loop with the drift term; event-timed, inputs resident."""
    import torch
    import post_quantization_02_amd as kq
    s = w.sublayers[0]
    m, n, N = s.m, s.n, w.N
    lib = kq.load()
    stream = torch.cuda.current_stream()
    Xd = path.Xd
    Xfd = w.gen_xfp_dev(s.x)
    C = torch.empty((n, n), dtype=torch.float32, device=dev)
    P = torch.empty((n, n), dtype=torch.float32, device=dev)
    ws_d = torch.empty(lib.kronq_drift_cross_ws(N, n), dtype=torch.uint8, device=dev)
    ws_p = torch.empty(lib.kronq_gptaq_correction_ws(n), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(lib.kronq_gptaq_ws(m, n), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(1, lib.kronq_biip_ws(n, n)), dtype=torch.uint8, device=dev)
    Wk = path.Wk_last
    names = ("drift_cross", "rotate_c", "correction_p", "gptaq_loop")

    def one(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        kq.kronq_drift_cross(Xfd, Xd, C, ws=ws_d)
        mark(1)
        kq.kronq_biip_rotate(C, None, None, path.si, s.in_block, path.si, s.in_block, 0.0, ws=ws_b)
        mark(2)
        kq.kronq_gptaq_correction(C, path.R, path.perm, 0.25, P, ws=ws_p)
        mark(3)
        kq.kronq_gptaq_quantize(Wk, path.R, path.perm, s.bits, s.group, P, What=path.What, ws=ws_q,
                                codes=path.codes, scales=path.scales, zeros=path.zeros)
        mark(4)

    one()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for k in range(steps):
        one(evs[k])
    torch.cuda.synchronize()
    st = {nm: float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(steps)]))
          for i, nm in enumerate(names)}
    cross_flops = 4.0 * N * n * n            # hi^T X and lo^T X, all n^2 entries
    p_flops = 2.0 * n ** 3 / 2 + 2.0 * n ** 3 / 6   # triangular K = C_p R^T, P = triu1(K) R
    return {"workload": w.name + " with a drifted input stream (drift %.2f)" % w.drift,
            "alpha": 0.25, "stage_ms": st,
            "drift_cross_tflops": cross_flops / (st["drift_cross"] * 1e-3) / 1e12,
            "correction_tflops_fp32": p_flops / (st["correction_p"] * 1e-3) / 1e12,
            "loop_ms": st["gptaq_loop"]}


def sublayer_record(w, s, st):
    m, n, N = s.m, s.n, w.N
    return {
        "sublayer": s.name, "m": m, "n": n, "bits": s.bits, "group": s.group,
        "hadamard_in": s.in_block, "hadamard_out": s.out_block, "act_order": s.act_order,
        "ms": sum(st.values()), "stage_ms": st,
        "gram_x_tflops": N * n * (n + 1) / (st["gram_x"] * 1e-3) / 1e12,
        "gram_g_tflops": N * m * (m + 1) / (st["gram_g"] * 1e-3) / 1e12,
        "fwht_gbs": 16.0 * (m * n + n * n + m * m) / (st["biip"] * 1e-3) / 1e9,
        "chol_tflops_fp32": 2.0 * n ** 3 / 3 / (st["chol_inv"] * 1e-3) / 1e12,
        "gptq_tflops_fp64": float(m) * n * n / (st["gptq"] * 1e-3) / 1e12,
        "gptq_min_bytes_gbs": (9.0 * m * n + 2.0 * n * n) / (st["gptq"] * 1e-3) / 1e9,
    }


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(args)
        return
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.library_gram:
        library_gram([int(x) for x in args.library_gram.split(",")])
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library runs the whole path on a single MI355X "
              "and does not shard it across GPUs (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.configs:
        log("configs leg only")
        print(json.dumps({"configs": configs_leg(args.config_steps, 1)}), flush=True)
        return
    if args.decode_only:
        log("decode leg only")
        print(json.dumps({"decode": decode_leg(args.decode_steps, 3),
                          "decode_stacked": decode_leg(args.decode_steps, 3, sublayers=DECODE_STACKED,
                                                       name="llama2_7b_linear_stack_qkv_gateup"),
                          "decode_noalloc": decode_leg(args.decode_steps, 3, noalloc=True)}),
              flush=True)
        return
    import torch
    import post_quantization_02_amd as kq
    from synth import workloads as WL

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kq.load()
    w = WL.C5
    log("headline workload", w.name)
    wall_ms, per_sub, t_gen, paths = run_workload(w, args.steps, args.warmup, dev)
    L = len(w.sublayers)
    subs = [sublayer_record(w, s, st) for s, st in zip(w.sublayers, per_sub)]
    N = w.N
    # roofline: the Gram launches at d = 28672 (G of gate_proj, X of down_proj)
    big = []
    for s, st in zip(w.sublayers, per_sub):
        if s.m == 28672:
            big.append(st["gram_g"])
        if s.n == 28672:
            big.append(st["gram_x"])
    d = 28672
    gram_ms = float(np.mean(big))
    gram_flops = float(N) * d * (d + 1)
    gram_tflops = gram_flops / (gram_ms * 1e-3) / 1e12
    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            with open(args.traffic_json) as f:
                tj = json.load(f)
            if tj.get("gram_source_sha256") == gram_source_hash():
                traffic = tj.get("bytes_per_launch")
        except Exception:
            traffic = None
    fwht_bytes = sum(16.0 * (s.m * s.n + s.n * s.n + s.m * s.m) for s in w.sublayers)
    fwht_ms = sum(st["biip"] for st in per_sub)
    out = {
        "metric": "sublayer quantize wall time (s) + Gram TFLOP/s & FWHT GB/s vs MI355X peak",
        "value": wall_ms / 1e3 / L,
        "unit": "s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_ms,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "N": N, "sublayers": ["%s %dx%d" % (s.name, s.m, s.n)
                                                             for s in w.sublayers],
                   "x_dtype": "bf16", "bits": 2, "group": 128, "hadamard": "7x4096 on 28672, 8192 full",
                   "alpha": w.alpha, "damp": w.lam, "act_order": False,
                   "value_is": "step wall time / %d sublayers" % L},
        "sublayers": subs,
        "stage_dtypes": {"gram": "bf16 products, fp32 accumulate", "biip": "fp32",
                         "chol_inv": "fp32 (diagonal blocks fp64)", "gptq": "fp64",
                         "sensitivity": "fp64 sums"},
        "gram_tflops": gram_tflops,
        "gram_frac_bf16_peak": gram_tflops / PEAK_BF16_TFLOPS,
        "fwht_gbs": fwht_bytes / (fwht_ms * 1e-3) / 1e9,
        "fwht_frac_hbm_peak": fwht_bytes / (fwht_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "roofline": {"kernel": "gram_bf16_lds_sync_kernel, kronq_gram at d = 28672 (one launch, no split-K)",
                     "bound": "mfma", "achieved": gram_tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": gram_tflops / PEAK_BF16_TFLOPS,
                     "traffic": traffic,
                     "algorithmic_flops_per_launch": gram_flops,
                     "algorithmic_bytes_per_launch": 2.0 * N * d + 4.0 * d * d},
        "input_gen_s": t_gen,
    }
    del paths
    torch.cuda.empty_cache()
    # host-only allocation on the Llama-3-8B block's seven scores (3.0-bit budget)
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "allocation_llama3_8b_block.json")))
    t0 = time.perf_counter()
    for _ in range(1000):
        kq.kronq_allocate_bits(g["scores"], g["n_params"], g["bmin"], g["bmax"], g["budget_bits"])
    out["allocation"] = {"workload": "llama3_8b_block scores, 7 sublayers, {2,3,4} bits, 3.0 average",
                         "us_per_call": (time.perf_counter() - t0) * 1e3}
    if not args.no_secondary:
        w2 = WL.C2
        log("secondary workload", w2.name)
        wall2, per2, _, p2 = run_workload(w2, max(args.steps, 5), args.warmup, dev)
        s2 = w2.sublayers[0]
        r2 = sublayer_record(w2, s2, per2[0])
        gms = 0.5 * (per2[0]["gram_x"] + per2[0]["gram_g"])
        gt = w2.N * s2.n * (s2.n + 1) / (gms * 1e-3) / 1e12
        r2.update({"workload": w2.name, "ms_per_step": wall2, "gram_frac_bf16_peak": gt / PEAK_BF16_TFLOPS,
                   "fwht_frac_hbm_peak": r2["fwht_gbs"] / PEAK_HBM_GBS})
        out["secondary"] = r2
        out["gptaq"] = gptaq_leg(w2, p2[0], dev)
        # CV_in / CV_out of W before and after BiIP, and the diagnostic's own rate
        # (one read of W: 4 m n algorithmic bytes per call)
        m, n = s2.m, s2.n
        lib = kq.load()
        W0, Wk = p2[0].W0, p2[0].Wk_last
        cv_out = torch.empty(2, dtype=torch.float64, device=dev)
        ws_cv = torch.empty(lib.kronq_weight_cv_ws(m, n), dtype=torch.uint8, device=dev)
        cv_before = [float(v) for v in kq.kronq_weight_cv(W0, out=cv_out, ws=ws_cv).cpu()]
        cv_after = [float(v) for v in kq.kronq_weight_cv(Wk, out=cv_out, ws=ws_cv).cpu()]
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        for _ in range(3):
            kq.kronq_weight_cv(W0, out=cv_out, ws=ws_cv)
        e0.record(stream)
        for _ in range(20):
            kq.kronq_weight_cv(W0, out=cv_out, ws=ws_cv)
        e1.record(stream)
        torch.cuda.synchronize()
        cv_ms = e0.elapsed_time(e1) / 20
        out["weight_cv"] = {"workload": w2.name, "cv_in_before": cv_before[0],
                            "cv_out_before": cv_before[1], "cv_in_after_biip": cv_after[0],
                            "cv_out_after_biip": cv_after[1], "ms_per_call": cv_ms,
                            "gbs": 4.0 * m * n / (cv_ms * 1e-3) / 1e9,
                            "frac_hbm_peak": 4.0 * m * n / (cv_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
        out["incoherence"] = incoherence_leg(w2, p2[0], dev)
        del p2
        torch.cuda.empty_cache()
    if not args.no_decode:
        log("decode leg")
        out["decode"] = decode_leg(args.decode_steps, 3)
        out["decode_stacked"] = decode_leg(args.decode_steps, 3, sublayers=DECODE_STACKED,
                                           name="llama2_7b_linear_stack_qkv_gateup")
        out["decode_noalloc"] = decode_leg(args.decode_steps, 3, noalloc=True)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle sample)")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_budget_s)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
