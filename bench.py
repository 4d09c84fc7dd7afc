"""Benchmark of the KronQ per-sublayer quantization path on one MI355X.

One step = the whole hot path for one sublayer, inputs resident in HBM:
  H_X = X^T X / N, H_G = G^T G / N            (kronq_gram x 2, bf16 matrix cores)
  BiIP: S_G rescale + Hadamard both sides      (kronq_biip_rotate)
  sensitivity tr(H_X') tr(H_G')                (kronq_sensitivity)
  damping + inverse Cholesky factor            (kronq_chol_inv, synchronizes)
  column-wise OBS quantize-and-compensate      (kronq_gptq_quantize)
  bit allocation                               (kronq_allocate_bits, host)
Workload: Llama-2-7B q_proj shape -- W 4096 x 4096, X and G 262144 x 4096 bf16
(128 sequences x 2048 tokens), 2-bit asymmetric groups of 128, Hadamard 4096 on
both sides, alpha 0.25, damping 1% of the mean diagonal.  Synthetic inputs
(heavy-tailed activations with outlier channels, log-normal gradient channel
scales) stand in for the calibration set.

Prints one JSON line.  `value` is the wall time of one sublayer quantization
(seconds, lower is better).  Per-stage times come from HIP events recorded on
the stream the kernels run on; `roofline` is for the Gram kernel call.
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
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "gram_bf16_llama2_7b_q_proj_traffic.json"))
    ap.add_argument("--copy-probe", type=int, metavar="BYTES", default=0,
                    help="only run a plain device copy of BYTES five times (calibrates the HBM byte "
                         "counters) and exit")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                             "COPY_WRITE_CSV"),
                    help="only turn four rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE and "
                         "WRITE_SIZE of this benchmark, then of --copy-probe) into the traffic file "
                         "(--traffic-json) and exit")
    ap.add_argument("--copy-bytes", type=int, default=256 * 1024 * 1024,
                    help="BYTES the copy-probe runs used (for --summarize-traffic)")
    return ap.parse_args()


GRAM_SRC = os.path.join(ROOT, "post_quantization_02_amd", "csrc", "gram.hip")
GRAM_KERNELS = ("gram_bf16_lds_kernel", "gram_finalize_kernel", "gram_bf16_kernel")


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


def _pmc_mean(path, kernel_pred, counter):
    import csv
    per_dispatch = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and kernel_pred(r["Kernel_Name"]):
                key = r["Dispatch_Id"]
                per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    vals = list(per_dispatch.values())
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def summarize_traffic(args):
    """HBM bytes per kronq_gram call (the Gram kernel and its split-K finalize)
    from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled so that the
    same counter over a plain copy of known size reads that size."""
    f_csv, w_csv, cf_csv, cw_csv = args.summarize_traffic
    copy = lambda k: "copyBuffer" in k
    cf, _ = _pmc_mean(cf_csv, copy, "FETCH_SIZE")
    cw, _ = _pmc_mean(cw_csv, copy, "WRITE_SIZE")
    kib = args.copy_bytes / 1024.0
    f_scale, w_scale = kib / cf, kib / cw
    out = {"counters": {}, "copy_probe": {"bytes": args.copy_bytes, "fetch_kib": cf, "write_kib": cw,
                                          "fetch_scale": f_scale, "write_scale": w_scale}}
    total = 0.0
    for k in GRAM_KERNELS:
        pred = lambda name, k=k: k in name
        fk, nf = _pmc_mean(f_csv, pred, "FETCH_SIZE")
        wk, nw = _pmc_mean(w_csv, pred, "WRITE_SIZE")
        if fk is None or wk is None:
            continue
        b = (fk * f_scale + wk * w_scale) * 1024.0
        out["counters"][k] = {"fetch_kib": fk, "write_kib": wk, "dispatches": nf,
                              "hbm_bytes_per_dispatch": b}
        total += b
    out["bytes_per_launch"] = total
    out["unit"] = "bytes per kronq_gram call (sum over its kernels, scaled counters)"
    out["gram_source_sha256"] = gram_source_hash()
    run = "python3 -u bench.py --steps 1 --warmup 0 --no-cpu-baseline"
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


def cpu_baseline(w, X, G, W, budget_s):
    """The oracle (numpy float64, as it stands) on a bounded sample of the same
    workload, extrapolated to one sublayer:
      Gram: a token prefix of X and of G (the Gram is linear in N),
      BiIP: full W, H_X, H_G rotations (sample-free),
      damping + inverse Cholesky: full,
      column loop: a row sample (rows are independent), all columns."""
    import synth
    from oracle import kronq_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    s = w.sub("q_proj")
    N = w.N
    t0 = time.perf_counter()
    Np = 4096
    xs = synth.bf16_to_f64(X[:Np])
    gs = synth.bf16_to_f64(G[:Np])
    t_g0 = time.perf_counter()
    HXs = O.gram(xs)
    HGs = O.gram(gs)
    t_gram = (time.perf_counter() - t_g0) * (N / Np)
    # BiIP: the three 4096 x 4096 rotations cost the same; W's is timed, x3
    t_b0 = time.perf_counter()
    Wp, _, _, sg = O.biip(synth.bf16_to_f64(W), None, HGs, w.in_signs("x"), s.in_block,
                          w.out_signs("q_proj"), s.out_block, w.alpha)
    t_biip = 3.0 * (time.perf_counter() - t_b0)
    t_s0 = time.perf_counter()
    O.sensitivity(HXs, HGs)
    t_sens = time.perf_counter() - t_s0
    t_c0 = time.perf_counter()
    perm, H = O.prepare_hessian(HXs, w.lam, s.act_order)
    R, _ = O.chol_inv_upper(H)
    t_chol = time.perf_counter() - t_c0
    rows = 16
    t_q0 = time.perf_counter()
    O.gptq(Wp[:rows], R, perm, s.bits, s.group)
    t_gptq = (time.perf_counter() - t_q0) * (s.m / rows)
    total = t_gram + t_biip + t_sens + t_chol + t_gptq
    wall = time.perf_counter() - t0
    return {
        "value": total, "unit": "s", "cores": int(cores), "kind": "oracle",
        "sample": ("Gram on the first %d of %d tokens of X and G, scaled x%d; BiIP rotation of W "
                   "timed and scaled x3 (H_X, H_G cost the same); sensitivity and damped inverse "
                   "Cholesky in full; column loop on %d of %d rows, scaled x%d; float64 numpy; "
                   "%.1f s of host time") % (Np, N, N // Np, rows, s.m, s.m // rows, wall),
        "stages_s": {"gram_x_g": t_gram, "biip": t_biip, "sensitivity": t_sens, "chol_inv": t_chol,
                     "gptq": t_gptq},
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
               name="llama2_7b_linear_stack"):
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
    share an input are timed as if each computed its own X Gram (the method
    computes it once per input)."""
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
        Xd, xname = None, None
        held = {}
        rows = []
        for s in w.sublayers:
            if s.x != xname:
                Xd = None
                torch.cuda.empty_cache()
                Xd, xname = w.gen_x_dev(s.x), s.x
            log("  rotate, score, factor:", s.name, s.m, "x", s.n)
            Gd = w.gen_g_dev(s.name)
            W0 = torch.from_numpy(w.w_f32(s.name)).to(dev)
            si = torch.from_numpy(w.in_signs(s.x)).to(dev)
            so = torch.from_numpy(w.out_signs(s.name)).to(dev)
            m, n = s.m, s.n
            HX = torch.empty((n, n), dtype=torch.float32, device=dev)
            HG = torch.empty((m, m), dtype=torch.float32, device=dev)
            Wk = torch.empty_like(W0)
            sg = torch.empty(m, dtype=torch.float32, device=dev)
            tr = torch.empty(3, dtype=torch.float64, device=dev)
            R = torch.empty((n, n), dtype=torch.float32, device=dev)
            perm = torch.empty(n, dtype=torch.int32, device=dev)

            def phase_a(ev):
                if ev is not None:
                    ev[0].record(stream)
                kq.kronq_gram(Xd, HX)
                if ev is not None:
                    ev[1].record(stream)
                kq.kronq_gram(Gd, HG)
                if ev is not None:
                    ev[2].record(stream)
                Wk.copy_(W0)
                if ev is not None:
                    ev[3].record(stream)
                kq.kronq_biip_rotate(Wk, HX, HG, si, s.in_block, so, s.out_block, w.alpha, sg)
                if ev is not None:
                    ev[4].record(stream)
                kq.kronq_sensitivity(HX, HG, out=tr)
                if ev is not None:
                    ev[5].record(stream)
                kq.kronq_chol_inv(HX, w.lam, s.act_order, perm=perm, R=R)
                if ev is not None:
                    ev[6].record(stream)

            ta = timed(phase_a, 7)
            held[s.name] = (Wk, R, perm)
            rows.append({"sublayer": s.name, "m": m, "n": n, "in_block": s.in_block,
                         "out_block": s.out_block, "group": s.group, "act_order": s.act_order,
                         "score": float(tr[2].item()),
                         "stage_ms": dict(zip(("gram_x", "gram_g", "w_restore", "biip", "sensitivity",
                                               "chol_inv"), ta)),
                         "gram_x_tflops": N * n * (n + 1) / (ta[0] * 1e-3) / 1e12,
                         "gram_g_tflops": N * m * (m + 1) / (ta[1] * 1e-3) / 1e12,
                         "fwht_gbs": 16.0 * (m * n + n * n + m * m) / (ta[3] * 1e-3) / 1e9})
            del Gd, HX, HG, sg, tr, W0
            torch.cuda.empty_cache()
        Xd = None
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


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(args)
        return
    if args.copy_probe:
        copy_probe(args.copy_probe)
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
                                                       name="llama2_7b_linear_stack_qkv_gateup")}),
              flush=True)
        return
    import torch
    import post_quantization_02_amd as kq
    import synth
    from synth import workloads as WL

    w = WL.C2
    s = w.sub("q_proj")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating inputs", w.name)
    t0 = time.perf_counter()
    X = w.gen_x("x")
    G = w.gen_g("q_proj")
    W = w.gen_w("q_proj")
    t_gen = time.perf_counter() - t0
    t0 = time.perf_counter()
    Xd = torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).to(dev)
    Gd = torch.from_numpy(G.view(np.int16)).view(torch.bfloat16).to(dev)
    W0 = torch.from_numpy(synth.bf16_to_f32(W)).to(dev)
    si = torch.from_numpy(w.in_signs("x")).to(dev)
    so = torch.from_numpy(w.out_signs("q_proj")).to(dev)
    torch.cuda.synchronize()
    t_h2d = time.perf_counter() - t0
    m, n, N = s.m, s.n, w.N

    HX = torch.empty((n, n), dtype=torch.float32, device=dev)
    HG = torch.empty((m, m), dtype=torch.float32, device=dev)
    Wk = torch.empty_like(W0)
    sg = torch.empty(m, dtype=torch.float32, device=dev)
    tr = torch.empty(3, dtype=torch.float64, device=dev)
    R = torch.empty((n, n), dtype=torch.float32, device=dev)
    perm = torch.empty(n, dtype=torch.int32, device=dev)
    What = torch.empty((m, n), dtype=torch.float32, device=dev)
    codes = torch.empty((m, n), dtype=torch.uint8, device=dev)
    ng = n // s.group
    scales = torch.empty((m, ng), dtype=torch.float32, device=dev)
    zeros = torch.empty((m, ng), dtype=torch.float32, device=dev)
    lib = kq.load()
    ws_g = torch.empty(max(1, lib.kronq_gram_ws(N, n, kq.KRONQ_BF16)), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(1, lib.kronq_biip_ws(m, n)), dtype=torch.uint8, device=dev)
    ws_c = torch.empty(max(1, lib.kronq_chol_inv_ws(n)), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(max(1, lib.kronq_gptq_ws(m, n)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    names = ["gram_x", "gram_g", "biip", "sensitivity", "chol_inv", "gptq", "allocate"]

    def step(Wk, ev=None):
        """One pass of the path; Wk (rotated in place) holds the step's own copy of W."""
        if ev is not None:
            ev[0].record(stream)
        kq.kronq_gram(Xd, HX, ws=ws_g)
        if ev is not None:
            ev[1].record(stream)
        kq.kronq_gram(Gd, HG, ws=ws_g)
        if ev is not None:
            ev[2].record(stream)
        kq.kronq_biip_rotate(Wk, HX, HG, si, s.in_block, so, s.out_block, w.alpha, sg, ws=ws_b)
        if ev is not None:
            ev[3].record(stream)
        kq.kronq_sensitivity(HX, HG, out=tr)
        if ev is not None:
            ev[4].record(stream)
        kq.kronq_chol_inv(HX, w.lam, s.act_order, perm=perm, R=R, ws=ws_c)
        if ev is not None:
            ev[5].record(stream)
        kq.kronq_gptq_quantize(Wk, R, perm, s.bits, s.group, What=What, ws=ws_q, codes=codes,
                               scales=scales, zeros=zeros)
        if ev is not None:
            ev[6].record(stream)
        score = float(tr[2].item())
        bits = kq.kronq_allocate_bits([score], [m * n], s.bits, s.bits, s.bits * m * n)
        if ev is not None:
            ev[7].record(stream)
        return bits

    log("warmup", args.warmup)
    for _ in range(args.warmup):
        Wk.copy_(W0)
        step(Wk)
    # the rotation works in place: every timed step gets its own copy of W,
    # resident before the timed region like X and G
    Wts = [W0.clone() for _ in range(args.steps)]
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(args.steps)]
    log("timing", args.steps, "steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(Wts[k], evs[k])
        log("  step", k + 1, "done")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = {nm: float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)]))
                for i, nm in enumerate(names)}
    ms_step = wall * 1e3 / args.steps
    Wk = Wts[-1]
    del Wts[:-1]

    gram_flops = float(N) * n * (n + 1)        # one factor, unique triangle
    gram_ms = 0.5 * (stage_ms["gram_x"] + stage_ms["gram_g"])
    gram_tflops = gram_flops / (gram_ms * 1e-3) / 1e12
    fwht_bytes = 16.0 * (m * n + n * n + m * m)   # two one-sided passes, 8 B per element each
    fwht_gbs = fwht_bytes / (stage_ms["biip"] * 1e-3) / 1e9
    chol_flops = 2.0 * n ** 3 / 3
    gptq_flops = float(m) * n * n
    gptq_bytes = 9.0 * m * n + 2.0 * n * n

    # HBM traffic per Gram call from the committed counter summary, null when the
    # Gram source has changed since the counters were taken
    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            with open(args.traffic_json) as f:
                tj = json.load(f)
            if tj.get("gram_source_sha256") == gram_source_hash():
                traffic = tj.get("bytes_per_launch")
        except Exception:
            traffic = None

    out = {
        "metric": "sublayer quantize wall time (s) + Gram TFLOP/s & FWHT GB/s vs MI355X peak",
        "value": ms_step / 1e3,
        "unit": "s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "N": N, "m": m, "n": n, "x_dtype": "bf16", "bits": s.bits,
                   "group": s.group, "hadamard_in": s.in_block, "hadamard_out": s.out_block,
                   "alpha": w.alpha, "damp": w.lam, "act_order": s.act_order},
        "stage_ms": stage_ms,
        "stage_dtypes": {"gram": "bf16 products, fp32 accumulate", "biip": "fp32",
                         "chol_inv": "fp32 (diagonal blocks fp64)", "gptq": "fp64",
                         "sensitivity": "fp64 sums"},
        "gram_tflops": gram_tflops,
        "gram_frac_bf16_peak": gram_tflops / PEAK_BF16_TFLOPS,
        "fwht_gbs": fwht_gbs,
        "fwht_frac_hbm_peak": fwht_gbs / PEAK_HBM_GBS,
        "chol_tflops_fp32": chol_flops / (stage_ms["chol_inv"] * 1e-3) / 1e12,
        "gptq_tflops_fp64": gptq_flops / (stage_ms["gptq"] * 1e-3) / 1e12,
        "gptq_min_bytes_gbs": gptq_bytes / (stage_ms["gptq"] * 1e-3) / 1e9,
        "roofline": {"kernel": "kronq_gram call (gram_bf16_kernel + gram_finalize_kernel)",
                     "bound": "mfma", "achieved": gram_tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": gram_tflops / PEAK_BF16_TFLOPS,
                     "traffic": traffic},
        "input_gen_s": t_gen,
        "h2d_s": t_h2d,
    }
    # CV_in / CV_out of W before and after BiIP, and the diagnostic's own rate
    # (one read of W: 4 m n algorithmic bytes per call)
    cv_out = torch.empty(2, dtype=torch.float64, device=dev)
    ws_cv = torch.empty(lib.kronq_weight_cv_ws(m, n), dtype=torch.uint8, device=dev)
    cv_before = [float(v) for v in kq.kronq_weight_cv(W0, out=cv_out, ws=ws_cv).cpu()]
    cv_after = [float(v) for v in kq.kronq_weight_cv(Wk, out=cv_out, ws=ws_cv).cpu()]
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
    out["weight_cv"] = {"cv_in_before": cv_before[0], "cv_out_before": cv_before[1],
                        "cv_in_after_biip": cv_after[0], "cv_out_after_biip": cv_after[1],
                        "ms_per_call": cv_ms, "gbs": 4.0 * m * n / (cv_ms * 1e-3) / 1e9,
                        "frac_hbm_peak": 4.0 * m * n / (cv_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    if not args.no_decode:
        log("decode leg")
        out["decode"] = decode_leg(args.decode_steps, 3)
        out["decode_stacked"] = decode_leg(args.decode_steps, 3, sublayers=DECODE_STACKED,
                                           name="llama2_7b_linear_stack_qkv_gateup")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle sample)")
        out["cpu_baseline"] = cpu_baseline(w, X, G, W, args.cpu_budget_s)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
