"""Benchmark: quantize one down_proj-shaped layer end to end on one MI355X.

A step is one whole quant_layer call on device-resident inputs: H = 2 X X^T
(bf16 MFMA SYRK), dead features + damping, blocked Cholesky, grid steps,
the back-to-front nearest-plane sweep with lazy MFMA block updates, and the
loss/bound reduction.  Default workload (--config 4), the largest layer with
every stage: W 4096 x 14336 bf16 N(0, 0.01^2), X 14336 x 262144 bf16
(Laplace(0, 1) times LogNormal(0, 1) channel scales) stored token-major
(262144 rows of 14336 channels; --x-layout channels stores it
14336 x 262144), symmetric 2-bit, group 64, block 128, damp 0.01 --
synthetic, seeded.  --config 2 / 3 time the q_proj / up_proj layers,
--config 5 the spectral layer (H given, fp64 factor and sweep, no SYRK:
`roofline` is null there).

Prints ONE JSON line.  `roofline` is for the dominant kernel (the Hessian
SYRK tiles): algorithmic flops n(n+1)N per launch over its average duration,
measured with HIP events that the library records around each launch of that
kernel during the timed steps, on the stream it launches on.
`stage_rooflines` gives the same for the other stages: the lazy block
updates (m n (n - 128) flop against the fp32 or fp64 MFMA peak) and the
column sweeps (14 bytes per weight against HBM), both from the library's HIP
events around each of their launches in the timed steps, and the Cholesky
(n^3/3 flop, stage time).  Each carries the published peak and the
achievable one measured on the device by the peak probe
(post_weight_quantization_19_amd/peak_probe, dense MFMA from registers and a
1 GiB copy), run in its own process first; the SYRK's line also carries the
bf16 rate the device sustains over a long launch on random operands.
`cpu_baseline` times the fp64 oracle on a bounded sample of the same
workload on the host cores.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3          # MI355X fp32 MFMA
PEAK_F64_TFLOPS = 78.6           # MI355X fp64 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "layer quantize time (s) & weights quantized/s; MFMA util of SYRK+update"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4, help="workload table entry")
    ap.add_argument("--x-layout", choices=["channels", "tokens"], default="tokens",
                    help="storage of the activations: token-major [ntok, n] (one row per "
                         "token, as a layer's inputs are captured; the default) or [n, ntok]")
    ap.add_argument("--order", default="back_to_front",
                    choices=["back_to_front", "front_to_back", "act_order", "min_pivot"],
                    help="processing order of the timed layer (the natural back-to-front "
                         "order by default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ssqr", type=float, default=None, metavar="DENSITY",
                    help="time the overflow-tolerant layer (SSQR: scale search for this "
                         "outlier density) instead of the plain one")
    ap.add_argument("--ssqr-iters", type=int, default=12)
    ap.add_argument("--oaem", action="store_true",
                    help="time OA-EM codebook initialisation of the layer (groups of 8, "
                         "K = 256, M = 2 codebooks, --oaem-rounds EM rounds per codebook) "
                         "instead of the quantizer")
    ap.add_argument("--oaem-rounds", type=int, default=10)
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the achievable-peak probe (MFMA and copy microbenchmarks)")
    ap.add_argument("--cpu-token-fraction", type=int, default=0,
                    help="oracle Hessian is timed on 1/k of the tokens, scaled by k "
                         "(0: the smallest k that keeps the sample near 2e12 flop)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="context for the Hessian's roofline: time the vendor library's "
                         "bf16 GEMM (torch.mm, hipBLASLt) computing the whole X^T X of the "
                         "layer's token-major X beside this library's Hessian on the same X, "
                         "in one process; prints its own JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (the reference kernel "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


KERNEL_SOURCE = os.path.join(ROOT, "post_weight_quantization_19_amd", "csrc", "hessian.hip")


def traffic_file(cfg):
    """Committed rocprofv3 counter summary of the SYRK tiles for a layer."""
    tag = cfg.name.replace("_", "")
    return os.path.join(ROOT, "profiles", f"syrk_tiles256_{tag}_{cfg.m}x{cfg.n}_traffic.json")


def input_hashes(lay):
    """sha256 of the generated inputs as stored on the host (bf16 bits of W
    and X, or the float32 H), so that runs can be checked to use the same
    data."""
    import hashlib

    def h(a):
        return hashlib.sha256(a.tobytes()).hexdigest()
    out = {}
    if lay.W_bits is not None:
        out["W_bf16"] = h(lay.W_bits)
    elif lay.W is not None:
        out["W_f32"] = h(lay.W)
    if lay.X_bits is not None:
        out["X_bf16"] = h(lay.X_bits)
    elif lay.X is not None:
        out["X_f32"] = h(lay.X)
    if lay.H is not None:
        out["H_f32"] = h(lay.H)
    return out


def measured_traffic(cfg, x_layout):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary, or None if the kernel source has changed since
    the counters were taken or they were taken for the other X layout."""
    import hashlib
    try:
        with open(traffic_file(cfg)) as f:
            t = json.load(f)
        with open(KERNEL_SOURCE, "rb") as f:
            h = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if t.get("kernel_source_sha256") != h or t.get("x_layout") != x_layout:
        return None
    return t.get("hbm_bytes_per_launch")


def spacing_constant(cfg):
    """The spectral layer's spacing constant c (mean code entropy 2.5 bits),
    as searched on the oracle's codes and stored with the tests."""
    path = os.path.join(ROOT, "tests", "golden", "spectral_layer_spacing.json")
    with open(path) as f:
        return float(json.load(f)["c"])


def blas_threads():
    """(vendor string, threads) of the BLAS numpy calls, from threadpoolctl."""
    try:
        from threadpoolctl import threadpool_info
        b = [d for d in threadpool_info() if d.get("user_api") == "blas"]
    except Exception:       # threadpoolctl missing or failing: unknown
        return "unknown", None
    if not b:
        return "unknown", None
    return (", ".join(f"{d.get('internal_api')} {d.get('version')}" for d in b),
            max(int(d.get("num_threads") or 0) for d in b))


def cpu_baseline(lay, cfg, frac):
    """Time the fp64 oracle on a bounded sample and project the whole layer:
    the Hessian over 1/frac of the tokens (x frac), the full Cholesky, and
    the blocked sweep over all rows, or over a row sample (x m / rows) when
    the sweep would take more than about 10 s."""
    import math

    import numpy as np

    import oracle as O
    import synth
    affinity = len(os.sched_getaffinity(0))
    vendor, nthreads = blas_threads()
    if frac <= 0 and lay.X_bits is not None:
        frac = max(1, math.ceil(2.0 * cfg.n * cfg.n * cfg.ntok / 2e12))
    t_h = 0.0
    if lay.X_bits is not None:
        ntok_s = cfg.ntok // frac
        Xs = synth.gen.bf16_bits_to_f32(lay.X_bits[:, :ntok_s])
        t0 = time.perf_counter()
        H_s = O.hessian(Xs)
        t_h = (time.perf_counter() - t0) * frac
        H = H_s * frac  # stand-in Hessian of the right scale for timing the rest
        h_txt = f"Hessian on the first {ntok_s} of {cfg.ntok} tokens, time x{frac}; "
    else:
        H = lay.H.astype(np.float64)
        h_txt = "H given; "
    t0 = time.perf_counter()
    Hd, W0, lam, _ = O.fix_dead_and_damp(H, lay.W64(), cfg.damp)
    L, info = O.cholesky_lower(Hd)
    t_c = time.perf_counter() - t0
    rows = min(cfg.m, max(64, int(4e11 / (2.0 * cfg.n * cfg.n))))
    t0 = time.perf_counter()
    if cfg.grid_kind == "colspacing":
        S = np.broadcast_to(O.colspacing_steps(L, spacing_constant(cfg))[None, :],
                            (rows, cfg.n))
    else:
        s_grp, z = O.grid_steps(W0[:rows], cfg.grid_kind, cfg.bits, cfg.group)
        S = O.expand_group_steps(s_grp, cfg.n)
    O.nearest_plane_sweep_blocked(W0[:rows], L, S, cfg.block)
    t_s = (time.perf_counter() - t0) * cfg.m / rows
    total = t_h + t_c + t_s
    return {
        "value": cfg.m * cfg.n / total, "unit": "weights/s",
        "cores": nthreads if nthreads else affinity, "kind": "oracle",
        "blas": vendor, "blas_threads": nthreads, "cpus_in_affinity": affinity,
        "os_cpu_count": os.cpu_count(),
        "sample": (f"fp64 numpy oracle ({vendor}, {nthreads} BLAS threads, {affinity} CPUs in "
                   f"the affinity mask): {h_txt}full Cholesky; blocked sweep of "
                   f"{rows} of {cfg.m} rows (x{cfg.m / rows:.3g}); projected whole-layer "
                   f"time {total:.2f} s (H {t_h:.2f} s, chol {t_c:.2f} s, sweep {t_s:.2f} s)"),
    }


def update_group_cols(prec):
    """Columns of a lazy-update group in the library's sweep (256 in fp32,
    512 in fp64)."""
    return 512 if prec == "f64" else 256


def sweep_launches(n, B, prec):
    """(sweep-block launches, lazy updates, update flops / m) of one sweep, in
    the order the library issues them: blocks from the back, sub-blocks of at
    most 128 columns, an in-block update after every sub-block but the
    block's first column group; blocks in groups of update_group_cols
    columns, each block's errors applied at once to the open columns of its
    group and each group's errors to every column before the group once its
    last block is swept."""
    bi = min(B, 128)
    grp = update_group_cols(prec) // B
    nblk = (n + B - 1) // B
    nsweep = nupd = 0
    flops_per_row = 0.0
    for b in range(nblk - 1, -1, -1):
        jb0 = b * B
        jb1 = min(n, jb0 + B)
        cg0 = (b // grp) * grp * B
        nsub = (jb1 - jb0 + bi - 1) // bi
        for s in range(nsub - 1, -1, -1):
            js0 = jb0 + s * bi
            nsweep += 1
            if s > 0:
                nupd += 1
                flops_per_row += 2.0 * min(jb1 - js0, bi) * (js0 - jb0)
        if jb0 > cg0:
            nupd += 1
            flops_per_row += 2.0 * (jb1 - jb0) * (jb0 - cg0)
        if jb0 == cg0 and cg0 > 0:
            kg = min(n, cg0 + grp * B) - cg0
            nupd += 1
            flops_per_row += 2.0 * kg * cg0
    return nsweep, nupd, flops_per_row


def measure_peaks():
    """Achievable peaks from the committed probe (a separate process, run
    before this one touches the GPU), or None."""
    import subprocess
    exe = os.path.join(ROOT, "post_weight_quantization_19_amd", "peak_probe")
    if not os.path.exists(exe):
        return None
    try:
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    except subprocess.TimeoutExpired:
        return None
    if r.returncode != 0:
        print(f"[bench] peak probe failed: {r.stderr.strip()}", file=sys.stderr)
        return None
    return json.loads(r.stdout.strip().splitlines()[-1])


def stage_roofline(achieved, peak, achievable, unit, bound, work, how):
    return {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak, "achievable": achievable,
            "frac_of_achievable": (achieved / achievable) if achievable else None,
            "work_per_step": work, "timed_by": how}


def library_gemm_bench(args):
    """The vendor library's bf16 GEMM (torch.mm, which hipBLASLt serves)
    computing the whole product X^T X (2 n^2 N flop, fp32 output) of the
    layer's token-major X, and this library's Hessian (n(n+1)N flop, the
    lower triangle, mirrored) on the same X in the same process, launches
    alternating.  Context for the Hessian's roofline, not a stage of the
    quantizer.  Prints one JSON line of its own."""
    import numpy as np
    import torch

    import post_weight_quantization_19_amd as P
    import synth

    cfg = synth.config(args.config)
    n, N = cfg.n, cfg.ntok
    if cfg.ntok == 0 or cfg.xdtype != "bf16":
        print(f"bench.py --library-gemm: config {args.config} has no bf16 X", file=sys.stderr)
        sys.exit(2)
    print(f"[bench] generating X of {cfg.name} n={n} ntok={N}", file=sys.stderr, flush=True)
    lay = synth.make_layer(cfg, keep_x_f32=False)
    dev = torch.device("cuda:0")
    X = torch.from_numpy(lay.X_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    X = X.t().contiguous()              # token-major [N, n]
    del lay
    H = torch.empty((n, n), dtype=torch.float32, device=dev)
    G = torch.empty((n, n), dtype=torch.float32, device=dev)

    def lib_gemm():
        torch.mm(X.t(), X, out_dtype=torch.float32, out=G)

    def ours():
        P.hessian_accum(X, H, x_layout="tokens")

    for _ in range(max(1, args.warmup)):
        lib_gemm()
        ours()
    torch.cuda.synchronize()
    t_lib, t_ours = [], []
    for _ in range(args.steps):
        for f, ts in ((lib_gemm, t_lib), (ours, t_ours)):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
    # both compute X^T X: the library's fp32 product and half of this
    # library's H agree to fp32 rounding of differently ordered sums
    rel = (torch.linalg.norm(2.0 * G - H) / torch.linalg.norm(H)).item()
    ml, mo = float(np.median(t_lib)), float(np.median(t_ours))
    fl_lib, fl_ours = 2.0 * n * n * N, float(n) * (n + 1) * N
    line = {
        "metric": "bf16 X^T X: vendor-library GEMM against this library's Hessian",
        "value": ml / mo, "unit": "x (library GEMM time / Hessian time)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "library_gemm": {"call": "torch.mm(X.t(), X, out_dtype=torch.float32)",
                         "ms_median": ml, "ms_min": min(t_lib), "flop": fl_lib,
                         "tflops": fl_lib / ml / 1e9},
        "hessian": {"call": "pwq_hessian_accum (token-major X)", "ms_median": mo,
                    "ms_min": min(t_ours), "flop": fl_ours, "tflops": fl_ours / mo / 1e9},
        "rel_fro_2G_vs_H": rel,
        "dtype": "bf16 products, f32 accumulate", "data": "synthetic (seeded)",
        "config": {"workload": f"{cfg.name}: X {N}x{n} bf16 token-major", "n": n, "ntok": N},
    }
    print(json.dumps(line))


def ssqr_bench(args):
    """The overflow-tolerant layer (SSQR): one call = the Hessian once, then
    iters + 2 (or 3) quantizations of the bisection of the step multiplier,
    and the outlier list.  Prints one JSON line of its own."""
    import numpy as np
    import torch

    import post_weight_quantization_19_amd as P
    import synth

    cfg = synth.config(args.config)
    if cfg.grid_kind not in ("sym", "asym"):
        raise SystemExit("SSQR needs a layer with a SYM or ASYM grid (--config 2, 3 or 4)")
    m, n, N = cfg.m, cfg.n, cfg.ntok
    print(f"[bench] generating workload {cfg.name} m={m} n={n} ntok={N}", file=sys.stderr,
          flush=True)
    lay = synth.make_layer(cfg, keep_x_f32=False)
    hashes = input_hashes(lay)
    dev = torch.device("cuda:0")
    W = torch.from_numpy(lay.W_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    X = torch.from_numpy(lay.X_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    xl = args.x_layout
    if xl == "tokens":
        X = X.t().contiguous()
    grid = P.Grid(cfg.grid_kind, cfg.bits, cfg.group)

    def call():
        return P.ssqr_quant_layer(W, X=X, grid=grid, damp=cfg.damp, block=cfg.block,
                                  density=args.ssqr, iters=args.ssqr_iters, x_layout=xl)
    out = call()                                   # warm-up (synchronous)
    reps = max(1, args.steps // 5)
    t0 = time.perf_counter()
    for _ in range(reps):
        out = call()
    dt = (time.perf_counter() - t0) / reps
    # the outlier list alone (two passes over the codes: 8 bytes per weight)
    stream = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    P.overflow_entries(out["codes"], out["scales"], grid, out["zeros"])
    a.record(stream)
    for _ in range(5):
        P.overflow_entries(out["codes"], out["scales"], grid, out["zeros"])
    b.record(stream)
    torch.cuda.synchronize()
    t_list = a.elapsed_time(b) / 5 / 1e3
    gbs = 8.0 * m * n / t_list / 1e9
    nq = args.ssqr_iters + 2
    line = {
        "metric": "SSQR layer time (scale search) & weights quantized/s",
        "value": m * n / dt, "unit": "weights/s", "n_gpus": 1, "steps": reps, "warmup": 1,
        "ms_per_step": dt * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 products, f32 accumulate/factor/sweep",
        "data": "synthetic (seeded)",
        "config": {"workload": f"{cfg.name} (SSQR, outlier density {args.ssqr}, "
                               f"{args.ssqr_iters} halvings of log2 kappa in [-8, 0])",
                   "m": m, "n": n, "ntok": N, "x_layout": xl, "input_sha256": hashes},
        "ssqr": {"kappa": out["kappa"], "n_outliers": out["n_outliers"],
                 "density": out["n_outliers"] / (m * n),
                 "quantizations_per_call": f"{nq} or {nq + 1}",
                 "ms_per_quantization": dt * 1e3 / nq},
        "roofline": {"bound": "hbm", "kernel": "overflow_rows + overflow_scan + "
                     "overflow_write (the outlier list)", "achieved": gbs, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "traffic": None,
                     "avg_launch_ms": t_list * 1e3, "bytes_per_launch": 8.0 * m * n},
    }
    print(json.dumps(line), flush=True)


def oaem_bench(args):
    """OA-EM initialisation of the layer's codebooks: one call = the Hessian
    once, then M = 2 residual stages of `rounds` E/M rounds and a final
    E-step each.  The E-step (fp64 Mahalanobis distances to every centroid)
    is the dominant kernel; it is timed with HIP events around its launches
    in a run of its own.  Prints one JSON line of its own."""
    import numpy as np
    import torch

    import post_weight_quantization_19_amd as P
    import synth

    cfg = synth.config(args.config)
    if cfg.ntok == 0:
        raise SystemExit("OA-EM needs calibration activations (--config 1 to 4)")
    m, n, N = cfg.m, cfg.n, cfg.ntok
    g, K, M, T = 8, 256, 2, args.oaem_rounds
    ng = n // g
    print(f"[bench] generating workload {cfg.name} m={m} n={n} ntok={N}", file=sys.stderr,
          flush=True)
    lay = synth.make_layer(cfg, keep_x_f32=False)
    hashes = input_hashes(lay)
    dev = torch.device("cuda:0")
    W = torch.from_numpy(lay.W_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    X = torch.from_numpy(lay.X_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    xl = args.x_layout
    if xl == "tokens":
        X = X.t().contiguous()
    rng = np.random.default_rng(2024)
    seeds = torch.from_numpy(np.stack([rng.choice(m * ng, K, replace=False)
                                       for _ in range(M)])).to(dev)
    H = torch.empty((n, n), dtype=torch.float32, device=dev)

    def call():
        P.hessian_accum(X, H=H, x_layout=xl)
        return P.oaem_init(W, H, seeds, g=g, iters=T, damp=cfg.damp)
    books, codes, obj, res = call()                # warm-up
    torch.cuda.synchronize()
    reps = max(1, args.steps // 5)
    t0 = time.perf_counter()
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    # the E-step alone: one round of one stage is qtable + E-step; time a
    # run without M-steps (iters 0: one E-step per stage) against events
    stream = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    one = seeds[:1].contiguous()
    P.oaem_init(W, H, one, g=g, iters=0, damp=cfg.damp, want_objective=False)
    a.record(stream)
    for _ in range(5):
        P.oaem_init(W, H, one, g=g, iters=0, damp=cfg.damp, want_objective=False)
    b.record(stream)
    torch.cuda.synchronize()
    t_e = a.elapsed_time(b) / 5 / 1e3
    flops_e = 2.0 * m * ng * (g * g + K * g)
    o = obj.cpu().numpy().tolist()
    line = {
        "metric": "OA-EM codebook initialisation time & weights/s",
        "value": m * n / dt, "unit": "weights/s", "n_gpus": 1, "steps": reps, "warmup": 1,
        "ms_per_step": dt * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64 (distances, sums, solves); bf16 Hessian products",
        "data": "synthetic (seeded)",
        "config": {"workload": f"{cfg.name} (OA-EM: groups of {g}, K {K}, M {M} codebooks, "
                               f"{T} EM rounds each, seeded initial groups)",
                   "m": m, "n": n, "ntok": N, "x_layout": xl, "input_sha256": hashes},
        "oaem": {"objective_per_stage": o, "info": P.read_result(res)["info"]},
        "roofline": {"bound": "alu (fp64 vector FMA)",
                     "kernel": "oaem_estep (+ its damping, load and norm table, timed as one "
                               "E-step-only call)",
                     "achieved": flops_e / t_e / 1e12, "peak": PEAK_F64_TFLOPS,
                     "unit": "TFLOP/s", "frac": flops_e / t_e / 1e12 / PEAK_F64_TFLOPS,
                     "traffic": None, "avg_call_ms": t_e * 1e3, "flops_per_estep": flops_e},
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    import synth
    if synth.config(args.config).wdtype != "bf16":
        print(f"bench.py: config {args.config} ({synth.config(args.config).name}, fp32 weights "
              "and activations) is a parity-test size; the timed layers are configs 2-5 "
              "(bf16 weights)", file=sys.stderr)
        sys.exit(2)
    if args.ssqr is not None and args.gpus == 1:
        ssqr_bench(args)
        return
    if args.oaem and args.gpus == 1:
        oaem_bench(args)
        return
    if args.library_gemm and args.gpus == 1:
        library_gemm_bench(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the "
              "quantizer's rows are independent, and a multi-GPU run would shard them "
              "with one all-reduce of H, which this library does not implement.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import post_weight_quantization_19_amd as P
    import synth

    peaks = None
    if not args.no_peaks:
        print("[bench] achievable peaks (probe)", file=sys.stderr, flush=True)
        peaks = measure_peaks()
    cfg = synth.config(args.config)
    m, n, N = cfg.m, cfg.n, cfg.ntok
    print(f"[bench] generating workload {cfg.name} m={m} n={n} ntok={N}", file=sys.stderr,
          flush=True)
    lay = synth.make_layer(cfg, keep_x_f32=False)
    hashes = input_hashes(lay)
    dev = torch.device("cuda:0")
    W = torch.from_numpy(lay.W_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    has_x = lay.X_bits is not None
    X = torch.from_numpy(lay.X_bits.view(np.int16)).view(torch.bfloat16).to(dev) if has_x else None
    xl = args.x_layout
    if has_x and xl == "tokens":
        X = X.t().contiguous()          # the same matrix, one row per token
    Hin = None if has_x else torch.from_numpy(lay.H).to(dev)
    if cfg.grid_kind == "colspacing":
        grid = P.Grid("colspacing", 0, 0, spacing_constant(cfg))
    else:
        grid = P.Grid(cfg.grid_kind, cfg.bits, cfg.group)
    prec = "f32" if has_x else "f64"     # the spectral layer is factored and swept in fp64
    order = args.order
    ws = P.workspace_for_layer(m, n, N, has_x, order, cfg.block, prec, dev)
    out = P.quant_layer(W, X=X, H=Hin, grid=grid, damp=cfg.damp, block=cfg.block, prec=prec,
                        workspace=ws, x_layout=xl, order=order)
    torch.cuda.synchronize()
    res0 = P.read_result(out["result"])
    if res0["info"] != 0:
        raise RuntimeError(f"Cholesky failed: {res0}")

    def step():
        P.quant_layer(W, X=X, H=Hin, grid=grid, damp=cfg.damp, block=cfg.block, prec=prec,
                      workspace=ws, out=out, x_layout=xl, order=order)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    # The dominant kernel (the Hessian SYRK tiles) records a HIP event pair
    # around each of its launches inside the timed steps, on the stream the
    # library launches it on.
    timer = P.HessianTileTimer(args.steps if has_x else 0)
    torch.cuda.synchronize()
    # one HIP event between consecutive steps on the library's stream (events
    # only: no synchronisation inside the timed region) for the per-step
    # median and minimum
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    with timer:
        t0 = time.perf_counter()
        step_ev[0].record()
        for i in range(args.steps):
            step()
            step_ev[i + 1].record()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
    step_ms = [step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(args.steps)]
    roofline = None
    if has_x:
        tiles_ms = timer.durations_ms()
        t_tiles = sum(tiles_ms) / len(tiles_ms) / 1e3
        flops_h = float(n) * (n + 1) * N
        achieved = flops_h / t_tiles / 1e12
        roofline = {"bound": "mfma",
                    "kernel": "syrk_tiles256 (bf16 SYRK tiles of H = 2 X X^T)",
                    "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": achieved / PEAK_BF16_TFLOPS,
                    "traffic": measured_traffic(cfg, xl),
                    "avg_launch_ms": t_tiles * 1e3, "launches_timed": len(tiles_ms),
                    "flops_per_launch": flops_h}

    stream = torch.cuda.current_stream()

    # the lazy updates and block sweeps are timed in a separate pass of as
    # many steps (their 2 x 63 event records per step would perturb the
    # headline timing above)
    nsweep, nupd, upd_flops_row = sweep_launches(n, cfg.block, prec)
    t_upd = P.KernelTimer("lazy_update", args.steps * nupd + 1)
    t_swp = P.KernelTimer("sweep_block", args.steps * nsweep + 1)
    torch.cuda.synchronize()
    with t_upd, t_swp:
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
    # one spare slot each: a launch schedule that differs from the model
    # above shows up as a count mismatch instead of silently dropped events
    if t_upd.count != args.steps * nupd or t_swp.count != args.steps * nsweep:
        raise RuntimeError(f"timed launches {t_upd.count} updates / {t_swp.count} sweeps, "
                           f"expected {args.steps * nupd} / {args.steps * nsweep}")

    # stage breakdown (same library calls, separately)
    def timed(fn, r=3):
        fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(r):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / r
    if has_x:
        H = torch.empty((n, n), dtype=torch.float32, device=dev)
        P.hessian_accum(X, H=H, x_layout=xl)
        t_hess = timed(lambda: P.hessian_accum(X, H=H, x_layout=xl))
    else:
        H, t_hess = Hin, 0.0
    Lf, dead, _ = P.damp_cholesky(H, damp=cfg.damp, prec=prec)
    s, z = (None, None) if cfg.grid_kind == "colspacing" else P.grid_steps(W, grid)
    t_chol = timed(lambda: P.damp_cholesky(H, damp=cfg.damp, prec=prec))
    t_sweep = timed(lambda: P.babai_sweep(W, Lf, grid, scales=s, zeros=z, block=cfg.block))
    t_order = None
    if order == "min_pivot":
        t_order = timed(lambda: P.min_pivot_order(H, damp=cfg.damp), r=2)
    if has_x:
        stored = "stored token-major [ntok, n]" if xl == "tokens" else "stored [n, ntok]"
        inputs = (f"X {n}x{N} bf16 {stored} " + ("Student-t(4)" if cfg.x_kind == "student_t" else
                                        "Laplace x LogNormal(0,1) channel scales")
                  + (f" with {cfg.outliers} outlier channels x20" if cfg.outliers else ""))
        grid_txt = f"{cfg.grid_kind} {cfg.bits}-bit group {cfg.group}"
    else:
        inputs = f"H {n}x{n} fp32 = L0 diag(k^-1.2) L0^T"
        grid_txt = f"column spacing c/l_kk, c = {grid.c:.6g}"

    # per-stage rooflines: SYRK and lazy update against their MFMA peaks,
    # Cholesky n^3/3 against its MFMA peak (stage time), the sweep's
    # ~14 bytes per weight against HBM
    pk = peaks or {}
    mf_peak, mf_key = (PEAK_F32_TFLOPS, "mfma_f32_tflops") if prec == "f32" else \
        (PEAK_F64_TFLOPS, "mfma_f64_tflops")
    upd_ms = sum(t_upd.durations_ms()) / args.steps
    swp_ms = sum(t_swp.durations_ms()) / args.steps
    upd_flops = m * upd_flops_row
    stages = {
        "cholesky": stage_roofline(n ** 3 / 3.0 / (t_chol / 1e3) / 1e12, mf_peak, pk.get(mf_key),
                                   "TFLOP/s", "mfma", n ** 3 / 3.0,
                                   "stage time (damp + factor), CUDA events"),
        "lazy_update": stage_roofline(upd_flops / (upd_ms / 1e3) / 1e12, mf_peak,
                                      pk.get(mf_key), "TFLOP/s", "mfma", upd_flops,
                                      f"library HIP events around each of the {nupd} updates "
                                      "of a step (separate pass)"),
        "sweep": stage_roofline(14.0 * m * n / (swp_ms / 1e3) / 1e9, PEAK_HBM_GBS,
                                pk.get("copy_gbs"), "GB/s", "hbm (latency: serial columns)",
                                14.0 * m * n,
                                f"library HIP events around each of the {nsweep} block sweeps "
                                "of a step (separate pass)"),
    }
    if roofline is not None:
        stages["hessian_tiles"] = stage_roofline(
            roofline["achieved"], PEAK_BF16_TFLOPS, pk.get("mfma_bf16_tflops"), "TFLOP/s",
            "mfma", roofline["flops_per_launch"], "library HIP events around each launch")
        roofline["achievable"] = pk.get("mfma_bf16_tflops")
        # the rate the device holds over a long launch of random-operand bf16
        # MFMAs of the form the SYRK issues (16x16x32; the power limit lowers
        # the clock); the SYRK runs as long
        sus = pk.get("mfma_bf16_16x16x32_sustained_random_tflops")
        roofline["achievable_sustained"] = sus
        roofline["frac_of_sustained"] = (roofline["achieved"] / sus) if sus else None
        stages["hessian_tiles"]["achievable_sustained"] = sus
        stages["hessian_tiles"]["frac_of_sustained"] = roofline["frac_of_sustained"]

    line = {
        "metric": METRIC,
        "value": m * n / dt,
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dt * 1e3,
        "step_ms": {"median": float(np.median(step_ms)), "min": min(step_ms),
                    "max": max(step_ms)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 products, f32 accumulate/factor/sweep" if has_x else
                  "f64 factor and sweep"),
        "data": "synthetic (seeded)",
        "config": {"workload": f"{cfg.name}: W {m}x{n} bf16, {inputs}; {grid_txt}, "
                               f"block {cfg.block}, damp {cfg.damp}"
                               + ("" if order == "back_to_front" else f", order {order}"),
                   "m": m, "n": n, "ntok": N, "x_layout": xl if has_x else None,
                   "layer_quantize_time_s": dt, "input_sha256": hashes},
        "roofline": roofline,
        "stages_ms": {"hessian_accum": t_hess, "damp_cholesky": t_chol,
                      "sweep_and_update": t_sweep, "lazy_updates_in_step": upd_ms,
                      "block_sweeps_in_step": swp_ms,
                      **({"min_pivot_order": t_order} if t_order is not None else {})},
        "stage_rooflines": stages,
        "achievable_peaks": peaks,
        "loss": res0["loss"], "bound": res0["bound"],
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(lay, cfg, args.cpu_token_fraction)
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        src.fill_(1.0)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
