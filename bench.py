"""Benchmark of the Muon per-owner update step on one MI355X.

A step is one muon_step over every matrix of the workload (momentum, norm,
Newton-Schulz, scale / weight decay / apply).  Inputs are synthetic and
already resident in HBM when timing starts.  Default workload: the
Llama-style 7B matrix set (32 layers, d=4096, ffn=11008; 160 bf16 matrices,
fp32 momentum), the largest matrix set that fits one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4] [--no-cpu-baseline]

Prints one JSON line.  `value` is the NS throughput of the whole step:
algorithmic (symmetric-aware) NS flops per step / measured step time.
"""
import argparse
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 400 for workloads 1 and 2, 20 otherwise)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: 40 for workloads 1 and 2 when timing, 5 otherwise)")
    ap.add_argument("--config", type=int, default=4, help="workload number 1..5 (default 4, the Llama-7B set)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tune", default="once", choices=["off", "once", "force"])
    ap.add_argument("--form", default="auto", choices=["auto", "direct", "gram"])
    ap.add_argument("--tile", type=int, default=None, help="force a tile plan (0..9)")
    ap.add_argument("--lanes", type=int, default=None, help="force the NS lane count (1..4)")
    ap.add_argument("--workspace-cap-gib", type=float, default=0,
                    help="plan workspace cap in GiB (0: the library default)")
    ap.add_argument("--adamw", action="store_true",
                    help="time the fused AdamW step over the non-matrix parameters of the "
                         "4-layer d=1024 transformer model (vocab 32000 embedding and classifier, norms)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time torch.matmul (hipBLASLt) on the workload's NS product shapes with random "
                         "bf16 operands, batched per shape as the library batches them")
    ap.add_argument("--owners", type=int, default=1,
                    help="assign the workload's matrices to this many owners (makespan-balanced) "
                         "and time one owner's share")
    ap.add_argument("--owner-rank", type=int, default=0, help="the owner whose share is timed")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run 2 steps and a 1 GiB device copy (for rocprofv3 --pmc passes), print nothing")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc output dirs (FETCH_SIZE, WRITE_SIZE passes over "
                         "--traffic-probe) into profiles/traffic.json for the workload's dominant kernel")
    ap.add_argument("--core-sweep", action="store_true",
                    help="time the NT core probe at its settled clock on random 8192 x 8192 x K bf16 "
                         "products for K = 8192, 4096, 2048, 1024 (per-tile start-up cost)")
    ap.add_argument("--epilogue-probe", action="store_true",
                    help="time the NT core probe on random 8192 x 8192 x 4096 bf16 products without an "
                         "output, with a bf16 row pass, with row and column passes, and with those "
                         "stores nontemporal (what writing a 256x256 tile costs)")
    ap.add_argument("--clock-from", metavar="PMC_DIR", default=None,
                    help="per-kernel engine clock and MFMA busy fraction from a rocprofv3 --pmc "
                         "pass with GRBM_GUI_ACTIVE and SQ_VALU_MFMA_BUSY_CYCLES")
    ap.add_argument("--kernel", default=None, help="kernel instance for --traffic-from, e.g. k_nt<128,128,bf16>")
    ap.add_argument("--cache", default=os.path.join(os.path.expanduser("~"), ".cache", "muon_mi355x",
                                                    "tune.txt"))
    ap.add_argument("--no-kernel-times", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="run the steps on a side stream with graph replay (muon_plan_set_graph)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured ceilings (dense bf16 MFMA loop, 1 GiB HBM copy)")
    args = ap.parse_args()
    # the sub-millisecond steps of workloads 1 and 2 get enough steps for a
    # timed region of about half a second; the --pmc probe keeps 5 + 2 steps
    short = args.config in (1, 2) and not args.adamw and not args.traffic_probe and not args.traffic_from
    if args.steps is None:
        args.steps = 400 if short else 20
    if args.warmup is None:
        args.warmup = 40 if short else 5
    return args


def source_digest():
    """sha256 of the kernel sources and of the planner (whose work-item order
    sets how much a launch re-reads): a recorded traffic figure is only valid
    for them."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "matrix_orthogonalizing_optimizer_muon_amd", "csrc")
    for f in ("kernels.hip", "mfma_nt.hpp", "kernels.hpp", "plan.cpp"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, workload, launches_per_step):
    """HBM bytes per launch of `kernel` from a committed counter summary
    (profiles/traffic.json, written from two rocprofv3 --pmc passes), or None
    when none matches this kernel, workload, kernel-source digest and launches
    per step (the plan's lane count sets how much one launch covers)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    digest = source_digest()
    for r in rec.get("entries", []):
        if (r.get("kernel") == kernel and r.get("workload") == workload and r.get("source") == digest
                and abs(r.get("launches_per_step", -1) - launches_per_step) < 1e-6):
            return {"fetch_bytes": r["fetch_bytes_per_launch"], "write_bytes": r["write_bytes_per_launch"],
                    "bytes": r["fetch_bytes_per_launch"] + r["write_bytes_per_launch"],
                    "copy_factor": r.get("copy_factor"), "source": digest}
    return None


COPY_BYTES = 1 << 30   # bytes read and written by the calibration copy
NT_CORE_DIM = 8192          # m = n = k of the NT core probe's product


def demangled(label):
    """Pattern of rocprofv3's name of a kernel instance label such as
    k_nt<128,128,bf16> or k_nt<256,256,bf16,qt> (the template also carries the
    block's wave grid and the k-major read flag)."""
    base, _, args = label.partition("<")
    args = args.rstrip(">").split(",") if args else []
    conv = {"bf16": "unsigned short", "f32": "float"}
    if base == "k_nt":
        qt = "true" if len(args) > 3 and args[3] == "qt" else "false"
        return re.compile(rf"k_nt<{args[0]}, {args[1]}, \d+, \d+, {conv[args[2]]}, {qt}>")
    return re.compile(re.escape(base))


def counter_rows(dirpath, counter):
    import csv
    import glob
    out = []
    for path in glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def write_traffic(args, wl, path=None):
    """Per-launch HBM bytes of one kernel from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled so that the calibration copy reads as COPY_BYTES.
    The passes ran --traffic-probe with the same --warmup (warmup + 2 steps, the
    plan from the tune cache), which gives the launches per step."""
    import statistics
    name = demangled(args.kernel)
    entry = {"kernel": args.kernel, "workload": wl.name, "source": source_digest()}
    for key, d, counter in (("fetch", args.traffic_from[0], "FETCH_SIZE"),
                            ("write", args.traffic_from[1], "WRITE_SIZE")):
        rows = counter_rows(d, counter)
        kern = [v for n, v in rows if name.search(n)]
        copy = [v for n, v in rows if "elementwise_kernel" in n]
        copy = [v for v in copy if v * 1024 > COPY_BYTES / 2]
        if not kern or not copy:
            raise SystemExit(f"{counter}: no rows for {name.pattern} or for the calibration copy in {d}")
        factor = COPY_BYTES / (statistics.median(copy) * 1024)
        entry[f"{key}_bytes_per_launch"] = statistics.mean(kern) * 1024 * factor
        entry[f"{key}_copy_factor"] = factor
        entry[f"{key}_dispatches"] = len(kern)
    if entry["fetch_dispatches"] != entry["write_dispatches"] or entry["fetch_dispatches"] % (args.warmup + 2):
        raise SystemExit(f"dispatch counts {entry['fetch_dispatches']} / {entry['write_dispatches']} "
                         f"do not fit {args.warmup} + 2 steps")
    entry["launches_per_step"] = entry["fetch_dispatches"] / (args.warmup + 2)
    entry["copy_factor"] = [entry["fetch_copy_factor"], entry["write_copy_factor"]]
    path = path or os.path.join(ROOT, "profiles", "traffic.json")
    rec = {"entries": []}
    if os.path.exists(path):
        with open(path) as fh:
            rec = json.load(fh)
    rec["entries"] = [e for e in rec["entries"]
                      if not (e["kernel"] == entry["kernel"] and e["workload"] == entry["workload"])]
    rec["entries"].append(entry)
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
    print(json.dumps(entry))


def core_sweep(torch, MU):
    """The NT core probe (the 256x256 main loop without an epilogue) on random
    N(0, 0.02^2) bf16 products 8192 x 8192 x K, K from 8192 down to 1024: a
    tile's start-up cost (block launch, the first k-tiles' copies) shows as
    the rate lost at short K.  About 0.2 s of untimed launches come first,
    then each K twice (about 60 ms each), in alternation."""
    gen = torch.Generator(device="cuda").manual_seed(11)
    n = NT_CORE_DIM
    p = (torch.randn(n, n, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    q = (torch.randn(n, n, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    views = {k: (p[:, :k].contiguous(), q[:, :k].contiguous()) for k in (8192, 4096, 2048, 1024)}
    MU.probe_nt_bf16(*views[8192], reps=100)
    MU.probe_nt_bf16(*views[8192], reps=100)
    rates = {k: [] for k in views}
    for _ in range(2):
        for k, (a, b) in views.items():
            reps = max(1, min(100, int(60e-3 / (2.0 * n * n * k / 1.3e15))))
            tf, _ = MU.probe_nt_bf16(a, b, reps=reps)
            rates[k].append(round(tf, 1))
    print(json.dumps({"metric": "NT core probe, TFLOP/s (settled clock)", "m": n, "n": n,
                      "operands": "random N(0, 0.02^2) bf16",
                      "k": {str(k): v for k, v in rates.items()}}))


def epilogue_probe(torch, MU):
    """The NT core probe (256x256 tiles, K = 4096 as in the Llama-7B set's A A
    and B X launches) with the outputs the NS products write: none (the sum
    of each thread's accumulators), a bf16 row pass (128 KB per tile), row and
    column passes (256 KB, a transposed copy or a mirrored tile), and the same
    with nontemporal stores.  About 0.2 s of untimed launches first; each
    variant twice in alternation, 100 timed launches after 20 untimed."""
    gen = torch.Generator(device="cuda").manual_seed(11)
    n, k = NT_CORE_DIM, 4096
    p = (torch.randn(n, k, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    q = (torch.randn(n, k, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    ct = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    MU.probe_nt_bf16(p, q, reps=100)
    MU.probe_nt_bf16(p, q, reps=100)
    names = {0: "no output", 1: "row pass", 2: "row and column passes", 3: "row and column passes, nontemporal"}
    rates = {m: [] for m in names}
    for _ in range(2):
        for mode in names:
            if mode == 0:
                MU.probe_nt_bf16(p, q, reps=20)
                tf, _ = MU.probe_nt_bf16(p, q, reps=100)
            else:
                MU.probe_nt_out_bf16(p, q, c, ct, mode=mode, reps=20)
                tf = MU.probe_nt_out_bf16(p, q, c, ct, mode=mode, reps=100)
            rates[mode].append(tf)
    waves = (n // 256) ** 2 / 256            # 256x256 tiles per CU per launch
    fl = 2.0 * n * n * k
    out = []
    for mode, name in names.items():
        best = max(rates[mode])
        out.append({"mode": mode, "epilogue": name, "tflops": [round(t, 1) for t in rates[mode]],
                    "us_per_tile": round(fl / (best * 1e12) / waves * 1e6, 2)})
    print(json.dumps({"metric": "NT core probe with output epilogues, TFLOP/s (settled clock)",
                      "m": n, "n": n, "k": k, "operands": "random N(0, 0.02^2) bf16", "variants": out}))


def clock_report(dirpath):
    """Engine clock and MFMA busy fraction per kernel from one rocprofv3 --pmc
    pass with GRBM_GUI_ACTIVE and SQ_VALU_MFMA_BUSY_CYCLES.  GRBM_GUI_ACTIVE
    sums the busy engine-clock cycles of all XCDs over a dispatch, so divided
    by the XCD count and the dispatch's duration it is the mean clock; the
    MFMA busy cycles are summed over all SIMDs.  At a clock f and busy fraction
    u the bf16 MFMA pipes issue PEAK * (f / 2.4 GHz) * u.  Dispatches shorter
    than 200 us are left out: the counters' window exceeds their timestamps."""
    import csv
    import glob
    import statistics
    xcc, simds = None, None
    disp = {}
    for path in glob.glob(os.path.join(dirpath, "**", "*agent_info.csv"), recursive=True):
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r.get("Name", "").startswith("gfx"):
                    xcc, simds = int(r["Num_Xcc"]), int(r["Simd_Count"])
    for path in glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as fh:
            for r in csv.DictReader(fh):
                d = disp.setdefault((path, r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
                d[r["Counter_Name"]] = float(r["Counter_Value"])
                d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    if not xcc or not disp:
        raise SystemExit(f"no agent info or counter rows in {dirpath}")
    groups = {}
    for d in disp.values():
        if "GRBM_GUI_ACTIVE" not in d or "SQ_VALU_MFMA_BUSY_CYCLES" not in d or d["ns"] < 200_000:
            continue
        name = d["name"].replace("void ", "").replace("muon::(anonymous namespace)::", "")
        m = re.match(r"[\w:]+(<[^()]*>)?", name)
        key = m.group(0) if m else name[:60]
        clk = d["GRBM_GUI_ACTIVE"] / xcc / d["ns"]               # GHz
        busy = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (d["GRBM_GUI_ACTIVE"] / xcc * simds)
        groups.setdefault(key, []).append((d["ns"] * 1e-3, clk, busy))
    out = []
    for key, v in sorted(groups.items(), key=lambda kv: -sum(x[0] for x in kv[1])):
        clk = [x[1] for x in v]
        busy = [x[2] for x in v]
        out.append({"kernel": key, "dispatches": len(v), "avg_us": round(statistics.mean(x[0] for x in v), 1),
                    "clock_ghz": round(statistics.mean(clk), 3), "clock_range": [round(min(clk), 3), round(max(clk), 3)],
                    "mfma_busy": round(statistics.mean(busy), 3), "busy_range": [round(min(busy), 3), round(max(busy), 3)],
                    "bf16_mfma_tflops_issued": round(PEAK_BF16_TFLOPS * statistics.mean(clk) / 2.4
                                                     * statistics.mean(busy), 1)})
    print(json.dumps({"source": dirpath, "xcds": xcc, "simds": simds, "kernels": out}))


def make_inputs(wl, torch):
    """Device-resident params / grads (workload's laws, fixed torch generator) and zero momenta."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234 + wl.cfg)
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    P, G, B = [], [], []
    for (r, c) in wl.shapes:
        w = torch.randn(r, c, device="cuda", generator=gen) * wl.w_scale
        if wl.grad_law == "student_t":
            # t(3) = N / sqrt(chi2_3 / 3)
            z = torch.randn(r, c, device="cuda", generator=gen)
            chi = sum(torch.randn(r, c, device="cuda", generator=gen) ** 2 for _ in range(3))
            g = z / torch.sqrt(chi / 3.0) * wl.grad_scale
        else:
            g = torch.randn(r, c, device="cuda", generator=gen) * wl.grad_scale
        P.append(w.to(dt).contiguous())
        G.append(g.to(dt).contiguous())
        B.append(torch.zeros(r, c, device="cuda", dtype=torch.float32))
    return P, G, B


def baseline_sample(wl):
    """Matrices the oracle leg times and checks, each with the number of
    matrices of the full set it stands for (the timed sample is scaled by
    these weights to a full step, labelled extrapolated when any weight > 1):
    one layer of each repeated block, every matrix of the small sets."""
    shapes = wl.shapes
    if wl.cfg == 3:      # backbone layer 0 (x24) and action-expert layer 0 (x12)
        return [(i, 24) for i in range(4)] + [(96 + i, 12) for i in range(4)]
    if wl.cfg == 4:      # layer 0: QKV, O, gate, up, down (x32)
        return [(i, 32) for i in range(5)]
    if wl.cfg == 5:      # expert 0's gate, up, down (x512 each) and one 512x16384 (x8)
        return [(0, 512), (1, 512), (2, 512), (len(shapes) - 8, 8)]
    return [(i, 1) for i in range(len(shapes))]


def parity_inputs(wl, sample, P, G, torch):
    """Writes the host-drawn seeded weights and gradients of the sampled
    matrices (step 0 of the workload's generator) over their device tensors;
    returns the stored host values for the oracle."""
    import numpy as np
    import workloads as WL
    host = {}
    for i, _w in sample:
        W, Gs = WL.draw(wl, i, 0, WL.KIND_W), WL.draw(wl, i, 0, WL.KIND_G)
        host[i] = (W, Gs)
        for st, t in ((W, P[i]), (Gs, G[i])):
            raw = np.ascontiguousarray(st.raw)
            src = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16) if st.dtype == WL.BF16 \
                else torch.from_numpy(raw)
            t.copy_(src.to(t.device))
    return host


def parity_step(plan, wl, sample, P, G, B, torch, h):
    """One step from zero momenta with the fp32 update of the sampled matrices
    captured; returns (U, W_new, momentum) per sampled matrix on the host."""
    cap = [None] * wl.n_matrices
    for i, _w in sample:
        cap[i] = torch.empty(wl.shapes[i], dtype=torch.float32, device="cuda")
    plan.set_update_capture(cap)
    plan.step(P, G, B, lr=h.lr, beta=h.beta, wd=h.wd, ns_steps=h.ns_steps, coeffs=h.coeffs)
    torch.cuda.synchronize()
    plan.set_update_capture(None)
    out = {}
    for i, _w in sample:
        wnew = P[i].view(torch.int16).cpu() if P[i].dtype == torch.bfloat16 else P[i].cpu()
        out[i] = (cap[i].cpu().numpy(), wnew.numpy(), B[i].cpu().numpy())
    return out, plan.flags()


def line_errors(d, ref):
    """Largest error of a row and of a column of d against ref: the norm of the
    line's error over max(the line's own norm, the RMS norm of the lines)."""
    import numpy as np
    out = []
    for ax in (1, 0):
        err = np.sqrt(np.sum(d * d, axis=ax))
        nrm = np.sqrt(np.sum(ref * ref, axis=ax))
        rms = np.sqrt(np.mean(nrm * nrm))
        out.append(float(np.max(err / np.maximum(nrm, rms))) if rms > 0 else 0.0)
    return out


def ulp_fraction_bf16(w_bits, ref_stored):
    """Fraction of bf16 weights within one bf16 ulp of the oracle's rounded W_new."""
    import numpy as np
    import workloads as WL
    w = WL.bf16_bits_to_f64(np.asarray(w_bits).view(np.uint16))
    _m, e = np.frexp(ref_stored)
    ulp = np.ldexp(1.0, e - 8)             # bf16: 8 significant bits
    ulp = np.where(ref_stored == 0, np.ldexp(1.0, -133), ulp)
    return float(np.mean(np.abs(w - ref_stored) <= ulp))


def cpu_baseline(wl, ns_flops_per_step, sample, host, gpu, flags):
    """The fp64 oracle on the host cores over a bounded sample of the same
    workload (one layer of each repeated block), scaled to the whole step by
    the sample weights; the same oracle results grade the GPU's parity step on
    those matrices (relative Frobenius error of the fp32 update, of the stored
    weight delta and of the momentum; largest row / column error; bf16
    fraction of weights within one ulp of the oracle's rounded value)."""
    import numpy as np
    from oracle import muon_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        threads = os.cpu_count()
    h = wl.hyper

    def rel(a, b):
        nb = np.linalg.norm(b)
        return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))

    oracle_s, ext_s, parity = 0.0, 0.0, []
    for i, weight in sample:
        W, Gs = host[i]
        t0 = time.perf_counter()
        ref = O.muon_step_ref(W.value, Gs.value, np.zeros(W.value.shape), lr=h.lr, beta=h.beta,
                              wd=h.wd, ns_steps=h.ns_steps, coeffs=h.coeffs, eps=h.eps,
                              param_dtype=wl.dtype)
        dt = time.perf_counter() - t0
        oracle_s += dt
        ext_s += dt * weight
        U, wnew, buf = gpu[i]
        U = U.astype(np.float64)
        if wl.dtype == "bf16":
            import workloads as WL
            wn = WL.bf16_bits_to_f64(wnew.view(np.uint16))
        else:
            wn = wnew.astype(np.float64)
        row, col = line_errors(U - ref["U"], ref["U"])
        rec = {"matrix": i, "shape": list(wl.shapes[i]), "oracle_s": round(dt, 2),
               "err_update": rel(U, ref["U"]), "err_dW": rel(wn - W.value, ref["U"]),
               "err_momentum": rel(buf.astype(np.float64), ref["buf_new"]),
               "max_row_err": row, "max_col_err": col}
        if wl.dtype == "bf16":
            rec["bf16_within_1ulp"] = ulp_fraction_bf16(wnew, ref["W_new_stored"])
        parity.append(rec)
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), None)
    except OSError:
        pass
    extrapolated = any(w > 1 for _i, w in sample)
    worst = {k: max(r[k] for r in parity) for k in ("err_update", "err_dW", "err_momentum",
                                                    "max_row_err", "max_col_err")}
    if wl.dtype == "bf16":
        worst["bf16_within_1ulp_min"] = min(r["bf16_within_1ulp"] for r in parity)
    return {"value": ns_flops_per_step / ext_s / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "ms_per_step": ext_s * 1e3, "extrapolated": extrapolated,
            "oracle_s": round(oracle_s, 2), "host_cpus": os.cpu_count(),
            "cpu_model": model, "blas_threads": int(threads),
            "sample": (f"{len(sample)} of the {wl.n_matrices} matrices of the {wl.name} set "
                       f"({', '.join(f'{wl.shapes[i][0]}x{wl.shapes[i][1]} x{w}' for i, w in sample)}), "
                       f"one step each, fp64 numpy, input generation excluded"
                       + ("; the full step is extrapolated from the sample by the weights" if extrapolated else "")),
            "parity": {"flags": flags, "worst": worst, "matrices": parity,
                       "how": "GPU step from zero momenta on the sampled matrices' seeded host inputs, "
                              "fp32 update captured, against the fp64 oracle on the same stored inputs"}}


ADAMW_VOCAB, ADAMW_D, ADAMW_LAYERS = 32000, 1024, 4


def bench_adamw(args, torch, MU):
    """The AdamW half of the hybrid on the 4-layer d=1024 transformer model's non-matrix
    parameters (bf16 params and grads, fp32 moments): one fused launch per step."""
    numels = [ADAMW_VOCAB * ADAMW_D, ADAMW_VOCAB * ADAMW_D] + [ADAMW_D] * (2 * ADAMW_LAYERS + 1)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(99)
    P = [(torch.randn(n, device="cuda", generator=gen) * 0.02).to(torch.bfloat16) for n in numels]
    G = [(torch.randn(n, device="cuda", generator=gen) * 0.02).to(torch.bfloat16) for n in numels]
    Mo = [torch.zeros(n, device="cuda") for n in numels]
    Vo = [torch.zeros(n, device="cuda") for n in numels]
    plan = MU.AdamWPlan(numels, "bf16")
    t = [0]

    def step():
        t[0] += 1
        plan.step(P, G, Mo, Vo, lr=2e-2, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.01, step=t[0])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    elems = sum(numels)
    nbytes = elems * (2 + 2 + 4 + 4 + 2 + 4 + 4)   # p, g, m, v in; p, m, v out
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "fused AdamW step GB/s (% of MI355X 8 TB/s HBM)", "value": round(gbs, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"non-matrix parameters of the 4-layer d={ADAMW_D} transformer: "
                               f"{ADAMW_VOCAB}x{ADAMW_D} embedding and classifier, "
                               f"{2 * ADAMW_LAYERS + 1} norm vectors",
                   "tensors": len(numels), "elements": elems, "bytes_per_step": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}}))
    plan.close()


def bench_vendor_gemm(args, wl, torch):
    """Reference rates of the vendor GEMM (torch.matmul on ROCm, hipBLASLt) for
    the products of one NS step of the workload, per canonical shape: X X^T
    (m x n times n x m; the full product, the library computes the upper
    triangle), A A (m x m times m x m) and B X (m x m times m x n), batched
    over the matrices of that shape, random N(0, 1) bf16 operands, both operands
    contiguous, timed at the settled clock.  Flops counted as issued by the
    vendor product (2 m n k)."""
    shapes = {}
    for r, c in wl.shapes:
        shapes.setdefault((min(r, c), max(r, c)), 0)
        shapes[(min(r, c), max(r, c))] += 1
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    out = []
    for (m, n), count in sorted(shapes.items()):
        batch = min(count, 32)
        X = torch.randn(batch, m, n, device="cuda", generator=gen).to(torch.bfloat16)
        Xt = X.transpose(1, 2).contiguous()
        A = torch.randn(batch, m, m, device="cuda", generator=gen).to(torch.bfloat16)
        prods = (("X X^T", X, Xt, 2.0 * m * m * n), ("A A", A, A, 2.0 * m * m * m), ("B X", A, X, 2.0 * m * m * n))
        for name, p, q, fl in prods:
            for _ in range(3):
                torch.matmul(p, q)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            torch.matmul(p, q)
            e1.record()
            torch.cuda.synchronize()
            one = max(e0.elapsed_time(e1), 1e-3)
            # sustained MFMA work settles the part's clock within a few ms: about
            # 0.1 s of untimed calls, then at least 20 ms (and 10 calls) timed
            for _ in range(min(20000, int(100.0 / one))):
                torch.matmul(p, q)
            reps = max(10, min(20000, int(20.0 / one)))
            e0.record()
            for _ in range(reps):
                torch.matmul(p, q)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            out.append({"shape": f"{m}x{n}", "product": name, "batch": batch, "ms": round(ms, 4),
                        "tflops": round(batch * fl / (ms * 1e-3) / 1e12, 1)})
        del X, Xt, A
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "vendor GEMM reference (torch.matmul / hipBLASLt), TFLOP/s",
                      "workload": wl.name, "operands": "random N(0,1) bf16, contiguous",
                      "products": out}))


def owner_share(args, wl, MU):
    """The matrices one owner gets when the workload is balanced over
    args.owners owners by estimated step time (plan costs, muon_assign_owners)."""
    import dataclasses
    if not 0 <= args.owner_rank < args.owners:
        raise SystemExit("--owner-rank must be in [0, --owners)")
    full = MU.MuonPlan(wl.shapes, wl.dtype, tune=args.tune, cache_path=args.cache, form=args.form,
                       tile=args.tile, lanes=args.lanes)
    costs = [full.matrix_cost(i) for i in range(wl.n_matrices)]
    full.close()
    owner, span, optimal = MU.assign_owners(costs, args.owners)
    idx = [i for i, o in enumerate(owner) if o == args.owner_rank]
    if not idx:
        raise SystemExit(f"owner {args.owner_rank} of {args.owners} gets no matrix")
    share = dataclasses.replace(wl, shapes=tuple(wl.shapes[i] for i in idx),
                                name=f"{wl.name}, owner {args.owner_rank} of {args.owners}")
    info = {"owners": args.owners, "rank": args.owner_rank, "matrices": len(idx),
            "est_share_us": round(sum(costs[i] for i in idx), 1), "est_makespan_us": round(span, 1),
            "est_lower_bound_us": round(max(max(costs), sum(costs) / args.owners), 1),
            "optimal": optimal}
    return share, info


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs the per-owner step on one GPU; multi-GPU runs are not "
                                   "supported (matrices would be sharded whole across owners)"}))
        sys.exit(2)
    import workloads as WL
    wl = WL.workload(args.config)
    if args.traffic_from:
        write_traffic(args, wl)
        return
    if args.clock_from:
        clock_report(args.clock_from)
        return
    import torch
    import matrix_orthogonalizing_optimizer_muon_amd as MU

    torch.cuda.init()
    if args.adamw:
        bench_adamw(args, torch, MU)
        return
    if args.vendor_gemm:
        bench_vendor_gemm(args, wl, torch)
        return
    if args.core_sweep:
        core_sweep(torch, MU)
        return
    if args.epilogue_probe:
        epilogue_probe(torch, MU)
        return
    os.makedirs(os.path.dirname(args.cache), exist_ok=True)
    owner_info = None
    if args.owners > 1:
        wl, owner_info = owner_share(args, wl, MU)
    t0 = time.perf_counter()
    plan = MU.MuonPlan(wl.shapes, wl.dtype, tune=args.tune, cache_path=args.cache, form=args.form,
                       tile=args.tile, lanes=args.lanes, workspace_cap=int(args.workspace_cap_gib * (1 << 30)))
    plan_s = time.perf_counter() - t0
    info = plan.info()
    choices = {}
    for i, (r, c) in enumerate(wl.shapes):
        ch = plan.matrix_choice(i)
        choices.setdefault(f"{min(r, c)}x{max(r, c)}", f"{ch['form']}/tile{ch['tile']}")
    P, G, B = make_inputs(wl, torch)
    h = wl.hyper
    # parity step of the oracle leg: seeded host inputs on a sample of the
    # matrices, one step from zero momenta, before any other step
    parity = None
    if not args.no_cpu_baseline and not args.traffic_probe and not args.graph:
        sample = baseline_sample(wl)
        host = parity_inputs(wl, sample, P, G, torch)
        gpu, flags = parity_step(plan, wl, sample, P, G, B, torch, h)
        parity = (sample, host, gpu, flags)
        print(f"# parity step done on {len(sample)} sampled matrices", file=sys.stderr, flush=True)
    if args.graph:
        # graph capture needs a stream other than the null stream; the inputs
        # were made on the default stream, so let that work finish first
        torch.cuda.synchronize()
        torch.cuda.set_stream(torch.cuda.Stream())
        plan.set_graph(True)
    stream = torch.cuda.current_stream()

    def step():
        plan.step(P, G, B, lr=h.lr, beta=h.beta, wd=h.wd, ns_steps=h.ns_steps, coeffs=h.coeffs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.traffic_probe:
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)   # one plain read and one plain write of COPY_BYTES
        torch.cuda.synchronize()
        plan.close()
        return
    print(f"# warmup done ({args.warmup} steps), timing {args.steps}", file=sys.stderr, flush=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per = []
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        step()
        s1.record(stream)
        per.append((s0, s1))
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = e0.elapsed_time(e1)
    ms = total_ms / args.steps
    step_ms = sorted(a.elapsed_time(b) for a, b in per)
    p = lambda q: step_ms[min(len(step_ms) - 1, int(q * len(step_ms)))]

    # per-kernel dispatch times over as many steps again, after the timed
    # region: while profiling the library records each kernel's dispatch start
    # and end and runs the NS lanes one after another, so each time is the
    # kernel's own
    kt = []
    if not args.no_kernel_times:
        plan.set_profiling(True)
        plan.kernel_times(reset=True)
        for _ in range(args.steps):
            step()
        kt = plan.kernel_times(reset=False)
        plan.kernel_times(reset=True)
        plan.set_profiling(False)
    # measured ceilings of this device, after the timed region: a dense bf16
    # MFMA loop without memory traffic, and a 1 GiB device-to-device copy
    ceil = None
    if not args.no_ceilings:
        mfma_tf, _ = MU.probe_mfma_bf16(iters=100000)              # about 17 ms
        mfma_sus, _ = MU.probe_mfma_bf16(iters=1000000)            # about 170 ms
        mfma_rnd, _ = MU.probe_mfma_bf16(iters=1000000, random_operands=True)
        # the NT contraction core alone (no epilogue) on a random 8192^3 product
        gen = torch.Generator(device="cuda").manual_seed(11)
        pa = (torch.randn(NT_CORE_DIM, NT_CORE_DIM, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
        qa = (torch.randn(NT_CORE_DIM, NT_CORE_DIM, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
        # sustained MFMA work lowers the part's clock within a few ms (its power
        # limit), so 100 untimed launches (about 0.1 s) come before the 100 timed
        MU.probe_nt_bf16(pa, qa, reps=100)
        nt_core, _ = MU.probe_nt_bf16(pa, qa, reps=100)
        del pa, qa
        a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        copy_gbs = MU.probe_hbm_copy(b, a, reps=10)
        del a, b
        ceil = {"mfma_bf16_tflops": round(mfma_tf, 1), "mfma_bf16_tflops_sustained": round(mfma_sus, 1),
                "mfma_bf16_tflops_random_operands": round(mfma_rnd, 1),
                "nt_core_bf16_tflops": round(nt_core, 1),
                "hbm_copy_gbs": round(copy_gbs, 1),
                "how": "muon_probe_mfma_bf16 (2 blocks of 4 waves per CU, 4 independent "
                       "32x32x16 bf16 MFMA chains per wave, no memory traffic; 1e5 and 1e6 "
                       "rounds; and 1e6 rounds with eight random operand pairs per wave, "
                       "muon_probe_mfma_bf16_random, the switching activity of real data "
                       "under the part's power limit), muon_probe_nt_bf16 (the 256x256 NT "
                       "contraction core without an epilogue on a random 8192^3 bf16 product, "
                       "100 launches after 100 untimed ones) and muon_probe_hbm_copy (1 GiB copy, read + written bytes, "
                       "best of 8 launch variants)"}
    ns_flops = info["ns_flops_min"]
    bf16 = wl.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS
    # per kernel instance (what rocprofv3 lists as one kernel), summed over stages
    by_kernel = {}
    for k in kt:
        d = by_kernel.setdefault(k["kernel"], {"launches": 0, "total_ms": 0.0, "flops": 0.0,
                                               "bytes": 0.0, "stages": []})
        d["launches"] += k["launches"]
        d["total_ms"] += k["total_ms"]
        d["flops"] += k["flops"]
        d["bytes"] += k["bytes"]
        d["stages"].append(k["name"])
    ns_kern = {n: d for n, d in by_kernel.items() if d["flops"] > 0}
    ew_kern = {n: d for n, d in by_kernel.items() if d["bytes"] > 0}
    ns_ms = sum(d["total_ms"] for d in ns_kern.values()) / max(args.steps, 1)
    roofline = None
    if ns_kern:
        name, dom = max(ns_kern.items(), key=lambda kv: kv[1]["total_ms"])
        avg_ms = dom["total_ms"] / dom["launches"]
        fpl = dom["flops"] / dom["launches"]
        ach = fpl / (avg_ms * 1e-3) / 1e12
        tr = traffic_for(name, wl.name, dom["launches"] / args.steps)
        roofline = {"bound": "mfma", "kernel": name, "stages": sorted(set(dom["stages"])),
                    "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(ach / peak, 4),
                    # measured HBM bytes per launch (fetch + write), null when
                    # no counter record matches these kernel sources and plan
                    "traffic": tr["bytes"] if tr else None,
                    "traffic_detail": tr,
                    "avg_launch_us": round(avg_ms * 1e3, 2), "flops_per_launch": fpl,
                    "launches_per_step": dom["launches"] / args.steps,
                    "share_of_step": round(dom["total_ms"] / args.steps / ms, 4),
                    "lanes": info["n_lanes"]}
        # the same launches credited with GEMM-equivalent flops (the symmetric
        # products X X^T and A A counted as whole products, 2 m^2 n and 2 m^3)
        geq = sum(k["flops"] * (2.0 if k["name"] in ("ns_syrk", "ns_comb") else 1.0)
                  for k in kt if k["kernel"] == name)
        a_geq = geq / dom["launches"] / (avg_ms * 1e-3) / 1e12
        roofline["achieved_gemm_equivalent"] = round(a_geq, 2)
        roofline["frac_gemm_equivalent"] = round(a_geq / peak, 4)
        if ceil and bf16:
            roofline["frac_of_measured_mfma"] = round(ach / ceil["mfma_bf16_tflops"], 4)
            roofline["frac_of_measured_mfma_random_operands"] = round(
                ach / ceil["mfma_bf16_tflops_random_operands"], 4)
            roofline["frac_of_nt_core"] = round(ach / ceil["nt_core_bf16_tflops"], 4)
    # every NS kernel instance against the same peak (profiling pass, per launch)
    ns_rooflines = []
    for n, d in sorted(ns_kern.items(), key=lambda kv: -kv[1]["total_ms"]):
        a_ms = d["total_ms"] / d["launches"]
        a = d["flops"] / d["launches"] / (a_ms * 1e-3) / 1e12
        ns_rooflines.append({"kernel": n, "stages": sorted(set(d["stages"])), "achieved": round(a, 2),
                             "frac": round(a / peak, 4), "avg_launch_us": round(a_ms * 1e3, 2),
                             "launches_per_step": d["launches"] / args.steps,
                             "ms_per_step": round(d["total_ms"] / args.steps, 4)})
    ew = {}
    for n, d in ew_kern.items():
        avg_ms = d["total_ms"] / d["launches"]
        gbs = d["bytes"] / d["launches"] / (avg_ms * 1e-3) / 1e9
        ew[n] = {"GB/s": round(gbs, 1), "frac_of_hbm": round(gbs / PEAK_HBM_GBS, 4),
                 "avg_launch_us": round(avg_ms * 1e3, 2), "bytes_per_launch": d["bytes"] / d["launches"],
                 "traffic": traffic_for(n, wl.name, d["launches"] / args.steps)}
        if ceil:
            ew[n]["frac_of_measured_copy"] = round(gbs / ceil["hbm_copy_gbs"], 4)
    value = ns_flops / (ms * 1e-3) / 1e12
    # direct-form GEMM-equivalent NS flops, T (4 m^2 n + 2 m^3) per matrix (m the
    # smaller side): every product counted whole, whatever form or symmetry
    # the plan uses
    geq_flops = float(sum(h.ns_steps * (4.0 * min(r, c) ** 2 * max(r, c) + 2.0 * min(r, c) ** 3)
                          for r, c in wl.shapes))
    geq_value = geq_flops / (ms * 1e-3) / 1e12
    out = {
        "metric": "Muon optimizer-step ms + NS TFLOP/s (% of MI355X bf16 MFMA peak)",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "matrices": wl.n_matrices, "elements": wl.n_elements,
                   **({"owner": owner_info} if owner_info else {}),
                   "ns_steps": h.ns_steps, "coeffs": list(h.coeffs), "lr": h.lr, "beta": h.beta,
                   "wd": h.wd, "parallelism": "single GPU"},
        "step_ms_p10_p50_p90": [round(p(0.1), 4), round(p(0.5), 4), round(p(0.9), 4)],
        "ns_flops_per_step": ns_flops, "ns_flops_issued_per_step": info["ns_flops_issued"],
        # NS kernels' own dispatch times summed over a step (profiling pass:
        # lanes one after another), and the rate over that sum
        "ns_kernel_ms_per_step_serial": round(ns_ms, 4) if kt else None,
        "ns_tflops_kernels_serial": round(ns_flops / (ns_ms * 1e-3) / 1e12, 2) if ns_ms else None,
        "step_frac_of_peak": round(value / peak, 4),
        "ns_flops_gemm_equivalent_per_step": geq_flops,
        "step_tflops_gemm_equivalent": round(geq_value, 2),
        "step_frac_of_peak_gemm_equivalent": round(geq_value / peak, 4),
        "elementwise": ew, "roofline": roofline, "ns_kernel_rooflines": ns_rooflines, "ceilings": ceil,
        "kernels": [{"stage": k["name"], "kernel": k["kernel"],
                     "launches_per_step": k["launches"] / args.steps,
                     "ms_per_step": round(k["total_ms"] / args.steps, 4)} for k in kt],
        "plan": {"choices": choices, "groups": info["n_groups"], "chunks": info["n_chunks"], "gram": info["n_gram"],
                 "lanes": info["n_lanes"],
                 "workspace_gb": round(info["workspace_bytes"] / 1e9, 3),
                 "create_s": round(plan_s, 3), "hash": info["plan_hash"], "graph_replay": args.graph},
        "wall_s_timed": round(wall, 3),
        "cpu_baseline": None,
    }
    if parity is not None:
        print("# cpu baseline (fp64 oracle on the sampled matrices)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, ns_flops, *parity)
    plan.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
