"""Benchmark of the block-scaled FP4 quantizer on one MI355X.

One step = one fp4q_quantize call on the headline workload: NVFP4 ScaleSweep
with importance-weighted MSE (offsets [-8, 7]) of a bf16 14336x4096 weight
matrix (Student-t(4) * 0.02, lognormal(0,1) per-column importance), global
scale computed on the device -- a pass of partial maxima, then the sweep
quantizer, whose workgroups each reduce those maxima to S.  Inputs are
resident in HBM before timing starts; the step cycles
through several input copies so that no step reads data a previous step left
in the 256 MB Infinity Cache.

Printed: one JSON line (rank 0).  `value` is quantized Gelem/s of the whole
call; `roofline` is the dominant kernel (the sweep quantizer) timed alone
with HIP events on the stream it runs on.  That kernel is bound by its
vector-ALU work, so the roofline is the VALU's: the exact estimate of all 16
candidates needs 48 binary32 operations, 8 FP4 encodes and 8 FP4 decodes per
element, the conversions weighted by their issue cost relative to an FMA
(measured by block_scaled_fp4_fp4q_amd/valu_issue, a microbenchmark run as a
child process), against the published 157.3 TFLOP/s binary32 vector peak
(78.6 T FMA lane-ops/s); the 8 TB/s HBM roofline of the same kernel is
reported beside it;
`cpu_baseline` is the CPU oracle on a bounded row sample of the same
workload, and `parity_sample` compares the GPU's bytes on those rows with the
oracle's; every other workload carries a `parity_sample` of its leading rows
(about 2^18 elements) as well.  `configs` times the other workloads with their own rules (c1
NVFP4 AbsMax and ScaleSweep MSE, c3 MXFP4 with and without a 32-point
Hadamard, c4 IF4); `extensions` times Four Over Six, the MXFP4 exponent
window, the IF4 pattern window and the FOCUS deploy encode.  `secondary` holds the 2 GiB
KV-cache workload (NVFP4 ScaleSweep MSE
[-3, 7] with a fused 16-point Hadamard; quantize and dequantize timed
separately).  A plain 1 GiB device copy is the achievable-bandwidth yardstick.
"""
import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "quantized Gelem/s + achieved HBM GB/s (% of peak), NVFP4 ScaleSweep MSE"


COUNTERS = os.path.join(ROOT, "profiles", "nvfp4_sweep_wmse_hbm_counters.md")
VALU_COUNTERS = os.path.join(ROOT, "profiles", "nvfp4_sweep_valu_counters.md")
VALU_ISSUE = os.path.join(ROOT, "block_scaled_fp4_fp4q_amd", "valu_issue")
# published binary32 vector peak, 157.3 TFLOP/s, as FMA lane-ops/s: 256 CUs x
# 4 SIMDs x 2.4 GHz x 32 lanes per cycle (a wave64 FMA issues in 2 cycles)
PEAK_FP32_LANE_OPS = 157.3e12 / 2
# per element of the sweep over 16 patterns in 8 exactly doubling pairs: per
# pair, y = |x| r and b y (shared), two residual FMAs and two accumulating
# FMAs (6 binary32 ops), one encode and one decode instruction (each converts
# two elements of one candidate, two candidates per pair)
SWEEP16_MIX = {"fp32": 48, "encode": 8, "decode": 8}
KERNEL_SOURCES = ["block_scaled_fp4_fp4q_amd/csrc/fp4q_kernels.hip",
                  "block_scaled_fp4_fp4q_amd/csrc/fp4q_device.h"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the sweep kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary, or None when the kernel sources changed
    since those counters were taken."""
    import re
    try:
        text = open(COUNTERS).read()
    except OSError:
        return None
    h = re.search(r"Kernel sources sha256\[:16\] = `([0-9a-f]+)`", text)
    t = re.search(r"traffic_bytes_per_launch \S+ = (\d+)", text)
    if not h or not t or h.group(1) != kernel_source_hash():
        return None
    return int(t.group(1))


def measured_valu():
    """Executed VALU lane-ops per element, AMD's VALUBusy and the fraction of
    the VALU's measured issue capacity used by the sweep kernel, from the
    committed rocprofv3 SQ counter summary, or None when the kernel sources
    changed since."""
    import re
    try:
        text = open(VALU_COUNTERS).read()
    except OSError:
        return None
    h = re.search(r"Kernel sources sha256\[:16\] = `([0-9a-f]+)`", text)
    ops = re.search(r"lane_ops_per_elem nvfp4_sweep_wmse_bf16_14336x4096 = ([0-9.]+)", text)
    busy = re.search(r"valu_busy nvfp4_sweep_wmse_bf16_14336x4096 = ([0-9.]+)", text)
    util = re.search(r"issue_capacity_used nvfp4_sweep_wmse_bf16_14336x4096 = ([0-9.]+)", text)
    if not h or not ops or not busy or not util or h.group(1) != kernel_source_hash():
        return None
    return {"lane_ops_per_elem": float(ops.group(1)), "valu_busy": float(busy.group(1)),
            "issue_capacity_used": float(util.group(1)),
            "source": "profiles/nvfp4_sweep_valu_counters.md (SQ_INSTS_VALU, "
                      "SQ_ACTIVE_INST_VALU, GRBM_GUI_ACTIVE)"}


def valu_issue_costs():
    """Issue cost of one wave64 instruction per class, in core-clock cycles of
    one SIMD, measured by the valu_issue microbenchmark in a child process; None
    when it is not built or fails."""
    if not os.path.exists(VALU_ISSUE):
        log(f"{VALU_ISSUE} is not built: no ALU roofline (run __graft_entry__.build())")
        return None
    try:
        r = subprocess.run([VALU_ISSUE], capture_output=True, text=True, timeout=120, check=True)
        return json.loads(r.stdout.strip().splitlines()[-1])
    except (subprocess.SubprocessError, ValueError, IndexError) as e:
        log(f"valu_issue failed: {e}")
        return None


def roofline(n, ms_k, kernel_gbps, bytes_per_elem, issue):
    """The sweep kernel against the VALU roof (its binding resource), with the
    HBM roof beside it; the HBM roof alone when the issue costs are missing."""
    hbm = {"bound": "hbm", "achieved": kernel_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
           "frac": kernel_gbps / PEAK_HBM_GBPS,
           "algorithmic_bytes_per_launch": n * bytes_per_elem}
    common = {"kernel": "nvfp4_sweep<bf16, no rotation, wmse>", "kernel_ms": ms_k,
              "traffic": measured_traffic(),
              "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                              "copy-calibrated)",
              "valu_counters": measured_valu()}
    if issue is None:
        return {**hbm, **common}
    c = issue["cycles_per_wave64_instr"]
    w_enc = c["v_cvt_scalef32_pk_fp4_f32"] / c["v_fma_f32"]
    w_dec = c["v_cvt_scalef32_pk_f32_fp4"] / c["v_fma_f32"]
    ops = SWEEP16_MIX["fp32"] + SWEEP16_MIX["encode"] * w_enc + SWEEP16_MIX["decode"] * w_dec
    achieved = n * ops / (ms_k * 1e-3) / 1e12
    peak = PEAK_FP32_LANE_OPS / 1e12
    return {"bound": "alu", "achieved": achieved, "peak": peak,
            "unit": "T VALU lane-ops/s (binary32 FMA equivalents)", "frac": achieved / peak,
            **common,
            "algorithmic_lane_ops_per_elem": ops,
            "algorithmic_lane_ops_per_launch": n * ops,
            "instruction_mix_per_elem": SWEEP16_MIX,
            "conversion_weights": {"encode": w_enc, "decode": w_dec},
            "issue_costs": issue,
            "hbm": hbm}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=200,
                   help="untimed steps first (the core clock settles over ~20-30 ms of load, "
                        "about 150 steps)")
    p.add_argument("--copies", type=int, default=4, help="input copies cycled per step")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--no-cpu", action="store_true",
                   help="skip the CPU oracle leg: the baseline timing and every parity sample")
    p.add_argument("--cpu-rows", type=int, default=6144)
    p.add_argument("--no-issue", action="store_true",
                   help="skip the VALU issue-cost microbenchmark (the roofline falls back to HBM)")
    return p.parse_args()


def to_dev(x, dev):
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(x).to(dev)


SETTLE_MS = 30.0  # GPU time of untimed calls before a secondary timing (clock settling)


def event_time(fn, steps, warmup, settle_ms=0.0):
    """Average ms per call of fn(i) over `steps` calls, HIP events on the
    current stream (the stream every library call is issued on).  `warmup`
    untimed calls come first; with settle_ms > 0, more untimed calls follow
    until about that much GPU time has run, so that a short workload timed
    after an idle stretch (input generation on the host) is not measured
    while the core clock is still rising, and at least settle_ms / 3 of calls
    are timed."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    if settle_ms > 0.0:
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(3):
            fn(i)
        e.record()
        torch.cuda.synchronize()
        per = max(s.elapsed_time(e) / 3, 1e-3)
        for i in range(int(settle_ms / per) + 1):
            fn(i)
        torch.cuda.synchronize()
        # and a timed region of at least a third of that, so that a short
        # workload is not timed over a fraction of a millisecond
        steps = max(steps, int(settle_ms / 3 / per) + 1)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    s.record()
    for i in range(steps):
        fn(i)
    e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return s.elapsed_time(e) / steps, wall


SAMPLE_ELEMS = 1 << 18  # elements of the leading rows re-quantized by the oracle per workload


def sample_parity(x_h, spec, codes, scales, gs, importance=None, relaxed=None):
    """The oracle on the leading rows of a workload (about SAMPLE_ELEMS
    elements), under the global scale the GPU computed for the whole tensor,
    against the GPU's bytes for those rows: mismatch counts and the oracle's
    near-tie blocks (second-best error within 1e-6 relative of the best)."""
    from oracle import ref
    rows, cols = x_h.shape
    r = max(1, min(rows, SAMPLE_ELEMS // cols))
    xs = np.ascontiguousarray(x_h[:r])
    S = None if spec.format == 1 else float(gs.item())  # MXFP4 has no global scale
    cores = len(os.sched_getaffinity(0))
    if relaxed is not None:
        coef, group = relaxed
        want = ref.quantize_relaxed(xs, np.ascontiguousarray(coef[:r]), group, fmt=spec.format,
                                    global_scale=S, nthreads=cores)
    else:
        want = ref.quantize(xs, fmt=spec.format, rule=spec.scale_rule, objective=spec.objective,
                            window=(spec.sweep_lo, spec.sweep_hi), rotate=spec.rotate,
                            global_scale=S, importance=importance, nthreads=cores, errors=True)
    nb = r * cols // spec.block
    got_s = scales.cpu().numpy()[:nb]
    got_c = codes.cpu().numpy()[: r * cols // 2]
    out = {"rows": r, "blocks": nb, "scale_mismatches": int(np.sum(got_s != want["scales"])),
           "code_bytes_mismatched": int(np.sum(got_c != want["codes"]))}
    if "best" in want:
        live = want["best"] > 0
        gap = np.where(live, (want["second"] - want["best"]) / np.where(live, want["best"], 1),
                       np.inf)
        out["oracle_near_tie_blocks"] = int(np.sum(gap < 1e-6))
    return out


def extensions(args, B, synth, dev, x2, imp, ws, x2_h, imp_h):
    """The other workloads (c1, c3, c4) and the rules beyond ScaleSweep, each
    timed as one quantize call (global scale computed) on its workload, with
    its error next to a baseline rule's and, unless --no-cpu, the oracle's
    bytes on a row sample.  Returns (configs, extensions)."""
    import torch
    steps = max(5, args.steps // 5)
    out = {}

    def run(name, workload, x, spec, importance=None, base_spec=None, err_imp=None, rotate=0,
            bytes_per_elem=None, base_rotate=None, x_h=None, imp_host=None):
        rows, cols = x.shape
        n = rows * cols
        codes = torch.empty(n // 2, dtype=torch.uint8, device=dev)
        scales = torch.empty(n // spec.block, dtype=torch.uint8, device=dev)
        gs = torch.empty(1, dtype=torch.float32, device=dev)
        # enough copies (>= 512 MiB) that no step finds its input in the Infinity Cache
        ncopy = max(2, -(-(512 << 20) // (x.numel() * x.element_size())))
        xc = [x] + [x.clone() for _ in range(ncopy - 1)]
        ms, _ = event_time(lambda i: B.fp4q_quantize(spec, xc[i % ncopy], importance, codes, scales,
                                                     gs, ws), steps, 2, SETTLE_MS)
        del xc
        # the oracle on a row sample, before the baseline below overwrites gs
        ps = None
        if x_h is not None and not args.no_cpu:
            ps = sample_parity(x_h, spec, codes, scales, gs, importance=imp_host)
        espec = B.make_spec(spec.format, rotate=rotate)
        e = B.fp4q_error(espec, x, err_imp, codes, scales, gs, ws)
        base_rot = rotate if base_rotate is None else base_rotate
        bcodes = torch.empty(n // 2, dtype=torch.uint8, device=dev)
        bscales = torch.empty(n // base_spec.block, dtype=torch.uint8, device=dev)
        B.fp4q_quantize(base_spec, x, importance, bcodes, bscales, gs, ws)
        eb = B.fp4q_error(B.make_spec(base_spec.format, rotate=base_rot), x, err_imp, bcodes, bscales,
                          gs, ws)
        k = 1 if err_imp is not None else 0
        gbps = n * bytes_per_elem / (ms * 1e-3) / 1e9
        out[name] = {"workload": workload, "quantize_ms": ms,
                     "quantize_gelem_s": n / (ms * 1e-3) / 1e9, "quantize_gbps": gbps,
                     "quantize_frac_of_peak": gbps / PEAK_HBM_GBPS,
                     "error": e[k], "baseline_error": eb[k],
                     "error_kind": "wmse" if k else "mse"}
        if ps is not None:
            out[name]["parity_sample"] = ps
        log(f"{name}: {ms:.3f} ms, {gbps:.0f} GB/s, err {e[k]:.6g} vs baseline {eb[k]:.6g}"
            + (f", parity {out[name]['parity_sample']}" if "parity_sample" in out[name] else ""))
        del codes, scales, bcodes, bscales

    nv = 2 * 2.0 + 0.5 + 1.0 / 16          # global max read + read + codes + scales
    mx = 2.0 + 0.5 + 1.0 / 32

    # ---- the other configurations with their own rules
    x1_h = synth.c1()
    x1 = to_dev(x1_h, dev)
    f1 = 2 * 4.0 + 0.5 + 1.0 / 16
    run("c1_nvfp4_absmax", "NVFP4 AbsMax, fp32 256x1024 N(0,1) with 1% x20 (cache-resident: "
        "latency-bound, no roofline claim)", x1, B.make_spec(), base_spec=B.make_spec(),
        bytes_per_elem=f1, x_h=x1_h)
    run("c1_nvfp4_sweep_mse", "NVFP4 ScaleSweep MSE [-3,7], fp32 256x1024 (cache-resident); "
        "baseline AbsMax", x1, B.make_spec(B.FP4Q_NVFP4, B.FP4Q_SCALE_SWEEP, window=(-3, 7)),
        base_spec=B.make_spec(), bytes_per_elem=f1, x_h=x1_h)
    del x1
    x3_h = synth.c3()
    x3 = to_dev(x3_h, dev)
    run("c3_mxfp4_rtn", "MXFP4 OCP scale + RTN, bf16 activations 8192x4096, 8 outlier channels x50",
        x3, B.make_spec(B.FP4Q_MXFP4), base_spec=B.make_spec(B.FP4Q_MXFP4), bytes_per_elem=mx,
        x_h=x3_h)
    run("c3_mxfp4_rtn_hadamard32", "MXFP4 with 32-point block Hadamard + RTN, same tensor; "
        "baseline without rotation", x3, B.make_spec(B.FP4Q_MXFP4, rotate=32),
        base_spec=B.make_spec(B.FP4Q_MXFP4), rotate=32, base_rotate=0, bytes_per_elem=mx,
        x_h=x3_h)
    x4_h = synth.c4()[0]
    x4 = to_dev(x4_h, dev)
    run("c4_if4", "IF4 (FP4 or INT4 per block, indicator in the scale's sign bit), bf16 "
        "8192x8192, half uniform / half spiky-Laplace blocks; baseline NVFP4 AbsMax",
        x4, B.make_spec(B.FP4Q_IF4), base_spec=B.make_spec(), bytes_per_elem=nv, x_h=x4_h)
    configs = dict(out)
    out.clear()
    run("nvfp4_four_over_six_wmse_c2",
        "NVFP4 Four Over Six (max onto 6 or 4), WMSE, bf16 weight 14336x4096; baseline AbsMax",
        x2, B.make_spec(B.FP4Q_NVFP4, B.FP4Q_SCALE_FOUR_OVER_SIX, B.FP4Q_OBJ_WMSE),
        importance=imp, base_spec=B.make_spec(), err_imp=imp, bytes_per_elem=nv, x_h=x2_h,
        imp_host=imp_h)

    for rot in (0, 32):
        run(f"mxfp4_exponent_window_rot{rot}_c3",
            f"MXFP4 E8M0 exponent window [0,1], MSE, rotation {rot}, bf16 activations "
            "8192x4096 with 8 outlier channels; baseline the OCP exponent",
            x3, B.make_spec(B.FP4Q_MXFP4, B.FP4Q_SCALE_SWEEP, window=(0, 1), rotate=rot),
            base_spec=B.make_spec(B.FP4Q_MXFP4, rotate=rot), rotate=rot, bytes_per_elem=mx,
            x_h=x3_h)
    c_h = np.random.default_rng(12).lognormal(0.0, 0.08, (8192, 4096 // 8)).astype(np.float32)
    c = torch.from_numpy(c_h).to(dev)
    r3 = torch.empty(8192 * 4096 // 2, dtype=torch.uint8, device=dev)
    s3 = torch.empty(8192 * 4096 // 32, dtype=torch.uint8, device=dev)
    spec_r = B.make_spec(B.FP4Q_MXFP4)
    x3c = [x3] + [x3.clone() for _ in range(7)]
    ms, _ = event_time(lambda i: B.fp4q_quantize_relaxed(spec_r, x3c[i % 8], c, 8, False, r3, s3,
                                                         None, ws), steps, 2, SETTLE_MS)
    del x3c
    gb = 8192 * 4096 * (mx + 4.0 / 8) / (ms * 1e-3) / 1e9
    out["mxfp4_focus_deploy_g8_c3"] = {
        "workload": "FOCUS deploy encode, MXFP4, one coefficient per 8 elements "
                    "(lognormal(0,0.08)), bf16 8192x4096", "quantize_ms": ms,
        "quantize_gbps": gb, "quantize_frac_of_peak": gb / PEAK_HBM_GBPS}
    if not args.no_cpu:
        B.fp4q_quantize_relaxed(spec_r, x3, c, 8, False, r3, s3, None, ws)
        out["mxfp4_focus_deploy_g8_c3"]["parity_sample"] = sample_parity(
            x3_h, spec_r, r3, s3, None, relaxed=(c_h, 8))
    log(f"mxfp4 focus g8: {ms:.3f} ms, {gb:.0f} GB/s, "
        f"parity {out['mxfp4_focus_deploy_g8_c3'].get('parity_sample')}")
    del x3, c, r3, s3

    run("if4_pattern_window_c4",
        "IF4 (FP4 or INT4 per block) over E4M3 patterns [-3,7], MSE, bf16 8192x8192 "
        "half uniform / half spiky-Laplace blocks; baseline plain IF4",
        x4, B.make_spec(B.FP4Q_IF4, B.FP4Q_SCALE_SWEEP, window=(-3, 7)),
        base_spec=B.make_spec(B.FP4Q_IF4), bytes_per_elem=nv, x_h=x4_h)
    del x4
    torch.cuda.empty_cache()
    return configs, out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X only: there is no multi-GPU path (the "
              "quantizer would shard by rows with one all-reduce(max) of the global "
              "scale).  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    # VALU issue costs first, in a child process, before this one opens the GPU
    issue = None if args.no_issue else valu_issue_costs()
    if issue is not None:
        log("VALU issue cycles per wave64 instruction:", issue["cycles_per_wave64_instr"])

    import torch
    from block_scaled_fp4_fp4q_amd import binding as B
    from block_scaled_fp4_fp4q_amd import synth

    dev = torch.device("cuda:0")
    B.lib()
    log("device", torch.cuda.get_device_name(0))

    # ---------------- headline: NVFP4 ScaleSweep WMSE on bf16 14336x4096 ----------------
    rows, cols = synth.SHAPES["c2"]
    t = time.time()
    x_h, imp_h = synth.c2()
    log(f"generated c2 {rows}x{cols} in {time.time() - t:.1f}s")
    n = rows * cols
    xs = [to_dev(x_h, dev)]
    for _ in range(args.copies - 1):
        xs.append(xs[0].clone())
    imp = to_dev(imp_h, dev)
    spec = B.make_spec(B.FP4Q_NVFP4, B.FP4Q_SCALE_SWEEP, B.FP4Q_OBJ_WMSE, (-8, 7))
    spec_given = B.make_spec(B.FP4Q_NVFP4, B.FP4Q_SCALE_SWEEP, B.FP4Q_OBJ_WMSE, (-8, 7),
                             global_scale_given=True)
    ws = B.alloc_workspace(spec, rows, cols, dev)
    outs = [(torch.empty(n // 2, dtype=torch.uint8, device=dev),
             torch.empty(n // 16, dtype=torch.uint8, device=dev),
             torch.empty(1, dtype=torch.float32, device=dev)) for _ in range(args.copies)]

    def step(i):
        c, s, g = outs[i % args.copies]
        B.fp4q_quantize(spec, xs[i % args.copies], imp, c, s, g, ws)

    ms, wall = event_time(step, args.steps, args.warmup)
    log(f"full call: {ms * 1e3:.1f} us/step (wall {wall:.3f}s for {args.steps})")

    def sweep_only(i):
        c, s, g = outs[i % args.copies]
        B.fp4q_quantize(spec_given, xs[i % args.copies], imp, c, s, g, ws)

    ms_k, _ = event_time(sweep_only, args.steps, args.warmup)
    bytes_per_elem_kernel = 2.0 + 0.5 + 1.0 / 16       # read bf16, write codes + scales
    bytes_per_elem_call = 2 * 2.0 + 0.5 + 1.0 / 16     # + the global-max read
    kernel_gbps = n * bytes_per_elem_kernel / (ms_k * 1e-3) / 1e9
    call_gbps = n * bytes_per_elem_call / (ms * 1e-3) / 1e9
    log(f"sweep kernel alone: {ms_k * 1e3:.1f} us, {kernel_gbps:.0f} GB/s")

    # reference: a plain device copy of 1 GiB (read + write, larger than the
    # Infinity Cache) -- the achievable-bandwidth yardstick, and the kernel
    # whose FETCH_SIZE / WRITE_SIZE calibrate the HBM traffic counters
    ref_src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    ref_dst = torch.empty_like(ref_src)
    cms, _ = event_time(lambda i: ref_dst.copy_(ref_src), 10, 2, SETTLE_MS)
    copy_gbps = 2 * ref_src.numel() / (cms * 1e-3) / 1e9
    del ref_src, ref_dst
    log(f"device copy 1 GiB: {copy_gbps:.0f} GB/s")

    # quality: ScaleSweep vs AbsMax MSE on the same tensor
    c, s, g = outs[0]
    B.fp4q_quantize(spec, xs[0], imp, c, s, g, ws)
    mse_sweep, wmse_sweep = B.fp4q_error(B.make_spec(), xs[0], imp, c, s, g, ws)
    ca, sa, ga = B.quantize(xs[0])
    mse_abs, wmse_abs = B.error(xs[0], ca, sa, ga, importance=imp)
    torch.cuda.synchronize()

    result = {
        "metric": METRIC,
        "value": n / (ms * 1e-3) / 1e9,
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "NVFP4 ScaleSweep WMSE [-8,7], bf16 weight 14336x4096 (t(4)*0.02), "
                        "lognormal(0,1) column importance, global scale computed on device",
            "rows": rows, "cols": cols, "block": 16, "input_dtype": "bf16",
            "input_copies_cycled": args.copies,
        },
        "achieved_gbps": call_gbps,
        "device_copy_gbps": copy_gbps,
        "frac_of_peak": call_gbps / PEAK_HBM_GBPS,
        "algorithmic_bytes_per_elem": bytes_per_elem_call,
        "nvfp4_sweep_mse": mse_sweep,
        "nvfp4_sweep_wmse": wmse_sweep,
        "nvfp4_absmax_mse": mse_abs,
        "nvfp4_absmax_wmse": wmse_abs,
        "roofline": roofline(n, ms_k, kernel_gbps, bytes_per_elem_kernel, issue),
    }

    # ---------------- CPU oracle on a row sample of the same workload ----------------
    if not args.no_cpu:
        from oracle import ref
        cores = len(os.sched_getaffinity(0))
        r = min(args.cpu_rows, rows)
        xs_h = np.ascontiguousarray(x_h[:r])
        t = time.perf_counter()
        ref.quantize(xs_h, rule=ref.SWEEP, objective=ref.WMSE, importance=imp_h, nthreads=cores)
        dt = time.perf_counter() - t
        result["cpu_baseline"] = {
            "value": r * cols / dt / 1e9, "unit": "Gelem/s", "cores": cores, "kind": "oracle",
            "sample": f"first {r} of {rows} rows ({r * cols} elements), same quantize "
                      f"(global max + ScaleSweep WMSE), {dt:.2f}s wall",
        }
        log(f"cpu oracle: {r * cols / dt / 1e6:.2f} Melem/s on {cores} threads")
        # the same rows re-quantized by the oracle under the GPU's global scale
        c, s_, g = outs[0]
        B.fp4q_quantize(spec, xs[0], imp, c, s_, g, ws)
        torch.cuda.synchronize()
        S = float(g.item())
        want = ref.quantize(xs_h, rule=ref.SWEEP, objective=ref.WMSE, importance=imp_h,
                            global_scale=S, nthreads=cores, errors=True)
        gs_rows = s_.cpu().numpy()[: r * cols // 16]
        gc_rows = c.cpu().numpy()[: r * cols // 2]
        live = want["best"] > 0
        gap = np.where(live, (want["second"] - want["best"]) / np.where(live, want["best"], 1), np.inf)
        result["parity_sample"] = {
            "blocks": int(gs_rows.size),
            "scale_mismatches": int(np.sum(gs_rows != want["scales"])),
            "code_bytes_mismatched": int(np.sum(gc_rows != want["codes"])),
            "oracle_near_tie_blocks": int(np.sum(gap < 1e-6)),
        }
        log(f"parity on the sample: {result['parity_sample']}")

    # ---------------- extensions: 4/6, MXFP4 exponent window, IF4 window, FOCUS ----------------
    if not args.no_secondary:
        result["configs"], result["extensions"] = extensions(args, B, synth, dev, xs[0], imp, ws,
                                                             x_h, imp_h)

    # ---------------- secondary: KV cache, sweep MSE + fused Hadamard ----------------
    if not args.no_secondary:
        del xs, outs
        torch.cuda.empty_cache()
        t = time.time()
        kv_h = synth.c5()
        log(f"generated c5 {kv_h.shape} in {time.time() - t:.1f}s")
        kv = to_dev(kv_h, dev)
        kv_head = np.ascontiguousarray(kv_h[: SAMPLE_ELEMS // kv_h.shape[1]])
        del kv_h
        kr, kc = kv.shape
        kn = kr * kc
        kspec = B.make_spec(B.FP4Q_NVFP4, B.FP4Q_SCALE_SWEEP, B.FP4Q_OBJ_MSE, (-3, 7), rotate=16)
        kspec_g = B.make_spec(B.FP4Q_NVFP4, B.FP4Q_SCALE_SWEEP, B.FP4Q_OBJ_MSE, (-3, 7), rotate=16,
                              global_scale_given=True)
        kc_, ks_, kg_ = (torch.empty(kn // 2, dtype=torch.uint8, device=dev),
                         torch.empty(kn // 16, dtype=torch.uint8, device=dev),
                         torch.empty(1, dtype=torch.float32, device=dev))
        ksteps = max(5, args.steps // 5)
        kms, _ = event_time(lambda i: B.fp4q_quantize(kspec, kv, None, kc_, ks_, kg_, ws), ksteps, 2,
                            SETTLE_MS)
        kms_k, _ = event_time(lambda i: B.fp4q_quantize(kspec_g, kv, None, kc_, ks_, kg_, ws), ksteps,
                              2, SETTLE_MS)
        y = torch.empty_like(kv)
        dms, _ = event_time(lambda i: B.fp4q_dequantize(kspec, kc_, ks_, kg_, kr, kc, 16, y), ksteps, 2,
                            SETTLE_MS)
        kmse, _ = B.fp4q_error(kspec, kv, None, kc_, ks_, kg_, ws)
        ka, kas, kag = B.quantize(kv, rotate=16)
        kmse_abs, _ = B.error(kv, ka, kas, kag, rotate=16)
        del ka, kas
        torch.cuda.synchronize()
        result["secondary"] = {
            "kv_cache_sweep_mse_hadamard16": {
                "workload": "NVFP4 ScaleSweep MSE [-3,7] + fused 16-point Hadamard, bf16 KV cache "
                            "[64,32,4096,128] (2 GiB), global scale computed on device",
                "quantize_ms": kms,
                "quantize_gelem_s": kn / (kms * 1e-3) / 1e9,
                "quantize_gbps": kn * 4.5625 / (kms * 1e-3) / 1e9,
                "quantize_frac_of_peak": kn * 4.5625 / (kms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                "sweep_kernel_ms": kms_k,
                "sweep_kernel_gbps": kn * 2.5625 / (kms_k * 1e-3) / 1e9,
                "dequantize_ms": dms,
                "dequantize_gbps": kn * 2.5625 / (dms * 1e-3) / 1e9,
                "nvfp4_sweep_mse": kmse,
                "nvfp4_absmax_mse": kmse_abs,
            },
        }
        if not args.no_cpu:
            # kc_, ks_, kg_ hold the last quantize of kv (S given: the S of the full call)
            result["secondary"]["kv_cache_sweep_mse_hadamard16"]["parity_sample"] = sample_parity(
                kv_head, kspec, kc_, ks_, kg_)
        log(f"c5 quantize {kms:.3f} ms, sweep kernel {kms_k:.3f} ms, dequant {dms:.3f} ms, parity "
            f"{result['secondary']['kv_cache_sweep_mse_hadamard16'].get('parity_sample')}")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
