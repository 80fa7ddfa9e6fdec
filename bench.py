"""Benchmark of the Muon bank step on one MI355X.

One step = one full pass of the hot path over every bank of the workload: momentum + Nesterov,
Frobenius pre-scale, five quintic Newton-Schulz rounds (Gram, polynomial, update contractions on bf16
MFMA), and the mixed-precision apply.  Inputs are seeded synthetic banks (no dataset), resident in
HBM before the timed region.  The default workload is the largest that one GPU holds whole: the 350M
model's banks (96, 1024, 1024) + (48, 4096, 1024) + (24, 2816, 768) with view slots 14-15 dead.

Prints one JSON line.  ``value`` is the step's throughput in algorithmic Newton-Schulz TFLOP/s: live
slots x 5*(m(m+1)n + m^2(m+1) + 2m^2 n) per step (symmetric Gram and A*A counted once) / wall time of
the whole step.  The timed region holds the K steps and nothing else; each kernel's average duration
comes from a separate pass in which every launch is bracketed by events.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

METRIC = "Muon bank-step ms and NS TFLOP/s (% bf16 MFMA peak), 1×MI355X"
PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 2.4 GHz x 4096 bf16 flop/clk/CU (dense)
PEAK_HBM_GBPS = 8000.0

HERE = os.path.dirname(os.path.abspath(__file__))


def ns_flops_per_slot(rows: int, cols: int, steps: int = 5) -> dict:
    m, n = min(rows, cols), max(rows, cols)
    return {"ns_gram": steps * m * (m + 1) * n, "ns_poly": steps * m * m * (m + 1), "ns_update": steps * 2 * m * m * n}


def ns_dense_flops_per_slot(rows: int, cols: int, steps: int = 5) -> int:
    """Dense-equivalent flops of the same rounds, symmetric products counted in full (reported beside the
    algorithmic count, never in place of it)."""
    m, n = min(rows, cols), max(rows, cols)
    return steps * (4 * m * m * n + 2 * m ** 3)


def bank_bytes(spec) -> dict:
    numel = spec.batch * spec.rows * spec.cols
    g = 4 if spec.grad_dtype == "f32" else 2
    return {"momentum": numel * (g + 2 * g + 2), "apply": numel * 10}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=4,
                   help="workload id 0..7 (4 = the 350M banks, the largest that fits one GPU; 1 = the attention "
                        "bank; 5, 6 = one GPU's share of workloads 3, 4 on 8 GPUs; 7 = workload 4 with the other "
                        "dead-slot reading)")
    p.add_argument("--kernel-steps", type=int, default=10,
                   help="steps of the separate pass whose kernel launches are each bracketed by events")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-parity", action="store_true")
    p.add_argument("--no-probes", action="store_true", help="skip the measured-peak probes")
    p.add_argument("--workload", default="bank", choices=("bank", "transpose", "vendor-gemm"),
                   help="bank: the Muon bank step (the headline); transpose: the tied-embedding transposes of "
                        "one optimizer step at the LM-head size; vendor-gemm: the vendor library's dense bf16 "
                        "batched products (torch.bmm) on the shapes of the Newton-Schulz contractions, for "
                        "comparison only")
    p.add_argument("--ns-path", type=int, default=0, choices=(0, 1),
                   help="0: persistent Newton-Schulz kernel where the shape allows it; 1: one launch per contraction")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run one device-to-device copy of MIB MiB (the known-size reference that the "
                        "FETCH_SIZE / WRITE_SIZE counters of the kernels are scaled by) and exit")
    return p.parse_args()


# Dense products with the shapes of the Newton-Schulz contractions (batch, m, k, n): X Xᵀ or Gᵀ G, A·A and the
# update of each bank, as plain batched products with every output computed, and one large square product.
VENDOR_GEMM_SHAPES = [
    ("attention bank 40 x 768^2: Gram, polynomial and update", 40, 768, 768, 768),
    ("MLP bank 24 x 3072x768: Gram (k = 3072)", 24, 768, 3072, 768),
    ("MLP bank 24 x 3072x768: update (3072 x 768 by 768 x 768)", 24, 3072, 768, 768),
    ("350M attention 96 x 1024^2: Gram, polynomial and update", 96, 1024, 1024, 1024),
    ("350M MLP 48 x 4096x1024: Gram (k = 4096)", 48, 1024, 4096, 1024),
    ("350M MLP 48 x 4096x1024: update (4096 x 1024 by 1024 x 1024)", 48, 4096, 1024, 1024),
    ("single 8192^3", 1, 8192, 8192, 8192),
]


def bench_vendor_gemm(args, torch):
    """torch.bmm (the vendor BLAS) in bf16 on contiguous operands, each shape timed over back-to-back calls
    between two events after warm-up; dense flops 2*b*m*k*n.  A comparison for the Newton-Schulz launch, not
    part of the step."""
    out = []
    gen = torch.Generator(device="cuda").manual_seed(0)
    for name, b, m, k, n in VENDOR_GEMM_SHAPES:
        x = torch.randn((b, m, k), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        y = torch.randn((b, k, n), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        x, y = x.contiguous(), y.contiguous()
        for _ in range(max(args.warmup, 3)):
            torch.bmm(x, y)
        reps = max(args.steps, 10)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(reps):
            torch.bmm(x, y)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / reps
        tf = 2.0 * b * m * k * n / (ms * 1e-3) / 1e12
        out.append({"shape": name, "batch": b, "m": m, "k": k, "n": n, "ms": round(ms, 4),
                    "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
        print(f"vendor gemm {name}: {ms:.4f} ms, {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
        del x, y
    print(json.dumps({"metric": "vendor bf16 batched GEMM (torch.bmm) on the Newton-Schulz contraction shapes",
                      "unit": "TFLOP/s", "peak": PEAK_BF16_TFLOPS, "reps": max(args.steps, 10),
                      "results": out}), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the bank step is measured on a single MI355X; "
                          "--gpus must be 1"}), flush=True)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (HIP device)")
    if args.workload == "vendor-gemm":
        bench_vendor_gemm(args, torch)
        return
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}), flush=True)
        return
    sys.path.insert(0, HERE)
    from newton_schulz_bank_amd import api
    from newton_schulz_bank_amd.workloads import WORKLOAD_NAMES, WORKLOADS, make_bank

    api.lib()    # fails loudly if libmuonbank.so is missing
    if args.workload == "transpose":
        bench_transpose(args, torch, api)
        return
    api.mb_ns_set_path(args.ns_path)
    specs = WORKLOADS[args.config]
    hosts = [make_bank(args.config, i) for i in range(len(specs))]

    def upload():
        banks = []
        for spec, h in zip(specs, hosts):
            bf = spec.grad_dtype == "bf16"

            def dev(a, as_bf16=False):
                t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()
                return t.view(torch.bfloat16) if as_bf16 and a.dtype == np.uint16 else t
            banks.append(api.Bank(grad=dev(h["grad"], bf), momentum=dev(h["momentum"], bf), w_hi=dev(h["w_hi"]),
                                  w_lo=dev(h["w_lo"])))
        return banks

    banks = upload()
    ws = torch.empty(api.mb_step_workspace_bytes(banks), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    # ---- one whole step of every bank on fresh copies of the inputs, in the launch configuration timed
    # below; the first and last live slot of each bank are compared with the oracle in the CPU-baseline
    # leg (the full parity checks live in the test suite)
    sample = None
    if not args.no_parity and not args.no_cpu_baseline:
        sample = gpu_sample_step(api, specs, upload)

    # ---- timed region: K whole steps back to back between two events on the launch stream, nothing
    # else inside it
    for _ in range(args.warmup):
        api.muon_bank_step(banks, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        api.muon_bank_step(banks, workspace=ws, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(stop) / args.steps

    # ---- per-kernel durations: a separate pass in which every launch is bracketed by the library's
    # pooled events (created before the pass); one unbracketed step first, so that no bracketed launch
    # follows a host synchronization
    api.mb_timing_enable(True)
    api.mb_timing_read()
    api.mb_timing_enable(False)
    api.muon_bank_step(banks, workspace=ws, stream=stream)
    api.mb_timing_enable(True)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for _ in range(args.kernel_steps):
        api.muon_bank_step(banks, workspace=ws, stream=stream)
    k1.record(stream)
    api.mb_timing_enable(False)
    torch.cuda.synchronize()
    per_kernel = api.mb_timing_read()
    sampled = args.kernel_steps
    kernel_pass_ms = k0.elapsed_time(k1) / args.kernel_steps

    # ---- spread of single steps: a separate pass, each step between two events of its own (outside
    # the timed region above, which ms_per_step comes from)
    n_dist = 20
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_dist + 1)]
    evs[0].record(stream)
    for k in range(n_dist):
        api.muon_bank_step(banks, workspace=ws, stream=stream)
        evs[k + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([evs[k].elapsed_time(evs[k + 1]) for k in range(n_dist)])

    # ---- the apply alone on the largest bank, cold: a 1 GiB buffer is written (then, separately, read)
    # first, so that neither the L2s nor the 256 MB MALL hold the weights (the in-step apply may find them
    # there).  After the write the MALL is full of dirty lines of that buffer, which the apply's own
    # traffic evicts to HBM; after the read it is clean.
    cold = None
    big = max(range(len(specs)), key=lambda i: specs[i].numel)
    if banks[big].w_hi.numel() > 0:
        scrub = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        gen = torch.Generator(device="cuda")
        gen.manual_seed(7)
        v = (torch.randn(banks[big].w_hi.shape, generator=gen, device="cuda") * 1e-2).to(torch.bfloat16)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0 = bank_bytes(specs[big])["apply"]
        cold = {"bank": specs[big].name, "bytes": b0, "note": "median of 3 launches, each after a 1 GiB buffer "
                "write (after_write) or read (after_read)"}
        for key, prep in (("after_write", lambda k: scrub.fill_(k + 1)),
                          ("after_read", lambda k: scrub.view(torch.int64).sum())):
            cold_ms = []
            for k in range(3):
                prep(k)
                e0.record(stream)
                api.mp_apply_update(banks[big].w_hi, banks[big].w_lo, v, 1e-3, 1.0 - 1e-4, stream=stream)
                e1.record(stream)
                torch.cuda.synchronize()
                cold_ms.append(e0.elapsed_time(e1))
            med = float(np.median(cold_ms))
            cold[key] = {"us": round(med * 1e3, 2), "gbps": round(b0 / (med * 1e-3) / 1e9, 1)}
        del scrub, v

    peaks = None if args.no_probes else measure_peaks(torch, stream)

    live_slots = sum(len(s.live_slots) for s in specs)
    # algorithmic flops by the kernel that does them: banks whose sides are multiples of 128 run
    # all their rounds in the persistent kernel (unless --ns-path 1), the rest (gates, ragged shapes)
    # in the small-slot kernel or one launch per contraction
    alg = {"ns_persist": 0, "ns_gram": 0, "ns_poly": 0, "ns_update": 0}
    for s in specs:
        f = ns_flops_per_slot(s.rows, s.cols)
        persistent = args.ns_path == 0 and s.rows % 128 == 0 and s.cols % 128 == 0
        for k in ("ns_gram", "ns_poly", "ns_update"):
            alg["ns_persist" if persistent else k] += f[k] * len(s.live_slots)
    alg = {k: v for k, v in alg.items() if v > 0}
    ns_flops = sum(alg.values())
    ns_dense = sum(ns_dense_flops_per_slot(s.rows, s.cols) * len(s.live_slots) for s in specs)
    bytes_ = {"momentum": sum(bank_bytes(s)["momentum"] for s in specs),
              "apply": sum(bank_bytes(s)["apply"] for s in specs)}

    kernels = {}
    for name, (n, tot) in per_kernel.items():
        per_launch = tot / n
        kernels[name] = {"launches_per_step": n / sampled, "avg_us": per_launch * 1e3, "ms_per_step": tot / sampled}
    ns_ms = sum(kernels.get(k, {"ms_per_step": 0})["ms_per_step"] for k in alg)
    for k in alg:
        if k in kernels:
            flops_per_launch = alg[k] / kernels[k]["launches_per_step"]
            kernels[k]["alg_tflops"] = flops_per_launch / (kernels[k]["avg_us"] * 1e-6) / 1e12
    for k in ("momentum", "apply"):
        if k in kernels:
            kernels[k]["gbps"] = bytes_[k] / (kernels[k]["ms_per_step"] * 1e-3) / 1e9
            if peaks:
                kernels[k]["frac_of_measured_copy"] = kernels[k]["gbps"] / peaks["copy_gbps"]

    dominant = max(alg, key=lambda k: kernels.get(k, {"ms_per_step": 0})["ms_per_step"])
    achieved = kernels[dominant]["alg_tflops"]
    roofline = {"bound": "mfma", "kernel": dominant, "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": read_traffic(dominant, args.config)}
    if peaks:
        roofline["measured_peak"] = peaks["mfma_bf16_tflops"]
        roofline["frac_of_measured"] = round(achieved / peaks["mfma_bf16_tflops"], 4)

    value = ns_flops / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.config], "config_id": args.config,
                   "banks": [[s.batch, s.rows, s.cols] for s in specs], "live_slots": live_slots,
                   "ns_steps": 5, "grad_dtype": specs[0].grad_dtype, "ns_path": args.ns_path},
        "matrices_per_s": round(live_slots / (ms_per_step * 1e-3), 1),
        "ns_ms_per_step": round(ns_ms, 4),
        "ns_tflops": round(ns_flops / (ns_ms * 1e-3) / 1e12, 2) if ns_ms > 0 else None,
        "ns_frac_of_peak": round(ns_flops / (ns_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4) if ns_ms > 0 else None,
        "ns_dense_equiv_tflops": round(ns_dense / (ns_ms * 1e-3) / 1e12, 2) if ns_ms > 0 else None,
        "step_ms_distribution": {"steps": n_dist, "p10": round(float(np.percentile(step_ms, 10)), 4),
                                 "median": round(float(np.median(step_ms)), 4),
                                 "p90": round(float(np.percentile(step_ms, 90)), 4)},
        "apply_gbps": round(kernels.get("apply", {}).get("gbps", 0.0), 1),
        "apply_cold": cold,
        "apply_frac_of_hbm": round(kernels.get("apply", {}).get("gbps", 0.0) / PEAK_HBM_GBPS, 4),
        "momentum_gbps": round(kernels.get("momentum", {}).get("gbps", 0.0), 1),
        "momentum_frac_of_hbm": round(kernels.get("momentum", {}).get("gbps", 0.0) / PEAK_HBM_GBPS, 4),
        "measured_peaks": peaks,
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "wall_s_timed": round(wall, 4),
        "kernel_timing": {"steps_bracketed": sampled, "ms_per_step_bracketed": round(kernel_pass_ms, 4),
                          "note": "every launch of a separate pass after the timed region bracketed by events"},
        "roofline": roofline,
        "device_fault": api.mb_device_fault(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"], out["parity"] = cpu_baseline(specs, hosts, sample)
        # the same whole step's Newton-Schulz work at the oracle's rate
        out["cpu_baseline"]["s_per_step_equiv"] = round(ns_flops / (out["cpu_baseline"]["value"] * 1e12), 2)
    print(json.dumps(out), flush=True)


def measure_peaks(torch, stream):
    """The measured-peak probes: a register-only bf16 MFMA loop over the whole chip and a 1 GiB device copy
    in 16-byte vectors (median of 5 launches each, events on the launch stream)."""
    from newton_schulz_bank_amd import probes
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn, reps=5):
        fn()
        out = []
        for _ in range(reps):
            ev[0].record(stream)
            fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            out.append(ev[0].elapsed_time(ev[1]))
        return float(np.median(out))
    wgs, iters = 256 * 8, 4096
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    ms = timed(lambda: probes.mb_probe_mfma_bf16(iters, wgs, sink, stream=stream))
    mfma = probes.mfma_flops(iters, wgs) / (ms * 1e-3) / 1e12
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms_c = timed(lambda: probes.mb_probe_copy(dst, src, stream=stream))
    del src, dst, sink
    return {"mfma_bf16_tflops": round(mfma, 1), "mfma_frac_of_nominal": round(mfma / PEAK_BF16_TFLOPS, 4),
            "copy_gbps": round(2 * n / (ms_c * 1e-3) / 1e9, 1), "copy_frac_of_nominal":
            round(2 * n / (ms_c * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "note": "mb_probe_mfma_bf16: 2048 workgroups x 4 wavefronts x 4 independent v_mfma_f32_32x32x16_bf16 "
                    "chains x 4096 iterations, no memory traffic; mb_probe_copy: 1 GiB device copy, 16-byte vectors "
                    "(2 GiB of traffic)"}


def gpu_sample_step(api, specs, upload):
    """One whole step of every bank on fresh copies of its inputs (the same banks, workspace size and
    launches as the timed steps, plus the v_out copy of the Newton-Schulz output); returns, for the first
    and the last live slot of each bank, the raw output bits."""
    import torch
    banks = upload()
    for b in banks:
        b.v_out = torch.empty(b.w_hi.shape, dtype=torch.int16, device="cuda")
    ws = torch.empty(api.mb_step_workspace_bytes(banks), dtype=torch.uint8, device="cuda")
    api.muon_bank_step(banks, workspace=ws)
    torch.cuda.synchronize()
    out = []
    for spec, b in zip(specs, banks):
        bf = spec.grad_dtype == "bf16"
        for slot in dict.fromkeys(spec.live_slots[:1] + spec.live_slots[-1:]):
            mom = b.momentum[slot:slot + 1]
            mom = mom.view(torch.int16).cpu().numpy().view(np.uint16) if bf else mom.cpu().numpy()
            out.append({"bank": spec.name, "slot": slot,
                        "v": b.v_out[slot:slot + 1].cpu().numpy().view(np.uint16),
                        "w_hi": b.w_hi[slot:slot + 1].cpu().numpy().view(np.uint16),
                        "w_lo": b.w_lo[slot:slot + 1].cpu().numpy().view(np.uint16), "momentum": mom})
    del banks, ws
    return out


def _sample_parity(oracle, spec, h, sample):
    """One slot the GPU stepped against the oracle's step of that slot on the same inputs (every slot of a
    bank takes the bank's scalars; the oracle's step is per slot)."""
    slot = sample["slot"]
    bf = spec.grad_dtype == "bf16"
    sl = lambda a: np.ascontiguousarray(a[slot:slot + 1])
    vals = (lambda a: a.astype(np.float64)) if not bf else oracle.bf16_bits_to_f64
    ref = oracle.muon_bank_step(vals(sl(h["grad"])), vals(sl(h["momentum"])), sl(h["w_hi"]), sl(h["w_lo"]),
                                oracle.F32 if not bf else oracle.BF16)
    v = oracle.bf16_bits_to_f64(sample["v"])
    err = float(np.linalg.norm(v - ref["v64"]) / max(np.linalg.norm(ref["v64"]), 1e-30))
    want = oracle.mp_apply_update(sl(h["w_hi"]), sl(h["w_lo"]), v, ref["scalars"].eta, ref["scalars"].decay)
    ok_apply = bool(np.array_equal(sample["w_hi"], want[0]) and np.array_equal(sample["w_lo"], want[1]))
    mom = vals(sample["momentum"]) if bf else sample["momentum"].astype(np.float64)
    ok_mom = bool(np.array_equal(mom, ref["momentum"]))
    if not (ok_apply and ok_mom and err <= 3e-2):
        raise SystemExit(f"parity failure on {spec.name} slot {slot}: ns rel err {err}, apply {ok_apply}, "
                         f"momentum {ok_mom}")
    # for information: against the oracle's iteration on u before its rounding to bf16 (the Nesterov sum
    # of the stored buffer taken in binary64), which adds the input's rounding to the error
    sc = ref["scalars"]
    u_unrounded = sc.nu * vals(sl(h["grad"])) + sc.mu * ref["momentum"]
    v_unrounded = oracle.newton_schulz(u_unrounded)
    err_u = float(np.linalg.norm(v - v_unrounded) / max(np.linalg.norm(v_unrounded), 1e-30))
    return {"bank": spec.name, "slot": slot, "ns_rel_fro_err": round(err, 5),
            "ns_rel_fro_err_vs_unrounded_u": round(err_u, 5), "apply_bit_exact": ok_apply,
            "momentum_bit_exact": ok_mom}


def _parity(oracle, specs, hosts, samples):
    """Every sampled slot against the oracle: the worst Newton-Schulz error and the per-slot results."""
    by_name = {s.name: (s, h) for s, h in zip(specs, hosts)}
    checked = [_sample_parity(oracle, *by_name[smp["bank"]], smp) for smp in samples]
    worst = max(checked, key=lambda c: c["ns_rel_fro_err"])
    return {"ns_rel_fro_err_max": worst["ns_rel_fro_err"], "worst": {"bank": worst["bank"], "slot": worst["slot"]},
            "ns_rel_fro_err_vs_unrounded_u_max": max(c["ns_rel_fro_err_vs_unrounded_u"] for c in checked),
            "apply_bit_exact": all(c["apply_bit_exact"] for c in checked),
            "momentum_bit_exact": all(c["momentum_bit_exact"] for c in checked),
            "tolerance": 3e-2, "slots": checked}


def cpu_baseline(specs, hosts, sample=None):
    """The oracle as it stands, on a bounded sample of the same workload, on the host's cores.  With a
    GPU sample (gpu_sample_step), the oracle's step of each sampled slot is also compared with it; returns
    (baseline, parity or None)."""
    sys.path.insert(0, HERE)
    import oracle
    parity = _parity(oracle, specs, hosts, sample) if sample is not None else None
    try:
        from threadpoolctl import threadpool_info
        info = [t for t in threadpool_info() if t.get("user_api") == "blas"]
        threads = max([t.get("num_threads", 1) for t in info] or [1])
        blas = ", ".join(sorted({f"{t.get('internal_api')} {t.get('version')}" for t in info})) or None
    except Exception:
        threads = os.cpu_count() or 1
        blas = None
    budget_s = 12.0
    flops, elapsed, counts = 0, 0.0, {}
    passes = 0
    while elapsed < budget_s and passes < 16:
        passes += 1
        f_, e_, c_ = _oracle_pass(oracle, specs, hosts, budget_s - elapsed)
        flops += f_
        elapsed += e_
        for k, v in c_.items():
            counts[k] = counts.get(k, 0) + v
    desc = [f"{counts[spec.name]} slot-steps over the {len(spec.live_slots)} live slots of {spec.name} "
            f"({spec.rows}x{spec.cols})" for spec in specs if spec.name in counts]
    out = {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
           "sample": f"full oracle step (momentum, fp64 NS5, exact apply), one slot at a time: {'; '.join(desc)}",
           "seconds": round(elapsed, 2), "host": platform.processor() or platform.machine(), "blas": blas}
    # one slot of the first bank with BLAS held to one thread
    try:
        from threadpoolctl import threadpool_limits
        spec, h = specs[0], hosts[0]
        s = spec.live_slots[0]
        with threadpool_limits(limits=1, user_api="blas"):
            t0 = time.perf_counter()
            _oracle_slot(oracle, spec, h, s)
            out["single_thread_s_per_slot"] = round(time.perf_counter() - t0, 3)
    except ImportError:
        pass
    return out, parity


def _oracle_slot(oracle, spec, h, s):
    sl = np.ascontiguousarray
    bf = spec.grad_dtype == "bf16"
    vals = (lambda a: a.astype(np.float64)) if not bf else oracle.bf16_bits_to_f64
    oracle.muon_bank_step(vals(sl(h["grad"][s:s + 1])), vals(sl(h["momentum"][s:s + 1])),
                          sl(h["w_hi"][s:s + 1]), sl(h["w_lo"][s:s + 1]), oracle.F32 if not bf else oracle.BF16)


def _oracle_pass(oracle, specs, hosts, budget_s):
    """One pass over the live slots of every bank, taking the banks in turn (one slot of each, then the
    next slot of each, ...), until the budget runs out: (flops, seconds, slots per bank)."""
    flops, elapsed, counts = 0, 0.0, {spec.name: 0 for spec in specs}
    order = []
    lives = [list(spec.live_slots) for spec in specs]
    for k in range(max(len(l) for l in lives)):
        order += [(i, l[k]) for i, l in enumerate(lives) if k < len(l)]
    for i, s in order:
        if elapsed >= budget_s:
            break
        spec, h = specs[i], hosts[i]
        t0 = time.perf_counter()
        _oracle_slot(oracle, spec, h, s)
        elapsed += time.perf_counter() - t0
        flops += sum(ns_flops_per_slot(spec.rows, spec.cols).values())
        counts[spec.name] += 1
    return flops, elapsed, {k: v for k, v in counts.items() if v}


def bench_transpose(args, torch, api):
    """The tied-embedding transposes of one optimizer step: the LM head's gradient (768, 50304) added
    transposed into the embedding's (50304, 768), and the embedding's weights copied transposed into
    the LM head, bf16, seeded synthetic data."""
    from newton_schulz_bank_amd.workloads import random_bf16_matrices
    rows, cols = 768, 50304
    lm_grad = random_bf16_matrices(7001, 1, rows, cols, 1e-3)[0]
    embed_grad = random_bf16_matrices(7002, 1, cols, rows, 1e-3)[0]
    embed_w = random_bf16_matrices(7003, 1, cols, rows, 0.02)[0]

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    d_lm_grad, d_embed_grad, d_embed_w = dev(lm_grad), dev(embed_grad), dev(embed_w)
    d_lm_w = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    # one call of each on the inputs, kept for the CPU-baseline leg's comparison with the oracle
    api.transpose_add(d_embed_grad, d_lm_grad)
    api.transpose_copy(d_lm_w, d_embed_w)
    torch.cuda.synchronize()
    got_add = d_embed_grad.view(torch.int16).cpu().numpy().view(np.uint16)
    got_copy = d_lm_w.view(torch.int16).cpu().numpy().view(np.uint16)
    d_embed_grad = dev(embed_grad)
    for _ in range(args.warmup):
        api.transpose_add(d_embed_grad, d_lm_grad)
        api.transpose_copy(d_lm_w, d_embed_w)
    torch.cuda.synchronize()

    def timed(fns):
        """K back-to-back calls of fns between two HIP events on the launch stream: ms per call of fns."""
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(args.steps):
            for fn in fns:
                fn()
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / args.steps

    def add():
        api.transpose_add(d_embed_grad, d_lm_grad)

    def copy():
        api.transpose_copy(d_lm_w, d_embed_w)
    # the step (both transposes), then each kernel alone: a per-launch event pair would add
    # microseconds to kernels this short
    ms_per_step = timed([add, copy])
    n = rows * cols * 2
    alg = {"transpose_add": 3 * n, "transpose_copy": 2 * n}       # bytes per launch
    kernels = {}
    for name, fn in (("transpose_add", add), ("transpose_copy", copy)):
        us = timed([fn]) * 1e3
        kernels[name] = {"avg_us": round(us, 3), "gbps": round(alg[name] / (us * 1e-6) / 1e9, 1)}
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"])
    achieved = kernels[dom]["gbps"]
    cpu, parity = (None, None) if args.no_cpu_baseline else _transpose_cpu_baseline(
        lm_grad, embed_grad, embed_w, got_add, got_copy)
    out = {
        "metric": "tied-embedding transposes (transpose_add + transpose_copy) HBM GB/s, 1xMI355X",
        "value": round(5 * n / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "LM head (768, 50304) <-> embedding (50304, 768), bf16", "rows": rows, "cols": cols},
        "kernels": kernels,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": read_traffic(dom, "transpose")},
    }
    if cpu is not None:
        out["cpu_baseline"], out["parity"] = cpu, parity
    print(json.dumps(out), flush=True)


def _transpose_cpu_baseline(lm_grad, embed_grad, embed_w, got_add, got_copy):
    """The oracle's transposes on a bounded slab of the same matrices, timed on one host core; the
    GPU's results are compared with the oracle's on 64 sampled embedding rows (add) and in full (copy)."""
    sys.path.insert(0, HERE)
    import oracle
    rows, cols = lm_grad.shape
    pick = np.sort(np.random.default_rng(7000).choice(cols, 64, replace=False))
    want_add = oracle.transpose_add(embed_grad[pick], np.ascontiguousarray(lm_grad[:, pick]), oracle.BF16)
    parity = {"transpose_add_bit_exact_sampled": bool(np.array_equal(got_add[pick], want_add)),
              "transpose_copy_bit_exact": bool(np.array_equal(got_copy, oracle.transpose_copy(embed_w)))}
    if not all(parity.values()):
        raise SystemExit(f"transpose parity failure: {parity}")
    t0, moved, slabs = time.perf_counter(), 0, 0
    while time.perf_counter() - t0 < 10.0 and slabs < 400:
        c0 = (slabs * 2048) % cols
        sl = slice(c0, min(c0 + 2048, cols))
        oracle.transpose_add(embed_grad[sl], np.ascontiguousarray(lm_grad[:, sl]), oracle.BF16)
        oracle.transpose_copy(np.ascontiguousarray(embed_w[sl]))
        moved += 5 * rows * (sl.stop - sl.start) * 2
        slabs += 1
    cpu_s = time.perf_counter() - t0
    return ({"value": round(moved / cpu_s / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
             "sample": f"{slabs} slabs of 2048 embedding rows (add + copy)", "seconds": round(cpu_s, 2)}, parity)


def read_traffic(kernel: str, config):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(HERE, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        entry = data.get(f"{kernel}:config{config}" if isinstance(config, int) else f"{kernel}:{config}")
        if not entry:
            return None
        import hashlib
        names = entry["sources"] if "sources" in entry else [entry["source"]]
        h = hashlib.sha256()
        for name in names:
            h.update(open(os.path.join(HERE, "newton_schulz_bank_amd", "csrc", name), "rb").read())
        if h.hexdigest() != entry["source_sha256"]:
            return None
        return entry["bytes_per_launch"]
    except Exception:
        return None


if __name__ == "__main__":
    main()
