"""Benchmark of the Muon-family optimizer step on one MI355X.

Default workload (the largest configuration): LionMuon on 8 x 4096x4096 +
8 x 4096x11008 bf16 matrices (494,927,872 parameters), M = 16 simulated
workers with Student-t(3) gradients, dual EMA (beta1 0.9, beta2 0.99), a
Muon step (5 cubic Newton-Schulz iterations on G_hat) every P = 4 steps and
Lion sign steps otherwise, 1-bit packed majority vote.  A step is one
sm_step call over all 16 matrices; the timed region starts on a P-cycle
boundary and holds whole cycles by default, so `value` is the P-averaged
steps/s.  Inputs are synthetic and resident in HBM before timing starts.

Prints one JSON line: steps/s (value), per-step-type times and rooflines
(Muon step: NS GEMMs against the bf16 MFMA peak; Lion step: the fused Lion
kernel against HBM), the roofline of the dominant kernel measured with HIP
events on the step's stream over the timed region, the CPU oracle timed on a
bounded sample on this host, and sub-objects for the other configurations:
`gpt2_small` (Sign-Muon, M = 5; with the int8 encoding and the polar step on
the vote as variants), `gpt2_large_cache_muon` (CacheMuon at gamma 2, 15, a
mixed-rate gamma and always-fresh, with refresh rates and executed
orthogonalisation FLOPs), `resnet50` (53 float32 convolution matrices, M =
4, one NS iteration) and `single_256` (one float32 256 x 256 matrix, M = 3).
Each Sign-Muon sub-object also times the same step replayed from one HIP
graph (`graph`: sm_step_graph, then sm_graph_launch per step).

  python bench.py [--steps K] [--warmup W] [--config {1..5}] [--no-cpu] [--no-sub]
  python bench.py --copy-calibration   # plain device copy of known size, for
                                       # scaling rocprofv3 FETCH_SIZE / WRITE_SIZE
  python bench.py --attainable         # MFMA ceiling probe and device copy only
  python bench.py --fidelity [--gamma G] # CacheMuon fidelity diagnostic (config 4)

roofline.traffic is the dominant kernel's HBM bytes per launch from the
rocprofv3 counter summary under profiles/ (FETCH_SIZE and WRITE_SIZE, each
scaled by what the counter reads for the plain copy); it is reported only
while the kernel source still hashes to the value recorded with the
counters, and is null otherwise.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
METRIC = "optimizer steps/s per layer set; NS TFLOP/s (MFMA %); vote+update GB/s (HBM %)"
DEFAULT_CONFIG = 5


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 20 for LionMuon = 5 P-cycles, 30 otherwise)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: one P-cycle for LionMuon, else 3)")
    ap.add_argument("--config", type=int, default=DEFAULT_CONFIG)
    ap.add_argument("--gamma", type=float, default=None, help="CacheMuon threshold override")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="budget of the CPU oracle sample")
    ap.add_argument("--no-sub", action="store_true",
                    help="skip the sub-objects of the other configurations")
    ap.add_argument("--sub-steps", type=int, default=20,
                    help="timed steps of each sub-object run")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (counter scaling)")
    ap.add_argument("--no-attainable", action="store_true",
                    help="skip the MFMA ceiling probe and device copy of the benchmark line "
                         "(kernel-statistics runs)")
    ap.add_argument("--attainable", action="store_true",
                    help="run only the MFMA ceiling probe and the device copy (the `attainable` "
                         "object of the benchmark line)")
    ap.add_argument("--fidelity", action="store_true",
                    help="CacheMuon fidelity diagnostic instead of the benchmark line: per step, "
                         "the residual and the spectral distance of the cached direction from a "
                         "fresh solve, and the refresh rate (default config 4)")
    ap.add_argument("--fidelity-steps", type=int, default=12)
    ap.add_argument("--fidelity-iters", type=int, default=30,
                    help="power-method iterations of the spectral distance")
    ap.add_argument("--fidelity-matrices", type=int, default=0,
                    help="diagnose only the first N matrices (0 = all)")
    ap.add_argument("--variant-steps", type=int, default=10,
                    help="timed steps of each step variant (int8 encoding, polar step on the "
                         "vote) of the Sign-Muon runs; 0 skips them")
    return ap.parse_args()


KINDS = ["ema", "norm", "gemm_gram", "gemm_apply", "gemm_rr", "probe", "sign_pack",
         "vote_update", "lion", "polar_update", "misc"]


def read_kinds(sm, steps):
    """Per-kind kernel time, algorithmic work and algorithmic HBM bytes from the
    library's HIP events."""
    kinds = {}
    for kind in KINDS:
        ms, n, work = sm.profile_read(kind)
        if n:
            kinds[kind] = {"ms_per_step": ms / steps, "launches_per_step": n / steps,
                           "avg_launch_ms": ms / n, "work_per_launch": work / n,
                           "flops" if kind.startswith(("gemm", "probe")) else "bytes":
                               work / steps}
            if kind.startswith(("gemm", "probe")):
                hb = sm.profile_read_bytes(kind)
                kinds[kind]["hbm_bytes"] = hb / steps
                kinds[kind]["bytes_per_launch"] = hb / n
    return kinds


def kind_roofline(kinds, kind, mdt):
    """Roofline of one kernel kind.  The NS / Gram GEMMs are dense
    contractions and sit under the MFMA roof of their operand type:
    `achieved` = algorithmic flops per launch / average launch time.  Their
    arithmetic intensity (algorithmic flops / algorithmic HBM bytes) and the
    HBM view (algorithmic bytes per launch / launch time against 8 TB/s) are
    reported beside it.  Streaming kinds sit under the HBM roof."""
    dk = kinds[kind]
    out = {"kernel": kind, "avg_launch_ms": dk["avg_launch_ms"],
           "work_per_launch": dk["work_per_launch"]}
    secs = dk["avg_launch_ms"] * 1e-3
    if kind.startswith(("gemm", "probe")):
        peak_f = PEAK_TFLOPS[mdt]
        ai = dk["flops"] / dk["hbm_bytes"] if dk.get("hbm_bytes") else float("inf")
        ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
        achieved = dk["work_per_launch"] / secs / 1e12
        out.update(bound="mfma", achieved=achieved, peak=peak_f, unit="TFLOP/s",
                   arith_intensity=ai, ridge=ridge, bytes_per_launch=dk.get("bytes_per_launch"))
        if dk.get("bytes_per_launch"):
            gbs = dk["bytes_per_launch"] / secs / 1e9
            out["hbm_view"] = {"achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": gbs / PEAK_HBM_GBS}
    else:
        achieved = dk["work_per_launch"] / secs / 1e9
        out.update(bound="hbm", achieved=achieved, peak=PEAK_HBM_GBS, unit="GB/s")
    out["frac"] = out["achieved"] / out["peak"]
    return out


def timed_steps(sm, torch, call, t, warmup, steps):
    """warmup untimed steps, `steps` timed ones, then as many again with the
    kernel-time accounting on (its event pairs around every launch would
    slow a launch-bound step, so they stay out of the timed region)."""
    for _ in range(warmup):
        call(t)
        t += 1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call(t)
        t += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sm.profile_enable(True)
    sm.profile_reset()
    for _ in range(steps):
        call(t)
        t += 1
    torch.cuda.synchronize()
    sm.profile_enable(False)
    return t, wall, read_kinds(sm, steps)


def stream_roofline(kinds, names):
    """HBM roofline of the slowest of the named streaming kernels."""
    have = [k for k in names if k in kinds]
    if not have:
        return None
    dom = max(have, key=lambda k: kinds[k]["ms_per_step"])
    dk = kinds[dom]
    achieved = dk["work_per_launch"] / (dk["avg_launch_ms"] * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": None,
            "avg_launch_ms": dk["avg_launch_ms"], "work_per_launch": dk["work_per_launch"]}


def gemm_totals(kinds):
    ms = sum(kinds.get(k, {}).get("ms_per_step", 0.0) for k in ("gemm_gram", "gemm_apply",
                                                               "gemm_rr"))
    fl = sum(kinds.get(k, {}).get("flops", 0.0) for k in ("gemm_gram", "gemm_apply", "gemm_rr"))
    return ms, fl


def measure_variants(sm, torch, wl, cfg, mats, t, args, base_ms, base_kinds):
    """The step variants the pages describe besides the default 1-bit vote:
    the int8 sign encoding and the optional polar step on the vote.  Each runs
    on the same state, warmed up and timed like the main step."""
    import dataclasses
    out = {}
    if wl.update != sm.UPDATE_VOTE or args.variant_steps <= 0:
        return out, t
    n = args.variant_steps
    # int8 encoding: sign kernel (int8 out) and the integer-sum vote
    c8 = dataclasses.replace(cfg, encoding=sm.ENC_INT8)
    t, wall, kinds = timed_steps(sm, torch, sm.StepCall(c8, mats), t, 2, n)
    out["int8_encoding"] = {
        "value": n / wall, "unit": "steps/s", "ms_per_step": 1000.0 * wall / n,
        "roofline": stream_roofline(kinds, ["sign_pack", "vote_update"]),
        "kernels": {k: kinds[k] for k in ("sign_pack", "vote_update") if k in kinds}}
    # polar step on the vote: vote as a matrix, its NS, the dense update
    cp = dataclasses.replace(cfg, vote_polar=True)
    t, wall, kinds = timed_steps(sm, torch, sm.StepCall(cp, mats), t, 2, n)
    g_ms, g_fl = gemm_totals(kinds)
    b_ms, b_fl = gemm_totals(base_kinds)
    extra_ms, extra_fl = g_ms - b_ms, g_fl - b_fl
    achieved = extra_fl / (extra_ms * 1e-3) / 1e12 if extra_ms > 0 else None
    peak = PEAK_TFLOPS[wl.mdt]
    out["vote_polar"] = {
        "value": n / wall, "unit": "steps/s", "ms_per_step": 1000.0 * wall / n,
        "extra_ms_per_step": 1000.0 * wall / n - base_ms,
        "roofline": {"bound": "mfma", "kernel": "ns_of_vote (gemm launches beyond the main "
                     "step's)", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak if achieved else None, "traffic": None,
                     "ms_per_step": extra_ms, "flops_per_step": extra_fl},
        "stream_roofline": stream_roofline(kinds, ["vote_update", "polar_update"]),
        "kernels": {k: kinds[k] for k in ("vote_update", "polar_update", "norm") if k in kinds}}
    return out, t


# Kernel source behind each GEMM kind, and the counter summary of the
# default workload's dominant kernel.
KERNEL_SOURCES = {"gemm_gram": "k_gemm_ns.hip", "gemm_apply": "k_gemm_ns.hip",
                  "gemm_rr": "k_gemm_ns.hip"}
TRAFFIC_SUMMARY = "profiles/{workload}.{kind}.hbm_traffic.md"


def source_sha256(kind):
    name = KERNEL_SOURCES.get(kind)
    if not name:
        return None
    path = os.path.join(ROOT, "matrix_aware_optimizer_momentum_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def recorded_traffic(workload, kind):
    """HBM bytes per launch recorded in the counter summary, if the kernel is unchanged."""
    path = os.path.join(ROOT, TRAFFIC_SUMMARY.format(workload=workload, kind=kind))
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != source_sha256(kind):
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None



def copy_calibration():
    """A plain device-to-device copy of known size, timed; its rocprofv3 FETCH_SIZE
    and WRITE_SIZE give the counters' scale (bytes moved / counter reading)."""
    import torch
    nbytes = 1 << 30
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
    y = torch.empty_like(x)
    for _ in range(2):
        y.copy_(x)
    torch.cuda.synchronize()
    reps = 10
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes,
                      "launches": reps + 2, "ms_per_copy": ms,
                      "copy_gbs": 2 * nbytes / (ms * 1e-3) / 1e9}))



def attainable_rates(sm, torch):
    """What the chip reaches at all on this machine, beside its nominal peaks: the
    MFMA ceiling probe (a bf16 GEMM k loop of the NS kernels' tile shape with
    its fragments read from LDS, or rotated in registers, and no global
    memory; and the same loop with the NS kernels' operand staging from an
    L2-sized buffer) and a plain 1 GiB device copy.  Medians of three timed
    runs after one warm-up."""
    out = torch.empty(256 * 256, dtype=torch.float32, device="cuda")
    src = torch.empty(1 << 19, dtype=torch.float32, device="cuda").uniform_()   # 2 MB
    res = {}
    for mode, key in ((1, "lds_operands"), (0, "register_operands"),
                      (2, "lds_operands_with_ns_staging")):
        rates = []
        for rep in range(4):
            e0, e1 = _events(torch)
            e0.record()
            flops = sm.mfma_ceiling(out, 256, 100000, mode, src)
            e1.record()
            torch.cuda.synchronize()
            if rep:
                rates.append(flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        res[key] = sorted(rates)[1]
    nbytes = 1 << 30
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
    y = torch.empty_like(x)
    y.copy_(x)
    rates = []
    for _ in range(3):
        e0, e1 = _events(torch)
        e0.record()
        y.copy_(x)
        e1.record()
        torch.cuda.synchronize()
        rates.append(2 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del x, y, out, src
    return {"mfma_loop_tflops": res, "copy_gbs": sorted(rates)[1],
            "probe": "sm_mfma_ceiling: 256 workgroups x 4 waves, each 100000 k16 slices of "
                     "16 v_mfma_f32_32x32x16_bf16 on a 128x128 float32 block (fragments from "
                     "LDS / registers; with staging: 8 direct-to-LDS loads per wave per k32 "
                     "step from a 2 MB buffer, each awaited three steps later, and one "
                     "barrier); device copy 1 GiB"}


def add_attainable(rl, att):
    """Attach the measured ceiling to a roofline object (its `peak` and `frac`
    stay the nominal ones)."""
    if not rl or att is None:
        return rl
    if rl.get("bound") == "mfma" and rl.get("unit") == "TFLOP/s" and rl.get("peak") == 2500.0:
        ceil = att["mfma_loop_tflops"]["lds_operands"]
        stg = att["mfma_loop_tflops"]["lds_operands_with_ns_staging"]
        rl["attainable"] = {"peak": ceil, "frac": rl["achieved"] / ceil,
                            "source": "MFMA ceiling probe, LDS operands",
                            "with_ns_staging": {"peak": stg, "frac": rl["achieved"] / stg}}
    elif rl.get("bound") == "hbm":
        ceil = att["copy_gbs"]
        rl["attainable"] = {"peak": ceil, "frac": rl["achieved"] / ceil,
                            "source": "plain 1 GiB device copy"}
    return rl


def _tdt(dt):
    import torch
    return torch.bfloat16 if dt == "bf16" else torch.float32


def build_state(wl, device="cuda"):
    """Weights, momentum, gradients (and CacheMuon caches) generated on the GPU."""
    import torch
    import matrix_aware_optimizer_momentum_amd as sm
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed)
    mats = []
    for (m, n) in wl.shapes:
        w = (0.02 * torch.randn(m, n, generator=gen, device=device)).to(_tdt(wl.wdt))
        mom = torch.zeros(wl.M, m, n, device=device, dtype=_tdt(wl.mdt))
        if wl.grad_kind == "student_t":
            z = torch.randn(wl.M, m, n, generator=gen, device=device)
            chi = torch.zeros_like(z)
            for _ in range(3):
                chi += torch.randn(wl.M, m, n, generator=gen, device=device) ** 2
            g = wl.grad_std * z / torch.sqrt(chi / 3.0)
            del z, chi
        else:
            g = wl.grad_std * torch.randn(wl.M, m, n, generator=gen, device=device)
        mb = sm.MatrixBuffers(w=w, mom=mom, grad=g.to(_tdt(wl.gdt)))
        del g
        if wl.algo == sm.CACHE_MUON:
            r = min(m, n)
            mb.q_cache = torch.zeros(wl.M, r, r, device=device)
            mb.cache_state = torch.zeros(wl.M, 2, dtype=torch.int32, device=device)
        mats.append(mb)
    return mats


def step_config(wl, gamma=None):
    import matrix_aware_optimizer_momentum_amd as sm
    return sm.StepConfig(algo=wl.algo, update=wl.update, M=wl.M, wdt=_tdt(wl.wdt),
                         mdt=_tdt(wl.mdt), gdt=_tdt(wl.gdt), lr=wl.lr, beta1=wl.beta1,
                         beta2=wl.beta2, period=wl.period,
                         ns=sm.NSParams(wl.ns_iters, wl.ns_a, wl.ns_b, wl.ns_c, wl.ns_eps),
                         gamma=wl.gamma if gamma is None else gamma, cache_mode=wl.cache_mode)



def _pearson(xs, ys):
    import math
    n = len(xs)
    if n < 2:
        return None
    mx, my = sum(xs) / n, sum(ys) / n
    sxy = sum((x - mx) * (y - my) for x, y in zip(xs, ys))
    sxx = sum((x - mx) ** 2 for x in xs)
    syy = sum((y - my) ** 2 for y in ys)
    return sxy / math.sqrt(sxx * syy) if sxx > 0 and syy > 0 else None


def _ranks(xs):
    order = sorted(range(len(xs)), key=lambda i: xs[i])
    r = [0.0] * len(xs)
    i = 0
    while i < len(order):
        j = i
        while j + 1 < len(order) and xs[order[j + 1]] == xs[order[i]]:
            j += 1
        for k in range(i, j + 1):
            r[order[k]] = (i + j) / 2.0
        i = j + 1
    return r


def fidelity(args, sm, torch, W):
    """CacheMuon fidelity diagnostic (the residual trigger against the spectral
    distance of the cached direction from a fresh solve, and the refresh rate)
    on an AR(1) gradient stream G_t = rho G_{t-1} + sqrt(1 - rho^2) sigma xi_t.
    After each step, for every diagnosed matrix: the cache as it was before the
    step is applied to the step's own momentum (forced reuse: D_hat and err),
    a fresh solve runs on a copy (D_fresh), and ||D_hat - D_fresh||_sp is
    estimated by the power method from a seeded start vector."""
    import math
    cfg_n = args.config if args.config != 2 else 4
    wl = W.WORKLOADS[cfg_n]
    if wl.algo != sm.CACHE_MUON:
        raise SystemExit("--fidelity needs a CacheMuon configuration")
    mats = build_state(wl)
    cfg = step_config(wl, args.gamma)
    nd = len(mats) if args.fidelity_matrices <= 0 else min(args.fidelity_matrices, len(mats))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed + 4242)
    rho = wl.ar1_rho
    diag = torch.zeros(len(mats), wl.M, 2, device="cuda")
    call = sm.StepCall(cfg, mats, diag=diag)
    # the diagnosed matrices, grouped by shape so each diagnostic call is batched
    groups = {}
    for j, mb in enumerate(mats[:nd]):
        groups.setdefault(tuple(mb.w.shape), []).append(j)
    v0s = {sh: torch.randn(len(js) * wl.M, sh[1], generator=gen, device="cuda")
           for sh, js in groups.items()}
    curve, pairs = [], []
    spec_ms, spec_work, spec_n = 0.0, 0.0, 0
    for t in range(1, args.fidelity_steps + 1):
        if t > 1:
            for mb in mats:
                xi = torch.randn(mb.grad.shape, generator=gen, device="cuda")
                g = rho * mb.grad.float() + math.sqrt(1 - rho * rho) * wl.grad_std * xi
                mb.grad.copy_(g.to(mb.grad.dtype))
                del xi, g
        before = [(mb.q_cache.clone(), mb.cache_state.clone()) for mb in mats[:nd]]
        call(t)
        torch.cuda.synchronize()
        refreshed = diag[:, :, 1].float().mean().item()
        errs, dists = [], []
        if t > 1:
            sm.profile_enable(True)
            sm.profile_reset()
            for sh, js in groups.items():
                x = torch.cat([mats[j].mom for j in js])
                q0 = torch.cat([before[j][0] for j in js])
                c0 = torch.cat([before[j][1] for j in js])
                d_hat, err, _ = sm.gram_ns_cached(x, q0.clone(), c0.clone(), t, 0.0,
                                                  mode=sm.MODE_FORCE_REUSE, params=cfg.ns)
                d_fr, _, _ = sm.gram_ns_cached(x, q0, c0, t, 0.0,
                                               mode=sm.MODE_FORCE_FRESH, params=cfg.ns)
                dist = sm.spectral_norm(d_hat, d_fr, v0s[sh], args.fidelity_iters)
                errs += err.cpu().tolist()
                dists += dist.cpu().tolist()
                del x, q0, c0, d_hat, d_fr
            ms, n, work = sm.profile_read("spectral")
            spec_ms, spec_work, spec_n = spec_ms + ms, spec_work + work, spec_n + n
            sm.profile_enable(False)
            pairs += list(zip(errs, dists))
        curve.append({"t": t, "refresh_rate": refreshed,
                      "err_mean": sum(errs) / len(errs) if errs else None,
                      "err_max": max(errs) if errs else None,
                      "dist_mean": sum(dists) / len(dists) if dists else None,
                      "dist_max": max(dists) if dists else None})
        print(json.dumps({"fidelity_step": t, **curve[-1]}), file=sys.stderr, flush=True)
    e = [p[0] for p in pairs]
    d = [p[1] for p in pairs]
    achieved = spec_work / (spec_ms * 1e-3) / 1e9 if spec_ms > 0 else None
    out = {
        "metric": "CacheMuon fidelity: residual err vs ||D_hat - D_fresh||_sp, refresh rate",
        "workload": wl.name, "gamma": cfg.gamma, "steps": args.fidelity_steps,
        "diagnosed_matrices": nd, "power_iters": args.fidelity_iters,
        "grad": f"AR(1) rho={rho} sigma={wl.grad_std}",
        "pearson_err_dist": _pearson(e, d),
        "spearman_err_dist": _pearson(_ranks(e), _ranks(d)) if len(e) > 1 else None,
        "refresh_rate_mean": sum(c["refresh_rate"] for c in curve) / len(curve),
        "spectral_roofline": {"bound": "hbm", "kernel": "k_pm_av / k_pm_atv (+ norms)",
                              "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": achieved / PEAK_HBM_GBS if achieved else None,
                              "launches": spec_n, "ms": spec_ms},
        "curve": curve,
    }
    print(json.dumps(out))


def host_info():
    """CPU model, BLAS library and the BLAS threads NumPy uses on this host."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    blas, threads = None, os.cpu_count()
    try:
        import threadpoolctl
        libs = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            threads = max(int(i.get("num_threads", 1)) for i in libs)
            blas = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in libs)
    except Exception:  # pragma: no cover
        pass
    return model, blas, threads


def _oracle_inputs(wl, m, n, rng):
    import numpy as np
    from matrix_aware_optimizer_momentum_amd import workloads as W
    w = W.as_storage((0.02 * rng.standard_normal((m, n))).astype(np.float32), wl.wdt)
    if wl.grad_kind == "student_t":
        g = rng.standard_t(3, size=(m, n))
    else:
        g = rng.standard_normal((m, n))
    g = W.as_storage((wl.grad_std * g).astype(np.float32), wl.gdt)
    return w, g


def cpu_baseline(wl, budget_s):
    """The oracle timed on this host on a bounded sample of the workload.

    One worker on one matrix of each distinct shape, per step type (LionMuon:
    a Muon step and a Lion step; CacheMuon: a fresh step, then a reuse step
    with the workload's gamma; Sign-Muon: one step); each time is scaled by
    the shape's matrix count times the worker count, and the step types are
    combined as the step schedule mixes them (LionMuon: (Muon + (P-1) Lion)
    / P).  Shapes not reached within the budget are extrapolated from the
    measured seconds per parameter."""
    import numpy as np
    from oracle import sm_oracle as O
    model, blas, threads = host_info()
    counts = {}
    for sh in wl.shapes:
        counts[sh] = counts.get(sh, 0) + 1
    order = sorted(counts, key=lambda sh: sh[0] * sh[1])
    ocfg = O.StepConfig(algo=wl.algo, update=wl.update, workers=1, wdtype=wl.wdt,
                        mdtype=wl.mdt, lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2,
                        period=wl.period, ns=O.NSParams(wl.ns_iters, wl.ns_a, wl.ns_b, wl.ns_c,
                                                        wl.ns_eps),
                        gamma=wl.gamma, cache_mode=wl.cache_mode)
    if wl.algo == O.LION_MUON:
        types = ([("muon", wl.period)] if wl.period > 0 else []) + [("lion", 1)]
    elif wl.algo == O.CACHE_MUON:
        types = [("fresh", 1), ("reuse", 2)]
    else:
        types = [("step", 1)]
    rng = np.random.default_rng(wl.seed)
    spent = 0.0
    per_type = {}
    covered = {typ: {} for typ, _ in types}
    for sh in order:
        m, n = sh
        w, g = _oracle_inputs(wl, m, n, rng)
        st = O.MatrixState(w=w.astype(np.float64), mom=[np.zeros((m, n))])
        for typ, t in types:
            if spent >= budget_s:
                break
            if typ == "reuse":        # continues from the fresh step's cache
                pass
            elif typ == "fresh":
                st = O.MatrixState(w=w.astype(np.float64), mom=[np.zeros((m, n))])
            t0 = time.perf_counter()
            O.step_matrix(st, [g], ocfg, t)
            dt = time.perf_counter() - t0
            spent += dt
            covered[typ][sh] = dt
    for typ, _ in types:
        done = covered[typ]
        if not done:
            continue
        secs = sum(counts[sh] * wl.M * done[sh] for sh in done)
        done_params = sum(counts[sh] * sh[0] * sh[1] for sh in done)
        per_param = secs / done_params
        missing = sum(counts[sh] * sh[0] * sh[1] for sh in counts if sh not in done)
        per_type[typ] = {"seconds_per_step": secs + per_param * missing,
                         "measured_shapes": [f"{a}x{b}" for a, b in done],
                         "seconds_measured": sum(done.values())}
    if wl.algo == O.LION_MUON and "muon" in per_type and "lion" in per_type:
        P = wl.period
        sec = (per_type["muon"]["seconds_per_step"] +
               (P - 1) * per_type["lion"]["seconds_per_step"]) / P
        how = f"P-averaged over P = {P} (one Muon step, {P - 1} Lion steps)"
    elif wl.algo == O.CACHE_MUON and "reuse" in per_type:
        sec = per_type["reuse"]["seconds_per_step"]
        how = "reuse step (gamma %g), fresh step reported beside it" % wl.gamma
    else:
        sec = next(iter(per_type.values()))["seconds_per_step"]
        how = "one step"
    total = sum(len(v) for v in covered.values())
    return {"value": 1.0 / sec, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"one worker on one matrix of each of {len(counts)} distinct shapes "
                       f"({total} oracle steps, {spent:.1f} s on the host), scaled by matrix "
                       f"count x {wl.M} workers; {how}; extrapolated"),
            "extrapolated": True, "seconds_per_step": sec, "cpu_model": model, "blas": blas,
            "per_step_type": per_type}


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def headline_roofline(kinds, mdt, wl_name, ms_per_step):
    dom = max(kinds, key=lambda k: kinds[k]["ms_per_step"])
    rl = kind_roofline(kinds, dom, mdt)
    roofline = {k: rl[k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    roofline["traffic"] = recorded_traffic(wl_name, dom)
    roofline.update({k: v for k, v in rl.items() if k not in roofline})
    others = {k: kind_roofline(kinds, k, mdt) for k in kinds
              if k != dom and kinds[k]["ms_per_step"] > 0.05 * ms_per_step}
    return roofline, others


def ns_summary(kinds, mdt, wl, ms_per_step, muon_fraction=1.0):
    out = {}
    ms, fl = gemm_totals(kinds)
    if ms > 0:
        out["ns_tflops"] = fl / (ms * 1e-3) / 1e12
        out["ns_mfma_frac"] = out["ns_tflops"] / PEAK_TFLOPS[mdt]
        # the direct iteration's flop count over the whole step time: the
        # rate the pages' form of the iteration would need to match this step
        out["ns_direct_form_equivalent_tflops"] = (wl.ns_flops_per_step() * muon_fraction /
                                                   (ms_per_step * 1e-3) / 1e12)
    if "vote_update" in kinds:
        vu = kinds["vote_update"]
        out["vote_update_gbs"] = vu["bytes"] / (vu["ms_per_step"] * 1e-3) / 1e9
        out["vote_update_hbm_frac"] = out["vote_update_gbs"] / PEAK_HBM_GBS
    return out


def graph_steps(sm, torch, cfg, mats, ws, t, steps):
    """The same Sign-Muon step recorded once as a HIP graph (sm_step_graph)
    and replayed `steps` times, timed by the wall clock like the direct calls:
    what a step costs once its kernel launches are not issued one by one."""
    g = sm.StepGraph(cfg, mats, t, ws=ws)
    for _ in range(3):
        g()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    g.close()
    return {"steps_per_s": steps / wall, "ms_per_step": 1000.0 * wall / steps, "steps": steps}


def sign_muon_sub(sm, torch, W, args, index=2, steps=None, variants=True):
    """A Sign-Muon configuration timed like the headline (wall clock over the
    timed steps), with its dominant-kernel roofline and the step variants."""
    wl = W.WORKLOADS[index]
    steps = steps or args.sub_steps
    mats = build_state(wl)
    cfg = step_config(wl)
    call = sm.StepCall(cfg, mats)
    t, wall, kinds = timed_steps(sm, torch, call, 1, 3, steps)
    ms = 1000.0 * wall / steps
    roofline, others = headline_roofline(kinds, wl.mdt, wl.name, ms)
    out = {"workload": wl.name, "value": steps / wall, "unit": "steps/s",
           "ms_per_step": ms, "steps": steps, "roofline": roofline,
           **ns_summary(kinds, wl.mdt, wl, ms), "other_rooflines": others, "kernels": kinds}
    out["graph"] = graph_steps(sm, torch, cfg, mats, call.ws, t, steps)
    if variants:
        v, t = measure_variants(sm, torch, wl, cfg, mats, t, args, ms, kinds)
        if v:
            out["variants"] = v
    del mats, call
    torch.cuda.empty_cache()
    return out


def _cache_flops(shapes, K):
    """Algorithmic orthogonalisation flops per problem: fresh Gram-NS solve
    2r^2c + 6Kr^3 + 2r^2c; cached candidate + residual probe 4r^2c."""
    fresh, probe = [], []
    for m, n in shapes:
        r, c = min(m, n), max(m, n)
        fresh.append(4.0 * r * r * c + 6.0 * K * r ** 3)
        probe.append(4.0 * r * r * c)
    return fresh, probe


def cache_muon_run(sm, torch, wl, gamma, mode, steps, warmup, label):
    """CacheMuon on an AR(1) gradient stream advanced before every step
    (outside the timed interval): per-step HIP events around sm_step, the
    refresh decisions and residuals read back after each step; then as many
    steps again on the same stream with the kernel-time accounting on (kept
    out of the timed steps)."""
    mats = build_state(wl)
    cfg = step_config(wl, gamma)
    cfg.cache_mode = mode
    M = wl.M
    diag = torch.zeros(len(mats), M, 2, device="cuda")
    call = sm.StepCall(cfg, mats, diag=diag)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed + 99)
    rho = wl.ar1_rho
    fresh_f, probe_f = _cache_flops(wl.shapes, wl.ns_iters)
    always_fresh = M * sum(fresh_f)
    rec = {"ms": [], "refreshed": [], "executed_flops": [], "errs": []}

    def advance():
        for mb in mats:
            xi = torch.randn(mb.grad.shape, generator=gen, device="cuda")
            g = rho * mb.grad.float() + math.sqrt(1 - rho * rho) * wl.grad_std * xi
            mb.grad.copy_(g.to(mb.grad.dtype))
            del xi, g

    for t in range(1, warmup + steps + 1):
        if t > 1:
            advance()
        timed = t > warmup
        e0, e1 = _events(torch)
        e0.record()
        call(t)
        e1.record()
        torch.cuda.synchronize()
        d = diag.cpu()
        refreshed = d[:, :, 1]
        probed = (d[:, :, 0] >= 0)
        if timed:
            rec["ms"].append(e0.elapsed_time(e1))
            rec["refreshed"].append(float(refreshed.mean()))
            ex = 0.0
            for j in range(len(mats)):
                ex += float(probed[j].sum()) * probe_f[j] + float(refreshed[j].sum()) * fresh_f[j]
            rec["executed_flops"].append(ex)
        rec["errs"] += [float(e) for e in d[:, :, 0].flatten() if e >= 0]
    sm.profile_enable(True)
    sm.profile_reset()
    for t in range(warmup + steps + 1, warmup + 2 * steps + 1):
        advance()
        call(t)
    torch.cuda.synchronize()
    kinds = read_kinds(sm, steps)
    sm.profile_enable(False)
    ms = sum(rec["ms"]) / steps
    ex = sum(rec["executed_flops"]) / steps
    gms, gfl = gemm_totals(kinds)
    gms += kinds.get("probe", {}).get("ms_per_step", 0.0)
    gfl += kinds.get("probe", {}).get("flops", 0.0)
    out = {"label": label, "gamma": gamma, "mode": ["trigger", "force_fresh", "force_reuse"][mode],
           "value": 1000.0 / ms, "unit": "steps/s (sum of per-step HIP event intervals)",
           "ms_per_step": ms, "steps": steps, "warmup": warmup,
           "refresh_rate": sum(rec["refreshed"]) / steps,
           "orth_flops_per_step": ex,
           "always_fresh_orth_flops_per_step": always_fresh,
           "orth_flop_reduction_vs_always_fresh": 1.0 - ex / always_fresh,
           "gemm_executed_tflops": gfl / (gms * 1e-3) / 1e12 if gms > 0 else None,
           "gemm_mfma_frac": (gfl / (gms * 1e-3) / 1e12 / PEAK_TFLOPS[wl.mdt]) if gms > 0 else None,
           "kernels": {k: {"ms_per_step": v["ms_per_step"], "launches_per_step":
                           v["launches_per_step"]} for k, v in kinds.items()}}
    errs = rec["errs"]
    del mats, call, diag
    torch.cuda.empty_cache()
    return out, errs


def cache_muon_sub(sm, torch, W, args):
    """CacheMuon (GPT-2 large, M = 1) at the pages' gamma = 2 and 15, at a
    mixed-rate gamma (the median residual of a calibration run, so that both
    branches run in the timed steps), and always-fresh (GramMuon)."""
    wl = W.WORKLOADS[4]
    steps, warmup = args.sub_steps, 2
    runs = {}
    for g in (2.0, 15.0):
        runs[f"gamma_{g:g}"], _ = cache_muon_run(sm, torch, wl, g, 0, steps, warmup, f"gamma {g:g}")
    # calibration: forced reuse, residuals of every cached candidate
    _, errs = cache_muon_run(sm, torch, wl, 0.0, 2, 3, 1, "calibration")
    errs.sort()
    g_mixed = errs[len(errs) // 2] if errs else 1.0
    runs["gamma_mixed"], _ = cache_muon_run(sm, torch, wl, g_mixed, 0, steps, warmup,
                                            "mixed-rate gamma (median residual)")
    runs["always_fresh"], _ = cache_muon_run(sm, torch, wl, 0.0, 1, steps, warmup,
                                             "always fresh (GramMuon)")
    return {"workload": wl.name, "grad": f"AR(1) rho={wl.ar1_rho} sigma={wl.grad_std}",
            "mixed_gamma": g_mixed, "runs": runs}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library "
              "has no multi-GPU exchange", file=sys.stderr)
        sys.exit(2)
    import torch
    import matrix_aware_optimizer_momentum_amd as sm
    from matrix_aware_optimizer_momentum_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration()
        return
    if args.attainable:
        print(json.dumps(attainable_rates(sm, torch)))
        return
    if args.fidelity:
        fidelity(args, sm, torch, W)
        return
    wl = W.WORKLOADS[args.config]
    P = wl.period if wl.algo == sm.LION_MUON else 0
    warmup = args.warmup if args.warmup is not None else (P if P else 3)
    steps = args.steps if args.steps is not None else (5 * P if P else 30)
    is_muon = (lambda t: P > 0 and t % P == 0) if wl.algo == sm.LION_MUON else (lambda t: True)

    mats = build_state(wl)
    cfg = step_config(wl, args.gamma)
    call = sm.StepCall(cfg, mats)
    torch.cuda.synchronize()
    print(f"bench: {wl.name}, warmup {warmup}, timed {steps}", file=sys.stderr, flush=True)

    t = 1
    for _ in range(warmup):
        call(t)
        t += 1
    torch.cuda.synchronize()

    sm.profile_enable(True)
    sm.profile_reset()
    evs = [_events(torch) for _ in range(steps)]
    types = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record()
        call(t)
        evs[i][1].record()
        types.append("muon" if is_muon(t) else "lion")
        t += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sm.profile_enable(False)
    step_ms = [a.elapsed_time(b) for a, b in evs]
    ms_per_step = 1000.0 * wall / steps
    value = steps / wall
    kinds = read_kinds(sm, steps)
    roofline, others = headline_roofline(kinds, wl.mdt, wl.name, ms_per_step)
    n_muon = types.count("muon")
    extra = ns_summary(kinds, wl.mdt, wl, ms_per_step, n_muon / steps)
    if others:
        extra["other_rooflines"] = others

    if wl.algo == sm.LION_MUON:
        # per step type: its mean time over the timed region, and a kernel
        # attribution of one more step of that type
        per = {}
        for typ in ("muon", "lion"):
            ms_t = [m for m, ty in zip(step_ms, types) if ty == typ]
            if not ms_t:
                continue
            while ("muon" if is_muon(t) else "lion") != typ:
                call(t)
                t += 1
            torch.cuda.synchronize()
            sm.profile_enable(True)
            sm.profile_reset()
            call(t)
            t += 1
            k1 = read_kinds(sm, 1)
            sm.profile_enable(False)
            ms1 = sum(ms_t) / len(ms_t)
            if typ == "muon":
                rl, oth = headline_roofline(k1, wl.mdt, wl.name, ms1)
                summ = ns_summary(k1, wl.mdt, wl, ms1)
            else:
                rl = stream_roofline(k1, ["lion"])
                oth = {k: kind_roofline(k1, k, wl.mdt) for k in k1 if k != "lion"
                       and k1[k]["ms_per_step"] > 0.05 * ms1}
                summ = ns_summary(k1, wl.mdt, wl, ms1, 0.0)
            per[typ] = {"steps_timed": len(ms_t), "ms_per_step": ms1,
                        "steps_per_s": 1000.0 / ms1, "roofline": rl, "other_rooflines": oth,
                        **summ, "kernels": k1}
        extra["per_step_type"] = per
        if "muon" in per and "lion" in per and P > 0:
            extra["p_averaged_steps_per_s"] = 1000.0 * P / (per["muon"]["ms_per_step"] +
                                                            (P - 1) * per["lion"]["ms_per_step"])
    if wl.algo == sm.CACHE_MUON:
        refreshed = sum(int(mb.cache_state[:, 1].eq(t - 1).sum().item()) for mb in mats)
        extra["last_step_refreshed_matrices"] = refreshed
    if wl.algo == sm.SIGN_MUON:
        variants, t = measure_variants(sm, torch, wl, cfg, mats, t, args, ms_per_step, kinds)
        if variants:
            extra["variants"] = variants
    del mats, call
    torch.cuda.empty_cache()
    att = None if args.no_attainable else attainable_rates(sm, torch)
    add_attainable(roofline, att)
    if att is not None and "ns_tflops" in extra and wl.mdt == "bf16":
        extra["ns_attainable_frac"] = extra["ns_tflops"] / att["mfma_loop_tflops"]["lds_operands"]
    for typ, rec in extra.get("per_step_type", {}).items():
        add_attainable(rec.get("roofline"), att)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "gpu_ms_per_step": sum(step_ms) / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.mdt,
        "data": "synthetic (seeded on-GPU Gaussian / AR(1) / Student-t gradients; no dataset)",
        "config": {"workload": wl.name, "matrices": len(wl.shapes), "params": wl.params,
                   "workers": wl.M, "ns_iters": wl.ns_iters, "algo": ["sign_muon", "cache_muon",
                                                                       "lion_muon"][wl.algo],
                   "period": wl.period, "muon_steps_timed": n_muon,
                   "weights": wl.wdt, "momentum": wl.mdt, "grads": wl.gdt},
        "roofline": roofline,
        "attainable": att,
        **extra,
        "kernels": kinds,
    }
    if not args.no_sub and args.config == DEFAULT_CONFIG:
        print("bench: sub-object gpt2_small", file=sys.stderr, flush=True)
        out["gpt2_small"] = sign_muon_sub(sm, torch, W, args, 2)
        print("bench: sub-object gpt2_large_cache_muon", file=sys.stderr, flush=True)
        out["gpt2_large_cache_muon"] = cache_muon_sub(sm, torch, W, args)
        print("bench: sub-objects resnet50, single_256", file=sys.stderr, flush=True)
        out["resnet50"] = sign_muon_sub(sm, torch, W, args, 3, variants=False)
        out["single_256"] = sign_muon_sub(sm, torch, W, args, 1, steps=100, variants=False)
        for key in ("gpt2_small", "resnet50", "single_256"):
            add_attainable(out[key].get("roofline"), att)
    if not args.no_cpu:
        print("bench: cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
