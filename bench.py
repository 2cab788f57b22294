"""Benchmark of the Muon-family optimizer step on one MI355X.

Default workload: the GPT-2-small layer set (12 layers x {768x2304, 768x768,
768x3072, 3072x768}, 84,934,656 parameters), Sign-Muon with M = 5 simulated
workers, bf16 momentum / Newton-Schulz operands with float32 accumulation,
5 cubic NS iterations, 1-bit packed majority vote.  A step is one sm_step
call: momentum EMA + norm, NS, sign + pack, vote + update for all 48
matrices.  Inputs are synthetic and resident in HBM before timing starts.

Prints one JSON line: steps/s (value), the roofline of the dominant kernel
measured with HIP events on the step's stream over the timed region, and the
CPU oracle timed on a bounded sample on this host.  After the main timed
region, `variants` times the same step with the int8 sign encoding and with
the optional polar step on the vote (--variant-steps each, default 10; the
main `value` is always the 1-bit vote step).

  python bench.py [--steps K] [--warmup W] [--config {1..5}] [--no-cpu]
  python bench.py --copy-calibration   # plain device copy of known size, for
                                       # scaling rocprofv3 FETCH_SIZE / WRITE_SIZE
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
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
METRIC = "optimizer steps/s per layer set; NS TFLOP/s (MFMA %); vote+update GB/s (HBM %)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--gamma", type=float, default=None, help="CacheMuon threshold override")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (counter scaling)")
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
                         "vote); 0 skips them")
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
    """Roofline of one kernel kind.  A GEMM kind sits under the MFMA roof when
    its arithmetic intensity (algorithmic flops / algorithmic HBM bytes) is at
    least the ridge point peak_flops / peak_bandwidth, else under the HBM roof;
    `achieved` is then algorithmic bytes per launch / average launch time."""
    dk = kinds[kind]
    out = {"kernel": kind, "avg_launch_ms": dk["avg_launch_ms"],
           "work_per_launch": dk["work_per_launch"]}
    secs = dk["avg_launch_ms"] * 1e-3
    if kind.startswith(("gemm", "probe")):
        peak_f = PEAK_TFLOPS[mdt]
        ai = dk["flops"] / dk["hbm_bytes"] if dk.get("hbm_bytes") else float("inf")
        ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
        out.update(arith_intensity=ai, ridge=ridge, bytes_per_launch=dk.get("bytes_per_launch"))
        if ai >= ridge:
            achieved = dk["work_per_launch"] / secs / 1e12
            out.update(bound="mfma", achieved=achieved, peak=peak_f, unit="TFLOP/s")
        else:
            achieved = dk["bytes_per_launch"] / secs / 1e9
            out.update(bound="hbm", achieved=achieved, peak=PEAK_HBM_GBS, unit="GB/s",
                       tflops=dk["work_per_launch"] / secs / 1e12)
    else:
        achieved = dk["work_per_launch"] / secs / 1e9
        out.update(bound="hbm", achieved=achieved, peak=PEAK_HBM_GBS, unit="GB/s")
    out["frac"] = out["achieved"] / out["peak"]
    return out


def timed_steps(sm, torch, call, t, warmup, steps):
    """warmup untimed steps, then `steps` timed ones with kernel accounting on."""
    for _ in range(warmup):
        call(t)
        t += 1
    torch.cuda.synchronize()
    sm.profile_enable(True)
    sm.profile_reset()
    t0 = time.perf_counter()
    for _ in range(steps):
        call(t)
        t += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
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


def stream_bytes(wl, kind):
    """Algorithmic bytes per step of one streaming kernel kind (whole layer set)."""
    es = {"bf16": 2, "f32": 4}
    n = wl.params
    if kind == "ema":        # read G and M, write M and the NS input copy
        return n * wl.M * (es[wl.gdt] + 2 * es[wl.mdt] + es[wl.mdt])
    if kind == "sign_pack":  # read D, write 1 bit
        return n * wl.M * (es[wl.mdt] + 1 / 8)
    if kind == "vote_update":
        return n * (wl.M / 8 + 2 * es[wl.wdt])
    return 0.0


def cpu_baseline(wl, seconds):
    """The oracle's step on a bounded sample of the layer set, on this host's cores."""
    import numpy as np
    from matrix_aware_optimizer_momentum_amd import workloads as W
    from oracle import sm_oracle as O
    try:
        import threadpoolctl
        threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()),
                      default=os.cpu_count())
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    ocfg = O.StepConfig(algo=wl.algo, update=wl.update, workers=wl.M, wdtype=wl.wdt,
                        mdtype=wl.mdt, lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2,
                        period=wl.period, ns=O.NSParams(wl.ns_iters, wl.ns_a, wl.ns_b, wl.ns_c,
                                                        wl.ns_eps),
                        gamma=wl.gamma, cache_mode=wl.cache_mode)
    done_params = 0
    elapsed = 0.0
    nmat = 0
    rng = np.random.default_rng(wl.seed)
    for (m, n) in wl.shapes:
        w = W.as_storage((0.02 * rng.standard_normal((m, n))).astype(np.float32), wl.wdt)
        g = [W.as_storage((wl.grad_std * rng.standard_normal((m, n))).astype(np.float32), wl.gdt)
             for _ in range(wl.M)]
        st = O.MatrixState(w=w.astype(np.float64), mom=[np.zeros((m, n)) for _ in range(wl.M)])
        t0 = time.perf_counter()
        O.step_matrix(st, g, ocfg, 1)
        elapsed += time.perf_counter() - t0
        done_params += m * n
        nmat += 1
        if elapsed >= seconds:
            break
    scale = wl.params / done_params
    sec_per_step = elapsed * scale
    return {"value": 1.0 / sec_per_step, "unit": "steps/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"{nmat} of {len(wl.shapes)} matrices ({done_params} of {wl.params} "
                       f"parameters) x {wl.M} workers, one step, {elapsed:.1f} s; "
                       f"{'extrapolated x%.2f to the whole layer set' % scale if scale > 1 else 'whole layer set'}"),
            "seconds_per_step": sec_per_step}


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
    if args.fidelity:
        fidelity(args, sm, torch, W)
        return
    wl = W.WORKLOADS[args.config]
    mats = build_state(wl)
    cfg = step_config(wl, args.gamma)
    call = sm.StepCall(cfg, mats)
    torch.cuda.synchronize()

    t = 1
    for _ in range(args.warmup):
        call(t)
        t += 1
    torch.cuda.synchronize()

    sm.profile_enable(True)
    sm.profile_reset()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        call(t)
        t += 1
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sm.profile_enable(False)
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = 1000.0 * wall / args.steps
    value = args.steps / wall

    kinds = read_kinds(sm, args.steps)
    dom = max(kinds, key=lambda k: kinds[k]["ms_per_step"])
    rl = kind_roofline(kinds, dom, wl.mdt)
    roofline = {k: rl[k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    roofline["traffic"] = recorded_traffic(wl.name, dom)
    roofline.update({k: v for k, v in rl.items() if k not in roofline})
    others = {k: kind_roofline(kinds, k, wl.mdt) for k in kinds
              if k != dom and kinds[k]["ms_per_step"] > 0.05 * ms_per_step}

    ns_ms = sum(kinds.get(k, {}).get("ms_per_step", 0.0) for k in ("gemm_gram", "gemm_apply",
                                                                   "gemm_rr"))
    ns_flops = sum(kinds.get(k, {}).get("flops", 0.0) for k in ("gemm_gram", "gemm_apply",
                                                               "gemm_rr"))
    extra = {}
    if ns_ms > 0:
        extra["ns_tflops"] = ns_flops / (ns_ms * 1e-3) / 1e12
        extra["ns_mfma_frac"] = extra["ns_tflops"] / PEAK_TFLOPS[wl.mdt]
        # the direct iteration's flop count over the whole step time: the
        # rate the pages' form of the iteration would need to match this step
        extra["ns_direct_form_equivalent_tflops"] = (wl.ns_flops_per_step() /
                                                     (ms_per_step * 1e-3) / 1e12)
    if others:
        extra["other_rooflines"] = others
    if "vote_update" in kinds:
        vu = kinds["vote_update"]
        extra["vote_update_gbs"] = vu["bytes"] / (vu["ms_per_step"] * 1e-3) / 1e9
        extra["vote_update_hbm_frac"] = extra["vote_update_gbs"] / PEAK_HBM_GBS
    if wl.algo == sm.CACHE_MUON:
        refreshed = sum(int(mb.cache_state[:, 1].eq(t - 1).sum().item()) for mb in mats)
        extra["last_step_refreshed_matrices"] = refreshed
    variants, t = measure_variants(sm, torch, wl, cfg, mats, t, args, ms_per_step, kinds)
    if variants:
        extra["variants"] = variants

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "gpu_ms_per_step": gpu_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.mdt,
        "data": "synthetic (seeded on-GPU Gaussian / AR(1) / Student-t gradients; no dataset)",
        "config": {"workload": wl.name, "matrices": len(wl.shapes), "params": wl.params,
                   "workers": wl.M, "ns_iters": wl.ns_iters, "algo": ["sign_muon", "cache_muon",
                                                                       "lion_muon"][wl.algo],
                   "weights": wl.wdt, "momentum": wl.mdt, "grads": wl.gdt},
        "roofline": roofline,
        **extra,
        "kernels": kinds,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
