"""Benchmark of the SSB phase-variance evaluation on one MI355X.

One step = one exact phase-variance loss evaluation (one trial) of the full
workload: 512 x 512 scan x 8,937 BF pixels, from cached complex64 spectra
already resident in HBM.  Prints one JSON line (rank 0, one GPU).

Also reported: the object redraw, the loss and object from one call, the per-trial
time inside a 200-trial batch,
the spectrum build (prepare), per-stage device times measured with HIP events on
the library's stream, the roofline of the dominant kernel, and the float64
oracle timed on the host's cores over whole evaluations (a process pool over BF
ranges), with its results compared with the library's.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ms per phase-variance eval + BF×scan samples/s at 512²×8,937 BF (1 GPU)"
# Checkpoints page, "fftA intermediate and M5 hardware floor": 222.7 ms p50 per
# evaluation of 2,342,780,928 BF x scan samples on an Apple M5 (another machine;
# real data with 2,464 aperture-active BF, ours has all 8,937 active).
PAGES_MS = 222.7
PEAK_FP32_TFLOPS = 157.3    # MI355X FP32 vector (256 CU x 2.4 GHz, packed)
PEAK_HBM_GBS = 8000.0
# vector-instruction issue ceiling: a wave64 VALU instruction occupies a 16-lane SIMD for
# 4 cycles; 256 CUs x 4 SIMDs at 2.4 GHz
PEAK_VALU_ISSUE = 256 * 4 * 2.4e9 / 4


def algorithmic_work(n: int, info: dict) -> dict:
    """Algorithmic HBM bytes and FLOPs per active BF plane and trial, by stage.

    From the library's own support tables (ssb_query): pass 1 reads the
    nonzero-transfer spectrum entries (complex64) and writes the column results of
    the column tiles that hold any support; pass 2 reads the nonzero columns and
    writes one float phase-sum image per 32 BF.  FLOPs: 5 n log2 n per complex
    n-point transform, 45 per nonzero-transfer correction, 23 per phase sample
    (atan2 and moments).
    """
    act = max(1, info["n_active_bf"])
    sup = info["support_entries"] / act
    cw = info["columns_written"] / act
    cr = info["columns_read"] / act
    fft = 5.0 * n * math.log2(n)
    return {
        "pass1": {"bytes": 8.0 * sup + 8.0 * n * cw, "flops": cw * fft + 45.0 * sup},
        "pass2": {"bytes": 8.0 * n * cr + 4.0 * n * n / 32.0, "flops": (n // 2) * fft + 23.0 * n * n},
    }


def stage_rates(n: int, info: dict, prof: dict) -> dict:
    """Average launch time, algorithmic bytes and FLOPs per launch, and the rates they
    give, for pass 1 and pass 2 (launch counts and planes from ssb_profile)."""
    work = algorithmic_work(n, info)
    out = {}
    for k in ("pass1", "pass2"):
        launches = max(1, prof[k]["launches"])
        t = prof[k]["ms"] / launches * 1e-3
        units = prof[k]["units"] / launches
        b = work[k]["bytes"] * units
        f = work[k]["flops"] * units
        out[k] = {"avg_launch_ms": t * 1e3, "planes_per_launch": units, "bytes": b, "flops": f,
                  "gbs": b / t / 1e9, "tflops": f / t / 1e12}
    return out


def kernel_source_hash() -> str:
    """Hash of the HIP kernel sources the measured HBM traffic belongs to (code only:
    comments and blank lines are dropped, so a comment edit keeps the counters valid)."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "aberration_phase_variance_amd", "csrc")
    hsh = hashlib.sha256()
    for name in ("ssb_kernels.hip", "ssb_fft.hpp", "ssb_internal.hpp", "ssb_math.hpp"):
        with open(os.path.join(csrc, name)) as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        for line in text.splitlines():
            code = line.split("//", 1)[0].strip()
            if code:
                hsh.update(code.encode() + b"\n")
    return hsh.hexdigest()[:16]


def plain_stream_gbs(dev) -> float:
    """HBM rate of a plain elementwise add (2 GiB read + 2 GiB written per call), best of 5."""
    import torch
    x = torch.ones(1 << 29, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    torch.add(x, 1.0, out=y)
    best = float("inf")
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.add(x, 1.0, out=y)
        e1.record()
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del x, y
    return 2.0 * (1 << 31) / (best * 1e-3) / 1e9


def _counter_line(kernel: str):
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    want = kernel_source_hash()
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) >= 4 and not line.startswith("#") and parts[0] == kernel and parts[1] == want:
                return parts
    return None


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed counter summary, if it matches these sources."""
    parts = _counter_line(kernel)
    return float(parts[2]) + float(parts[3]) if parts else None


def issue_view(kernel: str, launch_ms: float):
    """Vector-instruction issue time of one launch (SQ_INSTS_VALU from the committed counter
    summary, if it matches these sources) against the measured launch time."""
    parts = _counter_line(kernel)
    if not parts or len(parts) < 5:
        return None
    insts = float(parts[4])
    issue_ms = insts / PEAK_VALU_ISSUE * 1e3
    return {"valu_wave_instructions": insts, "issue_ms": round(issue_ms, 4),
            "frac": round(issue_ms / launch_ms, 4), "peak_wave_instructions_per_s": PEAK_VALU_ISSUE}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="full", choices=["tiny", "small", "medium", "full", "full1024"])
    ap.add_argument("--batch", type=int, default=200, help="trials in the batched measurement (0 = skip)")
    ap.add_argument("--cpu-baseline", type=int, default=1,
                    help="time the float64 oracle on the host's cores (process pool over BF ranges): one whole "
                         "evaluation and the object of this workload, whole tiny/small/medium evaluations; 0 = skip")
    ap.add_argument("--detector", type=int, default=1,
                    help="also time the detector side on full frames (detector sum, probe fit, BF gather); 0 = skip")
    ap.add_argument("--scan1024", type=int, default=1,
                    help="also time the 1024^2 scan workload (8,937 BF, 1024-point transforms); 0 = skip")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy (3x) as a known-size reference "
                         "for hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path shards over BF pixels "
              "but this build runs on a single device.", file=sys.stderr)
        sys.exit(2)

    import torch

    import aberration_phase_variance_amd as ssb
    from synth import WORKLOADS, make_counts_numpy, make_counts_torch, trial_params

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    w = WORKLOADS[args.config]
    g = w.geometry
    n = g.scan_n
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)      # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log(f"[bench] generating {w.name} counts ({w.n_bf} BF x {n}^2)")
    t0 = time.perf_counter()
    if n >= 256:
        counts = make_counts_torch(w, dev)
    else:
        counts = torch.from_numpy(make_counts_numpy(w).view(np.int32)).to(dev)
    torch.cuda.synchronize()
    log(f"[bench] counts ready in {time.perf_counter() - t0:.1f} s")

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    h = ssb.ssb_prepare(g, counts, w.n_bf)
    torch.cuda.synchronize()
    prepare_ms = (time.perf_counter() - t0) * 1e3
    info = ssb.ssb_query(h)
    log(f"[bench] prepare {prepare_ms:.1f} ms, spectra {info['spectrum_bytes'] / 1e9:.2f} GB, chunk {info['chunk_bf']}")

    params = np.array([w.true_params], dtype=np.float32)
    for _ in range(args.warmup):
        ssb.ssb_loss(h, params)
    torch.cuda.synchronize()
    samples = w.n_bf * n * n
    times = []
    t_all = time.perf_counter()
    for _ in range(args.steps):
        t1 = time.perf_counter()
        loss = ssb.ssb_loss(h, params)[0]     # synchronizes the stream before returning
        times.append((time.perf_counter() - t1) * 1e3)
    torch.cuda.synchronize()
    total_s = time.perf_counter() - t_all
    ms_per_step = total_s * 1e3 / args.steps
    log(f"[bench] loss {loss:.9f}: {ms_per_step:.3f} ms/eval (p50 {np.median(times):.3f}, "
        f"p95 {np.percentile(times, 95):.3f}, min {min(times):.3f})")

    # the full-plane variant (every entry of the N x N plane corrected on its own)
    ssb.ssb_set_variant(h, ssb.SSB_VARIANT_FULL_PLANE)
    for _ in range(2):
        ssb.ssb_loss(h, params)
    fp_steps = max(3, min(args.steps, 10))
    t1 = time.perf_counter()
    for _ in range(fp_steps):
        fp_loss = ssb.ssb_loss(h, params)[0]
    fp_ms = (time.perf_counter() - t1) * 1e3 / fp_steps
    fp_phase = torch.empty((n, n), dtype=torch.float32, device=dev)
    ssb.ssb_object(h, params[0], fp_phase)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(3):
        ssb.ssb_object(h, params[0], fp_phase)
    torch.cuda.synchronize()
    fp_obj_ms = (time.perf_counter() - t1) * 1e3 / 3
    ssb.ssb_loss_object(h, params[0], fp_phase)
    t1 = time.perf_counter()
    for _ in range(3):
        fp_lo = ssb.ssb_loss_object(h, params[0], fp_phase)
    fp_lo_ms = (time.perf_counter() - t1) * 1e3 / 3
    ssb.ssb_set_variant(h, ssb.SSB_VARIANT_HALF_PLANE)
    del fp_phase
    full_plane = {"ms_per_eval": fp_ms, "loss": fp_loss, "object_ms": fp_obj_ms, "loss_object_ms": fp_lo_ms,
                  "loss_object_same_loss": bool(fp_lo == fp_loss),
                  "loss_rel_diff_vs_half_plane": abs(fp_loss - loss) / abs(loss)}
    log(f"[bench] full-plane variant: {fp_ms:.3f} ms/eval, loss {fp_loss:.9f}, object {fp_obj_ms:.3f} ms, "
        f"loss and object in one call {fp_lo_ms:.3f} ms")

    # per-stage device times (HIP events on the library's stream), separate pass
    ssb.ssb_profile(h, 1)
    prof_steps = max(3, min(args.steps, 10))
    for _ in range(prof_steps):
        ssb.ssb_loss(h, params)
    phase = torch.empty((n, n), dtype=torch.float32, device=dev)
    for _ in range(3):
        ssb.ssb_object(h, params[0], phase)
    prof = ssb.ssb_profile(h, 0)
    torch.cuda.synchronize()

    # object redraw, host clock
    ssb.ssb_object(h, params[0], phase)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    n_obj = 5
    for _ in range(n_obj):
        ssb.ssb_object(h, params[0], phase)
    torch.cuda.synchronize()
    object_ms = (time.perf_counter() - t1) * 1e3 / n_obj
    log(f"[bench] object {object_ms:.3f} ms")

    # loss and object from one pass (ssb_loss_object), host clock, synchronizing call
    lo_loss = ssb.ssb_loss_object(h, params[0], phase)
    t1 = time.perf_counter()
    for _ in range(n_obj):
        lo_loss = ssb.ssb_loss_object(h, params[0], phase)
    loss_object_ms = (time.perf_counter() - t1) * 1e3 / n_obj
    log(f"[bench] loss and object in one call {loss_object_ms:.3f} ms (loss bitwise ssb_loss's: {lo_loss == loss})")

    batch_ms_per_trial = None
    fit = None
    if args.batch > 0:
        bp = trial_params(w, args.batch)
        ssb.ssb_loss(h, bp[:2])
        t1 = time.perf_counter()
        bl = ssb.ssb_loss(h, bp)
        batch_ms_per_trial = (time.perf_counter() - t1) * 1e3 / args.batch
        log(f"[bench] batch of {args.batch}: {batch_ms_per_trial:.3f} ms/trial")
        # the full fit as the workload defines it: the same batch, then 34 scalar refinement
        # evaluations (Nelder-Mead from the batch's best trial, stopped after 34 physical
        # evaluations); and the same refinement run until its tolerances are met
        t1 = time.perf_counter()
        fr = ssb.ssb_fit(h, bp, {"max_evals": 34})
        fit_ms = (time.perf_counter() - t1) * 1e3
        t1 = time.perf_counter()
        fc = ssb.ssb_fit(h, bp)
        conv_ms = (time.perf_counter() - t1) * 1e3
        fit = {"ms": fit_ms, "trials": args.batch, "refine_evals": fr["evals"], "refine_requests": fr["requests"],
               "converged": bool(fr["converged"]), "batch_best": fr["batch_best"], "batch_loss": fr["batch_loss"],
               "best": fr["best"], "loss": fr["loss"], "true": list(w.true_params),
               "to_tolerance": {"ms": conv_ms, "refine_evals": fc["evals"], "converged": bool(fc["converged"]),
                                "best": fc["best"], "loss": fc["loss"]}}
        log(f"[bench] fit: {fit_ms:.1f} ms ({args.batch} trials + {fr['evals']} refinement evaluations), "
            f"best {[round(v, 3) for v in fr['best']]} loss {fr['loss']:.9f}; to tolerance {conv_ms:.1f} ms "
            f"({fc['evals']} evaluations), best {[round(v, 3) for v in fc['best']]}")

    # roofline of the dominant stage: algorithmic bytes (or FLOPs) per launch / average launch time
    share = info["support_entries"] / (info["n_bf"] * n * (n // 2 + 1))
    work = algorithmic_work(n, info)
    stage_ms = {k: prof[k]["ms"] / max(1, prof[k]["launches"]) for k in prof}
    dom = max(("pass1", "pass2"), key=lambda k: prof[k]["ms"])
    units_per_launch = prof[dom]["units"] / max(1, prof[dom]["launches"])
    t_launch = stage_ms[dom] * 1e-3
    bytes_launch = work[dom]["bytes"] * units_per_launch
    flops_launch = work[dom]["flops"] * units_per_launch
    hbm_bound = bytes_launch / (PEAK_HBM_GBS * 1e9) >= flops_launch / (PEAK_FP32_TFLOPS * 1e12)
    achieved_gbs = bytes_launch / t_launch / 1e9
    achieved_tf = flops_launch / t_launch / 1e12
    traffic = measured_traffic(dom)
    if hbm_bound:
        roofline = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved_gbs / PEAK_HBM_GBS, 4)}
    else:
        roofline = {"bound": "alu", "achieved": round(achieved_tf, 3), "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved_tf / PEAK_FP32_TFLOPS, 4)}
    roofline.update({"traffic": traffic, "kernel": dom, "avg_launch_ms": round(stage_ms[dom], 4),
                     "planes_per_launch": units_per_launch, "algorithmic_bytes_per_launch": bytes_launch,
                     "algorithmic_flops_per_launch": flops_launch,
                     "flops_view": {"achieved_tflops": round(achieved_tf, 3), "peak": PEAK_FP32_TFLOPS,
                                    "frac": round(achieved_tf / PEAK_FP32_TFLOPS, 4)},
                     "kernel_source": kernel_source_hash(),
                     "issue_view": issue_view(dom, stage_ms[dom])})
    # the practical HBM ceiling on this GPU for context: a plain elementwise add over 2 GiB
    # (one read and one write stream), timed with events on torch's stream
    stream_gbs = plain_stream_gbs(dev)
    roofline.update({"stream_gbs": round(stream_gbs, 1),
                     "frac_of_stream": round(achieved_gbs / stream_gbs, 4) if roofline["bound"] == "hbm" else None})
    other = "pass2" if dom == "pass1" else "pass1"
    t_other = stage_ms[other] * 1e-3
    other_units = prof[other]["units"] / max(1, prof[other]["launches"])
    stages_roofline = {other: {"avg_launch_ms": round(stage_ms[other], 4),
                               "achieved_gbs": round(work[other]["bytes"] * other_units / t_other / 1e9, 1),
                               "achieved_tflops": round(work[other]["flops"] * other_units / t_other / 1e12, 3),
                               "issue_view": issue_view(other, stage_ms[other])}}
    g_bytes = info["spectrum_bytes"]
    hbm = {"spectrum_read_gb": g_bytes / 1e9,
           "spectrum_read_frac_of_step": round(g_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    # the whole evaluation's counted HBM bytes (both passes, committed counters) per step
    t_pass1, t_pass2 = measured_traffic("pass1"), measured_traffic("pass2")
    if t_pass1 is not None and t_pass2 is not None:
        ev_gbs = (t_pass1 + t_pass2) / (ms_per_step * 1e-3) / 1e9
        hbm.update({"evaluation_counted_gb": round((t_pass1 + t_pass2) / 1e9, 3),
                    "evaluation_gbs": round(ev_gbs, 1), "evaluation_frac_of_peak": round(ev_gbs / PEAK_HBM_GBS, 4),
                    "evaluation_frac_of_stream": round(ev_gbs / stream_gbs, 4)})

    # oracle on the host: whole evaluations with the pooled float64 oracle (every BF pixel,
    # BF ranges over the host's cores), compared with the library's results
    cpu = None
    oracle_check = None
    if args.cpu_baseline:
        from oracle import ssb_oracle as O
        from oracle.pool import OraclePool
        from synth import cached_counts

        dc = info["dc"]
        og = O.OGeom.from_any(g)
        mp = torch.full((n, n), float("nan"), dtype=torch.float32, device=dev)
        gpu_loss = ssb.ssb_loss(h, params, mp)[0]
        gpu_phase = torch.full((n, n), float("nan"), dtype=torch.float32, device=dev)
        ssb.ssb_object(h, params[0], gpu_phase)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        pool = OraclePool(lambda b0, b1: counts[b0:b1].cpu().numpy().view(np.uint32), shape=(w.n_bf, n, n))
        stage_s = time.perf_counter() - t1
        try:
            log(f"[bench] oracle: whole {w.name} evaluation on {pool.workers} worker processes ...")
            t1 = time.perf_counter()
            r1, r2 = pool.moments(og, params[0], dc)
            eval_s = time.perf_counter() - t1
            ref_loss = O.loss_from_moments(r1, r2, w.n_bf)
            t1 = time.perf_counter()
            ref_phase, _ = pool.object_wave(og, params[0], dc)
            obj_s = time.perf_counter() - t1
        finally:
            pool.close()
        whole = {}
        for wn in ("tiny", "small", "medium"):
            if wn == w.name:
                continue
            ws = WORKLOADS[wn]
            if ws.geometry.scan_n >= 256:
                cs = make_counts_torch(ws, dev).cpu().numpy().view(np.uint32)
            else:
                cs = cached_counts(ws)
            with OraclePool(cs) as pw:
                t1 = time.perf_counter()
                pw.loss(O.OGeom.from_any(ws.geometry), ws.true_params, O.dc_value(cs))
                whole[wn] = {"s": time.perf_counter() - t1, "samples": ws.n_bf * ws.geometry.scan_n ** 2,
                             "workers": pw.workers}
            del cs
        cpu = {"value": samples / eval_s, "unit": "BF×scan samples/s", "cores": pool.workers, "kind": "oracle",
               "sample": f"one whole {w.name} evaluation ({w.n_bf} BF x {n}^2 scan, every BF pixel) of the float64 "
                         f"oracle at the true aberrations: {eval_s:.1f} s on {pool.workers} worker processes "
                         f"(BF ranges, one NumPy thread each); the object over every BF pixel took {obj_s:.1f} s",
               "eval_s": eval_s, "ms_per_eval": eval_s * 1e3, "object_s": obj_s, "staging_s": stage_s,
               "host_cores_available": len(os.sched_getaffinity(0)), "whole_evaluations": whole}
        d = np.angle(np.exp(1j * (gpu_phase.cpu().numpy() - ref_phase)))
        dm = mp.cpu().numpy() - r1 / w.n_bf
        oracle_check = {"bf_range": [0, w.n_bf], "loss_gpu": gpu_loss, "loss_oracle": ref_loss,
                        "loss_rel_err": abs(gpu_loss - ref_loss) / abs(ref_loss),
                        "mean_phase_max_abs_err": float(np.max(np.abs(dm))),
                        "object_phase_rms_rad": float(np.sqrt(np.mean(d * d)))}
        log(f"[bench] oracle whole evaluation {eval_s:.1f} s, object {obj_s:.1f} s; loss rel err "
            f"{oracle_check['loss_rel_err']:.2e}, object rms {oracle_check['object_phase_rms_rad']:.2e} rad")
        del gpu_phase, mp

    ssb.ssb_release(h)
    del counts
    torch.cuda.empty_cache()

    detector = None
    if args.detector:
        import dataclasses

        from synth import make_frames_torch
        log(f"[bench] generating {w.name} detector frames ({n * n} x {g.det_n}^2)")
        frames = make_frames_torch(w, dev)
        torch.cuda.synchronize()
        d2 = g.det_n * g.det_n
        sums = torch.empty(d2, dtype=torch.int64, device=dev)
        ssb.ssb_detector_sum(frames, n, g.det_n, sums)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record()
        for _ in range(reps):
            ssb.ssb_detector_sum(frames, n, g.det_n, sums)      # the library's null stream = torch's current
        e1.record()
        torch.cuda.synchronize()
        sum_ms = e0.elapsed_time(e1) / reps
        t1 = time.perf_counter()
        pfit = ssb.ssb_fit_probe_device(sums, n, g.det_n)            # synchronizes
        fit_ms = (time.perf_counter() - t1) * 1e3
        host_fit_same = pfit == ssb.ssb_fit_probe(sums.cpu().numpy().view(np.uint64), n, g.det_n)
        geom = dataclasses.replace(g, det_cy=pfit["det_cy"], det_cx=pfit["det_cx"], bf_r2=pfit["bf_r2"])
        bfc = torch.empty((pfit["n_bf"], n, n), dtype=torch.int32, device=dev)
        ssb.ssb_gather_bf(frames, geom, bfc, pfit["n_bf"])
        t1 = time.perf_counter()
        for _ in range(3):
            ssb.ssb_gather_bf(frames, geom, bfc, pfit["n_bf"])   # synchronizes
        gather_ms = (time.perf_counter() - t1) * 1e3 / 3
        frame_bytes = n * n * d2 * 4
        detector = {"frames": [n * n, d2], "frame_bytes": frame_bytes,
                    "detector_sum_ms": sum_ms, "detector_sum_gbs": frame_bytes / sum_ms / 1e6,
                    "detector_sum_hbm_frac": round(frame_bytes / sum_ms / 1e6 / PEAK_HBM_GBS, 4),
                    "fit": pfit, "fit_ms_device": fit_ms, "fit_same_as_host": bool(host_fit_same),
                    "gather_ms_host_clock": gather_ms,
                    "gather_gbs": 2 * pfit["n_bf"] * n * n * 4 / gather_ms / 1e6}
        log(f"[bench] detector sum {sum_ms:.3f} ms ({detector['detector_sum_gbs']:.0f} GB/s), fit on the device "
            f"{fit_ms:.3f} ms (bitwise the host fit: {host_fit_same}) n_bf {pfit['n_bf']} r^2 {pfit['bf_r2']:.2f}, "
            f"gather {gather_ms:.3f} ms")
        del frames, bfc, sums
        torch.cuda.empty_cache()

    scan1024 = None
    if args.scan1024 and args.config == "full":
        w2 = WORKLOADS["full1024"]
        n2 = w2.geometry.scan_n
        log(f"[bench] generating {w2.name} counts ({w2.n_bf} BF x {n2}^2)")
        counts2 = make_counts_torch(w2, dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        h2 = ssb.ssb_prepare(w2.geometry, counts2, w2.n_bf)
        torch.cuda.synchronize()
        prep2 = (time.perf_counter() - t0) * 1e3
        del counts2
        torch.cuda.empty_cache()
        info2 = ssb.ssb_query(h2)
        p2 = np.array([w2.true_params], dtype=np.float32)
        for _ in range(args.warmup):
            ssb.ssb_loss(h2, p2)
        torch.cuda.synchronize()
        steps2 = max(3, min(args.steps, 10))
        t1 = time.perf_counter()
        for _ in range(steps2):
            loss2 = ssb.ssb_loss(h2, p2)[0]
        ms2 = (time.perf_counter() - t1) * 1e3 / steps2
        ssb.ssb_profile(h2, 1)
        for _ in range(3):
            ssb.ssb_loss(h2, p2)
        prof2 = ssb.ssb_profile(h2, 0)
        phase2 = torch.empty((n2, n2), dtype=torch.float32, device=dev)
        ssb.ssb_object(h2, p2[0], phase2)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(3):
            ssb.ssb_object(h2, p2[0], phase2)
        torch.cuda.synchronize()
        obj2 = (time.perf_counter() - t1) * 1e3 / 3
        ssb.ssb_loss_object(h2, p2[0], phase2)
        t1 = time.perf_counter()
        for _ in range(3):
            ssb.ssb_loss_object(h2, p2[0], phase2)
        lo2 = (time.perf_counter() - t1) * 1e3 / 3
        ssb.ssb_release(h2)
        del phase2
        torch.cuda.empty_cache()
        r2 = stage_rates(n2, info2, prof2)
        dom2 = max(("pass1", "pass2"), key=lambda k: r2[k]["avg_launch_ms"])
        scan1024 = {
            "workload": f"{w2.name}: {n2}x{n2} scan, {w2.geometry.det_n}x{w2.geometry.det_n} detector, "
                        f"{w2.n_bf} BF, one trial per evaluation",
            "ms_per_eval": ms2, "samples_per_s": w2.n_bf * n2 * n2 / (ms2 * 1e-3), "loss": loss2,
            "object_ms": obj2, "loss_object_ms": lo2, "prepare_ms": prep2, "spectrum_gb": info2["spectrum_bytes"] / 1e9,
            "chunk_bf": info2["chunk_bf"],
            "roofline": {"bound": "hbm", "kernel": dom2, "achieved": round(r2[dom2]["gbs"], 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(r2[dom2]["gbs"] / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic(dom2 + "@1024"),
                         "frac_of_stream": round(r2[dom2]["gbs"] / stream_gbs, 4),
                         "issue_view": issue_view(dom2 + "@1024", r2[dom2]["avg_launch_ms"])},
            "stages": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in r2[k].items()}
                       for k in r2},
            # notes page, "128 GB Apple M5 Max size-scaling follow-up": scalar evaluator
            # 168.5 ms at 1024 on 2,476 compact planes of Fourier-resized evidence
            "pages_context_ms": 168.538,
        }
        log(f"[bench] scan 1024: {ms2:.3f} ms/eval, pass1 {r2['pass1']['avg_launch_ms']:.3f} ms, "
            f"pass2 {r2['pass2']['avg_launch_ms']:.3f} ms, object {obj2:.3f} ms, loss and object {lo2:.3f} ms")

    value = samples * args.steps / total_s
    pages_rate = samples / (PAGES_MS * 1e-3) if args.config == "full" else None
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "BF×scan samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": (value / pages_rate) if pages_rate else None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {n}x{n} scan, {g.det_n}x{g.det_n} detector, {w.n_bf} BF, "
                               f"uint32 Poisson counts, one trial per step",
                   "scan_n": n, "det_n": g.det_n, "n_bf": w.n_bf, "trials_per_step": 1},
        "loss": loss,
        "ms_p50": float(np.median(times)),
        "ms_p95": float(np.percentile(times, 95)),
        "ms_min": float(min(times)),
        "object_ms": object_ms,
        "loss_object_ms": loss_object_ms,
        "loss_object_same_loss": bool(lo_loss == loss),
        "batch_trials": args.batch,
        "batch_ms_per_trial": batch_ms_per_trial,
        "fit": fit,
        "prepare_ms": prepare_ms,
        "stage_ms_per_launch": {k: round(v, 4) for k, v in stage_ms.items()},
        "support_share": share,
        "roofline": roofline,
        "other_stage": stages_roofline,
        "hbm": hbm,
        "cpu_baseline": cpu,
        "detector": detector,
        "full_plane_variant": full_plane,
        "scan1024": scan1024,
        "oracle_check": oracle_check,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
