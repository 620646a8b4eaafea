#!/usr/bin/env python3
"""Benchmark of one training iteration of tile-based differentiable 3D Gaussian splatting on one
MI355X: project -> bin (radix sort) -> fused forward + L1 gradient + backward, for all views.

Default workload: 1M Gaussians in 64 blobs, 1920x1080, a batch of 4 ring views, SH degree 3
(the synthetic stand-in for the pages' large-scene captures).  Prints ONE JSON line with
Gaussian-pixel blends per second (fwd+bwd), ms per iteration, the fused rasterizer's roofline
figures and the CPU oracle's rate on the host as a baseline.  Everything else goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Gaussian-pixel blends/s (fwd+bwd) and ms/iter, 1M Gaussians @1080p, 1 GPU"
# Algorithmic float32 operations (FMA = 2) of the fused rasterizer, per unit:
FLOPS_PER_ALPHA_PAIR = 16  # evaluate one (pixel, Gaussian) pair whose alpha reaches alpha_min
FLOPS_PER_BLEND = 81      # blend it in the forward (11) and back-propagate it (70)
# Float32 vector peak of MI355X, the published rate: 256 CUs x 128 FMA lanes per cycle (4 SIMDs,
# each issuing a wave64 float32 instruction every 2 cycles) x 2 flops x 2.4 GHz = 157.3 TFLOP/s.
# Non-packed instructions with vector operands come close to it (a dense stream of them issues
# about every 2.5 cycles); the kernels here use no packed float32 instructions.
ALU_PEAK_TFLOPS = 256 * 128 * 2 * 2.4e9 / 1e12
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_raster_fused_1m_1080p.md")
RASTER_SRC = os.path.join(ROOT, "differentiable_raster_amd", "csrc", "raster.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic():
    """HBM bytes per fused launch from the committed rocprofv3 counter summary, if it was taken
    on the current rasterizer source (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            vals[k.strip()] = v.strip()
    src = hashlib.sha256(open(RASTER_SRC, "rb").read()).hexdigest()
    if vals.get("raster.hip sha256") != src:
        return None
    try:
        return float(vals["hbm bytes per launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(scene, settings, views, single_views):
    """The oracle as it stands (float64 C with OpenMP, NumPy binning): one full iteration of the
    given views on all host threads, then of `single_views` on one thread.  Also returns the
    oracle's pair counts E_tile (list entries walked up to each pixel's stop) and E_box (those
    whose exact alpha_min box holds the pixel) of the all-thread views."""
    import oracle
    oracle.build(force=False)
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    res = oracle.iteration(scene, settings, loss_scale=1.0, views=views, backward=True)
    dt = time.perf_counter() - t0
    blends = sum(r["fwd"]["n_blended"] for r in res)
    e_tile = sum(r["fwd"]["n_evaluated"] for r in res)
    e_box = sum(r["fwd"]["n_box"] for r in res)
    del res
    oracle.set_num_threads(1)
    t1 = time.perf_counter()
    res1 = oracle.iteration(scene, settings, loss_scale=1.0, views=single_views, backward=True)
    dt1 = time.perf_counter() - t1
    blends1 = sum(r["fwd"]["n_blended"] for r in res1)
    del res1
    oracle.set_num_threads(threads)
    model = cpu_model()
    out = dict(value=blends / dt, unit="blends/s", cores=threads, kind="oracle",
               sample=f"{len(views)} of {len(scene.cameras)} views of the same workload, one full iteration "
                      f"(project, bin, forward, L1 gradient, backward) in float64 on {threads} threads: {blends} "
                      f"blends in {dt:.2f} s; CPU {model}",
               cpu_model=model,
               single_thread=dict(value=blends1 / dt1, unit="blends/s", cores=1,
                                  sample=f"{len(single_views)} view(s), the same iteration on one thread: {blends1} "
                                         f"blends in {dt1:.2f} s"))
    return out, e_tile, e_box


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    # 10 warm-up steps and 100 timed ones (about 0.13 s at 1M Gaussians): with 3 and 20 the mean
    # still carried about 30 us per step of warm-up against the per-iteration median
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3, help="synthetic workload 1..5 (3 = 1M Gaussians @1080p)")
    ap.add_argument("--cap", type=int, default=0, help="per-tile cap K (0 = off)")
    ap.add_argument("--cpu-views", type=int, default=4, help="views of the workload the CPU oracle times on all threads "
                                                             "(the first of them is also timed on one thread)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device-to-device copy (3x), the reference kernel that "
                         "scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings to bytes")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); the library "
              f"has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    from differentiable_raster_amd import gsmi, pipeline, scenes
    gsmi.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t = time.perf_counter()
    scene = scenes.make_scene(args.workload)
    settings = scene.settings(tile_cap=args.cap)
    log(f"[bench] workload {args.workload} ({scene.name}) generated in {time.perf_counter() - t:.1f} s")
    # lean: the optional per-field projection arrays are not requested (nothing downstream reads
    # them; the packed records hold the same values)
    r = pipeline.Renderer(scene, settings, device="cuda:0", lean=True)

    # sizing pass and algorithmic counts (outside the timed region)
    r.project()
    info = r.bin()
    r.forward(counters=True)
    torch.cuda.synchronize()
    E_eval, B, E_alpha, _ = [int(x) for x in r.counters.cpu().tolist()]
    vis = [info.vis_count[v] for v in range(r.V)]
    M = int(info.num_instances)
    log(f"[bench] visible {vis}, instances {M}, evaluated pairs {E_eval}, pairs past the alpha test {E_alpha}, "
        f"blends {B}")

    if args.copy_calibration:
        src = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copies: 3 x {src.numel() * 4} bytes read and written")
        del src, dst

    def stage_times(mode, passes=11):
        """Per stage, the median over `passes` event-timed iterations of that stage's time."""
        times = {k: [] for k in ("project", "bin", "raster")}
        for _ in range(passes):
            ev = {k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for k in times}
            ev["project"][0].record(); r.project(); ev["project"][1].record()
            ev["bin"][0].record(); r.bin(); ev["bin"][1].record()
            ev["raster"][0].record()
            if mode == "fused":
                r.fused(image=False)
            else:
                r.forward()
                r.backward(r.loss_grad(1.0))
            ev["raster"][1].record()
            torch.cuda.synchronize()
            for k, (a, b) in ev.items():
                times[k].append(a.elapsed_time(b))
        return {k: statistics.median(v) for k, v in times.items()}

    def run(mode, steps, warmup):
        for _ in range(warmup):
            r.iteration(mode=mode)
        torch.cuda.synchronize()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            r.project()
            r.bin()
            starts[k].record()
            if mode == "fused":
                r.fused(image=False)
            else:
                r.forward()
                r.backward(r.loss_grad(1.0))
            ends[k].record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        raster_ms = sum(a.elapsed_time(b) for a, b in zip(starts, ends)) / steps
        return (t1 - t0) * 1000.0 / steps, raster_ms

    def timed_median(mode, min_iters=20, min_s=1.0):
        """Per-iteration hipEvent times on the library's stream (torch's current stream): the
        median of at least min_iters iterations spanning at least min_s seconds of GPU time."""
        times = []
        while len(times) < min_iters or sum(times) < min_s * 1e3:
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(50)]
            for a, b in ev:
                a.record()
                r.iteration(mode=mode)
                b.record()
            torch.cuda.synchronize()
            times += [a.elapsed_time(b) for a, b in ev]
        times.sort()
        return times[len(times) // 2], len(times), sum(times) / 1e3

    ms_fused, raster_fused_ms = run("fused", args.steps, args.warmup)
    med_fused, n_med, s_med = timed_median("fused")
    log(f"[bench] fused: median {med_fused:.3f} ms/iter over {n_med} event-timed iterations ({s_med:.2f} s)")
    stages_fused = stage_times("fused")
    ms_sep, raster_sep_ms = run("separate", max(3, args.steps // 4), 1)
    stages_sep = stage_times("separate")
    log(f"[bench] fused: {ms_fused:.3f} ms/iter (raster call {raster_fused_ms:.3f} ms); "
        f"separate: {ms_sep:.3f} ms/iter (raster calls {raster_sep_ms:.3f} ms)")

    # the projection backward (2D gradients of all views -> parameter gradients), one kernel,
    # timed on its own and inside a full training iteration
    r.project_backward()
    torch.cuda.synchronize()
    pb_steps = max(5, args.steps // 2)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(pb_steps)]
    for a, b in ev:
        a.record()
        r.project_backward()
        b.record()
    torch.cuda.synchronize()
    pb_ms = sum(a.elapsed_time(b) for a, b in ev) / pb_steps
    for _ in range(2):
        r.iteration(mode="fused", project_bwd=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(pb_steps):
        r.iteration(mode="fused", project_bwd=True)
    torch.cuda.synchronize()
    full_ms = (time.perf_counter() - t0) * 1000.0 / pb_steps
    nk = (scene.sh_degree + 1) ** 2
    # algorithmic bytes: the parameters of each Gaussian some view sees read once, the gradient
    # row of every Gaussian written once (zeros for the others), 4 (10 + 3 nk) B each, and the
    # vis_ids entry (4 B) and 36 B of 2D gradients per visible slot
    seen = torch.zeros(scene.n, dtype=torch.bool, device=r.vis_ids.device)
    for v in range(r.V):
        seen[r.vis_ids[v * r.capacity: v * r.capacity + vis[v]].long()] = True
    n_seen = int(seen.sum().item())
    del seen
    pb_bytes = 4 * (10 + 3 * nk) * (n_seen + scene.n) + (4 + 36) * sum(vis)
    # the seen-only form (gs_project_bwd_seen): rows of the seen Gaussians only, plus one flag byte
    # per Gaussian
    r.project_backward(seen_only=True)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(pb_steps)]
    for a, b in ev:
        a.record()
        r.project_backward(seen_only=True)
        b.record()
    torch.cuda.synchronize()
    pbs_ms = sum(a.elapsed_time(b) for a, b in ev) / pb_steps
    pbs_bytes = 2 * 4 * (10 + 3 * nk) * n_seen + scene.n + (4 + 36) * sum(vis)
    log(f"[bench] projection backward: {pb_ms:.3f} ms (seen rows only: {pbs_ms:.3f} ms); "
        f"full iteration with it: {full_ms:.3f} ms")

    # sparse exchange of this iteration's 2D gradient records: the encoder compacts the non-zero
    # (view, slot) records, the decoder adds them into per-view owner arrays indexed by Gaussian
    from differentiable_raster_amd import sparse
    codec = sparse.GradCodec(r.V, r.capacity, scene.n)
    r.fused(image=False)
    codec.encode(r.vis_count, r.vis_ids, r.grads)
    codec.decode()
    torch.cuda.synchronize()
    kept = int(codec.view_offset[-1].item())
    sp_steps = max(5, args.steps // 2)
    ev_e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(sp_steps)]
    ev_d = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(sp_steps)]
    for (a, b), (c, d) in zip(ev_e, ev_d):
        a.record()
        codec.encode(r.vis_count, r.vis_ids, r.grads)
        b.record()
        c.record()
        codec.decode()
        d.record()
    torch.cuda.synchronize()
    enc_ms = sum(a.elapsed_time(b) for a, b in ev_e) / sp_steps
    dec_ms = sum(c.elapsed_time(d) for c, d in ev_d) / sp_steps
    n_rec = sum(vis)
    # algorithmic bytes: the encoder reads every visible slot's 9 components once and, per kept
    # record, its Gaussian index and writes the 40 B record; the decoder reads the 40 B record and
    # reads and writes the 36 B owner entry
    enc_bytes = 36 * n_rec + (4 + 40) * kept
    dec_bytes = (40 + 72) * kept
    log(f"[bench] sparse gradients: {kept} of {n_rec} records non-zero ({100.0 * (1 - kept / max(1, n_rec)):.1f} % "
        f"dropped); encode {enc_ms:.3f} ms, decode {dec_ms:.3f} ms")

    # composition of pixel-level partial renders: two partials (colour on black + transmittance)
    # of every view, composed over the background
    P_cmp = 2
    r.forward()
    parts_c = [r.image, r.image.clone()]
    parts_t = [r.t_final, r.t_final.clone()]
    out_img = torch.empty_like(r.image)
    out_t = torch.empty_like(r.t_final)
    bg = settings.bg
    gsmi.gs_compose(r.V, r.W, r.H, parts_c, parts_t, bg, out_img, out_t)
    torch.cuda.synchronize()
    ev_c = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(sp_steps)]
    for a, b in ev_c:
        a.record()
        gsmi.gs_compose(r.V, r.W, r.H, parts_c, parts_t, bg, out_img, out_t)
        b.record()
    torch.cuda.synchronize()
    cmp_ms = sum(a.elapsed_time(b) for a, b in ev_c) / sp_steps
    # algorithmic bytes: 16 B (colour + transmittance) read per partial and pixel, 16 B written
    cmp_bytes = (16 * P_cmp + 16) * r.V * r.W * r.H
    log(f"[bench] composition of {P_cmp} partial renders: {cmp_ms:.3f} ms")

    # Adam over all parameters with this iteration's parameter gradients: the dense step and the
    # deferred step (Gaussians whose gradient row is zero are left for a later replay)
    from differentiable_raster_amd import adam as adam_mod
    r.project_backward()
    torch.cuda.synchronize()
    nk = (scene.sh_degree + 1) ** 2
    rows = [3, 3, 4, 1, 3 * nk]
    lrs = [1.6e-4, 5e-3, 1e-3, 5e-2, 2.5e-3]
    grads3 = [r.d_means3, r.d_log_scales3, r.d_quats3, r.d_logits3, r.d_sh3]
    zero_rows = int(sum((g.view(k, scene.n) != 0).any(0).logical_not().int() for g, k in zip(grads3, rows))
                    .eq(len(rows)).sum().item())
    r.project_backward(seen_only=True)  # the seen flags of this iteration
    torch.cuda.synchronize()
    adam_ms = {}
    for kind in ("dense", "deferred", "seen"):
        params = [t.clone() for t in (r.means, r.log_scales, r.quats, r.logits, r.sh)]
        st = adam_mod.AdamState(scene.n, list(zip(params, grads3, rows, lrs)), deferred=kind != "dense")
        seen_arg = r.seen if kind == "seen" else None
        st.step(seen=seen_arg)
        torch.cuda.synchronize()
        ev_a = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(sp_steps)]
        for a, b in ev_a:
            a.record()
            st.step(seen=seen_arg)
            b.record()
        torch.cuda.synchronize()
        adam_ms[kind] = sum(a.elapsed_time(b) for a, b in ev_a) / sp_steps
        del st, params
    comps = sum(rows)
    # algorithmic bytes: per component of an updated Gaussian the parameter and both moments read
    # and written and the gradient read (28 B); the deferred step reads the whole gradient row of a
    # skipped Gaussian (4 B per component) and the step counter of every Gaussian (+4 B written
    # for the updated ones)
    dense_bytes = 28 * comps * scene.n
    lazy_bytes = 28 * comps * (scene.n - zero_rows) + 4 * comps * zero_rows + 4 * scene.n + 4 * (scene.n - zero_rows)
    # with seen flags: one flag byte per Gaussian, and the step counter read and written and the
    # 28 B per component for each seen one
    seen_bytes = 28 * comps * n_seen + scene.n + 8 * n_seen
    log(f"[bench] Adam: dense {adam_ms['dense']:.3f} ms, deferred {adam_ms['deferred']:.3f} ms "
        f"({zero_rows} of {scene.n} Gaussians without gradient), deferred with seen flags "
        f"{adam_ms['seen']:.3f} ms ({n_seen} seen)")

    flops = FLOPS_PER_ALPHA_PAIR * E_alpha + FLOPS_PER_BLEND * B
    achieved = flops / (raster_fused_ms * 1e-3) / 1e12
    # the committed counter summary was taken on the default workload (1M Gaussians, 1080p, 4
    # views, no cap); other workloads have no counter figure
    traffic = measured_traffic() if (args.workload == 3 and args.cap == 0) else None
    P = r.V * r.W * r.H
    M_K = int(info.num_instances_capped) if args.cap > 0 else M
    N_vis = sum(vis)
    # the minimum HBM bytes of the fused rasterizer: each (capped) list entry's record and slot
    # (40 B), the target of every pixel (12 B), the 2D gradient of every visible slot (36 B)
    alg_bytes = 40 * M_K + 12 * P + 36 * N_vis
    # this design's own: + per entry its instance index inputs (12 B) and its partial gradient
    # record written by the rasterizer and read back by the per-Gaussian reduction (2 x 36 B)
    design_bytes = (40 + 12 + 2 * 36) * M_K + 12 * P + 36 * N_vis
    hbm_achieved = alg_bytes / (raster_fused_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": B / (ms_fused * 1e-3),
        "unit": "blends/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_fused,
        "ms_per_iter_median": med_fused,
        "median_iterations": n_med,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{scene.name}: {scene.n} Gaussians, {r.W}x{r.H}, {r.V} views, SH degree "
                        f"{scene.sh_degree}, project + bin + fused fwd/L1/bwd"
                        + (f", tile cap {args.cap}" if args.cap else ""),
            "gaussians": scene.n, "width": r.W, "height": r.H, "views": r.V, "tile_cap": args.cap,
        },
        "roofline": {
            "kernel": "raster_fused (gs_raster_fused call: fused kernel, per-Gaussian reduction)",
            "bound": "alu",
            "achieved": achieved,
            "peak": ALU_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / ALU_PEAK_TFLOPS,
            "traffic": traffic,
            "algorithmic_flops": flops,
            "launch_ms": raster_fused_ms,
            "hbm": {"algorithmic_bytes": alg_bytes, "achieved": hbm_achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": hbm_achieved / HBM_PEAK_GBS, "design_bytes": design_bytes,
                    "target_frac": 0.5, "met": hbm_achieved / HBM_PEAK_GBS >= 0.5},
        },
        "counts": {"visible": vis, "instances": M, "instances_capped": M_K, "evaluated_pairs": E_eval,
                   "alpha_pairs": E_alpha, "blends": B, "e_box": None, "e_tile": None},
        "stages_ms": {"fused": stages_fused, "separate": stages_sep},
        "separate_path": {"ms_per_step": ms_sep, "blends_per_s": B / (ms_sep * 1e-3), "raster_ms": raster_sep_ms},
        "cpu_baseline": None,
        "sparse_grads": {
            "kernels": "encode_count/scan/encode_write (gs_grad_encode), decode_kernel (gs_grad_decode)",
            "records": n_rec, "kept": kept, "dropped_fraction": 1.0 - kept / max(1, n_rec),
            "page_figure": "ByteSplat: 65.8 % less backward inter-GPU communication volume (six real datasets)",
            "bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "encode": {"ms": enc_ms, "algorithmic_bytes": enc_bytes, "achieved": enc_bytes / (enc_ms * 1e-3) / 1e9,
                       "frac": enc_bytes / (enc_ms * 1e-3) / (HBM_PEAK_GBS * 1e9)},
            "decode": {"ms": dec_ms, "algorithmic_bytes": dec_bytes, "achieved": dec_bytes / (dec_ms * 1e-3) / 1e9,
                       "frac": dec_bytes / (dec_ms * 1e-3) / (HBM_PEAK_GBS * 1e9)},
        },
        "compose": {
            "kernel": "compose_kernel (gs_compose)", "partials": P_cmp, "ms": cmp_ms, "bound": "hbm",
            "algorithmic_bytes": cmp_bytes, "achieved": cmp_bytes / (cmp_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": cmp_bytes / (cmp_ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
        },
        "adam": {
            "kernel": "adam_step_kernel (gs_adam_step)", "gaussians": scene.n, "components": comps,
            "gaussians_without_gradient": zero_rows, "bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "dense": {"ms": adam_ms["dense"], "algorithmic_bytes": dense_bytes,
                      "achieved": dense_bytes / (adam_ms["dense"] * 1e-3) / 1e9,
                      "frac": dense_bytes / (adam_ms["dense"] * 1e-3) / (HBM_PEAK_GBS * 1e9)},
            "deferred": {"ms": adam_ms["deferred"], "algorithmic_bytes": lazy_bytes,
                         "achieved": lazy_bytes / (adam_ms["deferred"] * 1e-3) / 1e9,
                         "frac": lazy_bytes / (adam_ms["deferred"] * 1e-3) / (HBM_PEAK_GBS * 1e9)},
            "deferred_seen": {"kernel": "adam_step_kernel (gs_adam_step_seen)", "ms": adam_ms["seen"],
                              "gaussians_seen": n_seen, "algorithmic_bytes": seen_bytes,
                              "achieved": seen_bytes / (adam_ms["seen"] * 1e-3) / 1e9,
                              "frac": seen_bytes / (adam_ms["seen"] * 1e-3) / (HBM_PEAK_GBS * 1e9)},
        },
        "project_bwd": {
            "kernel": "project_bwd_kernel (gs_project_bwd)",
            "ms": pb_ms,
            "bound": "hbm",
            "algorithmic_bytes": pb_bytes,
            "gaussians_seen": n_seen,
            "achieved": pb_bytes / (pb_ms * 1e-3) / 1e9,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": pb_bytes / (pb_ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
            "full_iteration_ms": full_ms,
            "seen_only": {"kernel": "project_bwd_kernel (gs_project_bwd_seen)", "ms": pbs_ms,
                          "algorithmic_bytes": pbs_bytes,
                          "achieved": pbs_bytes / (pbs_ms * 1e-3) / 1e9,
                          "frac": pbs_bytes / (pbs_ms * 1e-3) / (HBM_PEAK_GBS * 1e9)},
            # one training step with frustum culling and deferred updates: the fused iteration,
            # the seen-only projection backward and the seen-flag Adam step
            "training_step_ms": med_fused + pbs_ms + adam_ms["seen"],
        },
    }
    if not args.no_cpu_baseline:
        views = list(range(min(args.cpu_views, r.V)))
        out["cpu_baseline"], e_tile, e_box = cpu_baseline(scene, settings, views, views[:1])
        if len(views) == r.V:
            out["counts"]["e_tile"], out["counts"]["e_box"] = e_tile, e_box
        log(f"[bench] cpu baseline: {out['cpu_baseline']}; E_tile {e_tile}, E_box {e_box}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
