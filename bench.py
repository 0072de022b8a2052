"""Benchmark: hierarchical local attention forward at the 8K workload on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 8k] [--cpu-seconds S]
                    [--radius R] [--guide-mode M] [--text T] [--backward] [--rope-at-load]
                    [--permute-free]

A step is one full uhla_forward (cos/sin table -> K, V permutation, K fused with RoPE ->
hi-res block-sparse attention with Q rotated at load and the inverse permutation fused
into its stores -> guide attention) over one batch of synthetic inputs already resident
in HBM.  Prints ONE JSON line.

value       effective TFLOP/s of the whole step: algorithmic FLOPs (4 * head_dim per
            unmasked (query, key) pair) / step time.  --radius / --guide-mode measure the
            mask variants of uhla_forward_masked instead (default: the pages' mask), and
            --text T a joint sequence with T text tokens (uhla_forward_text).
            --backward times a training step instead: uhla_forward_lse then uhla_backward
            (algorithmic FLOPs: 4*d per pair forward, 10*d per pair backward).
            --rope-at-load times uhla_forward_rope_at_load (K rotated at every K tile
            load instead of once in the prep pass), --permute-free
            uhla_forward_permute_free (no K/V prep pass: tiles copied from the raster
            K and V, K rotated at load, V read transposed from LDS).
roofline    the dominant kernel (hi-res attention pass) against the bf16 MFMA peak:
            its algorithmic FLOPs per launch / its mean launch duration, measured with
            HIP events recorded on the launch stream around each launch in as many steps
            again through uhla_forward_timed; stage_ms are those durations.  The timed
            steps themselves call the plain entry point (no timer events).
cpu_baseline  the fp64 oracle on a time-bounded, stratified sample of query rows of four
            heads of the same workload, on this host's cores, in the same unit, with the
            full oracle time extrapolated from it (labelled as such).
attention_passes  the same FLOPs over the attention passes alone (prep excluded).
permute     the standalone uhla_window_permute of the Q hi segment in GB/s, beside a plain
            device-to-device copy of the same bytes and uhla_copy_probe of the same bytes
            through each load path (plain, nontemporal, direct-to-LDS).
prep        the forward's own permutes (K rotated, V as V^T tiles; default mask): their
            algorithmic bytes (K and V of every row read and written once) over the prep
            stages' durations.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s (unmasked blocks) + tokens/s, 8K fwd; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
ATTN_SOURCE = os.path.join(ROOT, "global_attention_image_amd", "csrc", "attention.hip")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_hi_8k_hbm_traffic.md")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch of the hi attention kernel from the committed counter summary,
    or None when the summary is missing or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    fields = {}
    for line in open(TRAFFIC_PROFILE):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].rsplit(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("attention.hip sha256[:16]") != source_hash(ATTN_SOURCE):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def stratified_rows(geom, rng, n):
    """n query rows of one (batch, head), drawn class by class in proportion to each class's
    share of the L rows (at least one each): hi rows of corner, edge and interior windows,
    and guide rows."""
    nwy, nwx, w = geom.H // geom.w, geom.W // geom.w, geom.w
    r = np.arange(geom.N)
    wy, wx = (r // geom.W) // w, (r % geom.W) // w
    on_y, on_x = (wy == 0) | (wy == nwy - 1), (wx == 0) | (wx == nwx - 1)
    classes = [r[on_y & on_x], r[on_y ^ on_x], r[~on_y & ~on_x],
               np.arange(geom.N, geom.N + geom.M)]
    classes = [c for c in classes if len(c)]
    sizes = np.array([len(c) for c in classes], dtype=np.float64)
    take = np.maximum(1, np.round(n * sizes / sizes.sum()).astype(int))
    rows = [rng.choice(c, min(t, len(c)), replace=False) for c, t in zip(classes, take)]
    return np.sort(np.concatenate(rows))


def cpu_baseline(geom, q, k, v, seconds):
    """Time the oracle on stratified query rows of a few heads spread over the head range
    (batch 0), a share of the time budget per head, and extrapolate the full oracle time."""
    import oracle.uhla_oracle as orc
    from global_attention_image_amd.inputs import bf16_bits_to_f64
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(0)
    heads = sorted({0, geom.heads // 3, (2 * geom.heads) // 3, geom.heads - 1})
    t_start = time.perf_counter()
    rows_done, pairs, t_rot, t_rows = 0, 0, 0.0, 0.0
    block = 64
    for i, h in enumerate(heads):
        t0 = time.perf_counter()
        qs = bf16_bits_to_f64(q[0:1, :, h:h + 1, :])
        ks = bf16_bits_to_f64(k[0:1, :, h:h + 1, :])
        vs = bf16_bits_to_f64(v[0:1, :, h:h + 1, :])
        qk = orc.rotated_qk(qs, ks, geom, 0, 0)
        t1 = time.perf_counter()
        t_rot += t1 - t0
        budget = (seconds - (t1 - t_start)) / (len(heads) - i)
        while True:
            rows = stratified_rows(geom, rng, block)
            orc.attention_rows(qs, ks, vs, geom, 0, 0, rows, block=block, qk=qk)
            rows_done += len(rows)
            pairs += int(orc.allowed_key_count(geom, rows).sum())
            if time.perf_counter() - t1 >= budget:
                break
        t_rows += time.perf_counter() - t1
    dt = time.perf_counter() - t_start
    flops = 4 * geom.head_dim * pairs
    bh = geom.B * geom.heads
    full_s = bh * t_rot / len(heads) + t_rows / rows_done * bh * geom.L
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{rows_done} query rows of batch 0, heads {heads} of the {geom.name} "
                      f"workload, stratified by class in proportion to its share of the rows "
                      f"(corner / edge / interior windows, guide rows); per head the RoPE of "
                      f"that head, then explicit mask rows and a dense fp64 softmax over all "
                      f"{geom.L} keys; {dt:.1f} s wall; FLOPs counted as 4*d per unmasked pair",
            "seconds": round(dt, 3),
            "extrapolated_full_oracle_s": round(full_s, 1),
            "extrapolation": "extrapolated, not measured: mean RoPE time per head x B*heads + "
                             "mean time per query row x B*heads*L; an upper estimate (full "
                             "oracle runs at 2k and nonsquare took 0.89 and 0.63 of it)"}


def bench_backward(args, g):
    """Training step: uhla_forward_lse + uhla_backward on the workload, dO synthetic."""
    import torch
    from global_attention_image_amd import api
    from global_attention_image_amd.inputs import CONFIG_SEEDS, algorithmic_pairs, make_qkv_bits
    log(f"[bench] backward: generating seeded inputs for {g}")
    q, k, v = make_qkv_bits(g, CONFIG_SEEDS[g.name])
    do = make_qkv_bits(g, CONFIG_SEEDS[g.name] + 100)[0]
    dev = torch.device("cuda:0")
    up = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
    qt, kt, vt, gt = up(q), up(k), up(v), up(do)
    out = torch.empty_like(qt)
    lse = torch.empty((g.B, g.heads, g.L), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(qt), torch.empty_like(qt), torch.empty_like(qt)
    fws = api.alloc_workspace(g.B, g.H, g.W, g.w, g.H_lr, g.W_lr, g.heads, g.head_dim, dev,
                              rho=g.rho, radius=g.radius, guide_mode=g.guide_mode, T=g.T)
    nb = api.backward_workspace_bytes(g.B, g.T, g.H, g.W, g.w, g.H_lr, g.W_lr, g.rho, g.heads,
                                      g.head_dim, g.radius, g.guide_mode)
    bws = torch.empty(nb, dtype=torch.uint8, device=dev)
    fwd = lambda: api.forward_lse(qt, kt, vt, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho,
                                  theta=g.theta, radius=g.radius, guide_mode=g.guide_mode,
                                  T=g.T, out=out, lse=lse, workspace=fws)
    bwd = lambda: api.backward(qt, kt, vt, out, gt, lse, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho,
                               theta=g.theta, radius=g.radius, T=g.T, guide_mode=g.guide_mode,
                               dq=dq, dk=dk, dv=dv, workspace=bws)
    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record()
        fwd()
        e1.record()
        bwd()
        e2.record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    f_ms = sum(a.elapsed_time(b) for a, b, _ in ev) / args.steps
    b_ms = sum(b.elapsed_time(c) for _, b, c in ev) / args.steps
    pairs = algorithmic_pairs(g)["total"] * g.B * g.heads
    f_fl, b_fl = 4 * g.head_dim * pairs, 10 * g.head_dim * pairs
    res = {
        "metric": METRIC + " (training step: forward with LSE + backward)",
        "value": round((f_fl + b_fl) / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": g.name, "B": g.B, "heads": g.heads, "head_dim": g.head_dim,
                   "grid": f"{g.H}x{g.W}", "window": g.w, "guide_grid": f"{g.H_lr}x{g.W_lr}",
                   "rho": g.rho, "neighbourhood_radius": g.radius, "guide_mode": g.guide_mode,
                   "text_tokens": g.T, "parallelism": "single GPU"},
        "forward_ms": round(f_ms, 4), "backward_ms": round(b_ms, 4),
        "algorithmic_flops": {"forward": f_fl, "backward": b_fl},
        "roofline": {"kernel": "uhla_backward (all its kernels)", "bound": "mfma",
                     "achieved": round(b_fl / (b_ms * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(b_fl / (b_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="8k")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--radius", type=int, default=1)
    ap.add_argument("--guide-mode", type=int, default=0, choices=(0, 1, 2))
    ap.add_argument("--text", type=int, default=0, help="text tokens in the joint sequence")
    ap.add_argument("--backward", action="store_true", help="time forward (with LSE) + backward")
    ap.add_argument("--rope-at-load", action="store_true",
                    help="uhla_forward_rope_at_load: K rotated at every K tile load")
    ap.add_argument("--permute-free", action="store_true",
                    help="uhla_forward_permute_free: no K/V prep pass")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from global_attention_image_amd import api
    from global_attention_image_amd.inputs import (CONFIGS, CONFIG_SEEDS, algorithmic_flops,
                                                    algorithmic_pairs, make_qkv_bits)

    g = CONFIGS[args.config].with_(radius=args.radius, guide_mode=args.guide_mode, T=args.text)
    if args.backward:
        return bench_backward(args, g)
    variant = (args.radius != 1 or args.guide_mode != 0 or args.text != 0 or args.rope_at_load
               or args.permute_free)
    log(f"[bench] generating seeded inputs for {g}")
    t0 = time.perf_counter()
    q, k, v = make_qkv_bits(g, CONFIG_SEEDS[args.config])
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s; uploading")
    dev = torch.device("cuda:0")
    up = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
    qt, kt, vt = up(q), up(k), up(v)
    out = torch.empty_like(qt)
    ws = api.alloc_workspace(g.B, g.H, g.W, g.w, g.H_lr, g.W_lr, g.heads, g.head_dim, dev,
                             rho=g.rho, radius=g.radius, guide_mode=g.guide_mode, T=g.T,
                             permute_free=args.permute_free)
    fwd = lambda timer=None: api.forward(qt, kt, vt, g.H, g.W, g.w, g.H_lr, g.W_lr, rho=g.rho,
                                         theta=g.theta, out=out, workspace=ws, timer=timer,
                                         radius=g.radius, guide_mode=g.guide_mode, T=g.T,
                                         rope_at_load=args.rope_at_load,
                                         permute_free=args.permute_free)
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    log(f"[bench] warmup done; timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fwd()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # The spread of per-step device times, from as many steps again with HIP events
    # around each (kept out of the timed loop above, whose wall time is the value).
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for e_a, e_b in step_ev:
        e_a.record()
        fwd()
        e_b.record()
    torch.cuda.synchronize()
    step_list = sorted(a.elapsed_time(b) for a, b in step_ev)
    # Stage durations (HIP events on the launch stream around each kernel) from as many
    # steps again through the timed entry point.
    timer = api.Timer(args.steps)
    for _ in range(args.steps):
        fwd(timer)
    torch.cuda.synchronize()
    stage_ms, calls = timer.read()
    timer.close()
    ms_step = elapsed * 1e3 / args.steps
    stage_avg = {s: stage_ms[s] / calls for s in stage_ms}
    flops = algorithmic_flops(g)
    pairs = algorithmic_pairs(g)
    tflops = flops["total"] / (ms_step * 1e-3) / 1e12
    attn_hi_ms = stage_avg["attn_hi"]
    attn_ms = stage_avg["attn_hi"] + stage_avg["attn_lr"] + stage_avg["attn_text"]
    attn_tflops = flops["total"] / (attn_ms * 1e-3) / 1e12
    achieved = flops["hi"] / (attn_hi_ms * 1e-3) / 1e12
    log(f"[bench] {ms_step:.3f} ms/step; stages (ms/call): "
        + ", ".join(f"{s}={stage_avg[s]:.3f}" for s in stage_avg))

    # standalone permutation bandwidth (one of the four entry points), Q hi segment
    pdst = torch.empty((g.B, g.N, g.heads, g.head_dim), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        api.window_permute(qt, pdst, g.H, g.W, g.w, src_tokens_per_batch=g.L,
                           dst_tokens_per_batch=g.N)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        api.window_permute(qt, pdst, g.H, g.W, g.w, src_tokens_per_batch=g.L,
                           dst_tokens_per_batch=g.N)
    e1.record()
    torch.cuda.synchronize()
    perm_ms = e0.elapsed_time(e1) / reps
    perm_bytes = 2 * g.B * g.N * g.heads * g.head_dim * 2
    perm_gbs = perm_bytes / (perm_ms * 1e-3) / 1e9
    # a plain device-to-device copy of the same bytes, as a measured bandwidth ceiling
    psrc = torch.empty_like(pdst)
    for _ in range(3):
        pdst.copy_(psrc)
    e0.record()
    for _ in range(reps):
        pdst.copy_(psrc)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = perm_bytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    # uhla_copy_probe of the same bytes through each load path the kernels use: the
    # known-size copies the HBM traffic counters are calibrated against
    copy_paths = {}
    for mode, name in ((0, "plain"), (1, "nontemporal"), (2, "direct_to_lds")):
        api.copy_probe(psrc, pdst, mode)
        e0.record()
        for _ in range(3):
            api.copy_probe(psrc, pdst, mode)
        e1.record()
        torch.cuda.synchronize()
        copy_paths[name] = round(perm_bytes / (e0.elapsed_time(e1) / 3 * 1e-3) / 1e9, 1)
    del pdst, psrc

    traffic = None if variant else read_traffic()
    res = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        # per-step device time (HIP events around each step on the launch stream)
        "step_ms": {"median": round(float(np.median(step_list)), 4),
                    "min": round(step_list[0], 4), "max": round(step_list[-1], 4)},
        "config": {"workload": g.name, "B": g.B, "heads": g.heads, "head_dim": g.head_dim,
                   "grid": f"{g.H}x{g.W}", "window": g.w, "guide_grid": f"{g.H_lr}x{g.W_lr}",
                   "rho": g.rho, "rope_theta": g.theta, "tokens": g.L,
                   "neighbourhood_radius": g.radius, "guide_mode": g.guide_mode,
                   "text_tokens": g.T,
                   "k_rope": ("at every K tile load" if args.rope_at_load or args.permute_free
                              else "once, in the K prep pass"),
                   "kv_prep": "none: tiles copied from raster K, V" if args.permute_free
                              else "window-first K (rotated) and V^T tiles",
                   "parallelism": "single GPU"},
        "tokens_per_s": round(g.B * g.L / (ms_step * 1e-3), 1),
        "hi_tokens_per_s": round(g.B * g.N / (ms_step * 1e-3), 1),
        "algorithmic_flops": flops,
        "unmasked_pairs_per_head": pairs,
        "frac_bf16_peak_step": round(tflops / PEAK_BF16_TFLOPS, 4),
        # the same algorithmic FLOPs over the attention passes alone (hi, guide, text)
        "attention_passes": {"ms": round(attn_ms, 4), "TFLOP/s": round(attn_tflops, 2),
                             "frac_bf16_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4)},
        "stage_ms": {s: round(x, 4) for s, x in stage_avg.items()},
        "roofline": {"kernel": "attn_fwd_kernel<128, 8, hi%s> (hi-res pass)"
                               % (", raster tiles" if args.permute_free
                                  else ", K rotated at load" if args.rope_at_load else ""),
                     "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "permute": {"entry_point": "uhla_window_permute (Q hi segment, bf16)",
                    "ms": round(perm_ms, 4), "GB/s": round(perm_gbs, 1),
                    "frac_hbm_peak": round(perm_gbs / PEAK_HBM_GBS, 4),
                    "device_copy_GB/s": round(copy_gbs, 1),
                    "copy_probe_GB/s": copy_paths},
    }
    if not variant:
        # the forward's own permutes: K (rotated) and V (as V^T tiles) of every hi and guide
        # row read and written once, by prep_k_kernel and prep_v_kernel
        prep_ms = stage_avg["prep_hi"] + stage_avg["prep_lr"]
        prep_bytes = 2 * 2 * g.B * (g.N + g.H_lr * g.W_lr) * g.heads * g.head_dim * 2
        prep_gbs = prep_bytes / (prep_ms * 1e-3) / 1e9
        res["prep"] = {"kernels": "prep_k_kernel + prep_v_kernel", "ms": round(prep_ms, 4),
                       "algorithmic_bytes": prep_bytes, "GB/s": round(prep_gbs, 1),
                       "frac_hbm_peak": round(prep_gbs / PEAK_HBM_GBS, 4)}
    if not args.no_cpu_baseline:
        log(f"[bench] CPU baseline: oracle for ~{args.cpu_seconds:.0f} s")
        res["cpu_baseline"] = cpu_baseline(g, q, k, v, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
