"""Benchmark: one step of the spacetime-attention hot path at the Wan 480p shape.

One step, on synthetic seeded inputs already resident in HBM:
  1. patchify the block-input latent (1,16,21,60,104) bf16 with a 1x2x2
     Conv3d to [1, 32760, 1536] tokens (12 heads x 128);
  2. 3D RoPE [44,42,42] on those tokens (q = k);
  3. full 3D attention on independent N(0,1) Q/K/V [1, 32760, 12, 128];
  4. divided attention on the batch-2 (CFG pair) Q/K/V [2, 32760, 12, 128]:
     the spatial pass (504 frames of 1,560 tokens), then the temporal pass
     (37,440 sequences of 21 tokens).
`value` is the step's algorithmic attention FLOP (4*N^2*D per (b, head) for
full attention, its T*(HW)^2 and (HW)*T^2 parts for the two divided passes)
divided by the measured step time. Every pass is also reported on its own:
TFLOP/s against the bf16 matrix-core peak for the full and spatial passes,
GB/s against HBM for the temporal pass, RoPE and patchify.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
Prints one JSON line.
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

# MI355X published peaks (dense): bf16 matrix cores 2.5 PFLOP/s, which is
# 256 CUs x 2.4 GHz x 4,096 bf16 FLOP per CU per clock; HBM3E 8 TB/s.
PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12
PEAK_HBM_GBS = 8000.0
METRIC = "attention TFLOP/s + % bf16 MFMA peak (full/spatial), temporal GB/s + % HBM"


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the oracle timing (profiling runs)")
    p.add_argument("--no-720p", action="store_true",
                   help="skip the full-attention timing at the 14B-shaped 720p size [1,75600,40,128]")
    p.add_argument("--copy-probe", action="store_true",
                   help="run one plain 1 GiB device copy first (HBM counter calibration)")
    return p.parse_args()


def _dev(d):
    import torch
    return torch.from_numpy(np.ascontiguousarray(d.bits).view(np.int16)).view(torch.bfloat16).cuda()


def _source_hash(names: str) -> str:
    """sha256 (16 hex digits) of the "+"-joined kernel sources, concatenated."""
    h = hashlib.sha256()
    for name in names.split("+"):
        h.update(open(os.path.join(ROOT, "spacetime_attention_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def _traffic(kernel_file: str, per_launch_key: str):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs, if they were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(per_launch_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != _source_hash(kernel_file):
        return None
    return rec.get("bytes_per_launch")


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import spacetime_attention_amd as vd
    from synthetic_inputs import WORKLOADS

    torch.cuda.set_device(0)
    vd.load_library()

    wf, wd, wb = WORKLOADS["480p_full"], WORKLOADS["480p_divided"], WORKLOADS["block_input"]
    grid = (wf.T, wf.Hp, wf.Wp)
    HW = wf.Hp * wf.Wp
    D, H = wf.head_dim, wf.heads

    t0 = time.time()
    df = wf.draw_qkv()
    qf, kf, vf = (_dev(df[n]) for n in ("q", "k", "v"))
    dd = wd.draw_qkv()
    qd, kd, vd_ = (_dev(dd[n]) for n in ("q", "k", "v"))
    dl = wb.draw_latent()
    lat, wgt = _dev(dl["x"]), _dev(dl["w"])
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    tok = torch.empty((1, wb.N, wb.dim), dtype=torch.bfloat16, device="cuda")
    rot = torch.empty((1, wb.N, wb.heads, wb.head_dim), dtype=torch.bfloat16, device="cuda")
    of = torch.empty_like(qf)
    os_ = torch.empty_like(qd)
    ot = torch.empty_like(qd)

    if args.copy_probe:
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    passes = ["patchify", "rope", "full", "spatial", "temporal"]
    ev = {p: [] for p in passes}

    def step(record: bool):
        def run(name, fn):
            if record:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                ev[name].append((a, b))
            else:
                fn()
        run("patchify", lambda: vd.patchify(lat, wgt, heads=wb.heads, head_dim=wb.head_dim, out=tok))
        run("rope", lambda: vd.rope3d(tok.view(1, wb.N, wb.heads, wb.head_dim), grid, wb.rope_split,
                                      out=rot))
        run("full", lambda: vd.attn_full(qf, kf, vf, grid, out=of))
        run("spatial", lambda: vd.attn_spatial(qd, kd, vd_, grid, out=os_))
        run("temporal", lambda: vd.attn_temporal(qd, kd, vd_, grid, out=ot))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    # Timed region: K steps between two synchronisations. Per-launch events
    # are recorded on the same stream the library launches on.
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_step = elapsed * 1e3 / args.steps

    def avg_ms(name):
        return float(np.mean([a.elapsed_time(b) for a, b in ev[name]]))

    def spread(name):
        xs = [a.elapsed_time(b) for a, b in ev[name]]
        return {"ms_median": float(np.median(xs)), "ms_min": float(np.min(xs))}

    f_full = 4.0 * wf.B * H * wf.N * wf.N * D
    f_spatial = 4.0 * wd.B * H * wd.T * HW * HW * D
    f_temporal = 4.0 * wd.B * H * HW * wd.T * wd.T * D
    b_temporal = 4.0 * wd.B * wd.N * H * D * 2            # read Q, K, V, write O, bf16
    b_rope = 2.0 * wb.N * wb.dim * 2                       # read and write one tensor
    b_patch = (np.prod(wb.latent_shape) + np.prod(wb.weight_shape) + wb.N * wb.dim) * 2.0
    f_patch = 2.0 * wb.N * wb.dim * np.prod(wb.weight_shape[1:])
    attn_flop = f_full + f_spatial + f_temporal

    t = {p: avg_ms(p) for p in passes}
    per_pass = {
        "full": {"ms": t["full"], "tflops": f_full / t["full"] / 1e9,
                 "frac_bf16_peak": f_full / t["full"] / 1e9 / PEAK_BF16_TFLOPS,
                 "tokens_per_s": wf.B * wf.N / t["full"] * 1e3},
        "spatial": {"ms": t["spatial"], "tflops": f_spatial / t["spatial"] / 1e9,
                    "frac_bf16_peak": f_spatial / t["spatial"] / 1e9 / PEAK_BF16_TFLOPS,
                    "tokens_per_s": wd.B * wd.N / t["spatial"] * 1e3},
        "temporal": {"ms": t["temporal"], "gbs": b_temporal / t["temporal"] / 1e6,
                     "frac_hbm_peak": b_temporal / t["temporal"] / 1e6 / PEAK_HBM_GBS,
                     "tflops": f_temporal / t["temporal"] / 1e9,
                     "tokens_per_s": wd.B * wd.N / t["temporal"] * 1e3},
        "rope": {"ms": t["rope"], "gbs": b_rope / t["rope"] / 1e6,
                 "frac_hbm_peak": b_rope / t["rope"] / 1e6 / PEAK_HBM_GBS},
        "patchify": {"ms": t["patchify"], "gbs": b_patch / t["patchify"] / 1e6,
                     "frac_hbm_peak": b_patch / t["patchify"] / 1e6 / PEAK_HBM_GBS,
                     "tflops": f_patch / t["patchify"] / 1e9},
    }
    for p in passes:
        per_pass[p].update(spread(p))

    achieved = f_full / t["full"] / 1e9
    roofline = {"kernel": "flash_fwd_bf16<128,1,8,0> (vdit_attn_full, 480p)", "bound": "mfma",
                "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": _traffic("attn_flash_kernel.h+attn_flash_full.hip", "flash_full_480p")}

    result = {
        "metric": METRIC,
        "value": attn_flop / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "wan480p_attention_layer: patchify+RoPE of latent (1,16,21,60,104) -> "
                        "[1,32760,1536]; full attention [1,32760,12,128]; divided spatial+temporal "
                        "[2,32760,12,128]",
            "grid": list(grid), "heads": H, "head_dim": D, "seq_len": wf.N,
            "batch_full": wf.B, "batch_divided": wd.B, "parallelism": "single GPU",
        },
        "passes": per_pass,
        "roofline": roofline,
        "cpu_baseline": None,
    }

    result["temporal_alone"] = bench_temporal_alone(vd, torch, qd, kd, vd_, ot, grid, b_temporal)
    result["patchify_alone"] = bench_patchify_alone(vd, torch, lat, wgt, tok, wb, b_patch)
    # Six cold [1,32760,12,128] inputs: the two batch halves of the divided Q, K and V.
    rope_srcs = [t[i:i + 1] for t in (qd, kd, vd_) for i in range(2)]
    result["rope_alone"] = bench_rope_alone(vd, torch, rope_srcs, rot, grid, wb.rope_split, b_rope)
    result["next_rows"] = {"cross": bench_cross(vd, torch), "window": bench_window(vd, torch),
                           "qkv_proj": bench_qkv(vd, torch),
                           "rope_in_attention": bench_rope_in_attention(vd, torch, qf, kf, vf, of, qd, kd, vd_,
                                                                        os_, ot, grid, f_full, f_spatial,
                                                                        b_temporal)}
    if not args.no_720p:
        result["full_720p"] = bench_full_720p(vd, torch)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(df, wf)
        result["cpu_baseline"]["gpu_over_cpu"] = per_pass["full"]["tflops"] / result["cpu_baseline"]["value"]
    print(json.dumps(result), flush=True)


def _warm(torch, fn, min_ms: float = 100.0, at_least: int = 3):
    """Launch fn until at least min_ms of device time has passed (and at least
    `at_least` times). The passes timed on their own after the step follow
    host-side input generation, during which the device idles and its clock
    drops; the clock takes a few tens of milliseconds of load to come back."""
    import time
    t0 = time.perf_counter()
    n = 0
    while n < at_least or (time.perf_counter() - t0) * 1e3 < min_ms:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def bench_temporal_alone(vd, torch, q, k, v, o, grid, nbytes, iters: int = 20):
    """The temporal pass repeated on its own over the step's batch-2 tensors.
    Inside the step it follows the spatial pass on the same Q/K/V, so part of
    its reads can come from the 256 MB Infinity Cache; alone, its 805 MB
    working set cycles through that cache with little reuse."""
    _warm(torch, lambda: vd.attn_temporal(q, k, v, grid, out=o))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        vd.attn_temporal(q, k, v, grid, out=o)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / iters
    return {"ms": ms, "gbs": nbytes / ms / 1e6, "frac_hbm_peak": nbytes / ms / 1e6 / PEAK_HBM_GBS}


def bench_patchify_alone(vd, torch, lat, wgt, tok, wb, nbytes, iters: int = 20):
    """Patchify launched back to back on the step's latent and weight. The
    step's per-pass figure brackets a single ~20 us launch with a pair of
    events, which adds their processing and the dispatch of the launch
    (a few us) to the kernel's own time; here 20 launches run between one
    pair of events, so each carries only the gap between consecutive
    kernels. The 4 MB latent stays cached across launches; the bytes are
    dominated by the 100.6 MB of tokens written."""
    fn = lambda: vd.patchify(lat, wgt, heads=wb.heads, head_dim=wb.head_dim, out=tok)
    _warm(torch, fn)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        fn()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / iters
    return {"ms": ms, "gbs": nbytes / ms / 1e6, "frac_hbm_peak": nbytes / ms / 1e6 / PEAK_HBM_GBS}


def bench_rope_alone(vd, torch, srcs, out, grid, split, nbytes, iters: int = 24):
    """3D RoPE launched back to back, like patchify_alone, so each launch
    carries only the gap between kernels instead of an event pair. The
    launches cycle over six distinct 100.6 MB inputs (600 MB, more than the
    256 MB Infinity Cache), so every launch reads its input from HBM."""
    k = [0]

    def fn():
        vd.rope3d(srcs[k[0] % len(srcs)], grid, split, out=out)
        k[0] += 1

    _warm(torch, fn)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        fn()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / iters
    return {"ms": ms, "gbs": nbytes / ms / 1e6, "frac_hbm_peak": nbytes / ms / 1e6 / PEAK_HBM_GBS}


def bench_cross(vd, torch, iters: int = 20):
    """Cross-attention (the block's attn2), timed on its own after the step:
    32,760 video queries x 512 text keys, 12 heads x 128, bf16."""
    from synthetic_inputs import CROSS_WORKLOADS
    w = CROSS_WORKLOADS["cross_480p"]
    d = w.draw()
    q, k, v = (_dev(d[n]) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    _warm(torch, lambda: vd.attn_cross(q, k, v, out=o))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        vd.attn_cross(q, k, v, out=o)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / iters
    flop = 4.0 * w.B * w.heads * w.Nq * w.Nk * w.head_dim
    return {"workload": f"q [{w.B},{w.Nq},{w.heads},{w.head_dim}] x k/v [{w.B},{w.Nk},{w.heads},{w.head_dim}]",
            "ms": ms, "tflops": flop / ms / 1e9, "frac_bf16_peak": flop / ms / 1e9 / PEAK_BF16_TFLOPS}


def bench_full_720p(vd, torch, iters: int = 5):
    """Full attention at the 14B-shaped 720p size, timed on its own after the
    step: [1,75600,40,128] bf16 Q/K/V drawn N(0,1) on the device from a fixed
    seed (the sampled parity test covers the same shape with the host draw)."""
    from synthetic_inputs import WORKLOADS
    w = WORKLOADS["720p_full"]
    grid = (w.T, w.Hp, w.Wp)
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed)
    shape = (w.B, w.N, w.heads, w.head_dim)
    q, k, v = (torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
               for _ in range(3))
    o = torch.empty_like(q)
    _warm(torch, lambda: vd.attn_full(q, k, v, grid, out=o), at_least=2)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        vd.attn_full(q, k, v, grid, out=o)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / iters
    flop = 4.0 * w.B * w.heads * float(w.N) ** 2 * w.head_dim
    del q, k, v, o
    return {"workload": f"[{w.B},{w.N},{w.heads},{w.head_dim}] grid {grid}", "ms": ms,
            "tflops": flop / ms / 1e9, "frac_bf16_peak": flop / ms / 1e9 / PEAK_BF16_TFLOPS,
            "tokens_per_s": w.B * w.N / (ms * 1e-3)}


def window_flop(w, window) -> float:
    """4*|window|^2*head_dim FLOP per window and head, over the clipped windows."""
    total = 0
    for ext, win in zip((w.T, w.Hp, w.Wp), window):
        sizes = [min(win, ext - s) for s in range(0, ext, win)]
        total = sizes if total == 0 else [a * b for a in total for b in sizes]
    return 4.0 * w.B * w.heads * w.head_dim * float(sum(n * n for n in total))


def bench_window(vd, torch, iters: int = 20):
    """Windowed attention, timed on its own after the step: the 480p grid cut
    into 3 x 15 x 26 windows (28 windows of 1,170 tokens), 12 heads x 128."""
    from synthetic_inputs import WORKLOADS
    w = WORKLOADS["480p_window"]
    grid = (w.T, w.Hp, w.Wp)
    d = w.draw_qkv()
    q, k, v = (_dev(d[n]) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    _warm(torch, lambda: vd.attn_window(q, k, v, grid, w.window, out=o))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        vd.attn_window(q, k, v, grid, w.window, out=o)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / iters
    flop = window_flop(w, w.window)
    return {"workload": f"[{w.B},{w.N},{w.heads},{w.head_dim}] grid {grid} windows {w.window}",
            "ms": ms, "tflops": flop / ms / 1e9, "frac_bf16_peak": flop / ms / 1e9 / PEAK_BF16_TFLOPS}


def bench_rope_in_attention(vd, torch, qf, kf, vf, of, qd, kd, vd_, od, ot, grid, f_full, f_spatial, b_temporal,
                            rounds: int = 3, iters: int = 10):
    """RoPE applied inside the attention kernel against the separate RoPE
    pass on Q and on K followed by the plain kernel, on the step's full
    (batch 1) and divided (batch 2) inputs, timed on their own after the
    step in alternating blocks of `iters` launches so that both see the same
    clock. The FLOP rates count only the attention product; the temporal
    rate is its algorithmic bytes (Q, K, V read and O written once)."""
    split = (44, 42, 42)

    def sep(q, k, v, o, attn):
        qr, kr = torch.empty_like(q), torch.empty_like(k)

        def run():
            vd.rope3d(q, grid, split, out=qr)
            vd.rope3d(k, grid, split, out=kr)
            attn(qr, kr, v, grid, out=o)
        return run

    out = {}
    for name, q, k, v, o, plain, fused, flop in (
            ("full", qf, kf, vf, of, vd.attn_full, vd.attn_full_rope, f_full),
            ("spatial", qd, kd, vd_, od, vd.attn_spatial, vd.attn_spatial_rope, f_spatial),
            ("temporal", qd, kd, vd_, ot, vd.attn_temporal, vd.attn_temporal_rope, None)):
        runs = {"fused": lambda: fused(q, k, v, grid, split, out=o), "separate": sep(q, k, v, o, plain)}
        ms = {key: [] for key in runs}
        for key, fn in runs.items():
            _warm(torch, fn)
        for _ in range(rounds):
            for key, fn in runs.items():
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(iters):
                    fn()
                b.record()
                torch.cuda.synchronize()
                ms[key].append(a.elapsed_time(b) / iters)
        med = {key: float(np.median(v_)) for key, v_ in ms.items()}
        out[name] = {"fused_ms": med["fused"], "separate_ms": med["separate"],
                     "fused_over_separate": med["fused"] / med["separate"]}
        if flop is not None:
            out[name]["fused_tflops"] = flop / med["fused"] / 1e9
        else:
            out[name]["fused_gbs"] = b_temporal / med["fused"] / 1e6
        del runs
    out["workload"] = f"480p grid {grid}, 12 heads x 128, split {split}: full [1,32760,12,128], " \
                      f"spatial and temporal [2,32760,12,128]; separate = vdit_rope3d on q and on k, " \
                      f"then the plain pass"
    return out


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bench_qkv(vd, torch, iters: int = 20):
    """The projection in front of self-attention, timed on its own after the
    step: [1,32760,1536] tokens x fused [4608,1536] weight with bias, per-head
    RMSNorm and RoPE [44,42,42] on Q and K."""
    from synthetic_inputs import QKV_WORKLOADS
    w = QKV_WORKLOADS["qkv_480p"]
    d = w.draw()
    x, wt, b, gq, gk = (_dev(d[n]) for n in ("x", "w", "bias", "gq", "gk"))
    grid = (w.T, w.Hp, w.Wp)
    shape = (w.B, w.N, w.heads, w.head_dim)
    out = tuple(torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in range(3))

    def run():
        vd.qkv_proj(x, wt, b, gq, gk, grid=grid, heads=w.heads, head_dim=w.head_dim, split=w.rope_split, out=out)

    _warm(torch, run)
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        run()
    e.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(e) / iters
    flop = 2.0 * w.B * w.N * 3 * w.dim * w.dim
    return {"workload": f"x [{w.B},{w.N},{w.dim}] x w [{3 * w.dim},{w.dim}], RMSNorm + RoPE on Q/K",
            "ms": ms, "tflops": flop / ms / 1e9, "frac_bf16_peak": flop / ms / 1e9 / PEAK_BF16_TFLOPS}


def cpu_baseline(df, wf):
    """The fp64 oracle, untuned, on a bounded sample of the same workload:
    full attention at 480p for every 32nd query token (plus the last) of
    all 12 heads. Each sampled row costs exactly 4*N*head_dim FLOP."""
    import oracle
    from synthetic_inputs import sample_rows

    grid = (wf.T, wf.Hp, wf.Wp)
    rows = sample_rows(wf.N, 32)
    q, k, v = df["q"].f32, df["k"].f32, df["v"].f32
    t0 = time.perf_counter()
    oracle.attention(q, k, v, grid, "full", rows=rows)
    dt = time.perf_counter() - t0
    flop = 4.0 * wf.B * wf.heads * rows.size * wf.N * wf.head_dim
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": dt, "cpu_model": _cpu_model(),
            "sample": f"full attention 480p [1,32760,12,128], {rows.size} query rows "
                      f"(every 32nd token) x 12 heads, fp64 C oracle"}


if __name__ == "__main__":
    main()
