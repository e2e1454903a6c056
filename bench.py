"""Benchmark: projected tokens/s of the fused pixel-aligned conditioning path
on one MI355X, with the roofline of its dominant kernel and the CPU oracle
timed beside it.

One step = one pass of the whole path over the batch: the image-space token
order (p3d_token_order), then the fused kernel through it
(p3d_proj_cond_ordered) -- projection of every token, bilinear gather,
proj_linear on the matrix cores, mask, and the CFG null branch. Together the
two calls are p3d_proj_cond_ws; they are issued separately so that HIP events
bracket the fused kernel alone. The default workload is the largest one (a
1024^3 sparse shell of 100k tokens with a 100k-row null branch, bf16 map
1x512x512x2048, proj_linear 2048->1536); inputs are synthetic, seeded and
resident in HBM before the timed region starts.

Prints ONE JSON line. Fields beyond the common ones:
  roofline          dominant kernel (the fused gather+MFMA kernel, launched
                    once per step, null rows included): algorithmic flops per
                    launch / its mean duration (HIP events on the launch
                    stream around each launch of the timed steps) against the
                    bf16 dense MFMA peak; traffic = HBM bytes per launch from
                    the committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs, scaled
                    by a copy kernel of known size, or null if the sources
                    changed since.
  order_ms          the token order's share of the step (events likewise).
  cpu_baseline      the CPU oracle on a bounded prefix of the same tokens, on
                    every core of the affinity mask and on one thread.
  gather            the standalone bilinear gather on the same points, in
                    the step's token order when the step has one:
                    algorithmic bytes / duration against peak HBM bandwidth
                    and against the measured copy ceiling.
  hbm_copy_ceiling  a streaming device copy (p3d_stream_copy, 16-byte
                    non-temporal loads and stores): the achievable read plus
                    write HBM rate; the runtime's own copy beside it.
  null_fill         the null-branch fill alone: bytes written / duration.
  extra             the adjacent parts, each with its own roofline: the fused
                    call on every other workload (fp32 peak for fp32, bf16
                    for bf16), the headline without the order, cascade
                    requantization (HBM) and the fused kernel on grid nodes
                    (MFMA), the two-map texture stage (fused kernel, the
                    projection diagnostics and the gather-once samples, all
                    through one shared order, plus the per-block proj_linear
                    of 30 DiT blocks), and a plain GEMM reference.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
F32_PEAK_TFLOPS = 157.3        # MI355X fp32 MFMA, TFLOP/s
DEFAULT_WORKLOAD = "shell1024_cfg_bf16_c2048_d1536"
PROFILE_DIR = os.path.join(ROOT, "profiles")


# source files each measured kernel is built from, or that decide what it
# reads (the token order); its counters stay valid while these are unchanged
KERNEL_SOURCES = {
    "proj_cond_bf16_kernel": ["proj_cond_bf16.hip", "bf16_tile.h", "p3d_internal.h",
                              "order.hip"],
    "proj_cond_kernel": ["proj_cond.hip", "p3d_internal.h"],
    "sample_kernel": ["sample.hip", "p3d_internal.h", "order.hip"],
    "stats_kernel": ["stats.hip", "p3d_internal.h", "order.hip"],
}


def kernel_source_digest(kernel=None):
    """sha256 over the sources of `kernel` (all HIP sources of libp3d when
    None) and include/p3d.h: counters taken on one build are reused only
    while this matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "pixel_aligned_image_amd", "csrc")
    names = KERNEL_SOURCES.get(kernel) or sorted(
        f for f in os.listdir(csrc) if f.endswith((".hip", ".h")))
    for name in sorted(names):
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
    h.update(open(os.path.join(ROOT, "include", "p3d.h"), "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from profiles/, if the
    sources still match the digest recorded there."""
    path = os.path.join(PROFILE_DIR, "%s_%s_hbm_traffic.md" % (kernel, workload))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_digest = re.search(r"source_digest:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_digest and m_bytes) or m_digest.group(1) != kernel_source_digest(kernel):
        return None
    return float(m_bytes.group(1))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def unique_corner_rows(pixel, bidx, H, W):
    """Distinct map rows among the four corners of every point (what the
    gather must fetch at least once)."""
    import numpy as np
    x0 = pixel[:, 0].astype(np.int64)
    y0 = pixel[:, 1].astype(np.int64)
    x1 = np.minimum(x0 + 1, W - 1)
    y1 = np.minimum(y0 + 1, H - 1)
    b = bidx.astype(np.int64)
    rows = np.concatenate([(b * H + y) * W + x for y in (y0, y1) for x in (x0, x1)])
    return int(np.unique(rows).size)


def bf16_kernel_name(p3d, two_maps, n, D):
    """The fused bf16 kernel instantiation a launch of n tokens and D features
    runs, from the library's own tiling rule (p3d_proj_cond_plan): the round
    kernel for one round of 96-token tiles, else the kernel whose last
    template argument is its tail part size in 16-token blocks (4 for
    64-token parts, else 2)."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = p3d.p3d_proj_cond_plan(n, D, cus)
    two = "true" if two_maps else "false"
    if plan["tile_rows"] != 128:
        return "proj_cond_bf16_round_kernel<%s, true>" % two
    return "proj_cond_bf16_kernel<%s, true, %d>" % (two, 4 if plan["part_rows"] == 64 else 2)


def time_events(fn, reps, stream, lead=None):
    """Mean duration (ms) of fn() over reps launches, HIP events on stream.
    lead(), enqueued first and not timed, keeps the GPU busy while the host
    queues launches that are shorter than their own host-side call."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    if lead is not None:
        lead()
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def cpu_quota_cores():
    """CPU share the cgroup grants (cpu.max quota / period), or None."""
    try:
        q, per = open("/sys/fs/cgroup/cpu.max").read().split()
        return None if q == "max" else float(q) / float(per)
    except (OSError, ValueError):
        return None


def cpu_leg(o, inp, cams_o, threads, target_s):
    """The oracle over a prefix of the tokens on `threads` threads until about
    target_s seconds of CPU work: (tokens done, seconds, threads used)."""
    import numpy as np
    used = o.set_threads(threads)
    w = inp["w"]
    fo, do = cams_o
    done, t_total, chunk = 0, 0.0, max(64, 32 * used)
    while t_total < target_s and done < inp["n"]:
        rows = np.arange(done, min(inp["n"], done + chunk))
        t0 = time.perf_counter()
        o.proj_cond_rows(inp["coords"], inp["n"], w.resolution, fo, do, inp["feat"],
                         inp["weight"], inp["bias"], inp["n_null"], rows)
        t_total += time.perf_counter() - t0
        done += rows.size
        rate = rows.size / max(time.perf_counter() - t0, 1e-6)
        chunk = int(max(64, min(16384, rate * max(target_s - t_total, 0.0) * 0.5)))
    return done, t_total, used


def cpu_baseline(inp, cams_o, target_s=10.0):
    """The oracle, untuned, on a bounded prefix of the same tokens: one leg
    on every core this process may run on, one on a single thread; tokens/s
    is the rate over the prefix, and a full pass is extrapolated from it."""
    import oracle
    o = oracle.get()
    cores = len(os.sched_getaffinity(0))
    many = min(cores, 256)          # a sanity bound on threads, not a tuning
    d_all, t_all, used = cpu_leg(o, inp, cams_o, many, target_s)
    d_one, t_one, _ = cpu_leg(o, inp, cams_o, 1, target_s)
    quota = cpu_quota_cores()
    what = ("the full path per token: projection, gather, bf16 rounding, proj_linear in "
            "binary64 (rows of the oracle's proj_cond)")
    return {"value": d_all / t_all, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": "first %d of %d tokens of the same workload, %s, %.1f s on %d threads; "
                      "CPU %s, %d cores in the affinity mask%s" % (
                          d_all, inp["n"], what, t_all, used, cpu_model(), cores,
                          "" if quota is None else ", cgroup CPU quota %.1f cores" % quota),
            "extrapolated_full_pass_s": inp["n"] / (d_all / t_all),
            "single_thread": {"value": d_one / t_one, "unit": "tokens/s", "cores": 1,
                              "sample": "first %d tokens, %.1f s on 1 thread" % (d_one, t_one),
                              "extrapolated_full_pass_s": inp["n"] / (d_one / t_one)},
            "affinity_cores": cores, "cpu_quota_cores": quota, "cpu_model": cpu_model()}


def hbm_copy_ceiling(p3d, stream, reps, mib=2048):
    """The achievable HBM rate beside the datasheet peak: a streaming device
    copy of mib MiB (p3d_stream_copy: 16-byte non-temporal loads and stores),
    GB/s counted as bytes read plus bytes written per launch over its mean
    duration; the HIP runtime's own device-to-device copy (torch copy_) is
    reported beside it."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    sc = lambda: p3d.p3d_stream_copy(a, b)
    rt = lambda: b.copy_(a)
    for f in (sc, rt):
        for _ in range(3):
            f()
    ms = time_events(sc, reps, stream)
    ms_rt = time_events(rt, reps, stream)
    gbs = 2.0 * n * 4 / (ms * 1e-3) / 1e9
    gbs_rt = 2.0 * n * 4 / (ms_rt * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return {"kernel": "p3d_stream_copy (16-byte non-temporal loads and stores)",
            "bytes_per_launch": 2 * n * 4, "mean_ms": ms, "achieved": gbs, "unit": "GB/s",
            "frac_of_peak": gbs / HBM_PEAK_GBS,
            "runtime_copy": {"kernel": "torch copy_ (the HIP runtime's device-to-device copy)",
                             "mean_ms": ms_rt, "achieved": gbs_rt}}


def order_key(maps):
    """(H, W) of the map with the most texels: the key map of the order."""
    return max(((m.shape[1], m.shape[2]) for m in maps), key=lambda hw: hw[0] * hw[1])


def make_order(p3d, coords, n, R, cams, maps, points="cell_centres"):
    """Device order of the tokens and a closure that recomputes it."""
    import torch
    kH, kW = order_key(maps)
    order = torch.empty((n,), dtype=torch.int32, device="cuda")
    ws = torch.empty((p3d.p3d_token_order_workspace_size(n, len(cams), kH, kW),),
                     dtype=torch.uint8, device="cuda")
    run = lambda: p3d.p3d_token_order(coords, n, R, cams, kH, kW, order, workspace=ws,
                                      points=points)
    run()
    return order, run


def config_line(p3d, synth, name, stream, reps):
    """One workload's fused call, timed alone (HIP events), with its own
    roofline: fp32 MFMA peak for fp32 workloads, bf16 for bf16 ones. bf16
    workloads also report the ordered call (token order + fused kernel)."""
    import numpy as np
    import torch
    w = synth.workload(name)
    bf16 = w.dtype == "bf16"

    def dev(a):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.int16).view(torch.bfloat16) if bf16 and a.dtype == np.uint16
                else t).cuda()

    coords_np = synth.coords(w)
    coords = dev(coords_np)
    feat = dev(synth.feature_map(w))
    weight = dev(synth.weight(w))
    bias = dev(synth.bias(w))
    n, nn = w.n_tokens, w.n_null
    cams = [p3d.p3d_make_camera(a, w.distance if w.distance is not None else
                                p3d.p3d_distance_from_fov(a, w.width, 0)) for a in synth.fovs(w)]
    camarr = p3d.make_cameras(cams)
    out = torch.empty((n + nn, w.out_dim), dtype=feat.dtype, device="cuda")
    mask = torch.empty((n,), dtype=torch.uint8, device="cuda")
    fused = lambda: p3d.p3d_proj_cond(coords, n, w.resolution, camarr, feat, weight, out,
                                      bias=bias, n_null=nn, mask=mask)
    for _ in range(reps):
        fused()
    ms = time_events(fused, reps, stream)
    flops = 2.0 * n * w.channels * w.out_dim
    peak = BF16_PEAK_TFLOPS if bf16 else F32_PEAK_TFLOPS
    line = {"workload": w.name, "dtype": w.dtype, "tokens": n, "null_rows": nn,
            "map": "%dx%dx%dx%d" % tuple(feat.shape),
            "proj_linear": "%d->%d%s" % (w.channels, w.out_dim, " +bias" if bias is not None
                                         else ""),
            "kernel": bf16_kernel_name(p3d, False, n, w.out_dim) if bf16 else "proj_cond_kernel",
            "mean_ms": ms, "tokens_per_s": n / (ms * 1e-3), "bound": "mfma",
            "flops_per_launch": flops, "achieved": flops / (ms * 1e-3) / 1e12, "peak": peak,
            "unit": "TFLOP/s", "frac": flops / (ms * 1e-3) / 1e12 / peak}
    if bf16:
        line["tiling"] = p3d.p3d_proj_cond_plan(
            n, w.out_dim, torch.cuda.get_device_properties(0).multi_processor_count)
    if bf16 and coords is not None:
        order, run_order = make_order(p3d, coords, n, w.resolution, camarr, [feat], w.points)
        ordf = lambda: p3d.p3d_proj_cond(coords, n, w.resolution, camarr, feat, weight, out,
                                         bias=bias, n_null=nn, mask=mask, order=order)
        for _ in range(reps):
            ordf()
        oms = time_events(ordf, reps, stream)
        sort_ms = time_events(run_order, reps, stream)
        line["ordered"] = {"fused_ms": oms, "order_ms": sort_ms,
                           "frac": flops / (oms * 1e-3) / 1e12 / peak,
                           "tokens_per_s_incl_order": n / ((oms + sort_ms) * 1e-3)}
    del coords, feat, weight, bias, out, mask
    torch.cuda.empty_cache()
    return line


def channel_sweep(p3d, synth, stream, reps):
    """The 1024^3 shell's tokens (in the token order, no null rows) through
    the fused kernel on seeded 512 x 512 maps of 512 .. 2048 channels, D =
    1536; the least-squares line through the mean durations gives the
    launch's fixed cost and its time per 64-channel K chunk, and the MFMA
    rate of that steady state."""
    import numpy as np
    import torch
    w = synth.workload(DEFAULT_WORKLOAD)
    coords = torch.from_numpy(synth.coords(w)).cuda()
    n, D = w.n_tokens, w.out_dim
    cams = p3d.make_cameras([p3d.p3d_make_camera(a, p3d.p3d_distance_from_fov(a, w.width, 0))
                             for a in synth.fovs(w)])
    g = torch.Generator(device="cuda").manual_seed(1234)
    order = None
    chans, ms = [], []
    out = torch.empty((n, D), dtype=torch.bfloat16, device="cuda")
    for C in (512, 1024, 1536, 2048):
        feat = torch.randn((1, w.height, w.width, C), device="cuda", generator=g).to(torch.bfloat16)
        weight = (torch.randn((D, C), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        if order is None:
            order, _ = make_order(p3d, coords, n, w.resolution, cams, [feat], w.points)
        f = lambda: p3d.p3d_proj_cond(coords, n, w.resolution, cams, feat, weight, out,
                                      order=order)
        for _ in range(reps):
            f()
        chans.append(C)
        ms.append(time_events(f, reps, stream))
        del feat, weight
    slope, icpt = np.polyfit(np.array(chans, float), np.array(ms), 1)
    chunk_flops = 2.0 * n * 64 * D
    torch.cuda.empty_cache()
    return {"workload": w.name + " tokens, no null rows, seeded maps 512x512xC, D 1536",
            "channels": chans, "mean_ms": ms, "fixed_ms": float(icpt),
            "ms_per_k_chunk": float(slope * 64),
            "steady_state_frac": chunk_flops / (slope * 64 * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "fixed_share_at_2048": float(icpt / ms[-1])}


EXTRAS = ("configs", "variants", "channel_sweep", "cascade", "two_maps", "gemm_reference")


def run_extra(p3d, synth, stream, reps, lead_step, which, unordered_step=None,
              headline_flops=None, caller_order_gather=None):
    """Adjacent parts on their own workloads (the names in `which`):
      configs        the fused call on every other workload, own roofline;
      variants       the headline's fused kernel and its standalone gather
                     without the token order (the caller's order);
      channel_sweep  the headline's fused kernel (token order, no null rows)
                     on maps of 512 .. 2048 channels: a line through the
                     means splits the launch into a fixed cost (tile starts
                     and ends) and a rate per K chunk;
      cascade        requantization of a res-512 shell onto the 64-node grid,
                     and the fused kernel on those grid nodes;
      two_maps       the fused kernel over two concatenated maps, the
                     projection diagnostics and the gather-once samples over
                     those maps (all sharing one token order), the per-block
                     linears of 30 DiT blocks;
      gemm_reference one block of the plain product through the tile and
                     through a library GEMM."""
    import numpy as np
    import torch

    def dev(a, as_bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.int16).view(torch.bfloat16) if as_bf16 else t).cuda()

    def lead():
        for _ in range(2):
            lead_step()

    out = {}
    if "variants" in which and unordered_step is not None:
        for _ in range(reps):
            unordered_step()
        ums = time_events(unordered_step, reps, stream)
        out["unordered_fused"] = {
            "kernel": "proj_cond_bf16_kernel", "mean_ms": ums,
            "frac": headline_flops / (ums * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "note": "the headline's fused call without the token order (p3d_proj_cond): "
                    "tokens in the caller's (x, y, z) order"}
        if caller_order_gather is not None:
            g, gbytes = caller_order_gather
            for _ in range(reps):
                g()
            gms = time_events(g, reps, stream)
            out["caller_order_gather"] = {
                "kernel": "sample_kernel", "mean_ms": gms,
                "frac": gbytes / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "note": "the standalone gather at the same points in the caller's (x, y, z) "
                        "order (p3d_bilinear_sample)"}
    if "configs" in which:
        out["configs"] = [config_line(p3d, synth, w.name, stream, reps)
                          for w in synth.WORKLOADS if w.name != DEFAULT_WORKLOAD]
    if "channel_sweep" in which:
        out["channel_sweep"] = channel_sweep(p3d, synth, stream, reps)
    if "cascade" in which:
        w = synth.workload("cascade512_grid64_nodes_bf16_c2048_d1536")
        src = dev(synth.coords(w))
        n = src.shape[0]
        q = torch.empty_like(src)
        rq = lambda: p3d.p3d_requantize_coords(src, w.coords_resolution, w.resolution, q)
        rq()
        rq_ms = time_events(rq, reps, stream, lead)
        rq_bytes = 32 * n
        feat = dev(synth.feature_map(w), True)
        weight = dev(synth.weight(w), True)
        cams = [p3d.p3d_make_camera(a, p3d.p3d_distance_from_fov(a, w.width, 0))
                for a in synth.fovs(w)]
        camarr = p3d.make_cameras(cams)
        y = torch.empty((n, w.out_dim), dtype=torch.bfloat16, device="cuda")
        fused = lambda: p3d.p3d_proj_cond(q, n, w.resolution, camarr, feat, weight, y,
                                          points="grid_nodes")
        for _ in range(reps):
            fused()
        nodes_ms = time_events(fused, reps, stream)
        flops = 2.0 * n * w.k_total * w.out_dim
        out["requantize"] = {
            "workload": w.name, "kernel": "requant_kernel", "tokens": n, "mean_ms": rq_ms,
            "bound": "hbm", "bytes_per_launch": rq_bytes,
            "achieved": rq_bytes / (rq_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": rq_bytes / (rq_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "note": "100k tokens = 3.2 MB: launch-latency bound, far from the HBM roofline"}
        out["grid_nodes"] = {
            "workload": w.name, "kernel": bf16_kernel_name(p3d, False, n, w.out_dim), "tokens": n,
            "mean_ms": nodes_ms, "bound": "mfma", "flops_per_launch": flops,
            "achieved": flops / (nodes_ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": flops / (nodes_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "cascade_tokens_per_s": n / ((rq_ms + nodes_ms) * 1e-3)}
        del feat, weight, y, q, src
        torch.cuda.empty_cache()
    if "two_maps" in which or "gemm_reference" in which:
        out.update(run_two_maps(p3d, synth, stream, reps, which, dev))
    return out


def run_two_maps(p3d, synth, stream, reps, which, dev):
    """The texture stage's two-map workload: one token order per stage,
    shared by the fused call, the diagnostics and the gather-once samples."""
    import numpy as np
    import torch
    out = {}
    w = synth.workload("shell1024_cfg_twomap_bf16_c1024x2_d1536")
    coords = dev(synth.coords(w))
    n, nn = w.n_tokens, w.n_null
    maps = [dev(m, True) for m in synth.feature_maps(w)]
    weight = dev(synth.weight(w), True)
    cams = [p3d.p3d_make_camera(a, p3d.p3d_distance_from_fov(a, w.width, 0))
            for a in synth.fovs(w)]
    camarr = p3d.make_cameras(cams)
    K = sum(m.shape[3] for m in maps)
    order, run_order = make_order(p3d, coords, n, w.resolution, camarr, maps)
    order_ms = time_events(run_order, reps, stream)
    # algorithmic bytes: coords + each map's unique corner rows
    bidx = synth.coords(w)[:, 0].copy()
    uniq = 0
    for m in maps:
        pix = torch.empty((n, 2), dtype=torch.int32, device="cuda")
        p3d.p3d_project_points(coords, n, w.resolution, camarr, m.shape[1], m.shape[2],
                               pixel=pix)
        uniq += unique_corner_rows(pix.cpu().numpy(), bidx, m.shape[1], m.shape[2]) * \
            m.shape[3] * 2
    if "two_maps" in which:
        y = torch.empty((n + nn, w.out_dim), dtype=torch.bfloat16, device="cuda")
        flops = 2.0 * n * w.k_total * w.out_dim
        res = {}
        for key, o in (("plain", None), ("ordered", order)):
            f = lambda: p3d.p3d_proj_cond(coords, n, w.resolution, camarr, maps, weight, y,
                                          n_null=nn, order=o)
            for _ in range(reps):
                f()
            res[key] = time_events(f, reps, stream)
        out["two_maps"] = {
            "workload": w.name, "kernel": bf16_kernel_name(p3d, True, n, w.out_dim), "tokens": n,
            "null_rows": nn, "maps": ["%dx%dx%dx%d" % tuple(m.shape) for m in maps],
            "mean_ms": res["ordered"], "order_ms": order_ms, "unordered_ms": res["plain"],
            "tokens_per_s": n / ((res["ordered"] + order_ms) * 1e-3), "bound": "mfma",
            "flops_per_launch": flops, "achieved": flops / (res["ordered"] * 1e-3) / 1e12,
            "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": flops / (res["ordered"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "unordered_frac": flops / (res["plain"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
        del y
        # ---- diagnostics over the same two maps: coverage, per-map mean/std,
        # cosine between the maps' samples
        stats = torch.empty(8, dtype=torch.float64, device="cuda")
        res = {}
        for key, o in (("plain", None), ("ordered", order)):
            f = lambda: p3d.p3d_projection_stats(coords, n, w.resolution, camarr, maps, stats,
                                                 order=o)
            for _ in range(reps):
                f()
            res[key] = time_events(f, reps, stream)
        dbytes = 16 * n + uniq + 64
        out["diagnostics"] = hbm_part(
            w.name, "stats_kernel<true>", n, res, order_ms, dbytes,
            figures=p3d.p3d_stats_figures(stats, [m.shape[3] for m in maps]),
            traffic=recorded_traffic("stats_kernel", w.name))
        # ---- gather once per stage
        S = torch.empty((n, K), dtype=torch.bfloat16, device="cuda")
        res = {}
        for key, o in (("plain", None), ("ordered", order)):
            f = lambda: p3d.p3d_proj_sample(coords, n, w.resolution, camarr, maps, S, order=o)
            for _ in range(reps):
                f()
            res[key] = time_events(f, reps, stream)
        gbytes = 16 * n + uniq + n * K * 2
        out["gather_once"] = hbm_part(
            w.name, "sample_kernel<true, true, true> (both maps, one launch)", n, res, order_ms,
            gbytes, traffic=recorded_traffic("sample_kernel", w.name))
        # ---- every block's proj_linear over the gathered samples
        G = 30
        rng = np.random.default_rng(801)
        Wg = [torch.from_numpy(synth.bf16_bits((rng.standard_normal((w.out_dim, K)) * 0.02)
                                               .astype(np.float32))).view(torch.int16)
              .view(torch.bfloat16).cuda() for _ in range(G)]
        outs = [torch.zeros((n, w.out_dim), dtype=torch.bfloat16, device="cuda")
                for _ in range(G)]
        grp = lambda: p3d.p3d_proj_linear_grouped(S, Wg, outs, accumulate=True)
        for _ in range(max(3, reps // 4)):
            grp()
        grp_ms = time_events(grp, max(5, reps // 4), stream)
        gflops = 2.0 * n * K * w.out_dim * G
        out["grouped"] = {
            "workload": w.name + " x 30 blocks", "kernel": "grouped_kernel<true>", "tokens": n,
            "blocks": G, "mean_ms": grp_ms, "bound": "mfma", "flops_per_launch": gflops,
            "achieved": gflops / (grp_ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": gflops / (grp_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "note": "residual add: every block's output is read and rewritten (S 2048 -> 1536)"}
        del Wg, outs
    else:
        S = torch.empty((n, K), dtype=torch.bfloat16, device="cuda")
        p3d.p3d_proj_sample(coords, n, w.resolution, camarr, maps, S, order=order)
    if "gemm_reference" in which:
        # the same product, one block without the residual, through the tile
        # and through a library GEMM (torch.matmul, ROCm's BLAS): a reference
        # for what a plain bf16 GEMM of this shape reaches on this device
        rng = np.random.default_rng(802)
        W1 = torch.from_numpy(synth.bf16_bits((rng.standard_normal((w.out_dim, K)) * 0.02)
                                              .astype(np.float32))).view(torch.int16) \
            .view(torch.bfloat16).cuda()
        y1 = torch.empty((n, w.out_dim), dtype=torch.bfloat16, device="cuda")
        wt = W1.t().contiguous()
        one = lambda: p3d.p3d_proj_linear_grouped(S, [W1], [y1])
        lib_mm = lambda: torch.matmul(S, wt, out=y1)
        for f in (one, lib_mm):
            for _ in range(3):
                f()
        # alternating blocks, medians: the two are compared under the same clocks
        t_one, t_lib = [], []
        for _ in range(5):
            t_one.append(time_events(one, reps, stream))
            t_lib.append(time_events(lib_mm, reps, stream))
        one_ms, lib_ms = float(np.median(t_one)), float(np.median(t_lib))
        f1 = 2.0 * n * K * w.out_dim
        out["gemm_reference"] = {
            "shape": "[%d, %d] x [%d, %d] bf16" % (n, K, K, w.out_dim),
            "grouped_kernel_one_block_ms": one_ms,
            "grouped_kernel_frac": f1 / (one_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "library_gemm": "torch.matmul (ROCm BLAS)", "library_gemm_ms": lib_ms,
            "library_gemm_frac": f1 / (lib_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
        del W1, y1, wt
    del maps, weight, coords, S, order
    torch.cuda.empty_cache()
    return out


def hbm_part(workload, kernel, n, res, order_ms, nbytes, **more):
    """An HBM-bound part timed with and without the token order. The faster
    of the two is the one reported as mean_ms / frac (variant says which);
    with the order, frac_incl_order adds one order computation (one per
    stage, shared with the fused call)."""
    variant = "ordered" if res["ordered"] < res["plain"] else "plain"
    ms = res[variant]
    d = {"workload": workload, "kernel": kernel, "tokens": n, "variant": variant,
         "mean_ms": ms, "bound": "hbm",
         "bytes_per_launch": nbytes, "achieved": nbytes / (ms * 1e-3) / 1e9,
         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
         "order_ms": order_ms,
         "frac_incl_order": (nbytes / ((ms + order_ms) * 1e-3) / 1e9 / HBM_PEAK_GBS
                             if variant == "ordered" else None),
         "ordered_ms": res["ordered"], "unordered_ms": res["plain"],
         "ordered_frac": nbytes / (res["ordered"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
         "unordered_frac": nbytes / (res["plain"] * 1e-3) / 1e9 / HBM_PEAK_GBS}
    d.update(more)
    return d


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (profiling runs)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the adjacent-part measurements")
    ap.add_argument("--extras", default=",".join(EXTRAS),
                    help="comma-separated adjacent parts to measure (of %s)" % ", ".join(EXTRAS))
    ap.add_argument("--extras-only", action="store_true",
                    help="measure only the adjacent parts named by --extras (profiling runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB per launch (counter scale)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures a single GPU: the path shards by tokens with no per-call "
              "collective, and only the one-GPU share is measured. Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    which = set(x for x in args.extras.split(",") if x)
    unknown = which - set(EXTRAS)
    if unknown:
        ap.error("unknown extras: %s" % ", ".join(sorted(unknown)))

    import numpy as np
    import torch

    import p3d_synth as synth
    import pixel_aligned_image_amd as p3d

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    reps = max(args.steps, 20)

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(args.warmup + args.steps):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4,
                          "launches": args.warmup + args.steps}))
        return

    if args.extras_only:
        print(json.dumps({"extra": run_extra(p3d, synth, stream, reps, lambda: None, which)}),
              flush=True)
        return

    w = synth.workload(args.workload)
    bf16 = w.dtype == "bf16"
    t_gen = time.perf_counter()
    coords = synth.coords(w)
    feat_np = synth.feature_map(w)
    weight_np = synth.weight(w)
    bias_np = synth.bias(w)
    fovs = synth.fovs(w)
    n, n_null = w.n_tokens, w.n_null
    t_gen = time.perf_counter() - t_gen

    def dev(a, as_bf16=False):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a))
        if as_bf16:
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.cuda()

    coords_d = dev(coords)
    feat = dev(feat_np, bf16)
    weight = dev(weight_np, bf16)
    bias = dev(bias_np, bf16)
    dists = [w.distance] * w.batch
    cams = []
    for a, d in zip(fovs, dists):
        cams.append(p3d.p3d_make_camera(a, d if d is not None else
                                        p3d.p3d_distance_from_fov(a, w.width, 0)))
    camarr = p3d.make_cameras(cams)
    dt = torch.bfloat16 if bf16 else torch.float32
    out = torch.empty((n + n_null, w.out_dim), dtype=dt, device="cuda")
    mask = torch.empty((n,), dtype=torch.uint8, device="cuda")
    # bf16 sparse workloads take the tokens in image-space order: the step
    # computes the order (p3d_token_order) and runs the fused kernel through
    # it (p3d_proj_cond_ordered), which is what p3d_proj_cond_ws does in one
    # call; split here so that events bracket the fused kernel alone
    ordered = bf16 and coords_d is not None
    if ordered:
        order, run_order = make_order(p3d, coords_d, n, w.resolution, camarr, [feat], w.points)
    torch.cuda.synchronize()

    def fused():
        p3d.p3d_proj_cond(coords_d, n, w.resolution, camarr, feat, weight, out, bias=bias,
                          n_null=n_null, mask=mask, order=order if ordered else None)

    def step():
        if ordered:
            run_order()
        fused()

    def unordered_step():
        p3d.p3d_proj_cond(coords_d, n, w.resolution, camarr, feat, weight, out, bias=bias,
                          n_null=n_null, mask=mask)

    # An idle GPU takes tens of milliseconds of work to reach its working
    # clocks: untimed steps run for a fixed 0.3 s before the side
    # measurements and again before the timed steps.
    def settle():
        t_settle = time.perf_counter()
        while time.perf_counter() - t_settle < 0.3:
            for _ in range(10):
                step()
            torch.cuda.synchronize()

    # ---- side measurements first; the standalone gather on the same points
    settle()
    grid = torch.empty((n, 2), device="cuda")
    pixel = torch.empty((n, 2), dtype=torch.int32, device="cuda")
    p3d.p3d_project_points(coords_d, n, w.resolution, camarr, w.height, w.width, grid=grid,
                           pixel=pixel)
    bidx_np = coords[:, 0].copy() if coords is not None else np.repeat(
        np.arange(w.batch, dtype=np.int32), w.resolution ** 3)
    bidx = dev(bidx_np)
    s_out = torch.empty((n, w.channels), dtype=dt, device="cuda")

    # the standalone gather at the same points, in the step's token order
    # (p3d_bilinear_sample_ordered; the same points in the caller's order,
    # p3d_bilinear_sample, are timed with the adjacent parts)
    def gather_only():
        p3d.p3d_bilinear_sample(feat, grid, s_out, batch_index=bidx)

    def gather_ordered():
        p3d.p3d_bilinear_sample(feat, grid, s_out, batch_index=bidx, order=order)

    gather_line = gather_ordered if ordered else gather_only
    for _ in range(reps):
        gather_line()
    gather_ms = time_events(gather_line, reps, stream)

    # the null-branch fill alone (its own kernel when there are no tokens)
    out_null = out[n:]

    def null_only():
        p3d.p3d_proj_cond(None, 0, w.resolution, camarr, feat, weight, out_null, bias=bias,
                          n_null=n_null)

    def lead():
        for _ in range(4):
            step()

    null_ms = time_events(null_only, reps, stream, lead) if n_null else 0.0
    copy = hbm_copy_ceiling(p3d, stream, reps)
    torch.cuda.synchronize()

    # ---- the timed steps, after the clock settle and the W warmup steps
    settle()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # events on the launch stream around each launch: [start, after order,
    # after the fused kernel] per step
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev[k][0].record(stream)
        if ordered:
            run_order()
        ev[k][1].record(stream)
        fused()
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    fused_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    order_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps if ordered else 0.0
    gpu_step_ms = ev[0][0].elapsed_time(ev[-1][2]) / args.steps

    U = unique_corner_rows(pixel.cpu().numpy(), bidx_np, w.height, w.width)
    s = 2 if bf16 else 4
    C, D = w.channels, w.out_dim
    flops = 2.0 * n * C * D
    fused_bytes = 16 * n + U * C * s + D * C * s + (D * s if bias is not None else 0) \
        + n * D * s + n + n_null * D * s
    gather_bytes = 8 * n + 4 * n + U * C * s + n * C * s
    null_bytes = n_null * D * s
    peak = BF16_PEAK_TFLOPS if bf16 else F32_PEAK_TFLOPS
    achieved = flops / (fused_ms * 1e-3) / 1e12
    kname = "proj_cond_bf16_kernel" if bf16 else "proj_cond_kernel"
    traffic = recorded_traffic(kname, w.name)
    gather_gbs = gather_bytes / (gather_ms * 1e-3) / 1e9

    line = {
        "metric": "projected tokens/sec (project+sample+proj_linear); HBM GB/s & MFMA % of peak",
        "value": n / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": n, "null_rows": n_null,
                   "resolution": w.resolution, "batch": w.batch,
                   "map": "%dx%dx%dx%d %s NHWC" % (w.batch, w.height, w.width, C, w.dtype),
                   "proj_linear": "%d->%d%s" % (C, D, " +bias" if bias is not None else ""),
                   "unique_corner_rows": U,
                   "step": ("p3d_token_order + p3d_proj_cond_ordered (= p3d_proj_cond_ws)"
                            if ordered else "p3d_proj_cond")},
        "rows_per_sec_incl_null": (n + n_null) / (ms_per_step * 1e-3),
        "gpu_ms_per_step": gpu_step_ms,
        "order_ms": order_ms,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "kernel": kname, "mean_ms": fused_ms,
                     "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": fused_bytes,
                     "tiling": (p3d.p3d_proj_cond_plan(
                         n, D, torch.cuda.get_device_properties(0).multi_processor_count)
                                if bf16 else None)},
        "gather": {"bound": "hbm", "achieved": gather_gbs,
                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                   "frac": gather_gbs / HBM_PEAK_GBS,
                   "frac_of_copy_ceiling": gather_gbs / copy["achieved"],
                   "kernel": "sample_kernel", "mean_ms": gather_ms,
                   "call": ("p3d_bilinear_sample_ordered (the step's token order)" if ordered
                            else "p3d_bilinear_sample"),
                   "traffic": recorded_traffic("sample_kernel", w.name),
                   "algorithmic_bytes_per_launch": gather_bytes},
        "hbm_copy_ceiling": copy,
        "null_fill": {"bound": "hbm", "mean_ms": null_ms,
                      "achieved": null_bytes / (null_ms * 1e-3) / 1e9 if null_ms else None,
                      "unit": "GB/s", "bytes_per_launch": null_bytes},
        "input_generation_s": t_gen,
        "source_digest": {k: kernel_source_digest(k) for k in KERNEL_SOURCES},
    }
    if not args.no_extra:
        line["extra"] = run_extra(p3d, synth, stream, reps, step, which,
                                  unordered_step if ordered else None, flops,
                                  (gather_only, gather_bytes) if ordered else None)
    if not args.no_cpu_baseline:
        import oracle
        o = oracle.get()
        fo, do = o.cameras(fovs, [d if d is not None else o.distance_from_fov(a, w.width, 0)
                                  for a, d in zip(fovs, dists)])
        inp = dict(w=w, coords=coords, n=n, n_null=n_null, feat=feat_np, weight=weight_np,
                   bias=bias_np)
        line["cpu_baseline"] = cpu_baseline(inp, (fo, do))
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
