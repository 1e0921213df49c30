"""Benchmark of the per-latent-frame decode step on one MI355X.

One step = one fd_decode_frame call: the whole hot path (patchify, input
projection, every block's LayerNorm / QKV + ring write / attention / output
projection / MLP, final LayerNorm, unpatchify + pixel shuffle) for one latent
frame.  After warm-up frames the decoder is reset and the timed run decodes
frames 0 .. steps-1 of a stream (frame 0 attends to itself only, every later
frame to W = 2 cached frames).  Inputs are synthetic (seeded N(0,1)
latents, N(0, 0.02^2) bf16 weights) and resident in HBM before the timed
region.

Prints one JSON line.  `value` = decoded pixel frames per second
(4 pixel frames per latent frame) on the 1080p workload; 720p is reported
beside it.  `roofline` covers the dominant kernel (attention), timed with HIP
events on the library's stream over the timed region (one attention launch
per step, cycling through the blocks); the per-kernel breakdown comes from a
separate pass after it.  `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def flops_per_frame(cfg, n_valid: int) -> dict:
    """Algorithmic FLOPs (2 per multiply-add) of one frame, per kernel class.

    The refinement blocks of the upsampling tail run the same kernel classes
    as the backbone blocks on N4 = r_t N tokens (keys n_valid N4); the tail's
    last GEMM (spatial MLP output + pixel shuffle) counts as "unpatchify".
    Everything scales with the batch of streams."""
    N, D, F, L, R = cfg.n_tokens, cfg.d_model, cfg.mlp_dim, cfg.n_layers, cfg.n_refine
    N4 = cfg.n_sub_tokens if R else 0
    f = _flops_one_stream(cfg, n_valid, N, D, F, L, R, N4)
    return {k: v * cfg.batch for k, v in f.items()}


def _flops_one_stream(cfg, n_valid, N, D, F, L, R, N4) -> dict:
    f = {
        "inproj": 2.0 * N * D * cfg.c_in,
        "qkv": 2.0 * (L * N + R * N4) * cfg.qkv_dim * D,
        "attention": 4.0 * (L * N * n_valid * N + R * N4 * n_valid * N4) * D,  # QK^T, PV
        "oproj": 2.0 * (L * N + R * N4) * D * D,
        "fc1": 2.0 * (L * N + R * N4) * F * D,
        "fc2": 2.0 * (L * N + R * N4) * D * F,
    }
    if R:
        f["temporal"] = 2.0 * N * cfg.out_t * D * D
        f["spatial"] = 2.0 * N4 * cfg.up_dim * D
        f["unpatchify"] = 2.0 * N4 * cfg.sub_c_out * cfg.up_dim
    else:
        f["unpatchify"] = 2.0 * N * cfg.c_out * D
    return f


def backbone_attention_flops(cfg, n_valid: int) -> float:
    """FLOPs of one backbone block's attention launch (QK^T and PV), all streams."""
    return 4.0 * cfg.n_tokens * n_valid * cfg.n_tokens * cfg.d_model * cfg.batch


def log(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def run_gpu(cfg, steps: int, warmup: int, profile: bool = True, graph: bool = False):
    """Decode warmup + steps frames; time the last `steps` (the timed region).

    With graph, the decoder runs on a stream of its own and replays one
    recorded graph per frame (fd_graph_enable); a replay makes no per-launch
    records, so there is no profiling then.

    Inside the timed region the library records one HIP event pair per frame,
    around the attention launch of block (frame index mod n_layers), on its
    own stream: the dominant kernel's duration is measured live at a cost of
    one event pair per step.  The per-kernel breakdown comes from a separate
    pass after the timed region that times every launch (event pairs around
    all launches slow a step down by several percent, so they stay out of
    the timed region).
    """
    import torch
    import transformer_latent_pixel_amd as fd

    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    free0 = torch.cuda.mem_get_info()[0]
    weights = W.make_weights(cfg)
    stream = torch.cuda.Stream() if graph else None
    dec = fd.Decoder(cfg, weights, stream=stream)
    del weights
    if graph:
        profile = False
        dec.graph_enable(True)
    frames = warmup + steps
    if cfg.batch > 1:
        lat = [torch.from_numpy(z).cuda() for z in W.make_batched_latents(cfg, frames=frames)]
        pix = torch.empty((cfg.batch,) + cfg.pixel_shape, dtype=torch.float32, device="cuda")
    else:
        lat = [torch.from_numpy(z).cuda() for z in W.make_latents(cfg, frames=frames)]
        pix = torch.empty(cfg.pixel_shape, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    log(f"{cfg.name}: decoder created, arena {dec.query()['arena_bytes'] / 1e9:.2f} GB")

    for t in range(warmup):
        dec.decode_frame(lat[t], pix)
    # The timed run starts from frame 0 of a fresh stream (fd_reset), after
    # the warm-up frames above.
    dec.reset()
    torch.cuda.synchronize()
    if profile:
        dec.profile_read()            # drop anything recorded so far
        dec.profile_enable(True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if profile:
            # Frame 0 attends to one cached frame only: sample frames >= 1
            # (layer n_layers + n_refine is past the refinement blocks too,
            # so frame 0 records nothing).
            dec.profile_filter(["attention"],
                               i % cfg.n_layers if i > 0 else cfg.n_layers + cfg.n_refine)
        ev[i][0].record(stream)
        dec.decode_frame(lat[warmup + i], pix)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per_frame = np.array([a.elapsed_time(b) for a, b in ev])
    timed = dec.profile_read() if profile else None
    kernels = None
    if profile:
        # Breakdown pass (not timed): every launch of `steps` more frames.
        dec.profile_filter(None, -1)
        for i in range(steps):
            dec.decode_frame(lat[warmup + i], pix)
        kernels = dec.profile_read()
        dec.profile_enable(False)
    info = dec.query()
    free_min = torch.cuda.mem_get_info()[0]
    harness = sum(x.numel() * x.element_size() for x in lat) + pix.numel() * 4
    dec.close()
    log(f"{cfg.name}: {steps} frames in {elapsed:.3f} s")
    return {
        "elapsed_s": elapsed,
        "per_frame_ms": per_frame,
        "timed_attention": timed["attention"] if timed else None,
        "kernels": kernels,
        "info": info,
        "device_used_bytes": free0 - free_min,
        "harness_bytes": harness,
        "torch_peak_bytes": torch.cuda.max_memory_allocated(),
    }


def hbm_bytes_per_frame(cfg) -> dict:
    """Minimum HBM bytes per frame of the HBM-bound kernel classes."""
    N, D, L, R = cfg.n_tokens, cfg.d_model, cfg.n_layers, cfg.n_refine
    N4 = cfg.n_sub_tokens

    def ln(rows):        # read H (fp32) + gain/shift, write A (bf16)
        return rows * D * 4 + rows * D * 2 + 2 * D * 4

    if R:
        # read U (bf16) + W_s2 (bf16) + bias, write the pixel frame (fp32)
        unp = (N4 * cfg.up_dim * 2 + cfg.sub_c_out * cfg.up_dim * 2 + cfg.sub_c_out * 4
               + N4 * cfg.sub_c_out * 4)
    else:
        # read A (bf16) + W_out (bf16) + bias, write the pixel frame (fp32)
        unp = N * D * 2 + cfg.c_out * D * 2 + cfg.c_out * 4 + N * cfg.c_out * 4
    per = {
        "layernorm": (2 * L + 1) * ln(N) + ((2 * R + 1) * ln(N4) if R else 0),
        "unpatchify": unp,
        # read the latent frame (fp32), write tokens (bf16, K padded to 64)
        "patchify": cfg.latent_c * cfg.latent_h * cfg.latent_w * 4
                    + N * ((cfg.c_in + 63) // 64 * 64) * 2,
    }
    return {k: v * cfg.batch for k, v in per.items()}


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "attention_1080p_traffic.json")
ATTENTION_SOURCES = ("transformer_latent_pixel_amd/csrc/attention.hip",
                     "transformer_latent_pixel_amd/csrc/fd_common.h")


def attention_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in ATTENTION_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def attention_traffic(cfg):
    """HBM bytes per attention launch from the recorded FETCH_SIZE/WRITE_SIZE
    counters, each scaled by its plain-copy calibration factor; None when no
    record exists for this workload or the kernel source changed since."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != cfg.name or rec.get("source_sha256") != attention_source_digest():
        return None
    return (rec["fetch_kib"] * rec["fetch_factor"]
            + rec["write_kib"] * rec["write_factor"]) * 1024.0


def device_info() -> dict:
    """Name, compute units, memory and architecture of device 0, as the runtime
    reports them."""
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "compute_units": p.multi_processor_count,
            "memory_gb": round(p.total_memory / 1e9, 1),
            "arch": getattr(p, "gcnArchName", None)}


def gemm_compare(reps: int) -> dict:
    """The 1080p GEMM shapes through this library (fdk_gemm: QKV-sized with the
    fp32 epilogue, FC1 with GELU to bf16, FC2 and the out-projection with the
    residual epilogue) and through torch.nn.functional.linear (the vendor
    library, bf16 output, bias only), `reps` launches each.  Each launch is
    timed with HIP events and the median of launches 3..reps is reported (the
    first calls pay for library set-up).  For side-by-side counter runs under
    rocprofv3."""
    import torch
    import transformer_latent_pixel_amd as fd
    if reps < 3:
        raise SystemExit("--gemm-compare needs at least 3 launches per shape")
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    M, MA, D, F = 8160, 8192, 1024, 4096
    a = torch.randn(MA, F, device="cuda", generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(F, F, device="cuda", generator=g)).to(torch.bfloat16)
    bias = 0.02 * torch.randn(F, device="cuda", generator=g)
    u = torch.empty(MA, F, dtype=torch.bfloat16, device="cuda")
    h = torch.zeros(MA, D, device="cuda")
    hq = torch.zeros(MA, 3 * D, device="cuda")
    shapes = {"qkv_f32": (0, a[:, :D].contiguous(), w[:3 * D, :D].contiguous(), 3 * D, D, hq),
              "fc1_gelu": (2, a[:, :D].contiguous(), w[:, :D].contiguous(), F, D, u),
              "fc2_resid": (1, a, w[:D].contiguous(), D, F, h),
              "oproj_resid": (1, a[:, :D].contiguous(), w[:D, :D].contiguous(), D, D, h)}
    def per_launch(fn):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(reps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        t = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(2, reps))
        return round(t[len(t) // 2], 1)

    res = {}
    for name, (epi, A, W_, n, k, out) in shapes.items():
        A2, b2 = A[:M], bias[:n].to(torch.bfloat16)
        res[name] = {
            "this_library_us": per_launch(lambda: fd.fdk_gemm(
                epi, A.view(torch.int16), W_.view(torch.int16), bias, out, M, MA, n, k)),
            "vendor_linear_us": per_launch(lambda: torch.nn.functional.linear(A2, W_, b2))}
    return res


def mfma_probe(iters: int = 200000) -> dict:
    """Sustained bf16 matrix-core rate with register operands (fdk_mfma_probe),
    all-zero and random, with the shader clock the waves ran at."""
    import torch
    import transformer_latent_pixel_amd as fd
    wgs = fd.capi.PROBE_WORKGROUPS
    sink = torch.empty(wgs * 512, device="cuda")
    clocks = torch.zeros(wgs * 8 * 2, dtype=torch.int64, device="cuda")
    flops = 2.0 * 32 * 32 * 16 * 8 * iters * 8 * wgs
    res = {}
    for name, zero in (("zero_operands", True), ("random_operands", False)):
        fd.fdk_mfma_probe(zero, 100, sink, clocks)          # warm-up launch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        fd.fdk_mfma_probe(zero, iters, sink, clocks)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        c = clocks.view(-1, 2).cpu().numpy().astype(np.float64)
        ghz = c[:, 0] / c[:, 1] * 0.1
        res[name] = {"tflops": flops / (ms * 1e-3) / 1e12,
                     "frac_of_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                     "ms": ms, "shader_clock_ghz_mean": float(ghz.mean()),
                     "shader_clock_ghz_min": float(ghz.min()),
                     "shader_clock_ghz_max": float(ghz.max())}
    return res


def measure_copy_gbs(mib: int = 1024, reps: int = 10) -> float:
    """Device-to-device copy rate (GB/s, bytes read + bytes written) of a
    plain copy of `mib` MiB, larger than every cache level: the practical
    HBM ceiling that the HBM-bound kernels are also compared with."""
    import torch
    n = mib << 18                                   # float32 elements
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    secs = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    return 2.0 * 4 * n / secs / 1e9


def summarize(cfg, r, steps, copy_gbs=None):
    ms = r["elapsed_s"] * 1e3 / steps
    fpf = flops_per_frame(cfg, cfg.window)
    total_flops = sum(fpf.values())
    out = {
        "pixel_fps": cfg.batch * cfg.out_t * steps / r["elapsed_s"],
        # The pages count 1 + 4 (T' - 1) pixel frames for T' latent frames (the
        # first latent frame of the Wan VAE decodes to one frame).
        "pixel_fps_first_frame_single": cfg.batch * (1 + cfg.out_t * (steps - 1)) / r["elapsed_s"],
        "latent_fps": cfg.batch * steps / r["elapsed_s"],
        "ms_per_frame": ms,
        "latency_ms": {"p50": float(np.percentile(r["per_frame_ms"], 50)),
                       "p99": float(np.percentile(r["per_frame_ms"], 99)),
                       "max": float(r["per_frame_ms"].max()),
                       "frame0": float(r["per_frame_ms"][0]),
                       "p50_without_frame0": float(np.percentile(r["per_frame_ms"][1:], 50)),
                       "p99_without_frame0": float(np.percentile(r["per_frame_ms"][1:], 99))},
        "tflop_per_frame": total_flops / 1e12,
        "mfma_util_whole_step": total_flops / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "hbm_gb": {"arena": r["info"]["arena_bytes"] / 1e9,
                   "ring": r["info"]["ring_bytes"] / 1e9,
                   "weights": r["info"]["weight_bytes"] / 1e9,
                   "workspace": r["info"]["workspace_bytes"] / 1e9,
                   "harness_buffers": r["harness_bytes"] / 1e9,
                   "torch_peak_allocated": r["torch_peak_bytes"] / 1e9,
                   "device_used_delta": r["device_used_bytes"] / 1e9},
    }
    k = r["kernels"]
    if k:
        per = {}
        for name, v in k.items():
            if not v["launches"]:
                continue
            avg = v["ms"] / v["launches"]
            e = {"ms_per_frame": v["ms"] / steps, "avg_launch_ms": avg,
                 "launches": v["launches"]}
            if name in fpf:
                flops_launch = fpf[name] / (v["launches"] / steps)
                e["tflops"] = flops_launch / (avg * 1e-3) / 1e12
                e["mfma_frac"] = e["tflops"] / PEAK_BF16_TFLOPS
            hb = hbm_bytes_per_frame(cfg)
            if name in hb:
                e["hbm_gbs"] = hb[name] / (e["ms_per_frame"] * 1e-3) / 1e9
                e["hbm_frac"] = e["hbm_gbs"] / PEAK_HBM_GBS
                if copy_gbs:
                    e["hbm_frac_of_copy"] = e["hbm_gbs"] / copy_gbs
            per[name] = e
        out["kernels"] = per
        mm = [n for n in per if n in fpf]
        mm_ms = sum(per[n]["ms_per_frame"] for n in mm)
        out["mfma_util_gemm_attention"] = (
            sum(fpf[n] for n in mm) / (mm_ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12))
    return out


def cpu_baseline(cfg):
    """Time the CPU oracle on full frames of the same workload.

    The oracle decodes frames 0 and 1 of the same seeded stream at full depth
    and full spatial size; frame 1 is steady state (two frames in the window,
    like every later frame), and its wall time gives the reported rate.  The
    oracle is the float64 numpy one, unchanged; its BLAS and its per-head
    thread pool use the threads the host allots to this process
    (OMP_NUM_THREADS, else the CPUs in its affinity mask).
    """
    import oracle
    from threadpoolctl import threadpool_info

    weights = W.make_weights(cfg)
    zs = W.make_latents(cfg, frames=2)
    dec = oracle.StreamingDecoder(cfg, weights)
    secs = []
    for t, z in enumerate(zs):
        t0 = time.perf_counter()
        dec.decode_frame(z)
        secs.append(time.perf_counter() - t0)
        log(f"cpu baseline: {cfg.name} frame {t} ({cfg.n_layers} blocks) took {secs[-1]:.1f} s")
    blas = [p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max(blas + [oracle.host_threads()])
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    return {"value": cfg.out_t / secs[1], "unit": "pixel frames/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"{cfg.name}: measured full frames, float64 numpy oracle, all "
                       f"{cfg.n_layers} blocks at full spatial size: frame 0 (one cached "
                       f"frame) {secs[0]:.1f} s, frame 1 (steady state, two cached frames) "
                       f"{secs[1]:.1f} s; value = {cfg.out_t} pixel frames / frame 1 time"),
            "precision": "float64",
            "threads_used": threads,
            "cpus_available": affinity,
            "cpus_online": os.cpu_count(),
            "cpu_model": _cpu_model()}


def _cpu_model():
    """The /proc/cpuinfo model name of the first CPU, with its family, model,
    stepping, cache size and clock (a virtualised host may report only a
    short model name)."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if not line.strip():
                break
            k, _, v = line.partition(":")
            fields[k.strip()] = v.strip()
    except OSError:
        return "unknown"
    name = fields.get("model name", "unknown")
    extra = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping", "cache size",
                                          "cpu MHz") if k in fields]
    return f"{name} ({', '.join(extra)})" if extra else name


def describe(cfg):
    block = ""
    if cfg.kv_heads != cfg.n_heads or cfg.norm != "layer" or cfg.kv_norm or cfg.rope:
        block = (f", {cfg.kv_heads} KV heads, {cfg.norm.upper()}Norm"
                 f"{', KV-norm' if cfg.kv_norm else ''}{', 3D-RoPE' if cfg.rope else ''}")
    if cfg.batch > 1:
        block += f"; {cfg.batch} independent streams decoded together"
    if cfg.n_refine:
        block += (f"; temporal-first upsampling tail: D -> {cfg.out_t}D, {cfg.n_refine} "
                  f"refinement blocks over {cfg.n_sub_tokens} sub-frame tokens, spatial MLP "
                  f"{cfg.d_model} -> {cfg.up_dim} -> {cfg.sub_c_out}")
    return (f"{cfg.name}: latent {cfg.latent_c}x{cfg.latent_h}x{cfg.latent_w} patch "
            f"{cfg.patch} -> {cfg.n_tokens} tokens/frame, {cfg.n_layers} blocks, "
            f"D={cfg.d_model}, {cfg.n_heads}x{cfg.head_dim} heads{block}, MLP {cfg.mlp_dim}, "
            f"W={cfg.window}, {cfg.out_t}x{cfg.pix_h}x{cfg.pix_w}x{cfg.out_c} pixels "
            f"per latent frame")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="1080p",
                    choices=["480p", "720p", "1080p", "xl_720p", "xl_720p_tr", "480p_x8"],
                    help="xl_720p: the paper's block (RMSNorm, GQA, KV-norm, 3D-RoPE) at "
                         "FlashDecoder-XL size on the 720p latent; xl_720p_tr: the same with "
                         "the temporal-first upsampling tail (2 refinement blocks); 480p_x8: "
                         "eight 480p streams decoded together (pixel frames/s of all streams)")
    ap.add_argument("--window", type=int, default=0,
                    help="override the workload's window W (latent frames in the cache)")
    ap.add_argument("--secondary", default="720p",
                    help="also report this workload ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle timing (about a minute at 1080p)")
    ap.add_argument("--no-profile", action="store_true",
                    help="time without per-kernel events")
    ap.add_argument("--graph", action="store_true",
                    help="replay one recorded HIP graph per frame (fd_graph_enable); "
                         "no per-kernel events, so no roofline or kernel breakdown")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (a known-size "
                         "kernel for calibrating HBM byte counters)")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only measure the sustained bf16 matrix-core rate and shader "
                         "clock with register operands (zero and random), and exit")
    ap.add_argument("--gemm-compare", type=int, default=0, metavar="REPS",
                    help="only time the 1080p GEMM shapes through this library and "
                         "through torch.nn.functional.linear, REPS launches each, and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not "
              f"supported (independent video streams shard across GPUs with no "
              f"exchange, see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.mfma_probe:
        print(json.dumps({"mfma_probe": mfma_probe(), "device": device_info()}), flush=True)
        return
    if args.gemm_compare:
        print(json.dumps({"gemm_compare": gemm_compare(args.gemm_compare)}), flush=True)
        return
    if args.calibrate_copy:
        n = args.calibrate_copy << 18                  # float32 elements
        # Source uploaded from host memory and then pushed out of the caches
        # by 3 GiB of unrelated writes; the device-to-device copy (one runtime
        # blit kernel) then reads and writes exactly 4n bytes each.
        src = torch.from_numpy(np.ones(n, dtype=np.float32)).to("cuda")
        big = torch.empty(3 << 28, device="cuda")
        big.zero_()
        del big
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.calibrate_copy} MiB done")
        del src, dst
    cfg = W.CONFIGS[args.workload]
    if args.window:
        cfg = cfg.replace(window=args.window)
    copy_gbs = measure_copy_gbs()
    log(f"device copy: {copy_gbs:.0f} GB/s (read + write)")
    r = run_gpu(cfg, args.steps, args.warmup, profile=not args.no_profile, graph=args.graph)
    s = summarize(cfg, r, args.steps, copy_gbs)

    line = {
        "metric": "decoded pixel frames/s + p50/p99 per-frame latency at 720p/1080p; MFMA util",
        "value": round(s["pixel_fps"], 3),
        "unit": "pixel frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(s["ms_per_frame"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": describe(cfg), "global_batch": cfg.batch,
                   "seq_len": cfg.n_tokens * cfg.window, "parallelism": "single GPU"},
        "latency_ms": s["latency_ms"],
        "value_first_frame_single": s["pixel_fps_first_frame_single"],
        "value_first_frame_single_note": "the same run counting 1 + 4 (T' - 1) pixel frames "
                                         "for T' latent frames, as the pages count a clip",
        "mfma_util_whole_step": s["mfma_util_whole_step"],
        "mfma_util_gemm_attention": s.get("mfma_util_gemm_attention"),
        "tflop_per_frame": s["tflop_per_frame"],
        "device": device_info(),
        "hbm_gb": s["hbm_gb"],
        "kernels": s.get("kernels"),
        "kernels_pass": "per-kernel times from a pass after the timed region that times "
                        "every launch with HIP events",
        "launch_mode": "graph replay (fd_graph_enable)" if args.graph else "plain launches",
        "hbm_copy_gbs": copy_gbs,
        "hbm_copy_note": "device-to-device copy of 1 GiB (bytes read + written per second): "
                         "hbm_frac_of_copy compares the HBM-bound kernel classes with it, "
                         "hbm_frac with the published 8 TB/s",
    }
    ta = r.get("timed_attention")
    if ta and ta["launches"]:
        avg = ta["ms"] / ta["launches"]
        flops = backbone_attention_flops(cfg, cfg.window)
        achieved = flops / (avg * 1e-3) / 1e12
        line["roofline"] = {"kernel": "attention_hd64_kernel", "bound": "mfma",
                            "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                            "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                            "traffic": attention_traffic(cfg),
                            "avg_launch_ms": avg, "launches_timed": ta["launches"]}
    if args.secondary and args.secondary != args.workload:
        c2 = W.CONFIGS[args.secondary]
        r2 = run_gpu(c2, args.steps, args.warmup, profile=not args.no_profile,
                     graph=args.graph)
        s2 = summarize(c2, r2, args.steps, copy_gbs)
        line["secondary"] = {"workload": describe(c2),
                             "value": s2["pixel_fps"], "unit": "pixel frames/s",
                             "ms_per_step": s2["ms_per_frame"],
                             "latency_ms": s2["latency_ms"],
                             "mfma_util_whole_step": s2["mfma_util_whole_step"],
                             "mfma_util_gemm_attention": s2.get("mfma_util_gemm_attention"),
                             "hbm_gb": s2["hbm_gb"]}
    if "roofline" in line:
        # After the timed runs, so that the probe's power draw cannot touch them.
        probe = mfma_probe()
        sus = probe["random_operands"]["tflops"]
        line["roofline"]["sustained_peak"] = sus
        line["roofline"]["frac_of_sustained"] = line["roofline"]["achieved"] / sus
        line["roofline"]["sustained_note"] = (
            "register-only bf16 MFMA loop on random operands (fdk_mfma_probe), every CU "
            f"busy: shader clock {probe['random_operands']['shader_clock_ghz_mean']:.2f} GHz "
            f"against {probe['zero_operands']['shader_clock_ghz_mean']:.2f} GHz with zero "
            "operands; peak stays the published figure")
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
