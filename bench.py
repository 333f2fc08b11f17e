"""Benchmark of the STEPQuant packed-state decode step on one MI355X.

A step is one stepq_decode_step call over the whole batch: every (request,
head) tile is rebuilt from its packed codes, updated by the gated Delta rule,
read out, refitted and written back.  The default workload is the batch-512
serving shape (B=512, H=48, d_k=d_v=128, per-head gate, 6-bit nominal budget
with one FP16 pivot head): inputs drawn on the device, resident in HBM before
timing.  Row scales are the calibrated per-row constants (the headline).  Timed
beside it on the same GPU: the step with row scales refitted from the row RMS
at every step, uniform INT8 / INT4 with one scale per tile, the
per-key-channel (KDA) layout at batch 512, the split-phase schedule (readout
first, update on a second stream), the unquantised FP32-state step, plain HIP
streaming kernels (the attainable HBM rate), and the CPU oracle on a sample.
The roofline object carries the headline kernel's fraction of the HBM peak
(algorithmic bytes over its event-timed launch duration), its algorithmic
VALU fraction beside it and, when the committed counter summary matches the
kernel source, its measured HBM traffic.  Warm-up runs at least --warmup steps
and at least --warmup-ms of busy GPU time.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps 128] [--warmup 100] [--warmup-ms 1000] [--no-cpu-baseline] [--no-refit] [--no-fp32-state]
    python bench.py --copy-calibration     (plain device copy, for counter scaling)
    python bench.py --batch-sweep [--workload kimi-kda-b64]   (the step at batch 32 ... 4096)
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0                      # MI355X HBM3E, published
# FP32 vector FMA peak without packed-FP32 instructions (not used on this
# toolchain): 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz.
VALU_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
# Algorithmic floating-point work per state element and step.  Integer rows:
# dequantise r^ c^ q 2, decay 1, u and w 4 (two fma), update 2, clip-free
# maximum 1, quantise 2 (scale and round), least-squares column fit 5 (weight,
# two fma) = 17; the per-step row refit adds the row's sum of squares 2 and
# z = M' / r 1 = 20.  Binary16 / binary32 rows: decay 1, u and w 4, update 2 = 7.
# Uniform INT-b baseline (one scale per tile): dequantise 1, decay 1, u and w 4,
# update 2, maximum 1, quantise 2 = 11.
FLOPS_INT_ELEM = {"calibrated": 17, "refit": 20, "uniform": 11}
FLOPS_FLOAT_ELEM = 7
KERNEL_SOURCES = [ROOT / "quantized_recurrent_state_packed_amd" / "csrc" / n
                  for n in ("stepq_kernels.hip", "stepq_internal.hpp")]
PROFILE_TRAFFIC = ROOT / "profiles" / "decode_step_serving_b512_counters.md"


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(p.read_bytes())
    return h.hexdigest()[:16]


def kernel_name(lay) -> str:
    """The decode kernel a layout's step launches."""
    rb = lay.row_bits()
    mode = mode_of(lay)
    if lay.gate_mode == 1 and (rb.min(axis=1) != rb.max(axis=1)).any():
        return f"k_decode_rows<{mode}>" if lay.D == 128 else f"k_decode_mixed<{lay.D}, {mode}>"
    return f"k_decode_uniform<{lay.D}, {mode}>"


def mode_of(lay) -> str:
    return {0: "refit", 1: "calibrated", 2: "uniform"}[lay.row_mode]


def step_bytes(lay) -> dict:
    """Algorithmic HBM bytes of one decode step per request (one slot), by
    part: packed codes read + written, binary16 scales read + written
    (integer heads: column scales, and row scales when they are refitted),
    q/k/v read and o written (fp32), beta and gate, slot id."""
    D = lay.D
    rb = lay.row_bits()
    codes = scales = 0
    per_head_scales = {"refit": 2 * 2 * 2 * D, "calibrated": 2 * 2 * D, "uniform": 2 * 4}[mode_of(lay)]
    for h in range(lay.H):
        tile = ((int(rb[h].sum()) + 31) // 32) * D * 4
        codes += 2 * tile
        if (rb[h] <= 8).any():
            scales += per_head_scales
    qkvo = lay.H * 4 * 4 * D
    gate = lay.H * 4 * (1 if lay.gate_mode == 0 else D)
    small = lay.H * 4 + gate + 4
    return dict(codes=codes, scales=scales, qkvo=qkvo, small=small, total=codes + scales + qkvo + small)


def step_flops(lay) -> int:
    """Algorithmic floating-point operations of one decode step per request."""
    rb = lay.row_bits()
    n_int = int((rb <= 8).sum()) * lay.D
    n_flt = int((rb > 8).sum()) * lay.D
    return FLOPS_INT_ELEM[mode_of(lay)] * n_int + FLOPS_FLOAT_ELEM * n_flt


def read_traffic(expect_hash: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source."""
    if not PROFILE_TRAFFIC.exists():
        return None
    text = PROFILE_TRAFFIC.read_text()
    m = re.search(r"kernel source hash:\s*`?([0-9a-f]{16})", text)
    t = re.search(r"traffic_bytes_per_launch:\s*`?([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != expect_hash:
        return None
    return float(t.group(1))


def cpu_baseline(lay, pool_host, scales_host, inputs_host, n_req: int, n_steps: int) -> dict:
    """The oracle as it stands, on the host cores, over the first n_req
    requests of the same workload for n_steps steps."""
    from oracle import oracle as O
    ol = O.OracleLayout.from_workload(lay)
    slots = np.arange(n_req, dtype=np.int32)
    pool = pool_host[: n_req * ol.slot_bytes].copy()
    scales = scales_host[: n_req * ol.scale_halves].copy()
    O.lib()
    t0 = time.perf_counter()
    for t in range(n_steps):
        ol.step(slots, inputs_host[t], pool, scales)
    dt = time.perf_counter() - t0
    tiles = n_req * lay.H * n_steps
    return dict(value=tiles / dt, unit="state updates/s", cores=O.num_threads(), kind="oracle",
                cpu_model=cpu_model(),
                sample=f"first {n_req} of the batch's requests ({n_req * lay.H} tiles) x {n_steps} steps, "
                       f"same inputs as the GPU run; {dt:.1f} s")


def cpu_model() -> str:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def warm_up(launch, n_inputs: int, warmup: int, floor_ms: float) -> dict:
    """At least `warmup` untimed steps, and more until floor_ms of wall time has
    passed with the GPU busy (launches in chunks of 32, each chunk waited for):
    the first tens of milliseconds after a fresh start run slower than the
    steady state.  Step inputs are cycled."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < warmup or (time.perf_counter() - t0) * 1e3 < floor_ms:
        for _ in range(32 if n >= warmup else min(32, warmup - n)):
            launch(n % n_inputs)
            n += 1
        torch.cuda.synchronize()
    return dict(steps=n, ms=(time.perf_counter() - t0) * 1e3)


def timed_run(lay, steps, warmup: int, K: int, B: int, per_launch: bool = True, floor_ms: float = 0.0) -> dict:
    """Packs the workload's initial state under layout lay, runs warm-up steps
    (at least `warmup`, and at least floor_ms of busy GPU time), then times K
    decode steps with HIP events on the launch stream (the whole region, with
    nothing between launches), and -- per_launch -- K more steps with an event
    pair around every launch for the kernel's own duration."""
    import torch
    from quantized_recurrent_state_packed_amd import stepq as S
    from quantized_recurrent_state_packed_amd import workloads as W
    L = S.Layout.from_workload(lay)
    pool, scales = L.alloc(B)
    slots = torch.arange(B, dtype=torch.int32, device="cuda")
    S.stepq_pack(L.handle, B, slots, B, W.make_initial_state_torch(lay.cfg, B, "cuda", lay), pool, scales)
    o = torch.empty(B, lay.H, lay.D, dtype=torch.float32, device="cuda")

    def launch(t):
        d = steps[t]
        S.stepq_decode_step(L.handle, B, slots, B, d["q"], d["k"], d["v"], d["beta"], d["gate"], pool, scales, o)

    warm = warm_up(launch, max(1, warmup), warmup, floor_ms)
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for t in range(K):
        launch(warmup + t)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    launch_ms = None
    if per_launch:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        for t in range(K):
            ev[t][0].record(stream)
            launch(warmup + t)
            ev[t][1].record(stream)
        torch.cuda.synchronize()
        launch_ms = np.array([a.elapsed_time(b) for a, b in ev])
    return dict(total_ms=total_ms, launch_ms=launch_ms, layout=L, pool=pool, scales=scales, launch=launch,
                start=start, end=end, stream=stream, warm=warm)


SIDE_WARMUP_MS = 200.0          # warm-up floor of each side leg (--side-warmup-ms)


def side_run(lay, steps, warmup: int, K: int, B: int, packed_ms: float, note: str) -> dict:
    """Times the same steps under another layout (refit row scales, or every
    head in binary32) and releases its pool."""
    import torch
    r = timed_run(lay, steps, warmup, K, B, per_launch=False, floor_ms=SIDE_WARMUP_MS)
    ms = r["total_ms"] / K
    nbytes = step_bytes(lay)["total"] * B
    out = dict(ms_per_step=ms, bytes_per_step=nbytes,
               hbm_gbs=nbytes / (ms * 1e-3) / 1e9, hbm_frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
               time_vs_headline=ms / packed_ms, note=note)
    del r
    torch.cuda.empty_cache()
    return out


def split_phase_run(lay, steps, warmup: int, K: int, B: int, fused_ms: float) -> dict:
    """Split-phase schedule: stepq_readout (o only) on one stream, the update
    without readout (stepq_decode_step, o = NULL) on a second stream ordered
    after it, the next readout ordered after the update.  Reports the readout
    kernel's own duration (how long a consumer of o waits) and the schedule's
    time per step."""
    import torch
    from quantized_recurrent_state_packed_amd import stepq as S
    from quantized_recurrent_state_packed_amd import workloads as W
    L = S.Layout.from_workload(lay)
    pool, scales = L.alloc(B)
    slots = torch.arange(B, dtype=torch.int32, device="cuda")
    S.stepq_pack(L.handle, B, slots, B, W.make_initial_state_torch(lay.cfg, B, "cuda", lay), pool, scales)
    o = torch.empty(B, lay.H, lay.D, dtype=torch.float32, device="cuda")

    def pair(t):
        d = steps[t]
        args = (d["q"], d["k"], d["v"], d["beta"], d["gate"])
        S.stepq_readout(L.handle, B, slots, B, *args, pool, scales, o)
        S.stepq_decode_step(L.handle, B, slots, B, *args, pool, scales, None)

    warm_up(pair, max(1, warmup), 0, SIDE_WARMUP_MS)   # the side legs' warm-up floor
    s_read, s_upd = torch.cuda.Stream(), torch.cuda.Stream()
    ev_r = [torch.cuda.Event(enable_timing=True) for _ in range(warmup + K)]
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(warmup + K)]
    ev_u = [torch.cuda.Event() for _ in range(warmup + K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for t in range(warmup + K):
        d = steps[t]
        args = (d["q"], d["k"], d["v"], d["beta"], d["gate"])
        if t == warmup:
            start.record(s_read)
        if t > 0:
            s_read.wait_event(ev_u[t - 1])
        ev_a[t].record(s_read)
        S.stepq_readout(L.handle, B, slots, B, *args, pool, scales, o, stream=s_read)
        ev_r[t].record(s_read)
        s_upd.wait_event(ev_r[t])
        S.stepq_decode_step(L.handle, B, slots, B, *args, pool, scales, None, stream=s_upd)
        ev_u[t].record(s_upd)
    s_read.wait_event(ev_u[-1])
    end.record(s_read)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / K
    readout_us = float(np.mean([ev_a[t].elapsed_time(ev_r[t]) for t in range(warmup, warmup + K)])) * 1e3
    rb = step_bytes(lay)
    read_bytes = (rb["codes"] // 2 + rb["scales"] // 2 + rb["qkvo"] + rb["small"]) * B
    del pool, scales
    torch.cuda.empty_cache()
    return dict(readout_us_avg=readout_us, readout_hbm_gbs=read_bytes / (readout_us * 1e-6) / 1e9,
                schedule_ms_per_step=ms, fused_ms_per_step=fused_ms, readout_vs_fused=readout_us * 1e-3 / fused_ms,
                note="readout (o only) on one stream, update with o = NULL on a second stream after it")


def copy_calibration(nbytes: int = 1 << 30) -> None:
    """A plain device-to-device copy of known size, for scaling FETCH_SIZE /
    WRITE_SIZE counters."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes}))


def stream_reference(nbytes: int = 1 << 30, reps: int = 10) -> dict:
    """What plain HIP streaming kernels reach on this GPU (read-only, write-only
    and copy, 16-byte accesses, best of several grid sizes; libstreamprobe.so),
    to read the HBM figures against the attainable bandwidth as well as the
    published peak."""
    import ctypes
    lib = ctypes.CDLL(str(ROOT / "bench_probe" / "libstreamprobe.so"))
    lib.stepq_stream_probe.restype = ctypes.c_int
    lib.stepq_stream_probe.argtypes = [ctypes.c_size_t, ctypes.c_int] + [ctypes.POINTER(ctypes.c_double)] * 3
    r, w, c = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    rc = lib.stepq_stream_probe(nbytes, reps, ctypes.byref(r), ctypes.byref(w), ctypes.byref(c))
    if rc != 0:
        raise RuntimeError(f"stepq_stream_probe failed with HIP error {rc}")
    return {"read_gbs": r.value, "write_gbs": w.value, "copy_gbs": c.value,
            "read_frac": r.value / HBM_PEAK_GBS, "copy_frac": c.value / HBM_PEAK_GBS, "bytes": nbytes,
            "note": "plain HIP streaming kernels over 1 GiB buffers on the same GPU (copy counts bytes read "
                    "+ written); fractions of the published 8 TB/s"}


def batch_sweep(cfg: int, batches) -> list:
    """The decode step of workload cfg at several batch sizes (8 distinct input
    steps, cycled, so that large batches fit), with the pool resident before
    timing.  Every batch gets about 0.1 s of warm-up launches and at least
    30 ms of timed ones.  Reports the time per step over the timed region
    (launch gaps included: at small batches the Python launch path can show)
    and the kernel's own average duration from an event pair per launch,
    with state updates/s and the algorithmic HBM rate of each."""
    import torch
    from quantized_recurrent_state_packed_amd import workloads as W
    lay = W.make_layout(cfg)
    out = []
    for B in batches:
        est_s = 0.2e-3 * B / 512                        # rough step time, for the launch counts only
        warmup, K = max(20, int(0.1 / est_s)), max(50, int(0.03 / est_s))
        base = [W.make_step_inputs_torch(cfg, t, B, "cuda", lay) for t in range(8)]
        r = timed_run(lay, [base[t % 8] for t in range(warmup + K)], warmup, K, B, per_launch=True)
        ms = r["total_ms"] / K
        kernel_ms = float(r["launch_ms"].mean())
        nbytes = step_bytes(lay)["total"] * B
        out.append(dict(batch=B, tiles=B * lay.H, steps=K, ms_per_step=ms, kernel_us=kernel_ms * 1e3,
                        updates_per_s=B * lay.H / (ms * 1e-3), kernel_updates_per_s=B * lay.H / (kernel_ms * 1e-3),
                        hbm_gbs=nbytes / (ms * 1e-3) / 1e9, kernel_hbm_gbs=nbytes / (kernel_ms * 1e-3) / 1e9))
        del r, base
        torch.cuda.empty_cache()
    return out


def main() -> int:
    global SIDE_WARMUP_MS
    from quantized_recurrent_state_packed_amd import workloads as W

    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--warmup-ms", type=float, default=1000.0,
                    help="warm-up floor: untimed steps continue until this much busy GPU time has passed")
    ap.add_argument("--side-warmup-ms", type=float, default=SIDE_WARMUP_MS,
                    help="warm-up floor of each side leg (refit, uniform, KDA, FP32-state)")
    ap.add_argument("--workload", "--config", dest="config", metavar="NAME", type=W.workload_id, default="serving-b512-h48-d128",
                    help="workload name or index (workloads.CONFIGS)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-requests", type=int, default=128)
    ap.add_argument("--cpu-steps", type=int, default=80)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--batch", type=int, default=None,
                    help="requests per step (default: the workload's own batch)")
    ap.add_argument("--batch-sweep", action="store_true",
                    help="time the step of --workload at batch 32 ... 4096 instead (one JSON line)")
    ap.add_argument("--repeats", type=int, default=3,
                    help="timed K-step loops; the first gives value, all give the median")
    ap.add_argument("--no-refit", action="store_true",
                    help="skip the step with row scales refitted every step, timed at the same shape")
    ap.add_argument("--no-uniform", action="store_true",
                    help="skip the uniform INT8 / INT4 (one scale per tile) steps timed at the same shape")
    ap.add_argument("--no-split", action="store_true",
                    help="skip the split-phase (readout first, update on a second stream) schedule")
    ap.add_argument("--no-kda", action="store_true",
                    help="skip the per-key-channel (KDA) layout timed at batch --kda-batch")
    ap.add_argument("--kda-batch", type=int, default=512)
    ap.add_argument("--no-fp32-state", action="store_true",
                    help="skip the FP32-state (zero-loss) step timed at the same shape")
    ap.add_argument("--no-stream", action="store_true",
                    help="skip the plain streaming-bandwidth reference (frac_of_copy is then null)")
    args = ap.parse_args()
    SIDE_WARMUP_MS = args.side_warmup_ms

    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the decode step shards by request or by head with no exchange between tiles)", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration()
        return 0
    if args.batch_sweep:
        sweep = batch_sweep(args.config, (32, 64, 128, 256, 512, 1024, 2048, 4096))
        print(json.dumps({"workload": W.CONFIGS[args.config]["name"], "batch_sweep": sweep}))
        return 0

    import torch
    from quantized_recurrent_state_packed_amd import stepq as S

    cfg = args.config
    c = W.CONFIGS[cfg]
    B, H, D = args.batch or c["B"], c["H"], c["D"]
    K, Wm = args.steps, args.warmup
    dev = "cuda"
    lay = W.make_layout(cfg)                       # calibrated row scales
    steps = [W.make_step_inputs_torch(cfg, t, B, dev, lay) for t in range(Wm + K)]
    torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        from quantized_recurrent_state_packed_amd import stepq as S
        n_req = min(args.cpu_requests, B)
        L0 = S.Layout.from_workload(lay)
        pool0, scales0 = L0.alloc(n_req)
        S.stepq_pack(L0.handle, n_req, torch.arange(n_req, dtype=torch.int32, device=dev), n_req,
                     W.make_initial_state_torch(cfg, B, dev, lay)[:n_req].contiguous(), pool0, scales0)
        pool_h = pool0.cpu().numpy()
        scales_h = scales0.cpu().numpy().view(np.uint16)
        n_cpu = min(args.cpu_steps, K)          # the sample steps through the timed steps' inputs
        inp_h = [{k: v[:n_req].cpu().numpy() for k, v in steps[Wm + t].items()} for t in range(n_cpu)]
        cpu = cpu_baseline(lay, pool_h, scales_h, inp_h, n_req, n_cpu)
        del pool0, scales0

    run = timed_run(lay, steps, Wm, K, B, floor_ms=args.warmup_ms)
    total_ms, launch_ms = run["total_ms"], run["launch_ms"]
    warm = run["warm"]
    # the kernel's average duration: HIP events around the timed region of K
    # back-to-back launches on the launch stream (an event pair around every
    # launch, the loop after it, adds a few microseconds of its own per launch)
    avg_launch_s = total_ms / K * 1e-3

    # Further K-step loops over the same inputs (the state keeps evolving),
    # for the spread between repetitions (the per-launch loop ran in between).
    rep_ms = [total_ms / K]
    start, end, stream, launch = run["start"], run["end"], run["stream"], run["launch"]
    for _ in range(max(0, args.repeats - 1)):
        torch.cuda.synchronize()
        start.record(stream)
        for t in range(K):
            launch(Wm + t)
        end.record(stream)
        torch.cuda.synchronize()
        rep_ms.append(start.elapsed_time(end) / K)
    del run
    torch.cuda.empty_cache()

    refit = None
    if not args.no_refit:
        refit = side_run(dataclasses.replace(lay, row_mode=0), steps, Wm, K, B, total_ms / K,
                         "same shape and inputs; row scales refitted from the row RMS at every step")
    uniform = None
    if not args.no_uniform:
        uniform = {}
        for b in (8, 4):
            ul = dataclasses.replace(lay, unit_bits=np.full_like(lay.unit_bits, b), row_mode=2)
            uniform[f"int{b}"] = side_run(ul, steps, Wm, K, B, total_ms / K,
                                          f"same shape and inputs; uniform INT{b} with one absmax scale per tile")
    kda = None
    if not args.no_kda:
        kl = W.make_layout(2)
        kb = args.kda_batch
        ksteps = [W.make_step_inputs_torch(2, t, kb, dev, kl) for t in range(Wm + K)]
        kda = side_run(kl, ksteps, Wm, K, kb, total_ms / K,
                       f"per-key-channel gate, per-row widths (KDA workload recipe, H=32) at batch {kb}")
        kda["updates_per_s"] = kb * kl.H * 1e3 / kda["ms_per_step"]
        kda["flops_per_step"] = step_flops(kl) * kb
        kda["valu_tflops"] = kda["flops_per_step"] / (kda["ms_per_step"] * 1e-3) / 1e12
        kda["valu_frac"] = kda["valu_tflops"] / VALU_PEAK_TFLOPS
        if not args.no_refit:
            kda["refit_row_scales"] = side_run(dataclasses.replace(kl, row_mode=0), ksteps, Wm, K, kb,
                                               kda["ms_per_step"], "KDA layout, row scales refitted every step")
        if not args.no_uniform:
            ku = dataclasses.replace(kl, unit_bits=np.full_like(kl.unit_bits, 6), row_mode=2)
            kda["uniform_int6"] = side_run(ku, ksteps, Wm, K, kb, kda["ms_per_step"],
                                           "KDA gates, uniform INT6 with one absmax scale per tile")
            k6 = dataclasses.replace(kl, unit_bits=np.full_like(kl.unit_bits, 6))
            kda["all_rows_6bit"] = side_run(k6, ksteps, Wm, K, kb, kda["ms_per_step"],
                                            "KDA gates and calibrated row scales, every row 6-bit (the "
                                            "uniform-width kernel): what one width per head costs at this shape")
        del ksteps
        torch.cuda.empty_cache()
    split = None
    if not args.no_split:
        split = split_phase_run(lay, steps, Wm, K, B, total_ms / K)
    fp32 = None
    if not args.no_fp32_state:
        fp32 = side_run(dataclasses.replace(lay, unit_bits=np.full_like(lay.unit_bits, 32)), steps, Wm, K, B,
                        total_ms / K, "same shape, inputs and kernel; every head stored as binary32 (zero-loss rows)")
        fp32["speedup_packed_vs_fp32"] = fp32.pop("time_vs_headline")

    stream_ref = None if args.no_stream else stream_reference()

    per_req = step_bytes(lay)
    bytes_per_launch = per_req["total"] * B
    achieved = bytes_per_launch / avg_launch_s / 1e9
    flops_per_launch = step_flops(lay) * B
    tflops = flops_per_launch / avg_launch_s / 1e12
    hbm_frac, valu_frac = achieved / HBM_PEAK_GBS, tflops / VALU_PEAK_TFLOPS
    kh = kernel_hash()
    traffic = read_traffic(kh)
    updates = B * H * K / (total_ms * 1e-3)
    out = {
        "metric": "state updates/s (batch*heads per step) and HBM GB/s, 6-bit packed decode",
        "value": updates,
        "unit": "state updates/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "warmup_steps_run": warm["steps"],
        "warmup_ms": warm["ms"],
        "ms_per_step": total_ms / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded, drawn on device)",
        "config": {"workload": c["name"], "B": B, "H": H, "d_k": D, "d_v": D,
                   "gate": "per-head" if lay.gate_mode == 0 else "per-key-channel",
                   "bits": f"{c['avg_bits'] if 'avg_bits' in c else c['uniform_bits']}.0-bit nominal, "
                           f"FP16 pivot units counted inside", "storage": "packed int2-8 codes, fp16 scales and pivots",
                   "row_scales": "calibrated", "decode_steps": K},
        "hbm_gbs_algorithmic": achieved,
        "bytes_per_step": bytes_per_launch,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": hbm_frac, "traffic": traffic, "bytes_per_launch": bytes_per_launch,
                     "frac_of_copy": achieved / stream_ref["copy_gbs"] if stream_ref else None,
                     "valu": {"achieved": tflops, "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": valu_frac, "flops_per_launch": flops_per_launch,
                              "note": "algorithmic FP32 flops against the non-packed FP32 vector peak; "
                                      "the kernel's limiter is VALU issue (see profiles/)"},
                     "kernel": kernel_name(lay), "launch_us_avg": avg_launch_s * 1e6,
                     "event_pair_us_avg": float(launch_ms.mean()) * 1e3,
                     "launch_us_min": float(launch_ms.min()) * 1e3, "kernel_source_hash": kh},
        "repeats_ms_per_step": rep_ms,
        "median_ms_per_step": float(np.median(rep_ms)),
        "launch_us_median": float(np.median(launch_ms)) * 1e3,
        "cpu_baseline": cpu,
        "gpu_over_cpu": (updates / cpu["value"]) if cpu else None,
        "refit_row_scales": refit,
        "uniform_tile_scale": uniform,
        "split_phase": split,
        "kda_layout": kda,
        "fp32_state": fp32,
        "stream_reference": stream_ref,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
