"""Benchmark: fused linear cross-entropy forward + backward on one MI355X.

One step = one flce_fwd_bwd call over one batch (row compaction, the chunk
loop of logits GEMM -> softmax-gradient -> grad_input GEMM -> grad_weight
GEMM, loss reduction).  Default workload: the Llama-3-8B lm_head shape,
bf16, BT 8192, H 4096, V 128256, all rows labelled, mean, fp32 grad_weight,
chunk_size 2048.  Reported under "extra": the 256-row chunk of that shape,
masked SFT at labelled shares 100/75/50/10 %, the long-sequence shape at
chunk 256 for BT 8192 and 32768, and the fp32 same-dtype sweep.  Inputs are seeded synthetic tensors already resident in HBM
when the timed region starts.

Prints one JSON line.  ``value`` = tokens/s of the whole job (BT x steps /
elapsed).  ``roofline`` is for the dominant kernel, with its average launch
duration measured by HIP events on the stream it runs on, over the timed
steps; only that kernel is bracketed by events there.  The same steps are
also run with no kernel events (``ms_per_step_unbracketed``: each pair of
events costs about 12 us of stream time), and with every kernel bracketed
for the per-kernel table in ``detail``.
``cpu_baseline`` times the fp64 oracle on a bounded sample of rows of
the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}  # MI355X dense
HBM_PEAK_GBS = 8000.0
METRIC = "FLCE fwd+bwd tokens/sec + % bf16 MFMA peak @BT=8192,H=4096,V=128256"

WORKLOADS = {
    # name: BT, H, V, dtype, accum, reduction, chunk, labelled share
    "llama3_8b_lm_head": dict(BT=8192, H=4096, V=128256, dtype="bf16", accum="f32",
                              reduction="mean", chunk=2048, share=1.0, seed=1001),
    "llama3_8b_lm_head_c256": dict(BT=8192, H=4096, V=128256, dtype="bf16", accum="f32",
                                   reduction="mean", chunk=256, share=1.0, seed=1001),
    "same_dtype_sweep_bf16": dict(BT=16384, H=4096, V=32000, dtype="bf16", accum="same",
                                  reduction="mean", chunk=0, share=1.0, seed=1002),
    "same_dtype_sweep_f16": dict(BT=16384, H=4096, V=32000, dtype="f16", accum="same",
                                 reduction="mean", chunk=0, share=1.0, seed=1002),
    "same_dtype_sweep_f32": dict(BT=16384, H=4096, V=32000, dtype="f32", accum="same",
                                 reduction="mean", chunk=0, share=1.0, seed=1002),
    "long_seq_8k_c256": dict(BT=8192, H=5376, V=262144, dtype="bf16", accum="same",
                             reduction="mean", chunk=256, share=1.0, seed=1003),
    "long_seq_8k_default": dict(BT=8192, H=5376, V=262144, dtype="bf16", accum="same",
                                reduction="mean", chunk=0, share=1.0, seed=1003),
    "long_seq_32k_c256": dict(BT=32768, H=5376, V=262144, dtype="bf16", accum="same",
                              reduction="mean", chunk=256, share=1.0, seed=1003),
    "long_seq_32k_default": dict(BT=32768, H=5376, V=262144, dtype="bf16", accum="same",
                                 reduction="mean", chunk=0, share=1.0, seed=1003),
    **{f"masked_sft_{int(s * 100)}_{mode}": dict(BT=8192, H=2048, V=151936, dtype="bf16",
                                                 accum="same", reduction="sum", chunk=0, share=s,
                                                 seed=1004, frozen=(mode == "frozen"))
       for s in (1.0, 0.75, 0.5, 0.1) for mode in ("trained", "frozen")},
    # reduction none: a per-token upstream gradient in [0.5, 1.5), NaN at ignored rows
    **{f"masked_sft_{int(s * 100)}_{mode}_none": dict(BT=8192, H=2048, V=151936, dtype="bf16",
                                                      accum="same", reduction="none", chunk=0,
                                                      share=s, seed=1004,
                                                      frozen=(mode == "frozen"))
       for s in (1.0, 0.75, 0.5, 0.1) for mode in ("trained", "frozen")},
    # the same, as 8 packed sequences of 1024 tokens, each prompt-first
    **{f"masked_sft_packed_{int(s * 100)}_{mode}": dict(BT=8192, H=2048, V=151936, dtype="bf16",
                                                        accum="same", reduction="sum", chunk=0,
                                                        share=s, seed=1004, seq_len=1024,
                                                        frozen=(mode == "frozen"))
       for s in (0.75, 0.5, 0.1) for mode in ("trained", "frozen")},
}


# Measured with the headline workload by default: the 256-row chunk of the
# same shape, the ignored-token speed-up at each labelled share (trained
# weight; PR #1554, Summary: about 1 / labelled share faster), the 256-row
# chunk at BT 8192 and 32768 (PR #1439, Details: the 256-row slab is flat in
# BT), and the fp32 same-dtype sweep (issue #1323, comparison table).
DEFAULT_EXTRA = ["llama3_8b_lm_head_c256", "masked_sft_100_trained", "masked_sft_75_trained",
                 "masked_sft_50_trained", "masked_sft_10_trained", "long_seq_8k_c256",
                 "long_seq_32k_c256", "same_dtype_sweep_f32"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="llama3_8b_lm_head", choices=sorted(WORKLOADS))
    p.add_argument("--extra", default=",".join(DEFAULT_EXTRA),
                   help="comma-separated extra workloads reported under 'extra' ('' for none)")
    p.add_argument("--cpu-rows", type=int, default=256, help="rows in the oracle's timed sample")
    p.add_argument("--chunk-sweep", default="",
                   help="comma-separated chunk sizes (0: the MI355X default policy): time the "
                        "workload at each and print one JSON line with the curve, then exit")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--protocol", default="",
                   help="comma-separated workloads, or 'all': time them together, one step "
                        "each per round in a seeded random order (--steps rounds), with the "
                        "peak transient memory of each in two isolated samples, print one "
                        "{\"protocol\": ...} line and exit")
    p.add_argument("--protocol-seed", type=int, default=1234)
    p.add_argument("--sensor-seconds", type=float, default=1.5,
                   help="after each workload's timed steps, run it untimed this long while "
                        "reading the GPU's clock, temperature and power (0: skip)")
    p.add_argument("--autograd", action="store_true",
                   help="time the differentiable path instead (forward + loss.backward() "
                        "through fused_linear_cross_entropy, weight-dtype dW) and print "
                        "one {\"autograd\": ...} line")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the probes of what the chip sustains by itself (bf16 MFMA loop "
                        "with random and with zero operands, HBM read stream, device copy)")
    p.add_argument("--zero-operands", action="store_true",
                   help="diagnostic: run the workload with X and W zeroed, so that the MFMA "
                        "multipliers do not toggle and the power limit does not lower the "
                        "clock; the line is marked as such and is not a benchmark result")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run plain 1 GiB device copies (reference for HBM byte counters)")
    p.add_argument("--record-traffic", nargs=4, metavar=("KERNEL", "WORKLOAD", "FETCH_CSV",
                                                          "WRITE_CSV"),
                   help="write profiles/KERNEL_WORKLOAD.traffic.txt from FETCH_SIZE and "
                        "WRITE_SIZE collections that include --copy-calibration, and exit")
    p.add_argument("--summarize-profile", nargs="+", metavar="CSV",
                   help="print a text summary of rocprofv3 csv output (kernel stats, or "
                        "FETCH_SIZE / WRITE_SIZE counter collections) and exit")
    p.add_argument("--rates", metavar="JSON",
                   help="with --summarize-profile: also tabulate the per-kernel achieved "
                        "rates from the bench JSON line the profiled run printed")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


_HOST = {}


def make_inputs(cfg, dev):
    """Seeded host inputs of a workload and their device copies.  X, W and the
    targets are cached separately on the host (workloads that differ only in
    BT, the labelled share or the chunk size share them), only the last
    workload's device copies are kept."""
    import synthetic_inputs as si
    BT, H, V, dt, seed = cfg["BT"], cfg["H"], cfg["V"], cfg["dtype"], cfg["seed"]
    t0 = time.perf_counter()
    kx, kw = ("X", BT, H, dt, seed), ("W", V, H, dt, seed)
    kt = ("t", BT, V, seed, cfg["share"], cfg.get("seq_len", BT))
    keep = {kx, kw, kt}
    for k in [k for k in _HOST if k not in keep and k[0] != "W"]:
        del _HOST[k]
    if kx not in _HOST:
        log(f"generating X [{BT}, {H}] {dt}")
        _HOST[kx] = si.make_x(BT, H, dt, seed)
    if kw not in _HOST:
        for k in [k for k in _HOST if k[0] == "W"]:
            del _HOST[k]
        log(f"generating W [{V}, {H}] {dt}")
        _HOST[kw] = si.make_w(V, H, dt, seed)
    if kt not in _HOST:
        share = cfg["share"]
        if share >= 1.0:
            _HOST[kt] = si.make_targets(BT, V, seed)
        else:
            _HOST[kt] = si.make_targets(BT, V, seed, ignore="prompt_first", frac=1.0 - share,
                                        seq_len=cfg.get("seq_len", BT))
    host = (_HOST[kx], _HOST[kw], _HOST[kt])
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
    return host, tuple(h.to(dev) for h in host)


def prepare(cfg, dev, host_dev=None):
    """Inputs, outputs and the library call of one workload; the workspace is
    passed to each call, so that its allocation can be measured."""
    import types
    import torch
    import linear_cross_entropy_chunked_amd as pkg
    import synthetic_inputs as si
    BT, H, V = cfg["BT"], cfg["H"], cfg["V"]
    host, (X, W, t) = host_dev if host_dev is not None else make_inputs(cfg, dev)
    dt = {"bf16": pkg.BF16, "f16": pkg.F16, "f32": pkg.F32}[cfg["dtype"]]
    adt = pkg.F32 if cfg["accum"] == "f32" else dt
    frozen = bool(cfg.get("frozen", False))
    red = pkg.REDUCTIONS[cfg["reduction"]]
    tdt = {pkg.F32: torch.float32, pkg.F16: torch.float16, pkg.BF16: torch.bfloat16}
    loss = torch.empty(BT if red == pkg.NONE else 1, dtype=torch.float32, device=dev)
    gout = (si.make_grad_output(host[2], "none", cfg["seed"]).to(dev) if red == pkg.NONE
            else None)
    dX = torch.empty_like(X)
    dW = None if frozen else torch.empty(V, H, dtype=tdt[adt], device=dev)
    wsb = pkg.flce_workspace_bytes(BT, H, V, dt, cfg["chunk"], 1)
    stream = torch.cuda.current_stream(dev)
    st = pkg.FlceStats()

    def call(ws):
        rc = pkg.flce_fwd_bwd(X.data_ptr(), W.data_ptr(), t.data_ptr(), BT, H, V, dt, -100, red,
                              cfg["chunk"], 1, adt, int(frozen), 0,
                              None if gout is None else gout.data_ptr(), loss.data_ptr(),
                              dX.data_ptr(), None if frozen else dW.data_ptr(), ws.data_ptr(),
                              wsb, stream.cuda_stream, st)
        if rc != 0:
            raise pkg.FlceError(rc, "flce_fwd_bwd")
    return types.SimpleNamespace(host=host, call=call, wsb=wsb, st=st, stream=stream,
                                 frozen=frozen, flops_per_row=(4 if frozen else 6) * H * V)


def run_workload(name, cfg, steps, warmup, dev, host_dev=None, sensor_s=0.0):
    import torch
    import linear_cross_entropy_chunked_amd as pkg
    BT, H, V = cfg["BT"], cfg["H"], cfg["V"]
    p = prepare(cfg, dev, host_dev)
    host, st, stream, frozen = p.host, p.st, p.stream, p.frozen
    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    wsb = p.wsb
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def step():
        p.call(ws)

    log(f"{name}: {warmup} warmup step(s)")
    # The warmup is profiled to find the kernel that dominates a step.  The
    # timed steps bracket only that kernel with HIP events, for its launch
    # duration.  Each pair of events adds about 12 us of stream time (at 64
    # chunks that is 0.8 ms per step for one kernel kind, 4 ms for all six),
    # so the same steps are also run with no kernel events at all
    # (ms_per_step_unbracketed), and once more with every kernel bracketed for
    # the per-kernel table.
    pkg.flce_profile_begin()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    wprof = pkg.flce_profile_end()
    dominant = max(wprof, key=lambda k: wprof[k][1]) if any(v[0] for v in wprof.values()) \
        else "dw_gemm"
    log(f"{name}: {steps} timed step(s), events around {dominant}")
    # per-step HIP events on the library's stream, for the step-time spread
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    pkg.flce_profile_begin_kinds([dominant])
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    pct = lambda q: step_ms[min(len(step_ms) - 1, int(round(q * (len(step_ms) - 1))))]
    tprof = pkg.flce_profile_end()[dominant]
    log(f"{name}: {steps} step(s) with no kernel events")
    ev[0].record(stream)
    for i in range(steps):
        step()
    ev[1].record(stream)
    torch.cuda.synchronize()
    plain_ms = ev[0].elapsed_time(ev[1]) / steps
    log(f"{name}: {steps} step(s) with every kernel bracketed")
    pkg.flce_profile_begin()
    t1 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    profiled_ms = (time.perf_counter() - t1) / steps * 1e3
    prof = pkg.flce_profile_end()
    sensors = None
    if sensor_s > 0:
        # untimed: the same steps for about sensor_s seconds while the sampler reads the chip
        s = GpuSensors(dev.index or 0).start()
        t1 = time.perf_counter()
        while time.perf_counter() - t1 < sensor_s:
            step()
        torch.cuda.synchronize()
        sensors = s.stop()
        sensors["window"] = (f"untimed steps of the same workload for {sensor_s:.1f} s right "
                             f"after the timed region")
    peak_transient = torch.cuda.max_memory_allocated(dev) - mem0
    del ws
    n_lab = st.n_valid
    flops = (4 if frozen else 6) * n_lab * H * V
    ms = elapsed / steps * 1e3
    res = dict(
        workload=name, BT=BT, H=H, V=V, dtype=cfg["dtype"], accum_dtype=cfg["accum"],
        reduction=cfg["reduction"], frozen_weight=frozen, labelled_share=cfg["share"],
        seq_len=cfg.get("seq_len", BT), chunk_size=st.chunk_size, chunks_run=st.chunks_run, dx_splits=st.dx_splits,
        n_valid=n_lab, ms_per_step=ms, tokens_per_s=BT * steps / elapsed,
        ms_per_step_unbracketed=plain_ms,
        step_ms_p20_p50_p80=[pct(0.2), pct(0.5), pct(0.8)],
        algorithmic_tflops=flops / (ms * 1e-3) / 1e12,
        mfma_frac=flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[cfg["dtype"]],
        workspace_bytes=wsb, peak_transient_bytes=int(peak_transient),
        timed_kernel=dict(name=dominant, launches=tprof[0] // steps,
                          ms_per_launch=(tprof[1] / tprof[0] if tprof[0] else 0.0),
                          ms_per_step=tprof[1] / steps,
                          measured_in=f"{steps} steps right after the timed ones, with HIP events "
                                f"around this kernel only"),
        kernels={k: dict(launches=v[0] // steps, ms_per_launch=(v[1] / v[0] if v[0] else 0.0),
                         ms_per_step=v[1] / steps)
                 for k, v in prof.items() if v[0]},
        kernels_pass=(f"{steps} further steps with every kernel bracketed by HIP events "
                      f"({profiled_ms:.3f} ms per step)"),
        gpu_sensors=sensors,
    )
    return res, host


def kernel_work(kind, res, cfg):
    """Algorithmic work of one average launch of a kernel kind: (flops, HBM bytes).

    Per chunk of r labelled rows (r = n_valid / chunks_run on average),
    s = operand itemsize, a = grad_weight itemsize:
      logits_gemm   2 r H V flops; W V H s + rows r H s + slab r V s
      softmax_grad  slab read + write 2 r V s (+ the block maxima, 8 r V / 64)
      dx_gemm       2 r H V flops; W V H s + G r V s + dX rows r H s
      dx_reduce     split partials S r H 4 + dX rows r H s
      dw_gemm       2 r H V flops; G r V s + gathered rows r H s + dW written
                    once per call and read-modified-written by the later chunks
      gather_rows   X rows r H s read + the transposed copy r H s written
      mask_scan     targets 8 BT + row index 4 n_valid
      zero_ignored_rows  dX rows of the ignored rows (BT - n_valid) H s
      loss_finalize per-row losses 4 n_valid
    """
    H, V, BT = res["H"], res["V"], res["BT"]
    n, chunks = res["n_valid"], max(res["chunks_run"], 1)
    r = n / chunks
    s = 4 if cfg["dtype"] == "f32" else 2
    a = 4 if cfg["accum"] == "f32" else s
    if kind == "logits_gemm":
        return 2.0 * r * H * V, V * H * s + r * H * s + r * V * s
    if kind == "softmax_grad":
        return 0.0, 2.0 * r * V * s + 8.0 * r * V / 64
    if kind == "dx_gemm":
        return 2.0 * r * H * V, V * H * s + r * V * s + r * H * s
    if kind == "dx_reduce":
        return 0.0, res["dx_splits"] * r * H * 4 + r * H * s
    if kind == "dw_gemm":
        return 2.0 * r * H * V, r * V * s + r * H * s + V * H * a * (2.0 * chunks - 1) / chunks
    if kind == "gather_rows":
        return 0.0, 2.0 * r * H * s
    if kind == "mask_scan":
        return 0.0, 8.0 * BT + 4.0 * n
    if kind == "zero_ignored_rows":
        return 0.0, (BT - n) * H * s
    if kind == "loss_finalize":
        return 0.0, 4.0 * n
    return None


def kernel_rates(res, cfg):
    """Achieved rate of every kernel kind of a step against MI355X peak, from
    the per-kernel event table: HBM GB/s for all, MFMA TFLOP/s for the GEMMs,
    and which of the two rooflines bounds the kernel."""
    out = {}
    for kind, k in res["kernels"].items():
        w = kernel_work(kind, res, cfg)
        if w is None or not k["ms_per_launch"]:
            continue
        flops, byts = w
        sec = k["ms_per_launch"] * 1e-3
        e = dict(us_per_launch=k["ms_per_launch"] * 1e3, launches_per_step=k["launches"],
                 hbm_gbs=byts / sec / 1e9, hbm_frac=byts / sec / 1e9 / HBM_PEAK_GBS,
                 algorithmic_bytes=byts)
        if flops:
            peak = MFMA_PEAK_TFLOPS[cfg["dtype"]]
            e.update(tflops=flops / sec / 1e12, mfma_frac=flops / sec / 1e12 / peak,
                     algorithmic_flops=flops)
            e["bound"] = "mfma" if flops / (peak * 1e12) >= byts / (HBM_PEAK_GBS * 1e9) else "hbm"
        else:
            e["bound"] = "hbm"
        out[kind] = e
    return out


def roofline(res, cfg):
    """Roofline figures of the dominant kernel of one step, timed in the timed
    steps: against the MFMA peak when its algorithmic flops take longer at peak
    than its algorithmic bytes at 8 TB/s, else against HBM bandwidth."""
    k = res["timed_kernel"]
    name = k["name"]
    flops, byts = kernel_work(name, res, cfg)
    sec = k["ms_per_launch"] * 1e-3
    rows = res["n_valid"] / max(res["chunks_run"], 1)
    peak_f = MFMA_PEAK_TFLOPS[cfg["dtype"]]
    if flops and flops / (peak_f * 1e12) >= byts / (HBM_PEAK_GBS * 1e9):
        achieved = flops / sec / 1e12
        return dict(kernel=name, bound="mfma", achieved=achieved, peak=peak_f, unit="TFLOP/s",
                    frac=achieved / peak_f, traffic=None, rows_per_launch=rows,
                    hbm_frac_of_algorithmic_bytes=byts / sec / 1e9 / HBM_PEAK_GBS,
                    work_per_launch=f"2*c*H*V flops = {flops:.4g} (c={rows:g} rows on average)")
    achieved = byts / sec / 1e9
    out = dict(kernel=name, bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
               frac=achieved / HBM_PEAK_GBS, traffic=None, rows_per_launch=rows,
               work_per_launch=f"algorithmic bytes = {byts:.4g} (c={rows:g} rows on average)")
    if flops:
        out["mfma_frac"] = flops / sec / 1e12 / peak_f
    return out


def ceilings(dev):
    """What the chip sustains by itself, from the probe library (include/flce_probe.h):
    bf16 MFMA throughput of a loop with no memory traffic, with random operands (the
    multipliers toggle as in the GEMMs, and the power limit sets the clock) and with
    zero operands (no toggling); the HBM read rate of a plain streaming read of 2 GiB;
    a 1 GiB device copy (read + write).  Each is timed with HIP events on the current
    stream over several launches after one untimed launch."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "linear_cross_entropy_chunked_amd", "libflce_probe.so"))
    for f in (lib.flce_probe_mfma_loop, lib.flce_probe_mfma16_loop):
        f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                      ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.flce_probe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                           ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    st = torch.cuda.current_stream(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count

    def timed(launch, reps):
        launch()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            launch()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    def check(rc, what):
        if rc:
            raise RuntimeError(f"{what}: status {rc}")

    blocks, iters = 4 * cus, 4000
    sink = torch.empty(blocks * lib.flce_probe_mfma_threads(), dtype=torch.float32, device=dev)
    gen = torch.Generator().manual_seed(20240611)
    rnd = (torch.randn(8 << 20, generator=gen) * 0.05).to(torch.bfloat16).to(dev)
    flops = blocks * 8 * iters * 32 * 2 * 32 * 32 * 16  # the same for both shapes
    out = {}
    for loop, key in ((lib.flce_probe_mfma_loop, "mfma_loop"),
                      (lib.flce_probe_mfma16_loop, "mfma16_loop")):
        for kind, ops in (("random", rnd), ("zero", torch.zeros_like(rnd))):
            sec = timed(lambda: check(loop(
                ops.data_ptr(), ops.numel() * 2, sink.data_ptr(), sink.numel(), blocks, iters,
                st.cuda_stream), key), 12)
            out[f"{key}_bf16_{kind}_tflops"] = flops / sec / 1e12
    del rnd, sink
    nbytes = 2 << 30
    sblocks = nbytes >> 20  # 1 MiB per workgroup
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    ssink = torch.empty(sblocks * lib.flce_probe_stream_threads() * 16, dtype=torch.uint8,
                        device=dev)
    sec = timed(lambda: check(lib.flce_probe_read_stream(
        src.data_ptr(), nbytes, ssink.data_ptr(), ssink.numel(), sblocks, st.cuda_stream),
        "flce_probe_read_stream"), 10)
    out["hbm_read_stream_gbs"] = nbytes / sec / 1e9
    del src, ssink
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    sec = timed(lambda: b.copy_(a), 10)
    out["hbm_copy_gbs"] = 2 * COPY_BYTES / sec / 1e9
    del a, b
    torch.cuda.empty_cache()
    out["how"] = (f"probe library: {blocks} workgroups x 8 waves x {iters} iterations of 32 "
                  f"independent v_mfma_f32_32x32x16_bf16 (mfma16: 64 of "
                  f"v_mfma_f32_16x16x32_bf16) on register operands (random: "
                  f"N(0, 0.05) in bf16; zero: all zero), timed over 12 launches; a read of "
                  f"2 GiB in {sblocks} contiguous 1 MiB segments, one per workgroup of 256, "
                  f"16 B per lane, 4 loads in flight per lane, over 10 launches; torch copy "
                  f"of 1 GiB (2 GiB moved) over 10 launches")
    return out


# Which 16-bit GEMM launches run on 16x16x32 MFMAs (flce_gemm.hip): grad_input
# from DX_SUB16_ROWS rows per chunk; logits and grad_weight on their large tiles,
# i.e. more than LARGE_TILE_ROWS rows per chunk (logits also needs V >= 1024,
# grad_weight H >= 256).  Everything else runs on 32x32x16.
DX_SUB16_ROWS = 1024
LARGE_TILE_ROWS = 128


def runs_sub16(kernel, rows, H=None, V=None):
    if kernel == "dx_gemm":
        return rows >= DX_SUB16_ROWS
    if kernel == "logits_gemm":
        return rows > LARGE_TILE_ROWS and (V is None or V >= 1024)
    if kernel == "dw_gemm":
        return rows > LARGE_TILE_ROWS and (H is None or H >= 256)
    return False


def add_ceiling(rl, ceil, dtype, H=None, V=None):
    """The dominant kernel's rate against what the chip sustains by itself: the
    MFMA loop of the shape the kernel runs on (chosen by the average rows per
    launch), or the HBM read stream."""
    if not ceil:
        return
    if rl["bound"] == "mfma" and dtype in ("bf16", "f16"):
        sub16 = runs_sub16(rl.get("kernel"), rl.get("rows_per_launch", 0), H, V)
        key, shape = ("mfma16_loop", "16x16x32") if sub16 else ("mfma_loop", "32x32x16")
        c = ceil[f"{key}_bf16_random_tflops"]
        rl["ceiling"] = dict(value=c, unit="TFLOP/s", kind=f"bf16 {shape} MFMA loop, random operands")
        rl["frac_of_ceiling"] = rl["achieved"] / c
    elif rl["bound"] == "hbm":
        c = ceil["hbm_read_stream_gbs"]
        rl["ceiling"] = dict(value=c, unit="GB/s", kind="HBM read stream")
        rl["frac_of_ceiling"] = rl["achieved"] / c


def cpu_baseline(host, cfg, rows):
    """fp64 loop oracle on the first `rows` rows of the same batch (full H and V)."""
    import numpy as np
    import oracle
    X, W, t = host
    Xs, ts = X[:rows], t[:rows]
    log(f"cpu baseline: widening inputs, then {rows} rows through the oracle")
    Xd, Wd = oracle.widen(Xs), oracle.widen(W)
    t0 = time.perf_counter()
    oracle.flce(Xd, Wd, ts, reduction=cfg["reduction"], frozen=bool(cfg.get("frozen", False)))
    dt = time.perf_counter() - t0
    return dict(value=rows / dt, unit="tokens/s", cores=oracle.threads(), kind="oracle",
                sample=f"first {rows} of {cfg['BT']} rows of the same batch through the fp64 "
                       f"loop oracle (forward + backward, full H={cfg['H']}, V={cfg['V']}); "
                       f"{dt:.1f} s; widening the inputs to fp64 is not timed; host: "
                       f"{host_description()}")


class GpuSensors:
    """Shader clock, hotspot temperature and socket power of one GPU, read through the
    ROCm SMI library (amdsmi) every `interval` s from a background thread.

    Used over an untimed run of the same steps right after the timed region, so that
    the readings describe the chip under the measured load without touching the timed
    numbers.  Anything the platform does not expose is reported as unreadable."""

    def __init__(self, torch_index=0, interval=0.05):
        import threading
        self.interval, self.idx = interval, torch_index
        self.samples, self.error = [], None
        self._stop, self._ready = threading.Event(), threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _handle(self, amdsmi):
        import torch
        handles = amdsmi.amdsmi_get_processor_handles()
        p = torch.cuda.get_device_properties(self.idx)
        bus = getattr(p, "pci_bus_id", None)
        if bus is not None:
            want = f"{getattr(p, 'pci_domain_id', 0):04x}:{bus:02x}:{getattr(p, 'pci_device_id', 0):02x}"
            for h in handles:
                if amdsmi.amdsmi_get_gpu_device_bdf(h).lower().startswith(want):
                    return h
        if len(handles) == 1:
            return handles[0]
        raise RuntimeError(f"cannot match device {self.idx} among {len(handles)} SMI handles")

    def _read(self, amdsmi, h):
        def num(v):
            return float(v) if isinstance(v, (int, float)) else None
        clk = num(amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX).get("clk"))
        temp = None
        for kind in ("HOTSPOT", "JUNCTION", "EDGE"):
            t = getattr(amdsmi.AmdSmiTemperatureType, kind, None)
            if t is None:
                continue
            try:
                temp = num(amdsmi.amdsmi_get_temp_metric(
                    h, t, amdsmi.AmdSmiTemperatureMetric.CURRENT))
            except Exception:
                temp = None
            if temp is not None:
                break
        pw = amdsmi.amdsmi_get_power_info(h)
        power = next((num(pw.get(k)) for k in ("current_socket_power", "average_socket_power",
                                                 "socket_power") if num(pw.get(k))), None)
        return clk, temp, power

    def _run(self):
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            h = self._handle(amdsmi)
            while True:
                self.samples.append(self._read(amdsmi, h))
                self._ready.set()
                if self._stop.wait(self.interval):
                    break
        except Exception as e:  # no SMI access: report it, never fail the bench
            self.error = f"{type(e).__name__}: {e}"
        finally:
            self._ready.set()

    def start(self):
        self._thread.start()
        self._ready.wait(10.0)
        return self

    def stop(self):
        self._stop.set()
        if self._thread.ident is not None:
            self._thread.join(5.0)
        if not self.samples:
            return dict(readable=False, reason=self.error or "no sample within 10 s")

        def spread(i):
            v = sorted(s[i] for s in self.samples if s[i] is not None)
            return [v[0], v[len(v) // 2], v[-1]] if v else None
        return dict(readable=True, samples=len(self.samples),
                    gfx_clock_mhz_min_median_max=spread(0),
                    hotspot_temp_c_min_median_max=spread(1),
                    socket_power_w_min_median_max=spread(2), error=self.error)


def host_description() -> str:
    """CPU model and RAM of the machine the oracle runs on (Linux /proc)."""
    model, ram = "unknown CPU", "unknown RAM"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal"):
                ram = f"{int(line.split()[1]) / 2**20:.0f} GiB RAM"
                break
    except OSError:
        pass
    return f"{model}, {ram}"


# ---------------------------------------------------------------- profiling
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["linear_cross_entropy_chunked_amd/csrc/flce_gemm.hip",
                  "linear_cross_entropy_chunked_amd/csrc/flce_rowops.hip",
                  "linear_cross_entropy_chunked_amd/csrc/flce_device.hpp"]
COPY_BYTES = 1 << 30


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: comments and whitespace are dropped, so
    that recorded counter traffic stays valid across edits that change no code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def copy_calibration(dev):
    """Plain device copies of a known size: 1 GiB read + 1 GiB written per copy."""
    import torch
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def summarize_profile(paths):
    """Text summary of rocprofv3 csv files (kernel_stats or counter_collection)."""
    import csv
    import collections
    for path in paths:
        rows = list(csv.DictReader(open(path)))
        print(f"## {os.path.basename(path)}")
        if rows and "AverageNs" in rows[0]:
            print(f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'total_ms':>10s} {'pct':>6s}")
            for r in rows:
                print(f"{r['Name'][:70]:70s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e3:10.1f} "
                      f"{float(r['TotalDurationNs'])/1e6:10.2f} {float(r['Percentage']):6.2f}")
        else:
            agg = collections.defaultdict(list)
            for r in rows:
                agg[(r["Kernel_Name"][:70], r["Counter_Name"])].append(float(r["Counter_Value"]))
            print(f"{'kernel':70s} {'counter':12s} {'dispatches':>10s} {'avg_per_dispatch':>18s}")
            for (k, c), v in sorted(agg.items()):
                print(f"{k:70s} {c:12s} {len(v):10d} {sum(v)/len(v):18.1f}")
        print()


def summarize_rates(path):
    """Per-kernel achieved rates (HIP events in the profiled run) of every
    workload in a bench JSON line, against MI355X peak."""
    line = [l for l in open(path) if l.startswith("{")][-1]
    out = json.loads(line)
    runs = [(out["config"]["workload"], out["detail"])] + list(out.get("extra", {}).items())
    for name, res in runs:
        print(f"## achieved rates, {name}: chunk {res['chunk_size']}, {res['chunks_run']} "
              f"chunks, {res['n_valid']} labelled rows, {res['ms_per_step']:.3f} ms per step")
        print(f"{'kernel':18s} {'launches':>8s} {'us/launch':>10s} {'bound':>5s} "
              f"{'GB/s':>9s} {'of 8 TB/s':>9s} {'TFLOP/s':>9s} {'of peak':>8s}")
        for k, e in sorted(res.get("kernel_rates", {}).items(),
                           key=lambda kv: -kv[1]["us_per_launch"] * kv[1]["launches_per_step"]):
            tf = f"{e['tflops']:9.1f} {100 * e['mfma_frac']:7.1f}%" if "tflops" in e else ""
            print(f"{k:18s} {e['launches_per_step']:8d} {e['us_per_launch']:10.2f} "
                  f"{e['bound']:>5s} {e['hbm_gbs']:9.1f} {100 * e['hbm_frac']:8.1f}% {tf}")
        print()


def _per_dispatch(path, match):
    import csv
    return [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
            if match(r["Kernel_Name"])]


def record_traffic(kernel, workload, fetch_csv, write_csv):
    """Calibrated HBM bytes per launch of one kernel kind, from counter collections.

    FETCH_SIZE and WRITE_SIZE are in KiB per dispatch.  Each is scaled by
    (bytes a 1 GiB plain copy really moves) / (what the counter reports for
    that copy), taken from the --copy-calibration dispatches of the same run.
    """
    names = {"logits_gemm": "logits_kernel", "dx_gemm": "dx_kernel", "dw_gemm": "dw_kernel",
             "softmax_grad": "softmax_kernel", "gather_rows": "gather_t_kernel",
             "mask_scan": "mask_scan_kernel", "dx_reduce": "dx_reduce_kernel"}
    kname = names[kernel]
    copy_f = [v for v in _per_dispatch(fetch_csv, lambda n: "copyBuffer" in n) if v > 1e5]
    copy_w = [v for v in _per_dispatch(write_csv, lambda n: "copyBuffer" in n) if v > 1e5]
    ref_kib = COPY_BYTES / 1024
    f_scale = ref_kib / (sum(copy_f) / len(copy_f))
    w_scale = ref_kib / (sum(copy_w) / len(copy_w))
    kf = _per_dispatch(fetch_csv, lambda n: kname in n)
    kw = _per_dispatch(write_csv, lambda n: kname in n)
    fetch = sum(kf) / len(kf) * 1024 * f_scale
    write = sum(kw) / len(kw) * 1024 * w_scale
    path = os.path.join(PROFILES, f"{kernel}_{workload}.traffic.txt")
    with open(path, "w") as fh:
        fh.write(f"# HBM traffic per launch of {kernel} ({kname}), workload {workload}\n")
        fh.write("# from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE runs of:\n")
        fh.write(f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o fetch -- "
                 f"python bench.py --workload {workload} --steps 1 --warmup 1 "
                 f"--no-cpu-baseline --extra '' --sensor-seconds 0 --no-ceilings "
                 f"--copy-calibration\n")
        fh.write("#   (the same with --pmc WRITE_SIZE -o write)\n")
        fh.write("# counters are KiB per dispatch; each is scaled by the ratio of the bytes a\n")
        fh.write("# 1 GiB device copy moves to what the counter reports for it\n")
        fh.write(f"copy_fetch_kib_reported = {sum(copy_f) / len(copy_f):.1f}\n")
        fh.write(f"copy_write_kib_reported = {sum(copy_w) / len(copy_w):.1f}\n")
        fh.write(f"fetch_scale = {f_scale:.4f}\nwrite_scale = {w_scale:.4f}\n")
        fh.write(f"dispatches = {len(kf)}\n")
        fh.write(f"fetch_kib_per_dispatch = {sum(kf) / len(kf):.1f}\n")
        fh.write(f"write_kib_per_dispatch = {sum(kw) / len(kw):.1f}\n")
        fh.write(f"hbm_read_bytes_per_launch = {fetch:.6g}\n")
        fh.write(f"hbm_write_bytes_per_launch = {write:.6g}\n")
        fh.write(f"hbm_bytes_per_launch = {fetch + write:.6g}\n")
        fh.write(f"kernel_source_sha = {kernel_source_hash()}\n")
    print(open(path).read())


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch recorded from FETCH_SIZE / WRITE_SIZE counter runs, if current."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}.traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_hash():
        return None  # the kernel changed since the counters were taken
    return float(kv["hbm_bytes_per_launch"])


def autograd_bench(a, cfg, dev):
    """The differentiable path: loss = fused_linear_cross_entropy(...);
    loss.backward(), with dW accumulated in fp32 and returned in the weight dtype
    (the wrapper tail: the fp32 -> weight-dtype cast and the upstream scaling)."""
    import torch
    import linear_cross_entropy_chunked_amd as pkg
    host, (X, W, t) = make_inputs(cfg, dev)
    x = X.clone().requires_grad_(True)
    w = W.clone().requires_grad_(cfg.get("frozen", False) is False)
    accum = torch.float32 if cfg["accum"] == "f32" else None

    def step():
        x.grad = None
        w.grad = None
        loss = pkg.fused_linear_cross_entropy(x, w, t, reduction=cfg["reduction"],
                                              chunk_size=cfg["chunk"] or None,
                                              accum_dtype=accum)
        loss.backward()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / a.steps * 1e3
    # the per-kernel table from further steps (the events are kept out of the timed ones)
    pkg.flce_profile_begin()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    prof = pkg.flce_profile_end()
    wdt = w.grad.dtype if w.grad is not None else None
    # (backward runs on autograd's device thread, outside this thread's profile window)
    kernels = {k: dict(launches=v[0] // a.steps, ms_per_step=v[1] / a.steps)
               for k, v in prof.items() if v[0]}
    # the wrapper tail alone: the same scale/cast calls on tensors of the same sizes
    tail_ms = None
    if w.grad is not None and accum is not None and w.dtype != torch.float32:
        dw32 = torch.empty(w.shape, dtype=torch.float32, device=dev).normal_()
        dx = torch.empty_like(x)
        g = torch.ones(1, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for rep in range(3):
            e0.record()
            pkg.scale_cast(dw32, w.dtype, scale=g)
            pkg.scale_cast(dx, dx.dtype, scale=g, out=dx)
            e1.record()
            torch.cuda.synchronize()
            tail_ms = e0.elapsed_time(e1)
        del dw32, dx
    x.grad = None
    w.grad = None
    raw, _ = run_workload(a.workload, cfg, a.steps, a.warmup, dev, host_dev=(host, (X, W, t)))
    print(json.dumps({"autograd": {"workload": a.workload, "ms_per_step": ms,
                                   "tokens_per_s": cfg["BT"] / (ms * 1e-3),
                                   "raw_call_ms_per_step": raw["ms_per_step"],
                                   "wrapper_tail_ms": tail_ms,
                                   "weight_grad_dtype": str(wdt) if wdt is not None else None,
                                   "forward_kernels": kernels}}), flush=True)


PROTOCOL_WORKLOADS = [
    "llama3_8b_lm_head", "llama3_8b_lm_head_c256", "same_dtype_sweep_bf16",
    "same_dtype_sweep_f16", "same_dtype_sweep_f32", "long_seq_8k_c256", "long_seq_8k_default",
    "long_seq_32k_c256", "long_seq_32k_default",
    *[f"masked_sft_{p}_{m}" for m in ("trained", "frozen") for p in (100, 75, 50, 10)],
    *[f"masked_sft_{p}_{m}_none" for m in ("trained", "frozen") for p in (100, 75, 50, 10)],
    *[f"masked_sft_packed_{p}_{m}" for m in ("trained", "frozen") for p in (75, 50, 10)]]


def protocol(a, dev):
    """Every workload measured together: warmup steps for each, then rounds in
    which the workloads run in a seeded random order, one step each, timed with
    HIP events on the library's stream; the peak transient memory of each in two
    isolated samples (a fresh workspace allocated inside the measured window)."""
    import numpy as np
    import torch
    names = [n for n in a.protocol.split(",") if n] if a.protocol != "all" else PROTOCOL_WORKLOADS
    hosts, preps = {}, {}
    for n in names:
        cfg = WORKLOADS[n]
        key = tuple(cfg.get(k) for k in ("BT", "H", "V", "dtype", "seed", "share", "seq_len"))
        if key not in hosts:
            hosts[key] = make_inputs(cfg, dev)
        preps[n] = prepare(cfg, dev, hosts[key])
    wss = {n: torch.empty(p.wsb, dtype=torch.uint8, device=dev) for n, p in preps.items()}
    for n in names:
        for _ in range(a.warmup):
            preps[n].call(wss[n])
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(a.protocol_seed))
    samples = {n: [] for n in names}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    orders = []
    for r in range(a.steps):
        order = [names[i] for i in rng.permutation(len(names))]
        orders.append(order)
        for n in order:
            p = preps[n]
            e0.record(p.stream)
            p.call(wss[n])
            e1.record(p.stream)
            e1.synchronize()
            samples[n].append(e0.elapsed_time(e1))
        log(f"protocol round {r + 1}/{a.steps} done")
    del wss
    out = {}
    for n in names:
        p, cfg = preps[n], WORKLOADS[n]
        v = sorted(samples[n])
        q = lambda f: v[min(len(v) - 1, int(round(f * (len(v) - 1))))]
        mem = []
        for _ in range(2):
            torch.cuda.synchronize()
            m0 = torch.cuda.memory_allocated(dev)
            torch.cuda.reset_peak_memory_stats(dev)
            ws = torch.empty(p.wsb, dtype=torch.uint8, device=dev)
            p.call(ws)
            torch.cuda.synchronize()
            mem.append(int(torch.cuda.max_memory_allocated(dev) - m0))
            del ws
        med = q(0.5)
        flops = p.flops_per_row * p.st.n_valid
        out[n] = dict(step_ms_p20_p50_p80=[q(0.2), med, q(0.8)],
                      tokens_per_s_at_median=cfg["BT"] / (med * 1e-3),
                      mfma_frac_at_median=flops / (med * 1e-3) / 1e12
                      / MFMA_PEAK_TFLOPS[cfg["dtype"]],
                      chunk_size=p.st.chunk_size, chunks_run=p.st.chunks_run,
                      n_valid=p.st.n_valid, workspace_bytes=p.wsb,
                      peak_transient_bytes_two_samples=mem)
    print(json.dumps({"protocol": {"seed": a.protocol_seed, "warmup": a.warmup,
                                   "rounds": a.steps, "first_orders": orders[:2],
                                   "workloads": out}}), flush=True)


def chunk_sweep(a, cfg, dev):
    """Time one workload at several chunk sizes (same inputs); 0 = the MI355X policy."""
    import linear_cross_entropy_chunked_amd as pkg
    host = None
    rows = []
    adt = pkg.F32 if cfg["accum"] == "f32" else {"bf16": pkg.BF16, "f16": pkg.F16,
                                                 "f32": pkg.F32}[cfg["dtype"]]
    dt = {"bf16": pkg.BF16, "f16": pkg.F16, "f32": pkg.F32}[cfg["dtype"]]
    for c in [int(v) for v in a.chunk_sweep.split(",")]:
        policy = c == 0
        if policy:
            c = pkg.flce_chunk_size_mi355x(cfg["BT"], cfg["H"], cfg["V"], dt, adt,
                                           int(bool(cfg.get("frozen", False))), 0)
        ccfg = dict(cfg, chunk=c)
        res, host = run_workload(f"{a.workload}@{c}", ccfg, a.steps, a.warmup, dev,
                                 None if host is None else (host, tuple(h.to(dev) for h in host)))
        rows.append(dict(chunk=c, policy=policy, ms_per_step=res["ms_per_step"],
                         tokens_per_s=res["tokens_per_s"], mfma_frac=res["mfma_frac"],
                         workspace_bytes=pkg.flce_workspace_bytes(cfg["BT"], cfg["H"], cfg["V"],
                                                                  dt, c, 1),
                         kernels_ms_per_launch={k: round(v["ms_per_launch"], 4)
                                                for k, v in res["kernels"].items()}))
    print(json.dumps({"chunk_sweep": {"workload": a.workload, "steps": a.steps, "rows": rows}}),
          flush=True)


def extra_summaries(extras):
    """What the extra workloads show together: the ignored-token speed-up
    against 1 / labelled share (PR #1554, Summary), and the transient memory of
    a 256-row chunk at two sequence lengths (PR #1439, Details)."""
    out = {}
    base = extras.get("masked_sft_100_trained")
    if base:
        rows = []
        for sh in (0.75, 0.5, 0.1):
            e = extras.get(f"masked_sft_{int(sh * 100)}_trained")
            if e:
                rows.append(dict(labelled_share=sh, n_valid=e["n_valid"],
                                 chunks_run=e["chunks_run"],
                                 ms_per_step=e["ms_per_step_unbracketed"],
                                 speedup=base["ms_per_step_unbracketed"]
                                 / e["ms_per_step_unbracketed"],
                                 ideal_1_over_share=base["n_valid"] / e["n_valid"],
                                 chunk_ratio=base["chunks_run"] / e["chunks_run"]))
        out["ignored_token_speedup"] = dict(
            baseline_ms=base["ms_per_step_unbracketed"], rows=rows,
            timing="steps with no per-kernel events (ms_per_step_unbracketed)")
    a, b = extras.get("long_seq_8k_c256"), extras.get("long_seq_32k_c256")
    if a and b:
        out["flat_transient_c256"] = dict(
            bt_8192_peak_bytes=a["peak_transient_bytes"],
            bt_32768_peak_bytes=b["peak_transient_bytes"],
            bt_8192_workspace_bytes=a["workspace_bytes"],
            bt_32768_workspace_bytes=b["workspace_bytes"],
            workspace_difference_bytes=b["workspace_bytes"] - a["workspace_bytes"],
            row_index_and_loss_bytes=8 * (b["BT"] - a["BT"]),
            note="peak = max_memory_allocated - memory_allocated around a call whose workspace "
                 "is allocated inside the window (torch rounds that allocation up to 2 MiB); "
                 "the [256, V] slab and the other chunk buffers are the same at both BT, and "
                 "the workspace grows only by the int32 row index and fp32 per-row loss "
                 "(8 B per row)")
    return out


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {a.gpus}).", file=sys.stderr)
        sys.exit(2)
    if a.summarize_profile:
        summarize_profile(a.summarize_profile)
        if a.rates:
            summarize_rates(a.rates)
        return
    if a.record_traffic:
        record_traffic(*a.record_traffic)
        return
    import torch
    import linear_cross_entropy_chunked_amd as pkg
    pkg.load()
    dev = torch.device("cuda:0")
    if a.copy_calibration:
        log("copy calibration: 2 x 1 GiB device copies")
        copy_calibration(dev)
    if a.protocol:
        protocol(a, dev)
        return
    cfg = WORKLOADS[a.workload]
    if a.chunk_sweep:
        chunk_sweep(a, cfg, dev)
        return
    if a.autograd:
        autograd_bench(a, cfg, dev)
        return
    t_start = time.perf_counter()
    host_dev = None
    if a.zero_operands:
        host, (X, W, t) = make_inputs(cfg, dev)
        host_dev = (host, (torch.zeros_like(X), torch.zeros_like(W), t))
        del X, W
    main_res, host = run_workload(a.workload, cfg, a.steps, a.warmup, dev, host_dev=host_dev,
                                  sensor_s=a.sensor_seconds)
    del host_dev
    main_res["kernel_rates"] = kernel_rates(main_res, cfg)
    cpu = None
    if not a.no_cpu_baseline and not a.zero_operands:
        cpu = cpu_baseline(host, cfg, a.cpu_rows)
    del host
    extras = {}
    for name in [e for e in a.extra.split(",") if e and e != a.workload]:
        ecfg = WORKLOADS[name]
        res, _ = run_workload(name, ecfg, max(a.steps // 2, 2), a.warmup, dev,
                              sensor_s=a.sensor_seconds)
        erl = roofline(res, ecfg)
        erl["traffic"] = recorded_traffic(erl["kernel"], name)
        res["roofline"] = erl
        res["kernel_rates"] = kernel_rates(res, ecfg)
        extras[name] = res
        torch.cuda.empty_cache()
    summaries = extra_summaries(extras)
    ceil = None
    if not a.no_ceilings:
        log("ceilings: MFMA loop (random, zero operands), HBM read stream, device copy")
        ceil = ceilings(dev)
        for name, res in extras.items():
            add_ceiling(res["roofline"], ceil, WORKLOADS[name]["dtype"], WORKLOADS[name]["H"],
                        WORKLOADS[name]["V"])
    rl = roofline(main_res, cfg)
    rl["traffic"] = recorded_traffic(rl["kernel"], a.workload)
    sens = main_res["gpu_sensors"]
    if rl["bound"] == "mfma" and sens and sens.get("readable") and \
            sens["gfx_clock_mhz_min_median_max"]:
        # the published peak assumes 2.4 GHz; the same fraction at the clock the chip held
        mhz = sens["gfx_clock_mhz_min_median_max"][1]
        if mhz:
            rl["frac_at_measured_clock"] = rl["frac"] * 2400.0 / mhz
            rl["measured_clock_mhz"] = mhz
    add_ceiling(rl, ceil, cfg["dtype"], cfg["H"], cfg["V"])
    out = {
        "metric": METRIC,
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic" + (", X and W zeroed (diagnostic, not a benchmark result)"
                                if a.zero_operands else ""),
        "config": {"workload": a.workload, "BT": cfg["BT"], "H": cfg["H"], "V": cfg["V"],
                   "chunk_size": main_res["chunk_size"], "accum_dtype": cfg["accum"],
                   "reduction": cfg["reduction"], "labelled_share": cfg["share"],
                   "seq_len": main_res["seq_len"], "frozen_weight": main_res["frozen_weight"],
                   **({"operands": "zero"} if a.zero_operands else {})},
        "mfma_frac_of_peak": main_res["mfma_frac"],
        "algorithmic_tflops": main_res["algorithmic_tflops"],
        "roofline": rl,
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    if ceil is not None:
        out["ceilings"] = ceil
    out["detail"] = main_res
    out["summaries"] = summaries
    out["extra"] = extras
    out["wall_s"] = time.perf_counter() - t_start
    out["context"] = ("pages' figures on other hardware (not targets): BT 8192, H 4096, "
                      "V 128256 bf16 on H200, chunk 256: 53.039 ms; chunk 2048: 37.748 ms")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
