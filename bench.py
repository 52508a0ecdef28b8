"""Benchmark of the RSM mixer hot path on one MI355X.

A step is one rsm_forward_chunked call (route; then, per sequence segment, sparse decay,
chunk contractions, state scan and emit) over one batch of the 400M-scale layer workload: B=8, T=2048, Hh=8, M=64,
Dv=128, top-16, C=64, bf16 q/k/z/v, fp32 f/state/outputs.  Three input sets are rotated
so the ~154 MB working set cannot sit in the 256 MB last-level cache between steps.
The decode step (256 sequences x 16 heads, M64 Dv128 K16, prefill T=512) is timed in the
same run: 1024 back-to-back rsm_decode_step calls between two HIP events.  So are the
router / decay variants (softmax scores renormalised over the selected slots and one decay
rate per slot; with and without exploration noise on the logits) on both workloads.

Prints one JSON line.  Inputs are synthetic (seeded generator), already resident in HBM
when the timed region starts.  The benchmark runs on one GPU: `--gpus N` with N > 1 is refused.
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

METRIC = "RSM forward tokens/s (B8 T2048 M64) + decode-step µs; % HBM/MFMA roofline"
PEAK_HBM_GBS = 8000.0
COPY_BYTES = 256 << 20  # calibration copy: reads and writes this many bytes
# Sources of the forward kernels; the stored counter figures hold only for these bytes.
FWD_SOURCES = ["rsm_forward.hip", "rsm_route.hip", "rsm_route_row.h", "rsm_scan.h", "rsm_scan_args.h",
               "rsm_segstate.h", "rsm_scan_bf16_m64.hip", "rsm_device.h", "rsm_launch.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "forward_fwd_b8_t2048_traffic.txt")
# the forward configs besides the headline one (timed once each; parity cases in the tests)
CONFIG_NAMES = ("tiny_f32", "long_t32768", "sweep_dense", "sweep_swa", "sweep_topk")


def forward_bytes(B, T, Hh, M, Dv, es):
    """Algorithmic bytes of one forward: every input read once, outputs written once."""
    return (3 * B * T * Hh * M * es + B * T * Hh * Dv * es + B * T * Hh * 4
            + B * T * Hh * Dv * 4 + B * Hh * M * Dv * 4)


def decode_bytes(B, Hh, M, Dv, K, es):
    """Per step: full state read, K rows written back, inputs read, o written."""
    return (B * Hh * M * Dv * 4 + B * Hh * K * Dv * 4 + 3 * B * Hh * M * es + B * Hh * Dv * es
            + B * Hh * 4 + B * Hh * Dv * 4)


def variant_extra_bytes(rows, M):
    """Extra input bytes of the decode variant timed here: per-slot decay rates in place of
    one per token-head, and the fp32 noise on the logits."""
    return rows * (M - 1) * 4 + rows * M * 4


def forward_sources_sha256():
    h = hashlib.sha256()
    for name in FWD_SOURCES:
        with open(os.path.join(ROOT, "sparse_routed_slot_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per forward call from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (copy-calibrated), or None when the kernel sources changed since they were taken."""
    try:
        fields = dict(line.split(":", 1) for line in open(TRAFFIC_FILE) if ":" in line)
    except OSError:
        return None
    if fields.get("source_sha256", "").strip() != forward_sources_sha256():
        return None
    return float(fields["hbm_bytes_per_call"])


def measured_counters():
    """MFMA and VALU busy fractions of the two forward kernels from the committed rocprofv3
    counter runs, or None when the kernel sources changed since they were taken."""
    try:
        fields = dict(line.split(":", 1) for line in open(TRAFFIC_FILE) if ":" in line)
    except OSError:
        return None
    if fields.get("source_sha256", "").strip() != forward_sources_sha256():
        return None
    keys = ("mfma_busy_seg_state", "mfma_busy_pass_b", "valu_busy_seg_state", "valu_busy_pass_b")
    if not all(k in fields for k in keys):
        return None
    return {k: float(fields[k]) for k in keys}


def to_dev(d, torch):
    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return {"q": t(d["q"]), "k": t(d["k"]), "z": t(d["z"]), "v": t(d["v"]),
            "f": torch.from_numpy(d["f"]).cuda()}


def cpu_baseline(w, d, min_seconds=10.0):
    """The float64 oracle, as is, on the host cores: the whole forward workload, repeated
    until about ten seconds of wall time have passed."""
    from oracle import oracle
    from sparse_routed_slot_amd import inputs as gen
    r = {n: gen.as_f64(d[n], "bf16") for n in "qkzv"}
    f = d["f"].astype(np.float64)
    threads = oracle.max_threads()
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward(r["q"], r["k"], r["z"], r["v"], f, w.K)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    out = {"value": reps * w.B * w.T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{reps} x the full forward workload (B{w.B} T{w.T} Hh{w.Hh} M{w.M} Dv{w.Dv} "
                     f"K{w.K}), float64 recurrence, {dt:.1f} s wall on {threads} threads"}
    # one core: a bounded sample with the same work split (all batch rows and heads, the first
    # 32 tokens: 64 heads, so the oracle does not cut columns into blocks), repeated for about
    # two seconds
    sl = (slice(None), slice(0, 32))
    reps1 = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward(r["q"][sl], r["k"][sl], r["z"][sl], r["v"][sl], f[sl], w.K, nthreads=1)
        reps1 += 1
        dt1 = time.perf_counter() - t0
        if dt1 >= 2.0:
            break
    out["one_core"] = {"value": reps1 * w.B * 32 / dt1, "unit": "tokens/s", "cores": 1,
                       "sample": f"{reps1} x B{w.B} T32 Hh{w.Hh} of the same workload, {dt1:.1f} s on one thread"}
    # decode: one oracle step of the batched decode workload (256 sequences x 16 heads)
    wd = gen.WORKLOADS["decode_b256"]
    rng = np.random.default_rng(5)
    s = gen.decode_step_inputs(rng, wd.B, wd.Hh, wd.M, wd.Dv, "bf16")
    H = rng.standard_normal((wd.B, wd.Hh, wd.M, wd.Dv))
    args = [gen.as_f64(s[n], "bf16") for n in "qkzv"] + [s["f"].astype(np.float64)]
    steps = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 2.0:
        oracle.decode_step(*args, H, wd.K)
        steps += 1
    dtd = (time.perf_counter() - t0) / steps
    out["decode_us_per_step"] = {"value": dtd * 1e6, "cores": threads,
                                 "sample": f"{steps} steps of B{wd.B} Hh{wd.Hh} M{wd.M} Dv{wd.Dv} K{wd.K}"}
    return out


def time_forward_workload(name, torch, gen, rsm, steps):
    """One forward workload (every config besides the headline one): inputs generated once,
    2 warm-up calls, then `steps` calls between two HIP events.  Working sets of 300 MB and
    more exceed the last-level cache by themselves; the tiny one is launch-bound."""
    w = gen.WORKLOADS[name]
    d = gen.make_workload(name)
    es = 4 if w.dtype == "f32" else 2
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    if w.dtype == "f32":
        t = {n: torch.from_numpy(np.ascontiguousarray(d[n], np.float32)).cuda() for n in "qkzv"}
    else:
        t = {n: torch.from_numpy(np.ascontiguousarray(d[n]).view(np.int16)).view(torch.bfloat16).cuda()
             for n in "qkzv"}
    t["f"] = torch.from_numpy(d["f"]).cuda()
    del d
    o = torch.empty((w.B, w.T, w.Hh, w.Dv), dtype=torch.float32, device="cuda")
    H = torch.empty((w.B, w.Hh, w.M, w.Dv), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, rsm.forward_workspace_bytes(tdt, w.B, w.T, w.Hh, w.M, w.Dv, w.C, w.K)),
                     dtype=torch.uint8, device="cuda")

    def call():
        rsm.forward_chunked(t["q"], t["k"], t["z"], t["v"], t["f"], w.K, C=w.C, workspace=ws, out=o, state_out=H)

    for _ in range(2):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    nbytes = forward_bytes(w.B, w.T, w.Hh, w.M, w.Dv, es)
    c_run = 32 if (w.M == 128 and w.C > 32) else w.C
    rec = {"config": {"B": w.B, "T": w.T, "Hh": w.Hh, "M": w.M, "Dv": w.Dv, "K": w.K, "C": w.C,
                      "C_run": c_run, "dtype": w.dtype, "structure": w.note or "as the headline workload"},
           "us_per_call": us, "tokens_per_s": w.B * w.T / (us * 1e-6), "algorithmic_bytes_per_launch": nbytes,
           "achieved": nbytes / (us * 1e-6) / 1e9, "unit": "GB/s", "frac": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}
    if name == "tiny_f32":
        rec["note"] = "0.17 MB of data: launch-latency bound, absolute time only"
    print(f"[bench] forward {name}: {us:.1f} us/call, {rec['achieved']:.0f} GB/s "
          f"({rec['frac'] * 100:.1f}% of HBM peak), C run {c_run}", file=sys.stderr, flush=True)
    del t, o, H, ws
    return rec


def backward_bytes(B, T, Hh, M, Dv, es):
    """Algorithmic bytes of one backward: q, k, z, v, f, dO and dH_T read once; dq, dk, dz,
    dv, df and dH0 written once."""
    rows, heads = B * T * Hh, B * Hh
    return (3 * rows * M * es + rows * Dv * es + rows * 4 + rows * Dv * 4 + heads * M * Dv * 4
            + 3 * rows * M * 4 + rows * Dv * 4 + rows * 4 + heads * M * Dv * 4)


def time_backward(w, s, torch, rsm, steps):
    """rsm_backward on the headline workload (random upstream gradients), between HIP events."""
    g = torch.Generator(device="cuda").manual_seed(3)
    dO = torch.randn((w.B, w.T, w.Hh, w.Dv), device="cuda", generator=g)
    dHT = torch.randn((w.B, w.Hh, w.M, w.Dv), device="cuda", generator=g)
    ws = torch.empty(rsm.load().rsm_backward_workspace_bytes(1, w.B, w.T, w.Hh, w.M, w.Dv, w.K), dtype=torch.uint8,
                     device="cuda")

    def call():
        return rsm.backward(s["q"], s["k"], s["z"], s["v"], s["f"], w.K, dO, dHT=dHT, workspace=ws)

    call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    nbytes = backward_bytes(w.B, w.T, w.Hh, w.M, w.Dv, 2)
    print(f"[bench] backward {w.name}: {us:.1f} us/call, {w.B * w.T / us:.2f} M tok/s, "
          f"{nbytes / (us * 1e-6) / 1e9:.0f} GB/s", file=sys.stderr, flush=True)
    del dO, dHT, ws
    return {"workload": w.name, "us_per_call": us, "tokens_per_s": w.B * w.T / (us * 1e-6),
            "algorithmic_bytes_per_launch": nbytes, "achieved": nbytes / (us * 1e-6) / 1e9, "unit": "GB/s",
            "frac": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "form": "token-recurrent: route, rows forward (dq), rows backward (dk, dz, dg s, dH0), "
                    "columns backward (dv), df sum; see the design notes"}


def copy_bandwidth(torch, nbytes=1 << 30, reps=10):
    """Measured device-to-device copy rate (read + write bytes per second) of a 1 GiB buffer."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    return {"bytes_moved_per_copy": 2 * nbytes, "GB_per_s": 2 * nbytes / s / 1e9,
            "method": "torch copy_ of a 1 GiB fp32 buffer, 10 copies between HIP events"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the timing of the other forward configs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 256 MiB device copy (for scaling rocprofv3 byte counters)")
    ap.add_argument("--only-configs", action="store_true",
                    help="time only the other forward configs and print their records (for profiling them "
                         "apart from the headline workload); not the benchmark line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(heads, batch and value columns shard with no communication; see the sharding notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_routed_slot_amd import inputs as gen
    from sparse_routed_slot_amd import rsm

    if not os.path.exists(rsm.lib_path()):
        from sparse_routed_slot_amd import build
        build.build_library()
    rsm.load()
    torch.cuda.set_device(0)

    if args.only_configs:
        out = {name: time_forward_workload(name, torch, gen, rsm, 20 if name != "tiny_f32" else 200)
               for name in CONFIG_NAMES}
        print(json.dumps({"configs": out}), flush=True)
        return

    # ---------------------------------------------------------------- forward
    w = gen.WORKLOADS["fwd_b8_t2048"]
    print(f"[bench] generating inputs for {w.name}", file=sys.stderr, flush=True)
    host_sets = [gen.make_inputs(w.B, w.T, w.Hh, w.M, w.Dv, w.dtype, w.seed + 100 * i) for i in range(3)]
    sets = [to_dev(d, torch) for d in host_sets]
    o = torch.empty((w.B, w.T, w.Hh, w.Dv), dtype=torch.float32, device="cuda")
    Hs = torch.empty((w.B, w.Hh, w.M, w.Dv), dtype=torch.float32, device="cuda")
    ws = torch.empty(rsm.forward_workspace_bytes(torch.bfloat16, w.B, w.T, w.Hh, w.M, w.Dv, w.C, w.K),
                     dtype=torch.uint8, device="cuda")

    def fwd(i):
        s = sets[i % len(sets)]
        rsm.forward_chunked(s["q"], s["k"], s["z"], s["v"], s["f"], w.K, C=w.C, workspace=ws, out=o,
                            state_out=Hs)

    for i in range(args.warmup):
        fwd(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    # timed region: K calls back to back, bracketed by one pair of HIP events on the launch
    # stream (timing events between the calls would each add a few microseconds of wall time)
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    r0.record(stream)
    for i in range(args.steps):
        fwd(i)
    r1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    kernel_ms = r0.elapsed_time(r1) / args.steps
    # per-call spread, outside the timed region
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        fwd(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per_call_ms = [a.elapsed_time(b) for a, b in ev]
    tok = w.B * w.T
    fbytes = forward_bytes(w.B, w.T, w.Hh, w.M, w.Dv, 2)
    achieved = fbytes / (kernel_ms * 1e-3) / 1e9
    print(f"[bench] forward: wall {ms_per_step * 1e3:.1f} us/step, events over the timed region "
          f"{kernel_ms * 1e3:.1f} us/call, {achieved:.0f} GB/s; events per call (separate loop) mean "
          f"{np.mean(per_call_ms) * 1e3:.1f} min {min(per_call_ms) * 1e3:.1f} us", file=sys.stderr, flush=True)

    # router / decay variants on the same workload (softmax + renormalised + per-slot f + noise)
    vx = [gen.variant_inputs(np.random.default_rng(w.seed + 7 + i), host_sets[i]["z"].shape) for i in range(3)]
    vdev = [{"f": torch.from_numpy(x["f_slot"]).cuda(), "noise": torch.from_numpy(x["noise"]).cuda()} for x in vx]

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    var_fwd = {}
    for label, noisy in (("forward_inference", False), ("forward_training_noise", True)):
        def fwd_var(i):
            s, x = sets[i % len(sets)], vdev[i % len(vdev)]
            rsm.forward_chunked(s["q"], s["k"], s["z"], s["v"], x["f"], w.K, C=w.C, workspace=ws, out=o,
                                state_out=Hs, score="softmax", normalize=True, noise=x["noise"] if noisy else None)

        for i in range(3):
            fwd_var(i)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            fwd_var(i)
        e1.record(stream)
        torch.cuda.synchronize()
        var_ms = e0.elapsed_time(e1) / args.steps
        var_bytes = fbytes + w.B * w.T * w.Hh * (w.M - 1) * 4 + (w.B * w.T * w.Hh * w.M * 4 if noisy else 0)
        print(f"[bench] {label} (router/decay variant): {var_ms * 1e3:.1f} us, "
              f"{var_bytes / (var_ms * 1e-3) / 1e9:.0f} GB/s", file=sys.stderr, flush=True)
        var_fwd[label] = {"us_per_call": var_ms * 1e3, "algorithmic_bytes_per_launch": var_bytes,
                          "achieved": var_bytes / (var_ms * 1e-3) / 1e9, "unit": "GB/s",
                          "frac": var_bytes / (var_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    del vdev

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------------------------------------------------------- decode
    wd = gen.WORKLOADS["decode_b256"]
    print(f"[bench] decode: prefill T={wd.T} for {wd.B}x{wd.Hh} heads", file=sys.stderr, flush=True)
    dd = gen.make_inputs(wd.B, wd.T, wd.Hh, wd.M, wd.Dv, wd.dtype, wd.seed)
    pre = to_dev(dd, torch)
    del dd
    _, Hdec, _ = rsm.forward_chunked(pre["q"], pre["k"], pre["z"], pre["v"], pre["f"], wd.K, C=wd.C)
    del pre
    rng = np.random.default_rng(1000 + wd.seed)
    pool = [to_dev(gen.decode_step_inputs(rng, wd.B, wd.Hh, wd.M, wd.Dv, "bf16"), torch) for _ in range(16)]
    n_pool = len(pool)
    od = torch.empty((wd.B, wd.Hh, wd.Dv), dtype=torch.float32, device="cuda")

    def dec(i):
        s = pool[i % len(pool)]
        rsm.decode_step(s["q"], s["k"], s["z"], s["v"], s["f"], Hdec, wd.K, out=od)

    for i in range(16):
        dec(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.decode_steps):
        dec(i)
    e1.record(stream)
    torch.cuda.synchronize()
    dec_us = e0.elapsed_time(e1) * 1e3 / args.decode_steps
    dbytes = decode_bytes(wd.B, wd.Hh, wd.M, wd.Dv, wd.K, 2)
    print(f"[bench] decode: {dec_us:.2f} us/step, {dbytes / (dec_us * 1e-6) / 1e9:.0f} GB/s",
          file=sys.stderr, flush=True)

    # decode with the router / decay variant
    vpool = [{n: torch.from_numpy(x).cuda() for n, x in gen.variant_inputs(rng, (wd.B, wd.Hh, wd.M)).items()}
             for _ in range(16)]

    def dec_var(i):
        s, x = pool[i % len(pool)], vpool[i % len(vpool)]
        rsm.decode_step(s["q"], s["k"], s["z"], s["v"], x["f_slot"], Hdec, wd.K, out=od, score="softmax",
                        normalize=True, noise=x["noise"])

    for i in range(16):
        dec_var(i)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.decode_steps):
        dec_var(i)
    e1.record(stream)
    torch.cuda.synchronize()
    dvar_us = e0.elapsed_time(e1) * 1e3 / args.decode_steps
    dvar_bytes = dbytes + variant_extra_bytes(wd.B * wd.Hh, wd.M)
    print(f"[bench] decode, router/decay variant: {dvar_us:.2f} us/step, "
          f"{dvar_bytes / (dvar_us * 1e-6) / 1e9:.0f} GB/s", file=sys.stderr, flush=True)
    # decode over a state that cannot stay in the 256 MB last-level cache: three state
    # buffers (3 x 134 MB) rotated step by step
    Hrot = [Hdec] + [Hdec.clone() for _ in range(2)]

    def dec_rot(i):
        s = pool[i % len(pool)]
        rsm.decode_step(s["q"], s["k"], s["z"], s["v"], s["f"], Hrot[i % 3], wd.K, out=od)

    for i in range(6):
        dec_rot(i)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.decode_steps):
        dec_rot(i)
    e1.record(stream)
    torch.cuda.synchronize()
    drot_us = e0.elapsed_time(e1) * 1e3 / args.decode_steps
    print(f"[bench] decode, 3 rotated states (402 MB, past the last-level cache): {drot_us:.2f} us/step, "
          f"{dbytes / (drot_us * 1e-6) / 1e9:.0f} GB/s", file=sys.stderr, flush=True)
    del vpool, pool, Hdec, Hrot

    # decode step at the pages' default layer shape (4 heads, 256 slots, top-32, head dim 256),
    # 256 sequences; the state is drawn at random (the chunked forward takes M <= 128)
    LB, LHh, LM, LDv, LK = 256, 4, 256, 256, 32
    Hl = torch.randn((LB, LHh, LM, LDv), dtype=torch.float32, device="cuda")
    lpool = [to_dev(gen.decode_step_inputs(rng, LB, LHh, LM, LDv, "bf16"), torch) for _ in range(16)]
    n_lpool = len(lpool)
    ol = torch.empty((LB, LHh, LDv), dtype=torch.float32, device="cuda")

    def dec_layer(i):
        s = lpool[i % len(lpool)]
        rsm.decode_step(s["q"], s["k"], s["z"], s["v"], s["f"], Hl, LK, out=ol)

    for i in range(16):
        dec_layer(i)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.decode_steps):
        dec_layer(i)
    e1.record(stream)
    torch.cuda.synchronize()
    dl_us = e0.elapsed_time(e1) * 1e3 / args.decode_steps
    dl_bytes = decode_bytes(LB, LHh, LM, LDv, LK, 2)
    print(f"[bench] decode, default layer shape (B{LB} Hh{LHh} M{LM} Dv{LDv} K{LK}): {dl_us:.2f} us/step, "
          f"{dl_bytes / (dl_us * 1e-6) / 1e9:.0f} GB/s", file=sys.stderr, flush=True)

    # forward at the pages' default layer shape (M = 256, bf16, K = 32: chunked, chunks of 32)
    FB, FT, FHh, FM, FDv, FK = 16, 2048, 4, 256, 256, 32
    fl = to_dev(gen.make_inputs(FB, FT, FHh, FM, FDv, "bf16", 11), torch)
    fo = torch.empty((FB, FT, FHh, FDv), dtype=torch.float32, device="cuda")
    fH = torch.empty((FB, FHh, FM, FDv), dtype=torch.float32, device="cuda")
    fws = torch.empty(rsm.forward_workspace_bytes(torch.bfloat16, FB, FT, FHh, FM, FDv, 64, FK), dtype=torch.uint8,
                      device="cuda")

    def fwd_layer():
        rsm.forward_chunked(fl["q"], fl["k"], fl["z"], fl["v"], fl["f"], FK, workspace=fws, out=fo, state_out=fH)

    fwd_layer()
    torch.cuda.synchronize()
    n_fl = 5
    e0.record(stream)
    for _ in range(n_fl):
        fwd_layer()
    e1.record(stream)
    torch.cuda.synchronize()
    fl_us = e0.elapsed_time(e1) * 1e3 / n_fl
    fl_bytes = forward_bytes(FB, FT, FHh, FM, FDv, 2)
    print(f"[bench] forward, default layer shape (B{FB} T{FT} Hh{FHh} M{FM} Dv{FDv} K{FK}, chunked): "
          f"{fl_us:.0f} us/call, {FB * FT / fl_us:.2f} M tok/s", file=sys.stderr, flush=True)
    del fl, fo, fH, fws

    # backward pass (gradients for upstream dO and dH_T) on the headline workload
    bwd = time_backward(w, sets[0], torch, rsm, max(5, args.steps // 5))

    # every other forward config
    configs = {}
    if not args.no_configs:
        for name in CONFIG_NAMES:
            configs[name] = time_forward_workload(name, torch, gen, rsm, 20 if name != "tiny_f32" else 200)
    copy_bw = copy_bandwidth(torch)
    print(f"[bench] device copy: {copy_bw['GB_per_s']:.0f} GB/s", file=sys.stderr, flush=True)

    rec = {
        "metric": METRIC,
        "value": tok / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "Hh": w.Hh, "M": w.M, "Dv": w.Dv, "K": w.K,
                   "C": w.C, "inputs": "bf16 q,k,z,v; fp32 f, state, outputs", "input_sets_rotated": 3},
        "decode_us_per_step": dec_us,
        "decode_config": {"workload": wd.name, "B": wd.B, "Hh": wd.Hh, "M": wd.M, "Dv": wd.Dv, "K": wd.K,
                          "prefill_T": wd.T, "steps": args.decode_steps, "step_input_pool": n_pool},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(),
                     "kernel": "rsm_forward_chunked call = seg_state_kernel (routes each segment and "
                               "computes every segment state but the last's by the backward walk; one route-only "
                               "workgroup per head routes the last segment) + fwd_scan_kernel pass B (two "
                               "launches back to back on the caller's stream; the segment fold runs inside pass "
                               "B at 4 segments)",
                     "algorithmic_bytes_per_launch": fbytes, "avg_launch_ms": kernel_ms,
                     "counters": measured_counters()},
        "decode_roofline": {"bound": "hbm", "achieved": dbytes / (dec_us * 1e-6) / 1e9, "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": dbytes / (dec_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                            "kernel": "decode_step_kernel", "algorithmic_bytes_per_launch": dbytes,
                            "state_residency": "the 134 MB state fits in the 256 MB last-level cache across "
                                               "steps; decode_rotated_states is the figure with the state "
                                               "read from HBM"},
        "decode_rotated_states": {"us_per_step": drot_us, "states": 3, "working_set_bytes": 3 * wd.B * wd.Hh *
                                  wd.M * wd.Dv * 4, "achieved": dbytes / (drot_us * 1e-6) / 1e9, "unit": "GB/s",
                                  "frac": dbytes / (drot_us * 1e-6) / 1e9 / PEAK_HBM_GBS},
        "backward": bwd,
        "configs": configs,
        "device_copy": copy_bw,
        "decode_default_layer": {"config": {"B": LB, "Hh": LHh, "M": LM, "Dv": LDv, "K": LK,
                                            "state": "random fp32", "step_input_pool": n_lpool},
                                 "us_per_step": dl_us, "algorithmic_bytes_per_launch": dl_bytes,
                                 "achieved": dl_bytes / (dl_us * 1e-6) / 1e9, "unit": "GB/s",
                                 "frac": dl_bytes / (dl_us * 1e-6) / 1e9 / PEAK_HBM_GBS},
        "forward_default_layer": {"config": {"B": FB, "T": FT, "Hh": FHh, "M": FM, "Dv": FDv, "K": FK,
                                             "form": "chunked: the chunk router, then the chunk scan with chunks "
                                                     "of 32 and 64-column tiles (one segment)"},
                                  "us_per_call": fl_us, "tokens_per_s": FB * FT / (fl_us * 1e-6),
                                  "algorithmic_bytes_per_launch": fl_bytes,
                                  "achieved": fl_bytes / (fl_us * 1e-6) / 1e9, "unit": "GB/s",
                                  "frac": fl_bytes / (fl_us * 1e-6) / 1e9 / PEAK_HBM_GBS},
        "variants": {
            "router": "softmax scores renormalised over the selected slots and per-slot decay rates; "
                      "the training line and the decode add fp32 exploration noise on the logits",
            **var_fwd,
            "decode": {"us_per_step": dvar_us, "algorithmic_bytes_per_launch": dvar_bytes,
                       "achieved": dvar_bytes / (dvar_us * 1e-6) / 1e9, "unit": "GB/s",
                       "frac": dvar_bytes / (dvar_us * 1e-6) / 1e9 / PEAK_HBM_GBS},
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (float64 oracle)", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(w, host_sets[0])
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
