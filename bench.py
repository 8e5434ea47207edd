"""Benchmark of the MI355X FlashAttention forward.

One step = one bf16 attention forward (fa_fwd through the C ABI) over the
headline workload: B=4, H=16, N=8192, d=128, non-causal, N(0,1) inputs cast
to bf16, output bf16 O plus fp32 LSE.  Throughput counts 4*B*H*N^2*d FLOPs
(halved when causal).  Inputs are resident in device memory before the timed
region; the timed region is W untimed warm-up steps, then K steps bracketed
by device synchronisations, timed with HIP events recorded on the stream the
kernels are launched on.

Prints ONE JSON line (rank 0, one GPU) with the throughput, a roofline object
for the attention kernel (MFMA-bound; achieved FLOP/s over the dense bf16
peak), the oracle timed on the host cores on a bounded sample, and secondary
measurements of the other workloads (causal, GQA, fp8, quantisation).
"""

from __future__ import annotations

import argparse
import hashlib
import itertools
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
FP8_PEAK_TFLOPS = 5033.2    # dense fp8 MFMA: 256 CU x 8192 FLOP/clk x 2.4 GHz
HBM_PEAK_GBS = 8000.0

METRIC = "attention fwd TFLOP/s + % of MFMA peak (bf16, N=8192, d=128, 1 GPU)"


# Sources the headline kernel is built from (kernel, shared header, the
# launching entry point): the recorded HBM counters stay valid while these
# are unchanged.
HEADLINE_SOURCES = ("fa_api.hip", "fa_common.h", "fa_fwd_bf16.hip")


def _kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_attention_101_amd", "csrc")
    for name in HEADLINE_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def _traffic(kernel: str):
    """HBM bytes per launch from the committed PMC summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel)
    if not e or e.get("source_hash") != _kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


def _time_launches(fn, steps: int, warmup: int, min_warm_ms: float = 0.0):
    """Milliseconds per call of fn() over `steps` back-to-back calls, from
    HIP events on torch's current stream (the stream fn launches on): one
    event before the first call and one after each, so the mean (whole
    span / steps), median and minimum come from the same timed run.
    Warm-up: `warmup` calls, more if needed to fill at least min_warm_ms of
    back-to-back work (the clock ramps up over the first tens of ms of a
    burst)."""
    import torch
    if min_warm_ms > 0:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            fn()
        e1.record()
        torch.cuda.synchronize()
        per = max(e0.elapsed_time(e1) / 3, 1e-3)
        warmup = max(warmup, int(min_warm_ms / per) + 1)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    each = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    mid = steps // 2
    median = each[mid] if steps % 2 else 0.5 * (each[mid - 1] + each[mid])
    return {"mean": ev[0].elapsed_time(ev[steps]) / steps, "median": median,
            "min": each[0]}


def _progress(msg: str) -> None:
    """One line on stderr per finished measurement (stdout carries only the
    JSON result line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def _bf16_workload(name):
    """Seeded inputs of a named bf16 workload: device bf16 tensors plus the
    host bf16 tensors they were copied from."""
    import torch
    import workloads
    w = workloads.WORKLOADS[name]
    host = tuple(workloads.to_bf16(x) for x in workloads.workload_qkv(w))
    dev = torch.device("cuda:0")
    return w, tuple(t.to(dev) for t in host), host


def _cpu_baseline(w, host, budget_s: float):
    """The fp64 oracle on the host cores over a bounded sample of the same
    workload: whole heads (every query row against every key) of the same
    seeded inputs, as many as fit in the time budget."""
    import oracle
    import workloads
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        cores = max((p.get("num_threads", 1) for p in pools), default=1)
        if pools:
            blas = f"{pools[0].get('internal_api')} {pools[0].get('version')}"
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    qh, kh, vh = host
    t0 = time.perf_counter()
    n, secs = 0, 0.0
    while n < w.B * w.H and time.perf_counter() - t0 < budget_s:
        b, h = divmod(n, w.H)
        kvh = h // (w.H // w.Hkv)
        args = (workloads.bf16_values(qh[b:b + 1, h:h + 1]),
                workloads.bf16_values(kh[b:b + 1, kvh:kvh + 1]),
                workloads.bf16_values(vh[b:b + 1, kvh:kvh + 1]))
        t1 = time.perf_counter()
        oracle.attention(*args, causal=w.causal)
        secs += time.perf_counter() - t1
        n += 1
    flops = w.flops / (w.B * w.H) * n
    return {
        "value": round(flops / secs / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{n} of {w.B * w.H} heads of {w.name} (all {w.N} query "
                  f"rows of each head, fp64 numpy oracle, {secs:.1f} s); "
                  "same FLOP convention",
        "wall_s": round(secs, 2),
        "blas": blas,
        "affinity_cores": len(os.sched_getaffinity(0)),
    }


# Bodies of the issue-rate probes (exact_attention_101_amd/csrc/fa_probe_rates.hip):
# name -> (id, instructions per round, kind of instruction counted).
PROBE_BODIES = {
    "idle": (0, 0, ""),
    "fma": (1, 16, "v_fma_f32"),
    "exp": (2, 16, "v_exp_f32"),
    "exp+fma": (3, 16, "8 v_exp_f32 + 8 v_fma_f32"),
    "cvt_pk_fp8": (4, 16, "v_cvt_pk_fp8_f32"),
    "maximum3": (5, 16, "v_maximum3_f32"),
    "add": (6, 16, "v_add_f32"),
    "mfma_f8": (7, 4, "v_mfma_scale_f32_32x32x64_f8f6f4"),
    "mfma_bf16": (8, 4, "v_mfma_f32_32x32x16_bf16"),
    "mfma_f8+exp": (9, 4, "f8 MFMA, each with 8 exp or 8 fma"),
    "mfma_bf16+exp": (10, 4, "bf16 MFMA, each with 2 exp + 2 fma"),
    "exp_chain": (11, 16, "4 x (fma -> exp -> add) + 4 add"),
    "dot2_bf16": (14, 16, "v_dot2c_f32_bf16"),
    "mov_b64": (15, 16, "v_mov_b64"),
    "cvt_pk_bf16": (16, 16, "v_cvt_pk_bf16_f32"),
    "mfma_bf16+add": (17, 4, "bf16 MFMA, each with 4 v_add_f32"),
    "mfma_bf16+dot2": (18, 4, "bf16 MFMA, each with 4 v_dot2c_f32_bf16"),
    "mfma_bf16+mov64": (19, 4, "bf16 MFMA, each with 4 v_mov_b64"),
    "cvt_scalef32_pk_fp8": (20, 16, "v_cvt_scalef32_pk_fp8_f32"),
    "slot_bf16": (21, 4, "the bf16 forward's issue slot: scores MFMA, 2 x "
                         "(fma -> exp), P V MFMA, cvt_pk_bf16 + 2 add of the "
                         "exponentials (counted per slot)"),
    "lds_k": (22, 8, "ds_read_b128 at the bf16 forward's K fragment "
                     "addresses"),
    "lds_v": (23, 16, "ds_read_b64_tr_b16 at the bf16 forward's V fragment "
                      "addresses"),
    "lds_tr_seq": (24, 16, "ds_read_b64_tr_b16 at consecutive 8-byte units"),
    "exp2_fma": (25, 16, "the FMA-pipe exponential of the fp8 forward's "
                         "option (8 vector instructions; counted per "
                         "exponential)"),
    "slot_bf16_pipelined": (26, 4, "the same issue slot with its vector "
                                   "work pipelined across slots (fma of "
                                   "pair i+1 and exp of pair i after the "
                                   "first MFMA, pack and sums of pair i-1 "
                                   "after the second; counted per slot)"),
    "lds_dma_copy": (27, 16, "buffer_load_dwordx4 ... lds, 1 KB per wave, "
                             "from an L2-resident 16 KB buffer"),
    "mfma_bf16+copy": (28, 4, "bf16 MFMA, each followed by one LDS-DMA "
                              "copy (counted per MFMA)"),
    "slot_bf16+copy": (29, 4, "the bf16 forward's issue slot with one "
                              "LDS-DMA copy after its first MFMA (counted "
                              "per slot)"),
}
# Bodies that copy from (or multiply) the caller's data buffer.
PROBE_DATA_BODIES = (12, 13, 27, 28, 29)

# (body A, body B, waves per workgroup, A waves per SIMD): one workgroup per
# CU, four waves per SIMD at most (the SIMD of each wave is read from its
# HW_ID).
PROBE_CONFIGS = (
    [(b, "idle", 4 * n, n) for n in (1, 2, 4)
     for b in ("fma", "exp", "exp+fma", "add", "cvt_pk_fp8", "maximum3",
               "exp_chain", "dot2_bf16", "mov_b64", "cvt_pk_bf16",
               "cvt_scalef32_pk_fp8", "exp2_fma")]
    + [(b, "idle", 4 * n, n) for n in (1, 2)
       for b in ("mfma_f8", "mfma_bf16", "mfma_f8+exp", "mfma_bf16+exp",
                 "mfma_bf16+add", "mfma_bf16+dot2", "mfma_bf16+mov64")]
    + [("mfma_f8", b, 8, 1) for b in ("exp", "fma", "exp+fma", "exp_chain")]
    + [("mfma_bf16", b, 8, 1) for b in ("exp", "fma", "exp+fma", "exp_chain",
                                          "dot2_bf16", "mov_b64")]
    + [("mfma_f8", "exp+fma", 12, 1), ("mfma_f8", "exp_chain", 12, 1)]
    + [("mfma_f8", "exp2_fma", 8, 1), ("mfma_bf16", "exp2_fma", 8, 1)]
    + [(b, "idle", 4 * n, n) for n in (1, 2)
       for b in ("slot_bf16", "slot_bf16_pipelined", "lds_dma_copy",
                 "mfma_bf16+copy", "slot_bf16+copy")]
    + [(b, "idle", 4 * n, n) for n in (1, 2, 4)
       for b in ("lds_k", "lds_v", "lds_tr_seq")]
)


def _rates(iters: int) -> dict:
    """Cycles per wave64 instruction on one SIMD for each probe body, alone
    and mixed (see fa_probe_rates.hip)."""
    import ctypes
    import statistics
    import torch
    import exact_attention_101_amd as fa
    path = os.path.join(os.path.dirname(fa.__file__), "libfa_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built")
    lib = ctypes.CDLL(path)
    lib.fa_probe_rates.argtypes = [ctypes.c_int] * 6 + [ctypes.c_void_p] * 3
    lib.fa_probe_rates.restype = ctypes.c_int
    torch.cuda.set_device(0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream().cuda_stream
    rows = []
    # 16 KB of N(0, 1) values: the copy source of the LDS-DMA bodies.
    data = torch.randn(4096, device="cuda:0").contiguous()
    for a, b, waves, na in PROBE_CONFIGS:
        out = torch.zeros(cus * waves * 3, dtype=torch.int64, device="cuda:0")
        ia, na_i, _ = PROBE_BODIES[a]
        ib, nb_i, _ = PROBE_BODIES[b]
        dptr = data.data_ptr() if ia in PROBE_DATA_BODIES else None
        runs = []
        for rep in range(4):              # the first run warms the clock
            rc = lib.fa_probe_rates(ia, ib, waves, na, iters, cus,
                                    out.data_ptr(), dptr, stream)
            if rc != 0:
                raise RuntimeError(f"fa_probe_rates({a}, {b}) = {rc}")
            torch.cuda.synchronize()
            if rep:
                runs.append(out.view(cus, waves, 3).cpu())
        t = torch.stack(runs)              # [rep, cu, wave, 3]
        hw = t[0, :, :, 2]
        simd = ((hw >> 4) & 3).tolist()   # HW_ID bits 5:4
        is_a = [w < 4 * na for w in range(waves)]
        # Waves of body A and B on each (workgroup, SIMD); the rates below
        # come from the SIMDs with the most common composition.
        comp = {}
        for g in range(cus):
            per = {}
            for w in range(waves):
                key = per.setdefault(simd[g][w], [0, 0, []])
                key[0 if is_a[w] else 1] += 1
                key[2].append(w)
            for sm, (ka, kb, ws) in per.items():
                comp.setdefault((ka, kb), []).append((g, ws))
        (ka, kb), members = max(comp.items(), key=lambda kv: len(kv[1]))
        cyc = t[:, :, :, 0].double()
        ref = t[:, :, :, 1].double()
        ghz = float((cyc / ref).median()) * 0.1
        row = {"a": a, "b": b, "waves_per_wg": waves,
               "simd_compositions": {f"A{x}B{y}": len(m) for (x, y), m in
                                     sorted(comp.items())},
               "simd_a_waves": ka, "simd_b_waves": kb, "ghz": round(ghz, 3),
               "hw_id_wg0": [hex(int(x)) for x in hw[0].tolist()]}
        # A SIMD's throughput for a body is its waves' whole work over the
        # time its slowest wave of that body took (all waves start together
        # after a barrier); the fastest wave shows how issue was shared.
        for name, want_a, n_i, k in ((a, True, na_i, ka),
                                     (b, False, nb_i, kb)):
            if k == 0 or n_i == 0:
                continue
            slow, fast = [], []
            for r in range(cyc.shape[0]):
                for g, ws in members:
                    d = [float(cyc[r, g, w]) for w in ws if is_a[w] == want_a]
                    slow.append(max(d))
                    fast.append(min(d))
            norm = iters * n_i
            cs = float(statistics.median(slow)) / norm
            cf = float(statistics.median(fast)) / norm
            row[name + "_slowest_wave_cycles_per_instr"] = round(cs, 2)
            row[name + "_fastest_wave_cycles_per_instr"] = round(cf, 2)
            row[name + "_simd_cycles_per_instr"] = round(cs / k, 2)
        rows.append(row)
        _progress(json.dumps(row))
    return {"iters": iters, "cus": cus, "bodies": {k: v[2] for k, v in
                                                   PROBE_BODIES.items()},
            "rows": rows, "mfma_ceiling": _mfma_ceiling(lib)}


def _under_profiler() -> bool:
    """rocprofv3 preloads its library into every child process, and there
    it initialises the GPU, so a child that then replaces itself (a script
    run through `#!/usr/bin/env`) must not be started at all."""
    return any(k.startswith("ROCPROF") for k in os.environ) or \
        "rocprof" in os.environ.get("LD_PRELOAD", "")


def _amd_smi_sample():
    """(mean GFX clock over the XCDs in MHz, socket power in W) from one
    amd-smi call, or None.  amd-smi is a Python script: it is run by this
    interpreter directly, as one child process with no `env` hop."""
    import shutil
    import subprocess
    if _under_profiler():
        return None
    smi = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    try:
        with open(smi, "rb") as f:
            first = f.readline()
        cmd = [sys.executable, smi] if b"python" in first else [smi]
        r = subprocess.run(cmd + ["metric", "-g", "0", "--clock", "--power",
                                  "--json"], capture_output=True, text=True,
                           timeout=10)
        g = json.loads(r.stdout)["gpu_data"][0]
        clks = [v["clk"]["value"] for k, v in g["clock"].items()
                if k.startswith("gfx_") and isinstance(v.get("clk"), dict)]
        pw = g["power"]["socket_power"]["value"]
        return sum(clks) / len(clks), float(pw)
    except Exception:                     # tool missing or output changed
        return None


def _under_load(fn, seconds: float):
    """Calls fn() back to back for `seconds` while a thread samples the GPU
    clock and socket power with amd-smi (a subprocess); returns the medians
    over the samples taken wholly inside the load (started after its first
    third, when the clock has settled, and finished before the last launch
    completed), or None if none was."""
    import statistics
    import threading
    import torch
    samples = []
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            t_a = time.perf_counter()
            v = _amd_smi_sample()
            if v is not None:
                samples.append((t_a, time.perf_counter(), v))
            time.sleep(0.02)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()       # bound the queue
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stop.set()
    th.join()
    inside = [v for a, b, v in samples if a > t0 + seconds / 3 and b < t1]
    if not inside:
        return None
    return {"gfx_mhz": round(statistics.median(c for c, _ in inside), 1),
            "socket_w": round(statistics.median(p for _, p in inside), 1),
            "samples": len(inside), "launches": n,
            "how": "amd-smi metric --clock --power from a subprocess, median "
                   "of the samples taken wholly inside a span of back-to-back "
                   "launches (after its first third)"}


def _mfma_ceiling(lib) -> dict:
    """The matrix rate this card sustains under its power limit on operands
    like the attention's: every SIMD runs two waves of back-to-back MFMAs
    whose operands (2 A and 2 B fragments, paired in turn) hold N(0,1)
    values, for ~0.3 s.  TFLOP/s from HIP events; the shader clock from the
    probe's own s_memtime / s_memrealtime and from amd-smi."""
    import statistics
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream().cuda_stream
    g = torch.Generator(device="cuda:0").manual_seed(5)
    res = {}
    for name, body, flop, iters, make in (
            ("bf16_32x32x16", 12, 32 * 32 * 16 * 2, 100000,
             lambda: torch.randn(512 * 16, device="cuda:0", generator=g)
             .to(torch.bfloat16)),
            ("fp8_32x32x64", 13, 32 * 32 * 64 * 2, 50000,
             lambda: torch.randn(512 * 32, device="cuda:0", generator=g)
             .to(torch.float8_e4m3fn))):
        data = make().view(torch.uint8).contiguous()
        assert data.numel() == 512 * 32 and data.data_ptr() % 32 == 0
        waves = 8
        out = torch.zeros(cus * waves * 3, dtype=torch.int64, device="cuda:0")

        def launch():
            rc = lib.fa_probe_rates(body, 0, waves, 2, iters, cus,
                                    out.data_ptr(), data.data_ptr(), stream)
            if rc != 0:
                raise RuntimeError(f"fa_probe_rates({body}) = {rc}")

        for _ in range(2):
            launch()
        load = _under_load(launch, 1.0)
        tm = _time_launches(launch, 8, 2)
        t = cus * waves * iters * 4 * flop / (tm["mean"] * 1e-3) / 1e12
        o = out.view(cus, waves, 3).cpu().double()
        ghz = float((o[:, :, 0] / o[:, :, 1]).median()) * 0.1
        peak = BF16_PEAK_TFLOPS if body == 12 else FP8_PEAK_TFLOPS
        res[name] = {"TFLOP/s": round(t, 1), "frac_of_peak": round(t / peak, 4),
                     "shader_ghz": round(ghz, 3),
                     "frac_of_peak_at_that_clock": round(t / (peak * ghz / 2.4), 4),
                     "under_load": load}
        _progress(f"mfma ceiling {name}: {res[name]}")
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=25,
                    help="untimed launches first (the clock settles over "
                         "the first ~10 launches of a burst)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the secondary workloads")
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device-to-device copy "
                         "(reference point for HBM byte counters)")
    ap.add_argument("--rates", action="store_true",
                    help="instead of the benchmark: issue-rate probes of one "
                         "SIMD (cycles per wave64 v_fma_f32, v_exp_f32, "
                         "MFMA, alone and mixed); prints one JSON line")
    ap.add_argument("--rates-iters", type=int, default=4096)
    args = ap.parse_args()
    if args.rates:
        print(json.dumps(_rates(args.rates_iters)), flush=True)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the forward kernel runs on a "
              f"single device and this library has no multi-GPU path "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        return 2
    rank = int(os.environ.get("RANK", "0"))

    import numpy as np
    import torch
    import exact_attention_101_amd as fa
    import workloads

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    w, (q, k, v), host = _bf16_workload(workloads.HEADLINE)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

    def step():
        fa.forward(q, k, v, causal=w.causal, out=o, lse=lse)

    if args.copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    torch.cuda.synchronize()
    head = _time_launches(step, args.steps, args.warmup)
    ms = head["mean"]
    tflops = w.flops / (ms * 1e-3) / 1e12
    _progress(f"{w.name}: {ms:.4f} ms, {tflops:.1f} TFLOP/s")
    # The clock the card runs this kernel at (power-limited): amd-smi samples
    # while the same launches run back to back for a second.
    clock = _under_load(step, 3.0)
    if clock is not None:
        frac_clk = tflops / (BF16_PEAK_TFLOPS * clock["gfx_mhz"] / 2400.0)
        if frac_clk <= 1.0:
            clock["frac_of_peak_at_that_clock"] = round(frac_clk, 4)
        else:
            # The samples cannot describe the timed launches (more than the
            # whole matrix rate at that clock): amd-smi reported values from
            # before the load.
            clock["frac_of_peak_at_that_clock"] = None
            clock["inconsistent"] = (
                f"{frac_clk:.2f} of the peak at the sampled clock: the "
                "samples predate the load")
    _progress(f"clock under load: {clock}")

    extras = {}
    if not args.no_extras:
        for name in ("bf16_n4096", "bf16_causal_n8192",
                     "bf16_causal_gqa_n16384"):
            ww, (qq, kk, vv), _ = _bf16_workload(name)
            oo = torch.empty_like(qq)
            ll = torch.empty((ww.B, ww.H, ww.N), dtype=torch.float32,
                             device=dev)
            tm = _time_launches(lambda: fa.forward(qq, kk, vv, causal=ww.causal,
                                                   out=oo, lse=ll), 20, 20, min_warm_ms=30.0)
            m = tm["mean"]
            t = ww.flops / (m * 1e-3) / 1e12
            extras[name] = {"ms": round(m, 4), "ms_median": round(tm["median"], 4),
                            "ms_min": round(tm["min"], 4), "TFLOP/s": round(t, 1),
                            "frac_of_bf16_peak": round(t / BF16_PEAK_TFLOPS, 4)}
            _progress(f"{name}: {extras[name]}")
            del qq, kk, vv, oo, ll
        # Backward of the headline workload (dQ, dK, dV from the forward's O
        # and LSE and a seeded dO).  Throughput counts 2.5x the forward's
        # FLOPs, the usual convention for the five products of a backward
        # pass (the kernels recompute S and dP in both gradient kernels, so
        # they do seven).
        gd = torch.Generator(device=dev).manual_seed(11)
        dout = torch.randn(q.shape, device=dev, generator=gd).to(torch.bfloat16)
        dq, dk, dv = (torch.empty_like(x) for x in (q, k, v))
        ws = torch.empty(2 * w.B * w.H * w.N, dtype=torch.float32, device=dev)
        fa.forward(q, k, v, causal=w.causal, out=o, lse=lse)
        tm_b = _time_launches(
            lambda: fa.backward(q, k, v, o, lse, dout, causal=w.causal, dq=dq,
                                dk=dk, dv=dv, workspace=ws), 20, 10, min_warm_ms=30.0)
        tb = 2.5 * w.flops / (tm_b["mean"] * 1e-3) / 1e12
        extras["bf16_n8192_backward"] = {
            "ms": round(tm_b["mean"], 4), "ms_median": round(tm_b["median"], 4),
            "ms_min": round(tm_b["min"], 4), "TFLOP/s": round(tb, 1),
            "frac_of_bf16_peak": round(tb / BF16_PEAK_TFLOPS, 4),
            "flops": "2.5 x forward (10 B H N^2 d)"}
        _progress(f"bf16_n8192_backward: {extras['bf16_n8192_backward']}")
        del dout, dq, dk, dv, ws
        # Context for the HBM-bound rows: the read bandwidth a plain
        # streaming kernel reaches on this card (4 GiB read once per launch,
        # eight 16-byte loads in flight per thread, 64 workgroups per CU,
        # the best of 2-64 measured; fa_probe_read).
        read_gbs = None
        probe_r = os.path.join(os.path.dirname(fa.__file__), "libfa_probe.so")
        if os.path.exists(probe_r):
            import ctypes
            rlib = ctypes.CDLL(probe_r)
            rlib.fa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_ulonglong,
                                           ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p]
            rlib.fa_probe_read.restype = ctypes.c_int
            rbuf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
            rgrid = 64 * torch.cuda.get_device_properties(0).multi_processor_count
            rsink = torch.zeros(rgrid, dtype=torch.int32, device=dev)
            rstream = torch.cuda.current_stream().cuda_stream

            def _read_once():
                rc = rlib.fa_probe_read(rbuf.data_ptr(), rbuf.numel(), rgrid,
                                        rsink.data_ptr(), rstream)
                if rc != 0:
                    raise RuntimeError(f"fa_probe_read = {rc}")

            tm_r = _time_launches(_read_once, 10, 5, min_warm_ms=30.0)
            read_gbs = rbuf.numel() / (tm_r["mean"] * 1e-3) / 1e9
            extras["hbm_read_probe_4gib"] = {
                "ms": round(tm_r["mean"], 4), "GB/s": round(read_gbs, 1),
                "frac_of_hbm_peak": round(read_gbs / HBM_PEAK_GBS, 4),
                "what": "one streaming read of 4 GiB (fa_probe_read)"}
            _progress(f"hbm_read_probe_4gib: {extras['hbm_read_probe_4gib']}")
            del rbuf, rsink
        # Decode at long context through the split-KV forward: one query
        # per head, 32 query heads on 8 KV heads, 65536 keys, B = 8.  Bound
        # by HBM: K and V are read once (the algorithmic bytes).
        B_, H_, Hkv_, Nk_ = 8, 32, 8, 65536
        gk = torch.Generator(device=dev).manual_seed(13)
        qd = torch.randn((B_, H_, 1, 128), device=dev, generator=gk).to(torch.bfloat16)
        kd = torch.randn((B_, Hkv_, Nk_, 128), device=dev, generator=gk).to(torch.bfloat16)
        vd = torch.randn((B_, Hkv_, Nk_, 128), device=dev, generator=gk).to(torch.bfloat16)
        ns = fa.library().fa_splitkv_num_splits(B_, H_, Hkv_, 1, Nk_)
        od = torch.empty_like(qd)
        ld = torch.empty((B_, H_, 1), dtype=torch.float32, device=dev)
        wd = torch.empty(ns * B_ * H_ * 129, dtype=torch.float32, device=dev)
        tm_d = _time_launches(
            lambda: fa.forward_kv(qd, kd, vd, causal=True, num_splits=ns,
                                  out=od, lse=ld, workspace=wd), 20, 10, min_warm_ms=30.0)
        kv_bytes = 2 * kd.numel() * 2
        gbs = kv_bytes / (tm_d["mean"] * 1e-3) / 1e9
        extras["decode_b8_h32_hkv8_nk65536"] = {
            "ms": round(tm_d["mean"], 4), "ms_median": round(tm_d["median"], 4),
            "ms_min": round(tm_d["min"], 4), "GB/s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "frac_of_read_probe": round(gbs / read_gbs, 4) if read_gbs else None,
            "num_splits": ns, "bytes": "K and V once"}
        _progress(f"decode_b8_h32_hkv8_nk65536: {extras['decode_b8_h32_hkv8_nk65536']}")
        del qd, kd, vd, od, ld, wd
        # Variable-length batch with a causal sliding window (4096 keys to the
        # left): 8 sequences of 2K..16K tokens, 32 query heads on 8 KV heads.
        # FLOPs count 4 d per visible (query, key) pair.
        lens = [16384, 2048, 8192, 4096, 12288, 2048, 6144, 14336]
        win = 4096
        tot = sum(lens)
        gv = torch.Generator(device=dev).manual_seed(17)
        qv_ = torch.randn((32, tot, 128), device=dev, generator=gv).to(torch.bfloat16)
        kv_ = torch.randn((8, tot, 128), device=dev, generator=gv).to(torch.bfloat16)
        vv_ = torch.randn((8, tot, 128), device=dev, generator=gv).to(torch.bfloat16)
        cu = torch.tensor([0] + list(itertools.accumulate(lens)),
                          dtype=torch.int32, device=dev)
        ov_ = torch.empty_like(qv_)
        lv_ = torch.empty((32, tot), dtype=torch.float32, device=dev)
        tm_v = _time_launches(
            lambda: fa.forward_varlen(qv_, kv_, vv_, cu, cu, max(lens),
                                      causal=True, window=(win, -1),
                                      out=ov_, lse=lv_), 20, 10,
            min_warm_ms=30.0)
        pairs = sum(sum(min(i, win) + 1 for i in range(n)) for n in lens)
        tvl = 4 * 128 * 32 * pairs / (tm_v["mean"] * 1e-3) / 1e12
        extras["varlen_causal_window4096"] = {
            "ms": round(tm_v["mean"], 4), "ms_median": round(tm_v["median"], 4),
            "ms_min": round(tm_v["min"], 4), "TFLOP/s": round(tvl, 1),
            "frac_of_bf16_peak": round(tvl / BF16_PEAK_TFLOPS, 4),
            "flops": "4 d per visible (query, key) pair"}
        _progress(f"varlen_causal_window4096: {extras['varlen_causal_window4096']}")
        del qv_, kv_, vv_, ov_, lv_
        # Arbitrary masks on the headline shape (B4 H16 N8192 d128), one
        # mask shared by every (batch, head): a block-sparse pattern of
        # 128 x 128 squares (key block 0, the local band of three blocks and
        # 8 random blocks per query block), and the all-visible mask, whose
        # time against the unmasked kernel is the cost of masking itself.
        # FLOPs count 4 d per visible (query, key) pair.
        for mname, mbool in (
                ("masked_block_sparse_n8192",
                 workloads.block_sparse_mask(w.N, w.N, 128, 8, 23)),
                ("masked_all_visible_n8192",
                 np.ones((w.N, w.N), dtype=bool))):
            mw_ = torch.from_numpy(workloads.pack_mask(mbool)[None, None]
                                   .view(np.int32)).to(dev)
            tm_m = _time_launches(
                lambda: fa.forward_masked(q, k, v, mw_, out=o, lse=lse),
                20, 10, min_warm_ms=30.0)
            vis = float(mbool.sum())
            tmk = 4 * w.d * w.B * w.H * vis / (tm_m["mean"] * 1e-3) / 1e12
            extras[mname] = {
                "ms": round(tm_m["mean"], 4),
                "ms_median": round(tm_m["median"], 4),
                "ms_min": round(tm_m["min"], 4), "TFLOP/s": round(tmk, 1),
                "frac_of_bf16_peak": round(tmk / BF16_PEAK_TFLOPS, 4),
                "visible_fraction": round(vis / float(w.N) ** 2, 4),
                "flops": "4 d per visible (query, key) pair"}
            _progress(f"{mname}: {extras[mname]}")
            del mw_
        ww = workloads.WORKLOADS["fp8_n8192"]
        xq, xk, xv = (torch.from_numpy(x).to(dev)
                      for x in workloads.workload_qkv(ww))
        signs = workloads.hadamard_signs(ww.d, ww.seed(9))
        for rot in (False, True):
            s = signs if rot else None
            q8, sq = fa.quantize_fp8(xq, s)
            k8, sk = fa.quantize_fp8(xk, s)
            v8, sv = fa.quantize_fp8(xv, None)
            desc = torch.stack([sq[1], sk[1], sv[1]]).contiguous()
            oo = torch.empty((ww.B, ww.H, ww.N, ww.d), dtype=torch.bfloat16,
                             device=dev)
            ll = torch.empty((ww.B, ww.H, ww.N), dtype=torch.float32,
                             device=dev)
            tm = _time_launches(lambda: fa.forward_fp8(q8, k8, v8, desc,
                                                       out=oo, lse=ll), 20, 20, min_warm_ms=30.0)
            m = tm["mean"]
            t = ww.flops / (m * 1e-3) / 1e12
            key = "fp8_n8192" + ("_hadamard" if rot else "")
            extras[key] = {"ms": round(m, 4), "ms_median": round(tm["median"], 4),
                           "ms_min": round(tm["min"], 4), "TFLOP/s": round(t, 1),
                           "frac_of_fp8_peak": round(t / FP8_PEAK_TFLOPS, 4)}
            _progress(f"{key}: {extras[key]}")
            if rot:
                continue
            # Part of each tile's exponentials on the FMA pipe
            # (fa_fwd_fp8_exp2_fma), against v_exp_f32 above: 4, 8 or 16 of
            # a lane's 16 pairs per 64-key tile.
            for pairs in (4, 8, 16):
                tm = _time_launches(
                    lambda: fa.forward_fp8(q8, k8, v8, desc, out=oo, lse=ll,
                                           exp2_fma_pairs=pairs),
                    20, 20, min_warm_ms=30.0)
                t = ww.flops / (tm["mean"] * 1e-3) / 1e12
                key = f"fp8_n8192_exp2_fma_{pairs}_of_16_pairs"
                extras[key] = {
                    "ms": round(tm["mean"], 4),
                    "ms_median": round(tm["median"], 4),
                    "TFLOP/s": round(t, 1),
                    "frac_of_fp8_peak": round(t / FP8_PEAK_TFLOPS, 4),
                    "vs_v_exp_f32": round(m / tm["mean"], 4)}
                _progress(f"{key}: {extras[key]}")
        mq = _time_launches(lambda: fa.quantize_fp8(xq, signs), 20, 20, min_warm_ms=30.0)["mean"]
        nbytes = xq.numel() * (4 * 2 + 1)      # fp32 read twice, e4m3 write
        extras["fp8_quantize_hadamard_per_tensor"] = {
            "ms": round(mq, 4), "GB/s": round(nbytes / (mq * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (mq * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        _progress(f"fp8_quantize_hadamard_per_tensor: {extras['fp8_quantize_hadamard_per_tensor']}")
        del xq, xk, xv, q8, k8, v8, oo, ll
        # Context, not part of the path: the matrix rate the card sustains
        # under its power limit on N(0,1) operands (MFMAs only, no softmax,
        # no memory traffic).
        probe = os.path.join(os.path.dirname(fa.__file__), "libfa_probe.so")
        if os.path.exists(probe):
            import ctypes
            plib = ctypes.CDLL(probe)
            plib.fa_probe_rates.argtypes = [ctypes.c_int] * 6 + \
                [ctypes.c_void_p] * 3
            plib.fa_probe_rates.restype = ctypes.c_int
            extras["mfma_only_randn_ceiling"] = _mfma_ceiling(plib)
        # Context, not part of the path: the vendor bf16 GEMM (hipBLASLt via
        # torch.matmul) on N(0,1) operands of the same distribution, i.e. what
        # a tuned library contraction reaches on this card under its power
        # limit.
        g = torch.Generator(device=dev).manual_seed(7)
        a = torch.randn((8192, 8192), device=dev, generator=g).to(torch.bfloat16)
        bt = torch.randn((8192, 8192), device=dev, generator=g).to(torch.bfloat16)
        c = torch.empty((8192, 8192), device=dev, dtype=torch.bfloat16)
        mg = _time_launches(lambda: torch.matmul(a, bt, out=c), 20, 5, min_warm_ms=30.0)["mean"]
        tg = 2 * 8192 ** 3 / (mg * 1e-3) / 1e12
        extras["library_gemm_bf16_8192_randn"] = {
            "ms": round(mg, 4), "TFLOP/s": round(tg, 1),
            "frac_of_bf16_peak": round(tg / BF16_PEAK_TFLOPS, 4)}
        _progress(f"library_gemm_bf16_8192_randn: {extras['library_gemm_bf16_8192_randn']}")
        del a, bt, c

    cpu = None
    if not args.no_cpu and rank == 0:
        cpu = _cpu_baseline(w, host, args.cpu_budget)
        cpu["gpu_over_oracle"] = round(tflops / cpu["value"], 1)

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_median": round(head["median"], 4),
        "ms_min": round(head["min"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.Hkv,
                   "N": w.N, "d": w.d, "causal": w.causal},
        "frac_of_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
        "clock_under_load": clock,
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
            "traffic": _traffic("fwd_bf16_d128"),
            "kernel": "fwd_bf16_kernel<128, false, 2, false, false, 4>",
            "flops_per_launch": w.flops,
            "peak_basis": f"{cus} CUs x 4096 bf16 FLOP/clk x 2.4 GHz",
        },
        "cpu_baseline": cpu,
        "extras": extras,
        "gpu": torch.cuda.get_device_properties(0).name,
    }
    if rank == 0:
        print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
