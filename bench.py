"""Benchmark: throughput of the dense-BF16 MLP block at M = 5120 on one MI355X.

A step is the MLP block of a 2B-class decoder at one packed LoRA step (the
sm121a_matmul.py page's shape list): gate and up projections
A[5120,2048] x W[11008,2048]^T (two separate products with their own weights
and outputs, computed in one launch by gemm_bf16_dual), then the down projection
H[5120,11008] x W[2048,11008]^T through split-K (best k_splits of 1/2/4/8,
chosen during warm-up). Inputs are seeded synthetic BF16 tensors resident in
HBM before timing starts. `value` = 3 * 2*M*N*K flops per step / step time.

Every other row of the hot path is timed in the same run and reported under
"rows": attention projections, the fused LoRA fold (HBM roofline), the
order-preserving router GEMM (FP32 VALU roofline), the block-scaled FP4 GEMM
(and its M = 128 decode shapes through split-K), W4A16 and the small dense case, each warm and after a 1 GiB cache flush
(median with p20/p80), each with the oracle timed beside it on a bounded
sample of its rows (`oracle_*` fields, extrapolated to the full problem).

Output: one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0     # MI355X dense BF16 MFMA, published
FP4_PEAK_TFLOPS = 10100.0     # MI355X dense FP4 MFMA, published
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, published
# FP32 vector ALU without FMA: the published 157.3 TFLOP/s counts two flops
# per FMA lane, i.e. 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz FP32 operations;
# a plain multiply or add issues at the same lane rate, so a multiply plus an
# add per multiply-accumulate peaks at 78.6 TFLOP/s of GEMM flops.
VALU_NOFMA_PEAK_TFLOPS = 256 * 4 * 32 * 2.4e9 / 1e12

M, HID, INTER = 5120, 2048, 11008


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--splitk", default="auto", help="auto or a fixed k_splits for the down projection")
    p.add_argument("--no-rows", action="store_true", help="skip the per-row table")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--row-oracle-seconds", type=float, default=1.0,
                   help="oracle time budget per row (0 skips the per-row oracle timings)")
    p.add_argument("--calib-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (counter calibration) and exit")
    p.add_argument("--profile-rows", action="store_true",
                   help="only run every row's call 3 times, untimed (for counter passes), and exit")
    p.add_argument("--data-ceiling", action="store_true",
                   help="only time the gate+up dual call on random, constant and zero operands (same "
                        "kernels, different switching activity) with the engine clock, print JSON and exit")
    p.add_argument("--streamk", action="store_true",
                   help="only time gemm_bf16, gemm_bf16_streamk (both tiles) and gemm_bf16_splitk on the "
                        "attention, MLP and deep-K shapes, print JSON and exit")
    return p.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_scaled_fp4_gemm_amd as bg
    import synthetic

    dev = "cuda:0"
    torch.cuda.set_device(0)

    if args.calib_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 3 x 1 GiB device-to-device")
        return

    def up16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def u8(b):
        return torch.from_numpy(np.ascontiguousarray(b)).to(dev)

    if args.profile_rows:
        profile_rows(bg, synthetic, torch, up16, u8, dev)
        return

    if args.data_ceiling:
        print(json.dumps(data_ceiling(bg, synthetic, torch, np, up16, dev)), flush=True)
        return

    if args.streamk:
        print(json.dumps(streamk_compare(bg, synthetic, torch, np, up16, dev)), flush=True)
        return

    t_gen = time.time()
    x_np, wg_np = synthetic.mlp_gate_up()
    wu_np = synthetic.normal_bf16((INTER, HID), 0.02, 2, synthetic.TID_B2 + 10)
    h_np, wd_np = synthetic.mlp_down()
    X, Wg, Wu, H, Wd = up16(x_np), up16(wg_np), up16(wu_np), up16(h_np), up16(wd_np)
    G = torch.empty((M, INTER), dtype=torch.bfloat16, device=dev)
    U = torch.empty((M, INTER), dtype=torch.bfloat16, device=dev)
    D = torch.empty((M, HID), dtype=torch.bfloat16, device=dev)
    WS = torch.empty((8, M, HID), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"inputs generated and uploaded in {time.time() - t_gen:.1f}s")

    stream = torch.cuda.current_stream()

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def down(ks):
        bg.gemm_bf16_splitk(H, Wd, ks, workspace=WS, out=D)

    # Choose the down-projection split during warm-up, in context: whole
    # steps (gate, up, down) with each candidate, in interleaved rounds, so
    # the clock state the down GEMM sees is the one of the timed loop.
    # gate and up: two products of X in one launch (gemm_bf16_dual), so their
    # tiles share the rounds of one grid
    def gate_up():
        bg.gemm_bf16_dual(X, Wg, Wu, out0=G, out1=U)

    def step_with(ks):
        gate_up()
        down(ks)

    # The timed regions run with Python's cyclic garbage collector off (as
    # timeit does): a collection during a long unsynchronised launch sequence
    # was seen to block the host for tens of milliseconds while the queue
    # drained, leaving the GPU idle inside the timed region.
    gc.collect()
    gc.disable()

    if args.splitk == "auto":
        cands = (1, 2, 4, 8)
        times = {ks: [] for ks in cands}
        for _ in range(3):
            for ks in cands:
                step_with(ks)
                s = ev()
                for _ in range(5):
                    step_with(ks)
                e = ev()
                torch.cuda.synchronize()
                times[ks].append(s.elapsed_time(e) / 5)
        for ks in cands:
            log(f"step with down k_splits={ks}: {np.median(times[ks]) * 1e3:.1f} us (median of 3 rounds)")
        ks_down = min(cands, key=lambda k: float(np.median(times[k])))
    else:
        ks_down = int(args.splitk)

    def step(rec=None):
        e0 = ev() if rec is not None else None
        gate_up()
        e1 = ev() if rec is not None else None
        down(ks_down)
        if rec is not None:
            rec.append((e0, e1, ev()))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    rec = []
    start = ev()
    for _ in range(args.steps):
        step(rec)
    end = ev()
    torch.cuda.synchronize()
    gc.enable()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    flops_gemm = 2.0 * M * INTER * HID
    flops_step = 3 * flops_gemm
    value = flops_step / (ms_step * 1e-3) / 1e12

    gate_up_ms = [r[0].elapsed_time(r[1]) for r in rec]
    down_ms = [r[1].elapsed_time(r[2]) for r in rec]
    gu_avg = float(np.mean(gate_up_ms))
    achieved = 2 * flops_gemm / (gu_avg * 1e-3) / 1e12
    log(f"step {ms_step * 1e3:.1f} us: gate+up (dual) {gu_avg * 1e3:.1f} us avg, "
        f"down {np.mean(down_ms) * 1e3:.1f} us avg")

    # GPU engine clock while the same step runs on (outside the timed region):
    # the BF16 peak at the measured clock puts the achieved rate in context.
    clocks = sample_sclk(lambda: step(), seconds=0.3, sync=torch.cuda.synchronize)
    if clocks is not None:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        peak_at = cus * 4096 * clocks["sclk_mhz_mean"] * 1e6 / 1e12
        clocks["cus"] = cus
        clocks["bf16_peak_at_sclk_tflops"] = round(peak_at, 1)
        clocks["gate_up_frac_at_sclk"] = round(achieved / peak_at, 4)
        log(f"sclk {clocks['sclk_mhz_mean']:.0f} MHz mean over {clocks['samples']} samples: "
            f"BF16 peak at that clock {peak_at:.0f} TFLOP/s")

    roofline = {
        "bound": "mfma",
        "kernel": ("gemm_bf16_dual MLP gate+up call (two 5120x11008x2048 products of one X, per call): one "
                   "dispatch of gemm_mfma_direct_kernel 256x256 tiles, 1720 tiles"),
        "achieved": round(achieved, 1),
        "peak": BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
        "traffic": traffic_for_current_kernel(),
    }

    result = {
        "metric": "TFLOP/s and % of bf16 MFMA peak at M=5120 MLP gate/up/down shapes",
        "value": round(value, 1),
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
        "config": {
            "workload": "MLP block at M=5120: gate and up 5120x11008x2048, down 5120x2048x11008 split-K",
            "m": M, "hidden": HID, "intermediate": INTER, "down_k_splits": ks_down,
            "parallelism": "none (1 GPU)",
        },
        "pct_of_bf16_peak": round(100.0 * value / BF16_PEAK_TFLOPS, 2),
        "gate_up_dual_us": round(gu_avg * 1e3, 2),
        "down_us": round(float(np.mean(down_ms)) * 1e3, 2),
        "roofline": roofline,
        "clocks": clocks,
    }

    if not args.no_rows:
        result["rows"] = measure_rows(bg, synthetic, torch, np, up16, u8, dev, stream, args.row_oracle_seconds)

    del X, Wg, Wu, H, Wd, G, U, D, WS
    torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(
            [("gate", x_np, wg_np), ("up", x_np, wu_np), ("down", h_np, wd_np)], args.cpu_seconds)

    print(json.dumps(result), flush=True)


def sample_sclk(run_once, seconds, sync):
    """Runs run_once() back to back for about `seconds` while a thread reads
    the active engine-clock and memory-clock levels (the lines marked '*' in
    the driver's pp_dpm_sclk and pp_dpm_mclk files) every 2 ms. Returns the
    engine clock's mean, min and max MHz, the memory clock's mean MHz and the
    sample count, or None when no engine-clock file is readable."""
    import glob
    import threading
    cards = sorted(glob.glob("/sys/class/drm/card*/device"))

    def read(path):
        try:
            with open(path) as f:
                for line in f:
                    if "*" in line:
                        return float(line.split(":")[1].strip().lower().split("mhz")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    cards = [c for c in cards if read(c + "/pp_dpm_sclk") is not None]
    if not cards:
        return None
    samples = {c: [] for c in cards}
    msamples = {c: [] for c in cards}
    stop = threading.Event()

    def poll():
        while not stop.is_set():
            for c in cards:
                v = read(c + "/pp_dpm_sclk")
                if v is not None:
                    samples[c].append(v)
                m = read(c + "/pp_dpm_mclk")
                if m is not None:
                    msamples[c].append(m)
            time.sleep(0.002)

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t_end = time.time() + seconds
    while time.time() < t_end:
        for _ in range(10):
            run_once()
        sync()
    stop.set()
    th.join()
    # the GPU under load is the card whose engine clock ran highest
    best = max(cards, key=lambda c: sum(samples[c]) / max(1, len(samples[c])))
    v, mv = samples[best], msamples[best]
    if not v:
        return None
    res = {"sclk_mhz_mean": round(sum(v) / len(v), 1), "sclk_mhz_min": min(v), "sclk_mhz_max": max(v),
           "samples": len(v), "source": best + "/pp_dpm_sclk"}
    if mv:
        res["mclk_mhz_mean"] = round(sum(mv) / len(mv), 1)
    return res


def traffic_for_current_kernel():
    """HBM bytes per gate+up dual call from the committed counter
    summary, or None if the GEMM kernel source changed since the counters
    were taken."""
    path = os.path.join(ROOT, "profiles", "traffic_gate_up.json")
    src = os.path.join(ROOT, "block_scaled_fp4_gemm_amd", "csrc", "gemm_mfma.hip")
    try:
        rec = json.load(open(path))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if rec.get("kernel_source_sha256") != sha:
            return None
        return rec.get("traffic_bytes_per_launch")
    except (OSError, ValueError):
        return None


def data_ceiling(bg, synthetic, torch, np, up16, dev):
    """The gate+up dual call (2 x 5120x11008x2048) timed on three operand
    sets that run the identical instruction stream: the workload's random
    BF16 values, a constant (every element 1.0, so each MFMA sees the same
    operands) and all zeros. A GEMM whose time depends on the values it
    multiplies is limited by power (the engine clock falls with switching
    activity), not by its schedule. Each set: 5 warm-up calls, then 40 calls
    in 4 interleaved rounds of 10, while the engine clock is sampled."""
    x, wg = synthetic.mlp_gate_up()
    wu = synthetic.normal_bf16((INTER, HID), 0.02, 2, synthetic.TID_B2 + 10)
    sets = {
        "random": (up16(x), up16(wg), up16(wu)),
        "constant_one": tuple(torch.ones(s, dtype=torch.bfloat16, device=dev)
                              for s in ((M, HID), (INTER, HID), (INTER, HID))),
        "zero": tuple(torch.zeros(s, dtype=torch.bfloat16, device=dev)
                      for s in ((M, HID), (INTER, HID), (INTER, HID))),
    }
    G = torch.empty((M, INTER), dtype=torch.bfloat16, device=dev)
    U = torch.empty((M, INTER), dtype=torch.bfloat16, device=dev)
    flops = 2 * 2.0 * M * INTER * HID
    stream = torch.cuda.current_stream()
    times = {k: [] for k in sets}
    clocks = {}
    gc.collect()
    gc.disable()
    for name, (X, Wg, Wu) in sets.items():
        for _ in range(5):
            bg.gemm_bf16_dual(X, Wg, Wu, out0=G, out1=U)
        torch.cuda.synchronize()
        clocks[name] = sample_sclk(lambda: bg.gemm_bf16_dual(X, Wg, Wu, out0=G, out1=U), seconds=0.3,
                                   sync=torch.cuda.synchronize)
    for r in range(4):
        for name in (list(sets) if r % 2 == 0 else list(sets)[::-1]):
            X, Wg, Wu = sets[name]
            bg.gemm_bf16_dual(X, Wg, Wu, out0=G, out1=U)
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record(stream)
            for _ in range(10):
                bg.gemm_bf16_dual(X, Wg, Wu, out0=G, out1=U)
            e.record(stream)
            torch.cuda.synchronize()
            times[name].append(s.elapsed_time(e) / 10 * 1e3)
    gc.enable()
    out = {"call": "gemm_bf16_dual 2 x 5120x11008x2048 (gate+up)"}
    for name in sets:
        us = float(np.median(times[name]))
        out[name] = {"us": round(us, 1), "tflops": round(flops / us / 1e6, 1),
                     "frac_bf16_peak": round(flops / us / 1e6 / BF16_PEAK_TFLOPS, 4),
                     "sclk_mhz_mean": None if clocks[name] is None else clocks[name]["sclk_mhz_mean"]}
        log(f"data ceiling {name}: {out[name]}")
    return out


def streamk_compare(bg, synthetic, torch, np, up16, dev):
    """The stream-K entry point against the data-parallel one (and split-K
    with k = 2, 4, 8) on the attention and MLP shapes and two deep-K shapes
    with fewer tiles than CUs. Random BF16 operands (X ~ N(0,1), W ~
    N(0,0.02)); per variant the median of four interleaved rounds of 20
    back-to-back calls."""
    shapes = [(5120, 512, 2048), (5120, 2048, 2048), (5120, 2048, 11008), (5120, 11008, 2048),
              (1024, 1024, 8192), (512, 1024, 16384), (2048, 4096, 4096)]
    out = {"unit": "us per call (TFLOP/s)"}
    stream = torch.cuda.current_stream()

    def timed(fn, n=20):
        fn()
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(n):
            fn()
        e.record(stream)
        torch.cuda.synchronize()
        return s.elapsed_time(e) / n * 1e3

    for m, n, k in shapes:
        A = up16(synthetic.normal_bf16((m, k), 1.0, 1, 0))
        B = up16(synthetic.normal_bf16((n, k), 0.02, 2, 1))
        C = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        wss = {}
        for cfg in (23, 10):
            bg.tune_set(bg.TUNE_STREAMK_TILE, cfg)
            wss[cfg] = torch.empty(bg.gemm_bf16_streamk_workspace(m, n, k), dtype=torch.uint8, device=dev)
        bg.tune_set(bg.TUNE_STREAMK_TILE, -1)
        planes = torch.empty((8, m, n), dtype=torch.float32, device=dev)

        def sk(cfg):
            def f():
                bg.tune_set(bg.TUNE_STREAMK_TILE, cfg)
                bg.gemm_bf16_streamk(A, B, workspace=wss[cfg], out=C)
            return f

        variants = {"data_parallel": lambda: bg.gemm_bf16(A, B, out=C),
                    "streamk_128x128": sk(23), "streamk_256x128": sk(10)}
        for ks in (2, 4, 8):
            variants[f"splitk_{ks}"] = (lambda ks=ks: bg.gemm_bf16_splitk(A, B, ks, workspace=planes, out=C))
        res = {v: [] for v in variants}
        gc.collect()
        gc.disable()
        for r in range(4):
            for v in (list(variants) if r % 2 == 0 else list(variants)[::-1]):
                res[v].append(timed(variants[v]))
        gc.enable()
        bg.tune_set(bg.TUNE_STREAMK_TILE, -1)
        fl = 2.0 * m * n * k
        row = {v: f"{np.median(t):.1f} ({fl / np.median(t) / 1e6:.0f})" for v, t in res.items()}
        ws_default = bg.gemm_bf16_streamk_workspace(m, n, k)
        row["streamk_default_tile"] = "128x128" if ws_default == wss[23].numel() else "256x128"
        out[f"{m}x{n}x{k}"] = row
        log(f"streamk compare {m}x{n}x{k}: {row}")
        del A, B, C, wss, planes
    return out


def profile_rows(bg, synthetic, torch, up16, u8, dev):
    """Every row's library call on its workload, three times each, in the
    order of the per-row table (kernel names tell the rows apart in a
    counter pass)."""
    calls = []
    a, b = synthetic.attn_proj()
    A, B = up16(a), up16(b)
    calls.append(("attn_qo", lambda: bg.gemm_bf16(A, B)))
    a2, b2 = synthetic.attn_proj(n=512)
    A2, B2 = up16(a2), up16(b2)
    calls.append(("attn_kv", lambda: bg.gemm_bf16(A2, B2)))
    x, w = synthetic.mlp_gate_up()
    X, W = up16(x), up16(w)
    calls.append(("mlp_gate_up", lambda: bg.gemm_bf16(X, W)))
    W2 = up16(synthetic.normal_bf16((INTER, HID), 0.02, 2, synthetic.TID_B2 + 10))
    calls.append(("mlp_gate_up_dual", lambda: bg.gemm_bf16_dual(X, W, W2)))
    h, wd = synthetic.mlp_down()
    H, WD = up16(h), up16(wd)
    calls.append(("mlp_down_k1", lambda: bg.gemm_bf16(H, WD)))
    out, xl, bl, sc = synthetic.lora_fold()
    O, XL, BL = up16(out), up16(xl), up16(bl)
    calls.append(("lora_fold", lambda: bg.gemm_bf16_scaled_acc(XL, BL, O, sc)))
    for m in (4510, 2255):
        xr, wr = synthetic.router(m=m)
        XR, WR = up16(xr), up16(wr)
        calls.append((f"router_{m}", lambda XR=XR, WR=WR: bg.gemm_bf16_ordered(XR, WR)))
    fa, fsa, fb, fsb = synthetic.fp4_gemm()
    FA, FSA, FB, FSB = u8(fa), u8(fsa), u8(fb), u8(fsb)
    calls.append(("fp4", lambda: bg.gemm_fp4_blockscaled(FA, FSA, FB, FSB)))
    da, dsa, db, dsb = synthetic.fp4_decode()
    DA, DSA, DB, DSB = u8(da), u8(dsa), u8(db), u8(dsb)
    WS = torch.empty(8 * 128 * 7168, dtype=torch.float32, device=dev)
    calls.append(("fp4_decode_k8", lambda: bg.gemm_fp4_blockscaled_splitk(DA, DSA, DB, DSB, 8, workspace=WS)))
    ea, esa, eb, esb = synthetic.fp4_decode(m=128, n=4096, k=7168)
    EA, ESA, EB, ESB = u8(ea), u8(esa), u8(eb), u8(esb)
    WS2 = torch.empty(8 * 128 * 4096, dtype=torch.float32, device=dev)
    calls.append(("fp4_decode_4096_k8",
                  lambda: bg.gemm_fp4_blockscaled_splitk(EA, ESA, EB, ESB, 8, workspace=WS2)))
    wa, wb, wsb, s2 = synthetic.w4a16_gemm()
    WA, WB, WSB = up16(wa), u8(wb), u8(wsb)
    calls.append(("w4a16", lambda: bg.gemm_w4a16(WA, WB, WSB, s2)))
    for name, fn in calls:
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        log(f"profiled row {name}")


def oracle_timing(fn_rows, total_rows, block, seconds):
    """Runs the oracle on consecutive row blocks [r0, r1) until `seconds` of
    wall time (at least one block) and extrapolates to all rows."""
    if seconds <= 0:
        return {}
    t0 = time.time()
    done = 0
    while done < total_rows and (done == 0 or time.time() - t0 < seconds):
        r1 = min(total_rows, done + block)
        fn_rows(done, r1)
        done = r1
    dt = time.time() - t0
    return {"oracle_us_extrapolated": round(dt / done * total_rows * 1e6, 1),
            "oracle_sample": f"{done} of {total_rows} rows in {dt:.2f} s"}


def measure_rows(bg, synthetic, torch, np, up16, u8, dev, stream, oracle_seconds):
    import oracle

    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    spread = {}

    def timed(fn, reps=50, batch=10, batches=8):
        """Per-call time in us, warm and cold (p20/p80 kept in `spread`),
        after 5 untimed calls, with calls enqueued back to back (no host
        synchronisation between them). Warm: `batches` pairs of events on the
        stream, each around `batch` consecutive calls; the median per-call
        time of the batches. An event pair around every single call adds about
        2 us to each call (measured on 16-40 us calls), which a batch spreads
        over its calls; the step itself is timed the same way. Cold: `reps`
        calls, each preceded by a 1 GiB write that evicts the L2s and the
        256 MB Infinity Cache and inside its own pair of events; the median."""
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        res = {}
        gc.collect()
        gc.disable()
        pairs = []
        for _ in range(batches):
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record(stream)
            for _ in range(batch):
                fn()
            e.record(stream)
            pairs.append((s, e))
        torch.cuda.synchronize()
        us = [a.elapsed_time(b) * 1e3 / batch for a, b in pairs]
        res["warm"] = float(np.median(us))
        spread["warm"] = [round(float(np.percentile(us, 20)), 2), round(float(np.percentile(us, 80)), 2)]
        pairs = []
        for _ in range(reps):
            flush.zero_()
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record(stream)
            fn()
            e.record(stream)
            pairs.append((s, e))
        torch.cuda.synchronize()
        us = [a.elapsed_time(b) * 1e3 for a, b in pairs]
        res["cold"] = float(np.median(us))
        spread["cold"] = [round(float(np.percentile(us, 20)), 2), round(float(np.percentile(us, 80)), 2)]
        gc.enable()
        return res["warm"], res["cold"]

    def with_spread(d):
        d["us_warm_p20_p80"] = spread["warm"]
        d["us_cold_p20_p80"] = spread["cold"]
        return d

    rows = {}

    def dense_row(name, m, n, k, a, b):
        A, B = up16(a), up16(b)
        C = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        w, c = timed(lambda: bg.gemm_bf16(A, B, out=C))
        fl = 2.0 * m * n * k
        rows[name] = with_spread({"shape": [m, n, k], "us_warm": round(w, 2), "us_cold": round(c, 2),
                                  "tflops_warm": round(fl / w / 1e6, 1), "tflops_cold": round(fl / c / 1e6, 1),
                                  "frac_bf16_peak_warm": round(fl / w / 1e6 / BF16_PEAK_TFLOPS, 4)})
        rows[name].update(oracle_timing(lambda r0, r1: oracle.gemm_bf16_ref(a[r0:r1], b), m, 32, oracle_seconds))
        log(name, rows[name])

    a, b = synthetic.dense_small()
    dense_row("dense_128x256x512", 128, 256, 512, a, b)
    a, b = synthetic.attn_proj(n=2048)
    dense_row("attn_qo_5120x2048x2048", 5120, 2048, 2048, a, b)
    a, b = synthetic.attn_proj(n=512)
    dense_row("attn_kv_5120x512x2048", 5120, 512, 2048, a, b)

    def streamk_row(name, m, n, k, a, b):
        """The same product through the stream-K entry point (its workspace
        allocated once, outside the timed calls)."""
        A, B = up16(a), up16(b)
        C = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        need = bg.gemm_bf16_streamk_workspace(m, n, k)
        WS = torch.empty(need, dtype=torch.uint8, device=dev)
        w, c = timed(lambda: bg.gemm_bf16_streamk(A, B, workspace=WS, out=C))
        fl = 2.0 * m * n * k
        rows[name] = with_spread({"shape": [m, n, k], "us_warm": round(w, 2), "us_cold": round(c, 2),
                                  "tflops_warm": round(fl / w / 1e6, 1), "tflops_cold": round(fl / c / 1e6, 1),
                                  "frac_bf16_peak_warm": round(fl / w / 1e6 / BF16_PEAK_TFLOPS, 4),
                                  "workspace_bytes": need})
        log(name, rows[name])

    streamk_row("attn_kv_5120x512x2048_streamk", 5120, 512, 2048, a, b)
    a, b = synthetic.attn_proj(n=2048)
    streamk_row("attn_qo_5120x2048x2048_streamk", 5120, 2048, 2048, a, b)
    a, b = synthetic.mlp_gate_up()
    dense_row("mlp_gate_up_5120x11008x2048", 5120, 11008, 2048, a, b)
    # both projections in one launch (the step's form)
    A, B = up16(a), up16(b)
    B2 = up16(synthetic.normal_bf16((INTER, HID), 0.02, 2, synthetic.TID_B2 + 10))
    C1 = torch.empty((5120, 11008), dtype=torch.bfloat16, device=dev)
    C2 = torch.empty((5120, 11008), dtype=torch.bfloat16, device=dev)
    w, c = timed(lambda: bg.gemm_bf16_dual(A, B, B2, out0=C1, out1=C2))
    fl = 2 * 2.0 * 5120 * 11008 * 2048
    rows["mlp_gate_up_dual_2x5120x11008x2048"] = with_spread({
        "shape": [5120, 11008, 2048], "products": 2, "us_warm": round(w, 2), "us_cold": round(c, 2),
        "tflops_warm": round(fl / w / 1e6, 1), "tflops_cold": round(fl / c / 1e6, 1),
        "frac_bf16_peak_warm": round(fl / w / 1e6 / BF16_PEAK_TFLOPS, 4)})
    log("mlp_gate_up_dual", rows["mlp_gate_up_dual_2x5120x11008x2048"])
    del A, B, B2, C1, C2

    h, wd = synthetic.mlp_down()
    H, WD = up16(h), up16(wd)
    D = torch.empty((5120, 2048), dtype=torch.bfloat16, device=dev)
    WS = torch.empty((8, 5120, 2048), dtype=torch.float32, device=dev)
    fl = 2.0 * 5120 * 2048 * 11008
    for ks in (1, 2, 4, 8):
        w, c = timed(lambda: bg.gemm_bf16_splitk(H, WD, ks, workspace=WS, out=D))
        rows[f"mlp_down_5120x2048x11008_k{ks}"] = with_spread({
            "us_warm": round(w, 2), "us_cold": round(c, 2), "tflops_warm": round(fl / w / 1e6, 1),
            "tflops_cold": round(fl / c / 1e6, 1), "frac_bf16_peak_warm": round(fl / w / 1e6 / BF16_PEAK_TFLOPS, 4),
            "workspace_bytes": ks * 5120 * 2048 * 4 if ks > 1 else 0})
        log(f"down k{ks}", rows[f"mlp_down_5120x2048x11008_k{ks}"])
    # the oracle's split-K definition: FP64 planes, then the ascending FP32 reduce
    rows["mlp_down_5120x2048x11008_k8"].update(oracle_timing(
        lambda r0, r1: oracle.splitk_reduce(oracle.gemm_splitk_planes_ref(h[r0:r1], wd, 8).astype(np.float32)),
        5120, 16, oracle_seconds))
    del D, WS
    streamk_row("mlp_down_5120x2048x11008_streamk", 5120, 2048, 11008, h, wd)
    del H, WD

    out, x, bl, scale = synthetic.lora_fold()
    O, X, BL = up16(out), up16(x), up16(bl)
    w, c = timed(lambda: bg.gemm_bf16_scaled_acc(X, BL, O, scale))
    byts = 2 * 2048 * 17408 * 2 + (2048 + 17408) * 64 * 2
    rows["lora_fold_2048x17408x64"] = with_spread({
        "us_warm": round(w, 2), "us_cold": round(c, 2),
        "gbs_warm": round(byts / w / 1e3, 1), "gbs_cold": round(byts / c / 1e3, 1),
        "frac_hbm_warm": round(byts / w / 1e3 / HBM_PEAK_GBS, 4), "frac_hbm_cold": round(byts / c / 1e3 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes": byts})
    # the oracle's fold: FP64 delta, BF16 rounding, then the FP32 epilogue
    rows["lora_fold_2048x17408x64"].update(oracle_timing(
        lambda r0, r1: oracle.scaled_acc_epilogue(
            out[r0:r1], oracle.f32_to_bf16(oracle.gemm_bf16_ref(x[r0:r1], bl).astype(np.float32)), scale),
        2048, 16, oracle_seconds))
    log("lora", rows["lora_fold_2048x17408x64"])
    del O, X, BL

    for m in (4510, 2255):
        x, wr = synthetic.router(m=m)
        X, W = up16(x), up16(wr)
        C = torch.empty((m, 256), dtype=torch.bfloat16, device=dev)
        w, c = timed(lambda: bg.gemm_bf16_ordered(X, W, out=C))
        fl = 2.0 * m * 256 * 2048
        rows[f"router_ordered_{m}x256x2048"] = with_spread({
            "us_warm": round(w, 2), "us_cold": round(c, 2), "tflops_warm": round(fl / w / 1e6, 2),
            "frac_valu_nofma_peak": round(fl / w / 1e6 / VALU_NOFMA_PEAK_TFLOPS, 4)})
        # the strict FP32 recurrence of the oracle
        rows[f"router_ordered_{m}x256x2048"].update(oracle_timing(
            lambda r0, r1: oracle.gemm_ordered(x[r0:r1], wr), m, 16, oracle_seconds))
        log(f"router {m}", rows[f"router_ordered_{m}x256x2048"])

    a4, sfa, b4, sfb = synthetic.fp4_gemm()
    A4, SA, B4, SB = u8(a4), u8(sfa), u8(b4), u8(sfb)
    C = torch.empty((4096, 4096), dtype=torch.bfloat16, device=dev)
    w, c = timed(lambda: bg.gemm_fp4_blockscaled(A4, SA, B4, SB, out=C))
    fl = 2.0 * 4096 * 4096 * 8192
    rows["fp4_4096x4096x8192"] = with_spread({
        "us_warm": round(w, 2), "us_cold": round(c, 2), "tflops_warm": round(fl / w / 1e6, 1),
        "tflops_cold": round(fl / c / 1e6, 1),
        "frac_bf16_peak_warm": round(fl / w / 1e6 / BF16_PEAK_TFLOPS, 4),
        "frac_fp4_peak_warm": round(fl / w / 1e6 / FP4_PEAK_TFLOPS, 4)})
    rows["fp4_4096x4096x8192"].update(oracle_timing(
        lambda r0, r1: oracle.gemm_fp4_ref(a4[r0:r1], sfa[r0:r1], b4, sfb), 4096, 16, oracle_seconds))
    log("fp4", rows["fp4_4096x4096x8192"])
    del A4, SA, B4, SB, C

    # the kernelbot page's decode shapes (M = 128) through FP4 split-K, best
    # k_splits of 4/6/7/8/12/16. Bounds: the 16-bit MFMA rate (exact dequantization)
    # and HBM for the algorithmic bytes (A, B, scales read once, C written once).
    for m, n, k in ((128, 7168, 16384), (128, 4096, 7168)):
        ad, sad, bd, sbd = synthetic.fp4_decode(m=m, n=n, k=k)
        AD, SAD, BD, SBD = u8(ad), u8(sad), u8(bd), u8(sbd)
        C = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        WS = torch.empty((16, m, n), dtype=torch.float32, device=dev)
        best = None
        for ks in (4, 6, 7, 8, 12, 16):
            w, c = timed(lambda: bg.gemm_fp4_blockscaled_splitk(AD, SAD, BD, SBD, ks, workspace=WS[:ks], out=C))
            if best is None or w < best[1]:
                best = (ks, w, c, dict(spread))
        ks, w, c, sp = best
        fl = 2.0 * m * n * k
        byts = m * k // 2 + n * k // 2 + (m + n) * k // 16 + m * n * 2
        key = f"fp4_decode_{m}x{n}x{k}"
        rows[key] = {"us_warm": round(w, 2), "us_cold": round(c, 2), "k_splits": ks,
                     "us_warm_p20_p80": sp["warm"], "us_cold_p20_p80": sp["cold"],
                     "tflops_warm": round(fl / w / 1e6, 1), "frac_bf16_peak_warm": round(fl / w / 1e6 / BF16_PEAK_TFLOPS, 4),
                     "gbs_cold": round(byts / c / 1e3, 1), "frac_hbm_cold": round(byts / c / 1e3 / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": byts,
                     "bound_us": {"mfma_16bit": round(fl / BF16_PEAK_TFLOPS / 1e6, 2),
                                  "hbm": round(byts / HBM_PEAK_GBS / 1e3, 2)}}
        rows[key].update(oracle_timing(lambda r0, r1: oracle.gemm_fp4_ref(ad, sad, bd[r0:r1], sbd[r0:r1]),
                                       n, 64, oracle_seconds))
        rows[key]["oracle_sample"] += " (output columns)"
        log("fp4 decode", rows[key])
        del AD, SAD, BD, SBD, C, WS

    aw, bw, sw, s2 = synthetic.w4a16_gemm()
    AW, BW, SW = up16(aw), u8(bw), u8(sw)
    C = torch.empty((1016, 12288), dtype=torch.bfloat16, device=dev)
    w, c = timed(lambda: bg.gemm_w4a16(AW, BW, SW, s2, out=C))
    fl = 2.0 * 1016 * 12288 * 2048
    rows["w4a16_1016x12288x2048"] = with_spread({
        "us_warm": round(w, 2), "us_cold": round(c, 2), "tflops_warm": round(fl / w / 1e6, 1),
        "tflops_cold": round(fl / c / 1e6, 1), "frac_bf16_peak_warm": round(fl / w / 1e6 / BF16_PEAK_TFLOPS, 4)})
    rows["w4a16_1016x12288x2048"].update(oracle_timing(
        lambda r0, r1: oracle.gemm_w4a16_ref(aw[r0:r1], bw, sw, s2), 1016, 16, oracle_seconds))
    log("w4a16", rows["w4a16_1016x12288x2048"])
    del flush
    return rows


def cpu_baseline(gemms, seconds):
    """The plain C++ oracle's FP64 GEMM (oracle/cpu_oracle.cpp: decode, then
    one ascending-k FP64 dot product per output, rows split over host
    threads) on a bounded sample: for each of the step's three GEMMs, a run of
    consecutive output rows sized to take about seconds/3 of wall time. The
    numpy oracle (decode + BLAS FP64 matmul) is timed the same way for context."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from oracle import cpp

    threads = min(16, cpp.hardware_threads())   # the host share of one GPU

    def rate(fn, a, w, budget):
        """Calls fn on the leading r rows (r grows toward the budget, capped at
        all rows, so a fast oracle repeats whole passes) until `budget` seconds
        of wall time; returns flops, seconds and a description of the sample."""
        rows, t, flops, done, calls, top = 8, 0.0, 0.0, 0, 0, 0
        while t < budget:
            r = min(rows, a.shape[0])
            t0 = time.time()
            fn(a, w, r)
            dt = time.time() - t0
            t += dt
            flops += 2.0 * r * w.shape[0] * a.shape[1]
            done, calls, top = done + r, calls + 1, max(top, r)
            rows = max(8, int(r * max(1.0, (budget - t) / max(dt, 1e-3)) * 0.9))
        return flops, t, f"{done} output rows in {calls} calls on its first {top} of {a.shape[0]} rows"

    per = seconds / len(gemms)
    tot_f, tot_t, parts = 0.0, 0.0, []
    for name, a, w in gemms:
        f, t, n = rate(lambda a_, w_, r: cpp.gemm_bf16_ref_rows(a_, w_, np.arange(r), threads), a, w, per)
        tot_f, tot_t = tot_f + f, tot_t + t
        parts.append(f"{name}: {n}")
    # the same definition on one host thread (gate rows only)
    f1, t1, n1 = rate(lambda a_, w_, r: cpp.gemm_bf16_ref_rows(a_, w_, np.arange(r), 1), gemms[0][1], gemms[0][2],
                      min(per, 3.0))
    res = {"value": round(tot_f / tot_t / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
           "sample": f"C++ oracle orc_gemm_bf16_f64_rows (FP64, ascending k, {threads} threads) on the "
                     f"leading rows of the MLP step's GEMMs ({', '.join(parts)}; {tot_f / 1e9:.1f} GFLOP in {tot_t:.1f} s wall)"}

    res["one_thread"] = {"value": round(f1 / t1 / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                         "sample": f"{gemms[0][0]}: {n1}, {f1 / 1e9:.1f} GFLOP in {t1:.1f} s wall"}
    blas = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    nf, nt, nparts = 0.0, 0.0, []
    for name, a, w in gemms:
        f, t, n = rate(lambda a_, w_, r: oracle.gemm_bf16_ref(a_[:r], w_), a, w, min(per, 3.0))
        nf, nt = nf + f, nt + t
        nparts.append(f"{name}: {n}")
    res["numpy_oracle"] = {"value": round(nf / nt / 1e12, 4), "unit": "TFLOP/s", "cores": int(blas),
                           "sample": f"gemm_bf16_ref (decode + FP64 BLAS matmul) ({', '.join(nparts)}; "
                                     f"{nf / 1e9:.0f} GFLOP in {nt:.1f} s wall)"}
    return res


if __name__ == "__main__":
    main()
