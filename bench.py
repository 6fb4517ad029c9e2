#!/usr/bin/env python3
"""Benchmark of the FP8 P-cast attention forward on one MI355X.

One step is one pass of the whole hot path over the workload's input, which
is already resident in HBM: the V pre-pass (pcast_prepare_v) and the attention
kernel (attn_fwd_pcast_prepared) with the underflow counters on.  The default
workload is B=4, H=32, N=8192, d=128, causal, sink bias 7 on keys 0..3,
S = 256, reverse order.

Printed (one JSON line): throughput in TFLOP/s (algorithmic flops,
FlashAttention convention 2*B*H*N^2*d for causal), the attention kernel's own
time from HIP events on the launch stream, its fraction of the FP8 dense MFMA
peak, the CPU oracle timed on a bounded sample of the same workload, and the
output MSE against fp64 attention on that sample for S=256 reverse and S=1
forward.  The "qk_fp8" object times the variant with FP8 logits
(pcast_prepare_qk8 + attn_fwd_pcast_qk8_prepared) on the same input, and its
MSE against the same fp64 attention of the unquantised Q and K.  The "decode"
object times attn_decode_pcast (split KV) on the decode workload (16 sequences of
16384 cached keys, one new token each, GQA 32/8) against the HBM roofline; its V
copy is prepared once, outside the timed calls, as a cache would be; its "qk_fp8"
object times attn_decode_pcast_qk8 on an FP8 K cache prepared the same way.  The
"backward" object times attn_bwd_pcast on the same workload (its row-dot pre-pass
included), with the forward's O and lse as inputs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 P-cast attn fwd TFLOP/s + % MFMA peak; output MSE vs fp64 at Δ=7"
PEAK_FP8 = 5000.0    # TFLOP/s, MI355X dense FP8 MFMA
PEAK_BF16 = 2500.0   # TFLOP/s, MI355X dense bf16 MFMA
KERNEL_SRC = os.path.join(ROOT, "softmax_numerics_amd", "csrc", "attn_fwd_pcast.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attn_fwd_throughput.json")
TRAFFIC_FILE_QK8 = os.path.join(ROOT, "profiles", "traffic_attn_fwd_qk8_throughput.json")


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload: str, path: str = TRAFFIC_FILE):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash() or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch")


def causal_row_flops(rows, N: int, d: int, causal: bool):
    import numpy as np
    i = np.asarray(rows) % N
    keys = (i + 1) if causal else np.full(i.shape, N)
    return float(np.sum(4.0 * d * keys))


def cpu_baseline(w, qb, kb, vb, bias, out_rev, out_fwd1, target_s: float, seed: int = 0, out_qk8=None):
    """Time the oracle (kernel-mode block pipeline + exact attention, fp64, all
    host threads) on random 64-row blocks of the same workload, and use its
    exact result for the output-MSE comparison of the two GPU runs."""
    import numpy as np
    from oracle import core

    nthreads = os.cpu_count() or 1
    rng = np.random.default_rng(seed)
    nb = w.N // 64
    all_blocks = [(b, h, r) for b in range(w.B) for h in range(w.Hq) for r in range(nb)]

    def rows_of(blocks):
        return np.concatenate([np.arange(((b * w.Hq + h) * w.N + r * 64),
                                         ((b * w.Hq + h) * w.N + r * 64) + 64) for b, h, r in blocks])

    # grow a random block sample until one oracle call takes about target_s seconds
    order_ = rng.permutation(len(all_blocks))
    n = 8
    while True:
        blocks = [all_blocks[i] for i in sorted(order_[:n])]
        ids = rows_of(blocks)
        t0 = time.perf_counter()
        ref = core.rows(qb, kb, vb, bias, w.causal, 256.0, 1, "kernel", row_ids=ids, nthreads=nthreads)
        dt = time.perf_counter() - t0
        if dt >= 0.5 * target_s or n >= len(all_blocks):
            break
        n = min(len(all_blocks), int(n * min(16.0, max(2.0, target_s / max(dt, 1e-3)))))
    flops = causal_row_flops(ids, w.N, w.d, w.causal)
    o1 = ref["o1"]
    mse = {}
    runs = [("S256_reverse", out_rev), ("S1_forward", out_fwd1)]
    if out_qk8 is not None:
        runs.append(("qk_fp8_S256_reverse", out_qk8))
    for name, out in runs:
        got = out.reshape(-1, w.d)[ids].astype(np.float64)
        mse[name] = float(np.mean((got - o1) ** 2))
    mse["oracle_S256_reverse"] = float(np.mean((ref["o2"] - o1) ** 2))
    mse["ratio_S1fwd_over_S256rev"] = mse["S1_forward"] / mse["S256_reverse"]
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{n} random 64-row query blocks of {len(all_blocks)} ({ids.size} rows, "
                      f"{flops / w.flops * 100:.2f}% of the flops), kernel-mode P-cast emulation plus "
                      f"exact attention in fp64, {dt:.1f} s"}
    return base, mse


def bench_backward(sna, torch, np, synthetic, w, q, k, v, ws, bias_t, dev, stream, steps, warmup):
    sh = stream.cuda_stream
    S, order = 256.0, 1
    B, Hq, Hkv, N, d = w.B, w.Hq, w.Hkv, w.N, w.d
    o = torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    rc = sna.prepare_v(v.data_ptr(), B, Hkv, N, d, S, ws.data_ptr(), sh)
    rc = rc or sna.attn_fwd_pcast_rows(q.data_ptr(), k.data_ptr(), ws.data_ptr(), bias_t.data_ptr(), B, Hq, Hkv, N,
                                       d, int(w.causal), S, order, o.data_ptr(), 0, lse.data_ptr(), 0, sh)
    if rc != sna.PCAST_OK:
        raise sna.PcastError(rc, sna.strerror(rc))
    dob = synthetic.gaussian_bf16(w.seed, 3, (B, Hq, N, d))
    do = torch.from_numpy(dob.view(np.int16)).view(torch.bfloat16).to(dev)
    dq = torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev)
    dk = torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    wb = torch.empty(sna.bwd_workspace_bytes(B, Hq, Hkv, N, d), dtype=torch.uint8, device=dev)

    def call():
        r = sna.attn_bwd_pcast(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                               bias_t.data_ptr(), B, Hq, Hkv, N, d, int(w.causal), dq.data_ptr(), dk.data_ptr(),
                               dv.data_ptr(), wb.data_ptr(), sh)
        if r != sna.PCAST_OK:
            raise sna.PcastError(r, sna.strerror(r))

    def fwd_lse():
        r = sna.attn_fwd_pcast_rows(q.data_ptr(), k.data_ptr(), ws.data_ptr(), bias_t.data_ptr(), B, Hq, Hkv, N,
                                    d, int(w.causal), S, order, o.data_ptr(), 0, lse.data_ptr(), 0, sh)
        if r != sna.PCAST_OK:
            raise sna.PcastError(r, sna.strerror(r))

    def timed(fn):
        for _ in range(warmup):
            fn()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        for e in ev:
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))

    # the forward a training step runs before the backward: out and lse (no counters),
    # the attention kernel alone (the V copy is made once above)
    ms_fwd = timed(fwd_lse)
    ms = timed(call)
    flops = 2.5 * w.flops   # five products of the forward's two (FlashAttention convention)
    tf = flops / (ms * 1e-3) / 1e12
    print(f"[bench] backward: {ms:.4f} ms per call ({tf:.0f} TFLOP/s); forward with lse {ms_fwd:.4f} ms",
          file=sys.stderr, flush=True)
    return {"workload": f"{w.name}: B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal, sink bias 7 on keys 0..3, "
                        f"gradients of the S={S:g} {'reverse' if order else 'forward'} forward",
            "ms_per_call": round(ms, 5), "steps": steps,
            "kernels": "pcast_bwd_rowdot + pcast_attn_bwd_dq + pcast_attn_bwd_dkv",
            "forward_with_lse_ms": round(ms_fwd, 5),
            "forward_with_lse": "attn_fwd_pcast_rows with lost NULL (the pipelined forward, lse in its epilogue)",
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16, 4), "algorithmic_flops": flops,
                         "flops_rule": "2.5 x the forward's 2*B*H*N^2*d (causal)"}}


def bench_sweep_all(sna, torch, np, synthetic, w, q, k, v, dev, reps: int = 3):
    """The whole Sweep workload: every (delta, S, order) cell on the same Q, K, V through
    one attn_fwd_pcast_multi call (one launch per conversion mode and per 112 cells, the
    row blocks of all cells in one grid), each cell with its own out and counters.
    Returns the aggregate rate: all cells' flops over the call's time."""
    cells = [c for c in w.cases if c[1] > 0]
    ws = torch.empty(sna.workspace_bytes(w.B, w.Hkv, w.N, w.d, 256.0), dtype=torch.uint8, device=dev)
    main = torch.cuda.current_stream(dev)
    rc = sna.prepare_v(v.data_ptr(), w.B, w.Hkv, w.N, w.d, 256.0, ws.data_ptr(), main.cuda_stream)
    if rc != sna.PCAST_OK:
        raise sna.PcastError(rc, sna.strerror(rc))
    biases = {dl: torch.from_numpy(synthetic.sink_bias(w.N, dl)).to(dev) for dl in sorted({c[0] for c in cells})}
    outs = [torch.empty((w.B, w.Hq, w.N, w.d), dtype=torch.float32, device=dev) for _ in cells]
    sts = [torch.empty(sna.stats_words(w.B, w.Hq, w.N), dtype=torch.int64, device=dev) for _ in cells]
    args = dict(biases=[biases[c[0]].data_ptr() for c in cells], Ss=[c[1] for c in cells],
                orders=[c[2] for c in cells], outs=[o.data_ptr() for o in outs], stats=[x.data_ptr() for x in sts])
    torch.cuda.synchronize()

    def run():
        start, done = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(main)
        rc_ = sna.attn_fwd_pcast_multi(q.data_ptr(), k.data_ptr(), ws.data_ptr(), w.B, w.Hq, w.Hkv, w.N, w.d,
                                       int(w.causal), stream=main.cuda_stream, **args)
        if rc_ != sna.PCAST_OK:
            raise sna.PcastError(rc_, sna.strerror(rc_))
        done.record(main)
        done.synchronize()
        return start.elapsed_time(done)

    run()
    ms = sorted(run() for _ in range(reps))[reps // 2]
    flops = len(cells) * w.flops
    achieved = flops / (ms * 1e-3) / 1e12
    print(f"[bench] whole sweep: {len(cells)} cells in one multi-configuration call, {ms:.3f} ms "
          f"({achieved:.0f} TFLOP/s)", file=sys.stderr, flush=True)
    return {"cells": len(cells), "ms": round(ms, 4), "achieved": round(achieved, 2),
            "peak": PEAK_FP8, "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8, 4),
            "per_cell_us": round(ms * 1e3 / len(cells), 2),
            "what": "every cell of the Sweep (delta 0..10, S = 2^0..2^9 and 448, both orders) on the same Q, K, V "
                    "(one V pre-pass for all, outside the timed call), counters on, one attn_fwd_pcast_multi "
                    "call: one launch per conversion mode and per 112 cells"}


def bench_decode(sna, torch, np, synthetic, dev, stream, steps, warmup):
    w = synthetic.DECODE_WORKLOADS["decode"]
    delta, S, order = w.cases[0]
    qb, kb, vb = synthetic.decode_qkv_bf16(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.seed)
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    q, k, v = to(qb), to(kb), to(vb)
    bias = torch.from_numpy(synthetic.sink_bias(w.Nk, delta)).to(dev)
    sh = stream.cuda_stream
    vop = torch.empty(sna.workspace_bytes(w.B, w.Hkv, w.Nk, w.d, S), dtype=torch.uint8, device=dev)
    ws = torch.empty(sna.decode_workspace_bytes(w.B, w.Hkv, w.Nk, w.d, w.split_keys), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((w.B, w.Hq, w.Nq, w.d), dtype=torch.float32, device=dev)
    st = torch.empty(sna.stats_words(w.B, w.Hq, w.Nq), dtype=torch.int64, device=dev)
    rc = sna.prepare_v(v.data_ptr(), w.B, w.Hkv, w.Nk, w.d, S, vop.data_ptr(), sh)

    def call():
        r = sna.attn_decode_pcast(q.data_ptr(), k.data_ptr(), vop.data_ptr(), bias.data_ptr(), w.B, w.Hq, w.Hkv,
                                  w.Nq, w.Nk, w.d, S, order, w.split_keys, out.data_ptr(), st.data_ptr(),
                                  ws.data_ptr(), sh)
        if r != sna.PCAST_OK:
            raise sna.PcastError(r, sna.strerror(r))

    if rc != sna.PCAST_OK:
        raise sna.PcastError(rc, sna.strerror(rc))
    for _ in range(warmup):
        call()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record(stream)
        call()
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    gbs = w.bytes / (ms * 1e-3) / 1e9
    print(f"[bench] decode {w.name}: {ms:.4f} ms per call ({gbs:.0f} GB/s)", file=sys.stderr, flush=True)

    # the same decode with FP8 logits (K as E4M3 codes from pcast_prepare_qk8)
    ws8 = torch.empty(sna.workspace_bytes_qk8(w.B, w.Hkv, w.Nk, w.d), dtype=torch.uint8, device=dev)
    rc = sna.prepare_qk8(k.data_ptr(), v.data_ptr(), w.B, w.Hkv, w.Nk, w.d, ws8.data_ptr(), sh)
    if rc != sna.PCAST_OK:
        raise sna.PcastError(rc, sna.strerror(rc))

    def call8():
        r = sna.attn_decode_pcast_qk8(q.data_ptr(), ws8.data_ptr(), bias.data_ptr(), w.B, w.Hq, w.Hkv, w.Nq, w.Nk,
                                      w.d, S, order, w.split_keys, out.data_ptr(), st.data_ptr(), ws.data_ptr(), sh)
        if r != sna.PCAST_OK:
            raise sna.PcastError(r, sna.strerror(r))

    for _ in range(warmup):
        call8()
    torch.cuda.synchronize()
    for e in ev:
        e[0].record(stream)
        call8()
        e[1].record(stream)
    torch.cuda.synchronize()
    ms8 = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    gbs8 = w.bytes_qk8 / (ms8 * 1e-3) / 1e9
    print(f"[bench] decode {w.name}, FP8 logits: {ms8:.4f} ms per call ({gbs8:.0f} GB/s)", file=sys.stderr,
          flush=True)
    return {"workload": f"{w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} d={w.d}, "
                        f"split_keys={w.split_keys}, sink bias {delta} on keys 0..3, S={S:g}, "
                        f"{'reverse' if order else 'forward'} order, counters on",
            "ms_per_call": round(ms, 5), "kernels": "pcast_decode_split + pcast_decode_merge",
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                         "frac": round(gbs / 8000.0, 4), "algorithmic_bytes": w.bytes},
            "tflops": round(w.flops / (ms * 1e-3) / 1e12, 2),
            "qk_fp8": {"ms_per_call": round(ms8, 5), "kernels": "attn_decode_pcast_qk8 (K pre-pass not timed)",
                       "roofline": {"bound": "hbm", "achieved": round(gbs8, 1), "peak": 8000.0, "unit": "GB/s",
                                    "frac": round(gbs8 / 8000.0, 4), "algorithmic_bytes": w.bytes_qk8}}}


def smi_sample() -> dict:
    """One reading of socket power (W) and shader clock (MHz) from rocm-smi, with the raw
    power lines kept when no number can be read from them."""
    import re
    import subprocess
    try:
        txt = subprocess.run(["rocm-smi", "-a"], capture_output=True, text=True, timeout=30).stdout
    except (OSError, subprocess.SubprocessError) as e:
        return {"error": str(e)[:200]}
    out = {}
    for line in txt.splitlines():
        low = line.lower()
        if "power" in low and "(w)" in low and "max" not in low and "power_w" not in out:
            m = re.search(r"\(w\)\s*:\s*([0-9]+(?:\.[0-9]+)?)", low)
            if m:
                out["power_w"] = float(m.group(1))
            else:
                out.setdefault("raw", []).append(line.strip()[:160])
        if "sclk clock level" in low and "sclk_mhz" not in out:
            m = re.search(r"\((\d+)mhz\)", low)
            if m:
                out["sclk_mhz"] = float(m.group(1))
    return out


def run_sustained(launch, seconds: float, stream):
    """Call launch() back to back for about `seconds` (synchronising every 5 calls) while
    rocm-smi is sampled once a second after a short warm-up; returns (calls, ms, samples)."""
    import threading

    import torch

    samples, stop = [], threading.Event()

    def sampler():
        time.sleep(min(2.0, seconds / 3))
        while not stop.is_set():
            samples.append(smi_sample())
            stop.wait(1.0)
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n, t0 = 0, time.time()
    e0.record(stream)
    while time.time() - t0 < seconds:
        for _ in range(5):
            launch()
        n += 5
        torch.cuda.synchronize()
    e1.record(stream)
    e1.synchronize()
    stop.set()
    th.join()
    return n, e0.elapsed_time(e1), samples


def smi_summary(samples) -> dict:
    pw = sorted(x["power_w"] for x in samples if "power_w" in x)
    ck = sorted(x["sclk_mhz"] for x in samples if "sclk_mhz" in x)
    out = {"power_w_median": pw[len(pw) // 2] if pw else None, "sclk_mhz_median": ck[len(ck) // 2] if ck else None,
           "samples": len(samples)}
    if not pw and samples:
        out["smi"] = samples[0]
    return out


def bench_roof(seconds: float) -> dict:
    """Sustained matrix-core rates of the rate probe (libpcast_roof.so): bf16 32x32x16 only,
    FP8 32x32x64 only, the attention forward's mix (16 bf16 : 4 FP8 instructions per
    64-key block), the forward's softmax VALU work per block alone, and both interleaved
    as in the forward's steady step; each run back to back for `seconds` on every compute
    unit while rocm-smi samples socket power and shader clock."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "softmax_numerics_amd", "libpcast_roof.so"))
    lib.pcast_roof_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.pcast_roof_run.restype = ctypes.c_int
    lib.pcast_roof_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.pcast_roof_flops.restype = ctypes.c_double
    dev = torch.device("cuda:0")
    blocks = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    res = {"blocks": blocks, "threads": 256}
    waves_per_simd = blocks * 4 / (4 * torch.cuda.get_device_properties(dev).multi_processor_count)
    for mode, name, peak in ((0, "bf16_32x32x16", PEAK_BF16), (1, "fp8_32x32x64", PEAK_FP8),
                             (2, "forward_mix_16bf16_4fp8", None), (3, "forward_valu_per_block", None),
                             (4, "forward_mix_with_valu", None)):
        def launch(iters):
            rc = lib.pcast_roof_run(mode, iters, blocks, ctypes.c_void_p(sink.data_ptr()),
                                    ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"rate probe launch failed ({rc})")
        iters = 200
        launch(iters)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream); launch(iters); e1.record(stream); e1.synchronize()
        iters = max(1, int(iters * 20.0 / max(e0.elapsed_time(e1), 1e-3)))   # ~20 ms per launch
        n, ms, samples = run_sustained(lambda: launch(iters), seconds, stream)
        tflops = lib.pcast_roof_flops(mode, iters, blocks) * n / (ms * 1e-3) / 1e12
        entry = {"tflops": round(tflops, 1), "launches": n, "iters": iters, "seconds": round(ms * 1e-3, 2),
                 **smi_summary(samples)}
        # one iteration of every wave is one 64-key block of 32 query rows (modes 2-4); a
        # SIMD runs waves_per_simd of them side by side
        entry["ns_per_iteration_per_simd"] = round(ms * 1e6 / (n * iters * waves_per_simd), 2)
        if peak:
            entry["frac_of_peak"] = round(tflops / peak, 4)
        res[name] = entry
        print(f"[bench] rate probe {name}: {tflops:.0f} TFLOP/s, {entry['ns_per_iteration_per_simd']} ns per "
              f"iteration and SIMD, power {entry['power_w_median']} W, sclk {entry['sclk_mhz_median']} MHz",
              file=sys.stderr, flush=True)
    bf, f8 = res["bf16_32x32x16"]["tflops"], res["fp8_32x32x64"]["tflops"]
    # equal flops on each type, at the measured sustained rates
    res["mixed_roof_from_rates"] = round(1.0 / (0.5 / bf + 0.5 / f8), 1)
    t2, t3, t4 = (res[k]["ns_per_iteration_per_simd"] for k in
                  ("forward_mix_16bf16_4fp8", "forward_valu_per_block", "forward_mix_with_valu"))
    # 1 when the softmax's VALU work hides completely under the matrix cores, 0 when the
    # two only add up
    res["valu_overlap"] = round((t2 + t3 - t4) / min(t2, t3), 3)
    return res


ISSUE_KINDS = {1: "v_mfma_f32_32x32x16_bf16", 2: "softmax_work_per_block", 3: "v_exp_f32", 4: "v_fma_f32",
               5: "v_cvt_scalef32_pk_fp8_f32", 6: "v_cvt_pk_fp8_f32", 7: "v_max3_f32", 8: "v_add_f32",
               9: "v_or_b32+v_msad_u8", 10: "v_mul_f32"}


def bench_issue() -> dict:
    """Issue costs on one SIMD from the rate probe's second kernel (libpcast_roof.so): each
    instruction type of the forward's step alone with two waves per SIMD (ns per instruction
    and SIMD), the bf16 matrix-core stream and the softmax work per block alone with one
    wave per SIMD, and VALU waves beside a matrix-core wave on the same SIMD (how much of
    the matrix-core time the VALU wave loses)."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "softmax_numerics_amd", "libpcast_roof.so"))
    lib.pcast_issue_run.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p, ctypes.c_void_p]
    lib.pcast_issue_run.restype = ctypes.c_int
    lib.pcast_issue_count.argtypes = [ctypes.c_int]
    lib.pcast_issue_count.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count  # one 8-wave workgroup per CU
    sink = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def timed(klo, ilo, khi, ihi):
        def launch():
            rc = lib.pcast_issue_run(klo, ilo, khi, ihi, blocks, ctypes.c_void_p(sink.data_ptr()),
                                     ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"issue probe launch failed ({rc})")
        launch()
        best = float("inf")
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream); launch(); e1.record(stream); e1.synchronize()
            best = min(best, e0.elapsed_time(e1))
        return best

    it = 2000
    res = {"blocks": blocks, "threads": 512, "iterations": it, "two_waves_per_simd_ns_per_instruction": {}}
    for k in range(3, 11):
        ms = timed(k, it, k, it)
        res["two_waves_per_simd_ns_per_instruction"][ISSUE_KINDS[k]] = round(ms * 1e6 / (it * 2 * lib.pcast_issue_count(k)), 3)
    mf = timed(1, it, 0, 1)
    sm = timed(0, 1, 2, it)
    both = timed(1, it, 2, it)
    res["one_wave_ns_per_iteration"] = {"mfma_16_bf16": round(mf * 1e6 / it, 2),
                                        "softmax_work_per_block": round(sm * 1e6 / it, 2),
                                        "both_on_one_simd": round(both * 1e6 / it, 2)}
    res["overlap_mfma_wave_with_softmax_wave"] = round((mf + sm - both) / min(mf, sm), 3)
    # a VALU wave four times longer than the matrix-core wave beside it: the extra time
    # it takes, as a share of the matrix-core wave's time, is what the matrix cores cost it
    lost = {}
    for k in (3, 4, 5, 8, 2):
        alone1 = timed(0, 1, k, it)
        ih = max(1, int(it * 4.0 * mf / alone1))
        alone = timed(0, 1, k, ih)
        beside = timed(1, it, k, ih)
        lost[ISSUE_KINDS[k]] = round((beside - alone) / mf, 3)
    res["valu_wave_loses_share_of_mfma_time"] = lost
    print(f"[bench] issue probe: {json.dumps(res)}", file=sys.stderr, flush=True)
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="throughput", choices=["tiny", "sweep", "throughput", "gqa", "long"])
    ap.add_argument("--no-stats", action="store_true", help="time without the underflow counters")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time of the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-qk8", action="store_true", help="skip the FP8-logit variant")
    ap.add_argument("--no-decode", action="store_true", help="skip the split-KV decode measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurement")
    ap.add_argument("--sustain", type=float, default=0.0, metavar="SECONDS",
                    help="after the timed steps, run the attention kernel back to back for SECONDS with "
                         "power and clock samples")
    ap.add_argument("--roof", type=float, default=0.0, metavar="SECONDS",
                    help="only run the matrix-core rate probe (bf16, FP8 and the forward's mix), SECONDS "
                         "each, with power and clock samples")
    ap.add_argument("--issue", action="store_true",
                    help="only run the issue-cost probe (VALU instruction types of the forward's step, "
                         "matrix-core and VALU waves on one SIMD)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes, 3 times (scale for "
                         "the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.roof > 0:
        print(json.dumps({"roof": bench_roof(args.roof)}))
        return 0
    if args.issue:
        print(json.dumps({"issue": bench_issue()}))
        return 0
    if args.calibrate_copy:
        import torch
        x = torch.empty(args.calibrate_copy, dtype=torch.uint8, device="cuda:0").fill_(1)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.calibrate_copy}))
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the measured path runs on one GPU and needs no collective (sharding is by batch and kv head)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import softmax_numerics_amd as sna
    import synthetic

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    sna.load_library()
    w = synthetic.WORKLOADS[args.workload]
    delta, S, order = 7.0, 256.0, (0 if w.name == "tiny" else 1)   # tiny is non-causal, forward
    dev = torch.device("cuda:0")
    print(f"[bench] workload {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} causal={w.causal} "
          f"delta={delta} S={S} order={order}", file=sys.stderr, flush=True)
    qb, kb, vb = synthetic.qkv_bf16(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed)
    bias = synthetic.sink_bias(w.N, delta)
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    q, k, v = to(qb), to(kb), to(vb)
    bias_t = torch.from_numpy(bias).to(dev)
    out = torch.empty((w.B, w.Hq, w.N, w.d), dtype=torch.float32, device=dev)
    stats = None if args.no_stats else torch.empty(sna.stats_words(w.B, w.Hq, w.N), dtype=torch.int64, device=dev)
    ws = torch.empty(sna.workspace_bytes(w.B, w.Hkv, w.N, w.d, S), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def step(S_=S, order_=order, ev=None):
        if ev is not None:
            ev[0].record(stream)
        rc = sna.prepare_v(v.data_ptr(), w.B, w.Hkv, w.N, w.d, S_, ws.data_ptr(), sh)
        if ev is not None:
            ev[1].record(stream)
        rc = rc or sna.attn_fwd_pcast_prepared(
            q.data_ptr(), k.data_ptr(), ws.data_ptr(), bias_t.data_ptr(), w.B, w.Hq, w.Hkv, w.N, w.d,
            int(w.causal), S_, order_, out.data_ptr(), 0 if stats is None else stats.data_ptr(), sh)
        if ev is not None:
            ev[2].record(stream)
        if rc != sna.PCAST_OK:
            raise sna.PcastError(rc, sna.strerror(rc))

    ws8 = None if args.no_qk8 else torch.empty(sna.workspace_bytes_qk8(w.B, w.Hkv, w.N, w.d),
                                               dtype=torch.uint8, device=dev)

    def step_qk8(ev=None):
        if ev is not None:
            ev[0].record(stream)
        rc = sna.prepare_qk8(k.data_ptr(), v.data_ptr(), w.B, w.Hkv, w.N, w.d, ws8.data_ptr(), sh)
        if ev is not None:
            ev[1].record(stream)
        rc = rc or sna.attn_fwd_pcast_qk8_prepared(
            q.data_ptr(), ws8.data_ptr(), bias_t.data_ptr(), w.B, w.Hq, w.Hkv, w.N, w.d, int(w.causal), S, order,
            out.data_ptr(), 0 if stats is None else stats.data_ptr(), sh)
        if ev is not None:
            ev[2].record(stream)
        if rc != sna.PCAST_OK:
            raise sna.PcastError(rc, sna.strerror(rc))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev=events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prep_ms = [e[0].elapsed_time(e[1]) for e in events]
    attn_ms = [e[1].elapsed_time(e[2]) for e in events]
    ms_per_step = wall * 1e3 / args.steps
    print(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step (wall), attention kernel "
          f"{np.mean(attn_ms):.4f} ms, V pre-pass {np.mean(prep_ms):.4f} ms", file=sys.stderr, flush=True)

    flops = w.flops
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (float(np.mean(attn_ms)) * 1e-3) / 1e12
    mixed_roof = 1.0 / (0.5 / PEAK_BF16 + 0.5 / PEAK_FP8)

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3(P.V)+bf16(QK^T), fp32 softmax", "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} "
                               f"{'causal' if w.causal else 'non-causal'}, sink bias {delta} on keys 0..3, "
                               f"S={S:g}, {'reverse' if order else 'forward'} order, "
                               f"underflow counters {'off' if stats is None else 'on'}",
                   "global_batch": w.B, "seq_len": w.N, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8, 4),
                     "traffic": measured_traffic(w.name)},
        "attention_kernel_ms": round(float(np.mean(attn_ms)), 5),
        "v_prepass_ms": round(float(np.mean(prep_ms)), 5),
        "frac_bf16_peak": round(achieved / PEAK_BF16, 4),
        "frac_mixed_roof": round(achieved / mixed_roof, 4),
    }

    if args.sustain > 0:
        launch = lambda: sna.attn_fwd_pcast_prepared(  # noqa: E731
            q.data_ptr(), k.data_ptr(), ws.data_ptr(), bias_t.data_ptr(), w.B, w.Hq, w.Hkv, w.N, w.d,
            int(w.causal), S, order, out.data_ptr(), 0 if stats is None else stats.data_ptr(), sh)
        n, ms, samples = run_sustained(launch, args.sustain, stream)
        result["sustained"] = {"calls": n, "ms_per_call": round(ms / n, 5),
                               "tflops": round(flops * n / (ms * 1e-3) / 1e12, 1), **smi_summary(samples)}
        print(f"[bench] sustained: {result['sustained']}", file=sys.stderr, flush=True)

    out_rev = out.cpu().numpy() if not args.no_cpu_baseline else None
    st_rev = None if stats is None else stats.cpu().numpy().reshape(-1, 2)
    out_qk8 = None
    if ws8 is not None:
        # the FP8-logit variant on the same input, same configuration
        for _ in range(args.warmup):
            step_qk8()
        ev8 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step_qk8(ev=ev8[i])
        torch.cuda.synchronize()
        wall8 = time.perf_counter() - t0
        prep8 = float(np.mean([e[0].elapsed_time(e[1]) for e in ev8]))
        attn8 = float(np.mean([e[1].elapsed_time(e[2]) for e in ev8]))
        ach8 = flops / (attn8 * 1e-3) / 1e12
        print(f"[bench] FP8 logits: {wall8 * 1e3 / args.steps:.4f} ms/step (wall), attention kernel "
              f"{attn8:.4f} ms, K/V pre-pass {prep8:.4f} ms", file=sys.stderr, flush=True)
        # the same with Q and K rotated by diag(sigma) H before the rounding
        signs = torch.from_numpy(np.random.default_rng(w.seed).choice(np.array([-1, 1], dtype=np.int8), size=w.d)).to(dev)
        wsr = torch.empty(sna.workspace_bytes_qk8_rot(w.B, w.Hq, w.Hkv, w.N, w.d), dtype=torch.uint8, device=dev)

        def step_rot(ev=None):
            if ev is not None:
                ev[0].record(stream)
            rc = sna.prepare_qk8_rot(q.data_ptr(), k.data_ptr(), v.data_ptr(), signs.data_ptr(), w.B, w.Hq, w.Hkv,
                                     w.N, w.d, wsr.data_ptr(), sh)
            if ev is not None:
                ev[1].record(stream)
            rc = rc or sna.attn_fwd_pcast_qk8_rot_prepared(
                wsr.data_ptr(), bias_t.data_ptr(), w.B, w.Hq, w.Hkv, w.N, w.d, int(w.causal), S, order,
                out.data_ptr(), 0 if stats is None else stats.data_ptr(), sh)
            if ev is not None:
                ev[2].record(stream)
            if rc != sna.PCAST_OK:
                raise sna.PcastError(rc, sna.strerror(rc))

        for _ in range(2):
            step_rot()
        evr = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(min(args.steps, 10))]
        torch.cuda.synchronize()
        for e in evr:
            step_rot(ev=e)
        torch.cuda.synchronize()
        rot = {"prepass_ms": round(float(np.mean([e[0].elapsed_time(e[1]) for e in evr])), 5),
               "attention_kernel_ms": round(float(np.mean([e[1].elapsed_time(e[2]) for e in evr])), 5)}
        print(f"[bench] FP8 logits, rotated: attention kernel {rot['attention_kernel_ms']:.4f} ms, "
              f"pre-pass {rot['prepass_ms']:.4f} ms", file=sys.stderr, flush=True)
        del wsr
        result["qk_fp8"] = {"ms_per_step": round(wall8 * 1e3 / args.steps, 5),
                            "value": round(flops / wall8 * args.steps / 1e12, 2),
                            "attention_kernel_ms": round(attn8, 5), "prepass_ms": round(prep8, 5),
                            "achieved": round(ach8, 2), "peak": PEAK_FP8, "frac": round(ach8 / PEAK_FP8, 4),
                            "traffic": measured_traffic(w.name, TRAFFIC_FILE_QK8), "rotated": rot}
        step_qk8()                                   # the output of the unrotated variant
        torch.cuda.synchronize()
        out_qk8 = out.cpu().numpy()

    if w.name == "sweep":
        result["sweep_all"] = bench_sweep_all(sna, torch, np, synthetic, w, q, k, v, dev)
    if not args.no_backward:
        result["backward"] = bench_backward(sna, torch, np, synthetic, w, q, k, v, ws, bias_t, dev, stream,
                                            min(args.steps, 10), min(args.warmup, 2))
    if not args.no_decode:
        result["decode"] = bench_decode(sna, torch, np, synthetic, dev, stream, args.steps, args.warmup)

    if not args.no_cpu_baseline:
        # S = 1 forward, for the error contrast, with the per-row diagnostics (same out, bit for bit)
        lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
        lost = torch.empty_like(lse)
        st1 = torch.empty(sna.stats_words(w.B, w.Hq, w.N), dtype=torch.int64, device=dev)
        rc = sna.prepare_v(v.data_ptr(), w.B, w.Hkv, w.N, w.d, 1.0, ws.data_ptr(), sh)
        rc = rc or sna.attn_fwd_pcast_rows(q.data_ptr(), k.data_ptr(), ws.data_ptr(), bias_t.data_ptr(), w.B, w.Hq,
                                           w.Hkv, w.N, w.d, int(w.causal), 1.0, 0, out.data_ptr(), st1.data_ptr(),
                                           lse.data_ptr(), lost.data_ptr(), sh)
        if rc != sna.PCAST_OK:
            raise sna.PcastError(rc, sna.strerror(rc))
        torch.cuda.synchronize()
        out_fwd1 = out.cpu().numpy()
        s1 = st1.cpu().numpy().reshape(-1, 2)
        far = lost.cpu().numpy().reshape(w.B * w.Hq, w.N)[:, min(1024, w.N // 2):]
        result["collapse"] = {
            "delta": delta, "sink_keys": 4,
            "S1_forward": {"delta_critical": round(sna.delta_critical(1.0), 4),
                           "underflow_measured": float(s1[:, 1].sum() / s1[:, 0].sum()),
                           "underflow_model": round(sna.underflow_model(delta, 1.0), 4),
                           "lost_mass_measured": round(float(far.mean()), 4),
                           "lost_mass_model": round(sna.lost_mass_model(delta, 1.0), 4),
                           "lost_mass_rows": f"mean over all heads of rows {min(1024, w.N // 2)}..{w.N - 1}"},
            f"S{S:g}_{'reverse' if order else 'forward'}": {
                "delta_critical": round(sna.delta_critical(S), 4),
                "underflow_measured": None if st_rev is None else float(st_rev[:, 1].sum() / st_rev[:, 0].sum()),
                "underflow_model_forward": sna.underflow_model(delta, S)}}
        base, mse = cpu_baseline(w, qb, kb, vb, bias, out_rev, out_fwd1, args.cpu_seconds, out_qk8=out_qk8)
        result["cpu_baseline"] = base
        result["mse_vs_fp64_sampled"] = mse
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
