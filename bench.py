"""Benchmark of the FlashAttention backward pass on one MI355X.

Default workload: the long-context bf16 GQA causal backward (B=1, Hq=32,
Hkv=8, S=16384, D=128, scale 1/sqrt(128)), seeded synthetic inputs.  One
step = the whole backward path: Delta preprocess + dK/dV pass + dQ pass, all
inputs resident in HBM.  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long|extras|causal_f32|decode|copy]
                  [--path shared_ds|recompute] [--settle-ms MS] [--no-cpu-baseline] [--no-mfma-ceiling]
                  [--no-side-workloads]

O and L (inputs of the backward) are produced once, before timing, by the
library's own forward (fa_fwd, parity-tested against the oracle forward); they
are inputs only, never part of the timed path (the forward is timed
separately).  The cpu_baseline leg times the
CPU fp64 oracle on one GQA group of the same workload.

The default (long) run also times, in the same process and with the same
steps, the long workload on the other bf16 path (recompute vs shared dS) and
the two other prefill workloads (the bf16 GQA window + mask + dropout one and
the fp32 causal MHA one), each reported as a summary under its own key.  Their
steps are short (a few tenths of a millisecond), so before timing them the run
keeps the GPU busy for a while (the engine clock rises over some tens of
milliseconds of load after the idle input preparation), and their ms per step
comes from steps with no events between the kernels.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_F32_TFLOPS = 157.3     # fp32 matrix peak
PEAK_HBM_GBS = 8000.0       # HBM3E
# Untimed steps before a side workload's timed ones: its steps last well under a millisecond, and
# after the idle input preparation the engine clock takes some tens of milliseconds of load to rise.
SIDE_SETTLE_MS = 200.0


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long", choices=["long", "extras", "causal_f32", "decode", "copy"])
    ap.add_argument("--path", default="shared_ds", choices=["shared_ds", "recompute"],
                    help="bf16: the dQ pass reads the dS the dK/dV pass stored (shared_ds) or recomputes it")
    ap.add_argument("--settle-ms", type=float, default=0.0,
                    help="untimed steps after the warm-up ones until this much wall time has passed "
                         "(the side workloads always settle for %.0f ms)" % SIDE_SETTLE_MS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mfma-ceiling", action="store_true",
                    help="skip the calibration of the bf16 MFMA rate on N(0,1) operands (about 0.5 s)")
    ap.add_argument("--no-side-workloads", action="store_true",
                    help="long workload: skip the other bf16 path and the extras / fp32 causal summaries")
    return ap.parse_args()


def _mfma_ceiling():
    """TFLOP/s of back-to-back bf16 MFMAs on every SIMD with N(0,1) operand data.

    The published dense peak assumes the full engine clock; under a sustained
    MFMA load with random operand bits the chip holds a lower, power-limited
    clock.  This runs the library's calibration kernel (fa_bwd_calib_mfma_bf16:
    nothing but v_mfma_f32_32x32x16_bf16, operands rotating over registers as in
    the tile kernels) for a few hundred milliseconds and reports its rate, the
    ceiling the tile kernels can approach on this data.
    """
    import torch

    from flashattention_backward_pass_bwd_amd import api

    g = torch.Generator(device="cpu").manual_seed(1234)
    ops = torch.randn(2048 * 8, generator=g).to(torch.bfloat16).cuda()
    blocks = 4 * torch.cuda.get_device_properties(0).multi_processor_count  # four waves of one wave per SIMD
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    iters = 2000
    for _ in range(20):
        api.calib_mfma_bf16(ops, sink, blocks, iters)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 40
    e0.record()
    for _ in range(n):
        api.calib_mfma_bf16(ops, sink, blocks, iters)
    e1.record()
    torch.cuda.synchronize()
    flop = n * blocks * 4 * iters * 32 * 32768.0
    return flop / (e0.elapsed_time(e1) * 1e-3) / 1e12


def _visible_pairs(w) -> int:
    """Exact count of visible (i, j) pairs per (b, h), from the window/causal geometry."""
    import numpy as np

    i = np.arange(w.seq_q, dtype=np.int64)
    qa = i + w.causal_offset
    hi = np.minimum(w.seq_k, qa + 1) if w.causal else np.full_like(i, w.seq_k)
    lo = np.zeros_like(i)
    if w.window > 0:
        lo = np.maximum(0, qa - w.window + 1)
        if not w.causal:
            hi = np.minimum(w.seq_k, qa + w.window)
    return int(np.maximum(hi - lo, 0).sum())


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dkdv_bf16_long_traffic.txt")
TRAFFIC_SOURCES = ["fa_dkdv_bf16.hip", "fa_tiles.h", "fa_common.h", "fa_internal.h"]


def _dkdv_traffic_bytes():
    """HBM bytes per dK/dV launch from the committed FETCH_SIZE/WRITE_SIZE counters, scaled by the
    copy-kernel calibration; None when the kernel sources changed since the counters were taken."""
    import hashlib

    try:
        vals = dict(l.strip().split("=", 1) for l in open(TRAFFIC_FILE) if "=" in l and not l.startswith("#"))
        h = hashlib.sha256()
        for f in TRAFFIC_SOURCES:
            h.update(open(os.path.join(ROOT, "flashattention_backward_pass_bwd_amd", "csrc", f), "rb").read())
        if h.hexdigest()[:16] != vals["kernel_source_hash"]:
            return None
        return 1024.0 * (float(vals["fetch_kib"]) * float(vals["fetch_scale"]) +
                         float(vals["write_kib"]) * float(vals["write_scale"]))
    except (OSError, KeyError, ValueError):
        return None


def _cpu_baseline(w, q, k, v, o, do, lse):
    """Time the fp64 oracle backward on one GQA group (batch 0, KV head 0 and its query heads)."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    g = w.num_heads // w.num_kv_heads

    def heads(x, h0, n):  # [B,S,H,D] device -> logical [1,n,S,D] float64 host
        return x[0:1, :, h0:h0 + n, :].float().cpu().numpy().transpose(0, 2, 1, 3).astype(np.float64)

    qs, dos, os_ = heads(q, 0, g), heads(do, 0, g), heads(o, 0, g)
    ks, vs = heads(k, 0, 1), heads(v, 0, 1)
    ls = lse[0:1, 0:g, :].cpu().numpy().astype(np.float64)
    spec = oracle.Spec(scale=w.scale, causal=w.causal, causal_offset=w.causal_offset, window=w.window)
    t0 = time.perf_counter()
    oracle.backward(qs, ks, vs, os_, dos, ls, spec, None, chunk=2048)
    dt = time.perf_counter() - t0
    flops = 10.0 * g * w.seq_q * w.seq_k * w.head_dim * (0.5 if w.causal else 1.0)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"numpy fp64 oracle backward of one GQA group of the same workload (batch 0, KV head 0 "
                      f"and its {g} query heads, all {w.seq_q} rows; {g}/{w.batch * w.num_heads} of the job): "
                      f"{dt:.1f} s for {flops / 1e9:.1f} nominal GFLOP", "seconds": dt}


def _prepare(w):
    """Seeded inputs of workload w on the device, in its layout, and the O, L of its forward."""
    import torch

    from flashattention_backward_pass_bwd_amd import api, synth

    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    inp = synth.prefill_inputs(w)

    def up(x):  # logical [B,H,S,D] -> device view [B,S,H,D] in the workload layout
        t = torch.from_numpy(x)
        if w.layout == "bshd":
            return t.permute(0, 2, 1, 3).contiguous().to(tdt).to(dev)
        return t.contiguous().to(tdt).to(dev).transpose(1, 2)

    q, k, v, do = (up(inp[n]) for n in ("q", "k", "v", "do"))
    mask = torch.from_numpy(inp["mask"]).to(dev) if inp["mask"] is not None else None
    del inp
    p = api.make_params(q, k, scale=w.scale, causal=w.causal, causal_offset=w.causal_offset, window=w.window,
                        dropout_p=w.dropout_p, seed=w.dropout_seed, mask=mask)
    # O, L from the library's forward (parity-tested against the oracle forward)
    _log(f"inputs of {w.name} on device; forward for O, L")
    o, lse = api.forward(p, q, k, v)
    torch.cuda.synchronize()
    return {"q": q, "k": k, "v": v, "do": do, "mask": mask, "o": o, "lse": lse, "p": p, "dev": dev}


def _time_path(args, w, t, shared, settle_ms=0.0, split=False):
    """Event-timed steps (preprocess + dK/dV + dQ) of one path: (ms per step, per-kernel ms, workspace bytes).

    settle_ms: after the warm-up steps, further untimed steps until that much wall time has passed (a
    step of a fraction of a millisecond otherwise runs its timed steps while the engine clock is still
    rising after the idle input preparation).  split: ms per step from steps with no events between their
    kernels, the per-kernel times from a second batch of as many steps with events between them (each
    such event adds a few microseconds to a step)."""
    import torch

    from flashattention_backward_pass_bwd_amd import api

    dev, p = t["dev"], t["p"]
    q, k, v, do, o, lse = t["q"], t["k"], t["v"], t["do"], t["o"], t["lse"]
    delta = torch.empty((w.batch, w.num_heads, w.seq_q), dtype=torch.float32, device=dev)
    dq = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=dev)
    dk = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=dev)
    dv = torch.empty_strided(v.shape, v.stride(), dtype=v.dtype, device=dev)
    # shared dS: the dK/dV pass stores dS and the dQ pass reads it (the workspace
    # is allocated here, outside the timed steps); recompute: both passes recompute.
    ws = api.ds_workspace(p, dev) if shared else None
    ws_bytes = api.ds_workspace_bytes(p) if shared else 0

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        api.preprocess(p, o, do, delta)
        if ev is not None:
            ev[1].record()
        if shared:
            api.dkdv_ds(p, q, k, v, do, lse, delta, ws, dk, dv)
        else:
            api.dkdv(p, q, k, v, do, lse, delta, dk, dv)
        if ev is not None:
            ev[2].record()
        if shared:
            api.dq_ds(p, q, k, ws, dq)
        else:
            api.dq(p, q, k, v, do, lse, delta, dq)
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if settle_ms > 0:
        s0 = time.perf_counter()
        while (time.perf_counter() - s0) * 1e3 < settle_ms:
            for _ in range(8):
                step()
            torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for s_ in range(args.steps):
        step(None if split else evs[s_])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = start.elapsed_time(stop) / args.steps
    if split:
        for s_ in range(args.steps):
            step(evs[s_])
        torch.cuda.synchronize()
    kms = {"preprocess": sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps,
           "dkdv": sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps,
           "dq": sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps}
    del ws
    return ms, kms, ws_bytes, wall


def _work(w):
    """Nominal FLOP (the metric's count), visible pairs, peak and its dtype's name."""
    nominal = 10.0 * w.batch * w.num_heads * w.seq_q * w.seq_k * w.head_dim * (0.5 if w.causal else 1.0)
    pairs = _visible_pairs(w) * w.batch * w.num_heads
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    return nominal, pairs, peak


def _dkdv_roofline(w, t_dkdv, pairs, peak):
    # the dK/dV pass executes 4 of the contractions (QK^T, dO V^T, dV, dK): 8*D FLOP per visible pair
    achieved = 8.0 * w.head_dim * pairs / (t_dkdv * 1e-3) / 1e12
    return {"kernel": "dkdv_kernel", "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
            "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
            "per_unit": "8*D FLOP per visible (b,h,i,j) pair", "units": pairs}


def _dq_ds_roofline(w, t_dq, ws_bytes):
    # the dQ pass over stored dS streams the workspace once: HBM-bound
    dq_bytes = ws_bytes + (w.batch * w.num_kv_heads * w.seq_k * w.head_dim +
                           w.batch * w.num_heads * w.seq_q * w.head_dim) * 2
    gbs = dq_bytes / (t_dq * 1e-3) / 1e9
    return {"kernel": "dqs_kernel", "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "per_unit": "the stored dS (16 KB per visible 64x128 tile) + K read, dQ written",
            "algorithmic_bytes": dq_bytes}


def _summary(args, w):
    """Compact record of another prefill workload, timed the same way as the main line."""
    import torch

    t = _prepare(w)
    shared = w.dtype == "bf16"
    ms, kms, ws_bytes, _ = _time_path(args, w, t, shared, settle_ms=SIDE_SETTLE_MS, split=True)
    nominal, pairs, peak = _work(w)
    value = nominal / (ms * 1e-3) / 1e12
    out = {"workload": w.name, "dtype": w.dtype, "path": "shared_ds" if shared else "recompute",
           "ms_per_step": round(ms, 4), "value": round(value, 2), "unit": "TFLOP/s",
           "timing": f"{args.warmup} warm-up steps, then untimed steps for {SIDE_SETTLE_MS:.0f} ms (the clock "
                     f"settles), then {args.steps} timed steps with no events between the kernels; kernels_ms "
                     f"from {args.steps} further steps with events between them",
           "peak": peak, "pct_of_peak": round(100.0 * value / peak, 2),
           "nominal_gflop": round(nominal / 1e9, 3), "window_aware_gflop": round(10.0 * w.head_dim * pairs / 1e9, 3),
           "window_aware_pct_of_peak": round(100.0 * 10.0 * w.head_dim * pairs / (ms * 1e-3) / 1e12 / peak, 2),
           "kernels_ms": {k_: round(v_, 4) for k_, v_ in kms.items()},
           "roofline": _dkdv_roofline(w, kms["dkdv"], pairs, peak)}
    if shared:
        out["roofline_dq"] = _dq_ds_roofline(w, kms["dq"], ws_bytes)
    _log(f"{w.name}: {ms:.4f} ms/step ({out['pct_of_peak']}% of the {w.dtype} peak)")
    del t
    torch.cuda.synchronize()
    return out


def bench_prefill(args, w):
    import torch

    from flashattention_backward_pass_bwd_amd import api, synth

    t = _prepare(w)
    p, q, k, v, o, lse = t["p"], t["q"], t["k"], t["v"], t["o"], t["lse"]
    _log("O, L ready; timing")
    shared = w.dtype == "bf16" and args.path == "shared_ds"
    ms, kms, ws_bytes, wall = _time_path(args, w, t, shared, settle_ms=args.settle_ms)
    nominal, pairs, peak = _work(w)
    value = nominal / (ms * 1e-3) / 1e12
    roof = _dkdv_roofline(w, kms["dkdv"], pairs, peak)
    roof["traffic"] = _dkdv_traffic_bytes() if (w.name == synth.LONG_BF16.name and shared) else None
    roof["traffic_unit"] = "bytes per launch (HBM, FETCH_SIZE+WRITE_SIZE scaled by the copy calibration)"
    out = {
        "metric": "attention-backward TFLOP/s and % of MI355X bf16 MFMA peak, 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "pct_of_peak": round(100.0 * value / peak, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "wall_s_timed": round(wall, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs; O, L from the library's forward)",
        "config": {"workload": w.name, "batch": w.batch, "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads,
                   "seq_q": w.seq_q, "seq_k": w.seq_k, "head_dim": w.head_dim, "layout": w.layout,
                   "causal": w.causal, "window": w.window, "mask_density": w.mask_density,
                   "dropout_p": w.dropout_p, "nominal_gflop": round(nominal / 1e9, 3),
                   "path": "shared_ds" if shared else "recompute", "ds_workspace_bytes": ws_bytes,
                   "window_aware_gflop": round(10.0 * w.head_dim * pairs / 1e9, 3)},
        "kernels_ms": {k_: round(v_, 4) for k_, v_ in kms.items()},
        "roofline": roof,
    }
    if shared:
        out["roofline_dq"] = _dq_ds_roofline(w, kms["dq"], ws_bytes)
    _log(f"timed {args.steps} steps: {ms:.3f} ms/step")
    side = w.name == synth.LONG_BF16.name and not args.no_side_workloads
    if side and w.dtype == "bf16":
        # the same workload on the other bf16 path (no dS workspace on the recompute path)
        oms, okms, ows, _ = _time_path(args, w, t, not shared)
        out["other_path"] = {"path": "recompute" if shared else "shared_ds", "ms_per_step": round(oms, 4),
                             "value": round(nominal / (oms * 1e-3) / 1e12, 2),
                             "pct_of_peak": round(100.0 * nominal / (oms * 1e-3) / 1e12 / peak, 2),
                             "kernels_ms": {k_: round(v_, 4) for k_, v_ in okms.items()},
                             "ds_workspace_bytes": ows}
        _log(f"other path ({out['other_path']['path']}): {oms:.3f} ms/step")
    # the forward on the same inputs, timed on its own after the backward steps
    for _ in range(2):
        api.forward(p, q, k, v, o, lse)
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record()
    for _ in range(args.steps):
        api.forward(p, q, k, v, o, lse)
    f1.record()
    torch.cuda.synchronize()
    fms = f0.elapsed_time(f1) / args.steps
    ftf = 4.0 * w.head_dim * pairs / (fms * 1e-3) / 1e12
    out["forward"] = {"kernel": "fwd_kernel", "what": "O, L (fa_fwd)", "ms": round(fms, 4), "bound": "mfma",
                      "achieved": round(ftf, 2), "peak": peak, "unit": "TFLOP/s", "frac": round(ftf / peak, 4),
                      "per_unit": "4*D FLOP per visible (b,h,i,j) pair (QK^T and PV)", "units": pairs}
    _log(f"forward: {fms:.3f} ms")
    if w.dtype == "bf16" and not args.no_mfma_ceiling:
        ceiling = _mfma_ceiling()
        # a SIMD retires one v_mfma_f32_32x32x16_bf16 (32768 FLOP) per 32 engine clocks: the peak's
        # 1024 FLOP per clock per SIMD, so the MFMA-only rate gives the clock the chip holds under it
        simds = 4 * torch.cuda.get_device_properties(0).multi_processor_count
        out["roofline"]["mfma_ceiling"] = {
            "value": round(ceiling, 1), "unit": "TFLOP/s", "frac": round(roof["achieved"] / ceiling, 4),
            "engine_clock_ghz": round(ceiling * 1e12 / (simds * 1024.0) / 1e9, 3),
            "how": "back-to-back v_mfma_f32_32x32x16_bf16 on every SIMD, N(0,1) bf16 operands rotating "
                   "over registers (fa_bwd_calib_mfma_bf16), after the timed steps; engine_clock_ghz = "
                   "that rate / (1024 FLOP per clock per SIMD x SIMDs)"}
        _log(f"MFMA ceiling on N(0,1) operands: {ceiling:.1f} TFLOP/s")
    if not args.no_cpu_baseline:
        _log("cpu baseline: oracle on one GQA group")
        out["cpu_baseline"] = _cpu_baseline(w, q, k, v, o, t["do"], lse)
        _log(f"cpu baseline took {out['cpu_baseline']['seconds']:.1f} s")
    if side:
        del t, p, q, k, v, o, lse
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        out["side_workloads"] = {"extras": _summary(args, synth.EXTRAS_BF16),
                                 "causal_f32": _summary(args, synth.CAUSAL_F32)}
    return out


def bench_decode(args):
    import torch

    from flashattention_backward_pass_bwd_amd import api, synth

    w = synth.DECODE_F32
    dev = torch.device("cuda:0")
    N, H, Hkv, D, L = w.num_seqs, w.n_heads, w.n_kv_heads, w.head_dim, w.history_len
    k_hist = torch.empty((N, L, Hkv, D), dtype=torch.float32, device=dev)
    v_hist = torch.empty_like(k_hist)
    q = torch.empty((N, H, D), dtype=torch.float32, device=dev)
    d_out = torch.empty_like(q)
    for n in range(N):  # per-sequence seeded draws (same recipe as the tests)
        x = synth.decode_inputs(w, [n])
        k_hist[n].copy_(torch.from_numpy(x["k_hist"][0]))
        v_hist[n].copy_(torch.from_numpy(x["v_hist"][0]))
        q[n].copy_(torch.from_numpy(x["q"][0]))
        d_out[n].copy_(torch.from_numpy(x["d_out"][0]))
    g = H // Hkv
    # probs = softmax(q K^T), unscaled, from plain torch fp32 ops (input preparation only)
    probs = torch.empty((N, H, L), dtype=torch.float32, device=dev)
    for n in range(N):
        kk = k_hist[n].permute(1, 2, 0).contiguous()                 # [Hkv, D, L]
        qq = q[n].view(Hkv, g, D)
        probs[n] = torch.softmax(torch.matmul(qq, kk), dim=-1).reshape(H, L)
    d_scores = torch.empty_like(probs)
    d_q = torch.empty_like(q)
    for _ in range(args.warmup):
        api.decode_backward(k_hist, v_hist, probs, d_out, d_scores, d_q)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        api.decode_backward(k_hist, v_hist, probs, d_out, d_scores, d_q)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = start.elapsed_time(stop) / args.steps
    nbytes = 4 * (2 * N * L * Hkv * D + 2 * N * H * L + 2 * N * H * D)
    gbs = nbytes / (ms * 1e-3) / 1e9
    # pass 2 (history dK, dV from pass 1's d_scores), timed on its own after pass 1
    dk_hist = torch.empty_like(k_hist)
    dv_hist = torch.empty_like(v_hist)
    for _ in range(args.warmup):
        api.decode_dkdv(q, d_out, probs, d_scores, Hkv, dk_hist, dv_hist)
    torch.cuda.synchronize()
    s2, e2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s2.record()
    for _ in range(args.steps):
        api.decode_dkdv(q, d_out, probs, d_scores, Hkv, dk_hist, dv_hist)
    e2.record()
    torch.cuda.synchronize()
    ms2 = s2.elapsed_time(e2) / args.steps
    nbytes2 = 4 * (2 * N * L * Hkv * D + 2 * N * H * L + 2 * N * H * D)
    gbs2 = nbytes2 / (ms2 * 1e-3) / 1e9
    return {
        "metric": "decode-step attention-backward HBM GB/s, 1 GPU",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "wall_s_timed": round(wall, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": N, "n_heads": H, "n_kv_heads": Hkv, "head_dim": D,
                   "history_len": L, "algorithmic_bytes": nbytes},
        "roofline": {"kernel": "decode_kernel", "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "per_unit": "bytes of K,V rows + probs/d_scores + d_out/d_q", "units": nbytes},
        "pass2": {"kernel": "decode_kv_kernel", "what": "history dK, dV (fa_bwd_decode_dkdv)", "bound": "hbm",
                  "ms": round(ms2, 4), "achieved": round(gbs2, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                  "frac": round(gbs2 / PEAK_HBM_GBS, 4),
                  "per_unit": "dK,dV rows written + probs/d_scores + q/d_out read", "units": nbytes2},
    }


def bench_copy(args):
    """A plain elementwise copy kernel of known size (dst = -src, 1 GiB each way): calibrates the
    FETCH_SIZE / WRITE_SIZE counters.  (A same-dtype copy_ would be a DMA memcpy, not a kernel.)"""
    import torch

    n = 1 << 28  # 2^28 fp32 = 1 GiB read + 1 GiB written per launch
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        torch.neg(src, out=dst)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    nbytes = 2 * 4 * n
    return {"metric": "device copy GB/s (counter calibration)", "value": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic", "config": {"workload": "copy_1GiB", "bytes_read": 4 * n, "bytes_written": 4 * n}}


def main():
    args = _args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has no multi-GPU path; "
              "the per-GPU kernel is what one GPU runs when the work is sharded by (batch, KV head).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from flashattention_backward_pass_bwd_amd import synth

    if args.workload == "decode":
        out = bench_decode(args)
    elif args.workload == "copy":
        out = bench_copy(args)
    else:
        w = {"long": synth.LONG_BF16, "extras": synth.EXTRAS_BF16, "causal_f32": synth.CAUSAL_F32}[args.workload]
        out = bench_prefill(args, w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
