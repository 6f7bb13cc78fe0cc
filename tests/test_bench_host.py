"""Host-side logic of bench.py (no GPU): the FLOP counts its metric rests on,
the gating of the committed traffic counters, and the one-GPU refusal."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle
from flashattention_backward_pass_bwd_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("causal,offset,window,sq,sk", [
    (True, 0, 0, 70, 70), (True, 13, 0, 50, 90), (True, 0, 9, 64, 64), (True, 200, 0, 40, 30),
    (False, 0, 0, 33, 47), (False, 0, 7, 60, 40), (False, 0, 100, 20, 25), (True, 5, 300, 31, 80),
])
def test_visible_pairs_matches_brute_force(causal, offset, window, sq, sk):
    # the window-aware count equals the number of visible (i, j) in the oracle's definition
    w = synth.CAUSAL_F32.resized(seq_q=sq, seq_k=sk, causal=causal, causal_offset=offset, window=window)
    spec = oracle.Spec(scale=w.scale, causal=causal, causal_offset=offset, window=window)
    brute = int(oracle.visible(np.arange(sq), np.arange(sk), sq, sk, spec).sum())
    assert bench._visible_pairs(w) == brute


def test_nominal_flops_of_the_workloads():
    # 10 * B * H * Sq * Sk * D, halved when causal
    nominal, pairs, peak = bench._work(synth.LONG_BF16)
    assert nominal == 10.0 * 32 * 16384 * 16384 * 128 / 2 and peak == bench.PEAK_BF16_TFLOPS
    assert pairs == 32 * 16384 * 16385 // 2
    nominal, _, peak = bench._work(synth.CAUSAL_F32)
    assert nominal == 10.0 * 2 * 8 * 1024 * 1024 * 64 / 2 and peak == bench.PEAK_F32_TFLOPS
    nominal, pairs, _ = bench._work(synth.EXTRAS_BF16)
    assert nominal == 10.0 * 4 * 32 * 2048 * 2048 * 128 / 2
    # the window leaves far fewer pairs than the nominal causal count
    assert pairs == 4 * 32 * bench._visible_pairs(synth.EXTRAS_BF16) and pairs < 0.5 * 4 * 32 * 2048 * 2049 // 2


def test_traffic_counters_gated_by_the_kernel_sources(tmp_path, monkeypatch):
    got = bench._dkdv_traffic_bytes()
    assert got is None or got > 0
    lines = open(bench.TRAFFIC_FILE).read().splitlines()
    tampered = [("kernel_source_hash=0000000000000000" if l.startswith("kernel_source_hash=") else l) for l in lines]
    f = tmp_path / "traffic.txt"
    f.write_text("\n".join(tampered) + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench._dkdv_traffic_bytes() is None  # counters of other sources are not reported
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench._dkdv_traffic_bytes() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
