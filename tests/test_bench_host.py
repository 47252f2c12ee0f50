"""Host logic of bench.py (no GPU): the algorithmic FLOP and byte counts it
divides by, the kernel-source hash that decides whether the committed counter
runs still describe the kernels, the settle / warm-up / timed sequence of a
measurement (with torch's device calls replaced), and the refusal of more
than one GPU."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from attention_forward_online_amd.synth import SOFTMAX_WORKLOADS, WORKLOADS  # noqa: E402


def test_prefill_flops():
    # 4 B H N Nk d (QK^T and PV, 2 FLOPs per multiply-add), halved for causal
    w = WORKLOADS["causal_bf16_b4h16_n2048_d64"]
    assert bench.prefill_flops(w) == 2 * 4 * 16 * 2048 * 2048 * 64
    w = WORKLOADS["causal_bf16_b1h32_n8192_d128"]
    assert bench.prefill_flops(w) == 2 * 32 * 8192 * 8192 * 128
    w = WORKLOADS["tiny_f32_b1h1_n256_d64"]
    assert bench.prefill_flops(w) == 4 * 256 * 256 * 64
    # with key lengths only the visible keys count (clamped to [0, Nk])
    w = WORKLOADS["masked_bf16_b2h8_n4096_d128"]
    assert bench.prefill_flops(w, [1013, 0]) == 4 * 8 * 4096 * 128 * 1013
    assert bench.prefill_flops(w, [-5, 10 ** 9]) == 4 * 8 * 4096 * 128 * 4096


def test_prefill_bytes():
    # Q, K, V read once and O written (bf16), LSE written (fp32)
    w = WORKLOADS["causal_bf16_b1h32_n8192_d128"]
    assert bench.prefill_bytes(w) == 4 * 32 * 8192 * 128 * 2 + 32 * 8192 * 4
    # key lengths: only the visible K/V rows; a batch without keys reads no Q
    w = WORKLOADS["masked_bf16_b2h8_n4096_d128"]
    q_o = 2 * 8 * 4096 * 128 * 2 * 2 - 8 * 4096 * 128 * 2
    assert bench.prefill_bytes(w, [1013, 0]) == q_o + 2 * 8 * 1013 * 128 * 2 + 2 * 8 * 4096 * 4


def test_decode_bytes():
    # K and V read once, Q read, O and LSE written
    w = WORKLOADS["decode_bf16_b64h32_nk16384_d128"]
    kv = 2 * 64 * 32 * 16384 * 128 * 2
    assert bench.decode_bytes(w) == kv + 2 * 64 * 32 * 128 * 2 + 64 * 32 * 4
    assert bench.decode_bytes(w) == 17180925952


def test_softmax_bytes():
    w = next(iter(SOFTMAX_WORKLOADS.values()))
    el = 2 if w.dtype == "bf16" else 4
    assert bench.softmax_bytes(w) == 2 * w.rows * w.cols * el + w.rows * 4


def _hash_of(tree, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tree))
    return bench.kernel_source_hash()


def test_source_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    csrc = tmp_path / "attention_forward_online_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "attention_forward_online_amd", "csrc"), csrc,
                    ignore=shutil.ignore_patterns("*.o", "*.so"))
    h0 = _hash_of(tmp_path, monkeypatch)
    assert h0 == _hash_of(tmp_path, monkeypatch)          # deterministic
    f = csrc / "fa_decode.hip"
    text = f.read_text()
    f.write_text("// an added line comment\n/* and a\n   block comment */\n" +
                 text.replace("\n", "\n\n", 3))
    assert _hash_of(tmp_path, monkeypatch) == h0          # comments, blank lines: same
    f.write_text(text.replace("kUnroll = 16", "kUnroll = 8", 1))
    assert "kUnroll = 16" in text
    assert _hash_of(tmp_path, monkeypatch) != h0          # a code change: different
    # a record naming its own sources ignores changes to the others
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    fwd = bench.kernel_source_hash(bench.SOURCES_FWD)
    f.write_text(text)
    assert bench.kernel_source_hash(bench.SOURCES_FWD) == fwd
    assert bench.kernel_source_hash(bench.SOURCES_DECODE) != bench.kernel_source_hash(bench.SOURCES_FWD)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _replay_case(tile_values, d=64, n=32):
    """One wave of n query rows against len(tile_values) 64-key tiles whose
    scores (log2 units) are tile_values[t] for every key of tile t: q = e_0,
    k_j = x_j e_0 and scale = ln 2 make the log2-unit score exactly x_j."""
    import numpy as np
    nk = 64 * len(tile_values)
    q = np.zeros((1, n, d))
    q[0, :, 0] = 1.0
    k = np.zeros((1, nk, d))
    for t, x in enumerate(tile_values):
        k[0, 64 * t:64 * (t + 1), 0] = x
    return bench.replay_rescales(q, k, float(np.log(2.0)), False, None, d)


def test_rescale_replay_counts():
    # slowly growing tile maxima: the eager rule rescales on every step after
    # the first and moves the reference each time; the threshold (8) and the
    # guard (2^32) rules set it on the first tile only
    r = _replay_case([0.0, 0.5, 1.0, 1.5])
    assert r["wave_tile_steps"] == 4
    assert r["eager"] == {"rescaling_steps_frac": 0.75, "moves_per_row": 4.0}
    assert r["threshold"] == {"rescaling_steps_frac": 0.0, "moves_per_row": 1.0}
    assert r["guard"] == {"rescaling_steps_frac": 0.0, "moves_per_row": 1.0}
    # a jump of 20 on the third tile: past the threshold, but 32 weights of
    # 2^20 stay below the guard's 2^32
    r = _replay_case([0.0, 0.0, 20.0, 20.0])
    assert r["eager"]["moves_per_row"] == 2.0
    assert r["threshold"] == {"rescaling_steps_frac": 0.25, "moves_per_row": 2.0}
    assert r["guard"] == {"rescaling_steps_frac": 0.0, "moves_per_row": 1.0}
    # a jump of 40: weights of 2^40 would pass the guard's limit, so it moves
    # too (once: the later tile is then at its reference)
    r = _replay_case([0.0, 0.0, 40.0, 40.0])
    assert r["threshold"] == {"rescaling_steps_frac": 0.25, "moves_per_row": 2.0}
    assert r["guard"] == {"rescaling_steps_frac": 0.25, "moves_per_row": 2.0}
    # at d = 64 the guard checks the two 32-key halves of a tile separately:
    # a jump inside the second half of the first tile is caught there
    import numpy as np
    q = np.zeros((1, 32, 64)); q[0, :, 0] = 1.0
    k = np.zeros((1, 128, 64)); k[0, 32:64, 0] = 40.0; k[0, 64:, 0] = 40.0
    r = bench.replay_rescales(q, k, float(np.log(2.0)), False, None, 64)
    assert r["guard"]["moves_per_row"] == 1.0     # the first tile's max (40) is taken up front


def test_time_launches_settles_then_times(monkeypatch):
    """The settle phase (a call count from three timed calls, clamped to
    [10, 5000]) runs before the warm-ups, the timed region holds exactly the
    K steps, and the launch log records the untimed and timed counts."""
    import torch

    calls = []
    events = []

    class FakeEvent:
        def __init__(self, enable_timing=False):
            self.t = None
            events.append(self)

        def record(self):
            self.t = len(calls)

        def elapsed_time(self, other):
            return float(other.t - self.t)   # 1 ms per call in between

    monkeypatch.setattr(torch.cuda, "synchronize", lambda: None)
    monkeypatch.setattr(torch.cuda, "Event", FakeEvent)
    clock = iter([0.0, 0.003])
    monkeypatch.setattr(bench.time, "perf_counter", lambda: next(clock))
    monkeypatch.setattr(bench, "LAUNCH_LOG", [])
    ms = bench.time_launches(lambda: calls.append(1), 7, 2, settle_ms=60.0, label="x")
    # 3 estimate calls took 3 ms -> 1 ms per call -> 60 settle calls
    assert len(calls) == 3 + 60 + 2 + 7
    assert ms == 1.0
    assert bench.LAUNCH_LOG == [["x", 3 + 60 + 2, 7]]
    # no settle phase: only the warm-ups before the timed region
    del calls[:]
    bench.time_launches(lambda: calls.append(1), 5, 4, settle_ms=0, label="cold")
    assert len(calls) == 9 and bench.LAUNCH_LOG[-1] == ["cold", 4, 5]
