"""Throughput of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--only SECTION[,SECTION...]] [--copy-calibration]

A step is one fa_forward call on the long-context causal prefill
B=1 H=32 N=Nk=8192 d=128 bf16 (fp32 accumulation) -- the 8192-per-head,
32-head case whose score matrix would take 128 MiB per head -- with its inputs
resident in device memory before timing starts.  The headline value is
TFLOP/s with 4*B*H*N*Nk*d FLOPs halved for causal (QK^T and PV only).

The same run times, each for the same K steps after the same W warm-ups:
the other prefill workloads (causal d=64, masked high-dynamic-range d=128,
tiny fp32), the split-KV decode (GB/s), the row softmax (GB/s), the backward
on two causal shapes, the V1 loop-order ablation and the rescale-rule
ablation (the three rules timed in the same run, and how often each rescales,
replayed on the host).  It times the fp64 CPU oracle on the host's cores over the whole
headline workload as a reported baseline, and compares every element of the
timed run's output with it.  Prints one JSON line.

Kernel durations: the K timed launches run back to back between two HIP
events recorded on the stream the library launches on (torch's current
stream); one call is one kernel launch for the prefill workloads, so the
region divided by K is that kernel's average launch duration (plus the short
gaps between launches).  The forward and backward calls go through launchers
bound once (bind_forward / bind_backward: arguments checked when bound, not on
every call), so that the host keeps ahead of kernels of a few tens of
microseconds.  The cold-start diagnostic also records an event after every
launch to show the clock transient launch by launch.

Clock state.  After any idle gap (50 ms is enough) the MI355X's clock
controller answers a step to full matrix-core load with a dip: launches 3 to
~30 of the headline kernel run up to 30% slower (495 -> 640 -> 487 us) before
the clock settles, and the short workloads see the same dip after the host
work between sections.  Every measurement therefore first runs its own call
untimed back to back for about 60 ms (the count is in `launch_log`), then the
W warm-ups, then the K timed calls: each figure is the rate under sustained
load, the state the headline is timed in.  The headline is also timed once
at the very start with no such phase (`cold_start`, the same W and K), then
the split-KV decode runs (its own record; 2.5 ms of HBM-bound work per call),
then the headline is timed again: that is `value`.

Measured ceilings (`ceilings`): right after the decode, a bare streaming read
of the decode's K tensor; right after the headline, a bare stream of bf16
MFMAs with operands in registers; right after the row softmax, a bare
streaming copy of its input into its output (the probes of
include/fa_probe.h), each with the same W and K.  The published peaks assume a 2.4 GHz clock the chip does not
hold under sustained matrix-core load; each roofline record also gives its
rate as a fraction of the measured ceiling of its bound
(`frac_of_measured_ceiling`).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
METRIC = "fused attention fwd TFLOP/s + % bf16 MFMA peak; split-KV decode HBM GB/s"
HEADLINE = "causal_bf16_b1h32_n8192_d128"
PREFILLS = ("causal_bf16_b4h16_n2048_d64", "masked_bf16_b2h8_n4096_d128", "tiny_f32_b1h1_n256_d64")
DECODE = "decode_bf16_b64h32_nk16384_d128"
SOFTMAX = "softmax_f32_r1024_c262144"
BACKWARDS = ("causal_bf16_b4h16_n2048_d64", "causal_bf16_b1h32_n8192_d128")
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 512 * 1024 * 1024   # plain copy for counter calibration
PROBE_MFMA_BLOCKS = 512          # 2048 waves: two per SIMD, as the d=128 prefill runs
PROBE_MFMA_ITERS = 2000          # about half a millisecond per call
PROBE_READ_BLOCKS = 2048
PROBE_COPY_BLOCKS = 4096         # fastest of 512 .. 16384 in a sweep over a 1 GiB copy
SECTIONS = ("headline", "prefill", "decode", "softmax", "backward", "v1", "rescale")
RESCALE_WORKLOADS = ("causal_bf16_b4h16_n2048_d64", "causal_bf16_b1h32_n8192_d128", "masked_bf16_b2h8_n4096_d128")
GUARD_LOG2 = 32.0      # the guard rule keeps a pair group while its weight sum is below 2^32
TAU_LOG2 = 8.0         # the threshold rule's growth allowance (log2 units)

# kernel sources each measured path depends on (for the traffic records)
SOURCES_FWD = ("fa_fwd_bf16.hip", "fa_fwd_f32.hip", "fa_device.h", "fa_kernels.h", "fa_api.hip")
SOURCES_DECODE = ("fa_decode.hip", "fa_device.h", "fa_kernels.h", "fa_api.hip")
SOURCES_SOFTMAX = ("fa_softmax.hip", "fa_device.h", "fa_kernels.h", "fa_api.hip")
SOURCES_BWD = ("fa_bwd_bf16.hip", "fa_device.h", "fa_kernels.h", "fa_api.hip")


def prefill_flops(w, key_lens=None):
    """4*B*H*N*Nk*d (halved for causal); with key lengths the visible count."""
    if key_lens is not None:
        return 4.0 * w.H * w.N * w.d * float(sum(min(max(k, 0), w.Nk) for k in key_lens))
    f = 4.0 * w.B * w.H * w.N * w.Nk * w.d
    return f / 2 if w.causal else f


def prefill_bytes(w, key_lens=None):
    """Compulsory HBM bytes of one prefill call: Q, K, V read once (the visible
    keys only), O and LSE written."""
    el = 2 if w.dtype == "bf16" else 4
    qo = 2 * w.B * w.H * w.N * w.d * el
    if key_lens is None:
        kv = 2 * w.B * w.H * w.Nk * w.d * el
    else:
        kv = 2 * w.H * w.d * el * sum(min(max(k, 0), w.Nk) for k in key_lens)
        # a batch without keys reads no Q either
        qo -= w.H * w.N * w.d * el * sum(1 for k in key_lens if min(max(k, 0), w.Nk) == 0)
    return qo + kv + w.B * w.H * w.N * 4


def decode_bytes(w):
    """Compulsory HBM bytes of one decode call: K, V, Q read; O, LSE written."""
    el = 2 if w.dtype == "bf16" else 4
    return (2 * w.B * w.H * w.Nk * w.d + 2 * w.B * w.H * w.d) * el + w.B * w.H * 4


def softmax_bytes(w):
    """Compulsory HBM bytes of one row-softmax call: X read once, Y and LSE written."""
    el = 2 if w.dtype == "bf16" else 4
    return 2 * w.rows * w.cols * el + w.rows * 4


SETTLE_MS = 60.0       # untimed back-to-back load before each measurement (see time_launches)
LAUNCH_LOG = []        # [label, untimed calls, timed calls] per measurement, in run order


def time_launches(fn, steps, warmup, per_launch=False, settle_ms=SETTLE_MS, label=""):
    """Run `fn` back to back untimed for about `settle_ms` (a call count from
    three timed calls), then `warmup` untimed calls, a device synchronisation,
    then `steps` back-to-back calls between two HIP events recorded on torch's
    current stream (the stream the library launches on); synchronised again.
    Returns ms per step over that region.  The settle phase puts every
    measurement in the same sustained-load clock state the headline is timed
    in: after host work between sections the clock controller answers a step
    to full load with a dip lasting tens of milliseconds, longer than W
    warm-ups of a short kernel (settle_ms=0 times the dip on purpose).  With
    per_launch, an event is also recorded after every call and the per-call
    durations are returned too (each event between launches adds a few
    microseconds, so this is for diagnostics)."""
    import torch
    untimed = warmup
    if settle_ms > 0:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        per = max((time.perf_counter() - t0) / 3, 1e-6)
        n = min(max(int(settle_ms * 1e-3 / per + 0.5), 10), 5000)
        for _ in range(n):
            fn()
        untimed += 3 + n
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    LAUNCH_LOG.append([label, untimed, steps])
    n_ev = steps + 1 if per_launch else 2
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ev[0].record()
    for i in range(steps):
        fn()
        if per_launch:
            ev[i + 1].record()
    if not per_launch:
        ev[1].record()
    torch.cuda.synchronize()
    region = ev[0].elapsed_time(ev[-1]) / steps
    if not per_launch:
        return region
    return region, [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def launch_stats(per):
    return {"mean_ms": round(sum(per) / len(per), 5), "min_ms": round(min(per), 5),
            "median_ms": round(statistics.median(per), 5), "max_ms": round(max(per), 5),
            "last5_mean_ms": round(sum(per[-5:]) / len(per[-5:]), 5)}


def kernel_source_hash(files=None):
    """sha256 (first 16 hex digits) of kernel sources with comments and white
    space removed (all of csrc/*.hip|*.h, or the named files): a change to the
    code changes it, an edit to a comment alone does not."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_forward_online_amd", "csrc")
    names = sorted(files) if files else sorted(n for n in os.listdir(csrc) if n.endswith((".hip", ".h")))
    for name in names:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            code = re.sub(r"//[^\n]*|/\*.*?\*/", " ", f.read(), flags=re.S)
        h.update(name.encode() + "".join(code.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(key):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when the sources the record names changed after the counters were taken."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    rec = t.get(key)
    if not rec or rec.get("source_hash") != kernel_source_hash(rec.get("sources")):
        return None
    return rec.get("bytes_per_launch")


def replay_rescales(q, k, scale, causal, key_len, d, rows_per_wave=32, tile=64, heads=None):
    """Host replay of the three rescale rules over fp64 scores, in the kernel's
    grouping (waves of 32 query rows, tiles of 64 keys; the guard checks each
    pair group -- keys 0..31 and 32..63 of a tile at d=64, the whole tile at
    d=128 -- before using it).  Per rule: the fraction of (wave, tile) steps
    on which the wave rescales its accumulators, and per row the mean number
    of reference moves.  q, k: float64 [BH, N, d] / [BH, Nk, d]; key_len per
    head (None: all keys)."""
    import numpy as np
    BH, N, _ = q.shape
    Nk = k.shape[1]
    c = scale / np.log(2.0)
    groups = [(0, 32), (32, 64)] if d == 64 else [(0, 64)]
    steps = {"eager": 0, "threshold": 0, "guard": 0}
    moves = {"eager": 0.0, "threshold": 0.0, "guard": 0.0}
    total = 0
    for bh in (heads if heads is not None else range(BH)):
        kl = Nk if key_len is None else key_len[bh]
        if kl <= 0:
            continue
        s = (q[bh] @ k[bh, :kl].T) * c                      # log2 units
        j = np.arange(kl)[None, :]
        if causal:
            s = np.where(j <= np.arange(N)[:, None] + (Nk - N), s, -np.inf)
        for w0 in range(0, N, rows_per_wave):
            sw = s[w0:w0 + rows_per_wave]
            vis_any = np.isfinite(sw).any(axis=0)
            ntile = (int(np.nonzero(vis_any)[0].max()) // tile + 1) if vis_any.any() else 0
            m_eager = np.full(sw.shape[0], -np.inf)
            m_thr = np.full(sw.shape[0], -np.inf)
            m_grd = np.full(sw.shape[0], -np.inf)
            for t in range(ntile):
                st = sw[:, t * tile:(t + 1) * tile]
                mx = st.max(axis=1)
                total += 1
                if t > 0:
                    steps["eager"] += 1
                moves["eager"] += float(np.sum(mx > m_eager))
                m_eager = np.maximum(m_eager, mx)
                mv = mx > m_thr + TAU_LOG2
                if t == 0 or mv.any():
                    steps["threshold"] += 1 if t > 0 else 0
                moves["threshold"] += float(np.sum(mv))
                m_thr = np.where(mv, mx, m_thr)
                slow = False
                if t == 0:          # the first tile's max is always taken (prologue)
                    mvg = mx > m_grd
                    moves["guard"] += float(np.sum(mvg))
                    m_grd = np.where(mvg, mx, m_grd)
                for a, b in groups:
                    sg = st[:, a:b]
                    if sg.shape[1] == 0:
                        continue
                    ref = np.where(np.isfinite(m_grd), m_grd, 0.0)
                    with np.errstate(over="ignore", invalid="ignore"):
                        wsum = np.exp2(sg - ref[:, None]).sum(axis=1)
                    if not np.isfinite(m_grd).all() or (~(wsum < 2.0 ** GUARD_LOG2)).any():
                        gm = sg.max(axis=1)
                        mvg = gm > m_grd
                        moves["guard"] += float(np.sum(mvg))
                        m_grd = np.where(mvg, gm, m_grd)
                        slow = slow or t > 0
                if slow:
                    steps["guard"] += 1
    rows = sum(1 for bh in (heads if heads is not None else range(BH))
               if (Nk if key_len is None else key_len[bh]) > 0) * N
    return {r: {"rescaling_steps_frac": round(steps[r] / max(total, 1), 5),
                "moves_per_row": round(moves[r] / max(rows, 1), 3)} for r in steps} | {"wave_tile_steps": total}


def mfma_roofline(flops, ms, kernel, traffic_key, alg_bytes, peak=PEAK_BF16_TFLOPS):
    """Roofline record of a one-kernel-per-call workload: `ms` is the average
    launch duration over the timed region (HIP events around the back-to-back
    launches, so it also holds the short gaps between them)."""
    achieved = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma" if peak == PEAK_BF16_TFLOPS else "alu", "achieved": round(achieved, 2),
            "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(traffic_key), "algorithmic_bytes": alg_bytes,
            "kernel": kernel, "ms_per_launch": round(ms, 5),
            "timing": "HIP events around the timed region / launches (gaps between launches included); "
                      "the rocprofv3 kernel-trace mean of the same launches is at or below it"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None,
                    help="comma-separated sections to run (used under the profiler): "
                         + ", ".join(SECTIONS) + "; 'prefill:NAME' for one prefill workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy, whose FETCH_SIZE / WRITE_SIZE "
                         "counters scale the kernels' counters to bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(every workload here is measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    only = None
    if args.only:
        only = set()
        for s in args.only.split(","):
            if s.split(":")[0] not in SECTIONS:
                ap.error(f"unknown section {s!r}")
            only.add(s)

    def want(section, name=None):
        if only is None:
            return True
        return section in only or (name is not None and f"{section}:{name}" in only)

    import numpy as np
    import torch

    import attention_forward_online_amd as fa
    from attention_forward_online_amd import build as fabuild
    from attention_forward_online_amd.synth import (SOFTMAX_WORKLOADS, WORKLOADS, make_inputs,
                                                    make_softmax_input, randn_slices)

    if not os.path.exists(fabuild.LIB_PATH):
        fabuild.build()
    fa.load_library()
    torch.cuda.set_device(0)
    dev = "cuda"
    K, W = args.steps, args.warmup

    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    out = {"metric": METRIC}
    ceilings = {}
    # ---------------------------------------------------------------- headline
    w = WORKLOADS[HEADLINE]
    if want("headline") or want("backward") or not args.no_cpu_baseline:
        inp = make_inputs(w, device=dev)
        q, k, v = inp["q"], inp["k"], inp["v"]
        o = torch.empty_like(q)
        lse = torch.empty(w.B, w.H, w.N, device=dev, dtype=torch.float32)
    if want("headline"):
        # cold start: the same W and K right away (context only, see the module doc)
        ms_cold, per_cold = time_launches(fa.bind_forward(q, k, v, o, lse, causal=True), K, W,
                                          per_launch=True, settle_ms=0, label="headline cold")
        out["cold_start"] = {"ms_per_step": round(ms_cold, 5),
                             "tflops": round(prefill_flops(w) / (ms_cold * 1e-3) / 1e12, 2),
                             "launches": launch_stats(per_cold),
                             "note": "headline timed first in the run, W warm-ups after idle: inside "
                                     "the clock controller's dip; value is timed after the decode"}

    # ------------------------------------------------------------ decode
    if want("decode"):
        wd = WORKLOADS[DECODE]
        di = make_inputs(wd, device=dev)
        od = torch.empty_like(di["q"])
        ld = torch.empty(wd.B, wd.H, 1, device=dev, dtype=torch.float32)
        nb = fa.fa_decode_workspace_bytes(wd.B, wd.H, wd.d, wd.num_splits)
        ws = torch.empty(nb // 4, device=dev, dtype=torch.float32)
        ms_d = time_launches(
            lambda: fa.fa_decode_splitkv(di["q"], di["k"], di["v"], od, ld, wd.num_splits, ws), K, W,
            label="decode")
        nbytes = decode_bytes(wd)
        gbs = nbytes / (ms_d * 1e-3) / 1e9
        out["decode"] = {
            "workload": wd.describe(), "name": DECODE, "value": round(gbs, 1), "unit": "GB/s",
            "ms_per_call": round(ms_d, 4), "bytes_per_call": nbytes, "workspace_bytes": nb,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("decode/" + DECODE),
                         "kernels": "decode_split_kernel + decode_combine_kernel"},
        }
        # measured ceiling of the decode: a bare streaming read of its K tensor
        # (the same 16-byte nontemporal loads, no arithmetic, include/fa_probe.h)
        sink_r = torch.empty(PROBE_READ_BLOCKS * fa.PROBE_THREADS, dtype=torch.int32, device=dev)
        ms_r = time_launches(lambda: fa.probe_read(di["k"], PROBE_READ_BLOCKS, sink_r), K, W,
                             label="probe read")
        rbytes = di["k"].numel() * di["k"].element_size()
        read_gbs = rbytes / (ms_r * 1e-3) / 1e9
        ceilings["hbm_read_stream"] = {
            "gbs": round(read_gbs, 1), "frac_of_peak": round(read_gbs / PEAK_HBM_GBS, 4),
            "ms_per_call": round(ms_r, 4), "bytes_per_call": rbytes,
            "probe": f"fa_probe_read: {PROBE_READ_BLOCKS} workgroups of 256 threads reading 64 KiB chunks "
                     "in 16-byte nontemporal loads, the decode workload's K tensor, timed right after "
                     "the decode"}
        out["decode"]["roofline"]["frac_of_measured_ceiling"] = round(gbs / read_gbs, 4)
        del sink_r

    if want("headline"):
        # one fa_forward call launches exactly one kernel, fwd_bf16_kernel<128, causal>
        # (timed after the decode section: the clock has settled, see the module doc)
        ms_step = time_launches(fa.bind_forward(q, k, v, o, lse, causal=True), K, W, label="headline")
        flops = prefill_flops(w)
        value = flops / (ms_step * 1e-3) / 1e12
        out.update({
            "value": round(value, 2),
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": K,
            "warmup": W,
            "ms_per_step": round(ms_step, 5),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic: seeded iid N(0,1) bf16 Q, K, V drawn on the device",
            "config": {"workload": w.describe(), "name": HEADLINE, "B": w.B, "H": w.H, "N": w.N,
                       "Nk": w.Nk, "d": w.d, "causal": True, "scale": w.scale,
                       "flops_per_step": flops},
            "roofline": mfma_roofline(flops, ms_step, "fwd_bf16_kernel<128,true,1,2>",
                                      "forward/" + HEADLINE, prefill_bytes(w)),
        })
        # measured ceiling of the prefill: a bare stream of bf16 MFMAs (operands in
        # registers, no softmax, no memory traffic, include/fa_probe.h), timed
        # right after the headline with the same clock state, W and K
        sink_m = torch.empty(PROBE_MFMA_BLOCKS * fa.PROBE_THREADS, dtype=torch.float32, device=dev)
        ms_m = time_launches(lambda: fa.probe_mfma(PROBE_MFMA_BLOCKS, PROBE_MFMA_ITERS, sink_m), K, W,
                             label="probe mfma")
        mfl = PROBE_MFMA_BLOCKS * PROBE_MFMA_ITERS * fa.PROBE_MFMA_FLOPS
        mfma_tflops = mfl / (ms_m * 1e-3) / 1e12
        ceilings["mfma_bf16_stream"] = {
            "tflops": round(mfma_tflops, 2), "frac_of_peak": round(mfma_tflops / PEAK_BF16_TFLOPS, 4),
            "ms_per_call": round(ms_m, 4), "flops_per_call": mfl,
            "probe": f"fa_probe_mfma: {PROBE_MFMA_BLOCKS} workgroups of 4 waves (2 per SIMD), "
                     f"{PROBE_MFMA_ITERS} rounds of 8 v_mfma_f32_32x32x16_bf16 (4 chains) per wave on random bf16 "
                     "operands held in registers"}
        out["roofline"]["frac_of_measured_ceiling"] = round(value / mfma_tflops, 4)
        del sink_m
    if want("decode"):
        del di, od, ld, ws
        torch.cuda.empty_cache()

    # ------------------------------------------------------ other prefill workloads
    others = {}
    for name in PREFILLS:
        if not want("prefill", name):
            continue
        wo = WORKLOADS[name]
        oi = make_inputs(wo, device=dev)
        oo = torch.empty_like(oi["q"])
        ol = torch.empty(wo.B, wo.H, wo.N, device=dev, dtype=torch.float32)
        kl = oi["key_lens"]
        ms_o = time_launches(fa.bind_forward(oi["q"], oi["k"], oi["v"], oo, ol, causal=wo.causal,
                                             key_lens=kl), K, W, label=name)
        kll = kl.tolist() if kl is not None else None
        fl = prefill_flops(wo, kll)
        peak = PEAK_F32_TFLOPS if wo.dtype == "f32" else PEAK_BF16_TFLOPS
        kname = ("fwd_f32_kernel" if wo.dtype == "f32" else
                 f"fwd_bf16_kernel<{wo.d},{'true' if wo.causal else 'false'},1,2>")
        rec = {"workload": wo.describe(), "ms_per_call": round(ms_o, 5),
               "tflops": round(fl / (ms_o * 1e-3) / 1e12, 2),
               "flops_per_call": fl,
               "roofline": mfma_roofline(fl, ms_o, kname, "forward/" + name, prefill_bytes(wo, kll), peak)}
        if "mfma_bf16_stream" in ceilings and wo.dtype != "f32":
            rec["roofline"]["frac_of_measured_ceiling"] = round(
                rec["roofline"]["achieved"] / ceilings["mfma_bf16_stream"]["tflops"], 4)
        if kll is not None:
            rec["key_lens"] = kll
            rec["flops_convention"] = "effective: 4*H*N*d*sum(key_lens) (visible keys only)"
            rec["tflops_nominal"] = round(prefill_flops(wo) / (ms_o * 1e-3) / 1e12, 2)
        others[name] = rec
        del oi, oo, ol
    if others:
        out["workloads"] = others

    # ------------------------------------------------------- row softmax
    if want("softmax"):
        wsm = SOFTMAX_WORKLOADS[SOFTMAX]
        xs = make_softmax_input(wsm, device=dev)
        ys = torch.empty_like(xs)
        ls = torch.empty(wsm.rows, device=dev, dtype=torch.float32)
        nb = fa.fa_softmax_workspace_bytes(wsm.rows, wsm.cols, xs.dtype)
        wss = torch.empty(max(nb, 16) // 4, device=dev, dtype=torch.float32)
        ms_s = time_launches(lambda: fa.fa_softmax(xs, ys, ls, wss), K, W, label="softmax")
        nbytes = softmax_bytes(wsm)
        gbs = nbytes / (ms_s * 1e-3) / 1e9
        out["softmax"] = {
            "workload": wsm.describe(), "name": SOFTMAX, "value": round(gbs, 1), "unit": "GB/s",
            "ms_per_call": round(ms_s, 4), "bytes_per_call": nbytes, "workspace_bytes": nb,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("softmax/" + SOFTMAX),
                         "kernels": "softmax_reset_kernel + softmax_coop_kernel (one pass over X)"},
        }
        # measured ceiling of the softmax: a bare streaming copy of X into Y (the
        # same bytes read and written, 16-byte nontemporal loads and stores,
        # include/fa_probe.h)
        ms_c = time_launches(lambda: fa.probe_copy(xs, ys, PROBE_COPY_BLOCKS), K, W, label="probe copy")
        cbytes = 2 * xs.numel() * xs.element_size()
        copy_gbs = cbytes / (ms_c * 1e-3) / 1e9
        ceilings["hbm_copy_stream"] = {
            "gbs": round(copy_gbs, 1), "frac_of_peak": round(copy_gbs / PEAK_HBM_GBS, 4),
            "ms_per_call": round(ms_c, 4), "bytes_per_call": cbytes,
            "probe": f"fa_probe_copy: {PROBE_COPY_BLOCKS} workgroups of 256 threads copying 64 KiB chunks "
                     "in 16-byte nontemporal loads and stores, the softmax workload's X into its Y "
                     "(bytes read plus bytes written), timed right after the softmax"}
        out["softmax"]["roofline"]["frac_of_measured_ceiling"] = round(gbs / copy_gbs, 4)
        del xs, ys, ls, wss
        torch.cuda.empty_cache()

    # ------------------------------------------------- backward, two causal shapes
    if want("backward"):
        bw = {}
        for name in BACKWARDS:
            wb = WORKLOADS[name]
            if name == HEADLINE:
                bi, bo, bl = inp, o, lse
            else:
                bi = make_inputs(wb, device=dev)
                bo = torch.empty_like(bi["q"])
                bl = torch.empty(wb.B, wb.H, wb.N, device=dev, dtype=torch.float32)
            fa.fa_forward(bi["q"], bi["k"], bi["v"], bo, bl, causal=True)
            dob = randn_slices(tuple(bi["q"].shape), 1.0, torch.bfloat16, 0, wb.name, "do", dev)
            dq, dk, dv = (torch.empty_like(bi[t]) for t in ("q", "k", "v"))
            nbw = fa.fa_backward_workspace_bytes(wb.B, wb.H, wb.N)
            wsb = torch.empty(max(nbw, 16) // 4, device=dev, dtype=torch.float32)
            ms_b = time_launches(
                fa.bind_backward(bi["q"], bi["k"], bi["v"], bo, dob, bl, dq, dk, dv, wsb, causal=True),
                K, W, label="backward " + name)
            bflops = 2.5 * prefill_flops(wb)
            el = 2
            alg = 8 * wb.B * wb.H * wb.N * wb.d * el + wb.B * wb.H * wb.N * 4
            bw[name] = {
                "workload": wb.describe() + " backward (dQ, dK, dV from O, dO, LSE)",
                "ms_per_call": round(ms_b, 5), "tflops": round(bflops / (ms_b * 1e-3) / 1e12, 2),
                "flops_per_call": bflops,
                "flops_convention": "5 GEMMs (QK^T, dP, dV, dK, dQ) = 2.5 x forward, halved for causal",
                "roofline": mfma_roofline(bflops, ms_b, "bwd_dq_kernel + " + ("bwd_dkdv_kernel" if wb.d == 64 else "bwd_dkdv_paired_kernel"),
                                          "backward/" + name, alg),
            }
            del dob, dq, dk, dv, wsb
            if name != HEADLINE:
                del bi, bo, bl
        out["backward"] = bw

    # ------------------------------------ V1 loop order (ablation), d=64 causal shape
    if want("v1"):
        wv = WORKLOADS["causal_bf16_b4h16_n2048_d64"]
        vi = make_inputs(wv, device=dev)
        o1 = torch.empty_like(vi["q"])
        l1 = torch.empty(wv.B, wv.H, wv.N, device=dev, dtype=torch.float32)
        nv1 = fa.fa_forward_v1_workspace_bytes(wv.B, wv.H, wv.N, wv.d)
        wv1 = torch.empty(max(nv1, 16) // 4, device=dev, dtype=torch.float32)
        ms_v1 = time_launches(lambda: fa.fa_forward_v1(vi["q"], vi["k"], vi["v"], o1, l1, wv1, causal=True),
                              K, W, label="v1")
        ms_v2 = time_launches(fa.bind_forward(vi["q"], vi["k"], vi["v"], o1, l1, causal=True), K, W,
                              label="v1 ablation v2 leg")
        fl = prefill_flops(wv)
        out["v1_ablation"] = {
            "workload": wv.describe() + " in the V1 loop order (KV outer, Q inner, O/m/l via HBM)",
            "ms_per_call": round(ms_v1, 4), "tflops": round(fl / (ms_v1 * 1e-3) / 1e12, 2),
            "v2_ms_per_call": round(ms_v2, 5), "v1_over_v2_time": round(ms_v1 / ms_v2, 2),
            "workspace_bytes": nv1,
            "note": "one workgroup per (b, h) as in V1: 64 workgroups on 256 CUs",
        }
        del vi, o1, l1, wv1

    # ----------------------------- rescale rules (FA-4 ablation): timing + host replay
    if want("rescale"):
        rules = (("eager", fa.RESCALE_EAGER), ("threshold", fa.RESCALE_THRESHOLD), ("guard", fa.RESCALE_GUARD))
        ab = {}
        for name in RESCALE_WORKLOADS:
            wr = WORKLOADS[name]
            ri = inp if name == HEADLINE and want("headline") else make_inputs(wr, device=dev)
            ro = torch.empty_like(ri["q"])
            rl = torch.empty(wr.B, wr.H, wr.N, device=dev, dtype=torch.float32)
            kl = ri["key_lens"]
            rec = {"workload": wr.describe()}
            try:
                for rn, code in rules:
                    fa.testing_set_rescale_rule(code)
                    ms_r = time_launches(fa.bind_forward(ri["q"], ri["k"], ri["v"], ro, rl,
                                                         causal=wr.causal, key_lens=kl), K, W,
                                         label=f"rescale {rn} {name}")
                    rec[rn + "_ms"] = round(ms_r, 5)
            finally:
                fa.testing_set_rescale_rule(fa.RESCALE_GUARD)
            rec["guard_vs_eager_time"] = round(rec["guard_ms"] / rec["eager_ms"], 4)
            rec["guard_vs_threshold_time"] = round(rec["guard_ms"] / rec["threshold_ms"], 4)
            rec["threshold_vs_eager_time"] = round(rec["threshold_ms"] / rec["eager_ms"], 4)
            # replay: every head of the smaller workloads, 4 heads of the 8192-long one
            qd = ri["q"].reshape(-1, wr.N, wr.d).double().cpu().numpy()
            kd = ri["k"].reshape(-1, wr.Nk, wr.d).double().cpu().numpy()
            klh = None if kl is None else [int(x) for x in kl.tolist() for _ in range(wr.H)]
            heads = None if wr.B * wr.H * wr.N * wr.Nk <= 2 ** 29 else [0, 9, 18, 31]
            rec["replay"] = replay_rescales(qd, kd, wr.scale, wr.causal, klh, wr.d, heads=heads)
            rec["replay"]["heads"] = "all" if heads is None else heads
            ab[name] = rec
            del ro, rl, qd, kd
        out["rescale_ablation"] = ab

    # ----------------------------------------------- CPU oracle baseline + parity
    if not args.no_cpu_baseline:
        import oracle
        nthreads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
        if not want("headline"):
            fa.fa_forward(q, k, v, o, lse, causal=True)
        torch.cuda.synchronize()
        qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
        t = time.perf_counter()
        O_ref, L_ref = oracle.attention(qh, kh, vh, scale=float(np.float32(w.scale)), causal=True,
                                        nthreads=nthreads)
        dt = time.perf_counter() - t
        flops = prefill_flops(w)
        out["cpu_baseline"] = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s",
                               "cores": nthreads, "kind": "oracle",
                               "sample": f"the whole headline workload ({HEADLINE}): every one of its "
                                         f"{w.B * w.H * w.N} rows, one fp64 pass, {dt:.2f} s wall"}
        # the oracle's outputs double as an element-wise parity check of the timed run
        og = o.double().cpu().numpy()
        lg = lse.double().cpu().numpy()
        out["parity"] = {"rows_compared": int(w.B * w.H * w.N), "max_abs_O": float(np.abs(og - O_ref).max()),
                         "max_abs_LSE": float(np.abs(lg - L_ref).max()),
                         "nan": bool(np.isnan(og).any() or np.isnan(lg).any()),
                         "tolerance": {"O": 2e-2, "LSE": 1e-3}}
        del O_ref, L_ref, og, lg
    if ceilings:
        out["ceilings"] = ceilings
    out["launch_log"] = LAUNCH_LOG
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
