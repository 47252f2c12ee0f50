"""Throughput of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one fa_forward call on the causal prefill workload
B=4 H=16 N=Nk=2048 d=64 bf16 (fp32 accumulation); its inputs are resident in
device memory before timing starts.  The headline value is TFLOP/s with
4*B*H*N*Nk*d FLOPs halved for causal (QK^T and PV only).  The same run also
times the split-KV decode (B=64 H=32, Nk=16384, d=128, 16 splits) in HBM GB/s
and the other prefill workloads, and times the fp64 CPU oracle on the host's
cores on the headline workload as a reported baseline.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
METRIC = "fused attention fwd TFLOP/s + % bf16 MFMA peak; split-KV decode HBM GB/s"
HEADLINE = "causal_bf16_b4h16_n2048_d64"
DECODE = "decode_bf16_b64h32_nk16384_d128"
SOFTMAX = "softmax_f32_r1024_c262144"
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 512 * 1024 * 1024   # plain copy for counter calibration


def prefill_flops(w, key_lens=None):
    """4*B*H*N*Nk*d (halved for causal); with key lengths the visible count."""
    if key_lens is not None:
        return 4.0 * w.H * w.N * w.d * float(sum(min(max(k, 0), w.Nk) for k in key_lens))
    f = 4.0 * w.B * w.H * w.N * w.Nk * w.d
    return f / 2 if w.causal else f


def decode_bytes(w):
    """Compulsory HBM bytes of one decode call: K, V, Q read; O, LSE written."""
    el = 2 if w.dtype == "bf16" else 4
    return (2 * w.B * w.H * w.Nk * w.d + 2 * w.B * w.H * w.d) * el + w.B * w.H * 4


def softmax_bytes(w):
    """Compulsory HBM bytes of one row-softmax call: X read once, Y and LSE written."""
    el = 2 if w.dtype == "bf16" else 4
    return 2 * w.rows * w.cols * el + w.rows * 4


def time_region(fn, steps, warmup):
    """Milliseconds per call: HIP events on torch's current stream (the stream
    the library launches on) bracket `steps` back-to-back calls, after
    `warmup` untimed calls and a device synchronisation on both sides."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        fn()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def kernel_source_hash():
    """sha256 (first 16 hex digits) of the kernel sources with comments and
    white space removed: any change to the code changes it, an edit to a
    comment alone does not."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_forward_online_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), encoding="utf-8") as f:
                code = re.sub(r"//[^\n]*|/\*.*?\*/", " ", f.read(), flags=re.S)
            h.update(name.encode() + "".join(code.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when the kernels changed after the counters were taken."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    rec = t.get(kernel_key)
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-headline", action="store_true",
                    help="time only the headline prefill (used under the profiler)")
    ap.add_argument("--only-decode", action="store_true",
                    help="time only the split-KV decode (used under the profiler)")
    ap.add_argument("--only-backward", action="store_true",
                    help="time only the backward on the headline shape (used under the profiler)")
    ap.add_argument("--only-softmax", action="store_true",
                    help="time only the row softmax (used under the profiler)")
    ap.add_argument("--only-long", action="store_true",
                    help="time only the 8192-long d=128 causal prefill (used under the profiler)")
    ap.add_argument("--only-prefill", default=None,
                    choices=["causal_bf16_b1h32_n8192_d128", "masked_bf16_b2h8_n4096_d128",
                             "tiny_f32_b1h1_n256_d64"],
                    help="time only this prefill workload (used under the profiler)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy, whose FETCH_SIZE / WRITE_SIZE "
                         "counters scale the kernel's counters to bytes")
    args = ap.parse_args()
    if args.only_long:
        args.only_prefill = "causal_bf16_b1h32_n8192_d128"
    args.only_long = args.only_prefill is not None
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(every workload here is measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import attention_forward_online_amd as fa
    from attention_forward_online_amd import build as fabuild
    from attention_forward_online_amd.synth import (SOFTMAX_WORKLOADS, WORKLOADS, make_inputs,
                                                    make_softmax_input)

    if not os.path.exists(fabuild.LIB_PATH):
        fabuild.build()
    fa.load_library()
    torch.cuda.set_device(0)
    dev = "cuda"

    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------------------------------------------------------- headline
    w = WORKLOADS[HEADLINE]
    inp = make_inputs(w, device=dev)
    q, k, v = inp["q"], inp["k"], inp["v"]
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.N, device=dev, dtype=torch.float32)
    # one fa_forward call launches exactly one kernel, so the time per step is
    # that kernel's average launch duration (plus any gap between launches)
    side_only = args.only_decode or args.only_softmax or args.only_backward or args.only_long
    ms_step = time_region(lambda: fa.fa_forward(q, k, v, o, lse, causal=True),
                          args.steps if not side_only else 1,
                          args.warmup if not side_only else 0)
    flops = prefill_flops(w)
    avg_launch = ms_step
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (avg_launch * 1e-3) / 1e12
    traffic = measured_traffic("fwd_bf16_kernel<64,true,1>/" + HEADLINE)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded iid N(0,1) bf16 Q, K, V drawn on the device",
        "config": {"workload": w.describe(), "name": HEADLINE, "B": w.B, "H": w.H, "N": w.N,
                   "Nk": w.Nk, "d": w.d, "causal": True, "scale": w.scale,
                   "flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": "fwd_bf16_kernel<64,true,1>",
                     "avg_launch_ms": round(avg_launch, 5)},
    }
    head_out = (o, lse)

    if side_only:
        out = {"metric": METRIC}
    if not (args.only_headline or args.only_softmax or args.only_backward or args.only_long):
        # ------------------------------------------------------------ decode
        wd = WORKLOADS[DECODE]
        di = make_inputs(wd, device=dev)
        od = torch.empty_like(di["q"])
        ld = torch.empty(wd.B, wd.H, 1, device=dev, dtype=torch.float32)
        nb = fa.fa_decode_workspace_bytes(wd.B, wd.H, wd.d, wd.num_splits)
        ws = torch.empty(nb // 4, device=dev, dtype=torch.float32)
        dsteps = max(5, args.steps // 5)
        ms_d = time_region(
            lambda: fa.fa_decode_splitkv(di["q"], di["k"], di["v"], od, ld, wd.num_splits, ws),
            dsteps, max(2, args.warmup // 2))
        nbytes = decode_bytes(wd)
        gbs = nbytes / (ms_d * 1e-3) / 1e9
        gbs_launch = gbs   # split + combine, the whole call
        out["decode"] = {
            "workload": wd.describe(), "name": DECODE, "value": round(gbs, 1), "unit": "GB/s",
            "ms_per_call": round(ms_d, 4), "bytes_per_call": nbytes,
            "workspace_bytes": nb,
            "roofline": {"bound": "hbm", "achieved": round(gbs_launch, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs_launch / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("decode/" + DECODE),
                         "kernels": "decode_split_kernel + decode_combine_kernel"},
        }
        del di, od, ld, ws
        torch.cuda.empty_cache()

    if not (args.only_headline or args.only_decode or args.only_softmax or args.only_long):
        # ------------------------------------------------ backward (headline shape)
        from attention_forward_online_amd.synth import randn_slices
        dob = randn_slices((w.B, w.H, w.N, w.d), 1.0, torch.bfloat16, 0, w.name, "do", dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        nbw = fa.fa_backward_workspace_bytes(w.B, w.H, w.N)
        wsb = torch.empty(max(nbw, 16) // 4, device=dev, dtype=torch.float32)
        fa.fa_forward(q, k, v, o, lse, causal=True)
        ms_b = time_region(lambda: fa.fa_backward(q, k, v, o, dob, lse, dq, dk, dv, wsb, causal=True),
                           max(5, args.steps // 5), max(2, args.warmup // 2))
        bflops = 2.5 * flops
        out["backward"] = {
            "workload": w.describe() + " backward (dQ, dK, dV from O, dO, LSE)", "name": HEADLINE,
            "value": round(bflops / (ms_b * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_call": round(ms_b, 5), "flops_per_call": bflops,
            "flops_convention": "5 GEMMs (QK^T, dP, dV, dK, dQ) = 2.5 x forward, halved for causal",
            "roofline": {"bound": "mfma", "achieved": round(bflops / (ms_b * 1e-3) / 1e12, 2),
                         "peak": PEAK_BF16_TFLOPS,
                         "frac": round(bflops / (ms_b * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "unit": "TFLOP/s", "traffic": measured_traffic("backward/" + HEADLINE),
                         "kernels": "bwd_dq_kernel + bwd_dkdv_kernel"},
        }
        del dob, dq, dk, dv, wsb
        # ------------------------------------ V1 loop order (ablation), headline shape
        o1 = torch.empty_like(q)
        l1 = torch.empty_like(lse)
        nv1 = fa.fa_forward_v1_workspace_bytes(w.B, w.H, w.N, w.d)
        wv1 = torch.empty(max(nv1, 16) // 4, device=dev, dtype=torch.float32)
        ms_v1 = time_region(lambda: fa.fa_forward_v1(q, k, v, o1, l1, wv1, causal=True), 5, 1)
        ms_v2 = time_region(lambda: fa.fa_forward(q, k, v, o1, l1, causal=True), 20, 3)
        out["v1_ablation"] = {
            "workload": w.describe() + " in the V1 loop order (KV outer, Q inner, O/m/l via HBM)",
            "ms_per_call": round(ms_v1, 4), "tflops": round(flops / (ms_v1 * 1e-3) / 1e12, 2),
            "v2_ms_per_call": round(ms_v2, 5), "v1_over_v2_time": round(ms_v1 / ms_v2, 2),
            "workspace_bytes": nv1,
            "note": "one workgroup per (b, h) as in V1: 64 workgroups on 256 CUs",
        }
        del o1, l1, wv1

    if not (args.only_headline or args.only_decode or args.only_backward or args.only_long):
        # ------------------------------------------------------- row softmax
        wsm = SOFTMAX_WORKLOADS[SOFTMAX]
        xs = make_softmax_input(wsm, device=dev)
        ys = torch.empty_like(xs)
        ls = torch.empty(wsm.rows, device=dev, dtype=torch.float32)
        nb = fa.fa_softmax_workspace_bytes(wsm.rows, wsm.cols, xs.dtype)
        wss = torch.empty(max(nb, 16) // 4, device=dev, dtype=torch.float32)
        ms_s = time_region(lambda: fa.fa_softmax(xs, ys, ls, wss), max(5, args.steps // 5),
                           max(2, args.warmup // 2))
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
        del xs, ys, ls, wss
        torch.cuda.empty_cache()

    if not (args.only_headline or args.only_decode or args.only_softmax or args.only_backward):
        # ------------------------------------------------- other prefill shapes
        others = {}
        names = ("causal_bf16_b1h32_n8192_d128", "masked_bf16_b2h8_n4096_d128", "tiny_f32_b1h1_n256_d64")
        for name in (args.only_prefill,) if args.only_prefill else names:
            wo = WORKLOADS[name]
            oi = make_inputs(wo, device=dev)
            oo = torch.empty_like(oi["q"])
            ol = torch.empty(wo.B, wo.H, wo.N, device=dev, dtype=torch.float32)
            kl = oi["key_lens"]
            st = args.steps if args.only_long else max(5, args.steps // 5)
            ms_o = time_region(
                lambda: fa.fa_forward(oi["q"], oi["k"], oi["v"], oo, ol, causal=wo.causal,
                                      key_lens=kl), st, 3)
            nominal = prefill_flops(wo)
            rec = {"workload": wo.describe(), "ms_per_call": round(ms_o, 5),
                   "tflops_nominal": round(nominal / (ms_o * 1e-3) / 1e12, 2)}
            peak = PEAK_F32_TFLOPS if wo.dtype == "f32" else PEAK_BF16_TFLOPS
            if kl is not None:
                eff = prefill_flops(wo, kl.tolist())
                rec["key_lens"] = kl.tolist()
                rec["tflops_effective"] = round(eff / (ms_o * 1e-3) / 1e12, 2)
                rec["frac_effective"] = round(eff / (ms_o * 1e-3) / 1e12 / peak, 4)
            else:
                rec["frac"] = round(nominal / (ms_o * 1e-3) / 1e12 / peak, 4)
            rec["peak"] = peak
            if name == "causal_bf16_b1h32_n8192_d128" and not args.only_long:
                # backward of the same shape (5-GEMM convention, 2.5 x forward FLOPs)
                from attention_forward_online_amd.synth import randn_slices
                dg = randn_slices(tuple(oi["q"].shape), 1.0, torch.bfloat16, 0, wo.name, "do", dev)
                gq, gk, gv = (torch.empty_like(oi[t]) for t in ("q", "k", "v"))
                wsz = fa.fa_backward_workspace_bytes(wo.B, wo.H, wo.N)
                wsg = torch.empty(max(wsz, 16) // 4, device=dev, dtype=torch.float32)
                ms_g = time_region(lambda: fa.fa_backward(oi["q"], oi["k"], oi["v"], oo, dg, ol, gq, gk, gv,
                                                          wsg, causal=True), 3, 1)
                rec["backward_ms_per_call"] = round(ms_g, 4)
                rec["backward_tflops"] = round(2.5 * nominal / (ms_g * 1e-3) / 1e12, 2)
                del dg, gq, gk, gv, wsg
            others[name] = rec
            del oi, oo, ol
        out["workloads"] = others

    # ------------------------------------------------------- CPU oracle baseline
    if not args.no_cpu_baseline and not side_only:
        import oracle
        nthreads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
        qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
        t = time.perf_counter()
        O_ref, L_ref = oracle.attention(qh, kh, vh, scale=float(np.float32(w.scale)), causal=True,
                                        nthreads=nthreads)
        dt = time.perf_counter() - t
        out["cpu_baseline"] = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s",
                               "cores": nthreads, "kind": "oracle",
                               "sample": f"the whole headline workload ({HEADLINE}), one fp64 pass, "
                                         f"{dt:.2f} s wall"}
        # the oracle's outputs double as a full parity check of the timed run
        og = head_out[0].double().cpu().numpy()
        lg = head_out[1].double().cpu().numpy()
        out["parity"] = {"max_abs_O": float(np.abs(og - O_ref).max()),
                         "max_abs_LSE": float(np.abs(lg - L_ref).max()),
                         "tolerance": {"O": 2e-2, "LSE": 1e-3}}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
