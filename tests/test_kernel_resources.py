"""Register and scratch budget of every gfx950 kernel (no GPU: hipcc's resource
report for the device code, compiled here with the library's own flags).

No kernel may use scratch memory (per-lane stack: register spills or private
arrays the compiler could not keep in registers), and the kernels whose
occupancy the measured rates rest on must keep it: the bf16 prefill at d = 64
and the bf16 backward's dQ kernel at three waves per SIMD (at most 168 VGPRs of
the 512 a SIMD lane holds), the bf16 prefill at d = 128, the d = 64 dK/dV
kernel and the d = 128 paired dK/dV kernel (one 8-wave workgroup per CU) at
two."""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess

import pytest

from attention_forward_online_amd import build as B

REPORT = "-Rpass-analysis=kernel-resource-usage"
FIELD = re.compile(r"remark: +([A-Za-z][A-Za-z ]*?)(?: \[[^\]]*\])?: (\S+) \[" + re.escape(REPORT) + r"\]")


def _report(src: str, tmp: str) -> dict[str, dict[str, str]]:
    cmd = [B._hipcc(), *B.HIPCC_FLAGS, *B.FILE_FLAGS.get(src, []), "--cuda-device-only", "-c",
           os.path.join(B.CSRC, src), "-o", os.path.join(tmp, src + ".o"), REPORT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels: dict[str, dict[str, str]] = {}
    cur = None
    for line in r.stderr.splitlines():
        m = FIELD.search(line)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = kernels.setdefault(val, {})
        elif cur is not None:
            cur[key] = val
    return kernels


@pytest.fixture(scope="module")
def reports(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("res"))
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        parts = list(ex.map(lambda s: _report(s, tmp), B.SOURCES))
    return {src: p for src, p in zip(B.SOURCES, parts)}


def test_every_source_reports_its_kernels(reports):
    for src, kernels in reports.items():
        if src == "fa_api.hip":
            continue
        assert kernels, f"{src}: no kernel in the resource report"
        for name, f in kernels.items():
            assert {"VGPRs", "ScratchSize", "Occupancy"} <= f.keys(), (src, name, f)


def test_no_kernel_uses_scratch(reports):
    bad = [(src, name, f["ScratchSize"], f.get("VGPRs Spill"), f.get("SGPRs Spill"))
           for src, kernels in reports.items() for name, f in kernels.items()
           if f["ScratchSize"] != "0" or f.get("VGPRs Spill", "0") != "0"]
    assert not bad, f"kernels with scratch or spilled registers: {bad}"


# (source, demangled-name pattern, minimum waves per SIMD)
OCCUPANCY = [
    ("fa_fwd_bf16.hip", r"fwd_bf16_kernelILi64ELb[01]ELi1E", 3),
    ("fa_fwd_bf16.hip", r"fwd_bf16_kernelILi128ELb[01]ELi1E", 2),
    ("fa_bwd_bf16.hip", r"bwd_dq_kernelILi64ELb[01]ELi1E", 3),
    ("fa_bwd_bf16.hip", r"bwd_dq_kernelILi128ELb[01]ELi1E", 2),
    ("fa_bwd_bf16.hip", r"bwd_dkdv_kernelILi64ELb[01]ELi1E", 2),
    ("fa_bwd_bf16.hip", r"bwd_dkdv_paired_kernelILi128ELb[01]E", 2),
]


@pytest.mark.parametrize("src,pattern,waves", OCCUPANCY)
def test_hot_kernels_keep_their_occupancy(reports, src, pattern, waves):
    hits = {n: f for n, f in reports[src].items() if re.search(pattern, n)}
    assert hits, f"no kernel of {src} matches {pattern}"
    for name, f in hits.items():
        assert int(f["Occupancy"]) >= waves, f"{name}: {f['Occupancy']} waves/SIMD, {f['VGPRs']} VGPRs"
