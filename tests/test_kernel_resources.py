"""The consumer kernels' register and LDS footprints, read from the
compiler's own resource report, agree with what the host assumes: every
consumer kernel keeps enough of every SIMD's register file, and of the
CU's LDS, free for a producer wave, and no consumer kernel spills."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "communication_gemm_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and
                                not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc needed")


def resource_report(src):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-x", "hip", "--cuda-device-only", "-c", os.path.join(CSRC, src),
           "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, check=True).stderr
    kernels, cur = {}, None
    for line in out.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark: \s*(.+?): (\d+)", line)
        if m and cur:
            kernels[cur][m.group(1).strip()] = int(m.group(2))
    return kernels


def align8(x):
    return (x + 7) // 8 * 8


@pytest.fixture(scope="module")
def reports():
    return resource_report("consumer.hip"), resource_report("producer.hip")


def shape_table():
    """(kind, id) -> (BM, BN, SB, NS, WM, WN) from the sources."""
    plan = open(os.path.join(CSRC, "plan.cpp")).read()
    cons = open(os.path.join(CSRC, "consumer.hip")).read()
    cfg = {int(i): tuple(int(x) for x in v) for i, *v in re.findall(
        r"struct Cfg<(\d+)> \{ static constexpr int BM = (\d+), BN = (\d+), SB = (\d+), "
        r"NS = (\d+), WM = (\d+), WN = (\d+);", cons)}
    tables = {}
    for kind, name in (("F16", "kF16Shapes"), ("BF16", "kF16Shapes"), ("I8", "kI8Shapes"),
                       ("FP8", "kFP8Shapes")):
        body = plan[plan.index(name):]
        body = body[:body.index("};")]
        for i, tm, tn, threads, _ in re.findall(
                r"\{(\d+), (\d+), (\d+), (\d+), (true|false)\}", body):
            bm, bn, sb, ns, wm, wn = cfg[int(i)]
            assert (bm, bn) == (int(tm), int(tn))
            assert int(threads) == 64 * wm * wn
            tables[(kind, int(i))] = (bm, bn, sb, ns, wm, wn)
    return tables


# configurations built with the path's "x" traits (one rolling operand set:
# 16 x 16 MFMA blocks for fp16, bf16 and int8, 32 x 32 for fp8)
BLOCK16_IDS = (15,)


def consumer_report(cons, kind, bm, bn, sb, ns, wm, wn):
    key = (f"consumer_kernelINS0_{len(kind)}{kind}ELi{bm}ELi{bn}ELi{sb}ELi{ns}E"
           f"Li{wm}ELi{wn}EEEv")
    name = [k for k in cons if key in k]
    assert len(name) == 1, (kind, key)
    return cons[name[0]]


def test_every_consumer_leaves_room_for_the_producer(reports):
    """The pipelined mode launches a consumer grid that fills every CU and
    then the producer: each CU must still hold a producer workgroup (one
    wave per SIMD) beside the consumer workgroups that fit on it."""
    cons, prod = reports
    pk = [v for k, v in prod.items() if "producer_kernel" in k][0]
    prod_regs = align8(pk["VGPRs"]) + align8(pk.get("AGPRs", 0))
    prod_lds = pk.get("LDS Size [bytes/block]", 0)
    assert pk.get("ScratchSize [bytes/lane]", 0) == 0
    table = shape_table()
    assert len(table) == 54
    for (kind, i), (bm, bn, sb, ns, wm, wn) in table.items():
        r = consumer_report(cons, kind + ("x" if i in BLOCK16_IDS else ""),
                            bm, bn, sb, ns, wm, wn)
        regs = align8(r["VGPRs"]) + align8(r["AGPRs"])
        per_simd = wm * wn // 4          # waves of one workgroup on each SIMD
        # consumer workgroups on a CU: bounded by registers and by the LDS
        # ring (ns stages of (bm + bn) x sb bytes)
        lds = ns * sb * (bm + bn) + r.get("LDS Size [bytes/block]", 0)
        wgs = min(512 // (regs * per_simd), 163840 // lds, 8 // per_simd)
        assert wgs >= 1, (kind, i)
        waves = wgs * per_simd
        assert 512 - waves * regs >= prod_regs, (kind, i, regs, prod_regs)
        assert 163840 - wgs * lds >= prod_lds, (kind, i, lds)
        assert waves + 1 <= 8, (kind, i)


def test_no_consumer_kernel_spills(reports):
    cons, _ = reports
    for k, r in cons.items():
        assert r.get("ScratchSize [bytes/lane]", 0) == 0, k
        assert r.get("VGPRs Spill", 0) == 0, k
