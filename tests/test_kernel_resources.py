"""Register budget of the kernels whose occupancy the design relies on (no
GPU needed: hipcc reports the resource use of the gfx950 code objects).

The paired matrix-core products (QKV with RoPE, gate/up with SiLU) run 8-wave
workgroups; at most 128 VGPRs per lane and no scratch lets two of them share
a CU, which the verify's gate/up product depends on for its speed."""
import os
import re
import subprocess

import pytest

from layer_speculative_decoding_amd import build

CSRC = os.path.join(os.path.dirname(build.__file__), "csrc")


def _resources(src):
    cmd = [build.hipcc(), *[f for f in build.FLAGS if f not in ("-shared", "-fPIC")], "--cuda-device-only", "-c",
           "-Rpass-analysis=kernel-resource-usage", os.path.join(CSRC, src), "-o", os.devnull]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    out, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        m = re.search(r"remark: \s*([A-Za-z ]+?)(?: \[bytes/lane\])?: (\d+)", line)
        if cur and m:
            out[cur][m.group(1).strip()] = int(m.group(2))
    return out


def _assembly(src):
    cmd = [build.hipcc(), *[f for f in build.FLAGS if f not in ("-shared", "-fPIC")], "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stdout


def test_paired_matrix_core_products_fit_two_workgroups_per_cu():
    """At most 128 VGPRs (two 8-wave workgroups per CU).  The float32
    activation operand (two bfloat16 pieces per element) costs the paired
    products a few registers, which the compiler spills once per unit, outside
    the weight-streaming loop: no scratch access may sit between the first and
    the last matrix instruction."""
    res = _resources("gemm_mfma.hip")
    # k_gemm_mfma<1, EPI, 8, ...> for EPI 1 (QKV + RoPE) and 2 (SiLU gate/up)
    names = [n for n in res if re.search(r"k_gemm_mfmaILi1ELi[12]ELi8E", n)]
    assert len(names) == 2, sorted(res)
    asm = _assembly("gemm_mfma.hip")
    for n in names:
        assert res[n]["VGPRs"] + res[n].get("AGPRs", 0) <= 128, (n, res[n])
        assert res[n]["ScratchSize"] <= 32, (n, res[n])
        i = asm.index(n + ":")
        body = asm[i:asm.index(".Lfunc_end", i)].splitlines()
        mf = [j for j, l in enumerate(body) if "v_mfma" in l]
        assert mf, n
        inner = [l for l in body[mf[0]:mf[-1]] if "scratch_" in l]
        assert not inner, (n, inner[:4])
