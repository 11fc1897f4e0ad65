"""Static check of the library's own gfx950 assembly (CPU; needs hipcc, not a GPU).

MFMA instructions read every lane's operands whatever EXEC says.  An MFMA placed inside
a lane-divergent block (one the compiler entered by masking EXEC) therefore reads the
stale registers of the masked-off lanes: their scale operands, or values computed only
by the active lanes.  The kernels are written so that every MFMA sits on a wave-uniform
path; the compiler is free to sink an instruction into a branch when its result is
only used there, so this test compiles every source that holds MFMAs to assembly and
fails if an MFMA appears between an EXEC-masking instruction and the point where EXEC
is restored.
"""
import concurrent.futures
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from gemm_chains_amd import build

MFMA_SOURCES = ["attn.hip", "gemm_bf16.hip", "gemm_bf16_silu.hip", "gemm_e4m3.hip", "gemm_e4m3_silu.hip",
                "gemm_mxfp4.hip", "gemm_mxfp4_silu.hip"]


def _asm(src, out_dir):
    out = os.path.join(out_dir, src + ".s")
    cmd = [build._hipcc()] + [f for f in build.FLAGS if f != "-fPIC"] + [
        "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


def _masked_mfma(asm_text):
    """Names of kernels with an MFMA inside an EXEC-masked region."""
    bad = []
    for m in re.finditer(r"^(_Z[^:\s]+):", asm_text, re.M):
        end = asm_text.find(".Lfunc_end", m.end())
        body = asm_text[m.end():end]
        if "v_mfma" not in body:
            continue
        masked = False
        for line in body.splitlines():
            ins = line.split(";")[0].strip()
            if "saveexec" in ins or ins.startswith("s_and_b64 exec") or (
                    ins.startswith("s_mov_b64 exec,") and "-1" not in ins):
                masked = True
            elif ins.startswith(("s_or_b64 exec", "s_mov_b64 exec, -1", "s_barrier", "s_endpgm")):
                masked = False
            if masked and ins.startswith("v_mfma"):
                bad.append(m.group(1))
                break
    return bad


def test_masked_region_detector_flags_an_mfma_under_a_lane_mask():
    text = """_Zk1:
  s_and_saveexec_b64 s[0:1], vcc
  v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], 0
  s_or_b64 exec, exec, s[0:1]
.Lfunc_end0:
_Zk2:
  v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], 0
  s_and_saveexec_b64 s[0:1], vcc
  global_store_dwordx4 v[8:9], v[0:3], off
  s_or_b64 exec, exec, s[0:1]
.Lfunc_end1:
"""
    assert _masked_mfma(text) == ["_Zk1"]


@pytest.mark.slow
def test_no_mfma_on_a_lane_masked_path():
    try:
        build._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    tmp = tempfile.mkdtemp(prefix="frt_isa_")
    try:
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(MFMA_SOURCES))) as ex:
            outs = list(ex.map(lambda s: _asm(s, tmp), MFMA_SOURCES))
        n_kernels, bad = 0, []
        for path in outs:
            text = open(path).read()
            n_kernels += len(re.findall(r"^_Z[^:\s]+:", text, re.M))
            bad += _masked_mfma(text)
        assert n_kernels > 100
        assert not bad, f"MFMA inside an EXEC-masked region: {bad[:5]}"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
