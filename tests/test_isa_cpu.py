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


# ---------------------------------------------------------------------------------------
# Latency-bound kernels pay one memory round trip per batch of loads they wait on.  The
# single-round kernels on the chain are written so that every load of a workgroup goes out
# before the first wait on loads, and so that no kernel argument the loads or the records
# need arrives in a second, dependent round trip.  The compiler is free to sink a load
# toward its use (it did: the attention chunk kernel's V loads went out after the first
# Q.K^T MFMAs had waited for Q and K), so these checks read the assembly.

def _kernels(asm_text):
    for m in re.finditer(r"^(_Z[^:\s]+):", asm_text, re.M):
        end = asm_text.find(".Lfunc_end", m.end())
        yield m.group(1), asm_text[m.end():end]


def _loads_after_a_wait(body):
    """Vector-memory loads of 8 or 16 bytes per lane issued after the first wait on earlier
    vector loads.  (Single-dword loads are left out: they are the producers' read-ahead
    touches, whose later rounds wait on the earlier ones by design.)"""
    waited, late = False, 0
    for line in body.splitlines():
        ins = line.split(";")[0].strip()
        if re.match(r"(global|buffer)_load_dwordx[24]\b", ins) and waited:
            late += 1
        if ins.startswith("s_waitcnt") and "vmcnt" in ins:
            waited = True
    return late


_SMEM_BYTES = {"s_load_dword": 4, "s_load_dwordx2": 8, "s_load_dwordx4": 16, "s_load_dwordx8": 32,
               "s_load_dwordx16": 64}


def _late_argument_lines(body):
    """Kernel-argument cache lines (64 bytes) requested as a second dependent miss after
    the first vector load: first requested after a wait on vector loads, or after a wait
    that covered earlier first requests of lines (each such wait is a scalar round trip;
    a wait on lines already cached is not)."""
    fetched, vmem, missed, outstanding, late = set(), False, False, False, []
    for line in body.splitlines():
        ins = line.split(";")[0].strip()
        m = re.match(r"(s_load_dword\w*)\s+s\[?[\d:]+\]?,\s*s\[0:1\],\s*(0x[0-9a-f]+|\d+)", ins)
        if m:
            off = int(m.group(2), 0)
            lines = {off // 64, (off + _SMEM_BYTES[m.group(1)] - 1) // 64}
            if lines - fetched:
                if missed:
                    late.append(off)
                if vmem:
                    outstanding = True
            fetched |= lines
        if re.match(r"(global|buffer)_load", ins):
            vmem = True
        if vmem and ins.startswith("s_waitcnt") and ("vmcnt" in ins or outstanding):
            missed = True
    return late


def test_load_order_detectors():
    text = """_Zk1:
  s_load_dwordx2 s[4:5], s[0:1], 0x0
  s_waitcnt lgkmcnt(0)
  global_load_dwordx4 v[0:3], v4, s[4:5]
  s_waitcnt vmcnt(0)
  global_load_dword v12, v4, s[4:5]
  global_load_dwordx4 v[8:11], v4, s[4:5]
  s_load_dwordx2 s[6:7], s[0:1], 0x88
  s_load_dword s8, s[0:1], 0x8
.Lfunc_end0:
_Zk2:
  s_load_dwordx2 s[4:5], s[0:1], 0x0
  s_waitcnt lgkmcnt(0)
  global_load_dwordx4 v[0:3], v4, s[4:5]
  s_load_dword s9, s[0:1], 0x8
  s_waitcnt lgkmcnt(0)
  s_load_dwordx2 s[6:7], s[0:1], 0x88
  s_waitcnt lgkmcnt(0)
  global_load_dwordx4 v[8:11], v4, s[6:7]
.Lfunc_end1:
_Zk3:
  s_load_dwordx2 s[4:5], s[0:1], 0x80
  s_waitcnt lgkmcnt(0)
  global_load_dwordx4 v[0:3], v4, s[4:5]
  s_load_dwordx2 s[6:7], s[0:1], 0x0
  s_waitcnt lgkmcnt(0)
  s_load_dword s8, s[0:1], 0x110
  s_waitcnt lgkmcnt(0)
.Lfunc_end2:
"""
    (n1, b1), (n2, b2), (n3, b3) = list(_kernels(text))
    assert (n1, n2, n3) == ("_Zk1", "_Zk2", "_Zk3")
    assert _loads_after_a_wait(b1) == 1 and _loads_after_a_wait(b2) == 0
    assert _late_argument_lines(b1) == [0x88]  # first requested after a wait on the loads
    assert _late_argument_lines(b2) == []      # behind a wait on a cached line only
    assert _late_argument_lines(b3) == [0x110]  # a second dependent miss


# (family pattern, check): kernels that must issue every load before the first wait on
# loads, and (second list) fetch every kernel-argument line before their first load
_NO_LATE_LOADS = [
    r"attn_chunk_kernelILi\d+ELb0E",                        # one 32-key block per wave
    r"attn_merge_oproj_kernel",
    # producers with 0-8 split partials and K <= 1024 (with 16 partials and no operand
    # output the compiler interleaves sums with the loads; the chain never launches it)
    r"rnq_kernelILi[0-8]ELi1E",
    r"skinny_gemm_kernelILi1E(Li\d+E){4}Li2ELb",           # bf16 weights, plain single round
    r"skinny_gemm_kernelILi2E(Li\d+E){4}Li1ELb",           # e4m3 weights, single round, scales
]
_NO_LATE_ARGUMENTS = [
    r"attn_merge_oproj_kernel",
    r"skinny_gemm_kernelILi[12]E(Li\d+E){3}Li4ELi[12]ELb",  # QKV scatter epilogue
]


@pytest.mark.slow
def test_chain_kernels_issue_their_loads_in_one_batch():
    try:
        build._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    tmp = tempfile.mkdtemp(prefix="frt_isa_")
    srcs = MFMA_SOURCES + ["rnq.hip"]
    try:
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            outs = list(ex.map(lambda s: _asm(s, tmp), srcs))
        seen = {p: 0 for p in _NO_LATE_LOADS + _NO_LATE_ARGUMENTS}
        bad_loads, bad_args = [], []
        for path in outs:
            for name, body in _kernels(open(path).read()):
                for pat in _NO_LATE_LOADS:
                    if re.search(pat, name):
                        seen[pat] += 1
                        if _loads_after_a_wait(body):
                            bad_loads.append(name)
                for pat in _NO_LATE_ARGUMENTS:
                    if re.search(pat, name):
                        seen[pat] += 1
                        if _late_argument_lines(body):
                            bad_args.append(name)
        assert all(seen.values()), f"no kernel matched: {[p for p, n in seen.items() if not n]}"
        assert not bad_loads, f"loads issued after a wait on loads: {sorted(set(bad_loads))[:5]}"
        assert not bad_args, f"kernel-argument lines first fetched after the loads: {sorted(set(bad_args))[:5]}"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
