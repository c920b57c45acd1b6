"""Properties of the compiled tiled GEMM kernels (CPU only: hipcc cross-compiles for gfx950).

The K loop keeps later stages' transfers in flight by waiting, at each step, only for the
stage it is about to read.  A compiler decision can silently undo that (a register spill
reloaded inside the loop, a conservative alias assumption between LDS stores and the
transfers in flight, a register move of a load still in flight): each shows up as
`s_waitcnt vmcnt(0)`, a wait for every transfer, and the kernel still computes the right
result, only slower.  These tests compile w4a4_gemm.hip to gfx950 assembly and check, for the
production instantiations of the three code formats, that no scratch memory is used and
that the K loop waits only for the expected counts; and that the rotate+quantize kernels of
the benchmarked group sizes use no scratch either; and that the MXFP4 kernel issues its
scale loads where its waits count them.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from rotation_w4a4_quantized_convrot_amd import build as B

# kernel (mangled-name fragment of quant_gemm_kernel<false, QB, false>) -> vmcnt values
# allowed inside its K loop: transfers per wave per stage (4), plus one scale load (MXFP4)
KERNELS = {
    "int4": ("big17quant_gemm_kernelILb0ELi4ELb0E", {4}),
    "int8": ("big17quant_gemm_kernelILb0ELi8ELb0E", {4}),
    "mxfp4": ("big17quant_gemm_kernelILb0ELi1ELb0E", {4, 5}),
}
# int4 rows of 8 (mod 16) bytes: 4-byte transfers, sixteen per wave per stage (this form
# spills one register around the K loop, so it has no place in the scratch test)
KERNELS_T8 = {"int4-4-byte": ("big17quant_gemm_kernelILb0ELi4ELb1E", {16})}


# rotate+quantize instantiations of the benchmarked workloads (bf16 input, int4 codes):
# g = 256 (attention projection) and g = 1024 (MLP down-projection, proj_out)
RQ_KERNELS = {"g256": "16rht_quant_kernelILi256EtLi16ELi4ELi16E",
              "g1024": "16rht_quant_kernelILi1024EtLi16ELi4ELi8E"}


def _assemble(tmp_path_factory, src):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("isa") / (src + ".s"))
    cmd = [hipcc, *B.HIPCC_FLAGS, "-I", B.INCLUDE, "-I", B.CSRC, "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def isa(tmp_path_factory):
    return _assemble(tmp_path_factory, "w4a4_gemm.hip")


@pytest.fixture(scope="module")
def rq_isa(tmp_path_factory):
    return _assemble(tmp_path_factory, "rht_quant.hip")


def _function(text: str, fragment: str):
    names = [n for n in re.findall(r"^(\S+):", text, re.M) if fragment in n and n.startswith("_Z")]
    assert len(names) == 1, (fragment, names)
    start = text.index(names[0] + ":")
    end = text.index(".Lfunc_end", start)
    body = text[start:end].splitlines()
    meta = text[end:end + 4000]
    return body, meta


def _largest_loop(body):
    """Lines of the longest backward branch (the K loop)."""
    labels = {l.split(":")[0]: n for n, l in enumerate(body) if re.match(r"^\.LBB\S+:", l)}
    best = (0, 0)
    for n, line in enumerate(body):
        m = re.search(r"s_cbranch_\w+\s+(\.LBB\S+)", line)
        if m and m.group(1) in labels and labels[m.group(1)] < n:
            if n - labels[m.group(1)] > best[1] - best[0]:
                best = (labels[m.group(1)], n)
    return body[best[0]:best[1] + 1]


@pytest.mark.parametrize("fmt", sorted(KERNELS))
def test_no_scratch(isa, fmt):
    _, meta = _function(isa, KERNELS[fmt][0])
    scratch = int(re.search(r"ScratchSize:\s*(\d+)", meta).group(1))
    assert scratch == 0, f"{fmt}: {scratch} bytes of scratch per lane"


@pytest.mark.parametrize("fmt", sorted(KERNELS) + sorted(KERNELS_T8))
def test_k_loop_waits_for_one_stage(isa, fmt):
    frag, allowed = {**KERNELS, **KERNELS_T8}[fmt]
    body, _ = _function(isa, frag)
    loop = _largest_loop(body)
    assert sum("v_mfma" in l for l in loop) >= 64, f"{fmt}: the K loop was not found"
    waits = [int(w) for w in re.findall(r"s_waitcnt vmcnt\((\d+)\)", "\n".join(loop))]
    assert waits, f"{fmt}: no vmcnt wait in the K loop"
    assert set(waits) <= allowed, f"{fmt}: K-loop vmcnt waits {sorted(set(waits))}"
    assert all("scratch_" not in l for l in loop)


@pytest.mark.parametrize("which", sorted(RQ_KERNELS))
def test_rotate_quantize_no_scratch(rq_isa, which):
    _, meta = _function(rq_isa, RQ_KERNELS[which])
    scratch = int(re.search(r"ScratchSize:\s*(\d+)", meta).group(1))
    assert scratch == 0, f"rotate+quantize {which}: {scratch} bytes of scratch per lane"


def test_mxfp4_scale_loads_between_stages(isa):
    """The MXFP4 K loop's waits count each 16-byte scale load as issued after a whole stage's
    transfers; a scale load moved in among a stage's transfers would let a step read a
    stage before its last transfer landed.  Between two barriers the loop issues one
    stage's four transfers, then at most one scale load; the prologue issues the first
    scale load before stage 0 and the second between stages 1 and 2."""
    body, _ = _function(isa, KERNELS["mxfp4"][0])
    seq = []
    for line in body:
        t = line.strip()
        if t.startswith("buffer_load_dwordx4") and " lds" in t:
            seq.append("d")
        elif t.startswith("buffer_load_dwordx4 v["):
            seq.append("S")
        elif t.startswith("s_barrier"):
            seq.append("|")
    text = "".join(seq)
    first = text.index("|")
    assert text[:first] == "S" + "d" * 8 + "S" + "d" * 4, text[:first]
    for part in text[first + 1:].split("|"):
        assert re.fullmatch(r"(d{4}S?)?", part), f"transfers and scale loads between barriers: {part}"
