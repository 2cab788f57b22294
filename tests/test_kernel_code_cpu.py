"""Properties of the generated gfx950 code of the NS GEMM kernels, checked on
the CPU from hipcc's assembly output (no GPU needed).

* No scratch: the kernels keep everything in registers and LDS, and read
  their argument block in place (a private copy of it, or a spill, would
  put a scratch access, and a wait for every load in flight, in the loop).
* No MFMA under a lane mask without a skip: every branch in these kernels is
  uniform, but the compiler cannot tell, so it masks lanes; when it leaves
  out the `s_cbranch_execz` around a short masked block, an MFMA there still
  accumulates with no lane active (a both-sided identity fold went wrong
  that way).  The scan follows the straight-line order of the assembly: a
  region opened by a mask instruction counts as guarded once a conditional
  branch on the mask follows it.
"""
import os
import re
import subprocess

import pytest

from matrix_aware_optimizer_momentum_amd import build_lib

KERNEL_SRC = os.path.join(build_lib.CSRC, "k_gemm_ns.hip")


@pytest.fixture(scope="module")
def gemm_ns_asm(tmp_path_factory):
    try:
        hipcc = build_lib._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "k_gemm_ns.s"
    cmd = [hipcc, *build_lib.HIP_FLAGS, "--cuda-device-only", "-S", KERNEL_SRC, "-o", str(out)]
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert proc.returncode == 0, proc.stdout[-2000:]
    text = out.read_text()
    kernels = {}
    for m in re.finditer(r"^(_ZN2sm3nsg9k_gemm_nsILi(\d)EEEvNS0_4ArgsE):[^\n]*\n(.*?)^\s*s_endpgm",
                         text, re.S | re.M):
        kernels[int(m.group(2))] = m.group(3)
    assert set(kernels) == {0, 1}, sorted(kernels)
    return text, kernels


def test_gemm_ns_kernels_use_no_scratch(gemm_ns_asm):
    text, _ = gemm_ns_asm
    sizes = re.findall(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", text)
    assert len(sizes) >= 2
    assert all(int(v) == 0 for v in sizes), sizes


def masked_mfmas_without_skip(body: str):
    masked = guarded = False
    bad = []
    for n, line in enumerate(body.splitlines()):
        t = line.strip()
        if re.match(r"s_(and|andn2|or|xor)_saveexec_b64|s_(and|andn2|xor)_b64 exec,", t):
            masked, guarded = True, False
        elif t.startswith(("s_cbranch_execz", "s_cbranch_execnz")):
            guarded = True
        elif re.match(r"s_(or|mov)_b64 exec,", t):
            masked = False
        elif t.startswith("v_mfma") and masked and not guarded:
            bad.append((n, t))
    return bad


@pytest.mark.parametrize("role", [0, 1], ids=["symmetric", "apply"])
def test_no_mfma_under_a_lane_mask_without_skip(gemm_ns_asm, role):
    _, kernels = gemm_ns_asm
    bad = masked_mfmas_without_skip(kernels[role])
    assert not bad, bad[:5]


def test_scan_finds_a_masked_mfma():
    """The scan itself, on a hand-written fragment of the pattern it looks for."""
    body = "\n".join([
        "\ts_and_saveexec_b64 s[14:15], s[30:31]",
        "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[2:5], a[0:15]",
        "\ts_or_b64 exec, exec, s[14:15]",
        "\ts_and_saveexec_b64 s[14:15], s[16:17]",
        "\ts_cbranch_execz .LBB0_2",
        "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]",
        "\ts_or_b64 exec, exec, s[14:15]",
    ])
    bad = masked_mfmas_without_skip(body)
    assert [n for n, _ in bad] == [1]
