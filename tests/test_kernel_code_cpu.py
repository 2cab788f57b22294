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
* Wait states of the direct-to-LDS loads: their inline assembly sits outside
  the compiler's hazard recognizer, so the code must keep the distances that
  the hardware does not check itself: five instructions between a VALU
  write of an SGPR (v_readfirstlane, v_readlane, v_cmp ...) and a load that
  reads it as its base, and one between writing M0 and the load.
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
    # a kernel's whole body, up to its end label (an early exit puts an
    # s_endpgm ahead of the main loop)
    for m in re.finditer(r"^(_ZN2sm3nsg9k_gemm_nsILi(\d)EEEvNS0_4ArgsE):[^\n]*\n(.*?)^\.Lfunc_end",
                         text, re.S | re.M):
        kernels[int(m.group(2))] = m.group(3)
    assert all("v_mfma" in body for body in kernels.values())
    assert set(kernels) == {0, 1, 2}, sorted(kernels)
    return text, kernels


def test_gemm_ns_kernels_use_no_scratch(gemm_ns_asm):
    text, _ = gemm_ns_asm
    sizes = re.findall(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", text)
    assert len(sizes) >= 3
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


@pytest.mark.parametrize("role", [0, 1, 2], ids=["symmetric", "apply", "probe"])
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


def test_tile_walk_is_a_bijection(tmp_path):
    """The banded walk of a problem's 256 x 256 tiles (ns_tiles.hpp) visits
    every tile of the rectangle, or of the lower triangle, exactly once."""
    src = tmp_path / "walk.cpp"
    src.write_text(r'''
#include <cstdio>
#include <set>
#include <utility>
#include "ns_tiles.hpp"
int main() {
  int bad = 0;
  for (int sym = 0; sym < 2; ++sym)
    for (int tm = 1; tm <= 45; ++tm)
      for (int tn = 1; tn <= 45; ++tn) {
        if (sym && tn != tm) continue;
        const int total = sym ? tm * (tm + 1) / 2 : tm * tn;
        std::set<std::pair<int, int>> seen;
        for (int u = 0; u < total; ++u) {
          int a = -1, b = -1;
          sm::ns_tile_coords(u, tm, tn, sym, &a, &b);
          if (a < 0 || a >= tm || b < 0 || b >= tn || (sym && b > a)) ++bad;
          seen.insert({a, b});
        }
        if ((int)seen.size() != total) ++bad;
      }
  std::printf("%d\n", bad);
  return bad != 0;
}
''')
    exe = tmp_path / "walk"
    subprocess.run(["g++", "-std=c++17", f"-I{build_lib.CSRC}", str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "0", out.stdout


def _sgprs(spec: str):
    """SGPR numbers named by an operand such as s7 or s[40:41]."""
    m = re.fullmatch(r"s(\d+)", spec)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", spec)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def lds_dma_hazards(body: str):
    """Direct-to-LDS loads that read an SGPR a VALU instruction wrote within
    the five instructions before (wait states counted as s_nop's argument +
    1), or that follow an M0 write with no wait state between."""
    insts = []
    for line in body.splitlines():
        t = line.split(";")[0].strip()
        if not t or t.endswith(":") or t.startswith("."):
            continue
        insts.append(t)
    bad = []
    for n, t in enumerate(insts):
        if not t.startswith("global_load_lds"):
            continue
        ops = [o.strip() for o in t.split(None, 1)[1].split(",")]
        base = _sgprs(ops[1]) if len(ops) > 1 else set()
        dist = 0
        for back in range(n - 1, -1, -1):
            u = insts[back]
            if u.startswith("s_nop"):
                dist += int(u.split()[1], 0) + 1
                continue
            if back == n - 1 and re.match(r"s_mov_b32 m0,", u):
                bad.append((n, "M0 written just before", t))
            if u.startswith("v_"):
                dst = u.split(None, 1)[1].split(",")[0].strip() if " " in u else ""
                if _sgprs(dst) & base and dist < 5:
                    bad.append((n, u, t))
            dist += 1
            if dist >= 5:
                break
    return bad


@pytest.mark.parametrize("role", [0, 1, 2], ids=["symmetric", "apply", "probe"])
def test_lds_dma_wait_states(gemm_ns_asm, role):
    _, kernels = gemm_ns_asm
    assert "global_load_lds_dwordx4" in kernels[role]
    bad = lds_dma_hazards(kernels[role])
    assert not bad, bad[:5]


def test_lds_dma_scan_finds_the_hazards():
    """The scan itself, on hand-written fragments: a base written by a VALU
    instruction two instructions ahead, and M0 written with no wait state."""
    body = "\n".join([
        "\tv_readfirstlane_b32 s41, v7",
        "\ts_mov_b32 m0, s42",
        "\ts_nop 0",
        "\tglobal_load_lds_dwordx4 v62, s[40:41]",
        "\tv_readfirstlane_b32 s40, v7",
        "\ts_nop 4",
        "\ts_mov_b32 m0, s42",
        "\tglobal_load_lds_dwordx4 v61, s[40:41]",
    ])
    bad = lds_dma_hazards(body)
    assert [b[0] for b in bad] == [3, 7], bad
