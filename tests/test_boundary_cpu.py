"""C-ABI boundary checks that need no GPU.

The library must load, export every function include/sm.h declares, agree
with the Python binding on struct layouts, size its workspaces, and reject
bad arguments on the host before any HIP call.
"""
import ctypes
import os
import re
import subprocess

import pytest

from matrix_aware_optimizer_momentum_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_path_calls():
    names = declared_functions()
    for n in ("sm_step", "sm_ns_polar", "sm_gram_ns_cached", "sm_sign_pack", "sm_vote_update"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (sm_[a-z0-9_]+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    # the binding declares exactly the header's functions
    assert sorted(B.SIGNATURES) == declared_functions()


def test_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "sm.h"\n'
        "int main(void){printf(\"%zu %zu %zu %zu %zu %zu %zu %zu %zu\\n\", sizeof(sm_ns_params),"
        " sizeof(sm_matrix), sizeof(sm_config), offsetof(sm_config, ns),"
        " offsetof(sm_config, gamma), offsetof(sm_matrix, w), offsetof(sm_matrix, cache_state),"
        " offsetof(sm_config, encoding), offsetof(sm_config, vote_polar));"
        "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", "-I/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    want = [ctypes.sizeof(B.NSParams), ctypes.sizeof(B.Matrix), ctypes.sizeof(B.Config),
            B.Config.ns.offset, B.Config.gamma.offset, B.Matrix.w.offset,
            B.Matrix.cache_state.offset, B.Config.encoding.offset, B.Config.vote_polar.offset]
    assert vals == want


def test_status_strings_and_version():
    lib = B.lib()
    assert lib.sm_version() >= 1
    for code in range(7):
        assert lib.sm_status_string(code).decode().startswith(B.STATUS_NAMES[code])
    assert lib.sm_last_hip_error() == 0


def _ws(fn, *args):
    out = ctypes.c_size_t(0)
    code = fn(*args, ctypes.byref(out))
    return code, out.value


def test_workspace_queries():
    lib = B.lib()
    c1, a = _ws(lib.sm_ns_polar_ws, B.BF16, 5, 768, 3072)
    c2, b = _ws(lib.sm_ns_polar_ws, B.BF16, 10, 768, 3072)
    assert c1 == c2 == 0 and 0 < a < b
    # at least one iterate buffer plus the two r x r buffers
    assert a >= 5 * 768 * 3072 * 2 + 2 * 5 * 768 * 768 * 2
    c3, g = _ws(lib.sm_gram_ns_cached_ws, B.F32, 3, 100, 40)
    assert c3 == 0 and g >= 5 * 3 * 40 * 40 * 4
    assert _ws(lib.sm_ns_polar_ws, 7, 1, 4, 4)[0] == 3           # bad dtype
    assert _ws(lib.sm_ns_polar_ws, B.F32, 0, 4, 4)[0] == 2       # bad batch
    assert _ws(lib.sm_ns_polar_ws, B.F32, 1, 65536, 65536)[0] == 2


def _cfg(**kw):
    from matrix_aware_optimizer_momentum_amd.api import StepConfig
    return StepConfig(**kw).c_struct()


def test_step_ws_and_config_validation():
    import torch
    lib = B.lib()
    mats = (B.Matrix * 2)()
    mats[0] = B.Matrix(64, 147, None, None, None, None, None)
    mats[1] = B.Matrix(147, 64, None, None, None, None, None)
    ok = _cfg(M=4)
    code, nbytes = _ws(lib.sm_step_ws, ctypes.byref(ok), mats, 2)
    assert code == 0 and nbytes > 0
    for bad, want in ((dict(M=0), 5), (dict(M=65), 5), (dict(algo=7), 1),
                      (dict(update=1, M=1), 5),            # Sign-Muon with polar update
                      (dict(algo=1, update=1, M=2), 5),    # polar needs one worker
                      (dict(period=-1), 1), (dict(lr=float("nan")), 1),
                      (dict(cache_mode=3), 1), (dict(encoding=2), 1), (dict(vote_polar=2), 1)):
        c = _cfg(**bad)
        assert _ws(lib.sm_step_ws, ctypes.byref(c), mats, 2)[0] == want, bad
    c = _cfg(wdt=torch.float32)
    c.mdt = 9
    assert _ws(lib.sm_step_ws, ctypes.byref(c), mats, 2)[0] == 3
    c = _cfg()
    c.ns.iters = 0
    assert _ws(lib.sm_step_ws, ctypes.byref(c), mats, 2)[0] == 1


def test_host_validation_rejects_before_any_gpu_call():
    lib = B.lib()
    p = B.NSParams(5, 1.5, -0.5, 0.0, 1e-7)
    # null pointers
    assert lib.sm_ns_polar(None, None, B.F32, 1, 4, 4, 1, ctypes.byref(p), None, 0, None) == 1
    assert lib.sm_sign_pack(None, B.F32, 10, None, None) == 1
    assert lib.sm_sign_pack(None, B.F32, -1, None, None) == 2
    assert lib.sm_sign_pack(None, B.F32, 0, None, None) == 0      # empty: no-op
    assert lib.sm_vote_update(None, 0, 1, 64, None, B.F32, 1e-3, None, None) == 5
    assert lib.sm_vote_update(None, 65, 1, 64, None, B.F32, 1e-3, None, None) == 5
    assert lib.sm_vote_update(None, 3, 1, 64, None, 5, 1e-3, None, None) == 3
    # misaligned pointers (never dereferenced: rejected on the host)
    assert lib.sm_sign_pack(ctypes.c_void_p(0x1001), B.F32, 10, ctypes.c_void_p(0x2000),
                            None) == 1
    assert lib.sm_sign_pack(ctypes.c_void_p(0x1000), B.F32, 10, ctypes.c_void_p(0x2004),
                            None) == 1
    assert lib.sm_vote_update(ctypes.c_void_p(0x1000), 3, 1, 64, ctypes.c_void_p(0x2008),
                              B.F32, 1e-3, None, None) == 1
    # words_stride too small for the count
    assert lib.sm_vote_update(ctypes.c_void_p(0x1000), 3, 1, 65, ctypes.c_void_p(0x2000),
                              B.F32, 1e-3, None, None) == 1
    # int8 encoding, the vote as a matrix, the dense update
    assert lib.sm_sign_int8(None, B.F32, 10, None, None) == 1
    assert lib.sm_sign_int8(None, B.F32, -1, None, None) == 2
    assert lib.sm_sign_int8(None, B.F32, 0, None, None) == 0
    assert lib.sm_sign_int8(ctypes.c_void_p(0x1002), B.F32, 10, ctypes.c_void_p(0x2000),
                            None) == 1
    assert lib.sm_sign_int8(ctypes.c_void_p(0x1000), B.F32, 10, ctypes.c_void_p(0x1010),
                            None) == 1                              # overlap
    assert lib.sm_vote_update_int8(None, 0, 10, 10, None, B.F32, 1e-3, None, None) == 5
    assert lib.sm_vote_update_int8(ctypes.c_void_p(0x1000), 3, 9, 10, ctypes.c_void_p(0x2000),
                                   B.F32, 1e-3, None, None) == 1    # stride < count
    assert lib.sm_vote_update_int8(ctypes.c_void_p(0x1000), 3, 10, 10, ctypes.c_void_p(0x2000),
                                   B.F32, float("inf"), None, None) == 1
    assert lib.sm_vote(ctypes.c_void_p(0x1000), 2, 3, 10, 10, ctypes.c_void_p(0x2000), B.F32,
                       None) == 1                                   # bad encoding
    assert lib.sm_vote(ctypes.c_void_p(0x1004), 0, 3, 1, 64, ctypes.c_void_p(0x2000), B.F32,
                       None) == 1                                   # misaligned bits
    assert lib.sm_vote(ctypes.c_void_p(0x1000), 0, 3, 1, 65, ctypes.c_void_p(0x2000), B.F32,
                       None) == 1                                   # stride too small
    assert lib.sm_vote(ctypes.c_void_p(0x1000), 1, 70, 100, 10, ctypes.c_void_p(0x2000), B.F32,
                       None) == 5
    assert lib.sm_polar_update(ctypes.c_void_p(0x1000), B.F32, ctypes.c_void_p(0x1000), B.F32,
                               10, 1e-3, None) == 1                 # aliasing
    assert lib.sm_polar_update(ctypes.c_void_p(0x1000), B.F32, ctypes.c_void_p(0x2000), 4,
                               10, 1e-3, None) == 3
    # aliasing input/output of NS
    assert lib.sm_ns_polar(ctypes.c_void_p(0x10000), ctypes.c_void_p(0x10000), B.F32, 1, 4, 4,
                           1, ctypes.byref(p), ctypes.c_void_p(0x100000), 1 << 20, None) == 1
    # workspace too small
    assert lib.sm_ns_polar(ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000), B.F32, 1, 4, 4,
                           1, ctypes.byref(p), ctypes.c_void_p(0x100000), 16, None) == 4
    # bad NS params
    bad = B.NSParams(0, 1.5, -0.5, 0.0, 1e-7)
    assert lib.sm_ns_polar(ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000), B.F32, 1, 4, 4,
                           1, ctypes.byref(bad), ctypes.c_void_p(0x100000), 1 << 20, None) == 1
    # gram: bad mode, null cache
    assert lib.sm_gram_ns_cached(ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000), None, None,
                                 None, None, B.F32, 1, 4, 4, 1, ctypes.byref(p), 1.0, 0, 1,
                                 ctypes.c_void_p(0x100000), 1 << 20, None) == 1
    assert lib.sm_last_hip_error() == 0


def test_step_rejects_bad_matrices():
    lib = B.lib()
    c = _cfg(M=2)
    mats = (B.Matrix * 1)()
    mats[0] = B.Matrix(8, 8, None, None, None, None, None)
    assert lib.sm_step(ctypes.byref(c), mats, 1, 1, ctypes.c_void_p(0x100000), 1 << 20, None,
                       None) == 1
    mats[0] = B.Matrix(0, 8, 0x1000, 0x2000, 0x3000, None, None)
    assert lib.sm_step(ctypes.byref(c), mats, 1, 1, ctypes.c_void_p(0x100000), 1 << 20, None,
                       None) == 2
    mats[0] = B.Matrix(8, 8, 0x1000, 0x2000, 0x3000, None, None)
    assert lib.sm_step(ctypes.byref(c), mats, 1, 0, ctypes.c_void_p(0x100000), 1 << 20, None,
                       None) == 1     # t must be >= 1
    cc = _cfg(algo=1, M=2)
    assert lib.sm_step(ctypes.byref(cc), mats, 1, 1, ctypes.c_void_p(0x100000), 1 << 20, None,
                       None) == 1     # CacheMuon needs q_cache / cache_state
    assert lib.sm_step(ctypes.byref(c), mats, 1, 1, ctypes.c_void_p(0x100000), 8, None,
                       None) == 4


def test_step_graph_rejects_on_the_host():
    lib = B.lib()
    c = _cfg(M=2)
    ws = ctypes.c_void_p(0x100000)
    mats = (B.Matrix * 1)()
    mats[0] = B.Matrix(8, 8, 0x1000, 0x2000, 0x3000, None, None)
    h = ctypes.c_void_p(0x1234)
    assert lib.sm_step_graph(ctypes.byref(c), mats, 1, 1, ws, 1 << 20, None, None) == 1
    assert lib.sm_step_graph(ctypes.byref(c), mats, 1, 0, ws, 1 << 20, None,
                             ctypes.byref(h)) == 1      # t must be >= 1
    assert h.value is None                              # *out cleared on error
    cc = _cfg(algo=1, M=2)                              # CacheMuon records t in its state
    mc = (B.Matrix * 1)()
    mc[0] = B.Matrix(8, 8, 0x1000, 0x2000, 0x3000, 0x4000, 0x5000)
    assert lib.sm_step_graph(ctypes.byref(cc), mc, 1, 1, ws, 1 << 20, None,
                             ctypes.byref(h)) == 5
    assert h.value is None
    assert lib.sm_graph_launch(None, None) == 1
    assert lib.sm_graph_destroy(None) == 0
    assert lib.sm_last_hip_error() == 0


def test_python_front_end_needs_gpu_tensors():
    import torch
    import matrix_aware_optimizer_momentum_amd as sm
    with pytest.raises(ValueError):
        sm.sign_pack(torch.zeros(10))


def test_gram_ns_cached_rejects_workspace_aliasing():
    """The workspace may not overlap x, d, Q, the cache state, err or the
    refresh flags (checked on the host; nothing is launched)."""
    lib = B.lib()
    p = B.NSParams(5, 1.5, -0.5, 0.0, 1e-7)
    need = ctypes.c_size_t(0)
    assert lib.sm_gram_ns_cached_ws(B.F32, 2, 64, 96, ctypes.byref(need)) == 0
    x, d, q, cs = 0x100000, 0x200000, 0x300000, 0x400000
    err, rf = 0x500000, 0x600000
    big = 1 << 24
    for ws in (x, d, q, cs, err, rf, q - 256 * 16):
        args = [ctypes.c_void_p(v) for v in (x, d, q, cs, err, rf)]
        assert lib.sm_gram_ns_cached(*args, B.F32, 2, 64, 96, 1, ctypes.byref(p), 1.0, 0, 1,
                                     ctypes.c_void_p(ws), max(need.value, big), None) == 1, hex(ws)
    # Q aliasing the input
    assert lib.sm_gram_ns_cached(ctypes.c_void_p(x), ctypes.c_void_p(d), ctypes.c_void_p(x),
                                 ctypes.c_void_p(cs), None, None, B.F32, 2, 64, 96, 1,
                                 ctypes.byref(p), 1.0, 0, 1, ctypes.c_void_p(0x10000000),
                                 need.value, None) == 1
    assert lib.sm_last_hip_error() == 0


def _cpu_mats(M=3, m=8, n=12, wdt=None, mdt=None, gdt=None, mom_shape=None):
    import torch
    from matrix_aware_optimizer_momentum_amd.api import MatrixBuffers
    f = torch.float32
    return [MatrixBuffers(w=torch.zeros(m, n, dtype=wdt or f),
                          mom=torch.zeros(*(mom_shape or (M, m, n)), dtype=mdt or f),
                          grad=torch.zeros(M, m, n, dtype=gdt or f))]


@pytest.mark.parametrize("kw,msg", [
    (dict(mdt="bf16"), "mom must be torch.float32"),
    (dict(gdt="bf16"), "grad must be torch.float32"),
    (dict(wdt="bf16"), "w must be torch.float32"),
    (dict(mom_shape=(2, 8, 12)), "mom must have shape"),
    (dict(mom_shape=(3, 12, 8)), "mom must have shape"),
])
def test_step_front_end_checks_shapes_and_dtypes(kw, msg):
    """A bf16 momentum with a float32 configuration (and the like) is refused
    before any pointer reaches the library."""
    import torch
    from matrix_aware_optimizer_momentum_amd.api import StepCall, StepConfig
    kw = {k: (torch.bfloat16 if v == "bf16" else v) for k, v in kw.items()}
    with pytest.raises(ValueError, match=msg):
        StepCall(StepConfig(M=3), _cpu_mats(**kw))


def test_step_front_end_checks_cache_buffers_and_diag():
    import torch
    from matrix_aware_optimizer_momentum_amd.api import StepCall, StepConfig
    mats = _cpu_mats(M=1)
    cfg = StepConfig(algo=B.CACHE_MUON, update=B.UPDATE_POLAR, M=1)
    with pytest.raises(ValueError, match="needs q_cache"):
        StepCall(cfg, mats)
    mats[0].q_cache = torch.zeros(1, 8, 8, dtype=torch.float64)
    mats[0].cache_state = torch.zeros(1, 2, dtype=torch.int32)
    with pytest.raises(ValueError, match="q_cache must be torch.float32"):
        StepCall(cfg, mats)
    mats[0].q_cache = torch.zeros(1, 12, 12)
    with pytest.raises(ValueError, match="q_cache must have shape"):
        StepCall(cfg, mats)
    mats[0].q_cache = torch.zeros(1, 8, 8)
    mats[0].cache_state = torch.zeros(1, 2, dtype=torch.int64)
    with pytest.raises(ValueError, match="cache_state must be torch.int32"):
        StepCall(cfg, mats)
    with pytest.raises(ValueError, match="diag must hold at least 6"):
        StepCall(StepConfig(M=3), _cpu_mats(), diag=torch.zeros(5))
    with pytest.raises(ValueError, match="at least one matrix"):
        StepCall(StepConfig(M=3), [])


def test_noalloc_entry_point_rejects_oversized_problems_on_the_host():
    """The scratch limit is checked before any HIP call."""
    lib = B.lib()
    p = B.NSParams(5, 1.5, -0.5, 0.0, 1e-7)
    need = ctypes.c_size_t(0)
    assert lib.sm_ns_polar_ws(B.BF16, 4, 4096, 4096, ctypes.byref(need)) == 0
    assert need.value > B.NS_NOALLOC_MAX_WS
    assert lib.sm_ns_polar_noalloc(ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000000),
                                   B.BF16, 4, 4096, 4096, 1, ctypes.byref(p), None) == 4
    assert lib.sm_ns_polar_noalloc(None, None, B.BF16, 1, 8, 8, 1, ctypes.byref(p), None) == 1
    assert lib.sm_last_hip_error() == 0


def test_mfma_ceiling_probe_rejects_on_the_host():
    lib = B.lib()
    ok = ctypes.c_void_p(0x1000)
    assert lib.sm_mfma_ceiling(1, 256, 100, None, 0, None, None) == 1               # null out
    assert lib.sm_mfma_ceiling(1, 256, 100, None, 0, ctypes.c_void_p(0x1002), None) == 1
    assert lib.sm_mfma_ceiling(3, 256, 100, None, 0, ok, None) == 1                 # bad mode
    assert lib.sm_mfma_ceiling(-1, 256, 100, None, 0, ok, None) == 1
    assert lib.sm_mfma_ceiling(1, 0, 100, None, 0, ok, None) == 2
    assert lib.sm_mfma_ceiling(0, 65537, 100, None, 0, ok, None) == 2
    assert lib.sm_mfma_ceiling(0, 256, 0, None, 0, ok, None) == 2
    assert lib.sm_mfma_ceiling(0, 256, 10000001, None, 0, ok, None) == 2
    # mode 2: the source buffer is checked too
    assert lib.sm_mfma_ceiling(2, 256, 100, None, 1 << 21, ok, None) == 1          # null src
    assert lib.sm_mfma_ceiling(2, 256, 100, ctypes.c_void_p(0x2008), 1 << 21, ok, None) == 1
    assert lib.sm_mfma_ceiling(2, 256, 100, ctypes.c_void_p(0x2000), 3 << 20, ok, None) == 2
    assert lib.sm_mfma_ceiling(2, 256, 100, ctypes.c_void_p(0x2000), 1 << 15, ok, None) == 2
    assert lib.sm_mfma_ceiling(2, 256, 100, ctypes.c_void_p(0x2000), 1 << 27, ok, None) == 2
