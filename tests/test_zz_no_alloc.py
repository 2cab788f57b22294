"""sm_ns_polar_noalloc (the entry point that allocates nothing) against
sm_ns_polar, through the C ABI: two calls in a row on the library's fixed
scratch, the second with a smaller input, each bit-identical to the
workspace entry point's result on the same input."""
import ctypes

import numpy as np
import pytest
import torch

from matrix_aware_optimizer_momentum_amd import _binding as B
from tests.helpers import to_gpu

pytestmark = pytest.mark.gpu


def _call_ws(lib, x, u, dt, batch, m, n, p, stream):
    need = ctypes.c_size_t(0)
    assert lib.sm_ns_polar_ws(dt, batch, m, n, ctypes.byref(need)) == 0
    ws = torch.empty(need.value, dtype=torch.uint8, device="cuda")
    return lib.sm_ns_polar(x.data_ptr(), u.data_ptr(), dt, batch, m, n, 1, ctypes.byref(p),
                           ws.data_ptr(), need.value, stream)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_noalloc_equals_workspace_entry_point(gpu_lib, dt):
    lib = B.lib()
    code = B.BF16 if dt == "bf16" else B.F32
    p = B.NSParams(5, 1.5, -0.5, 0.0, 1e-7)
    stream = torch.cuda.current_stream().cuda_stream
    rng = np.random.default_rng(7)
    # a Gram-form batch (far from square), then a smaller direct-form one
    for batch, m, n in [(3, 384, 1536), (2, 200, 136)]:
        x = to_gpu(rng.standard_normal((batch, m, n)).astype(np.float32), dt)
        want = torch.empty_like(x)
        got = torch.full_like(x, float("nan"))
        assert _call_ws(lib, x, want, code, batch, m, n, p, stream) == 0
        assert lib.sm_ns_polar_noalloc(x.data_ptr(), got.data_ptr(), code, batch, m, n, 1,
                                       ctypes.byref(p), stream) == 0
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16) if dt == "bf16" else got.view(torch.int32),
                           want.view(torch.int16) if dt == "bf16" else want.view(torch.int32)), \
            (batch, m, n)


def test_noalloc_rejects_problems_beyond_its_scratch(gpu_lib):
    lib = B.lib()
    p = B.NSParams(5, 1.5, -0.5, 0.0, 1e-7)
    need = ctypes.c_size_t(0)
    assert lib.sm_ns_polar_ws(B.BF16, 8, 2048, 8192, ctypes.byref(need)) == 0
    assert need.value > B.NS_NOALLOC_MAX_WS
    x = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    assert lib.sm_ns_polar_noalloc(x.data_ptr(), x.data_ptr() + 4096, B.BF16, 8, 2048, 8192, 1,
                                   ctypes.byref(p), None) == 4
