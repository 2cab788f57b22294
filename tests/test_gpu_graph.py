"""A step recorded as a HIP graph (sm_step_graph / sm_graph_launch) against
the same step called directly (sm_step).

Two copies of one seeded state run side by side for several steps, with a
fresh gradient per step copied into the same gradient buffers of both: one
copy through sm_step, the other through replays of graphs recorded once.
Between replays the program does eager work of its own on the same stream
and synchronises, and after every step the weights and momenta of the two
copies must agree bit for bit.  Cases: the float32 single-matrix and mixed
ResNet shapes (generic GEMM path), a bf16 GPT-2 block (persistent NS kernel
with fused sign packing), the int8 encoding with the polar step on the vote,
and LionMuon with one graph per step type.
"""
import pytest
import torch

import matrix_aware_optimizer_momentum_amd as sm
from matrix_aware_optimizer_momentum_amd import workloads as W

pytestmark = pytest.mark.gpu


def _tdt(dt):
    return torch.bfloat16 if dt == "bf16" else torch.float32


def _cfg(wl, **kw):
    d = dict(algo=wl.algo, update=wl.update, M=wl.M, wdt=_tdt(wl.wdt), mdt=_tdt(wl.mdt),
             gdt=_tdt(wl.gdt), lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, period=wl.period,
             ns=sm.NSParams(wl.ns_iters, wl.ns_a, wl.ns_b, wl.ns_c, wl.ns_eps), gamma=wl.gamma,
             cache_mode=wl.cache_mode)
    d.update(kw)
    return sm.StepConfig(**d)


def _state(wl, shapes, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    mats = []
    for (m, n) in shapes:
        mats.append(sm.MatrixBuffers(
            w=(0.02 * torch.randn(m, n, generator=gen, device="cuda")).to(_tdt(wl.wdt)),
            mom=(1e-3 * torch.randn(wl.M, m, n, generator=gen, device="cuda")).to(_tdt(wl.mdt)),
            grad=torch.zeros(wl.M, m, n, device="cuda", dtype=_tdt(wl.gdt))))
    return mats


def _copy(mats):
    return [sm.MatrixBuffers(w=mb.w.clone(), mom=mb.mom.clone(), grad=mb.grad.clone())
            for mb in mats]


def _bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)


CASES = {
    "f32-256": (1, [(256, 256)], {}),
    "f32-resnet": (3, [(64, 147), (256, 64), (128, 1152), (512, 4608), (1024, 256)], {}),
    "bf16-gpt2-block": (2, W.gpt2_block_shapes(768, 1), {}),
    "bf16-int8-polar": (2, [(256, 768), (768, 256)], {"encoding": sm.ENC_INT8,
                                                       "vote_polar": 1}),
    "bf16-lion": (5, [(256, 256), (256, 704)], {}),
}


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replays_equal_direct_steps(gpu_lib, case):
    idx, shapes, kw = CASES[case]
    wl = W.WORKLOADS[idx]
    if wl.algo == sm.LION_MUON:
        wl = wl.scaled(M=4, period=3)
    cfg = _cfg(wl, **kw)
    direct = _state(wl, shapes, 1234 + idx)
    graphed = _copy(direct)
    call = sm.StepCall(cfg, direct)
    lion = wl.algo == sm.LION_MUON
    # one graph per step type (LionMuon: Muon iff t % P == 0), sharing a workspace
    first = sm.StepGraph(cfg, graphed, 1)
    graphs = {False: first}
    if lion:
        graphs[True] = sm.StepGraph(cfg, graphed, wl.period, ws=first.ws)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(99 + idx)
    side = torch.randn(512, 512, device="cuda")
    steps = 7 if lion else 5
    for t in range(1, steps + 1):
        for a, b in zip(direct, graphed):
            g = (wl.grad_std * torch.randn(a.grad.shape, generator=gen, device="cuda"))
            a.grad.copy_(g)
            b.grad.copy_(g)
        call(t)
        graphs[lion and t % wl.period == 0]()
        side = torch.tanh(side @ side.T * 1e-3)   # the program's own eager work in between
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(direct, graphed)):
            assert torch.equal(_bits(a.w), _bits(b.w)), (case, t, j, "w")
            assert torch.equal(_bits(a.mom), _bits(b.mom)), (case, t, j, "mom")
        assert direct[0].w.float().abs().sum() > 0
    for g in graphs.values():
        g.close()


def test_graph_recording_refused_while_kernel_times_are_recorded(gpu_lib):
    wl = W.WORKLOADS[1]
    mats = _state(wl, [(64, 64)], 7)
    sm.profile_enable(True)
    try:
        with pytest.raises(sm.SmError) as e:
            sm.StepGraph(_cfg(wl), mats, 1)
        assert e.value.code == 5
    finally:
        sm.profile_enable(False)
    g = sm.StepGraph(_cfg(wl), mats, 1)   # and accepted once they are off
    g()
    torch.cuda.synchronize()
    g.close()
    with pytest.raises(RuntimeError):
        g()


def test_cache_muon_is_not_recordable(gpu_lib):
    wl = W.WORKLOADS[4].scaled(M=2)
    (m, n) = (128, 256)
    r = min(m, n)
    mats = [sm.MatrixBuffers(w=torch.zeros(m, n, device="cuda", dtype=_tdt(wl.wdt)),
                             mom=torch.zeros(wl.M, m, n, device="cuda", dtype=_tdt(wl.mdt)),
                             grad=torch.zeros(wl.M, m, n, device="cuda", dtype=_tdt(wl.gdt)),
                             q_cache=torch.zeros(wl.M, r, r, device="cuda"),
                             cache_state=torch.zeros(wl.M, 2, device="cuda", dtype=torch.int32))]
    with pytest.raises(sm.SmError) as e:
        sm.StepGraph(_cfg(wl), mats, 1)
    assert e.value.code == 5
