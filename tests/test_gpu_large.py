"""GPU parity at the full shapes of the two largest layer sets.

* GPT-2 large (CacheMuon): the Gram Newton-Schulz solve with a cached Q at
  1280 x 3840, 1280 x 1280, 1280 x 5120 and 5120 x 1280 (bf16): a fresh
  solve (D and Q against the oracle's), a forced reuse of the oracle's own
  cache on a drifted input (candidate and residual against the oracle's),
  and the trigger on both sides of the oracle's residual.
* 7B-class LionMuon set (8 x 4096^2 + 8 x 4096 x 11008, M = 16, bf16,
  Student-t(3) gradients): sm_ns_polar at both shapes against the oracle's
  Newton-Schulz (the 4096 x 11008 problem runs in the Gram form); one whole
  Muon step and one whole Lion step in the launch configuration the
  benchmark times, checked on sampled matrices, workers and rows.
* The kernel-time accounting credits a predicated (skipped) fresh solve
  with no work.

The oracle side runs in float64 on the host; the largest case costs it a
few 4096 x 4096 x 11008 products.
"""
import sys

import numpy as np
import pytest
import torch

import matrix_aware_optimizer_momentum_amd as sm
from matrix_aware_optimizer_momentum_amd import workloads as W
from oracle import sm_oracle as O
from tests.helpers import (assert_ema_close, check_vote_within, f32, lion_band, rel_fro, to_gpu,
                           to_np)

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def _oriented(y):
    return (y.T, True) if y.shape[0] > y.shape[1] else (y, False)


# ------------------------------------------------------------------ GPT-2 large: CacheMuon

def test_cache_muon_full_size_steps_sampled(gpu_lib):
    """Two full config-4 steps as the benchmark runs them (144 matrices,
    707.8M parameters, M = 1, bf16, gamma = 2): the first refreshes every
    cache, the second reuses every one.  Sampled matrices (one per shape):
    the cached Q against the oracle's fresh solve on the step's own
    momentum; the second step's residual against the oracle's residual of
    the cached candidate on that step's momentum."""
    wl = W.WORKLOADS[4]
    say("cache muon full size: 144 matrices")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed)
    mats = []
    for (m, n) in wl.shapes:
        r = min(m, n)
        mats.append(sm.MatrixBuffers(
            w=(0.02 * torch.randn(m, n, generator=gen, device="cuda")).to(torch.bfloat16),
            mom=torch.zeros(1, m, n, dtype=torch.bfloat16, device="cuda"),
            grad=(wl.grad_std * torch.randn(1, m, n, generator=gen, device="cuda")).to(torch.bfloat16),
            q_cache=torch.zeros(1, r, r, dtype=torch.float32, device="cuda"),
            cache_state=torch.zeros(1, 2, dtype=torch.int32, device="cuda")))
    cfg = sm.StepConfig(algo=sm.CACHE_MUON, update=sm.UPDATE_POLAR, M=1, wdt=torch.bfloat16,
                        mdt=torch.bfloat16, gdt=torch.bfloat16, lr=wl.lr, beta1=wl.beta1,
                        ns=sm.NSParams(wl.ns_iters, wl.ns_a, wl.ns_b, wl.ns_c, wl.ns_eps),
                        gamma=wl.gamma, cache_mode=sm.MODE_TRIGGER)
    diag = torch.full((len(mats), 1, 2), 7.0, device="cuda")
    call = sm.StepCall(cfg, mats, diag=diag)
    op = O.NSParams(wl.ns_iters, f32(wl.ns_a), f32(wl.ns_b), f32(wl.ns_c), f32(wl.ns_eps))
    sample = [0, 1, 2, 3]                         # one matrix of each shape (first layer)
    w_before = [mb.w.clone() for mb in mats]
    call(1)
    torch.cuda.synchronize()
    assert diag[:, 0, 1].all()                    # no cache yet: every matrix refreshed
    assert all(mb.cache_state.cpu().tolist() == [[1, 1]] for mb in mats)
    for j, mb in enumerate(mats):                 # every weight matrix moved
        assert not torch.equal(mb.w, w_before[j]), j
    for j in sample:
        y = to_np(mats[j].mom)[0].astype(np.float64)
        xo, _ = _oriented(O.frobenius_normalize(y, op.eps))
        _, q_or = O.gram_ns_fresh_oriented(xo, op)
        eq = rel_fro(mats[j].q_cache.cpu().numpy()[0].astype(np.float64), q_or)
        say(f"  step 1 matrix {j} {wl.shapes[j]}: Q {eq:.2e}")
        assert eq <= TOL_BF16, (j, eq)
    # second step on a drifted gradient: gamma = 2 reuses every cache
    q1 = [mats[j].q_cache.clone() for j in sample]
    for mb in mats:
        mb.grad.mul_(0.99).add_((0.141 * wl.grad_std * torch.randn(mb.grad.shape, generator=gen,
                                                                    device="cuda")).to(torch.bfloat16))
    call(2)
    torch.cuda.synchronize()
    assert not diag[:, 0, 1].any()
    assert all(mb.cache_state.cpu().tolist() == [[1, 1]] for mb in mats)
    for i, j in enumerate(sample):
        assert torch.equal(mats[j].q_cache, q1[i])  # the cache is kept as it was
        y = to_np(mats[j].mom)[0].astype(np.float64)
        xo, _ = _oriented(O.frobenius_normalize(y, op.eps))
        cand = O.cache_reuse_oriented(q1[i].cpu().numpy()[0].astype(np.float64), xo)
        err_or = O.orth_residual(cand)
        err = float(diag[j, 0, 0].item())
        say(f"  step 2 matrix {j}: err gpu {err:.6f} oracle {err_or:.6f}")
        assert 0.0 <= err <= wl.gamma
        assert abs(err - err_or) <= 1e-3 * err_or, (j, err, err_or)


@pytest.mark.parametrize("shape", [(1280, 3840), (1280, 1280), (1280, 5120), (5120, 1280)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
def test_cache_muon_gpt2_large_shapes(gpu_lib, shape):
    m, n = shape
    r = min(m, n)
    say(f"cache muon {m}x{n}")
    rng = np.random.default_rng(m * 7 + n)
    p = sm.NSParams()
    op = O.NSParams(5, 1.5, -0.5, 0.0, f32(1e-7))
    q = torch.zeros(1, r, r, dtype=torch.float32, device="cuda")
    cs = torch.zeros(1, 2, dtype=torch.int32, device="cuda")
    x1 = W.as_storage((1e-2 * rng.standard_normal((1, m, n))).astype(np.float32), "bf16")

    def run(x, t, gamma, mode):
        d, err, refr = sm.gram_ns_cached(to_gpu(x, "bf16"), q, cs, t, gamma, mode=mode, params=p)
        torch.cuda.synchronize()
        return to_np(d)[0].astype(np.float64), float(err.item()), int(refr.item())

    # fresh solve
    d1, err1, refr1 = run(x1, 1, 2.0, 0)
    assert refr1 == 1 and err1 == -1.0
    xo, tr = _oriented(O.frobenius_normalize(x1[0], op.eps))
    d_or, q_or = O.gram_ns_fresh_oriented(xo, op)
    e = rel_fro(d1, d_or.T if tr else d_or)
    eq = rel_fro(q.cpu().numpy()[0].astype(np.float64), q_or)
    say(f"  fresh: D {e:.2e}, Q {eq:.2e}")
    assert e <= TOL_BF16 and eq <= TOL_BF16

    # forced reuse of the oracle's own cache on a drifted (AR(1)-like) input
    q.copy_(torch.from_numpy(q_or.astype(np.float32)[None]))
    x2 = W.as_storage((0.99 * x1 + 0.141 * 1e-2 *
                       rng.standard_normal((1, m, n))).astype(np.float32), "bf16")
    d2, err2, refr2 = run(x2, 2, -1.0, 2)
    assert refr2 == 0 and cs.cpu().tolist() == [[1, 1]]
    xo2, _ = _oriented(O.frobenius_normalize(x2[0], op.eps))
    q_or32 = q_or.astype(np.float32).astype(np.float64)
    cand = O.cache_reuse_oriented(q_or32, xo2)
    err_or = O.orth_residual(cand)
    e2 = rel_fro(d2, cand.T if tr else cand)
    say(f"  reuse: D_hat {e2:.2e}, err gpu {err2:.6f} oracle {err_or:.6f}")
    assert e2 <= TOL_BF16
    assert abs(err2 - err_or) <= 1e-3 * err_or
    own, _ = _oriented(d2)                      # the GPU's residual of its own candidate
    assert abs(err2 - O.orth_residual(own)) <= 1e-3 * O.orth_residual(own)

    # trigger: gamma just above the oracle's residual accepts, just below refreshes
    q.copy_(torch.from_numpy(q_or.astype(np.float32)[None]))
    cs.copy_(torch.tensor([[1, 1]], dtype=torch.int32))
    _, err3, refr3 = run(x2, 3, err_or * 1.01, 0)
    assert refr3 == 0 and cs.cpu().tolist() == [[1, 1]]
    d4, err4, refr4 = run(x2, 4, err_or * 0.99, 0)
    assert refr4 == 1 and cs.cpu().tolist() == [[1, 4]]
    d4_or, _ = O.gram_ns_fresh_oriented(xo2, op)
    assert rel_fro(d4, d4_or.T if tr else d4_or) <= TOL_BF16


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_predicated_fresh_solve_credits_no_work(gpu_lib, dt):
    """Kernel-time accounting: a fresh solve skipped on the device (forced
    reuse) is credited with no GEMM work; a forced fresh solve with all of
    it.  bf16 runs the Gram-form chain on the persistent kernels (gated
    launches; a symmetric product is credited with the half it computes),
    float32 the generic kernel (per-problem predicates, full products)."""
    m, n, batch = 256, 768, 3
    rng = np.random.default_rng(5)
    x = to_gpu((1e-2 * rng.standard_normal((batch, m, n))).astype(np.float32), dt)
    q = torch.zeros(batch, m, m, dtype=torch.float32, device="cuda")
    cs = torch.zeros(batch, 2, dtype=torch.int32, device="cuda")
    sm.gram_ns_cached(x, q, cs, 1, 2.0, mode=sm.MODE_FORCE_FRESH)
    torch.cuda.synchronize()
    work = {}
    for mode in (sm.MODE_FORCE_REUSE, sm.MODE_FORCE_FRESH):
        sm.profile_enable(True)
        try:
            sm.profile_reset()
            sm.gram_ns_cached(x, q, cs, 2, 2.0, mode=mode)
            torch.cuda.synchronize()
            work[mode] = {k: sm.profile_read(k) for k in ("gemm_gram", "gemm_rr", "gemm_apply",
                                                          "probe")}
        finally:
            sm.profile_enable(False)
    K = 5
    sym = 1.0 if dt == "bf16" else 2.0
    reuse, fresh = work[sm.MODE_FORCE_REUSE], work[sm.MODE_FORCE_FRESH]
    # forced reuse: the candidate (apply) and its probe ran, nothing of the solve
    assert reuse["gemm_gram"][2] == 0.0 and reuse["gemm_rr"][2] == 0.0
    assert reuse["gemm_apply"][2] == batch * 2.0 * m * m * n
    assert reuse["probe"][2] == batch * sym * m * m * n
    # forced fresh: no candidate, the whole solve
    assert fresh["probe"][2] == 0.0
    assert fresh["gemm_gram"][2] == batch * sym * m * m * n
    assert fresh["gemm_rr"][2] == batch * 3 * (K - 1) * sym * m ** 3
    assert fresh["gemm_apply"][2] == batch * 2.0 * m * m * n


# ------------------------------------------------------------------ 7B-class LionMuon set

def test_ns_polar_lion_muon_shapes(gpu_lib):
    """Newton-Schulz at 4096 x 4096 (direct form) and 4096 x 11008 (Gram form,
    a chain of bf16-rounded 4096 x 4096 products) against the oracle."""
    rng = np.random.default_rng(4096)
    for (m, n) in [(4096, 4096), (4096, 11008)]:
        say(f"ns_polar {m}x{n}")
        y = W.as_storage(rng.standard_t(3, size=(1, m, n)).astype(np.float32), "bf16")
        d = to_np(sm.ns_polar(to_gpu(y, "bf16")))[0]
        torch.cuda.synchronize()
        d_or = O.ns_polar(y[0], O.NSParams(5, 1.5, -0.5, 0.0, f32(1e-7)))
        e = rel_fro(d, d_or)
        say(f"  rel Frobenius {e:.2e}")
        assert e <= TOL_BF16


def _c5_state(seed):
    """The LionMuon layer set on the GPU: bf16 weights, momentum and
    Student-t(3) gradients drawn with a seeded torch generator."""
    wl = W.WORKLOADS[5]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    mats = []
    for (m, n) in wl.shapes:
        w = (0.02 * torch.randn(m, n, generator=gen, device="cuda")).to(torch.bfloat16)
        mom = (0.5 * torch.randn(wl.M, m, n, generator=gen, device="cuda")).to(torch.bfloat16)
        z = torch.randn(wl.M, m, n, generator=gen, device="cuda")
        chi = torch.zeros_like(z)
        for _ in range(3):
            chi += torch.randn(wl.M, m, n, generator=gen, device="cuda") ** 2
        g = (z / torch.sqrt(chi / 3.0)).to(torch.bfloat16)
        del z, chi
        mats.append(sm.MatrixBuffers(w=w, mom=mom, grad=g))
    return wl, mats


def _cfg5(wl):
    return sm.StepConfig(algo=wl.algo, update=wl.update, M=wl.M, wdt=torch.bfloat16,
                         mdt=torch.bfloat16, gdt=torch.bfloat16, lr=wl.lr, beta1=wl.beta1,
                         beta2=wl.beta2, period=wl.period,
                         ns=sm.NSParams(wl.ns_iters, wl.ns_a, wl.ns_b, wl.ns_c, wl.ns_eps))


def _vote_from_w(w_before, w_after, lr):
    """The vote each entry's bf16 update implies (9 where -1, 0, +1 coincide)."""
    cands = [O.update_vote(w_before, np.full(w_before.shape, v, np.int8), lr, "bf16")
             .astype(np.float32).view(np.uint32) for v in (-1, 0, 1)]
    got = w_after.astype(np.float32).view(np.uint32)
    hits = [c == got for c in cands]
    assert np.all(hits[0] | hits[1] | hits[2]), "update is not W - lr*v for any vote"
    v = np.full(w_before.shape, 9, np.int8)
    unique = (hits[0].astype(int) + hits[1] + hits[2]) == 1
    for val, h in zip((-1, 0, 1), hits):
        v[h & unique] = val
    return v


def test_lion_muon_full_size_steps_sampled(gpu_lib):
    """One Muon step (t = 4, P = 4) and the Lion step after it on the whole
    LionMuon layer set (M = 16), as the benchmark launches them.

    Muon step, on one matrix of each shape: each worker's G_hat is formed
    exactly from the pre-step state and rounded to bf16; sm_ns_polar of the
    16 G_hat gives directions (two of them checked against the oracle's
    Newton-Schulz); the step's vote equals the vote of their signs except
    where a direction is within the bf16 tolerance of zero; W moved by
    exactly that vote.  Lion step, on 64 sampled rows of both matrices: the
    vote of the exact signs of G_hat except inside the float32 band;
    momentum of every worker within the EMA bound."""
    wl, mats = _c5_state(20261203 + 5000 + 17)
    cfg = _cfg5(wl)
    lr = f32(cfg.lr)
    b1, b2 = f32(cfg.beta1), f32(cfg.beta2)
    sample = [0, 15]                    # a 4096 x 4096 and a 4096 x 11008 matrix
    pre = {j: (to_np(mats[j].w), mats[j].mom.clone(), mats[j].grad) for j in sample}
    w_all = [mb.w.clone() for mb in mats]
    call = sm.StepCall(cfg, mats)
    say("lion muon: Muon step t = 4")
    call(4)
    torch.cuda.synchronize()
    for j, mb in enumerate(mats):           # odd worker count aside, every entry moved or tied
        assert not torch.equal(mb.w.view(torch.int16), w_all[j].view(torch.int16)), j
    for j in sample:
        w0, mom0, g = pre[j]
        m, n = w0.shape
        # exact G_hat = b1 m + (1 - b1) g in float64 on the GPU, rounded once to bf16
        ghat = (b1 * mom0.double() + (1.0 - b1) * g.double()).float().to(torch.bfloat16)
        d = sm.ns_polar(ghat)
        torch.cuda.synchronize()
        dn = to_np(d)
        for k in (0, 7):
            d_or = O.ns_polar(to_np(ghat[k]), O.NSParams(5, 1.5, -0.5, 0.0, f32(1e-7)))
            e = rel_fro(dn[k], d_or)
            say(f"  matrix {j} {m}x{n} worker {k}: rel Frobenius {e:.2e}")
            assert e <= TOL_BF16
        # vote of the directions' signs: sign(M - 2 n_neg), ties 0
        n_neg = np.zeros((m, n), np.int32)
        for k in range(wl.M):
            n_neg += O.sign_negative(dn[k])
        v_chain = np.sign(wl.M - 2 * n_neg).astype(np.int8)
        v_gpu = _vote_from_w(w0, to_np(mats[j].w), lr)
        near0 = [np.abs(dn[k]) <= TOL_BF16 * np.sqrt(np.mean(dn[k].astype(np.float64) ** 2))
                 for k in range(wl.M)]
        nm = check_vote_within(v_gpu, v_chain, near0, f"Muon step matrix {j}", 1e-3)
        say(f"  matrix {j}: {nm} votes differ from the chain's, all near zero")
        # momentum after the step: beta2 EMA, sampled rows of every worker
        rows = slice(0, 64)
        m_new = to_np(mats[j].mom[:, rows])
        for k in range(wl.M):
            want = O.round_storage(O.lion_momentum(to_np(mom0[k, rows]), to_np(g[k, rows]), b2),
                                   "bf16")
            assert_ema_close(m_new[k], want, to_np(mom0[k, rows]), to_np(g[k, rows]), b2,
                             "bf16", f"matrix {j} worker {k}")
    del pre
    # the Lion step that follows (t = 5)
    say("lion muon: Lion step t = 5")
    rng = np.random.default_rng(55)
    rows = {j: torch.from_numpy(np.sort(rng.choice(mats[j].w.shape[0], size=64, replace=False)))
            .cuda() for j in sample}
    pre = {j: (to_np(mats[j].w[rows[j]]), to_np(mats[j].mom[:, rows[j]]),
               to_np(mats[j].grad[:, rows[j]])) for j in sample}
    call(5)
    torch.cuda.synchronize()
    for j in sample:
        w0, m0, g0 = pre[j]
        neg = [O.lion_sign_negative(m0[k], g0[k], b1) for k in range(wl.M)]
        v_or = O.vote_from_bits([O.pack_bits(x.reshape(-1)) for x in neg], w0.size)
        amb = [lion_band(m0[k], g0[k], b1) for k in range(wl.M)]
        w1 = to_np(mats[j].w[rows[j]])
        v_gpu = _vote_from_w(w0, w1, lr)
        nm = check_vote_within(v_gpu, v_or.reshape(w0.shape), amb, f"Lion step matrix {j}", 1e-4)
        ok = ~np.any(np.stack(amb), axis=0)
        want_w = O.update_vote(w0, v_or.reshape(w0.shape), lr, "bf16")
        np.testing.assert_array_equal(w1.view(np.uint32)[ok],
                                      want_w.astype(np.float32).view(np.uint32)[ok])
        m1 = to_np(mats[j].mom[:, rows[j]])
        for k in range(wl.M):
            want = O.round_storage(O.lion_momentum(m0[k], g0[k], b2), "bf16")
            assert_ema_close(m1[k], want, m0[k], g0[k], b2, "bf16", f"Lion matrix {j} worker {k}")
        say(f"  matrix {j}: {nm} votes inside the float32 band")
