"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test fixes one part of the method with something independent of the
oracle's own code: a closed form, an invariant, a library routine (NumPy SVD,
torch float32/bfloat16 arithmetic), a brute-force loop, or a number the pages
print.  A dropped term, wrong sign, wrong index or transposed operand in the
oracle fails at least one of them.
"""
import json
import math
import os
import struct

import numpy as np
import pytest
import torch

from oracle import sm_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _orthonormal(rng, rows, cols):
    q, _ = np.linalg.qr(rng.standard_normal((rows, cols)))
    return q[:, :cols]


def _known_svd(rng, r, c, s):
    u = _orthonormal(rng, r, r)
    v = _orthonormal(rng, c, r)
    return u, v, u @ np.diag(s) @ v.T


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ---------------------------------------------------------------- P-1 EMA

@pytest.mark.parametrize("beta", [0.0, 0.5, 0.9, 0.99])
def test_p1_ema_constant_gradient_closed_form(beta):
    rng = np.random.default_rng(1)
    g = rng.standard_normal((5, 7))
    m = np.zeros_like(g)
    for t in range(1, 30):
        m = O.ema(m, g, beta)
        np.testing.assert_allclose(m, (1 - beta ** t) * g, rtol=1e-13, atol=1e-15)


def test_p1_lion_buffers_closed_form():
    rng = np.random.default_rng(2)
    g = rng.standard_normal((3, 4))
    m = np.zeros_like(g)
    b1, b2 = 0.9, 0.99
    for t in range(1, 20):
        ghat = O.lion_interp(m, g, b1)
        # interpolation of M_{t-1} = (1 - b2^(t-1)) G with G
        np.testing.assert_allclose(ghat, (b1 * (1 - b2 ** (t - 1)) + (1 - b1)) * g, rtol=1e-13)
        m = O.lion_momentum(m, g, b2)
        np.testing.assert_allclose(m, (1 - b2 ** t) * g, rtol=1e-13)


# ---------------------------------------------------------------- P-2 norm

def test_p2_frobenius_unit_norm_and_zero():
    rng = np.random.default_rng(3)
    for shape in [(1, 1), (3, 8), (64, 17)]:
        y = rng.standard_normal(shape) * 7.0
        x = O.frobenius_normalize(y, 1e-7)
        assert abs(math.sqrt(float(np.sum(x ** 2))) - 1.0) < 1e-6
        # direction unchanged
        np.testing.assert_allclose(x * np.linalg.norm(y), y, rtol=1e-6)
    z = O.frobenius_normalize(np.zeros((4, 5)), 1e-7)
    assert np.all(z == 0)


# ---------------------------------------------------------------- P-3 NS on known SVD

@pytest.mark.parametrize("r,c", [(4, 4), (6, 10), (16, 40)])
@pytest.mark.parametrize("coef", [(1.5, -0.5, 0.0), (1.9, -0.7, 0.05), (1.2, -0.1, -0.08)])
def test_p3_ns_scalar_map_on_singular_values(r, c, coef):
    rng = np.random.default_rng(r * 100 + c)
    s = rng.uniform(0.05, 1.0, size=r)
    u, v, x = _known_svd(rng, r, c, s)
    a, b, cc = coef
    iters = 4
    p = O.NSParams(iters=iters, a=a, b=b, c=cc)
    got = O.ns_direct_oriented(x, p)
    # scalar recursion per singular value, written independently here
    sk = s.copy()
    for _ in range(iters):
        sk = a * sk + b * sk ** 3 + cc * sk ** 5
    want = u @ np.diag(sk) @ v.T
    assert _rel(got, want) < 1e-12


def test_p3_tall_orientation_matches_transpose_map():
    rng = np.random.default_rng(7)
    r, c = 5, 12
    s = rng.uniform(0.1, 0.9, size=r)
    u, v, x = _known_svd(rng, r, c, s)
    tall = x.T.copy()                      # 12 x 5
    p = O.NSParams(iters=3, a=1.5, b=-0.5, c=0.0)
    got = O.ns_polar(tall, p, normalize=False)
    sk = s.copy()
    for _ in range(3):
        sk = 1.5 * sk - 0.5 * sk ** 3
    want = (u @ np.diag(sk) @ v.T).T
    assert got.shape == tall.shape
    assert _rel(got, want) < 1e-12


# ---------------------------------------------------------------- P-4 textbook polar

@pytest.mark.parametrize("shape", [(4, 6), (8, 8), (6, 3)])
def test_p4_converges_to_svd_polar_factor(shape):
    rng = np.random.default_rng(sum(shape))
    m, n = shape
    r = min(m, n)
    s = rng.uniform(0.3, 1.0, size=r)
    uu = _orthonormal(rng, m, r)
    vv = _orthonormal(rng, n, r)
    y = uu @ np.diag(s) @ vv.T
    uf, _, vt = np.linalg.svd(y, full_matrices=False)
    polar = uf @ vt
    got = O.ns_polar(y, O.NSParams(iters=12), normalize=False)
    assert np.max(np.abs(got - polar)) < 1e-12


# ---------------------------------------------------------------- P-5 spectral norm <= 1

@pytest.mark.parametrize("shape", [(8, 8), (16, 48), (48, 16), (3, 100)])
def test_p5_spectral_norm_at_most_one(shape):
    rng = np.random.default_rng(shape[0] + 3 * shape[1])
    y = rng.standard_normal(shape)
    for iters in (1, 2, 5):
        d = O.ns_polar(y, O.NSParams(iters=iters), normalize=True)
        assert np.linalg.norm(d, 2) <= 1.0 + 1e-12


# ---------------------------------------------------------------- P-6 fixed point

@pytest.mark.parametrize("coef", [(1.5, -0.5, 0.0), (2.0, -1.5, 0.5)])
def test_p6_orthogonal_fixed_point(coef):
    rng = np.random.default_rng(11)
    x = _orthonormal(rng, 12, 5).T            # 5 x 12, orthonormal rows
    a, b, c = coef
    got = O.ns_direct_oriented(x, O.NSParams(iters=6, a=a, b=b, c=c))
    assert np.max(np.abs(got - x)) < 1e-12


# ---------------------------------------------------------------- P-7 Gram form

@pytest.mark.parametrize("r,c,coef", [(6, 6, (1.5, -0.5, 0.0)), (8, 20, (1.5, -0.5, 0.0)),
                                      (10, 33, (1.8, -0.6, 0.04))])
def test_p7_gram_equals_direct_and_q_properties(r, c, coef):
    rng = np.random.default_rng(r * c)
    x = O.frobenius_normalize(rng.standard_normal((r, c)), 1e-7)
    a, b, cc = coef
    p = O.NSParams(iters=5, a=a, b=b, c=cc)
    d_gram, q = O.gram_ns_fresh_oriented(x, p)
    d_direct = O.ns_direct_oriented(x, p)
    assert _rel(d_gram, d_direct) < 1e-12
    assert np.max(np.abs(q - q.T)) < 1e-12
    g0 = x @ x.T
    assert np.max(np.abs(q @ g0 - g0 @ q)) < 1e-12


def test_p7_gram_tall_orientation():
    rng = np.random.default_rng(5)
    y = rng.standard_normal((30, 9))
    st = O.CacheState()
    p = O.NSParams(iters=5)
    d, err, refr = O.cache_muon_direction(y, st, 1, p, gamma=1.0)
    assert refr and err == -1.0 and st.q.shape == (9, 9)
    want = O.ns_polar(y, p, normalize=True)
    assert d.shape == y.shape
    assert _rel(d, want) < 1e-12


# ---------------------------------------------------------------- P-8 residual

def test_p8_residual_brute_force_and_special_values():
    rng = np.random.default_rng(8)
    d = rng.standard_normal((4, 7))
    total = 0.0
    for i in range(4):
        for j in range(4):
            dot = sum(d[i, k] * d[j, k] for k in range(7))
            e = dot - (1.0 if i == j else 0.0)
            total += e * e
    assert abs(O.orth_residual(d) - math.sqrt(total) / 2.0) < 1e-12
    orth = _orthonormal(rng, 9, 4).T
    assert O.orth_residual(orth) < 1e-14
    assert abs(O.orth_residual(np.zeros((5, 8))) - 1.0) < 1e-15
    for cval in (0.0, 0.5, 1.0, 1.7):
        assert abs(O.orth_residual(cval * np.eye(6)) - abs(cval ** 2 - 1)) < 1e-14


def test_p8_acceptance_is_inclusive():
    """CacheMuon technical summary, core mechanism item 3: the cached candidate
    is kept while its residual is at most the threshold (err <= gamma, the
    boundary included); one ulp above it refreshes, and a NaN residual fails
    the comparison."""
    for gamma in (0.0, 0.5, 2.0, 15.0):
        assert O.accept_cached(gamma, gamma)
        assert not O.accept_cached(float(np.nextafter(gamma, np.inf)), gamma)
        assert O.accept_cached(float(np.nextafter(gamma, -np.inf)), gamma)
    assert not O.accept_cached(float("nan"), 2.0)
    assert O.accept_cached(0.0, 0.0)     # an exactly orthogonal candidate at gamma = 0


# ---------------------------------------------------------------- P-9 trigger

def _ar1_stream(rng, shape, steps, rho=0.99):
    g = rng.standard_normal(shape)
    out = [g]
    for _ in range(steps - 1):
        g = rho * g + math.sqrt(1 - rho * rho) * rng.standard_normal(shape)
        out.append(g)
    return out


def test_p9_negative_gamma_refreshes_every_step_equals_direct_ns():
    rng = np.random.default_rng(9)
    p = O.NSParams(iters=5)
    st = O.CacheState()
    for t, y in enumerate(_ar1_stream(rng, (6, 14), 5), start=1):
        d, err, refr = O.cache_muon_direction(y, st, t, p, gamma=-1.0)
        assert refr and st.a_t == t
        if t > 1:
            assert err >= 0.0
        assert _rel(d, O.ns_polar(y, p)) < 1e-12


def test_p9_infinite_gamma_refreshes_only_first_step():
    rng = np.random.default_rng(10)
    p = O.NSParams(iters=5)
    st = O.CacheState()
    flags = []
    for t, y in enumerate(_ar1_stream(rng, (6, 14), 6), start=1):
        _, _, refr = O.cache_muon_direction(y, st, t, p, gamma=float("inf"))
        flags.append(refr)
    assert flags == [True] + [False] * 5 and st.a_t == 1


def test_p9_constant_input_reuse_equals_fresh():
    rng = np.random.default_rng(12)
    y = rng.standard_normal((7, 11))
    p = O.NSParams(iters=5)
    st = O.CacheState()
    d1, _, _ = O.cache_muon_direction(y, st, 1, p, gamma=10.0)
    d2, err, refr = O.cache_muon_direction(y, st, 2, p, gamma=10.0)
    assert not refr
    assert _rel(d2, d1) < 1e-13
    assert abs(err - O.orth_residual(O.orient(d1)[0])) < 1e-12


def test_p9_force_modes():
    rng = np.random.default_rng(13)
    p = O.NSParams(iters=5)
    st = O.CacheState()
    ys = _ar1_stream(rng, (5, 9), 3)
    _, _, r1 = O.cache_muon_direction(ys[0], st, 1, p, gamma=-1.0, mode=O.MODE_FORCE_REUSE)
    assert r1   # no cache yet: fresh regardless of mode
    _, _, r2 = O.cache_muon_direction(ys[1], st, 2, p, gamma=-1.0, mode=O.MODE_FORCE_REUSE)
    assert not r2 and st.a_t == 1
    _, err, r3 = O.cache_muon_direction(ys[2], st, 3, p, gamma=1e9, mode=O.MODE_FORCE_FRESH)
    assert r3 and err == -1.0 and st.a_t == 3


# ---------------------------------------------------------------- P-10 sign

def test_p10_sign_special_values():
    vals = np.array([0.0, -0.0, np.nan, -np.nan, np.inf, -np.inf,
                     np.float32(1e-45), np.float32(-1e-45), 1.0, -1.0, 3e38, -3e38],
                    dtype=np.float32)
    want = [1, 1, 1, 1, 1, -1, 1, -1, 1, -1, 1, -1]
    got = O.sign_values(vals)
    assert list(got) == want
    # brute force over random bit patterns, sign decided by the IEEE sign bit
    # and "is not zero and not NaN"
    rng = np.random.default_rng(14)
    bits = rng.integers(0, 2 ** 32, size=4096, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    for xi, bi in zip(x, bits):
        sign_bit = int(bi) >> 31
        exp = (int(bi) >> 23) & 0xFF
        mant = int(bi) & 0x7FFFFF
        is_nan = exp == 0xFF and mant != 0
        is_zero = exp == 0 and mant == 0
        expect_neg = sign_bit == 1 and not is_nan and not is_zero
        assert bool(O.sign_negative(xi)) == expect_neg


# ---------------------------------------------------------------- P-11 pack

@pytest.mark.parametrize("n", [0, 1, 63, 64, 65, 130, 1000])
def test_p11_pack_brute_force(n):
    rng = np.random.default_rng(n + 5)
    x = rng.standard_normal(n).astype(np.float32)
    words = O.sign_pack(x)
    assert words.dtype == np.uint64 and words.size == (n + 63) // 64
    for w in range(words.size):
        expect = 0
        for j in range(64):
            i = 64 * w + j
            if i < n and x[i] < 0:
                expect |= 1 << j
        assert int(words[w]) == expect
    popcount = sum(bin(int(w)).count("1") for w in words)
    assert popcount == int(np.sum(x < 0))
    np.testing.assert_array_equal(O.unpack_bits(words, n), x < 0)


def test_p11_payload_ratio_matches_pages():
    with open(os.path.join(GOLDEN, "payload_ratios.json")) as f:
        gold = json.load(f)
    for n in (64, 4096, 768 * 2304):
        x = np.ones(n, dtype=np.float32)
        packed_bytes = O.sign_pack(x).nbytes
        assert (n * 4) // packed_bytes == gold["bitpack_vs_float32"]
        assert (n * 4) // (n * 1) == gold["int8_vs_float32"]


# ---------------------------------------------------------------- P-12 vote

@pytest.mark.parametrize("mw", [1, 2, 3, 4, 5, 16])
def test_p12_vote_brute_force_and_symmetries(mw):
    rng = np.random.default_rng(mw)
    n = 200
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(mw)]
    bits = [O.sign_pack(x) for x in xs]
    v = O.vote_from_bits(bits, n)
    for i in range(n):
        total = sum(-1 if xs[k][i] < 0 else 1 for k in range(mw))
        assert v[i] == (0 if total == 0 else (1 if total > 0 else -1))
    if mw % 2 == 1:
        assert np.all(v != 0)
    # flipping every worker's sign flips the vote (no exact zeros in xs)
    vneg = O.vote_from_bits([O.sign_pack(-x) for x in xs], n)
    np.testing.assert_array_equal(vneg, -v)
    perm = rng.permutation(mw)
    np.testing.assert_array_equal(O.vote_from_bits([bits[k] for k in perm], n), v)
    np.testing.assert_array_equal(O.vote_from_bits([bits[0]] * mw, n), O.sign_values(xs[0]))


# ---------------------------------------------------------------- P-13 update

def _f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def test_p13_update_matches_torch_float32_and_bf16():
    rng = np.random.default_rng(15)
    n = 5000
    w32 = (0.02 * rng.standard_normal(n)).astype(np.float32)
    v = rng.integers(-1, 2, size=n).astype(np.int8)
    lr = 1e-3
    tw = torch.from_numpy(w32.copy())
    tv = torch.from_numpy(v.astype(np.float32))
    want32 = (tw - torch.tensor(lr, dtype=torch.float32) * tv).numpy()
    got32 = O.update_vote(w32, v, lr, O.F32).astype(np.float32)
    np.testing.assert_array_equal(got32.view(np.uint32), want32.view(np.uint32))
    # bf16 weights: values exactly bf16, subtraction in float32, RNE to bf16
    wb = torch.from_numpy(w32).to(torch.bfloat16)
    wbf = wb.to(torch.float32)
    want_b = (wbf - torch.tensor(lr, dtype=torch.float32) * tv).to(torch.bfloat16)
    got_b = O.update_vote(wbf.numpy().astype(np.float64), v, lr, O.BF16)
    want_bits = want_b.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.bf16_bits_from_f32(got_b.astype(np.float32)), want_bits)


def test_p13_hand_derived_bf16_values():
    # 0.02 -> bf16 1.28125 * 2^-6 = 0x3CA4 (mantissa 36); minus 1e-3 in float32
    # is 0.0190195..., whose nearest bf16 is 1.21875 * 2^-6 = 0x3C9C (mantissa
    # 28); plus 1e-3 gives 0.0210195..., nearest bf16 1.34375 * 2^-6 = 0x3CAC.
    w = O.f32_from_bf16_bits(np.array([0x3CA4, 0x3CA4, 0x3CA4], dtype=np.uint16))
    got = O.update_vote(w, np.array([1, -1, 0], dtype=np.int8), 1e-3, O.BF16)
    assert list(O.bf16_bits_from_f32(got.astype(np.float32))) == [0x3C9C, 0x3CAC, 0x3CA4]
    # 1.0 - 1e-3 = 0.999 lies within half a bf16 spacing (2^-9) of 1.0
    got1 = O.update_vote(np.array([1.0]), np.array([1], np.int8), 1e-3, O.BF16)
    assert got1[0] == 1.0
    # float32 weights keep the update: bits of fp32(1.0 - fp32(1e-3))
    got2 = O.update_vote(np.array([1.0]), np.array([1], np.int8), 1e-3, O.F32)
    assert _f32_bits(float(got2[0])) == _f32_bits(1.0 - float(np.float32(1e-3)))


def test_bf16_rounding_matches_torch_on_random_bits():
    rng = np.random.default_rng(16)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    finite = np.isfinite(x)
    got = O.bf16_bits_from_f32(x[finite])
    want = torch.from_numpy(x[finite].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)
    # ties: 1 + 2^-8 lies halfway between bf16 1.0 and 1 + 2^-7 and rounds to even (1.0)
    assert O.bf16_bits_from_f32(np.array([1.0 + 2 ** -8], np.float32))[0] == 0x3F80
    assert O.bf16_bits_from_f32(np.array([1.0 + 3 * 2 ** -8], np.float32))[0] == 0x3F82
    nanb = O.bf16_bits_from_f32(np.array([np.nan], np.float32))[0]
    assert (nanb & 0x7F80) == 0x7F80 and (nanb & 0x7F) != 0


# ---------------------------------------------------------------- P-14 LionMuon reductions

def _grads(rng, shape, steps, workers):
    return [[rng.standard_normal(shape) for _ in range(workers)] for _ in range(steps)]


def _run(cfg, w0, grads):
    m, n = w0.shape
    st = O.MatrixState(w=w0.copy(), mom=[np.zeros((m, n)) for _ in range(cfg.workers)])
    for t, g in enumerate(grads, start=1):
        O.step_matrix(st, g, cfg, t)
    return st


def test_p14_period_one_equal_betas_is_ema_muon():
    rng = np.random.default_rng(17)
    w0 = 0.02 * rng.standard_normal((6, 10))
    gs = _grads(rng, (6, 10), 5, 3)
    lion = O.StepConfig(algo=O.LION_MUON, workers=3, beta1=0.9, beta2=0.9, period=1)
    sm = O.StepConfig(algo=O.SIGN_MUON, workers=3, beta1=0.9)
    a = _run(lion, w0, gs)
    b = _run(sm, w0, gs)
    np.testing.assert_array_equal(a.w, b.w)
    for x, y in zip(a.mom, b.mom):
        np.testing.assert_array_equal(x, y)


def test_p14_infinite_period_is_lion_and_signum_and_signsgd_mv():
    rng = np.random.default_rng(18)
    shape = (5, 8)
    w0 = 0.02 * rng.standard_normal(shape)
    gs = _grads(rng, shape, 6, 1)
    lr = 1e-3

    def textbook(beta1, beta2, grads_seq, workers=1):
        w = w0.astype(np.float32).copy()
        ms = [np.zeros(shape) for _ in range(workers)]
        for g in grads_seq:
            total = np.zeros(shape, dtype=np.int64)
            for k in range(workers):
                d = (beta1 * ms[k] + (1 - beta1) * g[k]).astype(np.float32)
                total += np.where(d < 0, -1, 1)
                ms[k] = (beta2 * ms[k] + (1 - beta2) * g[k]).astype(np.float32).astype(np.float64)
            w = (w - np.float32(lr) * np.sign(total).astype(np.float32)).astype(np.float32)
        return w

    lion = _run(O.StepConfig(algo=O.LION_MUON, workers=1, beta1=0.9, beta2=0.99, period=0, lr=lr), w0, gs)
    np.testing.assert_array_equal(lion.w.astype(np.float32), textbook(0.9, 0.99, gs))
    signum = _run(O.StepConfig(algo=O.LION_MUON, workers=1, beta1=0.9, beta2=0.9, period=0, lr=lr), w0, gs)
    np.testing.assert_array_equal(signum.w.astype(np.float32), textbook(0.9, 0.9, gs))
    gs3 = _grads(rng, shape, 4, 3)
    mv = _run(O.StepConfig(algo=O.LION_MUON, workers=3, beta1=0.0, beta2=0.5, period=0, lr=lr), w0, gs3)
    np.testing.assert_array_equal(mv.w.astype(np.float32), textbook(0.0, 0.5, gs3, workers=3))


def test_p14_schedule_phase():
    assert [O.lion_muon_is_muon_step(t, 4) for t in range(1, 9)] == \
        [False, False, False, True, False, False, False, True]
    assert all(O.lion_muon_is_muon_step(t, 1) for t in range(1, 5))
    assert not any(O.lion_muon_is_muon_step(t, 0) for t in range(1, 50))


def test_p14_lion_muon_muon_step_uses_ns_of_interpolation():
    rng = np.random.default_rng(19)
    shape = (6, 9)
    w0 = 0.02 * rng.standard_normal(shape)
    gs = _grads(rng, shape, 2, 1)
    cfg = O.StepConfig(algo=O.LION_MUON, workers=1, beta1=0.9, beta2=0.99, period=2)
    st = O.MatrixState(w=w0.copy(), mom=[np.zeros(shape)])
    O.step_matrix(st, gs[0], cfg, 1)        # Lion step
    m1 = st.mom[0].copy()
    out = O.step_matrix(st, gs[1], cfg, 2)  # Muon step
    ghat = 0.9 * m1 + 0.1 * gs[1][0]
    want = O.ns_polar(ghat.astype(np.float32).astype(np.float64), cfg.ns)
    assert _rel(out["d"][0], want) < 1e-6


# ---------------------------------------------------------------- P-15 Sign-Muon, one worker

def test_p15_single_worker_sign_muon():
    rng = np.random.default_rng(20)
    shape = (8, 12)
    w0 = (0.02 * rng.standard_normal(shape)).astype(np.float32).astype(np.float64)
    g = rng.standard_normal(shape)
    cfg = O.StepConfig(algo=O.SIGN_MUON, workers=1, beta1=0.9, lr=1e-3)
    st = O.MatrixState(w=w0.copy(), mom=[np.zeros(shape)])
    O.step_matrix(st, [g], cfg, 1)
    mom = (0.1 * g).astype(np.float32).astype(np.float64)
    d = O.ns_polar(mom, cfg.ns).astype(np.float32)
    want = (w0.astype(np.float32) - np.float32(1e-3) * np.where(d < 0, -1, 1).astype(np.float32))
    np.testing.assert_array_equal(st.w.astype(np.float32), want)


def test_cache_muon_trajectory_polar_mode():
    rng = np.random.default_rng(21)
    shape = (6, 16)
    w0 = 0.02 * rng.standard_normal(shape)
    gs = [[g] for g in _ar1_stream(rng, shape, 6)]
    cfg = O.StepConfig(algo=O.CACHE_MUON, update=O.UPDATE_POLAR, workers=1,
                       beta1=0.9, gamma=float("inf"))
    st = O.MatrixState(w=w0.copy(), mom=[np.zeros(shape)])
    refreshed = []
    for t, g in enumerate(gs, start=1):
        out = O.step_matrix(st, g, cfg, t)
        refreshed += out["refreshed"]
    assert refreshed == [True] + [False] * 5
    assert st.cache[0].a_t == 1


# ---------------------------------------------------------------- Lion sign decision

def _exact_lion_negative(m, g, beta1):
    """Brute force with exact rationals: beta1 as the float32 the ABI
    receives, m and g as the stored values."""
    from fractions import Fraction
    b = Fraction(float(np.float32(beta1)))
    return np.array([b * Fraction(float(mi)) + (1 - b) * Fraction(float(gi)) < 0
                     for mi, gi in zip(m, g)])


def test_lion_sign_is_the_exact_sign_of_the_interpolation():
    rng = np.random.default_rng(22)
    b = np.float32(0.9)
    b9 = float(b)     # the hyper-parameter as the float32 the C ABI receives
    c = np.float32(1) - b
    m = rng.standard_normal(3000).astype(np.float32)
    g = rng.standard_normal(3000).astype(np.float32)
    # near-cancellations: g ~ -(b/c) m rounded to float32, nudged by 0..3 ulp
    # either way, where the float32 rounding of c*g decides a float32 sign
    k = 1500
    g_c = (-(np.float64(b) / np.float64(c)) * m[:k].astype(np.float64)).astype(np.float32)
    nudge = rng.integers(-3, 4, size=k)
    g[:k] = np.array([np.nextafter(x, np.float32(np.inf) if s > 0 else np.float32(-np.inf))
                      if s else x for x, s in zip(g_c, nudge)], dtype=np.float32)
    for _ in range(2):
        g[:k] = np.where(np.abs(nudge) > 1,
                         np.nextafter(g[:k], np.where(nudge > 0, np.inf, -np.inf).astype(np.float32)),
                         g[:k])
        nudge = np.where(np.abs(nudge) > 1, nudge - np.sign(nudge), nudge)
    got = O.lion_sign_negative(m, g, b9)
    np.testing.assert_array_equal(got, _exact_lion_negative(m, g, 0.9))
    # bf16-valued state: same rule
    mb = torch.from_numpy(m).to(torch.bfloat16).float().numpy()
    gb = torch.from_numpy(g).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(O.lion_sign_negative(mb, gb, b9),
                                  _exact_lion_negative(mb, gb, 0.9))
    # exact cancellation g = -9 m: fp32(0.9) = 0.89999998 and 1 - fp32(0.9) =
    # 0.10000002, so G_hat = 0.89999998 - 0.90000021 < 0 for m = 1
    assert O.lion_sign_negative(np.array([1.0]), np.array([-9.0]), b9)[0]
    assert not O.lion_sign_negative(np.array([-1.0]), np.array([9.0]), b9)[0]
    # beta1 = 0.5 is exact: m = 1, g = -1 cancels to 0 -> +1
    assert not O.lion_sign_negative(np.array([1.0]), np.array([-1.0]), 0.5)[0]
    # beta1 = 0 is signSGD on the gradient, beta1 = 1 the sign of the buffer
    np.testing.assert_array_equal(O.lion_sign_negative(m, g, 0.0), g < 0)
    np.testing.assert_array_equal(O.lion_sign_negative(m, g, 1.0), m < 0)


def test_update_polar_matches_torch_float32_and_bf16():
    rng = np.random.default_rng(23)
    n = 5000
    w32 = (0.02 * rng.standard_normal(n)).astype(np.float32)
    d32 = (0.05 * rng.standard_normal(n)).astype(np.float32)
    lr = 1e-3
    tl = torch.tensor(lr, dtype=torch.float32)
    want32 = (torch.from_numpy(w32) - tl * torch.from_numpy(d32)).numpy()
    got32 = O.update_polar(w32, d32, lr, O.F32).astype(np.float32)
    np.testing.assert_array_equal(got32.view(np.uint32), want32.view(np.uint32))
    wbf = torch.from_numpy(w32).to(torch.bfloat16).to(torch.float32)
    want_b = (wbf - tl * torch.from_numpy(d32)).to(torch.bfloat16).view(torch.int16).numpy()
    got_b = O.update_polar(wbf.numpy(), d32, lr, O.BF16).astype(np.float32)
    np.testing.assert_array_equal(O.bf16_bits_from_f32(got_b), want_b.view(np.uint16))


# ---------------------------------------------------------------- P-16 int8 encoding

def test_p16_sign_int8_special_values_and_payload():
    x = np.array([0.0, -0.0, np.nan, -1e-30, 1e-30, -np.inf, np.inf, -2.5, 3.0], np.float32)
    want = np.array([1, 1, 1, -1, 1, -1, 1, -1, 1], np.int8)   # -1 iff x < 0
    s = O.sign_int8(x)
    assert s.dtype == np.int8
    np.testing.assert_array_equal(s, want)
    # one byte per entry: the int8 payload of the pages' 4x ratio
    with open(os.path.join(GOLDEN, "payload_ratios.json")) as f:
        gold = json.load(f)
    n = 768 * 2304
    assert (n * 4) // O.sign_int8(np.ones(n, np.float32)).nbytes == gold["int8_vs_float32"]


@pytest.mark.parametrize("mw", [1, 2, 3, 4, 5, 16])
def test_p16_int8_vote_brute_force_and_equals_bit_vote(mw):
    rng = np.random.default_rng(100 + mw)
    n = 300
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(mw)]
    xs[0][:5] = [0.0, -0.0, np.nan, -1e-30, 1e-30]
    v8 = O.vote_from_int8([O.sign_int8(x) for x in xs], n)
    for i in range(n):
        total = sum(-1 if xs[k][i] < 0 else 1 for k in range(mw))
        assert v8[i] == (0 if total == 0 else (1 if total > 0 else -1))
    # M - 2 n_neg (the bit path's popcount form) equals the plain integer sum
    np.testing.assert_array_equal(v8, O.vote_from_bits([O.sign_pack(x) for x in xs], n))


def test_p16_int8_vote_ties_for_even_workers():
    s = [np.array([1, 1, -1, -1, 1], np.int8), np.array([-1, 1, 1, -1, 1], np.int8)]
    np.testing.assert_array_equal(O.vote_from_int8(s, 5), [0, 1, 0, -1, 1])


# ---------------------------------------------------------------- P-17 polar step on the vote

def _hadamard(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def _scalar_ns(sigma, p):
    for _ in range(p.iters):
        sigma = p.a * sigma + p.b * sigma ** 3 + p.c * sigma ** 5
    return sigma


@pytest.mark.parametrize("coef", [(1.5, -0.5, 0.0), (3.4445, -4.775, 2.0315)])
@pytest.mark.parametrize("n,reps,tall", [(4, 1, False), (8, 1, False), (8, 2, False),
                                         (8, 3, True), (16, 1, False)])
def test_p17_vote_polar_on_hadamard_votes_closed_form(coef, n, reps, tall):
    """V made of Hadamard blocks has all singular values equal, so NS acts as
    one scalar map: D = phi^K(sigma0) V / s with s = sqrt(n reps), the common
    singular value, and sigma0 = s / (||V||_F + eps)."""
    p = O.NSParams(5, *coef, eps=1e-7)
    v = np.hstack([_hadamard(n)] * reps)
    if tall:
        v = v.T
    s = math.sqrt(n * reps)
    sigma0 = s / (math.sqrt(v.size) + p.eps)
    want = _scalar_ns(sigma0, p) * v / s
    d = O.vote_polar_direction(v.astype(np.int8), p)
    assert d.shape == v.shape
    np.testing.assert_allclose(d, want, rtol=1e-12, atol=1e-14)


def test_p17_vote_polar_rank_one_and_zero_votes():
    p = O.NSParams()
    rng = np.random.default_rng(7)
    u = rng.choice([-1, 1], size=12)
    w = rng.choice([-1, 1], size=20)
    v = np.outer(u, w)
    s = math.sqrt(v.size)                 # the one nonzero singular value
    sigma0 = s / (s + p.eps)
    np.testing.assert_allclose(O.vote_polar_direction(v, p), _scalar_ns(sigma0, p) * v / s,
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(O.vote_polar_direction(np.zeros((6, 9), np.int8), p),
                                  np.zeros((6, 9)))


def test_p17_step_with_unanimous_hadamard_vote():
    """Whole step: every worker's momentum is a positive multiple of a
    Hadamard matrix H, so every sign matrix, and the vote, is H; with the
    polar step the update is W - lr * rnd(phi^K(sigma0) H / sqrt(n)); with
    either encoding the plain vote update is W - lr * H."""
    n, mw = 8, 3
    h = _hadamard(n)
    w0 = (0.02 * np.random.default_rng(3).standard_normal((n, n))).astype(np.float32)
    grads = [(k + 1.0) * h for k in range(mw)]
    p = O.NSParams()
    base = dict(algo=O.SIGN_MUON, workers=mw, wdtype=O.F32, mdtype=O.F32, lr=1e-3, beta1=0.9,
                ns=p)
    # momentum after one step from zero: 0.1 (k+1) H, ||.||_F = 0.1 (k+1) n
    results = {}
    for enc in (O.ENC_BITS, O.ENC_INT8):
        for vp in (False, True):
            st = O.MatrixState(w=w0.astype(np.float64), mom=[np.zeros((n, n))] * mw)
            out = O.step_matrix(st, grads, O.StepConfig(encoding=enc, vote_polar=vp, **base), 1)
            np.testing.assert_array_equal(out["vote"], h.astype(np.int8))
            results[(enc, vp)] = st.w
    np.testing.assert_array_equal(results[(O.ENC_BITS, False)],
                                  O.update_vote(w0, h, 1e-3, O.F32))
    sigma0 = math.sqrt(n) / (n + p.eps)
    d = (_scalar_ns(sigma0, p) * h / math.sqrt(n)).astype(np.float32)
    want = (w0 - (np.float32(1e-3) * d).astype(np.float32)).astype(np.float32)
    np.testing.assert_array_equal(results[(O.ENC_BITS, True)].astype(np.float32), want)
    for vp in (False, True):
        np.testing.assert_array_equal(results[(O.ENC_INT8, vp)], results[(O.ENC_BITS, vp)])


# ---------------------------------------------------------------- P-18 spectral distance

@pytest.mark.parametrize("m,n", [(40, 40), (30, 70), (90, 20)])
def test_p18_power_method_converges_to_svd(m, n):
    rng = np.random.default_rng(m * 1000 + n)
    r = min(m, n)
    s = np.linspace(3.0, 0.5, r)              # a clear gap at the top
    u = _orthonormal(rng, m, r)
    v = _orthonormal(rng, n, r)
    e = u @ np.diag(s) @ v.T
    v0 = rng.standard_normal(n)
    est = O.spectral_norm_power(e, v0, 300)
    assert abs(est - np.linalg.svd(e, compute_uv=False)[0]) <= 1e-10 * 3.0
    # a lower bound at every iteration count, increasing
    prev = 0.0
    for k in (0, 1, 2, 5, 10):
        cur = O.spectral_norm_power(e, v0, k)
        assert cur <= 3.0 + 1e-12 and cur >= prev - 1e-12
        prev = cur


def test_p18_power_method_closed_forms():
    rng = np.random.default_rng(18)
    # rank one: one iteration is exact, sigma = |a| |b|
    a, b = rng.standard_normal(12), rng.standard_normal(9)
    v0 = rng.standard_normal(9)
    assert math.isclose(O.spectral_norm_power(np.outer(a, b), v0, 1),
                        np.linalg.norm(a) * np.linalg.norm(b), rel_tol=1e-13)
    # diagonal: v_k is proportional to d^(2k) * v0, so the estimate is
    # ||d^(2k+1) v0|| / ||d^(2k) v0||
    d = np.array([2.0, -1.5, 1.0, 0.25])
    v0 = np.array([0.1, 1.0, 1.0, 1.0])
    for k in (0, 1, 3, 8):
        w = d ** (2 * k) * v0
        want = np.linalg.norm(d * w) / np.linalg.norm(w)
        assert math.isclose(O.spectral_norm_power(np.diag(d), v0, k), want, rel_tol=1e-13)
    # zero matrix, zero start vector, start vector orthogonal to the row space
    assert O.spectral_norm_power(np.zeros((5, 7)), np.ones(7), 4) == 0.0
    assert O.spectral_norm_power(np.eye(3), np.zeros(3), 4) == 0.0
    e = np.zeros((3, 3)); e[0, 0] = 5.0
    assert O.spectral_norm_power(e, np.array([0.0, 1.0, 0.0]), 3) == 0.0


def test_p18_fidelity_of_a_fresh_cache_is_zero_and_tall_matches_wide():
    """A Q just produced by the fresh solve on the same input reproduces the
    fresh direction (distance 0), and a tall input gives the transpose's
    numbers."""
    rng = np.random.default_rng(81)
    p = O.NSParams()
    y = rng.standard_normal((24, 60))
    x = O.frobenius_normalize(y, p.eps)
    _, q = O.gram_ns_fresh_oriented(x, p)
    v0 = rng.standard_normal(60)
    err, dist = O.cache_fidelity(y, q, p, v0, 20)
    assert dist <= 1e-12
    assert math.isclose(err, O.orth_residual(q @ x), rel_tol=1e-12)
    # a stale Q (from another input) has a positive distance, and the tall
    # input's distance equals the wide one with the start vector in the
    # other dimension
    q_stale = O.gram_ns_fresh_oriented(O.frobenius_normalize(
        y + 0.3 * rng.standard_normal(y.shape), p.eps), p)[1]
    err_w, dist_w = O.cache_fidelity(y, q_stale, p, rng.standard_normal(60), 200)
    err_t, dist_t = O.cache_fidelity(y.T, q_stale, p, rng.standard_normal(24), 200)
    assert dist_w > 1e-3
    assert math.isclose(err_w, err_t, rel_tol=1e-12)
    assert math.isclose(dist_w, dist_t, rel_tol=1e-8)
    cand = q_stale @ x
    fresh = O.gram_ns_fresh_oriented(x, p)[0]
    assert math.isclose(dist_w, np.linalg.svd(cand - fresh, compute_uv=False)[0], rel_tol=1e-8)
