"""GPU parity of the C-ABI entry points against the CPU oracle, stage by stage.

Each entry point gets seeded inputs, and the oracle recomputes the same stage
from exactly the values the GPU was given.  Sign, pack, vote and update must
match bit for bit; Newton-Schulz and Gram factors must be within the relative
Frobenius tolerance of their operand type (float32 1e-4, bfloat16 2e-2).
"""
import math

import numpy as np
import pytest
import torch

from oracle import sm_oracle as O
from tests.helpers import rel_fro, to_gpu, to_np, words_np

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
# an identity coefficient that is exactly the sum of two bf16 values
# (1.296875 + 0.0031280517578125), unlike 1.3, which has no such split
A2 = 1.3000030517578125


def _special(rng, n):
    x = rng.standard_normal(n).astype(np.float32)
    specials = np.array([0.0, -0.0, np.nan, -np.nan, np.inf, -np.inf, 1e-45, -1e-45,
                         -1e-40, 3e38, -3e38], dtype=np.float32)
    if n >= 4 * len(specials):
        pos = rng.choice(n, size=len(specials), replace=False)
        x[pos] = specials
    return x


# ------------------------------------------------------------------ sign + pack

@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 63, 64, 65, 2047, 2048, 2049, 100003, (1 << 20) + 7])
def test_sign_pack_bit_exact(gpu_lib, dt, n):
    import matrix_aware_optimizer_momentum_amd as sm
    rng = np.random.default_rng(1000 + n)
    x = _special(rng, n)
    xt = to_gpu(x, dt)
    bits = sm.sign_pack(xt)
    torch.cuda.synchronize()
    want = O.sign_pack(to_np(xt))
    np.testing.assert_array_equal(words_np(bits)[: want.size], want)


# ------------------------------------------------------------------ vote + update

@pytest.mark.parametrize("wdt", ["f32", "bf16"])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 16, 64])
@pytest.mark.parametrize("count", [1, 64, 1000, 4097, 65539])
def test_vote_update_bit_exact(gpu_lib, wdt, M, count):
    import matrix_aware_optimizer_momentum_amd as sm
    rng = np.random.default_rng(M * 100003 + count)
    words = (count + 63) // 64
    stride = words + 3                       # a padded worker stride
    signs = [rng.standard_normal(count).astype(np.float32) for _ in range(M)]
    if M >= 4:                               # force exact ties on some entries
        k = min(count, 50)
        for j in range(M // 2):
            signs[j][:k] = -1.0
        for j in range(M // 2, 2 * (M // 2)):
            signs[j][:k] = 1.0
    packed = np.zeros((M, stride), dtype=np.uint64)
    for k in range(M):
        packed[k, :words] = O.sign_pack(signs[k])
        packed[k, words:] = np.uint64(0xDEADBEEFDEADBEEF)   # padding must be ignored
    w0 = (0.02 * rng.standard_normal(count)).astype(np.float32)
    wt = to_gpu(w0, wdt)
    w_before = to_np(wt)
    bits = torch.from_numpy(packed.view(np.int64)).cuda()
    vote = torch.empty(count, dtype=torch.int8, device="cuda")
    sm.vote_update(bits, wt, 1e-3, vote_out=vote)
    torch.cuda.synchronize()
    want_v = O.vote_from_bits([packed[k, :words] for k in range(M)], count)
    np.testing.assert_array_equal(vote.cpu().numpy(), want_v)
    want_w = O.update_vote(w_before, want_v, 1e-3, O.F32 if wdt == "f32" else O.BF16)
    np.testing.assert_array_equal(to_np(wt).view(np.uint32),
                                  want_w.astype(np.float32).view(np.uint32))


# ------------------------------------------------------------------ int8 encoding

@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 7, 8, 9, 2049, 100003, (1 << 20) + 5])
def test_sign_int8_bit_exact(gpu_lib, dt, n):
    import matrix_aware_optimizer_momentum_amd as sm
    rng = np.random.default_rng(2000 + n)
    x = _special(rng, n)
    xt = to_gpu(x, dt)
    s8 = sm.sign_int8(xt)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(s8.cpu().numpy(), O.sign_int8(to_np(xt)))


def test_sign_int8_unaligned_output(gpu_lib):
    """An output that is not 8-byte aligned takes the per-byte path."""
    import matrix_aware_optimizer_momentum_amd as sm
    x = _special(np.random.default_rng(5), 1001)
    xt = to_gpu(x, "f32")
    buf = torch.zeros(1010, dtype=torch.int8, device="cuda")
    sm.sign_int8(xt, out=buf[3:1004])
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    np.testing.assert_array_equal(got[3:1004], O.sign_int8(x))
    assert not got[:3].any() and not got[1004:].any()


def _signs_for_vote(rng, M, count):
    xs = [rng.standard_normal(count).astype(np.float32) for _ in range(M)]
    if M >= 4:                               # exact ties on some entries
        k = min(count, 50)
        for j in range(M // 2):
            xs[j][:k] = -1.0
        for j in range(M // 2, 2 * (M // 2)):
            xs[j][:k] = 1.0
    return xs


@pytest.mark.parametrize("wdt", ["f32", "bf16"])
@pytest.mark.parametrize("M", [1, 2, 3, 5, 16, 64])
@pytest.mark.parametrize("count", [1, 8, 1000, 4097, 65539])
def test_vote_update_int8_bit_exact_and_equal_to_bits(gpu_lib, wdt, M, count):
    import matrix_aware_optimizer_momentum_amd as sm
    rng = np.random.default_rng(M * 7919 + count)
    xs = _signs_for_vote(rng, M, count)
    stride = count + 5                       # padded, unaligned worker stride
    s8 = np.full((M, stride), 77, dtype=np.int8)   # padding must be ignored
    for k in range(M):
        s8[k, :count] = O.sign_int8(xs[k])
    w0 = (0.02 * rng.standard_normal(count)).astype(np.float32)
    wt = to_gpu(w0, wdt)
    w_before = to_np(wt)
    vote = torch.empty(count, dtype=torch.int8, device="cuda")
    sm.vote_update_int8(torch.from_numpy(s8).cuda(), wt, 1e-3, vote_out=vote)
    # the same signs through the 1-bit path
    words = (count + 63) // 64
    packed = np.stack([O.sign_pack(x) for x in xs]).astype(np.uint64)
    wb = to_gpu(w0, wdt)
    vote_b = torch.empty(count, dtype=torch.int8, device="cuda")
    sm.vote_update(torch.from_numpy(packed.view(np.int64)).cuda(), wb, 1e-3, vote_out=vote_b)
    torch.cuda.synchronize()
    want_v = O.vote_from_int8([s8[k, :count] for k in range(M)], count)
    np.testing.assert_array_equal(vote.cpu().numpy(), want_v)
    np.testing.assert_array_equal(vote_b.cpu().numpy(), want_v)
    want_w = O.update_vote(w_before, want_v, 1e-3, O.F32 if wdt == "f32" else O.BF16)
    np.testing.assert_array_equal(to_np(wt).view(np.uint32),
                                  want_w.astype(np.float32).view(np.uint32))
    assert torch.equal(wt, wb)
    assert words == packed.shape[1]


@pytest.mark.parametrize("vdt", ["f32", "bf16"])
@pytest.mark.parametrize("enc", ["bits", "int8"])
@pytest.mark.parametrize("M,count", [(1, 9), (4, 4097), (5, 65539), (16, 1000)])
def test_vote_matrix_bit_exact(gpu_lib, vdt, enc, M, count):
    import matrix_aware_optimizer_momentum_amd as sm
    rng = np.random.default_rng(31 * M + count)
    xs = _signs_for_vote(rng, M, count)
    if enc == "bits":
        signs = torch.from_numpy(np.stack([O.sign_pack(x) for x in xs]).view(np.int64)).cuda()
    else:
        signs = torch.from_numpy(np.stack([O.sign_int8(x) for x in xs])).cuda()
    out = torch.full((count,), 5.0, dtype=torch.float32 if vdt == "f32" else torch.bfloat16,
                     device="cuda")
    sm.vote(signs, count, out)
    torch.cuda.synchronize()
    want = O.vote_from_int8([O.sign_int8(x) for x in xs], count).astype(np.float64)
    np.testing.assert_array_equal(to_np(out), want)


@pytest.mark.parametrize("wdt,ddt", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32"),
                                     ("f32", "bf16")])
@pytest.mark.parametrize("count", [1, 1001, 65536])
def test_polar_update_bit_exact(gpu_lib, wdt, ddt, count):
    import matrix_aware_optimizer_momentum_amd as sm
    rng = np.random.default_rng(count + 17)
    wt = to_gpu((0.02 * rng.standard_normal(count)).astype(np.float32), wdt)
    dt_ = to_gpu((rng.standard_normal(count) / 30).astype(np.float32), ddt)
    w_before, d = to_np(wt), to_np(dt_)
    sm.polar_update(wt, dt_, 3e-3)
    torch.cuda.synchronize()
    want = O.update_polar(w_before, d, 3e-3, O.F32 if wdt == "f32" else O.BF16)
    np.testing.assert_array_equal(to_np(wt).view(np.uint32),
                                  want.astype(np.float32).view(np.uint32))


# ------------------------------------------------------------------ direct NS

NS_CASES = [
    # dt, batch, m, n, iters, (a, b, c)
    ("f32", 1, 256, 256, 5, (1.5, -0.5, 0.0)),
    ("f32", 3, 64, 147, 1, (1.5, -0.5, 0.0)),
    ("f32", 2, 147, 64, 5, (1.5, -0.5, 0.0)),
    ("f32", 2, 200, 300, 5, (1.5, -0.5, 0.0)),
    ("f32", 1, 129, 130, 3, (1.5, -0.5, 0.0)),
    ("f32", 4, 8, 8, 5, (1.5, -0.5, 0.0)),
    ("f32", 2, 96, 160, 4, (1.8, -0.6, 0.04)),
    ("f32", 1, 1, 5, 5, (1.5, -0.5, 0.0)),
    ("bf16", 2, 768, 2304, 5, (1.5, -0.5, 0.0)),
    ("bf16", 2, 3072, 768, 5, (1.5, -0.5, 0.0)),
    ("bf16", 3, 64, 576, 5, (1.5, -0.5, 0.0)),
    ("bf16", 2, 250, 130, 5, (1.5, -0.5, 0.0)),
    ("bf16", 2, 128, 384, 4, (1.8, -0.6, 0.04)),
    # 256-tile kernel: partial tiles in every dimension, tall and wide
    ("bf16", 2, 136, 520, 5, (1.5, -0.5, 0.0)),
    ("bf16", 2, 520, 136, 5, (1.5, -0.5, 0.0)),
    ("bf16", 1, 264, 264, 3, (1.5, -0.5, 0.0)),
    ("bf16", 2, 256, 1024, 5, (1.8, -0.6, 0.04)),
    ("bf16", 1, 1280, 1280, 5, (1.5, -0.5, 0.0)),
    # 256-tile NT kernel with partial tiles (dimensions multiples of 128):
    # identity fold with a = 1.5 (one bf16 term), A2 (two terms), and 1.3
    # (no exact split: the general path of separate products)
    ("bf16", 2, 384, 640, 5, (1.5, -0.5, 0.0)),
    ("bf16", 2, 640, 384, 5, (1.5, -0.5, 0.0)),
    ("bf16", 3, 128, 1152, 3, (1.5, -0.5, 0.0)),
    ("bf16", 2, 640, 768, 5, (A2, 1.0 - A2, 0.0)),
    ("bf16", 2, 768, 640, 4, (A2, 1.0 - A2, 0.0)),
    ("bf16", 2, 384, 640, 5, (1.3, -0.3, 0.0)),
    ("bf16", 2, 640, 384, 4, (1.3, -0.3, 0.0)),
    # cubic on far-from-square shapes: the Gram form (r x r products), one
    # and several tiles, partial tiles, the two-term identity split (A2),
    # the fewest iterations it takes (2), wide and tall
    ("bf16", 2, 256, 1024, 5, (1.5, -0.5, 0.0)),
    ("bf16", 2, 1024, 256, 4, (1.5, -0.5, 0.0)),
    ("bf16", 3, 384, 1152, 2, (A2, 1.0 - A2, 0.0)),
    ("bf16", 1, 128, 4096, 5, (1.5, -0.5, 0.0)),
    ("bf16", 2, 640, 1920, 3, (1.5, -0.5, 0.0)),
    ("bf16", 2, 1920, 640, 6, (A2, 1.0 - A2, 0.0)),
    ("bf16", 2, 1920, 640, 3, (1.3, -0.3, 0.0)),
    # lower-triangle storage of S_k, T_k, Q_k over several row blocks: each
    # panel read partly as stored rows, partly from the mirror tiles
    ("bf16", 1, 1280, 3840, 3, (1.5, -0.5, 0.0)),
    ("bf16", 2, 896, 2688, 3, (1.5, -0.5, 0.0)),
    ("bf16", 2, 2688, 896, 2, (1.5, -0.5, 0.0)),
]


@pytest.mark.parametrize("case", NS_CASES, ids=lambda c: f"{c[0]}-b{c[1]}-{c[2]}x{c[3]}-K{c[4]}")
def test_ns_polar_matches_oracle(gpu_lib, case):
    import matrix_aware_optimizer_momentum_amd as sm
    dt, batch, m, n, iters, (a, b, c) = case
    rng = np.random.default_rng(batch * 7919 + m * 31 + n)
    x = (0.01 * rng.standard_normal((batch, m, n))).astype(np.float32)
    xt = to_gpu(x, dt)
    p = sm.NSParams(iters=iters, a=a, b=b, c=c)
    u = sm.ns_polar(xt, normalize=True, params=p)
    torch.cuda.synchronize()
    xin = to_np(xt)
    got = to_np(u)
    op = O.NSParams(iters=iters, a=a, b=b, c=c)
    for k in range(batch):
        want = O.ns_polar(xin[k], op, normalize=True)
        err = rel_fro(got[k], want)
        assert err <= TOL[dt], (k, err)


def test_float32_ns_large_tiles_equal_small_tiles(gpu_lib):
    """Float32 NS on 16 problems of 1024 x 2048 runs its Gram, quintic and
    apply launches on 128 x 128 tiles (enough tiles to fill the chip: the
    lean interior epilogue with Cin, mirrored 16-byte stores and four blocks
    per wave); one of the problems alone takes 64 x 64 tiles.  Both tile
    sizes sum every product over k in the same order, so the results must be
    bit-identical; one problem is also checked against the oracle."""
    import matrix_aware_optimizer_momentum_amd as sm
    b, m, n = 16, 1024, 2048
    rng = np.random.default_rng(1128)
    x = torch.from_numpy((0.01 * rng.standard_normal((b, m, n))).astype(np.float32)).cuda()
    p = sm.NSParams(iters=2, a=1.8, b=-0.6, c=0.04)
    u = sm.ns_polar(x, params=p)
    torch.cuda.synchronize()
    for k in (0, 11):
        one = sm.ns_polar(x[k:k + 1].contiguous(), params=p)
        torch.cuda.synchronize()
        assert torch.equal(one[0].view(torch.int32), u[k].view(torch.int32)), k
    want = O.ns_polar(to_np(x[11]), O.NSParams(iters=2, a=1.8, b=-0.6, c=0.04), normalize=True)
    assert rel_fro(to_np(u[11]), want) <= TOL["f32"]


@pytest.mark.parametrize("m,n,iters,a,gram_form", [
    (768, 3072, 5, 1.5, True), (3072, 768, 5, 1.5, True), (384, 1152, 2, 1.5, True),
    (384, 640, 5, 1.5, True), (1920, 640, 6, A2, True), (768, 768, 5, 1.5, False),
    (640, 768, 5, 1.5, False), (768, 3072, 1, 1.5, False), (1920, 640, 6, 1.3, False)])
def test_ns_form_taken(gpu_lib, m, n, iters, a, gram_form):
    """Far-from-square cubic problems run as r x r products, others directly
    (and so does every problem whose a has no exact two-term bf16 split)."""
    import matrix_aware_optimizer_momentum_amd as sm
    x = torch.randn(2, m, n, device="cuda", dtype=torch.bfloat16)
    sm.profile_enable(True)
    try:
        sm.profile_reset()
        sm.ns_polar(x, params=sm.NSParams(iters=iters, a=a, b=1.0 - a, c=0.0))
        torch.cuda.synchronize()
        rr_launches = sm.profile_read("gemm_rr")[1]
        gram_launches = sm.profile_read("gemm_gram")[1]
        apply_launches = sm.profile_read("gemm_apply")[1]
    finally:
        sm.profile_enable(False)
    if gram_form:
        assert (gram_launches, apply_launches, rr_launches) == (1, 1, 2 * iters - 1)
    else:
        assert (gram_launches, apply_launches, rr_launches) == (iters, iters, 0)


def test_ns_gram_form_split_launches(gpu_lib):
    """300 one-tile problems: Q_{k+1} of the middle iterations is split between
    two launches by problems (the first ones fill a launch's last round of
    tiles); problems on both sides of the split match the oracle."""
    import matrix_aware_optimizer_momentum_amd as sm
    b, m, n = 300, 256, 512
    rng = np.random.default_rng(4242)
    x = (0.01 * rng.standard_normal((b, m, n))).astype(np.float32)
    xt = to_gpu(x, "bf16")
    sm.profile_enable(True)
    try:
        sm.profile_reset()
        u = sm.ns_polar(xt, params=sm.NSParams(iters=5))
        torch.cuda.synchronize()
        rr_launches = sm.profile_read("gemm_rr")[1]
    finally:
        sm.profile_enable(False)
    assert rr_launches >= 9
    xin, got = to_np(xt), to_np(u)
    for k in (0, 100, 211, 212, 213, 299):
        want = O.ns_polar(xin[k], O.NSParams(iters=5), normalize=True)
        assert rel_fro(got[k], want) <= TOL["bf16"], k


def test_profile_counts_algorithmic_bytes(gpu_lib):
    """Each GEMM launch is credited with its operands read once and its output written once."""
    import matrix_aware_optimizer_momentum_amd as sm
    b, m, n = 3, 256, 1024
    x = torch.randn(b, m, n, device="cuda", dtype=torch.bfloat16)
    sm.profile_enable(True)
    try:
        sm.profile_reset()
        sm.ns_polar(x, params=sm.NSParams(iters=1))
        torch.cuda.synchronize()
        gram = sm.profile_read_bytes("gemm_gram")
        apply_ = sm.profile_read_bytes("gemm_apply")
        ema = sm.profile_read("norm")[2], sm.profile_read_bytes("norm")
    finally:
        sm.profile_enable(False)
    assert gram == b * (2 * m * n + 2 * m * m)          # X once (A == B), B_0 written
    assert apply_ == b * (2 * m * m + 2 * m * n + 2 * m * n)   # B_0, X read; X_1 written
    assert ema[0] == ema[1]                              # streaming kinds: bytes = work


def test_profile_counts_lower_stored_gram_form(gpu_lib):
    """Gram form with a one-term identity: S_k, T_k, Q_k are kept as their
    256 x 256 tiles on and below the diagonal, and each launch is credited
    with those stored entries (read once, written once)."""
    import matrix_aware_optimizer_momentum_amd as sm
    b, m, n, K = 2, 640, 1920, 3
    x = torch.randn(b, m, n, device="cuda", dtype=torch.bfloat16)
    sm.profile_enable(True)
    try:
        sm.profile_reset()
        sm.ns_polar(x, params=sm.NSParams(iters=K))
        torch.cuda.synchronize()
        gram = sm.profile_read_bytes("gemm_gram")
        rr = sm.profile_read_bytes("gemm_rr")
        apply_ = sm.profile_read_bytes("gemm_apply")
    finally:
        sm.profile_enable(False)
    low = 256 * 256 + 256 * 512 + 128 * 640          # row blocks of 256, 256, 128
    assert gram == b * (2 * m * n + 2 * low)
    # T_0 = S_0 (S_0 + aI) and T_1 read one matrix; S_1, Q_2, S_2, Q_3 two
    assert rr == b * 2 * (2 * 2 + 4 * 3) * low
    assert apply_ == b * (2 * low + 2 * m * n + 2 * m * n)


def test_ns_polar_without_normalisation(gpu_lib):
    import matrix_aware_optimizer_momentum_amd as sm
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 40, 90)).astype(np.float32)
    x /= np.linalg.norm(x, axis=(1, 2), keepdims=True) * 1.3
    xt = to_gpu(x, "f32")
    u = sm.ns_polar(xt, normalize=False, params=sm.NSParams(iters=5))
    torch.cuda.synchronize()
    for k in range(2):
        want = O.ns_polar(x[k].astype(np.float64), O.NSParams(iters=5), normalize=False)
        assert rel_fro(to_np(u)[k], want) <= 1e-4


def test_ns_polar_zero_input_gives_zero(gpu_lib):
    import matrix_aware_optimizer_momentum_amd as sm
    xt = torch.zeros(2, 64, 96, device="cuda", dtype=torch.bfloat16)
    u = sm.ns_polar(xt)
    bits = sm.sign_pack(u)
    torch.cuda.synchronize()
    assert torch.count_nonzero(u.float()).item() == 0
    assert torch.count_nonzero(bits).item() == 0          # all signs +1


# ------------------------------------------------------------------ Gram NS with cache

GRAM_CASES = [
    ("f32", 2, 96, 160, (1.5, -0.5, 0.0)),
    ("f32", 2, 160, 96, (1.5, -0.5, 0.0)),
    ("f32", 1, 130, 129, (1.8, -0.6, 0.04)),
    ("bf16", 2, 256, 640, (1.5, -0.5, 0.0)),
    ("bf16", 2, 640, 256, (1.5, -0.5, 0.0)),
    ("bf16", 1, 200, 333, (1.8, -0.6, 0.04)),
]


def _oriented(y):
    return (y.T, True) if y.shape[0] > y.shape[1] else (y, False)


@pytest.mark.parametrize("case", GRAM_CASES, ids=lambda c: f"{c[0]}-b{c[1]}-{c[2]}x{c[3]}")
def test_gram_ns_cached_stages(gpu_lib, case):
    import matrix_aware_optimizer_momentum_amd as sm
    dt, batch, m, n, (a, b, c) = case
    r = min(m, n)
    tol = TOL[dt]
    rng = np.random.default_rng(m * n + batch)
    p = sm.NSParams(iters=5, a=a, b=b, c=c)
    op = O.NSParams(iters=5, a=a, b=b, c=c)
    q = torch.zeros(batch, r, r, dtype=torch.float32, device="cuda")
    cs = torch.zeros(batch, 2, dtype=torch.int32, device="cuda")
    x = 0.01 * rng.standard_normal((batch, m, n)).astype(np.float32)

    def run(xnp, t, gamma, mode):
        xt = to_gpu(xnp, dt)
        d, err, refr = sm.gram_ns_cached(xt, q, cs, t, gamma, mode=mode, params=p)
        torch.cuda.synchronize()
        return to_np(xt), to_np(d), err.cpu().numpy(), refr.cpu().numpy()

    # step 1: no cache -> fresh solve
    xin, d, err, refr = run(x, 1, 2.0, 0)
    assert list(refr) == [1] * batch and np.all(err == -1.0)
    assert cs.cpu().numpy().tolist() == [[1, 1]] * batch
    qg = q.cpu().numpy().astype(np.float64)
    q_or = []                     # the oracle's own caches (no GPU value feeds the oracle)
    for k in range(batch):
        xo, tr = _oriented(O.frobenius_normalize(xin[k], op.eps))
        dw, qw = O.gram_ns_fresh_oriented(xo, op)
        assert rel_fro(d[k], dw.T if tr else dw) <= tol
        assert rel_fro(qg[k], qw) <= tol
        q_or.append(qw)

    # step 2: forced reuse of the cached Q on a drifted input
    x2 = x + 0.002 * rng.standard_normal(x.shape).astype(np.float32)
    xin2, d2, err2, refr2 = run(x2, 2, -1.0, 2)
    assert list(refr2) == [0] * batch
    assert cs.cpu().numpy().tolist() == [[1, 1]] * batch
    for k in range(batch):
        xo, tr = _oriented(O.frobenius_normalize(xin2[k], op.eps))
        cand = O.cache_reuse_oriented(q_or[k], xo)
        assert rel_fro(d2[k], cand.T if tr else cand) <= tol
        # residual of the GPU's own candidate, brute force in float64
        got_cand, _ = _oriented(d2[k].astype(np.float64))
        assert abs(err2[k] - O.orth_residual(got_cand)) <= 1e-3 * O.orth_residual(got_cand)

    # step 3: trigger with gamma = 0 refreshes (err > 0)
    x3 = x2 + 0.002 * rng.standard_normal(x.shape).astype(np.float32)
    xin3, d3, err3, refr3 = run(x3, 3, 0.0, 0)
    assert list(refr3) == [1] * batch and np.all(err3 > 0)
    assert cs.cpu().numpy().tolist() == [[1, 3]] * batch
    for k in range(batch):
        xo, tr = _oriented(O.frobenius_normalize(xin3[k], op.eps))
        cand_err = O.orth_residual(O.cache_reuse_oriented(q_or[k], xo))
        assert abs(err3[k] - cand_err) <= max(tol, 1e-3) * cand_err
        dw, _ = O.gram_ns_fresh_oriented(xo, op)
        assert rel_fro(d3[k], dw.T if tr else dw) <= tol

    # step 4: huge gamma accepts; step 5: forced fresh
    _, _, err4, refr4 = run(x3, 4, 1e9, 0)
    assert list(refr4) == [0] * batch and np.all(err4 >= 0)
    assert cs.cpu().numpy().tolist() == [[1, 3]] * batch
    _, _, err5, refr5 = run(x3, 5, 1e9, 1)
    assert list(refr5) == [1] * batch and np.all(err5 == -1.0)
    assert cs.cpu().numpy().tolist() == [[1, 5]] * batch


def test_gram_reuse_on_identical_input_is_stable(gpu_lib):
    """A constant input: the reused candidate equals the fresh direction."""
    import matrix_aware_optimizer_momentum_amd as sm
    rng = np.random.default_rng(77)
    x = rng.standard_normal((2, 64, 200)).astype(np.float32)
    xt = to_gpu(x, "f32")
    q = torch.zeros(2, 64, 64, device="cuda")
    cs = torch.zeros(2, 2, dtype=torch.int32, device="cuda")
    d1, _, _ = sm.gram_ns_cached(xt, q, cs, 1, 10.0)
    d1 = d1.clone()
    d2, err, refr = sm.gram_ns_cached(xt, q, cs, 2, 10.0)
    torch.cuda.synchronize()
    assert refr.cpu().tolist() == [0, 0]
    assert rel_fro(to_np(d2), to_np(d1)) <= 1e-5
    for k in range(2):
        assert abs(err.cpu().numpy()[k] - O.orth_residual(to_np(d1)[k].astype(np.float64))) < 1e-4


# ------------------------------------------------------------------ spectral distance (CacheMuon fidelity)

SPEC_CASES = [
    # dt, batch, m, n, iters, with_b
    ("f32", 1, 37, 53, 0, True),
    ("f32", 2, 37, 53, 5, True),
    ("f32", 3, 64, 200, 30, False),
    ("f32", 2, 2100, 9, 12, True),
    ("bf16", 3, 64, 200, 30, True),
    ("bf16", 2, 520, 136, 20, True),
    ("bf16", 2, 768, 2304, 15, True),
    ("bf16", 1, 5, 4099, 8, True),
]


@pytest.mark.parametrize("case", SPEC_CASES, ids=lambda c: f"{c[0]}-b{c[1]}-{c[2]}x{c[3]}-it{c[4]}")
def test_spectral_norm_matches_oracle(gpu_lib, case):
    import matrix_aware_optimizer_momentum_amd as sm
    dt, batch, m, n, iters, with_b = case
    rng = np.random.default_rng(batch * 1009 + m + n + iters)
    a = to_gpu(rng.standard_normal((batch, m, n)).astype(np.float32), dt)
    b = to_gpu((rng.standard_normal((batch, m, n)) * 0.5).astype(np.float32), dt) if with_b else None
    v0 = torch.from_numpy(rng.standard_normal((batch, n)).astype(np.float32)).cuda()
    out = sm.spectral_norm(a, b, v0, iters)
    torch.cuda.synchronize()
    an, v0n = to_np(a).astype(np.float64), v0.cpu().numpy().astype(np.float64)
    bn = to_np(b).astype(np.float64) if with_b else np.zeros_like(an)
    for k in range(batch):
        want = O.spectral_norm_power(an[k] - bn[k], v0n[k], iters)
        got = float(out.cpu().numpy()[k])
        assert abs(got - want) <= 2e-4 * want, (k, got, want)


def test_spectral_norm_zero_difference_and_zero_start(gpu_lib):
    import matrix_aware_optimizer_momentum_amd as sm
    rng = np.random.default_rng(3)
    a = to_gpu(rng.standard_normal((2, 30, 40)).astype(np.float32), "f32")
    v0 = torch.from_numpy(rng.standard_normal((2, 40)).astype(np.float32)).cuda()
    assert sm.spectral_norm(a, a.clone(), v0, 6).cpu().tolist() == [0.0, 0.0]
    assert sm.spectral_norm(a, None, torch.zeros_like(v0), 6).cpu().tolist() == [0.0, 0.0]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(96, 256), (256, 96)])
def test_cache_fidelity_chain_matches_oracle(gpu_lib, dt, shape):
    """The diagnostic as a chain of entry points: the cached candidate
    (forced reuse) and the fresh direction (forced fresh, on a copy of the
    cache) of the same input, their spectral distance, and the residual,
    against the oracle's cache_fidelity with the same stale Q and start
    vector."""
    import matrix_aware_optimizer_momentum_amd as sm
    m, n = shape
    r = min(m, n)
    rng = np.random.default_rng(m + 7 * n)
    p = O.NSParams()
    y = rng.standard_normal((m, n)).astype(np.float32)
    y_old = y + 0.4 * rng.standard_normal((m, n)).astype(np.float32)
    xo, _ = O.orient(y_old)
    q_stale = O.gram_ns_fresh_oriented(O.frobenius_normalize(xo, p.eps), p)[1].astype(np.float32)
    yt = to_gpu(y, dt)
    y_used = to_np(yt).astype(np.float64)
    q = torch.from_numpy(q_stale[None]).cuda()
    cs = torch.tensor([[1, 1]], dtype=torch.int32, device="cuda")
    q2, cs2 = q.clone(), cs.clone()
    d_hat, err, _ = sm.gram_ns_cached(yt[None], q, cs, 2, 0.0, mode=sm.MODE_FORCE_REUSE)
    d_fresh, _, _ = sm.gram_ns_cached(yt[None], q2, cs2, 2, 0.0, mode=sm.MODE_FORCE_FRESH)
    v0 = torch.from_numpy(rng.standard_normal((1, n)).astype(np.float32)).cuda()
    dist = sm.spectral_norm(d_hat, d_fresh, v0, 50)
    torch.cuda.synchronize()
    err_or, dist_or = O.cache_fidelity(y_used, q_stale.astype(np.float64), p,
                                       v0.cpu().numpy()[0].astype(np.float64), 50)
    tol = 1e-3 if dt == "f32" else 3e-2
    assert abs(err.item() - err_or) <= tol * max(err_or, 1.0), (err.item(), err_or)
    assert abs(dist.item() - dist_or) <= tol, (dist.item(), dist_or)
    assert dist_or > 0.03                           # the stale cache is measurably off


# ------------------------------------------------------------------ measurement probe

@pytest.mark.parametrize("mode", [0, 1, 2])
def test_mfma_ceiling_probe_runs_and_is_deterministic(gpu_lib, mode):
    """The benchmark's MFMA ceiling probe (not a step of the method): it
    writes finite per-thread sums of its accumulators for every workgroup,
    the same bits on a second run, reports the flops it executes, and in
    mode 2 only reads its source buffer."""
    import matrix_aware_optimizer_momentum_amd as sm
    blocks, iters = 8, 64
    out = torch.full((blocks * 256 + 5,), -7.0, dtype=torch.float32, device="cuda")
    src = torch.arange(1 << 16, dtype=torch.int32, device="cuda")     # 256 KB
    src0 = src.clone()
    flops = sm.mfma_ceiling(out, blocks, iters, mode, src)
    first = out.clone()
    sm.mfma_ceiling(out, blocks, iters, mode, src)
    torch.cuda.synchronize()
    assert flops == blocks * 4 * iters * 16 * 32768
    body = first[: blocks * 256]
    assert torch.isfinite(body).all() and (body != 0).any()
    assert torch.equal(out, first)
    assert (out[blocks * 256:] == -7.0).all()          # nothing written past the end
    assert torch.equal(src, src0)
    with pytest.raises(ValueError):
        sm.mfma_ceiling(out[:100], blocks, iters, mode, src)
