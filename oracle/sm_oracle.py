"""CPU oracle for the Muon-family optimizer step (Sign-Muon, CacheMuon, LionMuon).

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain reference that the
HIP library is checked against.  Only the test-suite, the package smoke check
and the benchmark's CPU-baseline leg may import it; the library itself never
does, and this module imports nothing from the library.

Precision: every floating-point step of the method (momentum, normalisation,
Newton-Schulz, Gram Newton-Schulz, residual probe) runs in float64.  The
integer and bit steps (sign, pack, vote) are exact, and the update emulates
IEEE float32 arithmetic followed by round-to-nearest-even (RNE) to bfloat16
bit by bit, because the update is defined to be bit-exact.

Sources (the pages the method is taken from; cited below by short name):
  [SignMuon-ja]  "SignMuon: communication-efficient distributed Muon
                 optimisation" technical summary, gist.science/ja/paper/2605.16311
  [SignMuon-abs] "SignMuon: Communication-Efficient Distributed Muon
                 Optimization", abstract (fugumt.com/fugumt/paper_check/
                 2605.16311v1 and hotpaper.ai/paper/2605.16311)
  [CacheMuon-ja] "CacheMuon" technical summary, gist.science/ja/paper/2606.16371
  [LionMuon-pt]  "LionMuon" technical summary, gist.science/pt/paper/2605.19811

Readings taken where the pages are silent (each is repeated at its function):
  * Sign-Muon momentum is the single EMA  M <- beta*M + (1-beta)*G,  M_0 = 0.
  * Lion's buffer update is  M <- beta2*M + (1-beta2)*G, applied after the
    interpolation has used the previous M.
  * Normalisation is  X = Y / (||Y||_F + eps).
  * Newton-Schulz polynomial: X <- a X + b (X X^T) X + c (X X^T)^2 X, the
    coefficients are parameters (cubic default a=1.5, b=-0.5, c=0).
  * Tall matrices (m > n) are iterated on their transpose (r = min(m, n)).
  * Gram Newton-Schulz: G_0 = X X^T, Q_0 = I, P_k = aI + bG_k + cG_k^2,
    Q_{k+1} = P_k Q_k, G_{k+1} = P_k G_k P_k, direction Q_K X.
  * sign(x) = -1 if x < 0 else +1 (so +0, -0 and NaN give +1); vote ties give 0.
  * 1-bit layout: uint64 words, bit (i mod 64) of word i//64 is 1 iff entry i
    (row-major, original orientation) is negative; tail bits are 0.
  * Update: W <- rnd_W(fp32(W) - fp32(lr) * V) with one float32 rounding.
  * int8 encoding (the integer SUM all-reduce variant): one signed byte per
    entry, s in {-1, +1}; the vote sums them as integers, ties give 0.
  * Optional polar step on the vote: D = NS(V / (||V||_F + eps)) with the
    workers' Newton-Schulz settings, then W <- rnd_W(fp32(W) - fp32(lr * D)).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

# --------------------------------------------------------------------------
# Storage emulation (float32 and bfloat16 bit patterns)
# --------------------------------------------------------------------------

F32 = "f32"
BF16 = "bf16"


def bf16_bits_from_f32(x) -> np.ndarray:
    """Round float32 values to bfloat16 with round-to-nearest-even.

    Returns the uint16 bit patterns.  NaN stays NaN (quiet, sign kept).
    bfloat16 is the upper half of an IEEE float32; RNE adds 0x7FFF plus the
    lowest kept bit before truncating the low 16 bits.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    is_nan = np.isnan(x)
    nan_bits = ((u >> np.uint64(16)) | np.uint64(0x0040)) & np.uint64(0xFFFF)
    out = np.where(is_nan, nan_bits, rounded)
    return out.astype(np.uint16)


def f32_from_bf16_bits(bits) -> np.ndarray:
    """bfloat16 bit patterns -> exactly equal float32 values."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def round_storage(x, dtype: str) -> np.ndarray:
    """Round values to a storage type and return them as float64.

    Float32 storage rounds once (RNE).  bfloat16 storage rounds to float32
    first and then to bfloat16 (RNE), the way a kernel computing in float32
    stores bfloat16.
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == F32:
        return x32.astype(np.float64)
    if dtype == BF16:
        return f32_from_bf16_bits(bf16_bits_from_f32(x32)).astype(np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# --------------------------------------------------------------------------
# a1: momentum
# --------------------------------------------------------------------------

def ema(m_prev, g, beta: float) -> np.ndarray:
    """Single exponential moving average of the gradient.

    [SignMuon-ja] section 2, algorithm flow step 1: every worker refreshes
    its local momentum from its stochastic gradient.  No formula is printed;
    the reading taken is M <- beta*M + (1-beta)*G starting from M = 0.
    The same single buffer serves CacheMuon ([CacheMuon-ja] core mechanism:
    X_t is the normalised momentum).
    """
    m_prev = np.asarray(m_prev, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    return beta * m_prev + (1.0 - beta) * g


def lion_interp(m_prev, g, beta1: float) -> np.ndarray:
    """Lion interpolation  G_hat = beta1*M_{t-1} + (1-beta1)*G_t.

    [LionMuon-pt] Methodology, core algorithm item 2 (shared momentum): the
    update direction is this interpolation of the previous buffer and the
    fresh gradient.
    """
    return beta1 * np.asarray(m_prev, np.float64) + (1.0 - beta1) * np.asarray(g, np.float64)


def lion_momentum(m_prev, g, beta2: float) -> np.ndarray:
    """Lion buffer update  M_t = beta2*M_{t-1} + (1-beta2)*G_t.

    [LionMuon-pt] Methodology item 2 names a single dual-EMA buffer but prints
    only the interpolation; the second EMA with beta2 is the standard Lion
    rule that the page's "dual EMA" refers to, applied after the
    interpolation has read M_{t-1}.
    """
    return beta2 * np.asarray(m_prev, np.float64) + (1.0 - beta2) * np.asarray(g, np.float64)


def lion_sign_negative(m_prev, g, beta1: float) -> np.ndarray:
    """'Entry is negative' for the Lion direction sign(G_hat), G_hat exact.

    [LionMuon-pt] Methodology, core algorithm item 2: a Lion step moves by
    the sign of the interpolation G_hat = beta1*M_{t-1} + (1-beta1)*G_t.
    The sign is that of the exact value: with M_{t-1} and G_t the stored
    (float32 or bfloat16) values and beta1 a float32 hyper-parameter, both
    products and 1 - beta1 are exact in float64, and the one rounding of
    their float64 sum cannot change its sign (it is 0 only when the exact
    sum is 0, which counts as +1).
    """
    return sign_negative(lion_interp(m_prev, g, beta1))


# --------------------------------------------------------------------------
# a2: Frobenius normalisation
# --------------------------------------------------------------------------

def frobenius_normalize(y, eps: float) -> np.ndarray:
    """X = Y / (||Y||_F + eps).

    [CacheMuon-ja] core mechanism item 2 calls X_t the normalised momentum;
    [SignMuon-ja] section 4 (nanoGPT, hyper-parameters) says Frobenius
    scaling works.  The eps guard is a reading; the pages give none (Y = 0 gives X = 0).
    """
    y = np.asarray(y, dtype=np.float64)
    norm = math.sqrt(float(np.sum(y * y)))
    return y / (norm + eps)


# --------------------------------------------------------------------------
# a3: direct Newton-Schulz polar iteration
# --------------------------------------------------------------------------

@dataclass
class NSParams:
    iters: int = 5
    a: float = 1.5
    b: float = -0.5
    c: float = 0.0
    eps: float = 1e-7


def orient(y):
    """Return (X, transposed) with X wide (rows <= cols).

    Reading: a tall matrix is iterated on its transpose so the Gram matrix is
    r x r with r = min(m, n).  (X X^T) X = X (X^T X) in exact arithmetic, so
    the direct iterate is the same either way.
    """
    y = np.asarray(y, dtype=np.float64)
    if y.shape[0] > y.shape[1]:
        return y.T.copy(), True
    return y.copy(), False


def ns_direct_oriented(x, p: NSParams) -> np.ndarray:
    """Newton-Schulz iteration on a wide matrix (rows <= cols).

    [SignMuon-ja] section 2, core mechanism item 1: the polar factor of the
    momentum is approximated locally by a Newton-Schulz iteration that
    orthogonalises it; [LionMuon-pt] problem statement: Muon's update is the
    matrix sign msign(G_hat) computed by Newton-Schulz.  Each step applies
    X <- a X + b A X + c A^2 X with A = X X^T.
    """
    x = np.asarray(x, dtype=np.float64)
    for _ in range(p.iters):
        a_mat = x @ x.T
        b_mat = p.b * a_mat
        if p.c != 0.0:
            b_mat = b_mat + p.c * (a_mat @ a_mat)
        x = p.a * x + b_mat @ x
    return x


def ns_polar(y, p: NSParams, normalize: bool = True) -> np.ndarray:
    """Direct NS direction of an m x n matrix in its original orientation."""
    x, tr = orient(y)
    if normalize:
        x = frobenius_normalize(x, p.eps)
    d = ns_direct_oriented(x, p)
    return d.T.copy() if tr else d


# --------------------------------------------------------------------------
# a4 / a5: Gram Newton-Schulz with a cached left transform (CacheMuon)
# --------------------------------------------------------------------------

def gram_ns_fresh_oriented(x, p: NSParams):
    """Fresh Gram Newton-Schulz solve on a wide X; returns (D, Q).

    [CacheMuon-ja] core mechanism item 1: a refresh step runs the full Gram
    Newton-Schulz solver, which yields the approximate polar factor and the
    left transform Q that is cached.  The pages name the solver but print no
    steps; the reading is the Gram-space rewrite of the direct iteration:
    with G_k = X_k X_k^T and X_k = Q_k X, one direct step is X_{k+1} = P_k X_k
    with P_k = aI + bG_k + cG_k^2, so Q_{k+1} = P_k Q_k and
    G_{k+1} = P_k G_k P_k^T = P_k G_k P_k (P_k is symmetric).
    """
    x = np.asarray(x, dtype=np.float64)
    r = x.shape[0]
    eye = np.eye(r)
    g = x @ x.T
    q = eye.copy()
    for _ in range(p.iters):
        pk = p.a * eye + p.b * g
        if p.c != 0.0:
            pk = pk + p.c * (g @ g)
        q = pk @ q
        g = pk @ g @ pk
    return q @ x, q


def cache_reuse_oriented(q, x) -> np.ndarray:
    """Candidate direction D_hat = Q X from a cached Q.

    [CacheMuon-ja] core mechanism item 2: between refreshes the cached
    transform from the last refresh step a_t is applied to the current
    normalised momentum.
    """
    return np.asarray(q, np.float64) @ np.asarray(x, np.float64)


def orth_residual(d) -> float:
    """err = ||D D^T - I||_F / ||I||_F with I the r x r identity (r = rows).

    [CacheMuon-ja] core mechanism item 3 (residual trigger equation).  The
    identity's Frobenius norm is sqrt(r).
    """
    d = np.asarray(d, dtype=np.float64)
    r = d.shape[0]
    e = d @ d.T - np.eye(r)
    return math.sqrt(float(np.sum(e * e))) / math.sqrt(r)


def accept_cached(err: float, gamma: float) -> bool:
    """The candidate is accepted iff err <= gamma ([CacheMuon-ja] item 3).

    A NaN residual fails the comparison and forces a refresh.
    """
    return bool(err <= gamma)


MODE_TRIGGER = 0
MODE_FORCE_FRESH = 1
MODE_FORCE_REUSE = 2


@dataclass
class CacheState:
    """Per-matrix CacheMuon state: cached Q (oriented r x r) and refresh index."""
    has_cache: bool = False
    a_t: int = 0
    q: Optional[np.ndarray] = None


def cache_muon_direction(y, state: CacheState, t: int, p: NSParams, gamma: float,
                         mode: int = MODE_TRIGGER, normalize: bool = True):
    """One CacheMuon orthogonalisation; returns (D, err, refreshed).

    [CacheMuon-ja] core mechanism items 1-3.  With no cache (the first step),
    or mode FORCE_FRESH, a fresh solve runs.  Otherwise the cached candidate
    is probed and accepted iff err <= gamma (always accepted in FORCE_REUSE).
    On a refresh Q is replaced and a_t = t.  err is -1 when no candidate was
    probed.  D is returned in the original orientation; `state` is updated.
    """
    x, tr = orient(y)
    if normalize:
        x = frobenius_normalize(x, p.eps)
    err = -1.0
    d = None
    if state.has_cache and mode != MODE_FORCE_FRESH:
        cand = cache_reuse_oriented(state.q, x)
        err = orth_residual(cand)
        if mode == MODE_FORCE_REUSE or accept_cached(err, gamma):
            d = cand
    refreshed = d is None
    if refreshed:
        d, q = gram_ns_fresh_oriented(x, p)
        state.q = q
        state.has_cache = True
        state.a_t = t
    return (d.T.copy() if tr else d), err, refreshed


# --------------------------------------------------------------------------
# a6: LionMuon schedule
# --------------------------------------------------------------------------

def lion_muon_is_muon_step(t: int, period: int) -> bool:
    """Muon (NS) step iff P > 0 and t mod P == 0, t counted from 1.

    [LionMuon-pt] core algorithm item 1: one Muon step every P-th iteration,
    Lion sign steps for the other P-1.  P = 0 encodes P = infinity (pure
    Lion, item 4).
    """
    return period > 0 and t % period == 0


# --------------------------------------------------------------------------
# a7 / a8: sign and 1-bit packing
# --------------------------------------------------------------------------

def sign_negative(x) -> np.ndarray:
    """Boolean 'entry is negative' under sign(x) = -1 iff x < 0.

    [SignMuon-ja] section 2, algorithm flow step 2: entrywise sign with values
    in {-1, +1}.  +0, -0 and NaN map to +1 (the predicate x < 0 is false).
    """
    return np.asarray(x) < 0


def sign_values(x) -> np.ndarray:
    """The sign matrix S in {-1, +1} as int8."""
    return np.where(sign_negative(x), -1, 1).astype(np.int8)


def pack_bits(neg) -> np.ndarray:
    """Pack a flat boolean 'negative' array into uint64 words, LSB first.

    [SignMuon-ja] section 2, algorithm flow step 3 (all-gather variant): one
    bit per entry.  Word w holds entries 64w .. 64w+63; tail bits are zero.
    """
    neg = np.asarray(neg, dtype=bool).reshape(-1)
    n = neg.size
    nwords = (n + 63) // 64
    padded = np.zeros(nwords * 64, dtype=np.uint64)
    padded[:n] = neg.astype(np.uint64)
    weights = np.uint64(1) << np.arange(64, dtype=np.uint64)
    return (padded.reshape(nwords, 64) * weights).sum(axis=1, dtype=np.uint64)


def unpack_bits(words, count: int) -> np.ndarray:
    """Inverse of pack_bits: uint64 words -> boolean array of `count` entries."""
    words = np.asarray(words, dtype=np.uint64).reshape(-1)
    shifts = np.arange(64, dtype=np.uint64)
    bits = (words[:, None] >> shifts[None, :]) & np.uint64(1)
    return bits.reshape(-1)[:count].astype(bool)


def sign_pack(x) -> np.ndarray:
    """a7 + a8 on a flat array in its row-major order."""
    return pack_bits(sign_negative(np.asarray(x).reshape(-1)))


# --------------------------------------------------------------------------
# a9 / a10: majority vote and update
# --------------------------------------------------------------------------

def vote_from_bits(bits_per_worker: Sequence[np.ndarray], count: int) -> np.ndarray:
    """Majority vote V = sign(sum_m S^(m)) with ties -> 0.

    [SignMuon-ja] section 2, core mechanism item 3 and algorithm flow step 4:
    the workers' sign matrices are summed as integers and thresholded by
    sign().  With n_neg workers negative, sum = M - 2 n_neg.
    """
    m_workers = len(bits_per_worker)
    n_neg = np.zeros(count, dtype=np.int64)
    for words in bits_per_worker:
        n_neg += unpack_bits(words, count).astype(np.int64)
    return np.sign(m_workers - 2 * n_neg).astype(np.int8)


def update_vote(w_values, v, lr: float, wdtype: str) -> np.ndarray:
    """W <- rnd_W(fp32(W) - fp32(lr) * V), V in {-1, 0, +1}.

    [SignMuon-ja] section 2, algorithm flow step 4: W_{t+1} = W_t - eta_t *
    S_bar_t.  lr*V is exact in float32, so the only roundings are the
    float32 subtraction and, for bf16 weights, RNE to bfloat16.
    Returns float64 values exactly representable in the weight dtype.
    """
    w32 = np.asarray(w_values, dtype=np.float64).astype(np.float32)
    step = np.float32(lr) * np.asarray(v).astype(np.float32)
    out32 = (w32 - step).astype(np.float32)
    if wdtype == F32:
        return out32.astype(np.float64)
    return f32_from_bf16_bits(bf16_bits_from_f32(out32)).astype(np.float64)


def update_polar(w_values, d_values, lr: float, wdtype: str) -> np.ndarray:
    """W <- rnd_W(fp32(W) - fp32(fp32(lr) * D)) for a dense direction D.

    [CacheMuon-ja] problem statement: Muon replaces the momentum step by the
    orthogonalised direction; [LionMuon-pt] problem statement: W <- W - eta *
    msign(G_hat).  D is taken as stored (its storage dtype); the product and
    the difference are each rounded to float32.
    """
    w32 = np.asarray(w_values, dtype=np.float64).astype(np.float32)
    d32 = np.asarray(d_values, dtype=np.float64).astype(np.float32)
    step = (np.float32(lr) * d32).astype(np.float32)
    out32 = (w32 - step).astype(np.float32)
    if wdtype == F32:
        return out32.astype(np.float64)
    return f32_from_bf16_bits(bf16_bits_from_f32(out32)).astype(np.float64)


# --------------------------------------------------------------------------
# CacheMuon fidelity diagnostic: spectral distance of the cached direction
# --------------------------------------------------------------------------

def spectral_norm_power(e, v0, iters: int) -> float:
    """Power-iteration estimate of ||E||_2 (the largest singular value).

    [CacheMuon-ja] theoretical analysis: the deviation of the cached direction
    from the exact one is measured in the spectral norm, ||D_hat - D||_sp <=
    delta_t.  The estimate follows the plain power method on E^T E from the
    given start vector v0 (length n): v <- v0 / ||v0||; then `iters` times
    y = E v, z = E^T y, v = z / ||z|| (stopping at v = 0 if z = 0); the
    result is ||E v||.  It never exceeds ||E||_2 and reaches it as iters
    grows when v0 is not orthogonal to the top right singular vector.
    """
    e = np.asarray(e, dtype=np.float64)
    v = np.asarray(v0, dtype=np.float64).reshape(-1)
    nv = math.sqrt(float(v @ v))
    if nv == 0.0:
        return 0.0
    v = v / nv
    for _ in range(iters):
        z = e.T @ (e @ v)
        nz = math.sqrt(float(z @ z))
        if nz == 0.0:
            return 0.0
        v = z / nz
    y = e @ v
    return math.sqrt(float(y @ y))


def cache_fidelity(y, q, p: NSParams, v0, iters: int):
    """The diagnostic for one matrix: (err, distance) of a cached Q on Y.

    [CacheMuon-ja] core mechanism items 2-3 and the diagnostic findings of the
    experiments: the residual err of the cached candidate D_hat = Q X, and the
    spectral distance of D_hat from the fresh solve's direction on the same
    X, ||D_hat - D_fresh||_sp (estimated by the power method above), whose
    relation to err is what the pages report on.  X = Y / (||Y||_F + eps) in
    the wide orientation; the distance is taken on the difference in Y's own
    orientation (m x n), so v0 has n entries.
    """
    x, tr = orient(y)
    x = frobenius_normalize(x, p.eps)
    cand = cache_reuse_oriented(q, x)
    fresh, _ = gram_ns_fresh_oriented(x, p)
    diff = cand - fresh
    if tr:
        diff = diff.T
    return orth_residual(cand), spectral_norm_power(diff, v0, iters)


# --------------------------------------------------------------------------
# The int8 encoding, and the optional local polar step on the vote
# --------------------------------------------------------------------------

ENC_BITS = 0
ENC_INT8 = 1


def sign_int8(x) -> np.ndarray:
    """a7 in the int8 encoding: one signed byte per entry, s in {-1, +1}.

    [SignMuon-ja] section 2, algorithm flow step 3 (the integer SUM all-reduce
    variant) and "communication efficiency": instead of one packed bit, each
    entry's sign travels as an int8 (8 bits per entry, 4x fewer bytes than
    float32).  Same sign convention as the bit path: -1 iff x < 0.
    """
    return sign_values(np.asarray(x).reshape(-1))


def vote_from_int8(signs_per_worker: Sequence[np.ndarray], count: int) -> np.ndarray:
    """Majority vote from int8 signs: the integer sum over workers (what the
    SUM all-reduce hands every worker), then sign() with 0 on ties.

    [SignMuon-ja] section 2, core mechanism item 3 and algorithm flow step 4.
    """
    total = np.zeros(count, dtype=np.int64)
    for sv in signs_per_worker:
        total += np.asarray(sv, dtype=np.int64).reshape(-1)[:count]
    return np.sign(total).astype(np.int8)


def vote_polar_direction(v, p: NSParams) -> np.ndarray:
    """Optional local polar step on the aggregated sign matrix V (m x n).

    [SignMuon-ja] section 2, algorithm flow step 5, and [SignMuon-abs]: after
    the vote a worker may take a local polar step on the voted sign matrix,
    pushing the update toward orthogonality at no extra communication.
    Reading (the pages give no formula): the polar factor is approximated by
    the same Newton-Schulz iteration, coefficients and Frobenius
    normalisation as the workers' own directions, D = NS(V / (||V||_F + eps)),
    and the update is the dense one, W <- W - eta * D.  V = 0 gives D = 0.
    """
    return ns_polar(np.asarray(v, dtype=np.float64), p, normalize=True)


# --------------------------------------------------------------------------
# Whole steps (trajectory references)
# --------------------------------------------------------------------------

SIGN_MUON = 0
CACHE_MUON = 1
LION_MUON = 2
UPDATE_VOTE = 0
UPDATE_POLAR = 1


@dataclass
class StepConfig:
    algo: int = SIGN_MUON
    update: int = UPDATE_VOTE
    workers: int = 1
    wdtype: str = F32      # weight storage
    mdtype: str = F32      # momentum storage (also the NS operand dtype)
    lr: float = 1e-3
    beta1: float = 0.9     # single-EMA beta, or Lion's interpolation beta1
    beta2: float = 0.99    # Lion's buffer beta2
    period: int = 0        # LionMuon P (0 = infinity)
    ns: NSParams = field(default_factory=NSParams)
    gamma: float = 0.0
    cache_mode: int = MODE_TRIGGER
    encoding: int = ENC_BITS   # how the signs travel: packed bits or int8
    vote_polar: bool = False   # W <- W - lr * NS(V) instead of W - lr * V


@dataclass
class MatrixState:
    w: np.ndarray                      # m x n, values in wdtype
    mom: List[np.ndarray]              # per worker m x n, values in mdtype
    cache: List[CacheState] = field(default_factory=list)


def _direction_storage(d, cfg: StepConfig) -> np.ndarray:
    return round_storage(d, cfg.mdtype)


def step_matrix(st: MatrixState, grads: Sequence[np.ndarray], cfg: StepConfig, t: int):
    """One optimizer step of one weight matrix with cfg.workers workers.

    Returns a dict with the per-worker directions ('d'), packed bits ('bits'),
    int8 signs ('signs8'), the vote ('vote'), the polar direction of the vote
    ('vote_d', with vote_polar) and CacheMuon diagnostics; `st` is updated in
    place.
    Momentum and directions are rounded to their storage dtype between
    stages, the way a stored tensor is.
    """
    mw = cfg.workers
    assert len(grads) == mw and len(st.mom) == mw
    m, n = st.w.shape
    count = m * n
    out = {"d": [None] * mw, "bits": [None] * mw, "signs8": [None] * mw, "err": [],
           "refreshed": [], "vote_d": None}
    if cfg.algo == CACHE_MUON and not st.cache:
        st.cache = [CacheState() for _ in range(mw)]

    muon_step = True
    if cfg.algo == LION_MUON:
        muon_step = lion_muon_is_muon_step(t, cfg.period)

    for k in range(mw):
        g = np.asarray(grads[k], np.float64)
        if cfg.algo == LION_MUON:
            m_prev = st.mom[k]
            y = lion_interp(m_prev, g, cfg.beta1)
            st.mom[k] = round_storage(lion_momentum(st.mom[k], g, cfg.beta2), cfg.mdtype)
            if not muon_step:
                # Lion step: the exact sign of the interpolation.
                out["d"][k] = y
                neg = lion_sign_negative(m_prev, g, cfg.beta1).reshape(-1)
                out["bits"][k] = pack_bits(neg)
                out["signs8"][k] = np.where(neg, -1, 1).astype(np.int8)
                continue
            y = round_storage(y, cfg.mdtype)
        else:
            st.mom[k] = round_storage(ema(st.mom[k], g, cfg.beta1), cfg.mdtype)
            y = st.mom[k]
        if cfg.algo == CACHE_MUON:
            d, err, refr = cache_muon_direction(y, st.cache[k], t, cfg.ns, cfg.gamma,
                                                cfg.cache_mode)
            out["err"].append(err)
            out["refreshed"].append(refr)
        else:
            d = ns_polar(y, cfg.ns, normalize=True)
        d = _direction_storage(d, cfg)
        out["d"][k] = d
        out["bits"][k] = sign_pack(d)
        out["signs8"][k] = sign_int8(d)

    if cfg.update == UPDATE_POLAR and muon_step:
        assert mw == 1
        st.w = update_polar(st.w, out["d"][0], cfg.lr, cfg.wdtype)
        out["vote"] = None
        return out
    if cfg.encoding == ENC_INT8:
        v = vote_from_int8(out["signs8"], count).reshape(m, n)
    else:
        v = vote_from_bits(out["bits"], count).reshape(m, n)
    out["vote"] = v
    if cfg.vote_polar:
        dv = round_storage(vote_polar_direction(v, cfg.ns), cfg.mdtype)
        out["vote_d"] = dv
        st.w = update_polar(st.w, dv, cfg.lr, cfg.wdtype)
    else:
        st.w = update_vote(st.w, v, cfg.lr, cfg.wdtype)
    return out
