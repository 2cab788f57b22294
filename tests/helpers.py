"""Comparison helpers shared by the GPU parity tests (no method arithmetic)."""
import numpy as np
import torch


def to_np(t: torch.Tensor) -> np.ndarray:
    """GPU tensor -> float32 numpy holding exactly the stored values."""
    return t.detach().to(torch.float32).cpu().numpy()


def words_np(bits: torch.Tensor) -> np.ndarray:
    return bits.detach().cpu().numpy().view(np.uint64)


def storage_bits(x: np.ndarray, dt: str) -> np.ndarray:
    """Bit patterns of float32 values that are exact in the storage type."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.int64)
    return (u >> 16) if dt == "bf16" else u


def ordered(bits: np.ndarray, nbits: int) -> np.ndarray:
    """Map IEEE bit patterns to integers ordered like the values."""
    sign = bits >> (nbits - 1)
    mag = bits & ((1 << (nbits - 1)) - 1)
    return np.where(sign == 1, -mag, mag)


def ulp_distance(a: np.ndarray, b: np.ndarray, dt: str) -> np.ndarray:
    nb = 16 if dt == "bf16" else 32
    return np.abs(ordered(storage_bits(a, dt), nb) - ordered(storage_bits(b, dt), nb))


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def tdt(dt: str):
    return torch.bfloat16 if dt == "bf16" else torch.float32


def to_gpu(x: np.ndarray, dt: str, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device).to(tdt(dt))


def storage_ulp(x: np.ndarray, dt: str) -> np.ndarray:
    """Spacing of the storage type at |x| (bf16: 8 significant bits)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    if dt == "f32":
        return np.spacing(a.astype(np.float32)).astype(np.float64)
    _, e = np.frexp(np.maximum(a, 2.0 ** -126))
    return np.ldexp(1.0, e - 8)


def assert_ema_close(gpu, want, m_prev, g, beta, dt, what=""):
    """|gpu - want| <= 1 storage ulp + float32 rounding of the two EMA terms.

    The kernel evaluates beta*m + (1-beta)*g in float32 and stores it in dt;
    when the terms cancel, the float32 error is relative to the terms, not
    to the (small) result.
    """
    gpu = np.asarray(gpu, np.float64)
    want = np.asarray(want, np.float64)
    terms = np.abs(beta * np.asarray(m_prev, np.float64)) + \
        np.abs((1 - beta) * np.asarray(g, np.float64))
    tol = storage_ulp(want, dt) + 2.0 ** -22 * terms
    bad = np.abs(gpu - want) > tol
    assert not np.any(bad), f"{what}: {int(bad.sum())} momentum entries off by more than the bound"


def f32(v: float) -> float:
    """A hyper-parameter as the float32 the C ABI receives."""
    return float(np.float32(v))


def lion_band(m_prev, g, beta1: float) -> np.ndarray:
    """Entries whose Lion sign a float32 evaluation may decide either way.

    G_hat = b*m + (1-b)*g evaluated in float32 (b = fp32(beta1)) carries at
    most a few roundings of the size of its terms, so its sign can differ
    from the exact sign only where |G_hat| <= 2^-22 (|b m| + |(1-b) g|).
    """
    b = np.float64(np.float32(beta1))
    m = np.asarray(m_prev, np.float64)
    g = np.asarray(g, np.float64)
    exact = b * m + (1.0 - b) * g
    return np.abs(exact) <= 2.0 ** -22 * (np.abs(b * m) + np.abs((1.0 - b) * g))


def check_vote_within(v_gpu, v_or, ambiguous, what, max_frac):
    """The vote may differ from the oracle's only where some worker's sign is
    ambiguous (decided by rounding); the fraction of such entries is bounded.
    v_gpu may hold 9 where the update does not tell the vote apart."""
    v_gpu = np.asarray(v_gpu)
    amb = np.any(np.stack([np.asarray(a, bool).reshape(v_gpu.shape) for a in ambiguous]), axis=0)
    known = v_gpu != 9
    mism = known & (v_gpu != np.asarray(v_or).reshape(v_gpu.shape))
    bad = mism & ~amb
    assert not np.any(bad), f"{what}: {int(bad.sum())} vote mismatches outside the rounding band"
    assert mism.mean() <= max_frac, f"{what}: mismatch fraction {mism.mean():.2e}"
    return int(mism.sum())
