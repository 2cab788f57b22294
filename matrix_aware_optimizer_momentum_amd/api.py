"""torch-tensor front end of libsm: same names as the C ABI, marshalling only.

Tensors must be CUDA (HIP) tensors, contiguous, float32 or bfloat16 unless
stated otherwise.  Work is enqueued on torch's current stream.  Non-OK
status codes raise SmError.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import torch

from . import _binding as B

_DT = {torch.float32: B.F32, torch.bfloat16: B.BF16}
_TORCH_DT = {B.F32: torch.float32, B.BF16: torch.bfloat16}


@dataclass
class NSParams:
    iters: int = 5
    a: float = 1.5
    b: float = -0.5
    c: float = 0.0
    eps: float = 1e-7

    def c_struct(self) -> B.NSParams:
        return B.NSParams(self.iters, self.a, self.b, self.c, self.eps)


@dataclass
class StepConfig:
    algo: int = B.SIGN_MUON
    update: int = B.UPDATE_VOTE
    M: int = 1
    wdt: torch.dtype = torch.float32
    mdt: torch.dtype = torch.float32
    gdt: torch.dtype = torch.float32
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.99
    period: int = 0
    ns: NSParams = field(default_factory=NSParams)
    gamma: float = 0.0
    cache_mode: int = B.MODE_TRIGGER
    encoding: int = B.ENC_BITS
    vote_polar: bool = False

    def c_struct(self) -> B.Config:
        return B.Config(self.algo, self.update, self.M, _DT[self.wdt], _DT[self.mdt],
                        _DT[self.gdt], self.lr, self.beta1, self.beta2, self.period,
                        self.ns.c_struct(), self.gamma, self.cache_mode, self.encoding,
                        int(self.vote_polar))


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"dtype {t.dtype} not supported (float32 / bfloat16)")
    return _DT[t.dtype]


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _expect(t: torch.Tensor, name: str, shape=None, dtype=None, min_numel=None, dev=True):
    """Shape / dtype / size check of a caller tensor before its pointer
    crosses the C ABI (which sees only raw pointers and cannot check sizes);
    then (dev) that it is a contiguous GPU tensor."""
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} must hold at least {min_numel} elements, has {t.numel()}")
    if dev:
        _dev(t, name)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ws(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError("workspace too small")
        return ws
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _bmn(x: torch.Tensor):
    if x.dim() == 2:
        return 1, x.shape[0], x.shape[1]
    if x.dim() == 3:
        return x.shape[0], x.shape[1], x.shape[2]
    raise ValueError("expected [m, n] or [batch, m, n]")


# ------------------------------------------------------------------ sm_ns_polar

def ns_polar_ws(dtype: torch.dtype, batch: int, m: int, n: int) -> int:
    out = ctypes.c_size_t(0)
    B.check(B.lib().sm_ns_polar_ws(_DT[dtype], batch, m, n, ctypes.byref(out)), "sm_ns_polar_ws")
    return out.value


def ns_polar(x: torch.Tensor, out: Optional[torch.Tensor] = None, normalize: bool = True,
             params: Optional[NSParams] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    _dev(x, "x")
    batch, m, n = _bmn(x)
    p = params or NSParams()
    out = torch.empty_like(x) if out is None else out
    _expect(out, "out", x.shape, x.dtype)
    ws = _ws(ns_polar_ws(x.dtype, batch, m, n), x.device, ws)
    cp = p.c_struct()
    code = B.lib().sm_ns_polar(x.data_ptr(), out.data_ptr(), _dt(x), batch, m, n,
                               int(normalize), ctypes.byref(cp), ws.data_ptr(),
                               ws.numel() * ws.element_size(), _stream())
    B.check(code, "sm_ns_polar")
    return out


def ns_polar_noalloc(x: torch.Tensor, out: Optional[torch.Tensor] = None,
                     normalize: bool = True, params: Optional[NSParams] = None) -> torch.Tensor:
    """sm_ns_polar on the library's fixed scratch (no workspace argument).
    With out given, nothing is allocated here either."""
    _dev(x, "x")
    batch, m, n = _bmn(x)
    p = params or NSParams()
    out = torch.empty_like(x) if out is None else out
    _expect(out, "out", x.shape, x.dtype)
    cp = p.c_struct()
    code = B.lib().sm_ns_polar_noalloc(x.data_ptr(), out.data_ptr(), _dt(x), batch, m, n,
                                       int(normalize), ctypes.byref(cp), _stream())
    B.check(code, "sm_ns_polar_noalloc")
    return out


# ------------------------------------------------------------------ sm_gram_ns_cached

def gram_ns_cached_ws(dtype: torch.dtype, batch: int, m: int, n: int) -> int:
    out = ctypes.c_size_t(0)
    B.check(B.lib().sm_gram_ns_cached_ws(_DT[dtype], batch, m, n, ctypes.byref(out)),
            "sm_gram_ns_cached_ws")
    return out.value


def gram_ns_cached(x: torch.Tensor, q: torch.Tensor, cache_state: torch.Tensor, t: int,
                   gamma: float, mode: int = B.MODE_TRIGGER, normalize: bool = True,
                   params: Optional[NSParams] = None, d: Optional[torch.Tensor] = None,
                   err: Optional[torch.Tensor] = None, refreshed: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None):
    """Returns (d, err, refreshed); q and cache_state are updated in place."""
    _dev(x, "x")
    batch, m, n = _bmn(x)
    r = min(m, n)
    if q.dtype != torch.float32 or q.numel() != batch * r * r:
        raise ValueError("q must be float32 [batch, r, r]")
    if cache_state.dtype != torch.int32 or cache_state.numel() != 2 * batch:
        raise ValueError("cache_state must be int32 [batch, 2]")
    _dev(q, "q"); _dev(cache_state, "cache_state")
    p = params or NSParams()
    d = torch.empty_like(x) if d is None else d
    err = torch.empty(batch, dtype=torch.float32, device=x.device) if err is None else err
    refreshed = (torch.empty(batch, dtype=torch.int32, device=x.device)
                 if refreshed is None else refreshed)
    _expect(d, "d", x.shape, x.dtype)
    _expect(err, "err", dtype=torch.float32, min_numel=batch)
    _expect(refreshed, "refreshed", dtype=torch.int32, min_numel=batch)
    ws = _ws(gram_ns_cached_ws(x.dtype, batch, m, n), x.device, ws)
    cp = p.c_struct()
    code = B.lib().sm_gram_ns_cached(x.data_ptr(), d.data_ptr(), q.data_ptr(),
                                     cache_state.data_ptr(), err.data_ptr(),
                                     refreshed.data_ptr(), _dt(x), batch, m, n, int(normalize),
                                     ctypes.byref(cp), gamma, mode, t, ws.data_ptr(),
                                     ws.numel() * ws.element_size(), _stream())
    B.check(code, "sm_gram_ns_cached")
    return d, err, refreshed


# ------------------------------------------------------------------ sign / vote

def sign_pack(x: torch.Tensor, bits: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Packed signs as an int64 tensor holding the uint64 words."""
    _dev(x, "x")
    count = x.numel()
    words = (count + 63) // 64
    bits = torch.empty(max(words, 1), dtype=torch.int64, device=x.device) if bits is None else bits
    _expect(bits, "bits", dtype=torch.int64, min_numel=words)
    code = B.lib().sm_sign_pack(x.data_ptr(), _dt(x), count, bits.data_ptr(), _stream())
    B.check(code, "sm_sign_pack")
    return bits


def vote_update(bits: torch.Tensor, w: torch.Tensor, lr: float,
                vote_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bits: int64 [M, words_stride]; w updated in place; returns w."""
    _dev(bits, "bits"); _dev(w, "w")
    if bits.dtype != torch.int64 or bits.dim() != 2:
        raise ValueError("bits must be int64 [M, words_stride]")
    M, stride = bits.shape
    if stride * 64 < w.numel():
        raise ValueError("bits rows hold fewer than w.numel() signs")
    vp = 0
    if vote_out is not None:
        _dev(vote_out, "vote_out")
        if vote_out.dtype != torch.int8 or vote_out.numel() != w.numel():
            raise ValueError("vote_out must be int8 with w's element count")
        vp = vote_out.data_ptr()
    code = B.lib().sm_vote_update(bits.data_ptr(), M, stride, w.numel(), w.data_ptr(), _dt(w),
                                  lr, vp, _stream())
    B.check(code, "sm_vote_update")
    return w


def sign_int8(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int8 signs (-1 iff x < 0, else +1) of x's elements, flat [numel]."""
    _dev(x, "x")
    out = torch.empty(x.numel(), dtype=torch.int8, device=x.device) if out is None else out
    if out.dtype != torch.int8 or out.numel() < x.numel():
        raise ValueError("out must be int8 with at least x.numel() elements")
    code = B.lib().sm_sign_int8(x.data_ptr(), _dt(x), x.numel(), out.data_ptr(), _stream())
    B.check(code, "sm_sign_int8")
    return out


def vote_update_int8(signs: torch.Tensor, w: torch.Tensor, lr: float,
                     vote_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """signs: int8 [M, stride] (stride >= w.numel()); w updated in place; returns w."""
    _dev(signs, "signs"); _dev(w, "w")
    if signs.dtype != torch.int8 or signs.dim() != 2:
        raise ValueError("signs must be int8 [M, stride]")
    M, stride = signs.shape
    if stride < w.numel():
        raise ValueError("signs rows hold fewer than w.numel() signs")
    vp = 0
    if vote_out is not None:
        _dev(vote_out, "vote_out")
        if vote_out.dtype != torch.int8 or vote_out.numel() != w.numel():
            raise ValueError("vote_out must be int8 with w's element count")
        vp = vote_out.data_ptr()
    code = B.lib().sm_vote_update_int8(signs.data_ptr(), M, stride, w.numel(), w.data_ptr(),
                                       _dt(w), lr, vp, _stream())
    B.check(code, "sm_vote_update_int8")
    return w


def vote(signs: torch.Tensor, count: int, out: torch.Tensor) -> torch.Tensor:
    """The vote V in {-1, 0, +1} written to out ([count] float32/bfloat16).
    signs: int64 [M, words_stride] packed bits, or int8 [M, stride] signs."""
    _dev(signs, "signs"); _dev(out, "out")
    if signs.dim() != 2 or signs.dtype not in (torch.int64, torch.int8):
        raise ValueError("signs must be int64 (packed bits) or int8, shape [M, stride]")
    enc = B.ENC_BITS if signs.dtype == torch.int64 else B.ENC_INT8
    M, stride = signs.shape
    if out.numel() < count:
        raise ValueError("out is smaller than count")
    if stride * (64 if enc == B.ENC_BITS else 1) < count:
        raise ValueError("signs rows hold fewer than count signs")
    code = B.lib().sm_vote(signs.data_ptr(), enc, M, stride, count, out.data_ptr(), _dt(out),
                           _stream())
    B.check(code, "sm_vote")
    return out


def polar_update(w: torch.Tensor, d: torch.Tensor, lr: float) -> torch.Tensor:
    """w <- rnd(w - lr * d) in place (d has w's element count); returns w."""
    _dev(w, "w"); _dev(d, "d")
    if d.numel() != w.numel():
        raise ValueError("d must have w's element count")
    code = B.lib().sm_polar_update(w.data_ptr(), _dt(w), d.data_ptr(), _dt(d), w.numel(), lr,
                                   _stream())
    B.check(code, "sm_polar_update")
    return w


def spectral_norm(a: torch.Tensor, b: Optional[torch.Tensor], v0: torch.Tensor,
                  iters: int, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Power-method ||a - b||_2 per problem (b None: ||a||_2).

    a, b: [batch, m, n] or [m, n] (same dtype); v0: float32 [batch, n] start
    vectors.  Returns float32 [batch]."""
    _dev(a, "a"); _dev(v0, "v0")
    batch, m, n = _bmn(a)
    if b is not None:
        _dev(b, "b")
        if b.shape != a.shape or b.dtype != a.dtype:
            raise ValueError("b must match a in shape and dtype")
    if v0.dtype != torch.float32 or v0.numel() != batch * n:
        raise ValueError("v0 must be float32 with batch * n entries")
    out = torch.empty(batch, dtype=torch.float32, device=a.device)
    need = ctypes.c_size_t(0)
    B.check(B.lib().sm_spectral_norm_ws(batch, m, n, ctypes.byref(need)), "sm_spectral_norm_ws")
    ws = _ws(need.value, a.device, ws)
    code = B.lib().sm_spectral_norm(a.data_ptr(), b.data_ptr() if b is not None else None,
                                    _dt(a), batch, m, n, v0.data_ptr(), iters, out.data_ptr(),
                                    ws.data_ptr(), ws.numel() * ws.element_size(), _stream())
    B.check(code, "sm_spectral_norm")
    return out


# ------------------------------------------------------------------ sm_step

@dataclass
class MatrixBuffers:
    """Caller-owned state of one weight matrix (all on the GPU)."""
    w: torch.Tensor                       # [m, n]
    mom: torch.Tensor                     # [M, m, n]
    grad: torch.Tensor                    # [M, m, n]
    q_cache: Optional[torch.Tensor] = None      # [M, r, r] float32 (CacheMuon)
    cache_state: Optional[torch.Tensor] = None  # [M, 2] int32 (CacheMuon)

    def c_struct(self) -> B.Matrix:
        m, n = self.w.shape
        return B.Matrix(m, n, self.w.data_ptr(), self.mom.data_ptr(), self.grad.data_ptr(),
                        self.q_cache.data_ptr() if self.q_cache is not None else None,
                        self.cache_state.data_ptr() if self.cache_state is not None else None)


def _check_mats(cfg: StepConfig, mats: Sequence[MatrixBuffers], diag: Optional[torch.Tensor]):
    """Every tensor of every matrix has the shape and dtype the configuration
    implies (the library reads and writes them through raw pointers), and
    is a contiguous GPU tensor."""
    if len(mats) == 0:
        raise ValueError("a step needs at least one matrix")
    tensors = []
    for j, mb in enumerate(mats):
        if mb.w.dim() != 2:
            raise ValueError(f"matrix {j}: w must be [m, n]")
        m, n = mb.w.shape
        r = min(m, n)
        want = [(mb.w, "w", None, cfg.wdt), (mb.mom, "mom", (cfg.M, m, n), cfg.mdt),
                (mb.grad, "grad", (cfg.M, m, n), cfg.gdt)]
        if cfg.algo == B.CACHE_MUON:
            if mb.q_cache is None or mb.cache_state is None:
                raise ValueError(f"matrix {j}: CacheMuon needs q_cache and cache_state")
            want += [(mb.q_cache, "q_cache", (cfg.M, r, r), torch.float32),
                     (mb.cache_state, "cache_state", (cfg.M, 2), torch.int32)]
        for t, name, shape, dtype in want:
            _expect(t, f"matrix {j} {name}", shape, dtype, dev=False)
            tensors.append((t, f"matrix {j} {name}"))
    if diag is not None:
        _expect(diag, "diag", dtype=torch.float32, min_numel=len(mats) * cfg.M * 2, dev=False)
        tensors.append((diag, "diag"))
    for t, name in tensors:
        _dev(t, name)


def _mats_array(mats: Sequence[MatrixBuffers]):
    arr = (B.Matrix * len(mats))()
    for i, mb in enumerate(mats):
        arr[i] = mb.c_struct()
    return arr


def step_ws(cfg: StepConfig, mats: Sequence[MatrixBuffers]) -> int:
    out = ctypes.c_size_t(0)
    c = cfg.c_struct()
    arr = _mats_array(mats)
    B.check(B.lib().sm_step_ws(ctypes.byref(c), arr, len(mats), ctypes.byref(out)), "sm_step_ws")
    return out.value


class StepCall:
    """A prepared sm_step call: marshalled structs and a workspace, reusable per step."""

    def __init__(self, cfg: StepConfig, mats: Sequence[MatrixBuffers],
                 ws: Optional[torch.Tensor] = None, diag: Optional[torch.Tensor] = None):
        _check_mats(cfg, mats, diag)
        self.cfg = cfg
        self.mats = list(mats)
        self._c = cfg.c_struct()
        self._arr = _mats_array(self.mats)
        nbytes = step_ws(cfg, self.mats)
        self.ws = _ws(nbytes, self.mats[0].w.device, ws)
        self.diag = diag

    def __call__(self, t: int):
        code = B.lib().sm_step(ctypes.byref(self._c), self._arr, len(self.mats), t,
                               self.ws.data_ptr(), self.ws.numel() * self.ws.element_size(),
                               self.diag.data_ptr() if self.diag is not None else None,
                               _stream())
        B.check(code, "sm_step")


def step(cfg: StepConfig, mats: Sequence[MatrixBuffers], t: int,
         ws: Optional[torch.Tensor] = None, diag: Optional[torch.Tensor] = None):
    StepCall(cfg, mats, ws, diag)(t)


class StepGraph:
    """sm_step at step index t, recorded once as a HIP graph (sm_step_graph)
    and replayed on the current stream by each call (sm_graph_launch).

    The matrices' buffers, the workspace and diag are bound at recording and
    must stay in place while the graph lives.  A LionMuon step's type follows
    t: record one graph at a Muon step and one at a Lion step (they may share
    a workspace).  CacheMuon is not recordable (SmError SM_ERR_UNSUPPORTED).
    """

    def __init__(self, cfg: StepConfig, mats: Sequence[MatrixBuffers], t: int,
                 ws: Optional[torch.Tensor] = None, diag: Optional[torch.Tensor] = None):
        self._h = None
        self._call = StepCall(cfg, mats, ws, diag)   # holds the buffers and the workspace
        c = self._call
        h = ctypes.c_void_p()
        code = B.lib().sm_step_graph(ctypes.byref(c._c), c._arr, len(c.mats), t,
                                     c.ws.data_ptr(), c.ws.numel() * c.ws.element_size(),
                                     c.diag.data_ptr() if c.diag is not None else None,
                                     ctypes.byref(h))
        B.check(code, "sm_step_graph")
        self._h = h
        self.t = t

    @property
    def ws(self) -> torch.Tensor:
        return self._call.ws

    def __call__(self):
        if self._h is None:
            raise RuntimeError("StepGraph: replay after close()")
        B.check(B.lib().sm_graph_launch(self._h, _stream()), "sm_graph_launch")

    def close(self):
        """Destroys the graph once every replay enqueued so far has finished."""
        if self._h is not None:
            h, self._h = self._h, None
            torch.cuda.synchronize(self._call.ws.device)
            B.check(B.lib().sm_graph_destroy(h), "sm_graph_destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------------ kernel accounting

def mfma_ceiling(out: torch.Tensor, blocks: int, iters: int, mode: int = 1,
                 src: Optional[torch.Tensor] = None) -> int:
    """Enqueue the MFMA ceiling probe (sm_mfma_ceiling) on the current stream;
    returns the flops it executes.  `out` is a float32 device tensor of at
    least blocks * 256 entries; mode 2 reads `src` (a device tensor whose
    byte size is a power of two from 64 KB to 64 MB)."""
    _expect(out, "out", dtype=torch.float32, min_numel=blocks * 256)
    sp, sb = None, 0
    if mode == 2:
        if src is None:
            raise ValueError("mode 2 needs a source buffer")
        _dev(src, "src")
        sp, sb = ctypes.c_void_p(src.data_ptr()), src.numel() * src.element_size()
    B.check(B.lib().sm_mfma_ceiling(int(mode), blocks, iters, sp, sb,
                                    ctypes.c_void_p(out.data_ptr()), _stream()),
            "sm_mfma_ceiling")
    return blocks * 4 * iters * 16 * 32768


def profile_enable(on: bool = True):
    B.check(B.lib().sm_profile_enable(int(on)), "sm_profile_enable")


def profile_reset():
    B.check(B.lib().sm_profile_reset(), "sm_profile_reset")


def profile_read(kind: str):
    """(total_ms, launches, algorithmic work) for one kernel kind; waits on its events."""
    k = B.KERNEL_KINDS.index(kind)
    ms, n, work = ctypes.c_double(0), ctypes.c_int64(0), ctypes.c_double(0)
    B.check(B.lib().sm_profile_read(k, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(work)),
            "sm_profile_read")
    return ms.value, n.value, work.value


def profile_read_bytes(kind: str) -> float:
    """Algorithmic HBM bytes of one kernel kind (operands read once, outputs written once)."""
    k = B.KERNEL_KINDS.index(kind)
    b = ctypes.c_double(0)
    B.check(B.lib().sm_profile_read_bytes(k, ctypes.byref(b)), "sm_profile_read_bytes")
    return b.value
