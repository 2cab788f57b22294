"""Seeded synthetic workloads: shapes, hyper-parameters and input generators.

Holds none of the method's arithmetic.  Shapes follow the models the pages
train (ResNet-50 convolutions, GPT-2 small / large blocks, a 7B-class
4096 x 11008 block); the pages' datasets are not used -- seeded random
gradient streams with the stated distributions stand in for them.

Seeds: configuration c uses base seed 20261203 + 1000*c; the weights use the
base seed and worker k's gradient stream uses base + 1 + k, drawn step by
step in matrix order.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Iterator, List, Sequence, Tuple

import numpy as np

SIGN_MUON, CACHE_MUON, LION_MUON = 0, 1, 2
UPDATE_VOTE, UPDATE_POLAR = 0, 1


def resnet50_conv_shapes() -> List[Tuple[int, int]]:
    """The 53 ResNet-50 convolutions as (out, in*k*k) matrices (torchvision layout)."""
    shapes = [(64, 3 * 7 * 7)]
    inplanes = 64
    for width, blocks in ((64, 3), (128, 4), (256, 6), (512, 3)):
        out = 4 * width
        for bi in range(blocks):
            shapes.append((width, inplanes))          # 1x1 reduce
            shapes.append((width, width * 9))         # 3x3
            shapes.append((out, width))               # 1x1 expand
            if bi == 0:
                shapes.append((out, inplanes))        # downsample
            inplanes = out
    return shapes


def gpt2_block_shapes(d: int, layers: int) -> List[Tuple[int, int]]:
    """Per layer: qkv (d x 3d), attention out (d x d), fc (d x 4d), fc_out (4d x d)."""
    out = []
    for _ in range(layers):
        out += [(d, 3 * d), (d, d), (d, 4 * d), (4 * d, d)]
    return out


@dataclass
class Workload:
    name: str
    index: int
    algo: int
    update: int
    M: int
    wdt: str
    mdt: str
    gdt: str
    shapes: List[Tuple[int, int]]
    grad_kind: str = "gaussian"   # gaussian | ar1 | student_t
    grad_std: float = 1.0
    ar1_rho: float = 0.99
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.99
    period: int = 0
    ns_iters: int = 5
    ns_a: float = 1.5
    ns_b: float = -0.5
    ns_c: float = 0.0
    ns_eps: float = 1e-7
    gamma: float = 2.0
    cache_mode: int = 0
    steps: int = 10
    notes: str = ""

    @property
    def seed(self) -> int:
        return 20261203 + 1000 * self.index

    @property
    def params(self) -> int:
        return sum(m * n for m, n in self.shapes)

    def ns_flops_per_step(self, muon_step: bool = True) -> float:
        """NS flops per step of the direct iteration, counted as the kernels count them.

        Per cubic iteration and problem the two products are 2 r^2 c each
        (+2 r^3 for the quintic term).  The bf16 path computes the symmetric
        Gram product X X^T (and A^2) as one triangle, so it is credited with
        half of it: 3 r^2 c (+ r^3).  The f32 path computes full products.
        The library runs far-from-square cubic problems in the Gram form,
        which reaches the same X_K with fewer flops; this is the direct
        form's count, a reference figure, not the work done.
        """
        if not muon_step or self.algo == CACHE_MUON:
            return 0.0
        sym = self.mdt == "bf16"
        tot = 0.0
        for m, n in self.shapes:
            r, c = min(m, n), max(m, n)
            gram = (1.0 if sym else 2.0) * r * r * c
            quint = ((1.0 if sym else 2.0) * r ** 3) if self.ns_c != 0 else 0.0
            tot += (gram + 2.0 * r * r * c + quint) * self.ns_iters * self.M
        return tot

    def scaled(self, layers_fraction: float = None, shapes=None, **kw) -> "Workload":
        """A copy with fewer matrices (parity cases that the oracle finishes quickly)."""
        d = dict(self.__dict__)
        if shapes is not None:
            d["shapes"] = list(shapes)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    1: Workload("sign_muon_256x256_fp32_M3", 1, SIGN_MUON, UPDATE_VOTE, 3, "f32", "f32", "f32",
                [(256, 256)], "gaussian", 1.0, steps=10,
                notes="single fp32 256x256 matrix, N(0,1) gradients, 10 steps"),
    2: Workload("gpt2_small_sign_muon_bf16_M5", 2, SIGN_MUON, UPDATE_VOTE, 5, "bf16", "bf16",
                "bf16", gpt2_block_shapes(768, 12), "gaussian", 1e-2, steps=20,
                notes="12 GPT-2-small layers, bf16 momentum/NS, N(0, 1e-2^2) gradients"),
    3: Workload("resnet50_sign_muon_fp32_M4", 3, SIGN_MUON, UPDATE_VOTE, 4, "f32", "f32", "f32",
                resnet50_conv_shapes(), "gaussian", 1.0, ns_iters=1, steps=10,
                notes="53 ResNet-50 convolutions as (out, in*k*k), 1 NS iteration"),
    4: Workload("gpt2_large_cache_muon_bf16_M1", 4, CACHE_MUON, UPDATE_POLAR, 1, "bf16", "bf16",
                "bf16", gpt2_block_shapes(1280, 36), "ar1", 1e-2, gamma=2.0, steps=100,
                notes="36 GPT-2-large layers, Gram-NS with cached Q, AR(1) gradients"),
    5: Workload("lion_muon_4096_11008_bf16_M16", 5, LION_MUON, UPDATE_VOTE, 16, "bf16", "bf16",
                "bf16", [(4096, 4096)] * 8 + [(4096, 11008)] * 8, "student_t", 1.0,
                beta1=0.9, beta2=0.99, period=4, steps=8,
                notes="8 x 4096^2 + 8 x 4096x11008, LionMuon P=4, Student-t(3) gradients"),
}


# ---------------------------------------------------------------- NumPy generators (parity)

def init_weights(wl: Workload, shapes: Sequence[Tuple[int, int]] = None) -> List[np.ndarray]:
    rng = np.random.default_rng(wl.seed)
    shapes = shapes if shapes is not None else wl.shapes
    return [(0.02 * rng.standard_normal(s)).astype(np.float32) for s in shapes]


def grad_stream(wl: Workload, shapes: Sequence[Tuple[int, int]] = None,
                workers: int = None) -> Iterator[List[np.ndarray]]:
    """Yields, per step, a list over matrices of float32 arrays [M, m, n]."""
    shapes = list(shapes if shapes is not None else wl.shapes)
    mw = workers or wl.M
    rngs = [np.random.default_rng(wl.seed + 1 + k) for k in range(mw)]
    prev = None
    rho = wl.ar1_rho
    while True:
        step = []
        for j, (m, n) in enumerate(shapes):
            per = []
            for k in range(mw):
                if wl.grad_kind == "student_t":
                    g = rngs[k].standard_t(3, size=(m, n))
                else:
                    g = rngs[k].standard_normal((m, n))
                g = wl.grad_std * g
                if wl.grad_kind == "ar1" and prev is not None:
                    g = rho * prev[j][k] + math.sqrt(1 - rho * rho) * g
                per.append(g)
            step.append(np.stack(per).astype(np.float32))
        if wl.grad_kind == "ar1":
            prev = [s.astype(np.float64) for s in step]
        yield step


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 inputs to bfloat16 once (torch's conversion), as float32 values."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .to(torch.float32).numpy()


def as_storage(x: np.ndarray, dt: str) -> np.ndarray:
    """Input arrays as the values a tensor of storage type dt holds."""
    return round_bf16(x) if dt == "bf16" else np.asarray(x, dtype=np.float32)
