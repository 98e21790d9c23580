"""Seeded synthetic inputs and the workload table for the Sign-Muon step.

This module holds no arithmetic of the method: it only names the workloads
(weight-matrix shapes, worker counts, iteration counts, storage types) and
draws the random gradients and initial weights. Both the GPU path's tests
and benchmark and the CPU oracle's tests take their inputs from here.

The pages evaluate on CIFAR-10 / ResNet-50 and on nanoGPT (GPT-2 small). The
datasets and trained weights are not used: only the models' weight-matrix
shapes are kept, and gradients are seeded i.i.d. draws.

Every draw uses numpy's PCG64 seeded with
``SeedSequence([20260519, workload.seed_id, matrix_index, worker, step])``
(weights: ``[20260519, seed_id, matrix_index, 1_000_000]``). Samples are drawn
in fp64, multiplied by the scale and rounded to fp32 by ``astype``.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple

import numpy as np

ROOT_SEED = 20260519
W_STREAM = 1_000_000


def _gpt2_small_shapes():
    # nanoGPT GPT-2 small (124M): per layer the fused qkv projection, the
    # attention output projection, the MLP up and down projections.
    per_layer = [(768, 2304), (768, 768), (768, 3072), (3072, 768)]
    return tuple(per_layer * 12)


def _resnet50_conv_shapes():
    # Every ResNet-50 convolution weight flattened to (out, in*kh*kw).
    groups = [((64, 147), 1), ((64, 64), 1), ((64, 576), 3), ((256, 64), 4), ((64, 256), 2),
              ((128, 256), 1), ((128, 1152), 4), ((512, 128), 4), ((512, 256), 1),
              ((128, 512), 3), ((256, 512), 1), ((256, 2304), 6), ((1024, 256), 6),
              ((1024, 512), 1), ((256, 1024), 5), ((512, 1024), 1), ((512, 4608), 3),
              ((2048, 512), 3), ((2048, 1024), 1), ((512, 2048), 2)]
    out = []
    for shape, count in groups:
        out.extend([shape] * count)
    return tuple(out)


@dataclass(frozen=True)
class Workload:
    name: str
    seed_id: int
    shapes: Tuple[Tuple[int, int], ...]
    workers: int
    ns_iters: int
    grad_dist: str = "normal"          # "normal" or "student_t3"
    grad_scale: float = 1.0            # standard deviation (normal) or multiplier (t)
    grad_dtype: str = "f32"
    mom_dtype: str = "f32"
    ns_dtype: str = "f32"
    beta: float = 0.9
    eta: float = 1e-3
    w_scale: float = 0.02
    post_polar_iters: int = 0
    norm: str = "frobenius"            # or "spectral" (power iteration on the Gram matrix)
    power_iters: int = 0
    description: str = field(default="", compare=False)

    @property
    def params(self) -> int:
        return int(sum(r * c for r, c in self.shapes))

    def ns_flops(self) -> float:
        """Algorithmic Newton-Schulz flops of one step: per worker, matrix and
        iteration, r^2*c for the symmetric Gram plus 2*r^2*c for the product
        (r = min side, c = max side)."""
        tot = 0
        for r_, c_ in self.shapes:
            r, c = min(r_, c_), max(r_, c_)
            tot += 3 * r * r * c
        return float(tot) * self.workers * self.ns_iters

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "square256_mw4_k1": Workload(
        "square256_mw4_k1", 1, ((256, 256),), workers=4, ns_iters=1, grad_scale=1.0,
        description="one fp32 256x256 weight, 4 workers, grads N(0,1), 1 NS iteration"),
    "resnet50_4shapes_mw4_k1": Workload(
        "resnet50_4shapes_mw4_k1", 2, ((64, 576), (256, 2304), (512, 4608), (2048, 512)),
        workers=4, ns_iters=1, grad_scale=1e-2,
        description="four ResNet-50 conv weights as (out, in*kh*kw), fp32, 4 workers, 1 NS iter"),
    "resnet50_4shapes_mw4_k5": Workload(
        "resnet50_4shapes_mw4_k5", 2, ((64, 576), (256, 2304), (512, 4608), (2048, 512)),
        workers=4, ns_iters=5, grad_scale=1e-2,
        description="four ResNet-50 conv weights, fp32, 4 workers, 5 NS iters"),
    "resnet50_all_convs_mw4_k1": Workload(
        "resnet50_all_convs_mw4_k1", 6, _resnet50_conv_shapes(), workers=4, ns_iters=1,
        grad_scale=1e-2, description="all 53 ResNet-50 conv weights, fp32, 4 workers, 1 NS iter"),
    "gpt2s_mw8_k1": Workload(
        "gpt2s_mw8_k1", 3, _gpt2_small_shapes(), workers=8, ns_iters=1, grad_scale=1e-3,
        mom_dtype="bf16", ns_dtype="bf16",
        description="GPT-2 small 48 matrices (84.9M params), bf16 momentum and NS, fp32 W, "
                    "8 workers, grads N(0,1e-3), 1 NS iter"),
    "gpt2s_mw8_k1_spectral": Workload(
        "gpt2s_mw8_k1_spectral", 3, _gpt2_small_shapes(), workers=8, ns_iters=1, grad_scale=1e-3,
        mom_dtype="bf16", ns_dtype="bf16", norm="spectral", power_iters=8,
        description="as gpt2s_mw8_k1 with spectral scaling of the Newton-Schulz input "
                    "(8 power-iteration steps on the Gram matrix)"),
    "gpt2s_mw16_k5_t3": Workload(
        "gpt2s_mw16_k5_t3", 4, _gpt2_small_shapes(), workers=16, ns_iters=5,
        grad_dist="student_t3", grad_scale=1e-3, mom_dtype="bf16", ns_dtype="bf16",
        description="GPT-2 small, 16 workers (ties possible), 5 NS iters, Student-t(3) grads"),
    "gpt2s_mw16_k5_t3_postpolar": Workload(
        "gpt2s_mw16_k5_t3_postpolar", 4, _gpt2_small_shapes(), workers=16, ns_iters=5,
        grad_dist="student_t3", grad_scale=1e-3, mom_dtype="bf16", ns_dtype="bf16",
        post_polar_iters=5,
        description="as gpt2s_mw16_k5_t3 plus the post-vote local polar step (5 iters)"),
    "block4096_mw16_k5": Workload(
        "block4096_mw16_k5", 5, ((4096, 4096),) * 4 + ((4096, 11008), (11008, 4096)),
        workers=16, ns_iters=5, grad_scale=1e-3, mom_dtype="bf16", ns_dtype="bf16",
        description="large transformer block: 4x 4096x4096, 4096x11008, 11008x4096; bf16 NS, "
                    "16 workers, 5 NS iters"),
}


def rng_for(seed_id: int, *keys: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, seed_id,
                                                                        *keys])))


def draw(rng: np.random.Generator, dist: str, scale: float, shape) -> np.ndarray:
    """fp64 samples times scale, rounded to fp32."""
    if dist == "normal":
        x = rng.standard_normal(shape)
    elif dist == "student_t3":
        x = rng.standard_t(3, shape)
    else:
        raise ValueError(dist)
    return (x * scale).astype(np.float32)


def gradient(wl: Workload, j: int, worker: int, step: int) -> np.ndarray:
    """Gradient of matrix j for one worker at one step, fp32 [R][C]."""
    R, C = wl.shapes[j]
    return draw(rng_for(wl.seed_id, j, worker, step), wl.grad_dist, wl.grad_scale, (R, C))


def gradients(wl: Workload, j: int, step: int) -> np.ndarray:
    """All workers' gradients of matrix j, fp32 [Mw][R][C]."""
    return np.stack([gradient(wl, j, m, step) for m in range(wl.workers)])


def initial_weight(wl: Workload, j: int) -> np.ndarray:
    R, C = wl.shapes[j]
    return draw(rng_for(wl.seed_id, j, W_STREAM), "normal", wl.w_scale, (R, C))


def random_matrix(seed: int, shape, scale: float = 1.0, dist: str = "normal") -> np.ndarray:
    """A free-standing seeded fp32 array for unit tests."""
    return draw(rng_for(0, seed), dist, scale, shape)
