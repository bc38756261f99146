"""Seeded synthetic workloads shared by the oracle side and the GPU side.

This module only draws inputs (weights, gradients, momentum buffers, EMA
shadows, coefficient tables) and describes their shapes.  It holds none of the
optimizer's arithmetic.  Every array is drawn in float64 with NumPy's PCG64
(``default_rng``) and cast to float32 once, so the oracle and the GPU library
receive bit-identical inputs.

Shapes follow "Record: L_ParallelResiduals_UNetSkips_DepthRecur_Muon_ 1.0901"
(PR #1893), table "Architecture and training stack": 11 layers, width 512,
8 query heads and 4 KV heads (head dim 64), MLP 4x, 34,401,372 parameters,
SP4096 vocabulary, value embeddings of dimension 128.  The Muon matrix set per
layer is Q, K, V, O, MLP up and MLP down in PyTorch (out x in) layout.

The parameter list for the EMA is a reading: the page gives only the total, so
the list is the 66 matrices, a 4096 x d token embedding, a 4096 x 128 value
embedding, 118 gain/scale vectors of length d and one vector of length 92,
which sums to exactly 34,401,372 at d = 512.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

# Quintic coefficient triple used for every NS step unless a table is drawn.
# The pages name a per-step schedule (PR #1396, "Techniques Combined", Polar
# Express row) but print no values; this is the commonly used Muon triple.
STANDARD_TRIPLE = (3.4445, -4.7750, 2.0315)

# Seeds the pages run with (PR #1584 "Results"; PR #1893 "Results").
PRIMARY_SEED = 1337
ROBUST_SEEDS = (42, 2024)

PAGE_PARAM_COUNT_512 = 34_401_372  # PR #1893, "Architecture and training stack", Parameters row


def layer_shapes(d: int, kv_heads: int, head_dim: int = 64, mlp_mult: int = 4):
    """(name, rows, cols) of one transformer layer's Muon matrices, out x in."""
    kv = kv_heads * head_dim
    return [
        ("q", d, d),
        ("k", kv, d),
        ("v", kv, d),
        ("o", d, d),
        ("up", mlp_mult * d, d),
        ("down", d, mlp_mult * d),
    ]


def extra_param_shapes(d: int, vocab: int = 4096, ve_dim: int = 128,
                       n_vectors: int = 118, tail: int = 92):
    """Non-matrix parameters touched only by the EMA (reading, see module doc)."""
    shapes = [("tok_emb", (vocab, d)), ("value_emb", (vocab, ve_dim))]
    shapes += [(f"vec{i}", (d,)) for i in range(n_vectors)]
    shapes.append(("tail", (tail,)))
    return shapes


@dataclass
class Workload:
    name: str
    matrices: List[Tuple[str, int, int]]
    extras: List[Tuple[str, Tuple[int, ...]]]
    lr: float
    momentum: float
    nesterov: bool
    weight_decay: float
    row_norm: bool
    ns_steps: int
    ns_precision: int            # 0 = bf16 MFMA, 1 = fp32
    ema_decay: Optional[float]   # None: no EMA in this workload
    steps: int = 1
    weight_std: float = 0.02
    grad_std: float = 1.0
    mom_std: float = 0.0         # 0: zero initial momentum
    structured_rank: int = 0     # >0: gradient = rank-r outer products + noise
    noise_std: float = 0.0
    jitter_coeffs: bool = False  # draw the per-step table around the triple
    description: str = ""

    @property
    def n_matrix_elems(self) -> int:
        return sum(r * c for _, r, c in self.matrices)

    @property
    def n_params(self) -> int:
        return self.n_matrix_elems + sum(int(np.prod(s)) for _, s in self.extras)


def _model_matrices(d: int, kv_heads: int, layers: int = 11):
    out = []
    for layer in range(layers):
        for nm, r, c in layer_shapes(d, kv_heads):
            out.append((f"l{layer}.{nm}", r, c))
    return out


def workload(cfg: int) -> Workload:
    """The five workloads, numbered 0..4."""
    if cfg == 0:
        return Workload(
            name="single512_fp32ns", matrices=[("w", 512, 512)], extras=[],
            lr=0.022, momentum=0.99, nesterov=True, weight_decay=0.0, row_norm=False,
            ns_steps=5, ns_precision=1, ema_decay=None, grad_std=1.0, mom_std=0.0,
            description="one 512x512 matrix, N(0,1) gradient, zero momentum, fp32 NS")
    if cfg == 1:
        return Workload(
            name="layer512", matrices=[(f"l0.{n}", r, c) for n, r, c in layer_shapes(512, 4)],
            extras=[], lr=0.022, momentum=0.99, nesterov=True, weight_decay=0.105,
            row_norm=True, ns_steps=5, ns_precision=0, ema_decay=None,
            grad_std=1e-3, mom_std=1e-3,
            description="one layer's six matrices at d=512, bf16 NS")
    if cfg == 2:
        return Workload(
            name="model11L512", matrices=_model_matrices(512, 4), extras=extra_param_shapes(512),
            lr=0.022, momentum=0.99, nesterov=True, weight_decay=0.105, row_norm=True,
            ns_steps=5, ns_precision=0, ema_decay=0.9965, grad_std=1e-3, mom_std=1e-3,
            description="66 matrices of the 11L 512d model + EMA over 34,401,372 params")
    if cfg == 3:
        return Workload(
            name="model11L1024", matrices=_model_matrices(1024, 8), extras=extra_param_shapes(1024),
            lr=0.03, momentum=0.97, nesterov=True, weight_decay=0.105, row_norm=True,
            ns_steps=5, ns_precision=0, ema_decay=0.997, grad_std=1e-3, mom_std=1e-3,
            description="66 matrices of an 11L 1024d model + EMA over all params")
    if cfg == 4:
        return Workload(
            name="structured512", matrices=_model_matrices(512, 4), extras=extra_param_shapes(512),
            lr=0.022, momentum=0.99, nesterov=True, weight_decay=0.105, row_norm=True,
            ns_steps=4, ns_precision=0, ema_decay=0.9965, steps=10, mom_std=0.0,
            structured_rank=8, noise_std=1e-2, jitter_coeffs=True,
            description="rank-8 + noise gradients, 4 NS steps with a drawn table, 10 steps")
    raise ValueError(f"unknown workload {cfg}")


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def _normal32(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float64)
    if std != 1.0:
        x *= std
    return x.astype(np.float32)


def coeff_table(w: Workload, seed: int) -> np.ndarray:
    """(ns_steps, 3) float32 coefficient table."""
    base = np.array([STANDARD_TRIPLE] * w.ns_steps, dtype=np.float64).reshape(w.ns_steps, 3)
    if w.jitter_coeffs:
        rng = _rng(seed, 0xC0EF)
        base = base * (1.0 + rng.uniform(-0.05, 0.05, size=base.shape))
    return base.astype(np.float32)


def make_state(w: Workload, seed: int):
    """Initial weights, momentum buffers and EMA shadows (float32, C-contiguous).

    Returns dict(params=[matrices..., extras...], moms=[one per matrix],
    ema=[one per param]).  The EMA starts as a copy of the weights.
    """
    streams = np.random.SeedSequence(seed).spawn(len(w.matrices) + len(w.extras))
    params, moms = [], []
    for i, (_, r, c) in enumerate(w.matrices):
        rng = np.random.default_rng(streams[i])
        params.append(_normal32(rng, (r, c), w.weight_std))
        if w.mom_std > 0:
            moms.append(_normal32(rng, (r, c), w.mom_std))
        else:
            moms.append(np.zeros((r, c), dtype=np.float32))
    for j, (_, shape) in enumerate(w.extras):
        rng = np.random.default_rng(streams[len(w.matrices) + j])
        params.append(_normal32(rng, shape, w.weight_std))
    ema = [p.copy() for p in params] if w.ema_decay is not None else []
    return {"params": params, "moms": moms, "ema": ema}


def make_grads(w: Workload, seed: int, step: int = 0) -> List[np.ndarray]:
    """Gradients of the Muon matrices for one step (float32)."""
    out = []
    for i, (_, r, c) in enumerate(w.matrices):
        rng = _rng(seed, 0x6AD, step, i)
        if w.structured_rank > 0:
            k = w.structured_rank
            u = rng.standard_normal(size=(r, k))
            v = rng.standard_normal(size=(c, k))
            g = u @ v.T + w.noise_std * rng.standard_normal(size=(r, c))
            out.append(g.astype(np.float32))
        else:
            out.append(_normal32(rng, (r, c), w.grad_std))
    return out


# AdamW on the non-matrix parameters ("Architecture and training stack", Optimizer
# row, PR #1893, names the optimizer and nothing else).  Reading: the library
# defaults of torch.optim.AdamW; the step counter is past the first steps so
# that both bias corrections are live (0.9^1000 is negligible, 0.999^1000 is not).
ADAMW_HPARAMS = {"lr": 1e-3, "beta1": 0.9, "beta2": 0.999, "eps": 1e-8, "weight_decay": 0.01, "step": 1000}


def make_adamw_state(w: Workload, seed: int, step: int = 0):
    """Gradients and AdamW moments of the non-matrix parameters (float32).

    exp_avg ~ N(0, grad_std^2); exp_avg_sq is the square of an independent
    N(0, grad_std^2) draw (non-negative, as the second moment always is).
    """
    grads, m1, m2 = [], [], []
    for j, (_, shape) in enumerate(w.extras):
        rng = _rng(seed, 0xADA, step, j)
        grads.append(_normal32(rng, shape, w.grad_std))
        m1.append(_normal32(rng, shape, w.grad_std))
        m2.append(np.square(_normal32(rng, shape, w.grad_std)))
    return {"grads": grads, "exp_avg": m1, "exp_avg_sq": m2}


def make_independent_ema(w: Workload, seed: int) -> List[np.ndarray]:
    """EMA shadows drawn independently of the weights (so no element is trivial)."""
    out = []
    shapes = [(r, c) for _, r, c in w.matrices] + [s for _, s in w.extras]
    for i, shape in enumerate(shapes):
        out.append(_normal32(_rng(seed, 0xE3A, i), shape, w.weight_std))
    return out


def small_ragged_matrices() -> List[Tuple[str, int, int]]:
    """Odd shapes that leave ragged tails in every tiling (wide, tall, square)."""
    return [("a", 33, 65), ("b", 130, 70), ("c", 1, 300), ("d", 257, 129),
            ("e", 96, 96), ("f", 200, 1), ("g", 128, 384), ("h", 300, 520)]
