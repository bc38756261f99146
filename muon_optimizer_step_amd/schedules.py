"""Host-side schedules that feed muon_step per call (no device work).

"Record: L_ParallelResiduals_UNetSkips_DepthRecur_Muon_ 1.0901" (PR #1893),
table "Architecture and training stack", Optimizer row: Muon momentum 0.99,
warmed up from 0.92 over the first 1500 steps.  The library takes the momentum
as a per-call scalar and the Newton-Schulz coefficients as a per-call table,
so both schedules live here, on the host.
"""

from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

STANDARD_QUINTIC = (3.4445, -4.7750, 2.0315)


def muon_momentum(step: int, *, start: float = 0.92, end: float = 0.99, warmup_steps: int = 1500) -> float:
    """Momentum for training step `step` (counted from 0).

    Reading taken (the page gives the endpoints and the length only): linear in
    the step count from `start` at step 0 to `end` at step `warmup_steps`, and
    `end` from then on.
    """
    if step < 0:
        raise ValueError(f"step = {step} must be >= 0")
    if warmup_steps <= 0 or step >= warmup_steps:
        return float(end)
    frac = step / warmup_steps
    return float((1.0 - frac) * start + frac * end)


def ns_coefficients(ns_steps: int, table: Optional[Sequence[Sequence[float]]] = None) -> List[Tuple[float, float, float]]:
    """The per-iteration (a, b, c) table for muon_step.

    With `table`, its rows drive the iterations in order and it must hold
    exactly ns_steps rows (a per-step schedule such as Polar Express; the pages
    do not print its values).  Without it, every iteration uses the standard
    quintic (3.4445, -4.7750, 2.0315).
    """
    if ns_steps < 0:
        raise ValueError(f"ns_steps = {ns_steps} must be >= 0")
    if table is None:
        return [STANDARD_QUINTIC] * ns_steps
    rows = [tuple(float(v) for v in row) for row in table]
    if len(rows) != ns_steps or any(len(r) != 3 for r in rows):
        raise ValueError(f"table must hold {ns_steps} rows of (a, b, c)")
    return rows
