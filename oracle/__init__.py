"""Float64 CPU oracle for the Muon optimizer step and the batched weight EMA.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``muon_optimizer_step_amd``) never imports, calls or links it, and this package
imports nothing from the product path.

See ``oracle/muon.py`` for the method and its citations.
"""

from .muon import (  # noqa: F401
    EPS,
    momentum_update,
    row_normalize,
    frobenius_normalize,
    newton_schulz,
    orthogonalize,
    shape_scale,
    apply_update,
    muon_step_matrix,
    ema_update,
)
