"""MI355X (gfx950) Muon optimizer step, weight EMA and AdamW for the other parameters.

Thin Python binding over the C ABI of libmuonstep.so (include/muonstep.h):
it only turns torch tensors into device pointers plus the current HIP stream.
Every step of the computation runs in the library's HIP kernels.
"""

from ._lib import (  # noqa: F401
    MUON_NS_BF16, MUON_NS_FP32, MUON_NS_BF16X3, MUON_NS_SCHEDULE_PHASES, MUON_NS_SCHEDULE_CHAIN, MuonError, LIB_PATH,
    load, set_ns_schedule, plan_cache_stats,
)
from .api import (  # noqa: F401
    muon_step, muon_step_static, ema_update, ema_swap, adamw_step, workspace_size, profile_enable, profile_read, version,
    PreparedMuonStep, PreparedEma, PreparedAdamW,
)
