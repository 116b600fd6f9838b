"""MI355X-native balanced expert-parallel hot path: plan -> zero-copy dispatch ->
weighted combine -> replica-gradient reduce, as HIP kernels behind a C ABI
(include/moonep.h, libmoonep.so), with a thin ctypes binding."""

from .moonep import (moonep_query, moonep_plan, moonep_plan_noalloc, moonep_dispatch,  # noqa: F401
                     moonep_combine,
                     moonep_reduce_grad, moonep_plan_status, moonep_dispatch_bwd,
                     moonep_combine_bwd, moonep_prefetch_weight, moonep_expert_stub,
                     moonep_dispatch_staged, moonep_combine_staged, Plan,
                     Sizes, MoonepError, lib, LIB_PATH, EXPORTS)
