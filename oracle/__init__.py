"""Plain, slow, fp64 CPU oracle for the DeltaLog decode path.

TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the CPU
baseline leg of the benchmark may import anything under this directory; the
product path (the HIP library and its binding) never does, and the two share
no code.  The only thing both sides read is the seeded input generator in the
separate `inputs` package, which holds no recurrence arithmetic.

Modules:
  recurrences  eager dense recurrences (GDN, KDA, RWKV6), one step on all states
  deferred     base + bounded-log model of one state, with the merge schedule
  drive        loops over a seeded workload, and the relative-error measure
"""
from .recurrences import eager_step, gdn_step, kaczmarz_beta, kda_step, rwkv6_step  # noqa: F401
from .deferred import DeferredTile, round_to_bf16  # noqa: F401
from .drive import deferred_tiles, elem_rel_err, rel_err, run_deferred, run_eager, step_arrays  # noqa: F401
