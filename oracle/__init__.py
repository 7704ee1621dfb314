"""CPU oracle for probe-scored KV-cache compression and decode.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, fp64 restatement of
what the compression path computes, written from the pages (GraceKV project
page; DistillCache paper) step by step. Only the tests, the smoke check of
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
The GPU library never calls it, and it shares no code with the GPU library:
the only thing both sides consume is the seeded input generator in
``workload/``, which holds none of the method's arithmetic.

Conventions
-----------
* Every stage takes its inputs in the boundary dtypes (bf16/fp32 tensors,
  fp32 scores) and converts them exactly to float64; all arithmetic inside a
  stage is float64. Quantities that feed an integer decision downstream (token
  relevance, head sensitivity, operation utilities) are emitted as float32,
  which is also how the GPU library hands them from stage to stage.
* Stage functions operate on whole tensors in the layouts of the C ABI
  (documented in include/kvc.h) and loop over (sequence, layer, KV head) units.

Parity status of each function is stated in its docstring; every function
is pinned by a CPU test in tests/test_oracle_pins.py or
tests/test_oracle_pins_slips.py (the latter also plants plausible slips in the
oracle and checks that the pin fails) unless it says "parity unpinned".
"""
from .common import (regions, budgets, rope, rope_inv, to64, bf16_round,  # noqa: F401
                     round_to)
from .score import probe_scores  # noqa: F401
from .propagate import propagate  # noqa: F401
from .partition import (turning_score, slot_costs, dp_slots, fixed_slots,  # noqa: F401
                        slots_for)
from .trees import build_trees, tree_nodes  # noqa: F401
from .select import floor_select, auction, token_topk  # noqa: F401
from .pack import pack  # noqa: F401
from .decode import decode_step, decode_all, full_view  # noqa: F401
from .kl import kl_rows  # noqa: F401
from .pipeline import run_pipeline  # noqa: F401
