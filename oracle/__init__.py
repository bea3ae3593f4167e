"""CPU oracle for paged MLA decode.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call, link
or execute this package: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use it. It shares no code with the HIP library; the only
module both sides read is ``mla_inputs`` (seeded input draws, no attention
arithmetic).

Contents
  mla_oracle  naive expand-then-attend decode (the plain definition), the
              absorbed form used to pin it, split/merge and the streaming
              online-softmax recurrence.
  split_plan  integer model of the split-KV work plan (which pages each
              workgroup slot covers), pinned by coverage invariants.

Every function is pinned by a CPU test; none is "parity unpinned".
"""
from . import kv_quant, mla_oracle, split_plan  # noqa: F401
