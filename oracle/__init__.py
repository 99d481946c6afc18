"""CPU oracle for per-ubatch attention over a cell-granular F16 KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (``ubatch_attention_paged_amd``): every step here is restated
from the source pages in plain, slow numpy (fp64 for the attention) so that a
reader can check it against the pages by eye.

Sources (cited by page title and section throughout):

* "llama.cpp and the ubatch" (joelfernandes.org, 2026-08-14)
* "Batch、Ubatch 与解码主循环" (jonathanding.github.io, llm-learning #4)
* "What does llama.cpp's KV cache actually look like in memory?"
  (joelfernandes.org, 2026-10-05)
* "Iteration-Level Batching: Reforming the Batch at Every Token"
  (mercemay.com), cited as "Iteration-Level Batching"

Modules:

* ``batching``  -- parameter clamps, batch validation/auto-fill, split_simple,
  split_equal, output_ids.
* ``kvcache``   -- cell table, placement, commit, n_kv padding, KQ mask, F16
  store rounding, cache byte sizes and address arithmetic.
* ``attention`` -- masked-softmax grouped-query attention in fp64 (the plain
  definition) and an explicit-loop brute force over the token history.
* ``engine``    -- the decode loop that strings the above together.
* ``scheduler`` -- the iteration-level batching loop (retire, admit under
  token and cache budgets, assemble, advance; preemption by recompute).
* ``seqstate``  -- save / restore of one sequence's cached K/V in the record
  layout of the .bin dump.

Pinned against the pages' worked numbers, closed forms, brute force, a
library special case and invariants in ``tests/test_oracle_*.py``.
"""

from .batching import (clamp_params, fill_batch, split_simple, split_equal,
                       split_batch, split_seq, output_ids, SplitError)
from .kvcache import (CellTable, f16_round, row_bytes, cache_bytes,
                      k_elem_offset, N_PAD_FLOOR, MASK_VISIBLE, MASK_HIDDEN)
from .attention import masked_attention, brute_force_attention
from .engine import OracleEngine

__all__ = [
    "clamp_params", "fill_batch", "split_simple", "split_equal", "split_seq", "split_batch",
    "output_ids", "SplitError", "CellTable", "f16_round", "row_bytes",
    "cache_bytes", "k_elem_offset", "N_PAD_FLOOR", "MASK_VISIBLE", "MASK_HIDDEN",
    "masked_attention", "brute_force_attention", "OracleEngine",
]
