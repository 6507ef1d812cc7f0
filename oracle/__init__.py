"""Plain CPU oracle for paged attention -- TEST INFRASTRUCTURE ONLY.

This package is the slow, obviously-correct reference the HIP path is checked
against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it; the library and its Python binding never
do, and nothing here calls into them.  It shares no code with the HIP path.

Everything is NumPy in float64 unless a format fixes the precision.  Each
function cites the passage of the pages it follows:

* the vLLM encyclopedia article (itwiki "vLLM"), section "PagedAttention",
  sub-sections "Block table" and "Block-wise attention" (the block-sum
  formula and the remark that it equals ordinary attention);
* the vLLM 0.25 Model Runner V2 article (llm-wiki), section "Redesign 3"
  (block tables and slot mapping survive the kernel rewrite) and
  "Redesign 4" (query_start_loc, seq_lens, slot mapping as step inputs);
* the vLLM V1 article (techknowgenie), "Dynamic Chunked Prefill" (decode and
  prompt chunks share one step) and "FP8 KV cache quantization";
* the itwiki "vLLM" article's sections on block sharing with copy-on-write
  and on scheduling and preemption (whole-block copies, ``blocks``);
* the llm-wiki article's "Redesign 1", "Redesign 3" and "Redesign 4" (step
  inputs from persistent request slots and staged block-table writes,
  ``metadata``).

Pins: every function is checked in ``tests/test_oracle_*.py`` against
something other than itself (library casts, brute force, closed forms,
invariants the pages state).  No function here is "parity unpinned".
"""

from . import codecs, cache, attention, blocks, metadata  # noqa: F401
