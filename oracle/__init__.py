"""CPU oracle for KV-cache attention: plain, slow, obviously correct, fp64.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
link anything under this package; only the test-suite, the smoke check and
the CPU-baseline leg of the benchmark do.  It shares no code with the HIP
library: its inputs are plain numpy arrays holding the same bytes the GPU
receives.

Sources (cited by short key in every function of this package):
  [P1] "KV Cache, Flash Attention and Inference Optimization"
       (factory.pai-world.com lesson)
  [P2] "KV Cache Fully Explained: The Core of LLM Inference Memory"
       (techblog.paldyn.com)
  [P3] "KV Cache" (heepie.pages.dev concept note)
  [P4] "Transformer Attention Masks and KV-Cache Inference"
       (c86j224s.github.io interview note)

Modules:
  codec      - storage formats -> fp64 (fp32, bf16, OCP FP8 E4M3FN) and the
               E4M3FN encoder used by the fp8 cache
  attention  - scaled dot-product attention by its definition, decode,
               prefill, the running (max, sum) tiled route, split-K merge
  cache      - logical KV cache with the append contract, physical pool
               prediction for contiguous / 16-token paged layouts, byte
               closed forms, op counts
  paging     - block-table batch/beam reorder, block copies, a reference
               block pool (free list, reference counts, copy-on-write) and
               the contiguous vs paged reserved-memory closed forms
  pool       - runs the functions above over host processes (shared-memory
               inputs) to time the oracle on many cores; no arithmetic

Every function is pinned by tests/test_oracle_pins.py and
tests/test_oracle_paging.py against values the
pages print, closed forms, library routines or brute force.  Parity pinned
everywhere; no function here is "parity unpinned".
"""
from . import codec, attention, cache, paging  # noqa: F401  (pool is imported on demand)
