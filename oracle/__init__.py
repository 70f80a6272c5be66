"""Reference oracle for paged single-token decode attention (TEST INFRASTRUCTURE).

This package is a plain, slow, obviously-correct CPU model of what the paged
decode path computes, written in float64 numpy. It exists only to check the
HIP library: the test suite, the package's smoke check and the CPU-baseline
leg of the benchmark may import it; the library and its Python binding never
do, and nothing here imports the library or shares code with it.

Sources (web pages; cited by tag and section throughout this package):
  [SMTS] "Sub-Millisecond Token Scheduling: Inside Disaggregated KV-Cache
         Paging for Frontier LLMs" (factnode.online)
  [LLMI] "LLM inference: prefill, decode, KV cache" (systemcraft.online,
         lesson c03)
  [MTKV] "Architecting Multi-Tier Disaggregated KV-Cache Hierarchies for
         Terabyte-Scale LLM Inference" (ultrainstinct.tech)

Modules:
  fp8_e4m3     -- OCP FP8 E4M3FN decode / round-to-nearest-even saturating encode
  fp4_e2m1     -- FP4 E2M1 decode / round-to-nearest-even saturating encode,
                  two codes per byte
  bf16         -- exact widening of bfloat16 bit patterns
  paged        -- gather through block tables, dense decode attention, split-K
                  partials and their merge, slot mapping, kv_append, CoW copy,
                  multi-token-query attention, shared-prefix (cascade)
                  attention, swap-out / swap-in of blocks
  block_manager-- host block allocator model (ref counts, copy-on-write, swap,
                  radix prefix cache with LRU eviction)
  sizing       -- KV-cache byte closed form and the capacity model

Pin status (what each function is checked against in tests/, CPU only):
  every public function has at least one pin that is not a retyping of its
  own formula: closed forms, values the pages print, special cases with known
  answers, library routines (torch's bfloat16 / float8 conversions and
  scaled_dot_product_attention), exhaustive comparison and invariants. No
  function is "parity unpinned". Outputs at sizes the brute-force pins cannot
  reach come from `paged.decode_attention` itself, which those pins cover.
  tests/test_oracle_mutations.py plants 33 plausible mistakes in these
  modules, one at a time, and requires the pins to fail on each.
"""

from . import bf16, fp8_e4m3, fp4_e2m1, paged, block_manager, sizing  # noqa: F401
