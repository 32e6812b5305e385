"""Plain fp64 CPU reference of the causal GQA attention path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the entry
module and the CPU-baseline leg of the benchmark may import this package.  The
library under ``gqa_causal_flash_amd`` never imports it, and this package never
imports the library: the two share no code.  The seeded input generators live
in ``workloads`` (which holds none of the attention arithmetic) and feed both.

What is computed, in the notation of the pages (Hq query heads sharing Hkv K/V
heads, head dim D, softmax scale, causal positions):

* ``prefill_causal`` -- dense causal GQA prefill, softmax(scale*Q K^T + causal
  mask) V, as named in the purpose section of the long-prefill page
  ("[Kernel][SM70] Default long-prefill GQA architecture", Purpose: causal FP16
  Q=8000, KV=40000..128000, Hq=6, Hkv=1, D=256, scale 1/16).
* ``prefill_paged_sparse`` -- the same attention over the union of selected
  four-token blocks fetched through a page table, with stale slots at or past
  the live length clamped away ("[Kernel][SM70] Repair #378 on latest main",
  Changes: four-token block selection, locality-sorted pages, clamp to live
  request length, partial tail admitted only for real tokens).
* ``prefill_causal_varlen`` -- a batch of independent causal prefills packed
  end to end (per-sequence offsets), each with its queries at the last
  positions of its keys.
* ``verify_fp8kv`` -- a short causal verifier tail (2..8 query rows) over a K/V
  cache stored as OCP E4M3 bytes with one fp32 scale per tensor ("[Perf] Ship
  the qualified SM70 long-context layout...", What / Changes: grouped E4M3 FP32
  long-context operator, verifier tail query_rows 2..8).
* ``prefill_causal_e4m3`` -- the dense causal prefill with Q, K and V all given
  as E4M3 codes and one fp32 scale per tensor: the quantised-Q definition of an
  E4M3-cache long prefill whose Q K^T products run on FP8 matrix cores (same
  page, What: grouped E4M3 FP32 long-context operator).
* ``e4m3_decode`` -- the OCP 8-bit E4M3 ("E4M3FN") format definition.

Every function returns unrounded float64 outputs together with the per-row
log-sum-exp, so tests can compare a GPU fp16 result against exact values.
Parity pins for each function live in ``tests/test_oracle_pins.py``.
"""

from .attention import (
    attend,
    causal_visible,
    kv_head_of,
    prefill_causal,
    prefill_causal_e4m3,
    prefill_causal_varlen,
    prefill_paged_sparse,
    verify_fp8kv,
    visible_pairs_causal,
)
from .e4m3 import e4m3_decode, e4m3_table

__all__ = [
    "attend",
    "causal_visible",
    "kv_head_of",
    "prefill_causal",
    "prefill_causal_e4m3",
    "prefill_causal_varlen",
    "prefill_paged_sparse",
    "verify_fp8kv",
    "visible_pairs_causal",
    "e4m3_decode",
    "e4m3_table",
]
