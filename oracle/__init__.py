"""CPU oracle for the paged KV-cache hot path — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct statement of what the
GPU path computes.  It exists so that tests, the smoke check and the CPU
baseline leg of the benchmark can compare the HIP kernels against an
independent definition.  The product path never imports it: the Python
binding in ``paged_kv_cache_336_amd`` fails loudly when its HIP library is
missing instead of falling back to anything here.

The oracle shares no code with the HIP path (no kernels, headers, tables or
helpers), and it imports nothing from ``paged_kv_cache_336_amd``.  Inputs
come from the seeded generator module, which holds none of the method's
arithmetic.

Sources (cited by page title and section):

* "PagedAttention" (shubhamtatvamasi.com), section "How attention reads
  paged memory": the pool ``[num_blocks, block_size, kv_heads, head_dim]``,
  the per-sequence block table, the current length, and attention over the
  gathered keys/values.
* Same page, "Sharing and copy-on-write" and its FAQ entry on
  copy-on-write for parallel sampling: the block copy.
* "How PagedAttention Works in vLLM ..." (instagit.com), section
  "write_to_paged_cache: Direct In-Place Updates": the slot-mapped scatter,
  its ``kv_cache_dtype`` and per-tensor ``k_scale``/``v_scale``.
* OCP 8-bit floating point specification (E4M3 "fn" and E5M2 variants):
  the fp8 codecs.

Storage conventions shared with the generator (plain numpy dtypes):
``"f32"`` float32, ``"f16"`` float16, ``"bf16"`` uint16 holding bfloat16
bits, ``"fp8_e4m3"`` / ``"fp8_e5m2"`` uint8 holding OCP E4M3 / E5M2 codes;
fp8 scales per tensor, one per kv head, or one per (token slot, kv head)
in a float32 array shaped like the pool without its head_dim axis.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
something other than itself (library routines, closed forms, brute force
and the pages' worked example).  No function is "parity unpinned".
"""

from .fp8_e4m3 import e4m3_decode, e4m3_encode, E4M3_MAX
from .fp8_e5m2 import e5m2_decode, e5m2_encode, E5M2_MAX
from .storage import to_float64
from .attention import (paged_attention, paged_attention_rows,
                        gather_sequence, attention_one_head)
from .cache_ops import (cache_write, cache_write_token_scales,
                        copy_block_prefixes, copy_blocks, copy_token_scales)
from .multi_query import paged_attention_multi

__all__ = [
    "e4m3_decode",
    "e4m3_encode",
    "E4M3_MAX",
    "e5m2_decode",
    "e5m2_encode",
    "E5M2_MAX",
    "to_float64",
    "paged_attention",
    "paged_attention_rows",
    "gather_sequence",
    "attention_one_head",
    "cache_write",
    "cache_write_token_scales",
    "copy_token_scales",
    "copy_blocks",
    "copy_block_prefixes",
    "paged_attention_multi",
]
