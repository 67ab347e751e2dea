"""CPU oracle for the paged KV-cache hot path — TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct restatement of what the
paged KV-cache operations compute, written from the pages on PagedAttention:

* ``codecs``  — storage codes (fp32 / fp16 / bf16 / OCP FP8 E4M3FN) to exact
  float64 values, and the FP8 quantiser used by slot writes.
* ``paged``   — slot-mapped writes, whole-block copies, gathering a sequence's
  keys and values through its block table, and ordinary softmax attention
  over the gathered tokens in float64.
* ``blocks``  — a tiny block manager (free list, block tables, reference
  counts, copy-on-write, swap) used to replay the pages' worked example.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import it. The library under ``paged_kv_cache_44_amd`` never does, and this
package never imports that library: the two share no code. Nothing here is
tuned for speed.
"""

from . import blocks, codecs, paged  # noqa: F401
