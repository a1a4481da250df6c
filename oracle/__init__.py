"""CPU oracle for paged decode attention and the slot-mapped KV append.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (the HIP library under ``paged_kv_cache_187_amd/`` and its Python
binding) never imports, calls or links it, and this package never imports the
product path: the two share no code.  The only module both sides use is the
seeded input generator in ``synth/``, which holds no arithmetic of the method.

Everything here is plain numpy in float64 (bit patterns are decoded by this
package's own codecs), written to be checked by eye against the pages:

* "LLM推理引擎深度实战：从PagedAttention到分布式推理部署" (ybb.press), §2.2 and §2.3:
  the KV cache lives in fixed 16-token pages reached through a per-request page
  table, and the attention kernel translates logical token indices into
  physical page addresses, so that paging does not change what attention
  computes.  §5.3: KV-cache quantisation to FP8 at per-token granularity.
* "大模型推理引擎优化：KV Cache 与连续批处理" (devpress.csdn.net), §2.1 and §2.2: every
  decode step attends over the K/V of all previous tokens; blocks hold 16
  tokens and are allocated on demand.  §4.2: a block that several sequences
  share is copied before one of them writes into it (copy-on-write).  The
  ybb.press page §3.2: preempted requests' pages go to CPU memory and come back.

Pins (tests marked ``not gpu`` under ``tests/``) tie each function to something
other than itself: brute-force dense attention and torch's
``scaled_dot_product_attention`` in float64, block-permutation invariance,
closed-form special cases, hand-derived fixtures under ``tests/golden/``,
torch's own float16 / bfloat16 / float8_e4m3fn conversions, and exhaustive
codec round trips.
"""

from .codecs import (  # noqa: F401
    decode_f16,
    decode_bf16,
    e4m3_table,
    decode_e4m3,
    encode_e4m3,
    decode_bits,
)
from .kv_append import append_kv, quantize_tokens_e4m3, append_kv_e4m3  # noqa: F401
from .block_copy import copy_blocks, swap_blocks  # noqa: F401
from .paged_attention import (  # noqa: F401
    attend,
    attention_weights,
    gather_kv,
    paged_decode,
    paged_decode_multi,
    paged_decode_one,
    partial_attend,
    merge_partials,
)
