"""CPU float64 oracle for static KV-cache decode.

TEST INFRASTRUCTURE ONLY. This package is the slow, obviously correct
reference that the HIP path is checked against. Only the test suite, the
smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the product library never does, and this
package imports nothing from the product package (``static_kv_cache_amd``).

Everything here follows the four web pages on the subject directly:

* "KV-Cache Mechanics" (DantinoX documentation) -- static per-layer cache,
  memory formula, prefill/decode with ``cache_index``, disabling the cache.
* "Key-value cache" (AI Atlas lesson record) -- payload estimate and the
  per-token growth equation.
* "KV Cache Optimization: GQA Audit, In-Place Buffers, Persistent Prompts"
  -- the ``[B, nKvHeads, T, headDim]`` layout, in-place slice-assign append,
  reads sliced to the valid length, byte examples, saving the live prefix.
* "10.3 - KV cache implementation details" -- the exact byte formula and
  its variants (MQA, GQA, MLA, quantised), the decode loop (append, then
  single-query softmax attention over the cache), block tables and shared
  prefixes.

Modules
-------
cache_bytes   byte accounting (pinned to the pages' printed examples)
codec         bf16 / fp32 stored-bit decoding to float64
buffer        bit-exact model of the static cache buffer and its append
attention     decode attention (plain definition) and no-cache causal attention
mla           latent (MLA) decode, materialised and absorbed forms
quant         int8 storage with a float32 scale per row: codes, dequantisation, the cache model
paged         block-table layout: pools of fixed-size blocks, append and gather through tables
persist       the live-prefix image: save (pack) and load (unpack, shared prefixes)

Parity status: every function here has a pin in ``tests/test_oracle_*.py``
(printed worked examples, closed forms, invariants, library routines);
there is no function marked "parity unpinned".
"""

from . import cache_bytes, codec, buffer, attention, mla  # noqa: F401
