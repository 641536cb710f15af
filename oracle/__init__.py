"""CPU oracle for paged decode attention.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, calls or links anything here, and this
package imports nothing from the product path: the two share no kernels,
headers, helpers, tables or constants.

What it is: a plain, slow, obviously correct numpy implementation of what the
hot path computes, in float64 wherever the arithmetic is the method's own.

Sources (page titles as published; sections named on each page):

* "KV cache & continuous batching" (docs.masst.dev, ai/inference/kv-cache-batching)
  - section "KV cache memory math": the per-token KV byte formula, GQA/MQA head counts;
  - section "Visual: the lifecycle of a request in continuous batching": 16-token
    blocks, blocks per request;
  - section "2. PagedAttention (vLLM)": per-request block table mapping logical
    positions to physical blocks; the attention kernel gathers K and V through it;
  - section "The core insight": decode computes Q for the new token only and
    attends over every cached K and V;
  - section "5. Speculative decoding": the target verifies the drafted tokens in
    one pass at length current + K.
* "LLM Serving - KV Cache, Batching, Speculative Decoding" (dineshblog.com, session 124)
  - section "KV memory, paging and prefix identity": the byte formula's symbols
    and its worked 512 KiB / 1 GiB / 16 GiB example; physical blocks may be shared;
  - section "Hands-on: cache equivalence and scheduling oracles": cached decode
    equals the last row of full causal attention (the pin in the tests).
* "LLM Inference Optimization: KV Cache, Batching, and Speculative Decoding"
  (adaptiverecall.com) - section "Memory Bandwidth Optimization": decode reads
  the whole cache per token; KV quantization to one byte per element.

Modules
-------
``kv_math``   byte and block arithmetic the pages print (pinned by their numbers).
``fp8``       OCP E4M3 codec written from the format definition.
``int8``      symmetric int8 codec (round half to even, saturate to +-127).
``int4``      symmetric int4 codec (saturate to +-7), two codes per byte.
``pool``      host model of the pool byte layout: slot mapping, cache write, gather.
``attention`` float64 softmax attention over gathered K/V: decode and k-row verify.

Pins (what ties each function to something other than itself) live in
``tests/test_oracle_*.py``.  Every function here has at least one pin; see the
docstrings.
"""

from . import kv_math, fp8, int8, int4, pool, attention  # noqa: F401
