"""fp64 CPU oracle for RoPE + grouped-query causal/cross-document attention.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package; the product path (the C-ABI library and its Python binding) never
does. The oracle shares no code with the HIP path: it takes its inputs from the
``workloads`` package (seeded draws only) and computes everything else itself.

Sources (the web pages this library is built from):

* "Llama 3.1 Architecture: Dense Scaling to 405B and 128K Context",
  section "Context Expansion: From 8K to 128K via RoPE Frequency Scaling",
  subsection "1. High Base Frequency": the RoPE frequency bands
  theta_k = theta_base^(-2k/d), k in [0, d/2 - 1]; flowchart in "Architectural
  Deep Dive": 128 query heads over 8 KV heads (16:1);
* "The Llama 3 Herd of Models", Chapter Roadmap, "A Deliberately Standard Dense
  Transformer": GQA with 8 KV heads, RoPE base 500,000, cross-document mask;
* "How Meta's Llama 3.1 405B Architecture Actually Works", paragraph on GQA:
  several query heads share one key/value head, which shrinks the KV cache
  used while decoding.

Pins: every function here is checked by ``tests/test_oracle_pins.py`` against
brute force (``oracle.brute``), a library routine (PyTorch's
scaled_dot_product_attention in fp64 with complex-number RoPE) and invariants
and closed forms of the method. No function is "parity unpinned".
"""

from .reference import (  # noqa: F401
    attention,
    combine,
    decode,
    decode_partials,
    document_of,
    rope,
    rope_attention,
    rope_frequencies,
)
