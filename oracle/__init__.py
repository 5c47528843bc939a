"""CPU oracle for the Flint-shaped W4A16 MoE layer -- TEST INFRASTRUCTURE.

A plain, slow, float64 NumPy statement of what the decode MoE layer computes,
written from the pages that describe it ("Day-0 Support for Flint on vLLM",
its Spanish translation, and the arex-research write-up of the same
release).  It exists to check the HIP path and nothing else:

* only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
  ``bench.py`` may import it;
* it shares no code with the HIP path (``w4a16_moe_decode_amd``) and never
  imports it; the two meet only in the seeded generators of ``gen/``;
* the product path never falls back to it.

Modules:
  formats  E2M1 / UE4M3 value definitions and the source super-block decode
  bf16     float64 -> bfloat16 round-to-nearest-even
  moe      RMSNorm, router + sigmoid top-k, SwiGLU expert, combine, the
           decode layer, dense MLP, the multi-layer decode step, prefill
  attn     per-head Q/K RMSNorm, rotate-half RoPE and the KV-cache write
           of an attention layer's projected heads; decode attention with
           learned sinks over a sliding window or the whole context

Parity pins (tests/test_oracle_*.py) tie every function to something other
than itself.  Parity against values printed on the pages is unpinned: the
pages print no worked numerical example of the layer.
"""
from . import attn, bf16, formats, moe  # noqa: F401
