"""CPU oracle for dual-flow shared-KV decode -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 implementation of what the decode step computes, used
to check the GPU library. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the library never does, and the
oracle imports nothing from the library. It shares no code with the GPU path:
it decodes bf16 bit patterns itself and rounds to bf16 with its own routine.

Sources (web pages on arXiv 2608.12385, "Dual-Flow Transformers"):

* [DFT-pt] "Resumo Técnico: Dual-Flow Transformers" (gist.science, Portuguese
  technical summary). Sections "Arquitetura Central", "Mecanismos Chave",
  "Custos de Inferência vs. Treinamento".
* [DFT-news] "Dual-Flow Transformers: separando prefill e decode para reduzir
  custo" (omapapaper.com.br), section "O que aconteceu".

Modules:

* ``formats``   -- bf16/fp32 decoding and float64 -> bf16 round-to-nearest-even.
* ``attention`` -- exact softmax attention of both flows over the primary cache.
* ``layer``     -- one full dual-flow decoder layer at one decode step.
* ``brute``     -- scalar pure-Python versions of both, for tiny inputs.

Readings where the pages are silent (all pinned only to this stated choice,
"parity unpinned" with respect to the paper itself):

* query coupling: ``q2' = q2 + a * q1`` elementwise, a of shape [Hq, D];
* MLP couplings: ``z2' = z2 + b * z1`` on the SwiGLU product (the input of the
  down projection) and ``m2' = m2 + c * m1`` on the MLP output;
* no masking beyond the context length, no RoPE, no normalisation, no biases;
  query head h reads kv head ``h // (Hq / Hkv)``; scale ``1 / sqrt(D)``.
"""
