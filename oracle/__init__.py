"""Plain CPU oracle for DeepSeek-V4 indexer-Q preparation.

TEST INFRASTRUCTURE ONLY. This package is the slow, obviously-correct reference
that the HIP path is checked against. Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it; the product library never does,
and this package imports nothing from the product library.

What it computes (numpy, float64 unless a step fixes another precision):

* ``quant_fp8``   packed-UE8M0 FP8 1x128 activation quantization
  (tokenspeed PR "perf(deepseek-v4): accelerate indexer Q and packed FP8
  quantization", Summary and Risk and fallback).
* ``indexer_q``   block-scaled FP8 Q projection, RoPE on each head's rope slice,
  128-point Hadamard rotation, FP4 e2m1 quantization with UE8M0 block scales
  (same page, Summary; TensorRT-LLM PR "Fuse DeepSeek-V4 Indexer Q projection
  with CuTe DSL", sequence diagram and Description / Paths compared).
* ``formats``     OCP OFP8 E4M3, OCP MX E2M1 and E8M0 encodings, written from the
  public OCP format definitions.
* ``checker``     the acceptance rule that compares a device result with the
  oracle's.

Every function is pinned by tests against something other than itself
(closed forms, brute force, a library cast, invariants); none is
"parity unpinned".
"""
