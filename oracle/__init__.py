"""CPU oracle for the per-token NVFP4 routed-MoE path.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, numpy reference of
what the GPU path computes. Only the test suite, the smoke check of the build
entry and the CPU-baseline leg of the benchmark may import it; the product
library never does, and it shares no code with the HIP kernels.

Sources (three public pages; cited by page and section):
  * Megatron-LM pull request 8262, "per-token NVFP4 squared-ReLU and SwiGLU
    MoE via FlashInfer CuTe DSL" -- cited as [Megatron-LM #8262 . <section>].
  * FlashInfer pull request 5019, "CuTe DSL NVFP4 W4A16 MegaMoE" -- cited as
    [FlashInfer #5019 . <section>].

Where the pages leave a step open, the oracle takes one stated reading; each
is tagged R<n> in the docstrings and listed with its justification in the
design notes of the repository.

Modules:
  formats -- E2M1 / E4M3 / BF16 codecs.
  quant   -- per-token activation quantizer, FP32-row requantizer, weight
             quantizer, dequantizers.
  moe     -- gating detection, routing, FC1, activation, FC2, finalize, the
             whole pipeline, and two brute-force references used as pins.
  recipes -- the per-tensor NVFP4 (static calibrated input scales folded into
             the alphas) and weight-only W4A16 (BF16 activations) variants of
             the pipeline [Megatron-LM #8262 . How to extend], and the general
             pipeline with the layer options (SwiGLU clamp, fused finalize).
  layer   -- the router front (top-k, softmax weights), the SwiGLU clamp and
             the fused (order-free) finalize.

Parity pins: every function here is pinned by a CPU test against something
other than itself (hand enumerations, a library cast, brute force, closed
forms, invariants). None is "parity unpinned".
"""
