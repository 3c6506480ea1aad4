"""CPU oracle for draft-guided block-sparse mixed-precision attention.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, float64 restatement
of what the method computes, written to check the GPU library against. Only
the test suite, the smoke check of the build entry point and the CPU-baseline
leg of the benchmark may import it. The product path never calls it, and it
shares no code, tables or constants with the HIP sources.

Sources, cited by page title and section:

* [DA2] "DraftAttention2: Fast Video Diffusion with Low-Resolution-Guided
  Mixed-Precision Attention" (arXiv 2609.32628), abstract: a low-resolution
  draft attention map from 2D average- and max-pooled queries and keys scores
  the attention blocks; one shared ranking gives the most important blocks the
  higher precision, the next retained blocks the lower precision and skips the
  rest under configurable budgets; operands are prepared in one fused pass and
  one attention kernel runs precision-specific phases that share data
  movement, softmax statistics and the output accumulator; the precisions are
  4-bit and 8-bit.
* [DA1] "DraftAttention: Fast Video Diffusion via Low-Resolution Attention
  Guidance" (arXiv 2505.14708), abstract: each frame's latent feature map is
  down-sampled, the draft map comes from the draft queries and keys, Q/K/V are
  reordered so that the sparsity is structured for the hardware, and the
  original order is restored after attention.
* [DA1-article] the news write-up of DraftAttention (szmaozhuayin.com),
  method overview, steps 1-4: average pooling over 8x16 windows, draft map,
  top-scoring regions to a mask, token reordering for GPU memory layout.
* [OFP8] OCP 8-bit Floating Point Specification, E4M3 encoding; [OCP-MX] OCP
  Microscaling Formats v1.0, FP4 E2M1 elements and E8M0 shared scales. These
  fix the number formats; the pages only name 8-bit and 4-bit.

Where the pages leave a step open, the reading taken is stated in the
docstring of the function that takes it.

Parity status: every function here is pinned by tests under ``tests/`` that
do not re-derive it (format tables vs. torch's float8_e4m3fn cast and the
format definitions, closed forms, invariants, library softmax attention,
brute force on tiny inputs). The pages' own quality and speed claims are
"parity unpinned": they need trained models and other hardware.
"""

from . import formats, geometry, quant, draft, attention, pipeline  # noqa: F401
