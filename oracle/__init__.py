"""CPU oracle for the weight-only quantized GEMM  out[M,N] = A[M,K] . dequant(W)[K,N].

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU-baseline
leg of the benchmark may import anything in this package; the GPU library never does,
and this package imports nothing from the GPU library.

Every function is plain numpy, slow and written to be checked against the pages by eye:

* Low Bit Triton Kernels (GPU MODE lecture 034), section on the core low-bit GEMM
  pattern and the gemlite inner-loop snippet: INT4 codes are two nibbles per byte, the
  signed weight is nibble - 8, and it is multiplied by a per-(K-group, column) fp16
  scale to give the 16-bit operand of the matrix multiply.
* FlashInfer PR #7495 analysis (mm_bf16_fp8), introduction: FP8 e4m3 weights with one
  fp32 per-tensor scale that is applied to the fp32 accumulator, not to the weights.
* FlashInfer PR #4466 analysis (BF16 x FP4 GEMM), sections 1-3: FP4 weights held as
  [n, k/2] bytes with per-block scale factors and a separate fp32 alpha.

Module map: ``codecs`` (number formats), ``quant`` (quantizers + canonical packing),
``layout`` (model of the packed device layout), ``reference`` (dequant + fp64 GEMM),
``tolerance`` (the acceptance gates).

Parity status of each function is recorded in its docstring; nothing here is
"parity unpinned": every function has at least one pin in tests/test_oracle_*.py.
"""
from . import codecs, quant, layout, reference, tolerance  # noqa: F401
