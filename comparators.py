"""Vendor-library comparators for the weight-only quantized GEMM (measurement context only).

Two paths that the pages measure the method against, rebuilt on MI355X with torch's own
kernels (elementwise ops and hipBLASLt through ``torch.nn.functional.linear``):

* the 16-bit vendor GEMM on a weight that already sits in HBM at 16 bits, the "FP16
  baseline at batch 1 and 16" of Low Bit Triton Kernels (lecture 034, exercises);
* the cast-copy path that the FP8 work replaces (FlashInfer PR #7495 analysis,
  introduction): materialize the whole 16-bit weight -- for FP8 ``weight.to(dtype)`` times the
  scale cast to the activation type, so both the scale and the product are rounded -- then
  run the same vendor GEMM on it.  Its error against the exact product is the yardstick of
  that analysis's accuracy gate (the kernel's error may be at most a multiple of it).

Nothing here is on the library's path: the library never calls torch for arithmetic.  These
functions take the canonical (un-packed) codes and scales, as a cast-copy user holds them.
"""
import numpy as np


def _dev(x, torch):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


class CastCopy:
    """Device copies of one quantized weight in canonical form plus its dequantizer.

    fmt: 'int4' (codes uint8 [N, K/2], scales fp16 bits [K/G, N]), 'fp8' / 'fp8h' (codes
    uint8 [N, K], alpha), 'fp4' (codes uint8 [N, K/2], e4m3 scale codes [N, K/16], alpha).
    """

    def __init__(self, torch, fmt, N, K, G, codes, scales, alpha):
        self.torch, self.fmt, self.N, self.K, self.G = torch, fmt, N, K, G
        self.dtype = torch.float16 if fmt in ("int4", "fp8h") else torch.bfloat16
        self.codes = _dev(codes, torch)
        self.scales = None if scales is None else _dev(scales, torch)
        self.alpha = torch.tensor([alpha], dtype=torch.float32, device="cuda")
        if fmt == "fp4":
            # e2m1 code -> value, the 16 entries of the format (sign bit 3, exponent bits 2..1,
            # mantissa bit 0): +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}
            mag = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
            self.e2m1 = torch.tensor(mag + [-m for m in mag], dtype=self.dtype, device="cuda")

    def dequantize(self):
        """The 16-bit weight [N, K] in HBM, as the cast-copy path forms it."""
        t = self.torch
        N, K = self.N, self.K
        if self.fmt == "int4":
            # signed nibble to fp16, times the fp16 group scale (one rounding: RNE_fp16((n-8) s))
            q = t.stack((self.codes & 15, self.codes >> 4), dim=-1).reshape(N, K)
            s = self.scales.view(t.float16).t().repeat_interleave(self.G, dim=1)
            return (q.to(t.float16) - 8.0) * s
        if self.fmt in ("fp8", "fp8h"):
            # weight.to(dtype).mul_(scale.to(dtype)): the scale and the product are both rounded
            return self.codes.view(t.float8_e4m3fn).to(self.dtype).mul_(self.alpha.to(self.dtype))
        # FP4: e2m1 value times its e4m3 block scale (exact in bf16), then times alpha rounded
        # to bf16 (rounded product)
        q = t.stack((self.codes & 15, self.codes >> 4), dim=-1).reshape(N, K).long()
        sb = self.scales.view(t.float8_e4m3fn).to(self.dtype).repeat_interleave(16, dim=1)
        return (self.e2m1[q] * sb).mul_(self.alpha.to(self.dtype))

    def run(self, A):
        """Cast-copy GEMM: dequantize into HBM, then the vendor GEMM.  Returns [M, N] 16-bit."""
        return self.torch.nn.functional.linear(A, self.dequantize())


def dense_gemm(torch, A, W16):
    """The vendor 16-bit GEMM on a resident 16-bit weight W16 [N, K]: out = A . W16^T."""
    return torch.nn.functional.linear(A, W16)
