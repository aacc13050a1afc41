"""Shared machinery of the GPU parity tests: seeded inputs, oracle references, a runner
that calls the library through the C ABI, and the comparison against the oracle."""
import functools
import sys

import numpy as np

import synthetic
from oracle import codecs, quant, reference, tolerance

FMT_ACT = {"int4": "f16", "int2": "f16", "nf4": "f16", "fp8": "bf16", "fp8h": "f16", "fp4": "bf16"}
SIGMA = {"int4": 0.02, "int2": 0.02, "nf4": 0.02, "fp8": 0.05, "fp8h": 0.05, "fp4": 0.02}
GROUPED = ("int4", "int2", "nf4")        # formats with a group size (fp16 group scales, no alpha)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=8)
def oracle_weights(fmt, N, K, G, key):
    """Oracle quantization of seeded weights: canonical bytes, scales, alpha, dequant [N,K]."""
    return quantize_weights(fmt, synthetic.weights(N, K, SIGMA[fmt], key), G)


def quantize_weights(fmt, w, G):
    """Oracle quantization of fp32 weights w [N, K]: canonical bytes, scales, alpha, dequant [N,K]."""
    if fmt == "int4":
        codes, sbits = quant.quantize_int4(w, G)
        return quant.pack_nibbles(codes), sbits, 1.0, reference.dequant_int4(codes, sbits, G)
    if fmt == "int2":
        codes, sbits = quant.quantize_int2(w, G)
        return quant.pack_crumbs(codes), sbits, 1.0, reference.dequant_int2(codes, sbits, G)
    if fmt == "nf4":                     # canonical scales: the code book, then [K/G][N]
        codes, sbits, book = quant.quantize_nf4(w, G)
        return (quant.pack_nibbles(codes), np.concatenate([book, sbits.reshape(-1)]), 1.0,
                reference.dequant_nf4(codes, sbits, G, book))
    if fmt in ("fp8", "fp8h"):           # one quantization for both activation types
        codes, alpha = quant.quantize_fp8(w)
        return codes, None, alpha, reference.dequant_fp8(codes)
    codes, sf, alpha = quant.quantize_fp4(w)
    return quant.pack_nibbles(codes), sf, alpha, reference.dequant_fp4(codes, sf)


def a_values(A16):
    """fp64 values of a 16-bit torch CPU tensor (exact)."""
    import torch
    return A16.to(torch.float64).numpy()


class Prepared:
    """Device-resident packed weights for one (format, N, K, G)."""

    def __init__(self, q, fmt, N, K, G, key, alpha_override=None, weights=None):
        """key seeds the weights; or `weights` (fp32 [N, K]) gives them."""
        import torch
        self.fmt, self.N, self.K, self.G = fmt, N, K, G
        canon, scales, alpha, self.wdq = (oracle_weights(fmt, N, K, G, key) if weights is None
                                          else quantize_weights(fmt, weights, G))
        self.alpha = alpha if alpha_override is None else alpha_override
        p = q.problem(1, N, K, fmt, group_size=G if fmt in GROUPED else None)
        wpk, spk = q.pack(p, canon, scales)
        self.w = torch.from_numpy(wpk).cuda()
        self.s = None if spk is None else torch.from_numpy(spk).cuda()
        self.alpha_t = torch.tensor([self.alpha], dtype=torch.float32, device="cuda")


def run_gpu(q, prep, A16, out_dtype, kernel_hint=0, split_k_hint=0, workspace=None, tile_hint=0, bias=None):
    """Run through the C ABI; returns (out as numpy float64 or 16-bit bits, the workspace).

    bias: optional CPU tensor [N] (16-bit); it is passed in out_dtype (fp32 for F32 output,
    an exact widening), through qgemm_run_bias."""
    import torch
    M, K = A16.shape
    p = q.problem(M, prep.N, prep.K, prep.fmt, group_size=prep.G if prep.fmt in GROUPED else None,
                  out_dtype=out_dtype, kernel_hint=kernel_hint, split_k_hint=split_k_hint,
                  tile_hint=tile_hint)
    tdt = {q.DT_F32: torch.float32, q.DT_F16: torch.float16, q.DT_BF16: torch.bfloat16}[out_dtype]
    out = torch.full((M, prep.N), float("nan"), dtype=tdt, device="cuda")
    A = A16.cuda()
    if workspace is None:
        workspace = q.alloc_workspace(p)
    b = None if bias is None else bias.to(tdt).cuda()
    q.run(p, A, prep.w, prep.s, None if prep.fmt in GROUPED else prep.alpha_t, out, workspace, bias=b)
    torch.cuda.synchronize()
    o = out.cpu()
    if out_dtype == q.DT_F32:
        return o.numpy().astype(np.float64), workspace
    return o.view(torch.int16).numpy().view(np.uint16), workspace


def out16_kind(fmt):
    return "f16" if fmt in ("int4", "int2", "nf4", "fp8h") else "bf16"


def out16_dtype(q, fmt):
    return q.DT_F16 if out16_kind(fmt) == "f16" else q.DT_BF16


def out16_values(bits, fmt):
    return codecs.f16_from_bits(bits) if out16_kind(fmt) == "f16" else codecs.bf16_from_bits(bits)


def check_against_oracle(q, prep, A16, rows=None, kernel_hint=0, split_k_hint=0, tile_hint=0, bias=None,
                         chunk=2048):
    """E1/E2 on the fp32 output, E2 on the 16-bit output, E3 between them, over every row
    (or the given rows): the fp64 reference is formed in row chunks and the chunk
    statistics are combined, so full-size outputs are compared element by element.  E3
    also requires every element of both outputs to be finite (outputs start as NaN, so an
    output tile that no workgroup wrote fails here)."""
    M = A16.shape[0]
    rows = np.arange(M) if rows is None else np.asarray(rows)
    y32, ws = run_gpu(q, prep, A16, q.DT_F32, kernel_hint, split_k_hint, tile_hint=tile_hint, bias=bias)
    y16, _ = run_gpu(q, prep, A16, out16_dtype(q, prep.fmt), kernel_hint, split_k_hint, ws, tile_hint, bias=bias)
    tolerance.check_e3(y16, y32.astype(np.float32), out16_kind(prep.fmt))
    a = a_values(A16)
    w = np.asarray(prep.wdq, dtype=np.float64)
    b = None if bias is None else a_values(bias)
    parts32, parts16 = [], []
    for i in range(0, len(rows), chunk):
        rr = rows[i:i + chunk]
        r = reference.gemm_fp64(a[rr], w, prep.alpha, b)
        parts32.append(tolerance.error_stats(y32[rr], r))
        parts16.append(tolerance.error_stats(out16_values(y16[rr], prep.fmt), r))
    st = tolerance.combine_stats(parts32)
    if not tolerance.gates_pass(st):
        raise AssertionError(f"tolerance gates failed on the fp32 output: {st}")
    st16 = tolerance.combine_stats(parts16)
    if st16["nonfinite"] or st16["E2_fail_count"]:
        raise AssertionError(f"E2 failed on the 16-bit output: {st16}")
    st["rows_checked"] = int(len(rows))
    return st, y32
