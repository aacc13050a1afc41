"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds none of the method's arithmetic: it only draws Gaussian numbers and
casts activations to their 16-bit type with torch's own cast.  Quantization, packing and
the GEMM live in the library (GPU path) and, independently, in the oracle.

Workloads (LLM linear layers; no dataset or trained weights are involved):
  A ~ N(0, 1) cast to fp16 (INT4, INT2 and NF4 shapes, FP8 with fp16 activations) or bf16
  (FP8 / FP4 shapes);
  W ~ N(0, sigma) in fp32, sigma = 0.02 (INT4, INT2, NF4, FP4) or 0.05 (FP8), drawn in the
  "nt" orientation [N, K] (row n = output column n).
  a bias (the bias argument of mm_bf16_fp8 / mm_fp16_fp8) ~ N(0, 0.1) per output column,
  cast to the output's 16-bit type.
Seeds are numpy ``default_rng([workload, shape, role])`` with role 0 = A, 1 = W, 2 = bias.
"""
import numpy as np

ROLE_A, ROLE_W, ROLE_BIAS = 0, 1, 2

# named workloads: (name, format, list of (M, N, K), extra)
WORKLOADS = {
    "int4_tiny": dict(fmt="int4", shapes=[(1, 256, 512)], group_sizes=[128], sigma=0.02),
    "int4_decode": dict(fmt="int4", shapes=[(1, 4096, 4096), (16, 4096, 4096),
                                            (1, 11008, 4096), (16, 11008, 4096)],
                        group_sizes=[128], sigma=0.02),
    "int4_prefill": dict(fmt="int4", shapes=[(4096, 4096, 4096)],
                         group_sizes=[32, 64, 128, 256], sigma=0.02),
    "fp8": dict(fmt="fp8", shapes=[(1, 10240, 5120), (16, 10240, 5120), (8192, 10240, 5120),
                                   (32768, 3200, 5120), (16384, 12800, 5120)],
                group_sizes=[0], sigma=0.05),
    "fp4": dict(fmt="fp4", shapes=[(1, 8192, 8192), (128, 8192, 8192), (8192, 8192, 8192)],
                group_sizes=[16], sigma=0.02),
    # mm_fp16_fp8: the FP8 layer shapes with fp16 activations and a bias
    "fp8h": dict(fmt="fp8h", shapes=[(1, 10240, 5120), (16, 10240, 5120), (8192, 10240, 5120)],
                 group_sizes=[0], sigma=0.05),
    # W2A16: the INT4 decode and prefill layer shapes with 2-bit weights
    "int2": dict(fmt="int2", shapes=[(1, 4096, 4096), (16, 4096, 4096), (4096, 4096, 4096)],
                 group_sizes=[128], sigma=0.02),
    # NF4 (4-bit code-book index): the same shapes, so its table lookup is priced against INT4
    "nf4": dict(fmt="nf4", shapes=[(1, 4096, 4096), (16, 4096, 4096), (4096, 4096, 4096)],
                group_sizes=[128], sigma=0.02),
}
WORKLOAD_INDEX = {name: i for i, name in enumerate(WORKLOADS)}


def rng(*key):
    return np.random.default_rng([int(k) for k in key])


def activations(M, K, kind, key):
    """A ~ N(0,1) as a CPU torch tensor of dtype fp16 ('f16') or bf16 ('bf16')."""
    import torch
    x = rng(*key, ROLE_A).standard_normal((M, K), dtype=np.float32)
    t = torch.from_numpy(x)
    return t.to(torch.float16 if kind == "f16" else torch.bfloat16)


def weights(N, K, sigma, key):
    """W ~ N(0, sigma) as float32 [N, K] (row n holds output column n)."""
    w = rng(*key, ROLE_W).standard_normal((N, K), dtype=np.float32)
    w *= np.float32(sigma)
    return w


def bias(N, kind, key):
    """bias ~ N(0, 0.1) as a CPU torch tensor [N] of dtype fp16 ('f16') or bf16 ('bf16')."""
    import torch
    x = rng(*key, ROLE_BIAS).standard_normal(N, dtype=np.float32) * np.float32(0.1)
    return torch.from_numpy(x).to(torch.float16 if kind == "f16" else torch.bfloat16)
