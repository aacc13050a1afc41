"""Packed weights, and activations, larger than 4 GiB (GPU): every byte offset past 2^32 must be
formed in 64-bit arithmetic, in the decode and in the prefill kernels.

The packed layout stores each 16-column block (its weights and its scales) contiguously, so
the packed bytes of a matrix whose columns repeat with a period of three column blocks are
the packed bytes of those three blocks repeated.  A 48-column matrix is quantized by the
oracle and packed by the library, and its packed weights and scales are tiled on the GPU to
N = 48 T columns, past 4 GiB of weights.  Every output column must then equal the column of
the same phase bitwise (the arithmetic of a column does not depend on where it sits), and the
first 48 columns must pass the oracle gates.  A 32-bit wrap of a weight offset at 2^32 bytes
would read column block 2^32 / (K / 128 KiB) = 65536 for K = 8192 from block 0, whose phase
differs (65536 mod 3 = 1), and fail the comparison."""
import numpy as np
import pytest

import synthetic
from gpu_cases import GROUPED, Prepared, a_values, out16_kind, out16_values, say
from oracle import reference, tolerance

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

P = 48                                   # columns of the repeated pattern: three column blocks
K = 8192


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_only_quantized_qgemm_amd as lib
    return lib


# (format, M, repeats T, 16-bit output): N = 48 T columns, packed weights of 4.7 GB
CASES = [("int4", 1, 24000, False),     # decode, A staged
         ("int4", 64, 24000, True),     # prefill, 64 x 128 tile
         ("fp8", 16, 12000, False),     # decode, A by DMA in runs
         ("fp4", 128, 24000, True)]     # prefill, 128 x 128 tile


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_weights_past_4_gib(q, ci):
    fmt, M, T, out16 = CASES[ci]
    N = P * T
    G = 128 if fmt in GROUPED else 0
    p = q.problem(M, N, K, fmt, group_size=G or None, out_dtype=(q.DT_F16 if out16_kind(fmt) == "f16" else q.DT_BF16)
                  if out16 else q.DT_F32)
    wb, sb = q.packed_sizes(p)
    assert wb > (1 << 32), "the case must put weight offsets past 2^32"
    say(f"case large-weights#{ci} fmt={fmt} M={M} N={N} K={K} weights {wb / 1e9:.2f} GB plan={q.plan_describe(p)}")
    prep = Prepared(q, fmt, P, K, G, (75, ci))
    w = prep.w.repeat(T)
    s = None if prep.s is None else prep.s.repeat(T)
    assert w.numel() == wb and (s is None and not sb or s.numel() == sb)
    A16 = synthetic.activations(M, K, out16_kind(fmt), (75, ci, M))
    tdt = torch.float32 if not out16 else (torch.float16 if out16_kind(fmt) == "f16" else torch.bfloat16)
    out = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
    q.run(p, A16.cuda(), w, s, None if fmt in GROUPED else prep.alpha_t, out, q.alloc_workspace(p))
    torch.cuda.synchronize()
    del w, s
    bits = out.view(torch.int32 if tdt == torch.float32 else torch.int16).view(M, T, P)
    assert bool((bits == bits[:, :1, :]).all()), "a column differs from the column of the same phase"
    head = out[:, :P].cpu()
    y = head.numpy().astype(np.float64) if tdt == torch.float32 else out16_values(
        head.view(torch.int16).numpy().view(np.uint16), fmt)
    r = reference.gemm_fp64(a_values(A16), prep.wdq, prep.alpha)
    st = tolerance.error_stats(y, r)
    if tdt == torch.float32:
        assert tolerance.gates_pass(st), st
    else:
        assert not st["nonfinite"] and not st["E2_fail_count"], st
    say(f"  E1={st['E1']:.3e}")
    del out
    torch.cuda.empty_cache()


# (format, row repeats T, N, kernel_hint, 16-bit output): M = 48 T rows of A, 4.3 GB of activations
A_CASES = [("int4", 11000, 256, 0, False),     # one 256 x 256 tile per workgroup
           ("int4", 11000, 256, 3, False),     # persistent schedule with a stream-K tail
           ("fp8", 11000, 384, 0, False),      # ragged last tile column
           ("int4", 11000, 4096, 0, True)]     # and 4.3 GB of 16-bit output


@pytest.mark.parametrize("ci", range(len(A_CASES)))
def test_activations_past_4_gib(q, ci):
    # A repeats with a period of 48 rows, so every output row must equal the row of its phase
    # bitwise; a 32-bit wrap of A's offset at 2^32 bytes (row 524288 for K = 8192 bytes a row)
    # would read a row of another phase (524288 mod 48 = 32).
    fmt, T, N, hint, out16 = A_CASES[ci]
    M, Kq = P * T, 4096
    G = 128 if fmt in GROUPED else 0
    tdt = torch.float32 if not out16 else (torch.float16 if out16_kind(fmt) == "f16" else torch.bfloat16)
    odt = q.DT_F32 if not out16 else (q.DT_F16 if out16_kind(fmt) == "f16" else q.DT_BF16)
    p = q.problem(M, N, Kq, fmt, group_size=G or None, out_dtype=odt, kernel_hint=hint)
    assert M * Kq * 2 > (1 << 32), "the case must put activation offsets past 2^32"
    say(f"case large-activations#{ci} fmt={fmt} M={M} N={N} K={Kq} A {M * Kq * 2 / 1e9:.2f} GB "
        f"plan={q.plan_describe(p)}")
    prep = Prepared(q, fmt, N, Kq, G, (76, ci))
    A_small = synthetic.activations(P, Kq, out16_kind(fmt), (76, ci, P))
    A = A_small.cuda().repeat(T, 1)
    out = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
    q.run(p, A, prep.w, prep.s, None if fmt in GROUPED else prep.alpha_t, out, q.alloc_workspace(p))
    torch.cuda.synchronize()
    del A
    per = out.view(T, P, N)
    if hint != q.KERNEL_PREFILL_STREAMK:
        bits = out.view(torch.int32 if not out16 else torch.int16).view(T, P, N)
        assert bool((bits == bits[:1]).all()), "a row differs from the row of the same phase"
    else:
        # the stream-K tail sums a tile's K range in pieces handed between workgroups, so its
        # rows round differently from rows computed in one pass: equal to rounding, and bitwise
        # equal wherever both rows lie in whole tiles (the first dp_tiles tiles of the walk)
        d = (per - per[:1]).abs()
        rel = float((d / (per[:1].abs() + 1.0)).max())
        rows = int((d.amax(dim=2) > 0).sum())
        say(f"  stream-K: {rows} of {M} rows differ from the row of the same phase, by at most {rel:.2e}")
        assert rel < 1e-5, rel
    head = out[:P].cpu()
    y = head.numpy().astype(np.float64) if not out16 else out16_values(head.view(torch.int16).numpy().view(np.uint16), fmt)
    st = tolerance.error_stats(y, reference.gemm_fp64(a_values(A_small), prep.wdq, prep.alpha))
    if not out16:
        assert tolerance.gates_pass(st), st
    else:
        assert not st["nonfinite"] and not st["E2_fail_count"], st
    say(f"  E1={st['E1']:.3e}")
    del out, per
    torch.cuda.empty_cache()
