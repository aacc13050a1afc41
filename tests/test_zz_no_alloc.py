"""qgemm_run_no_alloc (GPU): the entry point without a workspace argument, whose split-K
partials live in the library's static per-GPU scratch, against qgemm_run_bias with a
caller workspace on the same problem (same plan, so bitwise the same result), called
several times in a row with decreasing sizes so that a later call meets what an earlier
one left in the scratch."""
import numpy as np
import pytest

import synthetic
from gpu_cases import Prepared, check_against_oracle, out16_dtype, out16_kind, run_gpu, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_only_quantized_qgemm_amd as lib
    return lib


def _no_alloc(q, prep, A16, out_dtype, kernel_hint=0, split_k_hint=0, tile_hint=0, bias=None):
    M, K = A16.shape
    p = q.problem(M, prep.N, prep.K, prep.fmt, group_size=prep.G if prep.fmt in ("int4", "int2", "nf4") else None,
                  out_dtype=out_dtype, kernel_hint=kernel_hint, split_k_hint=split_k_hint, tile_hint=tile_hint)
    tdt = {q.DT_F32: torch.float32, q.DT_F16: torch.float16, q.DT_BF16: torch.bfloat16}[out_dtype]
    out = torch.full((M, prep.N), float("nan"), dtype=tdt, device="cuda")
    b = None if bias is None else bias.to(tdt).cuda()
    q.run_no_alloc(p, A16.cuda(), prep.w, prep.s, None if prep.fmt in ("int4", "int2", "nf4") else prep.alpha_t,
                   out, bias=b)
    torch.cuda.synchronize()
    o = out.cpu()
    if out_dtype == q.DT_F32:
        return o.numpy().astype(np.float64)
    return o.view(torch.int16).numpy().view(np.uint16)


# (format, M, N, K, G, kernel_hint, split_k_hint, tile_hint, with bias); each runs after the
# previous one on the same scratch, sizes decreasing: the prefill split of FP4 M = 128 (8 MiB of
# partials, 64 tiles), a planned INT4 prefill split with 64-row tiles (4 MiB, 64 tiles), a
# prefill split with many tiles (so its tickets cover bytes that earlier calls used), a decode
# split, then a plan without a split.
SEQUENCE = [("fp4", 128, 8192, 8192, 0, 0, 0, 0, False),
            ("int4", 64, 4096, 4096, 128, 0, 0, 0, True),
            ("fp8", 300, 2048, 1024, 0, 2, 3, 64, False),
            ("int4", 1, 256, 128 * 64, 128, 1, 16, 0, False),
            ("nf4", 16, 512, 1024, 64, 0, 0, 0, False),
            ("int4", 5, 272, 1024, 32, 1, 3, 0, True)]


def test_no_alloc_matches_workspace_entry_point_bitwise(q):
    for rep in range(2):
        for fmt, M, N, K, G, hint, split, tile, with_bias in SEQUENCE:
            say(f"case no-alloc rep={rep} fmt={fmt} M={M} N={N} K={K} G={G} hint={hint} split={split} tile={tile}")
            prep = Prepared(q, fmt, N, K, G, (70, N, K))
            A = synthetic.activations(M, K, out16_kind(fmt), (70, M))
            b = synthetic.bias(N, out16_kind(fmt), (70, N)) if with_bias else None
            p = q.problem(M, N, K, fmt, group_size=G or None, kernel_hint=hint, split_k_hint=split, tile_hint=tile)
            ws_bytes = q.workspace_bytes(p)
            assert rep > 0 or fmt != "fp4" or ws_bytes > 0, "the sequence must exercise the scratch"
            for odt in (q.DT_F32, out16_dtype(q, fmt)):
                want, _ = run_gpu(q, prep, A, odt, hint, split, tile_hint=tile, bias=b)
                got = _no_alloc(q, prep, A, odt, hint, split, tile, bias=b)
                assert np.array_equal(got, want), f"no-alloc output differs ({fmt} M={M} out={odt})"
    # the result itself against the oracle once (the bitwise match carries it to the rest)
    prep = Prepared(q, "fp4", 8192, 8192, 0, (70, 8192, 8192))
    A = synthetic.activations(128, 8192, "bf16", (70, 128))
    y = _no_alloc(q, prep, A, q.DT_F32)
    st, ref32 = check_against_oracle(q, prep, A)
    assert np.array_equal(y, ref32)
    say(f"  fp4 128x8192x8192 E1={st['E1']:.3e}")


def test_no_alloc_runs_the_persistent_stream_k_schedule(q):
    # The persistent schedule with the 128- and 64-row tiles keeps its two partial slots per
    # resident workgroup (32 MiB) and its tail tickets inside the static scratch: bitwise the
    # result of qgemm_run_bias with a workspace, twice in a row; with the 256-row tile it needs
    # 128 MiB and is refused.
    M, N, K = 2176, 2048, 1024
    say("case no-alloc stream-k int4 2176x2048x1024")
    prep = Prepared(q, "int4", N, K, 128, (71, N, K))
    A = synthetic.activations(M, K, "f16", (71, M))
    for tile in (128, 64):
        assert 0 < q.workspace_bytes(q.problem(M, N, K, "int4", kernel_hint=3, tile_hint=tile)) <= q.NO_ALLOC_SCRATCH_BYTES
        for odt in (q.DT_F32, q.DT_F16):
            want, _ = run_gpu(q, prep, A, odt, kernel_hint=3, tile_hint=tile)
            for _ in range(2):
                got = _no_alloc(q, prep, A, odt, kernel_hint=3, tile_hint=tile)
                assert np.array_equal(got, want)
    big = q.problem(M, N, K, "int4", kernel_hint=3, tile_hint=256)
    assert q.workspace_bytes(big) > q.NO_ALLOC_SCRATCH_BYTES
    out = torch.full((M, N), 3.0, dtype=torch.float16, device="cuda")
    with pytest.raises(q.QgemmError) as ei:
        q.run_no_alloc(big, A.cuda(), prep.w, prep.s, None, out)
    assert ei.value.status == q.ERR_WORKSPACE_TOO_SMALL


def test_no_alloc_rejects_plans_beyond_the_scratch(q):
    # FP4 1024 x 8192 x 8192 plans 64 MiB of partial tiles, more than the static scratch holds:
    # the call is refused before anything is enqueued, and the workspace entry point is not.
    p = q.problem(1024, 8192, 8192, "fp4")
    assert q.workspace_bytes(p) > q.NO_ALLOC_SCRATCH_BYTES
    w = torch.zeros(8192 * 4096, dtype=torch.uint8, device="cuda")
    s = torch.zeros(8192 * 512, dtype=torch.uint8, device="cuda")
    A = torch.zeros((1024, 8192), dtype=torch.bfloat16, device="cuda")
    out = torch.full((1024, 8192), 3.0, dtype=torch.bfloat16, device="cuda")
    alpha = torch.ones(1, dtype=torch.float32, device="cuda")
    with pytest.raises(q.QgemmError) as ei:
        q.run_no_alloc(p, A, w, s, alpha, out)
    assert ei.value.status == q.ERR_WORKSPACE_TOO_SMALL
    assert "static scratch" in ei.value.detail
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
    # M = 0 and a problem without a split need no scratch at all
    q.run_no_alloc(q.problem(0, 8192, 8192, "fp4"), A, w, s, alpha, out)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
