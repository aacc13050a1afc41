"""HIP-graph capture of the library's launches (GPU).

qgemm_run, qgemm_run_bias and qgemm_run_no_alloc are captured into a graph and the graph is
replayed several times, with eager work between the replays (a fill of the output, an eager
launch of the same problem on its own workspace, host synchronisations).  Every replay's
output must equal the eager result bitwise.  This holds because a completed launch leaves its
split-K tickets at zero, so a replay finds its workspace as a fresh zero-filled one, and
because no memset is ever recorded (the no-alloc scratch is cleared by a fill kernel).  The
cases cover each launch path: decode (staged A, A by DMA in runs, split K), the three
prefill tiles with split K, the persistent stream-K schedule, the transform-wave kernel, a
bias, and the static scratch.  A second test captures several problems into one graph that
shares one workspace in stream order, which the workspace contract allows."""
import pytest

import synthetic
from gpu_cases import GROUPED, Prepared, out16_dtype, out16_kind, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_only_quantized_qgemm_amd as lib
    return lib


# (format, M, N, K, G, kernel_hint, split_k_hint, tile_hint, with bias, entry point)
CASES = [
    ("int4", 1, 4096, 4096, 128, 0, 0, 0, False, "run"),          # decode, A staged, early first load
    ("int4", 16, 11008, 4096, 128, 0, 0, 0, False, "run"),        # decode, A by DMA, runs of two sets
    ("int4", 4, 512, 8192, 128, 1, 4, 0, True, "run"),            # decode split K, bias
    ("fp8", 300, 2048, 1024, 0, 2, 3, 64, False, "run"),          # 64 x 128 tile, split 3, ragged M
    ("fp4", 128, 8192, 8192, 0, 0, 0, 0, False, "run"),           # planned split of the small tile
    ("int2", 33, 4096, 2048, 64, 2, 0, 256, False, "run"),        # 256 x 256 tile, planned split 4
    ("int4", 2176, 2048, 1024, 128, 3, 0, 128, False, "run"),     # persistent stream-K, 128 x 128 tile
    ("nf4", 100, 1024, 2048, 64, 4, 2, 0, False, "run"),          # transform waves, split 2
    ("fp8h", 64, 1024, 1024, 0, 2, 2, 0, True, "run"),            # fp16 activations, bias, split 2
    ("fp4", 128, 8192, 8192, 0, 0, 0, 0, False, "no_alloc"),      # static scratch, split
    ("int4", 5, 272, 1024, 32, 1, 3, 0, True, "no_alloc"),        # static scratch, decode split
]


def _case_inputs(q, fmt, M, N, K, G, with_bias, seed, out_torch_dtype):
    """Device inputs, all uploaded before any capture (a host copy cannot be captured); the
    bias is passed in the output type (fp32 for an fp32 output, an exact widening)."""
    prep = Prepared(q, fmt, N, K, G, (72, N, K))
    A = synthetic.activations(M, K, out16_kind(fmt), (72, seed, M)).cuda()
    bias = synthetic.bias(N, out16_kind(fmt), (72, seed)).to(out_torch_dtype).cuda() if with_bias else None
    return prep, A, bias


def _launch(q, entry, p, prep, A, out, ws, bias):
    alpha = None if prep.fmt in GROUPED else prep.alpha_t
    if entry == "run":
        q.run(p, A, prep.w, prep.s, alpha, out, ws, bias=bias)
    else:
        q.run_no_alloc(p, A, prep.w, prep.s, alpha, out, bias=bias)


def _bits(t):
    return t.view(torch.int32 if t.element_size() == 4 else torch.int16)


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_graph_replays_equal_eager(q, ci):
    fmt, M, N, K, G, hint, split, tile, with_bias, entry = CASES[ci]
    odt = q.DT_F32 if ci % 2 == 0 else out16_dtype(q, fmt)
    say(f"case graph#{ci} {entry} fmt={fmt} M={M} N={N} K={K} G={G} hint={hint} split={split} tile={tile} "
        f"bias={with_bias} out={odt}")
    tdt = {q.DT_F32: torch.float32, q.DT_F16: torch.float16, q.DT_BF16: torch.bfloat16}[odt]
    prep, A, bias = _case_inputs(q, fmt, M, N, K, G, with_bias, ci, tdt)
    p = q.problem(M, N, K, fmt, group_size=G or None, out_dtype=odt, kernel_hint=hint, split_k_hint=split,
                  tile_hint=tile)
    nan = float("nan")

    ws_e = q.alloc_workspace(p) if entry == "run" else None
    ref = torch.full((M, N), nan, dtype=tdt, device="cuda")
    _launch(q, entry, p, prep, A, ref, ws_e, bias)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(ref).all())

    out = torch.full((M, N), nan, dtype=tdt, device="cuda")
    ws_g = q.alloc_workspace(p) if entry == "run" else None
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _launch(q, entry, p, prep, A, out, ws_g, bias)
    torch.cuda.synchronize()
    again = torch.empty_like(ref)
    for r in range(REPLAYS):
        out.fill_(nan)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref)), f"replay {r} differs from the eager result"
        again.fill_(nan)
        _launch(q, entry, p, prep, A, again, ws_e, bias)     # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(_bits(again), _bits(ref)), f"eager launch after replay {r} differs"
    del g


def test_one_graph_of_several_problems_sharing_a_workspace(q):
    # Launches in one stream's order may share a workspace; captured together, each replay
    # runs them back to back on it, each finding the tickets the previous one left at zero.
    seq = [CASES[2], CASES[3], CASES[4], CASES[7], CASES[5]]
    probs = []
    for k, (fmt, M, N, K, G, hint, split, tile, with_bias, _) in enumerate(seq):
        odt = out16_dtype(q, fmt)
        tdt = torch.float16 if odt == q.DT_F16 else torch.bfloat16
        prep, A, bias = _case_inputs(q, fmt, M, N, K, G, with_bias, 100 + k, tdt)
        p = q.problem(M, N, K, fmt, group_size=G or None, out_dtype=odt, kernel_hint=hint, split_k_hint=split,
                      tile_hint=tile)
        probs.append((p, prep, A, bias, tdt, M, N))
    ws_bytes = max(q.workspace_bytes(p) for p, *_ in probs)
    assert ws_bytes > 0
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    refs = []
    for p, prep, A, bias, tdt, M, N in probs:
        r = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
        _launch(q, "run", p, prep, A, r, ws, bias)
        refs.append(r)
    torch.cuda.synchronize()
    outs = [torch.full_like(r, float("nan")) for r in refs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for (p, prep, A, bias, *_), o in zip(probs, outs):
            _launch(q, "run", p, prep, A, o, ws, bias)
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        say(f"case graph-sequence replay {rep}")
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for k, (o, r) in enumerate(zip(outs, refs)):
            assert torch.equal(_bits(o), _bits(r)), f"problem {k} differs on replay {rep}"
    del g
