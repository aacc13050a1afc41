"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: dequantized weights bit-exact (identity activations); GEMM outputs within
E1 <= 1e-3 and E2 (|y - r| <= max(5e-3 |r|, 2e-2)) of the fp64 oracle, 16-bit outputs
bitwise equal to the RNE cast of the fp32 output (E3), runs bitwise deterministic."""
import numpy as np
import pytest

import synthetic
from gpu_cases import (Prepared, check_against_oracle, oracle_weights, out16_dtype, out16_kind,
                       run_gpu, say)
from oracle import codecs, reference, tolerance

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_only_quantized_qgemm_amd as lib
    return lib


def _g(fmt):
    """Group size of the format in the generic cases (128 for the integer formats)."""
    return 128 if fmt in ("int4", "int2", "nf4") else 0


def _act(fmt, M, K, key):
    return synthetic.activations(M, K, out16_kind(fmt), key)


def _identity_rows(fmt, rows, K):
    import torch as T
    dt = T.float16 if out16_kind(fmt) == "f16" else T.bfloat16
    A = T.zeros((len(rows), K), dtype=dt)
    for i, k in enumerate(rows):
        A[i, k] = 1.0
    return A


def _dequant_16bit_values(fmt, prep):
    """The 16-bit operand the method feeds the MFMA, [N, K] float64."""
    canon, scales, _, wdq = oracle_weights(fmt, prep.N, prep.K, prep.G, (7, prep.N, prep.K))
    from oracle import quant
    if fmt == "int4":
        return reference.dequant_int4_f16(quant.unpack_nibbles(canon), scales, prep.G)
    if fmt == "nf4":                                     # RNE_fp16(T[code] s)
        return reference.dequant_nf4_f16(quant.unpack_nibbles(canon), scales[16:].reshape(-1, prep.N),
                                         prep.G, scales[:16])
    # INT2: (code - 2) s is exact in fp16; FP8 (alpha not applied), FP4: exact in 16 bits
    return wdq.astype(np.float64)


@pytest.mark.parametrize("fmt,G", [("int4", 32), ("int4", 64), ("int4", 128), ("int4", 256),
                                   ("int2", 32), ("int2", 64), ("int2", 128), ("int2", 256),
                                   ("nf4", 32), ("nf4", 64), ("nf4", 128), ("nf4", 256),
                                   ("fp8", None), ("fp8h", None), ("fp4", None)])
@pytest.mark.parametrize("hint,step", [(1, 16), (1, 4), (1, 1), (2, None)],
                         ids=["decode-M16", "decode-M4", "decode-M1", "prefill"])
def test_identity_activations_give_dequantized_weights_bit_exact(q, fmt, G, hint, step):
    N, K = 48, 512
    say(f"case identity fmt={fmt} G={G} hint={hint} rows={step}")
    prep = Prepared(q, fmt, N, K, G or 0, (7, N, K), alpha_override=1.0)
    step = step or K
    want = _dequant_16bit_values(fmt, prep)              # [N, K]
    if step == 1:
        k0s = list(range(0, K, 37)) + [K - 1]            # M = 1: a sample of single rows
    else:
        k0s = list(range(0, K, step))
    for k0 in k0s:
        rows = list(range(k0, k0 + step))
        A = _identity_rows(fmt, rows, K)
        y32, _ = run_gpu(q, prep, A, q.DT_F32, kernel_hint=hint)
        assert np.array_equal(y32, want[:, rows].T), f"fp32 dequant mismatch rows {k0}.."
        y16, _ = run_gpu(q, prep, A, out16_dtype(q, fmt), kernel_hint=hint)
        kind = out16_kind(fmt)
        want16 = codecs.f16_bits(want[:, rows].T) if kind == "f16" else codecs.bf16_bits(want[:, rows].T)
        assert np.array_equal(y16, want16)


CONFIGS = [
    # workload name, shape index, (M, N, K), G; every output element is compared
    ("int4_tiny", 0, (1, 256, 512), 128),
    ("int4_decode", 0, (1, 4096, 4096), 128),
    ("int4_decode", 1, (16, 4096, 4096), 128),
    ("int4_decode", 2, (1, 11008, 4096), 128),
    ("int4_decode", 3, (16, 11008, 4096), 128),
    ("int4_prefill", 0, (4096, 4096, 4096), 32),
    ("int4_prefill", 0, (4096, 4096, 4096), 64),
    ("int4_prefill", 0, (4096, 4096, 4096), 128),
    ("int4_prefill", 0, (4096, 4096, 4096), 256),
    ("fp8", 0, (1, 10240, 5120), None),
    ("fp8", 1, (16, 10240, 5120), None),
    ("fp8", 2, (8192, 10240, 5120), None),
    ("fp8", 3, (32768, 3200, 5120), None),
    ("fp8", 4, (16384, 12800, 5120), None),
    ("fp8h", 0, (1, 10240, 5120), None),
    ("fp8h", 1, (16, 10240, 5120), None),
    ("fp8h", 2, (8192, 10240, 5120), None),
    ("int2", 0, (1, 4096, 4096), 128),
    ("int2", 1, (16, 4096, 4096), 128),
    ("int2", 2, (4096, 4096, 4096), 128),
    ("nf4", 0, (1, 4096, 4096), 128),
    ("nf4", 1, (16, 4096, 4096), 128),
    ("nf4", 2, (4096, 4096, 4096), 128),
    ("fp4", 0, (1, 8192, 8192), None),
    ("fp4", 1, (128, 8192, 8192), None),
    ("fp4", 2, (8192, 8192, 8192), None),
]


@pytest.mark.parametrize("name,si,shape,G", CONFIGS,
                         ids=[f"{c[0]}-{c[2][0]}x{c[2][1]}x{c[2][2]}-G{c[3]}" for c in CONFIGS])
def test_workload_parity(q, name, si, shape, G):
    # Full size, in the launch configuration the benchmark times (automatic plan), every
    # row of the output against the fp64 oracle.
    M, N, K = shape
    fmt = synthetic.WORKLOADS[name]["fmt"]
    wi = synthetic.WORKLOAD_INDEX[name]
    say(f"case workload {name} M={M} N={N} K={K} G={G}")
    prep = Prepared(q, fmt, N, K, G or 0, (wi, si))
    A = _act(fmt, M, K, (wi, si))
    # the fp16-activation FP8 workload carries a bias (mm_fp16_fp8's bias argument)
    b = synthetic.bias(N, out16_kind(fmt), (wi, si)) if name == "fp8h" else None
    st, _ = check_against_oracle(q, prep, A, bias=b)
    assert st["rows_checked"] == M
    say(f"  E1={st['E1']:.3e} worstE2={st['E2_worst_ratio']:.3f} max_abs={st['max_abs']:.3e} "
        f"max_rel(|r|>=rms)={st['max_rel_rms']:.3e}")


@pytest.mark.parametrize("fmt,G", [("int4", 32), ("int4", 128), ("int4", 256), ("int2", 64), ("int2", 256),
                                   ("nf4", 32), ("nf4", 256), ("fp8", None), ("fp8h", None), ("fp4", None)])
@pytest.mark.parametrize("M", [1, 2, 7, 15, 16, 17, 33, 127, 128, 129])
def test_m_sweep_ragged(q, fmt, G, M):
    N, K = 272, 768          # N: 17 column blocks (ragged against 128-wide tiles); K: 6 k blocks
    say(f"case m-sweep fmt={fmt} G={G} M={M}")
    prep = Prepared(q, fmt, N, K, G or 0, (50, N, K))
    A = _act(fmt, M, K, (50, M))
    check_against_oracle(q, prep, A)


@pytest.mark.parametrize("fmt", ["int4", "int2", "nf4", "fp8", "fp4"])
@pytest.mark.parametrize("M,hint,split,tile", [(16, 1, 2, 0), (16, 1, 3, 1), (16, 1, 7, 2), (16, 1, 14, 4),
                                               (4, 1, 1, 4), (4, 1, 5, 1), (16, 1, 1, 3), (16, 1, 4, 3),
                                               (3, 1, 2, 3), (16, 2, 1, 0), (16, 2, 2, 0),
                                               (16, 2, 5, 0)])
def test_split_k_and_kernel_hints(q, fmt, M, hint, split, tile):
    N, K = 256, 1792    # 14 k blocks
    say(f"case hints fmt={fmt} M={M} kernel={hint} split={split} tile={tile}")
    prep = Prepared(q, fmt, N, K, _g(fmt), (51, N, K))
    A = _act(fmt, M, K, (51, M))
    check_against_oracle(q, prep, A, kernel_hint=hint, split_k_hint=split, tile_hint=tile)


@pytest.mark.parametrize("fmt,G", [("int4", 64), ("int2", 128), ("nf4", 32), ("fp8", None), ("fp4", None)])
@pytest.mark.parametrize("M,N,K", [(1, 256, 128 * 44), (3, 512, 128 * 60), (16, 256, 128 * 60), (16, 8192, 128 * 44),
                                   (9, 4352, 128 * 23)])
def test_decode_multi_run(q, fmt, G, M, N, K):
    # Wavefront shares longer than one run (the pipelined decode path), with uneven run
    # counts, shares that end mid-run, and staged / unstaged A.
    say(f"case decode-multirun fmt={fmt} G={G} M={M} N={N} K={K}")
    prep = Prepared(q, fmt, N, K, G or 0, (54, N, K))
    A = _act(fmt, M, K, (54, M))
    check_against_oracle(q, prep, A)


STAGED_CASES = [
    # (format, G, M, N, K, A path): staged A with the first weight block issued before the
    # staging loads ("staged-early": one column block, short runs, one workgroup per CU at
    # most) and after them ("staged")
    ("int4", 128, 1, 4096, 4096, "staged-early"),
    ("int4", 32, 4, 11008, 4096, "staged"),          # 688 workgroups
    ("fp4", None, 1, 8192, 8192, "staged"),          # runs of eight k blocks, 512 workgroups
    ("nf4", 64, 3, 1024, 2048, "staged-early"),      # split K
    ("fp8", None, 2, 4096, 5120, "staged-early"),    # runs of five
    ("int2", 256, 4, 8192, 4096, "staged"),          # 512 workgroups
]


@pytest.mark.parametrize("fmt,G,M,N,K,path", STAGED_CASES,
                         ids=[f"{c[0]}-{c[2]}x{c[3]}x{c[4]}" for c in STAGED_CASES])
def test_decode_staged_paths(q, fmt, G, M, N, K, path):
    d = q.plan_fields(q.problem(M, N, K, fmt, group_size=G))
    assert d["kernel"] == "decode" and d["a"] == path, d
    say(f"case decode-staged fmt={fmt} G={G} M={M} N={N} K={K} plan={d}")
    prep = Prepared(q, fmt, N, K, G or 0, (65, N, K))
    A = _act(fmt, M, K, (65, M))
    check_against_oracle(q, prep, A)


DMA_CASES = [
    # (format, G, M, N, K, expected plan: cb, kpw, runs, splits) -- every case takes A through
    # the DMA slots; together they cover one run per share (with wavefronts whose share is
    # empty), two slot sets alternating over 2 to 8 runs, shares ending mid-run, runs one
    # after another reusing one set, runs shortened to fit LDS, split K, 1 to 4 column blocks.
    ("int4", 128, 5, 256, 512, (1, 1, 1, 1)),       # 4 k blocks over 8 wavefronts
    ("int4", 64, 16, 2048, 5120, (1, 2, 3, 1)),     # share 5 in runs of 2
    ("nf4", 32, 9, 1024, 5120, (1, 2, 2, 2)),       # split K, share 3
    ("int4", 128, 16, 2048, 16384, (1, 2, 8, 1)),   # share 16: eight overlapped runs
    ("int4", 128, 16, 2048, 18432, (1, 2, 1, 1)),   # share 18: nine runs, one slot set
    ("int4", 32, 6, 9216, 6144, (3, 2, 6, 1)),      # six overlapped runs
    ("fp8", None, 16, 4096, 8192, (1, 2, 4, 1)),    # runs shortened from 8 to fit LDS
    ("fp4", None, 12, 4352, 2944, (2, 4, 2, 1)),
    ("int2", 32, 16, 8448, 2048, (3, 2, 2, 1)),
    ("fp8h", None, 7, 12288, 1024, (3, 2, 1, 1)),
    ("int4", 256, 16, 16384, 2048, (4, 2, 2, 1)),
    ("fp4", None, 16, 1024, 16384, (1, 2, 4, 2)),
    ("nf4", 128, 13, 4096, 3072, (1, 2, 2, 1)),
]


@pytest.mark.parametrize("fmt,G,M,N,K,plan", DMA_CASES,
                         ids=[f"{c[0]}-{c[2]}x{c[3]}x{c[4]}" for c in DMA_CASES])
def test_decode_dma_paths(q, fmt, G, M, N, K, plan):
    # The decode kernel with A in DMA-filled LDS slots, in each launch shape the planner makes
    # (checked through qgemm_plan_describe), every row against the fp64 oracle.
    d = q.plan_fields(q.problem(M, N, K, fmt, group_size=G))
    got = tuple(int(d[k]) for k in ("cb", "kpw", "runs", "splits"))
    assert d["kernel"] == "decode" and d["a"] == "dma" and got == plan, d
    say(f"case decode-dma fmt={fmt} G={G} M={M} N={N} K={K} plan={d}")
    prep = Prepared(q, fmt, N, K, G or 0, (64, N, K))
    A = _act(fmt, M, K, (64, M))
    check_against_oracle(q, prep, A)


TRANSFORM_CASES = [
    # (format, G, M, N, K, split): the prefill kernel with dedicated dequantization wavefronts
    # (64 x 128 tiles): ragged rows and columns (idle MFMA wavefronts past N), slices of one to
    # many k blocks, every format and group size family
    ("int4", 128, 100, 400, 1024, 1), ("int4", 32, 64, 256, 128, 1), ("int2", 64, 130, 528, 896, 2),
    ("nf4", 128, 64, 1024, 2048, 3), ("fp8", None, 200, 272, 640, 1), ("fp8h", None, 17, 400, 1664, 2),
    ("fp4", None, 128, 2048, 4096, 2), ("int4", 256, 300, 784, 2304, 4),
]


@pytest.mark.parametrize("fmt,G,M,N,K,split", TRANSFORM_CASES,
                         ids=[f"{c[0]}-{c[2]}x{c[3]}x{c[4]}-s{c[5]}" for c in TRANSFORM_CASES])
def test_prefill_transform_waves(q, fmt, G, M, N, K, split):
    # kernel_hint PREFILL_TRANSFORM: every element against the oracle, and bitwise the same
    # result on a second run.
    say(f"case transform fmt={fmt} G={G} M={M} N={N} K={K} split={split}")
    p = q.problem(M, N, K, fmt, group_size=G, kernel_hint=q.KERNEL_PREFILL_TRANSFORM, split_k_hint=split)
    d = q.plan_fields(p)
    assert d["kernel"] == "prefill" and d["transform"] == "1" and d["tile"] == "64x128", d
    assert int(d["splits"]) == split, d
    prep = Prepared(q, fmt, N, K, G or 0, (68, N, K))
    A = _act(fmt, M, K, (68, M))
    st, y0 = check_against_oracle(q, prep, A, kernel_hint=q.KERNEL_PREFILL_TRANSFORM, split_k_hint=split)
    y1, _ = run_gpu(q, prep, A, q.DT_F32, kernel_hint=q.KERNEL_PREFILL_TRANSFORM, split_k_hint=split)
    assert np.array_equal(y0, y1)


SMALL_WINDOW_CASES = [
    # (format, G, K, split): the 64-row tile meets at a barrier every second k block and keeps
    # six A stages, so slices of 1, 2, 3, 5 and 7 k blocks end on a full window, inside one, or
    # before the first barrier; with splits, the last slice is the shorter one.
    ("int4", 128, 128, 1), ("fp8", None, 256, 1), ("fp4", None, 384, 1), ("nf4", 32, 640, 1),
    ("int2", 64, 896, 1), ("fp8h", None, 128 * 13, 2), ("int4", 256, 128 * 18, 4), ("fp4", None, 128 * 11, 3),
]


@pytest.mark.parametrize("fmt,G,K,split", SMALL_WINDOW_CASES,
                         ids=[f"{c[0]}-K{c[2]}-s{c[3]}" for c in SMALL_WINDOW_CASES])
def test_prefill_small_tile_barrier_windows(q, fmt, G, K, split):
    # 100 rows (a full and a ragged 64-row tile) x 400 columns (three 128-column tiles, the
    # last one with its wavefronts past N idle): every element against the oracle.
    M, N = 100, 400
    say(f"case small-tile windows fmt={fmt} G={G} K={K} split={split}")
    p = q.problem(M, N, K, fmt, group_size=G, kernel_hint=2, tile_hint=64, split_k_hint=split)
    d = q.plan_fields(p)
    assert d["tile"] == "64x128" and int(d["splits"]) == split, d
    prep = Prepared(q, fmt, N, K, G or 0, (67, N, K))
    A = _act(fmt, M, K, (67, M))
    check_against_oracle(q, prep, A, kernel_hint=2, split_k_hint=split, tile_hint=64)


@pytest.mark.parametrize("fmt,G", [("int4", 32), ("int4", 128), ("int2", 32), ("nf4", 64), ("fp8", None),
                                   ("fp4", None)])
@pytest.mark.parametrize("tile,split", [(64, 1), (64, 3), (128, 1), (128, 3), (256, 1), (256, 3)])
def test_prefill_tile_shapes(q, fmt, G, tile, split):
    # The three prefill workgroup shapes on every format: 600 rows are ragged against 64-,
    # 128- and 256-row tiles, 784 columns (49 column blocks) against 128- and 256-column
    # tiles; 8 k blocks.
    M, N, K = 600, 784, 1024
    say(f"case prefill-tile fmt={fmt} G={G} tile={tile} split={split}")
    prep = Prepared(q, fmt, N, K, G or 0, (53, N, K))
    A = _act(fmt, M, K, (53, M))
    check_against_oracle(q, prep, A, kernel_hint=2, split_k_hint=split, tile_hint=tile)


@pytest.mark.parametrize("fmt", ["int4", "int2", "nf4", "fp8", "fp4"])
@pytest.mark.parametrize("M", [16, 256])
def test_deterministic_and_counters_reset(q, fmt, M):
    N, K = 512, 4096
    say(f"case determinism fmt={fmt} M={M}")
    prep = Prepared(q, fmt, N, K, _g(fmt), (52, N, K))
    A = _act(fmt, M, K, (52, M))
    outs = []
    ws = None
    for _ in range(3):
        y, ws = run_gpu(q, prep, A, q.DT_F32, workspace=ws)
        outs.append(y)
        if ws is not None:
            p = q.problem(M, N, K, fmt, group_size=_g(fmt) or None)
            assert q.workspace_bytes(p) > 0
            head = ws[:256].cpu().numpy()
            assert not head.any(), "split-K tickets must return to zero"
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])


@pytest.mark.parametrize("fmt", ["int4", "int2", "nf4", "fp8", "fp4"])
def test_minimum_shape_and_zero_weights(q, fmt):
    import torch as T
    N, K = 16, 128
    say(f"case minimum fmt={fmt}")
    prep = Prepared(q, fmt, N, K, _g(fmt), (53, N, K))
    for M in (1, 16, 17):
        check_against_oracle(q, prep, _act(fmt, M, K, (53, M)))
    # all-zero packed weights give exact zeros
    prep.w.zero_()
    if prep.s is not None:
        prep.s.zero_()
    y, _ = run_gpu(q, prep, _act(fmt, 5, K, (53, 5)), q.DT_F32)
    assert not y.any()


def test_int4_closed_form_equal_nibbles_unit_scales(q):
    import torch as T
    N, K, M = 64, 1024, 8
    say("case closed-form int4")
    p = q.problem(M, N, K, "int4", out_dtype=q.DT_F32)
    A16 = _act("int4", M, K, (54, 0))
    rowsum = A16.to(T.float64).sum(dim=1).numpy()
    for c in (0, 5, 8, 15):
        codes = np.full((N, K // 2), c | (c << 4), np.uint8)
        scales = np.full((K // 128, N), 0x3C00, np.uint16)        # 1.0
        wpk, spk = q.pack(p, codes, scales)
        out = T.empty((M, N), dtype=T.float32, device="cuda")
        q.run(p, A16.cuda(), T.from_numpy(wpk).cuda(), T.from_numpy(spk).cuda(), None, out,
              q.alloc_workspace(p))
        T.cuda.synchronize()
        y = out.cpu().numpy().astype(np.float64)
        want = np.repeat(((c - 8) * rowsum)[:, None], N, axis=1)
        if c == 8:
            assert not y.any()
        else:
            tolerance.check_e1_e2(y, want)


@pytest.mark.parametrize("fmt", ["int4", "fp8"])
@pytest.mark.parametrize("M,hint,tile,split", [(5, 1, 0, 1), (16, 1, 0, 3), (100, 2, 64, 1), (100, 2, 128, 2),
                                               (300, 2, 256, 1), (300, 2, 64, 3)])
@pytest.mark.parametrize("f32", [False, True])
def test_writes_stay_inside_the_output(q, fmt, M, hint, tile, split, f32):
    # The output handed over is the first M rows of a larger buffer whose remaining rows hold
    # sentinels: no kernel (decode, each prefill tile, split or not, 16-bit or fp32 output)
    # may write past row M - 1; N = 272 is ragged against every column tile.
    N, K = 272, 1024
    say(f"case bounds fmt={fmt} M={M} hint={hint} tile={tile} split={split} f32={f32}")
    prep = Prepared(q, fmt, N, K, _g(fmt), (63, N, K))
    A = _act(fmt, M, K, (63, M)).cuda()
    dt = torch.float32 if f32 else (torch.float16 if out16_kind(fmt) == "f16" else torch.bfloat16)
    odt = q.DT_F32 if f32 else out16_dtype(q, fmt)
    buf = torch.full((M + 80, N), -3.0, dtype=dt, device="cuda")
    p = q.problem(M, N, K, fmt, group_size=_g(fmt) or None, out_dtype=odt, kernel_hint=hint,
                  split_k_hint=split, tile_hint=tile)
    q.run(p, A, prep.w, prep.s, None if fmt == "int4" else prep.alpha_t, buf[:M], q.alloc_workspace(p))
    torch.cuda.synchronize()
    assert bool((buf[M:] == -3.0).all())
    assert bool(torch.isfinite(buf[:M]).all()) and not bool((buf[:M] == -3.0).all())


@pytest.mark.parametrize("fmt", ["int4", "nf4", "fp8", "fp4"])
def test_empty_m_enqueues_nothing(q, fmt):
    # M = 0 is an empty product: the call succeeds and writes nothing (the output buffer
    # handed over here has a row of sentinels that must survive).
    N, K = 256, 512
    say(f"case empty-m fmt={fmt}")
    prep = Prepared(q, fmt, N, K, _g(fmt), (55, N, K))
    dt = torch.float16 if out16_kind(fmt) == "f16" else torch.bfloat16
    A = torch.zeros((1, K), dtype=dt, device="cuda")
    out = torch.full((1, N), 7.0, dtype=dt, device="cuda")
    p = q.problem(0, N, K, fmt, group_size=_g(fmt) or None)
    q.run(p, A, prep.w, prep.s, None if fmt in ("int4", "int2", "nf4") else prep.alpha_t, out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


@pytest.mark.parametrize("fmt,G", [("int4", 128), ("fp8", None), ("fp4", None)])
@pytest.mark.parametrize("M,N,K", [(1, 256, 131072), (16, 256, 131072), (300, 32, 65536)])
def test_long_k(q, fmt, G, M, N, K):
    # Long reductions: M = 1 needs many K slices to keep its staged A slice within LDS;
    # M = 16 streams A fragments over a long share; the prefill case splits K deeply.
    say(f"case long-k fmt={fmt} G={G} M={M} N={N} K={K}")
    prep = Prepared(q, fmt, N, K, G or 0, (56, N, K))
    A = _act(fmt, M, K, (56, M))
    st, _ = check_against_oracle(q, prep, A)
    say(f"  E1={st['E1']:.3e} worstE2={st['E2_worst_ratio']:.3f}")


@pytest.mark.parametrize("fmt", ["int4", "int2", "nf4", "fp8", "fp8h", "fp4"])
@pytest.mark.parametrize("M,hint,split,tile", [(1, 0, 0, 0), (16, 0, 3, 0), (33, 0, 0, 0), (300, 2, 2, 0),
                                              (600, 2, 1, 256), (200, 2, 3, 64)])
def test_bias_epilogue(q, fmt, M, hint, split, tile):
    # qgemm_run_bias: out = A . dequant(W) (* alpha) + bias[n], the bias added in fp32 after
    # alpha and rounded once with the rest (mm_bf16_fp8 / mm_fp16_fp8 bias argument).
    # N = 272 columns are ragged against the 128- and 256-column prefill tiles.
    import torch as T
    N, K = 272, 1024
    say(f"case bias fmt={fmt} M={M} hint={hint} split={split} tile={tile}")
    prep = Prepared(q, fmt, N, K, _g(fmt), (57, N, K))
    A = _act(fmt, M, K, (57, M))
    b = synthetic.bias(N, out16_kind(fmt), (57, N))
    check_against_oracle(q, prep, A, kernel_hint=hint, split_k_hint=split, tile_hint=tile, bias=b)
    # zero activations: the output is exactly the bias in every row (both output types)
    y32, _ = run_gpu(q, prep, T.zeros_like(A), q.DT_F32, hint, split, bias=b, tile_hint=tile)
    assert np.array_equal(y32, np.tile(b.to(T.float64).numpy(), (M, 1)))
    y16, _ = run_gpu(q, prep, T.zeros_like(A), out16_dtype(q, fmt), hint, split, bias=b, tile_hint=tile)
    assert np.array_equal(y16, np.tile(b.view(T.int16).numpy().view(np.uint16), (M, 1)))


def test_bias_null_is_plain_run_bitwise(q):
    # qgemm_run_bias with a NULL bias is exactly qgemm_run
    import torch as T
    N, K, M = 256, 1024, 16
    prep = Prepared(q, "fp8h", N, K, 0, (58, N, K))
    A = _act("fp8h", M, K, (58, M)).cuda()
    p = q.problem(M, N, K, "fp8h", out_dtype=q.DT_F32)
    o1 = T.empty((M, N), dtype=T.float32, device="cuda")
    o2 = T.empty_like(o1)
    ws = q.alloc_workspace(p)
    q.run(p, A, prep.w, None, prep.alpha_t, o1, ws)
    st = q.run_bias_raw(p, A.data_ptr(), prep.w.data_ptr(), None, prep.alpha_t.data_ptr(), None, o2.data_ptr(),
                        None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel(),
                        T.cuda.current_stream().cuda_stream)
    assert st == q.OK, q.last_error()
    T.cuda.synchronize()
    assert T.equal(o1, o2)


@pytest.mark.parametrize("hint,M", [(1, 1), (1, 4), (1, 16), (2, 64)])
def test_nf4_any_code_book_bit_exact(q, hint, M):
    # The kernels read the code book from the packed scales: with a random book (every entry
    # its own sign and magnitude), random codes and random scales, identity activations must
    # return RNE_fp16(T[code] * s) exactly for every code in every nibble slot.
    import torch as T
    from oracle import quant
    N, K, G = 64, 512, 64
    say(f"case nf4-any-book hint={hint} M={M}")
    g = np.random.default_rng([59, hint, M])
    mag = np.exp2(g.uniform(-4, 2, 16))
    book = codecs.f16_bits(codecs.f16_round(mag * g.choice([-1.0, 1.0], 16)))
    codes = g.integers(0, 16, (N, K)).astype(np.uint8)
    sbits = codecs.f16_bits(codecs.f16_round(np.exp2(g.uniform(-8, 1, (K // G, N)))))
    p = q.problem(M, N, K, "nf4", group_size=G, out_dtype=q.DT_F32, kernel_hint=hint)
    wpk, spk = q.pack(p, quant.pack_nibbles(codes), np.concatenate([book, sbits.reshape(-1)]))
    want = reference.dequant_nf4_f16(codes, sbits, G, book)          # [N, K]
    w_d, s_d = T.from_numpy(wpk).cuda(), T.from_numpy(spk).cuda()
    ws = q.alloc_workspace(p)
    for k0 in range(0, K, M):
        rows = list(range(k0, min(k0 + M, K)))
        A = _identity_rows("nf4", rows, K)
        pr = q.problem(len(rows), N, K, "nf4", group_size=G, out_dtype=q.DT_F32, kernel_hint=hint)
        out = T.full((len(rows), N), float("nan"), dtype=T.float32, device="cuda")
        q.run(pr, A.cuda(), w_d, s_d, None, out, ws)
        T.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().astype(np.float64), want[:, rows].T), f"rows {k0}.."


@pytest.mark.parametrize("fmt,G,M,N,K", [("int4", 128, 1000, 4048, 1024), ("fp8", None, 2000, 2560, 640),
                                         ("int4", 64, 520, 4096, 2048), ("fp4", None, 1024, 2048, 2048),
                                         ("int4", 256, 200, 2048, 1024), ("fp8h", None, 300, 4112, 512),
                                         ("nf4", 128, 257, 1024, 2048), ("int4", 128, 17, 4096, 4096),
                                         ("fp4", None, 64, 8192, 2048), ("int2", 32, 100, 2064, 1024),
                                         ("fp8", None, 128, 3072, 1536)])
def test_mid_m_auto_plan(q, fmt, G, M, N, K):
    # Shapes between decode and the large tiles, where the planner's time model picks the tile
    # (64 x 128, 128 x 128 or 256 x 256) and the K split; every row is checked.
    say(f"case mid-m fmt={fmt} G={G} M={M} N={N} K={K}")
    prep = Prepared(q, fmt, N, K, G or 0, (61, N, K))
    A = _act(fmt, M, K, (61, M))
    st, _ = check_against_oracle(q, prep, A)
    say(f"  E1={st['E1']:.3e} worstE2={st['E2_worst_ratio']:.3f}")


STREAMK_CASES = [
    # (format, G, M, N, K, tile rows): tiles vs resident workgroups (256 for every tile: one
    # workgroup per CU, as each tile's A stages take at least 96 KiB of LDS): a tail of whole
    # rounds plus a part, and far fewer tiles than workgroups (every tile cut among several
    # workgroups)
    ("fp8", None, 4352, 4096, 1024, 256),      # 17 x 16 = 272 tiles: 16 whole + 16 split in K
    ("int4", 64, 4352, 4112, 768, 256),        # ragged N: 17 x 17 = 289 tiles
    ("fp4", None, 2176, 2048, 1024, 128),      # 17 x 16 = 272 medium tiles
    ("nf4", 128, 2112, 2048, 512, 64),         # 33 x 16 = 528 small tiles: 256 whole + 272 split
    ("int2", 32, 600, 784, 1024, 64),          # 10 x 7 = 70 tiles over 256 workgroups
    ("fp8h", None, 300, 272, 2048, 256),       # 2 x 2 tiles, 16 k blocks each, over 256 workgroups
    ("int4", 128, 1000, 4048, 1024, 128),      # 8 x 32 = 256 = one full round, no tail
]


@pytest.mark.parametrize("fmt,G,M,N,K,tile", STREAMK_CASES,
                         ids=[f"{c[0]}-{c[2]}x{c[3]}x{c[4]}-t{c[5]}" for c in STREAMK_CASES])
def test_prefill_persistent_stream_k(q, fmt, G, M, N, K, tile):
    # The persistent prefill schedule (whole tiles round-robin, then the tail tiles' k blocks
    # split evenly over the resident workgroups with a ticketed hand-off of fp32 partials):
    # every row against the oracle, bitwise identical on a second run, tickets back at zero.
    say(f"case stream-k fmt={fmt} G={G} M={M} N={N} K={K} tile={tile}")
    prep = Prepared(q, fmt, N, K, G or 0, (64, N, K))
    A = _act(fmt, M, K, (64, M))
    st, y0 = check_against_oracle(q, prep, A, kernel_hint=3, tile_hint=tile)
    y1, ws = run_gpu(q, prep, A, q.DT_F32, kernel_hint=3, tile_hint=tile)
    assert np.array_equal(y0, y1)
    p = q.problem(M, N, K, fmt, group_size=G, kernel_hint=3, tile_hint=tile)
    assert ws is not None and q.workspace_bytes(p) > 0
    T = -(-N // (256 if tile == 256 else 128)) * -(-M // tile)          # output tiles
    P = int(q.plan_fields(p)["persist"])                                 # resident workgroups
    assert P == 256, P
    tail = T - ((T // P - 1) * P if T > P else 0)                        # tiles with tickets
    assert not ws[:4 * tail].cpu().numpy().any(), "stream-K tickets must return to zero"
    say(f"  E1={st['E1']:.3e} worstE2={st['E2_worst_ratio']:.3f}")


def test_split_k_under_concurrent_load(q):
    # Split-K must not rely on its workgroups being resident together (FlashInfer PR #7495
    # analysis, section 3(d)): with a long GEMM occupying compute units from another stream,
    # split-K decode and prefill launches still finish and give bitwise the results of an
    # isolated run.
    import torch as T
    say("case split-k under concurrent load")
    cases = [("int4", 1, 256, 128 * 64, 128, 1, 16), ("fp4", 128, 2048, 8192, 0, 2, 4),
             ("fp8", 16, 512, 128 * 40, 0, 1, 5), ("fp8", 300, 272, 2048, 0, 3, 0)]
    preps = []
    for fmt, M, N, K, G, hint, split in cases:
        prep = Prepared(q, fmt, N, K, G, (62, N, K))
        A = _act(fmt, M, K, (62, M))
        y0, ws = run_gpu(q, prep, A, q.DT_F32, kernel_hint=hint, split_k_hint=split)
        preps.append((prep, A, hint, split, y0, ws))
    x = T.randn((8192, 8192), dtype=T.float16, device="cuda")
    y = T.randn((8192, 8192), dtype=T.float16, device="cuda")
    side = T.cuda.Stream()                       # default priority
    side.wait_stream(T.cuda.current_stream())
    with T.cuda.stream(side):
        for _ in range(8):
            z = T.mm(x, y)
    for _ in range(3):
        for prep, A, hint, split, y0, ws in preps:
            y1, _ = run_gpu(q, prep, A, q.DT_F32, kernel_hint=hint, split_k_hint=split, workspace=ws)
            assert np.array_equal(y1, y0)
            assert not ws[:256].cpu().numpy().any()
    side.synchronize()
    del z


@pytest.mark.parametrize("fmt,M,N,K,hint,split,tile", [("int4", 1, 256, 128 * 64, 1, 16, 0),
                                                       ("fp8", 16, 512, 128 * 40, 1, 5, 2),
                                                       ("fp4", 128, 2048, 8192, 2, 4, 128),
                                                       ("nf4", 300, 272, 1024, 2, 3, 64),
                                                       ("fp8", 4352, 4096, 1024, 3, 0, 256),
                                                       ("int2", 600, 784, 1024, 3, 0, 64)])
def test_workspace_guard_bytes_survive(q, fmt, M, N, K, hint, split, tile):
    # The workspace handed over is the planned size plus 64 KiB of guard bytes: no split-K or
    # stream-K hand-off (tickets or partial tiles) writes past the size qgemm_workspace_bytes
    # reports, and the tickets are back at zero afterwards.
    import torch as T
    G = {"int4": 128, "int2": 32, "nf4": 64}.get(fmt, 0)
    say(f"case workspace guard fmt={fmt} M={M} N={N} K={K} hint={hint} split={split} tile={tile}")
    prep = Prepared(q, fmt, N, K, G, (65, N, K))
    A = _act(fmt, M, K, (65, M))
    p = q.problem(M, N, K, fmt, group_size=G or None, kernel_hint=hint, split_k_hint=split, tile_hint=tile)
    need = q.workspace_bytes(p)
    assert need > 0
    ws = T.zeros(need + 65536, dtype=T.uint8, device="cuda")
    ws[need:] = 0xA5
    y = []
    for odt in (q.DT_F32, out16_dtype(q, fmt)):
        y.append(run_gpu(q, prep, A, odt, hint, split, workspace=ws, tile_hint=tile)[0])
    tail = ws[need:].cpu().numpy()
    assert (tail == 0xA5).all(), f"{int((tail != 0xA5).sum())} guard bytes overwritten"
    head = ws[:256].cpu().numpy()
    assert not head.any()
    # the fp32 result itself is right (the run with the exact workspace is covered elsewhere)
    from oracle import reference
    r = reference.gemm_fp64(A.to(T.float64).numpy(), prep.wdq, prep.alpha)
    tolerance.check_e1_e2(y[0], r)
