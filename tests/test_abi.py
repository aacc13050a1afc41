"""C-ABI contract on the CPU: exported symbols, status strings, validation errors that
return before anything is enqueued, workspace sizing.  No kernel is launched here."""
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import weight_only_quantized_qgemm_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(qgemm_[a-z_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert set(names) >= {"qgemm_pack", "qgemm_run", "qgemm_run_bias", "qgemm_workspace_bytes", "qgemm_quantize",
                          "qgemm_status_string", "qgemm_last_error", "qgemm_version"}
    for n in names:
        assert hasattr(q.lib, n), n


def test_import_fails_loudly_without_the_library():
    # no fallback: without the HIP library the binding refuses to load at all
    env = dict(os.environ, QGEMM_LIB_PATH=os.path.join(ROOT, "_no_such_dir", "libqgemm.so"))
    r = subprocess.run([sys.executable, "-c", "import weight_only_quantized_qgemm_amd"], capture_output=True,
                       text=True, cwd=ROOT, env=env, timeout=300)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "is missing" in r.stderr and "_build" in r.stderr


def test_status_strings_and_version():
    assert q.status_string(q.OK) == "QGEMM_OK"
    assert q.status_string(q.ERR_MISALIGNED) == "QGEMM_ERR_MISALIGNED"
    assert q.status_string(99) == "QGEMM_ERR_UNKNOWN_STATUS"
    assert q.version() >= 100


BAD = [
    (dict(M=-1, N=256, K=512, fmt="int4"), q.ERR_INVALID_ARGUMENT, "M must be"),
    (dict(M=(1 << 24) + 1, N=256, K=512, fmt="int4"), q.ERR_INVALID_ARGUMENT, "M must be"),
    (dict(M=1, N=(1 << 24) + 16, K=512, fmt="int4"), q.ERR_INVALID_ARGUMENT, "N must be"),
    (dict(M=1, N=256, K=(1 << 24) + 128, fmt="int4"), q.ERR_INVALID_ARGUMENT, "K must be"),
    (dict(M=4096, N=256, K=1 << 24, fmt="int4"), q.ERR_UNSUPPORTED, "prefill kernel needs"),
    (dict(M=4096, N=256, K=1 << 23, fmt="int4", tile_hint=128), q.ERR_UNSUPPORTED, "prefill kernel needs"),
    (dict(M=1, N=250, K=512, fmt="int4"), q.ERR_INVALID_ARGUMENT, "N must be"),
    (dict(M=1, N=256, K=500, fmt="int4"), q.ERR_INVALID_ARGUMENT, "K must be"),
    (dict(M=1, N=256, K=640, fmt="int4", group_size=256), q.ERR_INVALID_ARGUMENT, "multiple of group_size"),
    (dict(M=1, N=256, K=512, fmt="int4", group_size=48), q.ERR_UNSUPPORTED, "group_size"),
    (dict(M=1, N=256, K=512, fmt="int4", out_dtype=q.DT_BF16), q.ERR_UNSUPPORTED, "INT4 weights need"),
    (dict(M=1, N=256, K=512, fmt="int2", out_dtype=q.DT_BF16), q.ERR_UNSUPPORTED, "INT2 weights need"),
    (dict(M=1, N=256, K=512, fmt="int2", group_size=16), q.ERR_UNSUPPORTED, "INT2 group_size"),
    (dict(M=1, N=256, K=512, fmt="nf4", out_dtype=q.DT_BF16), q.ERR_UNSUPPORTED, "NF4 weights need"),
    (dict(M=1, N=256, K=512, fmt="nf4", group_size=16), q.ERR_UNSUPPORTED, "NF4 group_size"),
    (dict(M=1, N=256, K=640, fmt="nf4", group_size=256), q.ERR_INVALID_ARGUMENT, "multiple of group_size"),
    (dict(M=1, N=256, K=512, fmt="fp8", out_dtype=q.DT_F16), q.ERR_UNSUPPORTED, "FP8_E4M3 weights need"),
    (dict(M=1, N=256, K=512, fmt="fp8h", out_dtype=q.DT_BF16), q.ERR_UNSUPPORTED, "FP8_E4M3 weights need"),
    (dict(M=1, N=256, K=512, fmt="fp8", group_size=128), q.ERR_INVALID_ARGUMENT, "group_size 0"),
    (dict(M=1, N=256, K=512, fmt="fp4", group_size=32), q.ERR_INVALID_ARGUMENT, "group_size 16"),
    (dict(M=17, N=256, K=512, fmt="int4", kernel_hint=q.KERNEL_DECODE), q.ERR_INVALID_ARGUMENT, "DECODE needs"),
    (dict(M=1, N=256, K=512, fmt="int4", kernel_hint=7), q.ERR_INVALID_ARGUMENT, "kernel_hint"),
    (dict(M=1, N=256, K=512, fmt="int4", kernel_hint=5), q.ERR_INVALID_ARGUMENT, "kernel_hint"),
    (dict(M=100, N=256, K=512, fmt="fp4", kernel_hint=4, tile_hint=128), q.ERR_INVALID_ARGUMENT, "PREFILL_TRANSFORM"),
    (dict(M=1, N=256, K=512, fmt="int4", split_k_hint=5), q.ERR_INVALID_ARGUMENT, "split_k_hint"),
    (dict(M=1, N=256, K=512, fmt="int4", split_k_hint=-1), q.ERR_INVALID_ARGUMENT, "split_k_hint"),
]


@pytest.mark.parametrize("kw,status,text", BAD)
def test_validation_errors(kw, status, text):
    p = q.problem(**kw)
    with pytest.raises(q.QgemmError) as ei:
        q.workspace_bytes(p)
    assert ei.value.status == status
    assert text in ei.value.detail


def test_empty_product_needs_nothing_and_launches_nothing():
    # M = 0: no workspace; qgemm_run validates the descriptor and returns without touching
    # (or checking) any pointer, so it needs no GPU.
    for fmt in ("int4", "int2", "nf4", "fp8", "fp8h", "fp4"):
        p = q.problem(0, 256, 512, fmt)
        assert q.workspace_bytes(p) == 0
        assert q.run_raw(p, None, None, None, None, None, None, 0, None) == q.OK
        assert q.run_bias_raw(p, None, None, None, None, None, None, None, 0, None) == q.OK
    p = q.problem(0, 250, 512, "int4")               # the descriptor is still checked
    assert q.run_raw(p, None, None, None, None, None, None, 0, None) == q.ERR_INVALID_ARGUMENT


def test_bad_enums_and_hints():
    p = q.problem(1, 256, 512, "int4")
    p.a_dtype = 17
    assert q.run_raw(p, 16, 16, 16, None, 16, None, 0, None) == q.ERR_INVALID_ARGUMENT
    p = q.problem(1, 256, 512, "int4", tile_hint=5)
    assert q.run_raw(p, 16, 16, 16, None, 16, None, 0, None) == q.ERR_INVALID_ARGUMENT
    p = q.problem(64, 256, 512, "int4", tile_hint=1)
    assert q.run_raw(p, 16, 16, 16, None, 16, None, 0, None) == q.ERR_INVALID_ARGUMENT
    p = q.problem(1, 256, 512, "int4")
    p.w_dtype = q.DT_F16
    assert q.run_raw(p, 16, 16, 16, None, 16, None, 0, None) == q.ERR_UNSUPPORTED


def _valid_run_status(p, A=0x1000, W=0x2000, S=0x3000, alpha=0x4000, out=0x5000, ws=None, wsb=0):
    return q.run_raw(p, A, W, S, alpha, out, ws, wsb, None)


def test_null_and_misaligned_pointers_fail_before_launch():
    p = q.problem(1, 256, 512, "int4")
    assert _valid_run_status(p, A=None) == q.ERR_INVALID_ARGUMENT
    assert _valid_run_status(p, S=None) == q.ERR_INVALID_ARGUMENT
    assert _valid_run_status(p, A=0x1008) == q.ERR_MISALIGNED
    assert "A must be 16-byte aligned" in q.last_error()
    assert _valid_run_status(p, W=0x2004) == q.ERR_MISALIGNED
    assert _valid_run_status(p, out=0x5002) == q.ERR_MISALIGNED
    f8 = q.problem(1, 256, 512, "fp8")
    assert _valid_run_status(f8, alpha=None) == q.ERR_INVALID_ARGUMENT
    assert _valid_run_status(f8, alpha=0x4002) == q.ERR_MISALIGNED     # 2 mod 4
    f4 = q.problem(1, 256, 512, "fp4")
    assert _valid_run_status(f4, S=0x3008) == q.ERR_MISALIGNED


def test_bias_needs_16_byte_alignment():
    # the FlashInfer fix (PR #7495 analysis, section 3(a)): a bias is 16-byte aligned, the
    # scalar alpha only 4; a misaligned bias fails before anything is enqueued
    for fmt in ("int4", "int2", "nf4", "fp8", "fp8h", "fp4"):
        p = q.problem(1, 256, 512, fmt)
        st = q.run_bias_raw(p, 0x1000, 0x2000, 0x3000, 0x4004, 0x6008, 0x5000, None, 0, None)
        assert st == q.ERR_MISALIGNED and "bias must be 16-byte aligned" in q.last_error()


def test_fp8_weights_pack_the_same_for_both_activation_types():
    g = np.random.default_rng(3)
    w = (g.standard_normal((64, 256)) * 0.05).astype(np.float32)
    pb, ph = q.problem(1, 64, 256, "fp8"), q.problem(1, 64, 256, "fp8h")
    cb, _, ab = q.quantize(pb, w)
    ch, _, ah = q.quantize(ph, w)
    assert np.array_equal(cb, ch) and ab == ah
    assert np.array_equal(q.pack(pb, cb, None)[0], q.pack(ph, ch, None)[0])


def test_scalar_alpha_needs_only_4_byte_alignment():
    # alpha at addr % 16 == 4 passes the alignment check: the call then fails only on the
    # deliberately missing workspace (a check that also precedes any launch)
    p = q.problem(16, 256, 4096, "fp8")
    need = q.workspace_bytes(p)
    assert need > 0
    st = _valid_run_status(p, alpha=0x4004, ws=None, wsb=0)
    assert st == q.ERR_WORKSPACE_TOO_SMALL, q.last_error()


def test_workspace_too_small_and_misaligned():
    p = q.problem(16, 256, 4096, "int4")
    need = q.workspace_bytes(p)
    assert need > 0
    assert _valid_run_status(p, ws=0x100000, wsb=need - 1) == q.ERR_WORKSPACE_TOO_SMALL
    assert _valid_run_status(p, ws=0x100010, wsb=need) == q.ERR_MISALIGNED


def test_workspace_sizes_do_not_depend_on_out_dtype():
    for fmt, o in (("int4", q.DT_F32), ("fp8", q.DT_F32), ("fp4", q.DT_F32)):
        for M in (1, 16, 128, 4096):
            a = q.workspace_bytes(q.problem(M, 8192, 8192, fmt))
            b = q.workspace_bytes(q.problem(M, 8192, 8192, fmt, out_dtype=o))
            assert a == b


def test_prefill_tile_workspace_sizes():
    # A split prefill needs one ticket per output tile (rounded to 256 bytes) plus one fp32
    # partial tile per tile and slice; each tile shape gives its own count.
    M, N, K = 600, 784, 1024
    for tile, bn in ((64, 128), (128, 128), (256, 256)):
        p = q.problem(M, N, K, "int4", kernel_hint=2, split_k_hint=3, tile_hint=tile)
        tiles = -(-M // tile) * -(-N // bn)
        assert q.workspace_bytes(p) == -(-tiles * 4 // 256) * 256 + tiles * 3 * tile * bn * 4, tile
        p.split_k_hint = 1
        assert q.workspace_bytes(p) == 0


def test_prefill_rows_up_to_64_use_the_64_row_tile():
    # With M <= 64 only the 64 x 128 tile is a candidate (a taller one would compute padding
    # rows only): the split workspace has that tile's geometry for any format and split.
    for fmt, M, N, K in (("int4", 17, 4096, 4096), ("fp8", 64, 10240, 5120), ("fp4", 33, 8192, 8192)):
        for s in (2, 5):
            p = q.problem(M, N, K, fmt, kernel_hint=2, split_k_hint=s)
            tiles = -(-N // 128)
            assert q.workspace_bytes(p) == -(-tiles * 4 // 256) * 256 + tiles * s * 64 * 128 * 4, (fmt, M, s)


def test_pack_size_query():
    assert q.packed_sizes(q.problem(1, 256, 512, "int4")) == (256 * 256, 256 * 4 * 2)
    assert q.packed_sizes(q.problem(1, 256, 512, "int4", group_size=32)) == (256 * 256, 256 * 16 * 2)
    assert q.packed_sizes(q.problem(1, 256, 512, "fp8")) == (256 * 512, 0)
    assert q.packed_sizes(q.problem(1, 256, 512, "fp4")) == (256 * 256, 256 * 32)
    assert q.packed_sizes(q.problem(1, 256, 512, "int2")) == (256 * 128, 256 * 4 * 2)
    assert q.packed_sizes(q.problem(1, 256, 512, "nf4", group_size=64)) == (256 * 256, 256 + 256 * 8 * 2)


def test_nf4_needs_its_scale_layout():
    # NF4 scales carry the code book: the plain group layout is refused, and INT4 does not
    # take the code-book layout
    p = q.problem(1, 256, 512, "nf4")
    p.scale_layout = q.SCALE_GROUP_F16
    assert _valid_run_status(p) == q.ERR_UNSUPPORTED and "GROUP_F16_LUT16" in q.last_error()
    p = q.problem(1, 256, 512, "int4")
    p.scale_layout = q.SCALE_GROUP_F16_LUT16
    assert _valid_run_status(p) == q.ERR_UNSUPPORTED
    p = q.problem(1, 256, 512, "nf4")
    assert _valid_run_status(p, S=None) == q.ERR_INVALID_ARGUMENT
    assert _valid_run_status(p, S=0x3008) == q.ERR_MISALIGNED
    p.scale_layout = 4
    assert _valid_run_status(p) == q.ERR_INVALID_ARGUMENT


def test_planner_sweep_sizes_are_consistent():
    # The launch planner over a grid of shapes, formats and hints (run also under the host
    # sanitizers by test_host_asan.py): every valid problem gets a plan, the workspace size is
    # a multiple of 256 plus whole fp32 tiles or 0, and forcing the persistent stream-K
    # schedule always asks for a workspace (its tickets and partial slots).
    sizes = [1, 2, 15, 16, 17, 64, 65, 128, 255, 300, 1000, 4097, 9000, 70000]
    for fmt in ("int4", "int2", "nf4", "fp8", "fp8h", "fp4"):
        for M in sizes:
            for N, K in ((16, 128), (272, 768), (4096, 4096), (12800, 5120), (256, 131072)):
                for hint, tile in ((0, 0), (2, 64), (2, 128), (2, 256), (3, 0), (3, 64), (4, 0), (4, 64)):
                    if hint == 2 and tile and tile * K * 2 >= 2 ** 31:
                        continue
                    p = q.problem(M, N, K, fmt, kernel_hint=hint, tile_hint=tile)
                    try:
                        ws = q.workspace_bytes(p)
                    except q.QgemmError as e:
                        assert e.status == q.ERR_UNSUPPORTED and "prefill kernel needs" in e.detail
                        continue
                    assert ws >= 0
                    if hint == 3:
                        assert ws > 0


def test_plan_describe_fields_and_errors():
    # qgemm_plan_describe: one line naming the kernel and its launch; an invalid problem
    # returns the validation status, a buffer too small for the line QGEMM_ERR_INVALID_ARGUMENT.
    import ctypes
    assert q.plan_describe(q.problem(0, 256, 512, "int4")) == "empty"
    d = q.plan_fields(q.problem(16, 4096, 4096, "int4"))
    assert d["kernel"] == "decode" and d["a"] == "dma" and int(d["splits"]) >= 1
    assert q.plan_fields(q.problem(1, 4096, 4096, "int4"))["a"] == "staged-early"
    assert q.plan_fields(q.problem(1, 11008, 4096, "int4"))["a"] == "staged"        # 688 workgroups
    d = q.plan_fields(q.problem(4096, 4096, 4096, "int4"))
    assert d["kernel"] == "prefill" and d["tile"] in ("64x128", "128x128", "256x256")
    assert q.plan_fields(q.problem(2176, 2048, 1024, "int4", kernel_hint=3))["persist"] != "0"
    # dedicated dequantization wavefronts: the 64 x 128 tile, one-tile launch, any M (also M <= 16)
    for M in (1, 100, 4096):
        d = q.plan_fields(q.problem(M, 2048, 1024, "fp4", kernel_hint=q.KERNEL_PREFILL_TRANSFORM))
        assert d["kernel"] == "prefill" and d["transform"] == "1" and d["tile"] == "64x128" and d["persist"] == "0", d
    assert q.plan_fields(q.problem(4096, 4096, 4096, "int4"))["transform"] == "0"
    with pytest.raises(q.QgemmError) as e:
        q.plan_describe(q.problem(16, 250, 512, "int4"))
    assert e.value.status == q.ERR_INVALID_ARGUMENT
    p = q.problem(16, 4096, 4096, "int4")
    buf = ctypes.create_string_buffer(8)
    assert q.lib.qgemm_plan_describe(ctypes.byref(p), buf, 8) == q.ERR_INVALID_ARGUMENT
    assert len(buf.value) == 7                        # truncated, still NUL-terminated
    assert q.lib.qgemm_plan_describe(ctypes.byref(p), None, 64) == q.ERR_INVALID_ARGUMENT


def test_decode_plans_fit_lds_and_take_dma_above_staging():
    # Decode plans: A is staged for M <= 4 and goes through the DMA slots above; the slots (two
    # sets when runs overlap), the dynamic region and the 2 KiB reserve for the kernel's other
    # LDS fit the 160 KiB of a workgroup; runs of KPW k blocks cover each wavefront's share.
    for fmt in ("int4", "int2", "nf4", "fp8", "fp8h", "fp4"):
        for M in (1, 4, 5, 9, 16):
            for N, K in ((16, 128), (272, 768), (4096, 4096), (11008, 4096), (4096, 14336), (12800, 5120),
                         (28672, 8192), (256, 131072)):
                for tile, split in ((0, 0), (1, 0), (4, 0), (2, 3)):
                    p = q.problem(M, N, K, fmt, kernel_hint=q.KERNEL_DECODE, tile_hint=tile, split_k_hint=split)
                    try:
                        d = q.plan_fields(p)
                    except q.QgemmError as e:
                        # a split hint too coarse for staging, or finer than K
                        assert "stages at most" in e.detail or "exceeds the" in e.detail, e.detail
                        continue
                    assert d["kernel"] == "decode"
                    assert d["a"] in (("staged", "staged-early") if M <= 4 else ("dma",)), (fmt, M, N, K, d)
                    if d["a"] == "staged-early":
                        g = [int(x) for x in d["grid"].split("x")]
                        assert d["cb"] == "1" and int(d["kpw"]) <= 5 and g[0] * g[1] <= 256, d
                    waves, kpw, runs = int(d["waves"]), int(d["kpw"]), int(d["runs"])
                    share = -(-int(d["kb_per_split"]) // waves)
                    assert 1 <= kpw <= share or share == 0
                    assert runs == 1 or (2 <= runs <= (8 if d["a"] == "dma" else 4) and -(-share // kpw) == runs)
                    if d["a"] == "dma":
                        sets = 2 if runs > 1 else 1
                        assert sets * waves * kpw * 4096 + int(d["lds"]) + 2048 <= 160 * 1024, (fmt, M, N, K, d)


def test_errors_and_plans_are_per_thread():
    # qgemm_last_error is per calling thread and the validation / planning code keeps no shared
    # state: eight threads (ctypes releases the GIL, so the calls overlap) interleave failing and
    # valid queries, and each reads back its own message and the same plans as a lone caller
    import threading
    bad = [q.problem(1, 250 + 16 * i, 512, "int4") for i in range(8)]       # N not a multiple of 16
    good = [q.problem(1 + 97 * i, 4096, 4096, "int4") for i in range(8)]
    want = [q.plan_describe(p) for p in good]
    errors = []

    def worker(i):
        try:
            for _ in range(300):
                assert q.run_raw(bad[i], 16, 16, 16, None, 16, None, 0, None) == q.ERR_INVALID_ARGUMENT
                msg = q.last_error()
                assert "N must be" in msg and str(250 + 16 * i) in msg, msg
                assert q.plan_describe(good[i]) == want[i]
                assert q.last_error() == ""
        except Exception as e:                     # reported on the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[0]
