"""Planted mistakes in the oracle (CPU): the pins must catch them.

Each mutant replaces one oracle function with a plausible wrong version of it — an
off-by-one zero point, the scale of the neighbouring group, a dropped or mis-scaled factor,
a dropped K term, swapped nibbles or table entries, truncation for round-to-nearest-even, a
wrong exponent bias, a layout shifted by one lane — and runs the existing pins of that
part of the oracle (tests/test_oracle_*.py) against it: at least one pin must fail.  So the
pins constrain each function from outside (brute force, closed forms, library casts,
hand-worked fixtures) rather than restating it.  Mutants are planted only here, on the CPU,
through monkeypatch; nothing else sees them."""
import inspect

import numpy as np
import pytest

import test_oracle_codecs
import test_oracle_gemm
import test_oracle_layout
import test_oracle_quant
from oracle import codecs, layout, quant, reference


def _pins(*modules):
    """Every pin of the modules as (name, zero-argument call); a parametrized pin once per case."""
    out = []
    for mod in modules:
        for name, fn in inspect.getmembers(mod, inspect.isfunction):
            if not name.startswith("test_") or fn.__module__ != mod.__name__:
                continue
            marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
            if marks:
                names = [a.strip() for a in marks[0].args[0].split(",")]
                for v in marks[0].args[1]:
                    v = v if isinstance(v, tuple) else (v,)
                    out.append((f"{name}{v}", lambda fn=fn, v=v, names=names: fn(**dict(zip(names, v)))))
            elif not inspect.signature(fn).parameters:
                out.append((name, fn))
    return out


def _first_failing(pins):
    for name, call in pins:
        try:
            call()
        except Exception:        # an assertion, or an error the planted mistake causes
            return name
    return None


def _s_nk(scale_bits, group):
    return np.repeat(codecs.f16_from_bits(scale_bits).T, group, axis=1)


# (name, module, attribute, mutant factory taking the original function, pin modules)
MUTANTS = [
    # dequantization and the fp64 GEMM
    ("int4 zero point 7", reference, "dequant_int4",
     lambda f: lambda c, s, g: f(c, s, g) + _s_nk(s, g).astype(np.float32), [test_oracle_gemm]),
    ("int4 scale of the next group", reference, "dequant_int4",
     lambda f: lambda c, s, g: f(c, np.roll(s, 1, axis=0), g), [test_oracle_gemm]),
    ("int4 scale of the next column", reference, "dequant_int4",
     lambda f: lambda c, s, g: f(c, np.roll(s, 1, axis=1), g), [test_oracle_gemm]),
    ("int2 zero point 1", reference, "dequant_int2",
     lambda f: lambda c, s, g: f(c, s, g) + _s_nk(s, g).astype(np.float32), [test_oracle_gemm]),
    ("nf4 neighbouring book entry", reference, "dequant_nf4",
     lambda f: lambda c, s, g, b: f(np.asarray(c) ^ 1, s, g, b), [test_oracle_gemm]),
    ("fp8 sign dropped", reference, "dequant_fp8",
     lambda f: lambda c: np.abs(f(c)), [test_oracle_gemm]),
    ("fp4 block scale dropped", reference, "dequant_fp4",
     lambda f: lambda c, sf: codecs.e2m1_decode(c).astype(np.float32), [test_oracle_gemm]),
    ("fp4 scale of the next block", reference, "dequant_fp4",
     lambda f: lambda c, sf: f(c, np.roll(sf, 1, axis=1)), [test_oracle_gemm]),
    ("gemm alpha ignored", reference, "gemm_fp64",
     lambda f: lambda a, w, alpha=1.0, bias=None: f(a, w, 1.0, bias), [test_oracle_gemm]),
    ("gemm bias dropped", reference, "gemm_fp64",
     lambda f: lambda a, w, alpha=1.0, bias=None: f(a, w, alpha, None), [test_oracle_gemm]),
    ("gemm last K term dropped", reference, "gemm_fp64",
     lambda f: lambda a, w, alpha=1.0, bias=None: f(np.asarray(a)[:, :-1], np.asarray(w)[:, :-1], alpha, bias),
     [test_oracle_gemm]),
    ("gemm weight not transposed", reference, "gemm_fp64",
     lambda f: lambda a, w, alpha=1.0, bias=None: f(a, np.asarray(w)[::-1], alpha, bias), [test_oracle_gemm]),
    # quantizers and canonical packing
    ("int4 stored code off by one", quant, "quantize_int4",
     lambda f: lambda w, g: (lambda c, s: ((c.astype(np.int64) - 1).clip(0, 15).astype(np.uint8), s))(*f(w, g)),
     [test_oracle_quant]),
    ("int4 scale of the next group", quant, "quantize_int4",
     lambda f: lambda w, g: (lambda c, s: (c, np.roll(s, 1, axis=0)))(*f(w, g)), [test_oracle_quant]),
    ("nibbles swapped in a byte", quant, "pack_nibbles",
     lambda f: lambda c: (lambda b: ((b >> 4) | (b << 4)).astype(np.uint8))(f(c)), [test_oracle_quant]),
    ("crumbs reversed in a byte", quant, "pack_crumbs",
     lambda f: lambda c: (lambda b: (((b & 3) << 6) | ((b & 12) << 2) | ((b >> 2) & 12) | (b >> 6)).astype(np.uint8))(f(c)),
     [test_oracle_quant]),
    ("fp8 alpha halved", quant, "quantize_fp8",
     lambda f: lambda w: (lambda c, a: (c, a * 0.5))(*f(w)), [test_oracle_quant]),
    ("fp4 alpha off", quant, "quantize_fp4",
     lambda f: lambda w: (lambda c, sf, a: (c, sf, a * 1.5))(*f(w)), [test_oracle_quant]),
    ("nf4 book reversed", quant, "nf4_codebook",
     lambda f: lambda: f()[::-1].copy(), [test_oracle_quant]),
    ("int2 stored code off by one", quant, "quantize_int2",
     lambda f: lambda w, g: (lambda c, s: ((c.astype(np.int64) + 1).clip(0, 3).astype(np.uint8), s))(*f(w, g)),
     [test_oracle_quant]),
    # codecs
    ("fp16 truncation", codecs, "f16_round",
     lambda f: lambda x: f((np.asarray(x, np.float32).view(np.uint32) & np.uint32(0xFFFFE000)).view(np.float32)),
     [test_oracle_codecs]),
    ("bf16 truncation", codecs, "bf16_round",
     lambda f: lambda x: f((np.asarray(x, np.float32).view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)),
     [test_oracle_codecs]),
    ("e4m3 exponent bias 8", codecs, "e4m3_decode",
     lambda f: lambda c: f(c) * 0.5, [test_oracle_codecs]),
    ("e2m1 table entries 5 and 6 swapped", codecs, "e2m1_decode",
     lambda f: lambda c: f(np.where(np.asarray(c) % 8 == 5, np.asarray(c) + 1,
                                    np.where(np.asarray(c) % 8 == 6, np.asarray(c) - 1, np.asarray(c)))),
     [test_oracle_codecs]),
    # device layout model
    ("int4 fragment shifted one lane", layout, "device_int4_weights",
     lambda f: lambda *a, **k: np.roll(f(*a, **k), 16), [test_oracle_layout]),
    ("fp4 fragment shifted one lane", layout, "device_fp4_weights",
     lambda f: lambda *a, **k: np.roll(f(*a, **k), 16), [test_oracle_layout]),
    ("fp8 fragment shifted one lane", layout, "device_fp8_weights",
     lambda f: lambda *a, **k: np.roll(f(*a, **k), 16), [test_oracle_layout]),
    ("int2 fragment shifted one lane", layout, "device_int2_weights",
     lambda f: lambda *a, **k: np.roll(f(*a, **k), 8), [test_oracle_layout]),
    ("int4 scales shifted one column", layout, "device_int4_scales",
     lambda f: lambda *a, **k: np.roll(f(*a, **k), 2), [test_oracle_layout]),
    ("fp4 scales shifted one column", layout, "device_fp4_scales",
     lambda f: lambda *a, **k: np.roll(f(*a, **k), 8), [test_oracle_layout]),
]


def test_every_pin_passes_on_the_oracle_itself():
    # the premise: unmutated, no pin fails (so a failure below is the mutant's doing)
    assert _first_failing(_pins(test_oracle_gemm, test_oracle_quant, test_oracle_codecs, test_oracle_layout)) is None


@pytest.mark.parametrize("mi", range(len(MUTANTS)), ids=[m[0] for m in MUTANTS])
def test_a_planted_mistake_fails_a_pin(monkeypatch, mi):
    _, module, attr, factory, pin_modules = MUTANTS[mi]
    monkeypatch.setattr(module, attr, factory(getattr(module, attr)))
    assert _first_failing(_pins(*pin_modules)) is not None, "no pin caught the planted mistake"
