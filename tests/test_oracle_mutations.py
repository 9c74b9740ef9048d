"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of an oracle module (a dropped term, a
wrong sign, a swapped index, a wrong slice, a wrong constant) and reruns the
pin tests of that module against the copy.  At least one pin must fail for
every planted mistake.  Only the CPU oracle is mutated; nothing here touches
the HIP library.
"""

import importlib
import importlib.util
import inspect
import json
import os
import types

import pytest

from conftest import ROOT

# mutants may produce NaN or overflow on the way to failing a pin
pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _mutant(modname, old, new, extra=None):
    src = inspect.getsource(importlib.import_module(modname))
    assert src.count(old) == 1, (modname, old)
    src = src.replace(old, new)
    mod = types.ModuleType(modname + "_mutant")
    mod.__package__ = "oracle"
    exec(compile(src, modname + "_mutant.py", "exec"), mod.__dict__)
    for k, v in (extra or {}).items():
        setattr(mod, k, v)
    return mod


def _golden():
    with open(os.path.join(ROOT, "tests", "golden", "page_figures.json")) as f:
        return json.load(f)


_ARGS = {"golden": _golden, "cuts": lambda: [0, 5, 40], "seed": lambda: 3}


def _failures(test_modname, alias, mutant, monkeypatch):
    """Run every pin of ``test_modname`` with ``alias`` bound to ``mutant``;
    return the names of the pins that failed."""
    tm = importlib.import_module(test_modname)
    monkeypatch.setattr(tm, alias, mutant)
    failed = []
    for name, fn in inspect.getmembers(tm, inspect.isfunction):
        if not name.startswith("test_") or fn.__module__ != tm.__name__:
            continue
        kwargs = {p: _ARGS[p]() for p in inspect.signature(fn).parameters}
        try:
            fn(**kwargs)
        except Exception:
            failed.append(name)
    return failed


ATTENTION_MUTANTS = [
    ("dropped softmax scale", "s = scale * (qh @ K.T)", "s = (qh @ K.T)"),
    ("wrong sign in the exponent", "e = np.exp(s - m)", "e = np.exp(m - s)"),
    ("log2 instead of ln in lse", "lse = (m + np.log(l))[:, 0]", "lse = (m + np.log2(l))[:, 0]"),
    ("missing normalisation", "out = (e @ V) / l", "out = (e @ V)"),
    ("transposed score operand", "s = scale * (qh @ K.T)", "s = scale * (K @ qh.T).T[:, ::-1]"),
    ("V taken from the wrong dims", "o, ls = attend(qh, Kf, Kf[:, :D_V], softmax_scale)",
     "o, ls = attend(qh, Kf, Kf[:, D_QK - D_V:], softmax_scale)"),
    ("RoPE dims dropped from K", "o, ls = attend(qh, Kf, Kf[:, :D_V], softmax_scale)",
     "o, ls = attend(qh[:, :D_V], Kf[:, :D_V], Kf[:, :D_V], softmax_scale)"),
    ("page and offset swapped", "[t // BLOCK] * BLOCK + t % BLOCK", "[t % BLOCK] * BLOCK + t // BLOCK"),
    ("-1 indices not masked", "idx[(idx >= 0) & (idx < num_rows)]", "idx[(idx >= -1) & (idx < num_rows)]"),
    ("merge weights swapped", "a2 = np.where(safe, np.exp(np.where(safe, d2, 0.0)), 0.0) * l2",
     "a2 = np.where(safe, np.exp(np.where(safe, d1, 0.0)), 0.0) * l2"),
    ("online rescale dropped", "acc = acc * alpha + p * V[j]", "acc = acc + p * V[j]"),
    ("lse written to the wrong head", "lse[b, :, i] = ls", "lse[b, :, i] = ls[::-1]"),
]


@pytest.mark.parametrize("what,old,new", ATTENTION_MUTANTS, ids=[m[0] for m in ATTENTION_MUTANTS])
def test_attention_pins_catch(what, old, new, monkeypatch):
    mut = _mutant("oracle.attention", old, new)
    assert _failures("test_oracle_attention", "A", mut, monkeypatch), what


def test_causal_offset_mistake_is_caught(monkeypatch):
    sched_mut = _mutant("oracle.sched", "int(L) - s_q + 1 + i", "int(L) - s_q + i")
    mut = _mutant("oracle.attention", "D_QK = 576", "D_QK = 576", extra={"visible_len": sched_mut.visible_len})
    assert _failures("test_oracle_attention", "A", mut, monkeypatch)


FP8_MUTANTS = [
    ("scale tile of 64 dims", "tile_scale = np.repeat(scales, TILE, axis=1)",
     "tile_scale = np.repeat(scales, TILE // 2, axis=1)[:, :LATENT] if False else np.tile(scales, (1, TILE))"),
    ("RoPE read from the scale bytes", "rope_bits = np.ascontiguousarray(flat[:, ROPE_OFFSET:])",
     "rope_bits = np.ascontiguousarray(flat[:, SCALE_OFFSET:SCALE_OFFSET + 2 * ROPE])"),
    ("scale applied after rounding", "prod = (vals * tile_scale).astype(np.float32)",
     "prod = (f32_to_bf16_bits_rne(vals).astype(np.float32) * 0 + vals * tile_scale * 1.0001).astype(np.float32)"),
    # 528-byte records
    ("e8m0 bias 128", "out = np.ldexp(1.0, e - 127)", "out = np.ldexp(1.0, e - 128)"),
    ("528-byte scales in reverse order", "out = vals * np.repeat(scales, V41_GROUP, axis=1)",
     "out = vals * np.repeat(scales[:, ::-1], V41_GROUP, axis=1)"),
    # 288-byte FP4 records
    ("FP4 nibbles swapped", "codes[:, 0::2] = packed & 0xF          # even index: low nibble\n    codes[:, 1::2] = packed >> 4",
     "codes[:, 0::2] = packed >> 4\n    codes[:, 1::2] = packed & 0xF"),
    ("FP4 scale group of 32 values", "out = e2m1_decode(codes) * np.repeat(scales, FP4_GROUP, axis=1)",
     "out = e2m1_decode(codes) * np.repeat(scales[:, :16], 2 * FP4_GROUP, axis=1)"),
    ("FP4 scales read from the code bytes", "scales = e4m3fn_decode(flat[:, FP4_DIM // 2:])",
     "scales = e4m3fn_decode(flat[:, :FP4_DIM // 16])"),
    ("e2m1 exponent bias 0", "np.ldexp(1.0 + 0.5 * m, (e - 1).astype(np.int32))",
     "np.ldexp(1.0 + 0.5 * m, e.astype(np.int32))"),
    ("e2m1 subnormal read as normal", "mag = np.where(e == 0, 0.5 * m,", "mag = np.where(e == 0, 1.0 * m,"),
    ("e2m1 sign from bit 2", "sign = np.where(c & 8, -1.0, 1.0)", "sign = np.where(c & 4, -1.0, 1.0)"),
]


@pytest.mark.parametrize("what,old,new", FP8_MUTANTS, ids=[m[0] for m in FP8_MUTANTS])
def test_fp8_pins_catch(what, old, new, monkeypatch):
    src = inspect.getsource(importlib.import_module("oracle.fp8cache"))
    if src.count(old) != 1:
        pytest.fail(f"mutation site for '{what}' is not unique in oracle/fp8cache.py")
    mut = _mutant("oracle.fp8cache", old, new)
    assert _failures("test_oracle_numerics", "F8", mut, monkeypatch), what


SCHED_MUTANTS = [
    ("partition size rounded down", "q = max(1, -(-T // P))", "q = max(1, T // P)"),
    ("fixed cost not skipped at the end", "te = min(max(0, hi - int(C[je]) - F), int(n[je]))",
     "te = min(max(0, hi - int(C[je])), int(n[je]))"),
]


@pytest.mark.parametrize("what,old,new", SCHED_MUTANTS, ids=[m[0] for m in SCHED_MUTANTS])
def test_sched_pins_catch(what, old, new, monkeypatch):
    src = inspect.getsource(importlib.import_module("oracle.sched"))
    if src.count(old) != 1:
        pytest.fail(f"mutation site for '{what}' is not unique in oracle/sched.py")
    mut = _mutant("oracle.sched", old, new)
    assert _failures("test_oracle_sched", "S", mut, monkeypatch), what
