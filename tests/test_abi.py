"""The C-ABI library loads, exports every declared entry point, and validates
arguments on the host (no GPU needed: mla_plan with an explicit CU count and
the argument checks that fail before any launch)."""

import ctypes
import os
import re

import pytest

from conftest import ROOT


def _declared():
    names = []
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            names += re.findall(r"^\s*(?:[\w\s\*]+?)\b(mla_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    from mla_decode_amd import _lib
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    from mla_decode_amd import _lib
    names = _declared()
    assert set(names) == set(_lib.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings(lib):
    assert lib.mla_abi_version() == 6
    for s in range(6):
        assert lib.mla_status_string(s)
    assert lib.mla_status_string(99) == b"unknown status"


def _problem(**kw):
    import mla_decode_amd as mla
    base = dict(batch=64, s_q=1, h_q=128, num_blocks=4096, max_blocks_per_seq=64)
    base.update(kw)
    args = {k: base.pop(k) for k in ("batch", "s_q", "h_q", "num_blocks", "max_blocks_per_seq")}
    return mla.make_problem(**args, **base)


def test_plan_host_only():
    import mla_decode_amd as mla
    # dense decode over a bf16 cache: 64 heads per workgroup
    m = mla.plan(_problem(), num_cus=256)
    assert m.num_head_blocks == 2 and m.num_partitions == 128 and m.fixed_overhead == 0
    assert m.max_splits == 64 + 128
    assert m.bytes == (8 + 5 * 128 + 64 + 1) * 4
    assert mla.workspace_bytes(m) == 192 * 128 * 513 * 4
    m = mla.plan(_problem(h_q=192), num_cus=256)
    assert m.num_head_blocks == 3 and m.num_partitions == 85
    m = mla.plan(_problem(h_q=16, batch=2, num_blocks=8, max_blocks_per_seq=4), num_cus=256)
    assert m.num_head_blocks == 1 and m.num_partitions == 256
    # top-k over a bf16 cache whose row offsets fit 32 bits: 64 heads per workgroup
    m = mla.plan(_problem(h_q=192, topk=2048), num_cus=256)
    assert m.num_head_blocks == 3 and m.num_partitions == 85
    # quantised formats and larger bf16 top-k caches: 128 heads per workgroup
    m = mla.plan(_problem(kv_format="fp8"), num_cus=256)
    assert m.num_head_blocks == 1 and m.num_partitions == 256
    m = mla.plan(_problem(h_q=192, topk=2048, num_blocks=58254), num_cus=256)   # (64 n + 2) 1152 < 2^32
    assert m.num_head_blocks == 3
    m = mla.plan(_problem(h_q=192, topk=2048, num_blocks=58255), num_cus=256)
    assert m.num_head_blocks == 2 and m.num_partitions == 128
    # the largest batches: 16384 query groups in all
    for kw in (dict(batch=16384), dict(batch=8192, s_q=2), dict(batch=4096, s_q=4, topk=64)):
        m = mla.plan(_problem(**kw), num_cus=256)
        assert m.bytes == (8 + 5 * m.num_partitions + 16384 + 1) * 4
    for tau in (0.0, 6.0, 8.0, 30.0):   # lazy-rescale thresholds in range
        assert mla.plan(_problem(rescale_threshold=tau), num_cus=256).num_partitions == 128


def test_struct_layout_matches_header():
    """The ctypes Problem mirrors mla_problem_t: 13 int32 fields then two floats."""
    from mla_decode_amd import _lib
    names = [f[0] for f in _lib.Problem._fields_]
    assert names[-2:] == ["softmax_scale", "rescale_threshold"]
    assert ctypes.sizeof(_lib.Problem) == 15 * 4
    src = open(os.path.join(ROOT, "include", "mla_decode.h")).read()
    body = src[src.index("typedef struct {\n    int32_t batch;"):src.index("} mla_problem_t;")]
    fields = re.findall(r"^\s*(int32_t|float)\s+(\w+);", body, flags=re.M)
    assert [n for _, n in fields] == names
    assert [t for t, _ in fields] == ["int32_t"] * 13 + ["float"] * 2


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), 1), (dict(s_q=0), 1), (dict(h_q=0), 1), (dict(num_blocks=0), 1),
    (dict(max_blocks_per_seq=0), 1), (dict(topk=-1), 1), (dict(softmax_scale=float("nan")), 1), (dict(softmax_scale=0.0), 1), (dict(softmax_scale=-0.5), 1),
    (dict(topk=64, causal=True), 2), (dict(batch=20000), 2), (dict(batch=16385), 2), (dict(batch=8193, s_q=2), 2),
    (dict(batch=4097, s_q=4, topk=64), 2),
    (dict(rescale_threshold=-1.0), 1), (dict(rescale_threshold=30.5), 1), (dict(rescale_threshold=float("nan")), 1),
    (dict(rescale_threshold=float("inf")), 1),
])
def test_plan_rejects(kw, status):
    import mla_decode_amd as mla
    with pytest.raises(mla.MlaError) as e:
        mla.plan(_problem(**kw), num_cus=256)
    assert e.value.status == status


def test_unsupported_shapes(lib):
    import mla_decode_amd as mla
    for field, val in (("h_kv", 2), ("d_qk", 512), ("d_v", 256), ("block_size", 32)):
        p = _problem()
        setattr(p, field, val)
        m = mla.Metadata()
        assert lib.mla_plan(ctypes.byref(p), 256, ctypes.byref(m)) == 2


def test_decode_rejects_bad_arguments_before_launch(lib):
    import mla_decode_amd as mla
    p = _problem()
    m = mla.plan(p, num_cus=256)
    ws = mla.workspace_bytes(m)
    fake = ctypes.c_void_p(1 << 20)       # never dereferenced: validation fails first
    # metadata has no device buffer
    assert lib.mla_decode_fwd(ctypes.byref(p), fake, fake, fake, fake, None, ctypes.byref(m), fake, ws, fake, fake,
                              None) == 1
    m.dev = 1 << 20
    # workspace too small
    assert lib.mla_decode_fwd(ctypes.byref(p), fake, fake, fake, fake, None, ctypes.byref(m), fake, ws - 1, fake,
                              fake, None) == 3
    # misaligned q
    assert lib.mla_decode_fwd(ctypes.byref(p), ctypes.c_void_p((1 << 20) + 2), fake, fake, fake, None,
                              ctypes.byref(m), fake, ws, fake, fake, None) == 1
    # metadata planned for another problem
    p2 = _problem(batch=32)
    assert lib.mla_decode_fwd(ctypes.byref(p2), fake, fake, fake, fake, None, ctypes.byref(m), fake, ws, fake, fake,
                              None) == 4
    # sparse entry point on a dense problem
    assert lib.mla_sparse_decode_fwd(ctypes.byref(p), fake, fake, fake, None, None, ctypes.byref(m), fake, ws, fake,
                                     fake, None) == 1
    # combine argument checks
    assert lib.mla_combine(0, 128, 1, fake, fake, fake, None, 0, fake, fake, None) == 1
    assert lib.mla_combine(3, 128, 2, fake, fake, fake, None, 0, fake, fake, None) == 1
    assert lib.mla_combine(4, 128, 2, fake, fake, fake, None, 7, fake, fake, None) == 1


def test_prefill_rejects_bad_arguments_before_launch(lib):
    import mla_decode_amd as mla
    fake = ctypes.c_void_p(1 << 20)       # never dereferenced: validation fails first
    p = mla.make_problem(1, 300, 128, 16, topk=600)
    m = mla.plan(p, num_cus=256)
    m.dev = 1 << 20
    ws = mla.workspace_bytes(m)
    call = lambda prob, s_kv: lib.mla_sparse_prefill_fwd(ctypes.byref(prob), s_kv, fake, fake, fake, None, None,
                                                         ctypes.byref(m), fake, ws, fake, fake, None)
    assert call(p, 0) == 1                 # empty cache
    assert call(p, 16 * 64 + 1) == 1       # more rows than num_blocks*64
    p2 = mla.make_problem(2, 150, 128, 16, topk=600)
    assert call(p2, 1000) == 1             # prefill is one sequence
    p3 = mla.make_problem(1, 300, 128, 16, max_blocks_per_seq=16)
    assert call(p3, 1000) == 1             # dense problem


@pytest.mark.parametrize("fmt", ["fp8_528", "fp4_288"])
def test_512_wide_records_need_the_512_wide_head_and_top_k(fmt):
    import mla_decode_amd as mla
    p = mla.make_problem(4, 2, 128, 64, topk=2048, kv_format=fmt)
    assert p.d_qk == 512
    assert mla.plan(p, num_cus=256).num_partitions == 256
    with pytest.raises(mla.MlaError) as e:                       # dense paged decode is not offered
        mla.plan(mla.make_problem(4, 1, 128, 64, 16, kv_format=fmt), num_cus=256)
    assert e.value.status == 2
    p.d_qk = 576                                                  # wrong head width for the format
    with pytest.raises(mla.MlaError) as e:
        mla.plan(p, num_cus=256)
    assert e.value.status == 2


def test_noalloc_step_rejects_oversized_plans_before_touching_the_device(lib):
    import mla_decode_amd as mla
    fake = ctypes.c_void_p(1 << 20)       # never dereferenced: the size check fails first
    p = _problem(batch=2048, num_blocks=4096, max_blocks_per_seq=64)   # 2176 split slots of 128 heads
    assert lib.mla_decode_step_noalloc(ctypes.byref(p), 256, fake, fake, fake, fake, None, None, fake, fake,
                                       None) == 3
    p = _problem(batch=0)
    assert lib.mla_decode_step_noalloc(ctypes.byref(p), 256, fake, fake, fake, fake, None, None, fake, fake,
                                       None) == 1


def test_decode_step_rejects_bad_arguments_before_touching_the_device(lib):
    import mla_decode_amd as mla
    fake = ctypes.c_void_p(1 << 20)       # never dereferenced: every call below fails on the host
    p = _problem()
    m = mla.plan(p, num_cus=256)
    m.dev = 1 << 20
    ws = mla._lib.load().mla_workspace_bytes(ctypes.byref(m))
    step = lib.mla_decode_step
    # no block table
    assert step(ctypes.byref(p), fake, fake, None, fake, None, None, ctypes.byref(m), fake, ws, fake, fake,
                None) == 1
    # metadata planned for another problem
    other = mla.plan(_problem(batch=32), num_cus=256)
    other.dev = 1 << 20
    assert step(ctypes.byref(p), fake, fake, fake, fake, None, None, ctypes.byref(other), fake, ws, fake, fake,
                None) == 4
    # workspace smaller than the plan needs
    assert step(ctypes.byref(p), fake, fake, fake, fake, None, None, ctypes.byref(m), fake, ws - 16, fake, fake,
                None) == 3
    # sparse: the scheduler call checks the metadata first
    ps = _problem(topk=2048)
    assert step(ctypes.byref(ps), fake, fake, fake, None, None, None, ctypes.byref(other), fake, ws, fake, fake,
                None) == 4
