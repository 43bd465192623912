"""The C-ABI library loads, exports every symbol include/recsa.h declares, and
rejects bad arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest
import torch  # noqa: F401  -- load torch's HIP runtime first, as the binding does

import long_context_recsa_amd as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "recsa.h")).read()
    return re.findall(r"RECSA_API\s+[\w\s\*]+?\b(recsa_\w+)\s*\(", txt)


def test_library_exports_every_declared_symbol():
    lib = R.load_library()
    names = _declared()
    assert len(names) == len(R.EXPORTED) and set(names) == set(R.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_single_hip_runtime_mapped():
    R.load_library()
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(libs) == 1, libs


def _p(**kw):
    base = dict(n_kv_heads=8, n_q_heads=32, head_dim=128, fanout_b=32, budget_k=8,
                capacity=524288 + 4096)
    base.update(kw)
    return R.make_params(**base)


def test_geometry_queries():
    p = _p()
    assert R.recsa_num_levels(p) == 3          # 528384 / 32^3 = 16
    assert R.recsa_max_candidates(p) == 8 * 32 + 31
    ko, vo, nc = R.recsa_tree_layout(p, 1)
    assert nc == 528384 // 32 and ko % 256 == 0 and vo % 256 == 0 and vo > ko
    assert R.recsa_tree_layout(p, 3)[2] == 16
    nbytes = R.recsa_tree_bytes(p)
    assert nbytes % 256 == 0
    # summaries of 3 levels (bf16 keys + values, fp32 means below the top) + RoPE table
    n1, n2, n3 = 16512, 516, 16
    want = 8 * 128 * (4 * (n1 + n2 + n3) + 4 * (n1 + n2)) + 288 * 64 * 8
    assert want <= nbytes <= want + 256 * 12
    assert R.recsa_workspace_bytes(p, 1000) == 0           # few rows: one workgroup per row
    rows = 4096 * 32                                         # a 4096-query prefill chunk
    ws = R.recsa_workspace_bytes(p, rows)
    # at least the per-row logits and one partial sum per (row, parent) of a level
    assert ws >= rows * (8 * 32 + 31) * 4 + rows * 9 * 128 * 4
    assert ws % 256 == 0
    assert R.recsa_workspace_bytes(_p(store="f32"), rows) == 0
    with pytest.raises(R.RecsaError):
        R.recsa_tree_layout(p, 4)
    assert R.recsa_num_levels(_p(capacity=31)) == 0
    assert R.recsa_num_levels(_p(fanout_b=2, capacity=1 << 20)) == 20


@pytest.mark.parametrize("kw", [
    dict(n_kv_heads=0), dict(n_q_heads=12), dict(head_dim=96), dict(fanout_b=1),
    dict(budget_k=0), dict(capacity=0), dict(capacity=1 << 31), dict(rope_base=-1.0),
])
def test_invalid_params_rejected(kw):
    p = _p(**kw)
    assert R.recsa_tree_bytes(p) == 0
    assert R.recsa_num_levels(p) == -1


def test_unsupported_candidate_count():
    p = _p(budget_k=200)        # 200*32 + 31 candidates per level > 4096
    d = R.recsa_tree_desc(256, 256, 256, 256, 0)
    with pytest.raises(R.RecsaError) as e:
        R.recsa_build_tree(p, d, 0)
    assert e.value.status == R.RECSA_ERR_UNSUPPORTED


def test_calls_validate_before_any_hip_call():
    p = _p(capacity=1000)
    fake = 1 << 20          # never dereferenced: every case below fails validation
    d = R.recsa_tree_desc(fake, fake, fake, fake, 0)
    cases = [
        (lambda: R.recsa_build_tree(p, R.recsa_tree_desc(None, fake, fake, fake, 0), 0), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_build_tree(p, R.recsa_tree_desc(fake + 8, fake, fake, fake, 0), 0), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_build_tree(p, R.recsa_tree_desc(fake, fake, fake + 16, fake, 0), 0), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_build_tree(p, d, 1001), R.RECSA_ERR_CAPACITY),
        (lambda: R.recsa_build_tree(p, d, -1), R.RECSA_ERR_CAPACITY),
        (lambda: R.recsa_append(p, R.recsa_tree_desc(fake, fake, fake, fake, 990), fake, fake, 11), R.RECSA_ERR_CAPACITY),
        (lambda: R.recsa_append(p, d, None, fake, 5), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_append(p, d, fake, fake, -1), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_decode(p, d, fake, 1, fake), R.RECSA_ERR_INVALID_ARG),      # empty tree
        (lambda: R.recsa_decode(p, R.recsa_tree_desc(fake, fake, fake, fake, 10), fake, 0, fake), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_decode(p, R.recsa_tree_desc(fake, fake, fake, fake, 10), None, 1, fake), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_decode(p, R.recsa_tree_desc(fake, fake, fake, fake, 10), fake + 4, 1, fake), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_prefill(p, R.recsa_tree_desc(fake, fake, fake, fake, 10), fake, 11, fake), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_prefill(p, R.recsa_tree_desc(fake, fake, fake, fake, 10), fake, 0, fake), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_decode(_p(n_q_heads=12), d, fake, 1, fake), R.RECSA_ERR_INVALID_ARG),
        # a bf16 prefill of 200 x 32 rows runs parent-major and needs its workspace
        (lambda: R.recsa_prefill(p, R.recsa_tree_desc(fake, fake, fake, fake, 990), fake, 200, fake), R.RECSA_ERR_INVALID_ARG),
    ]
    for i, (fn, status) in enumerate(cases):
        with pytest.raises(R.RecsaError) as e:
            fn()
        assert e.value.status == status, (i, str(e.value))
        assert str(e.value)
    # a rejected call leaves the descriptor unchanged
    d2 = R.recsa_tree_desc(fake, fake, fake, fake, 990)
    with pytest.raises(R.RecsaError):
        R.recsa_append(p, d2, fake, fake, 11)
    assert d2.length == 990


def test_status_strings():
    lib = R.load_library()
    for s in range(5):
        assert lib.recsa_status_string(s).decode().startswith("RECSA_")


def test_params_struct_layout():
    # offsets must match the C struct: 8 int32, double, 2 floats, int64
    assert ctypes.sizeof(R.recsa_params) == 56
    assert R.recsa_params.rope_base.offset == 32
    assert R.recsa_params.capacity.offset == 48
    assert ctypes.sizeof(R.recsa_tree_desc) == 40


def test_multi_decode_validates_before_any_hip_call():
    p = _p(capacity=1000)
    fake = 1 << 20
    assert R.recsa_multi_workspace_bytes(0) == 0
    assert R.recsa_multi_workspace_bytes(32) == 0        # the table travels with the launch
    assert R.recsa_multi_workspace_bytes(33) >= 33 * 32
    good = (R.recsa_tree_desc * 2)(R.recsa_tree_desc(fake, fake, fake, fake, 10),
                                   R.recsa_tree_desc(fake, fake, fake, fake, 20))
    empty = (R.recsa_tree_desc * 2)(R.recsa_tree_desc(fake, fake, fake, fake, 10),
                                    R.recsa_tree_desc(fake, fake, fake, fake, 0))
    over = (R.recsa_tree_desc * 1)(R.recsa_tree_desc(fake, fake, fake, fake, 1001))
    cases = [
        (lambda: R.recsa_decode_multi(p, None, 2, fake, fake, ws=fake), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_decode_multi(p, good, 0, fake, fake, ws=fake), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_decode_multi(p, empty, 2, fake, fake, ws=fake), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_decode_multi(p, over, 1, fake, fake, ws=fake), R.RECSA_ERR_CAPACITY),
        (lambda: R.recsa_decode_multi(p, (R.recsa_tree_desc * 33)(*([good[0]] * 33)), 33, fake, fake,
                                      ws=None), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_decode_multi(p, good, 2, None, fake, ws=fake), R.RECSA_ERR_INVALID_ARG),
    ]
    for i, (fn, status) in enumerate(cases):
        with pytest.raises(R.RecsaError) as e:
            fn()
        assert e.value.status == status, (i, str(e.value))


def test_grouped_decode_validates_before_any_hip_call():
    fake = 1 << 20
    d = R.recsa_tree_desc(fake, fake, fake, fake, 10)
    cases = [
        # groups of 3 heads: the shared selection is built for 1, 2, 4 or 8
        (lambda: R.recsa_decode_grouped(_p(n_kv_heads=4, n_q_heads=12, capacity=1000), d, fake, 1, fake),
         R.RECSA_ERR_UNSUPPORTED),
        (lambda: R.recsa_decode_grouped(_p(n_kv_heads=1, n_q_heads=16, capacity=1000), d, fake, 1, fake),
         R.RECSA_ERR_UNSUPPORTED),
        (lambda: R.recsa_decode_grouped(_p(capacity=1000), R.recsa_tree_desc(fake, fake, fake, fake, 0),
                                        fake, 1, fake), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_decode_grouped(_p(capacity=1000), d, fake, 0, fake), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_decode_grouped(_p(capacity=1000), d, None, 1, fake), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_decode_grouped(_p(capacity=1000), d, fake, 1, fake + 8), R.RECSA_ERR_INVALID_ARG),
        # k = 64, b = 64 at G = 8: the group's logits and rotated queries exceed a CU's LDS
        (lambda: R.recsa_decode_grouped(_p(n_kv_heads=1, n_q_heads=8, fanout_b=64, budget_k=63,
                                           capacity=1 << 20), d, fake, 1, fake),
         R.RECSA_ERR_UNSUPPORTED),
    ]
    for i, (fn, status) in enumerate(cases):
        with pytest.raises(R.RecsaError) as e:
            fn()
        assert e.value.status == status, (i, str(e.value))


def test_backward_validates_before_any_hip_call():
    p = _p(capacity=1000)
    fake = 1 << 20
    d = R.recsa_tree_desc(fake, fake, fake, fake, 10)
    assert R.recsa_backward_workspace_bytes(p, 64) >= 2 * 8 * (1000 // 32) * 128 * 4
    # bf16 storage and >= 256 rows: the parent-major path's buffers come on top
    summaries = R.recsa_backward_workspace_bytes(p, 64)
    assert R.recsa_backward_workspace_bytes(p, 255) == summaries
    assert R.recsa_backward_workspace_bytes(p, 256) > summaries
    assert R.recsa_backward_workspace_bytes(p, 4096) >= R.recsa_backward_workspace_bytes(p, 256)
    # fp32 storage stays row-wise at any row count
    pf = _p(capacity=1000, store="f32")
    assert R.recsa_backward_workspace_bytes(pf, 4096) == R.recsa_backward_workspace_bytes(pf, 64)
    ws = fake
    ok = dict(q_ptr=fake, n_q=2, causal=0, dout_ptr=fake, dq_ptr=fake, dk_ptr=fake, dv_ptr=fake,
              dw_ptr=fake, ws=ws)
    cases = [
        (dict(n_q=0), R.RECSA_ERR_INVALID_ARG),
        (dict(causal=2), R.RECSA_ERR_INVALID_ARG),
        (dict(causal=1, n_q=11), R.RECSA_ERR_INVALID_ARG),       # more queries than tokens
        (dict(dout_ptr=None), R.RECSA_ERR_INVALID_ARG),
        (dict(dk_ptr=fake + 4), R.RECSA_ERR_INVALID_ARG),
        (dict(dw_ptr=None), R.RECSA_ERR_INVALID_ARG),
        (dict(ws=None), R.RECSA_ERR_INVALID_ARG),
        (dict(ws=fake + 128), R.RECSA_ERR_INVALID_ARG),
    ]
    for i, (kw, status) in enumerate(cases):
        args = dict(ok, **kw)
        with pytest.raises(R.RecsaError) as e:
            R.recsa_backward(p, d, args["q_ptr"], args["n_q"], args["causal"], args["dout_ptr"],
                             args["dq_ptr"], args["dk_ptr"], args["dv_ptr"], args["dw_ptr"], ws=args["ws"])
        assert e.value.status == status, (i, str(e.value))
    with pytest.raises(R.RecsaError) as e:
        R.recsa_backward(p, R.recsa_tree_desc(fake, fake, fake, fake, 0), fake, 1, 0, fake, fake, fake,
                         fake, fake, ws=ws)
    assert e.value.status == R.RECSA_ERR_INVALID_ARG


def test_dense_and_distill_validate_before_any_hip_call():
    p = _p(capacity=1000)
    fake = 1 << 20
    d = R.recsa_tree_desc(fake, fake, fake, fake, 10)
    # per-span states of up to 256 spans: 8 KV heads x 2 queries x 4 heads per group x (d + 2)
    assert R.recsa_dense_workspace_bytes(p, 2) >= 8 * 256 * 2 * 4 * 130 * 4
    assert R.recsa_distill_workspace_bytes(p, 2) > R.recsa_backward_workspace_bytes(p, 2 * 32)
    assert R.recsa_dense_workspace_bytes(p, 0) == 0 and R.recsa_distill_workspace_bytes(p, 0) == 0
    cases = [
        (lambda: R.recsa_dense_decode(p, R.recsa_tree_desc(fake, fake, fake, fake, 0), fake, 1, fake, fake),
         R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_dense_decode(p, d, fake, 0, fake, fake), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_dense_decode(p, d, fake, 1, fake, None), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_dense_decode(p, d, fake + 2, 1, fake, fake), R.RECSA_ERR_INVALID_ARG),
        # pool_w must be the descriptor's
        (lambda: R.recsa_distill_step(p, d, fake + 4096, fake, 1, fake, 0.1, 0.9, fake, fake, fake),
         R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_distill_step(p, d, fake, fake, 1, fake, 0.1, 1.0, fake, fake, fake),
         R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_distill_step(p, d, fake, fake, 1, fake, -0.1, 0.9, fake, fake, fake),
         R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_distill_step(p, d, fake, fake, 1, None, 0.1, 0.9, fake, fake, fake),
         R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_distill_step(p, d, fake, fake, 1, fake, 0.1, 0.9, fake, fake, fake + 16),
         R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_distill_step(p, d, fake, fake, 0, fake, 0.1, 0.9, fake, fake, fake),
         R.RECSA_ERR_INVALID_ARG),
    ]
    for i, (fn, status) in enumerate(cases):
        with pytest.raises(R.RecsaError) as e:
            fn()
        assert e.value.status == status, (i, str(e.value))


def test_path_field_sizes_and_runs_alike():
    """recsa_params.path picks the layout of prefill and backward work; the sizing
    calls read the same field as the running calls, and a parent-major request the
    path cannot serve is refused on the host."""
    fake = 1 << 20
    rows = 4096 * 32
    auto = _p()
    assert R.recsa_workspace_bytes(auto, rows) > 0                       # parent-major by default
    assert R.recsa_workspace_bytes(_p(path="rowwise"), rows) == 0
    assert R.recsa_workspace_bytes(_p(path="parent_major"), 64) > 0      # forced at few rows
    summaries = R.recsa_backward_workspace_bytes(_p(path="rowwise"), 4096)
    assert R.recsa_backward_workspace_bytes(auto, 4096) > summaries
    assert R.recsa_backward_workspace_bytes(_p(path="parent_major"), 8) > summaries
    bad = _p()
    bad.path = 7
    assert R.recsa_tree_bytes(bad) == 0
    # fp32 storage and fanouts above 128 have no parent-major layout
    for p in (_p(store="f32", path="parent_major", capacity=1000),
              _p(fanout_b=200, path="parent_major", capacity=100000)):
        assert R.recsa_workspace_bytes(p, rows) == 0
        d = R.recsa_tree_desc(fake, fake, fake, fake, 900)
        with pytest.raises(R.RecsaError) as e:
            R.recsa_prefill(p, d, fake, 4, fake, ws=fake)
        assert e.value.status == R.RECSA_ERR_UNSUPPORTED
        with pytest.raises(R.RecsaError) as e:
            R.recsa_backward(p, d, fake, 2, 0, fake, fake, fake, fake, fake, ws=fake)
        assert e.value.status == R.RECSA_ERR_UNSUPPORTED


def test_multi_noalloc_validates_before_any_hip_call():
    p = _p(capacity=1000)
    fake = 1 << 20
    good = (R.recsa_tree_desc * 40)(*([R.recsa_tree_desc(fake, fake, fake, fake, 10)] * 40))
    bad = (R.recsa_tree_desc * 40)(*([R.recsa_tree_desc(fake, fake, fake, fake, 10)] * 39 +
                                     [R.recsa_tree_desc(fake, fake, fake, fake, 0)]))
    many = (R.recsa_tree_desc * 4097)(*([good[0]] * 4097))
    cases = [
        (lambda: R.recsa_decode_multi_noalloc(p, many, 4097, fake, fake), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_decode_multi_noalloc(p, bad, 40, fake, fake), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_decode_multi_noalloc(p, good, 40, None, fake), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_decode_multi_noalloc(p, good, 0, fake, fake), R.RECSA_ERR_INVALID_ARG),
        (lambda: R.recsa_decode_multi_noalloc(_p(head_dim=96), good, 40, fake, fake), R.RECSA_ERR_UNSUPPORTED),
    ]
    for i, (fn, status) in enumerate(cases):
        with pytest.raises(R.RecsaError) as e:
            fn()
        assert e.value.status == status, (i, str(e.value))
