"""The C ABI without a GPU: the library loads, exports every function that
include/va.h declares, and va_plan / va_run reject bad arguments with the
documented status codes (no kernel is launched in any of these tests)."""
import ctypes
import os
import re

import pytest

import paged_gqa_attention_va_amd as va

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "va.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(va_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("va_plan", "va_plan_workspace_bytes", "va_run", "va_plan_destroy", "va_status_str"):
        assert n in names


def test_library_exports_every_declared_function():
    lib = va.library()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(va.EXPORTED)


def base_problem(**kw):
    d = dict(num_seqs=16, num_q_heads=16, num_kv_heads=1, max_seqlen_q=4, max_seqlen_k=32768,
             max_blocks_per_seq=2048, num_blocks=32768, total_q=64, kv_dtype="fp8", num_cus=256)
    d.update(kw)
    return d


def test_plan_accepts_the_workloads():
    for kw in (dict(), dict(num_q_heads=32, num_kv_heads=2), dict(num_q_heads=4, max_seqlen_q=1, total_q=16),
               dict(num_q_heads=8, kv_dtype="bf16", max_seqlen_q=3, total_q=48)):
        p = va.Plan(**base_problem(**kw))
        assert p.workspace_bytes > 0 and p.grid == 256


@pytest.mark.parametrize("kw,status", [
    (dict(num_q_heads=12), va.VA_ERR_UNSUPPORTED),          # G = 12
    (dict(num_q_heads=2, num_kv_heads=1), va.VA_ERR_UNSUPPORTED),
    (dict(num_q_heads=16, num_kv_heads=3), va.VA_ERR_UNSUPPORTED),
    (dict(head_dim=128), va.VA_ERR_UNSUPPORTED),
    (dict(page_size=32), va.VA_ERR_UNSUPPORTED),
    (dict(max_seqlen_q=5, total_q=64), va.VA_ERR_UNSUPPORTED),
    (dict(q_dtype="fp8"), va.VA_ERR_UNSUPPORTED),
    (dict(num_seqs=0), va.VA_ERR_INVALID_ARG),
    (dict(total_q=65), va.VA_ERR_INVALID_ARG),
    (dict(max_seqlen_q=0), va.VA_ERR_INVALID_ARG),
    (dict(num_blocks=0), va.VA_ERR_INVALID_ARG),
    (dict(max_seqlen_k=32769), va.VA_ERR_INVALID_ARG),
    (dict(num_cus=-1), va.VA_ERR_INVALID_ARG),
    (dict(force_grid=-1), va.VA_ERR_INVALID_ARG),
    (dict(force_grid=65537), va.VA_ERR_INVALID_ARG),
])
def test_plan_rejects(kw, status):
    with pytest.raises(va.VaError) as e:
        va.Plan(**base_problem(**kw))
    assert e.value.status == status


def test_plan_rejects_bad_dtype_enum_and_null():
    lib = va.library()
    pr = va._Problem(1, 16, 1, 256, 16, 4, 100, 7, 7, 4, 1, 9, 256, 0)   # kv_dtype 9
    h = ctypes.c_void_p()
    assert lib.va_plan(ctypes.byref(pr), ctypes.byref(h)) == va.VA_ERR_INVALID_ARG
    assert lib.va_plan(None, ctypes.byref(h)) == va.VA_ERR_INVALID_ARG
    pr.kv_dtype = 2
    assert lib.va_plan(ctypes.byref(pr), None) == va.VA_ERR_INVALID_ARG


def test_force_grid_sets_grid_and_workspace_grows_with_it():
    a = va.Plan(**base_problem(force_grid=7))
    b = va.Plan(**base_problem(force_grid=700))
    assert a.grid == 7 and b.grid == 700 and b.workspace_bytes > a.workspace_bytes


def _run_args(plan, ws_bytes, **over):
    fake = ctypes.c_void_p(0x10000)          # never dereferenced: argument checks fail first
    args = dict(q=fake, k=fake, v=fake, bt=fake, cu=fake, sk=fake, out=fake, ws=fake)
    args.update(over)
    return (plan._h, args["q"], args["k"], args["v"], args["bt"], args["cu"], args["sk"],
            ctypes.c_float(0.0625), None, None, args["out"], args["ws"],
            ctypes.c_size_t(ws_bytes), None)


def test_run_rejects_null_pointers_and_short_workspace():
    lib = va.library()
    plan = va.Plan(**base_problem())
    n = plan.workspace_bytes
    assert lib.va_run(*_run_args(plan, n, q=None)) == va.VA_ERR_INVALID_ARG
    assert lib.va_run(*_run_args(plan, n, out=None)) == va.VA_ERR_INVALID_ARG
    assert lib.va_run(*_run_args(plan, n, bt=None)) == va.VA_ERR_INVALID_ARG
    assert lib.va_run(*_run_args(plan, n - 1)) == va.VA_ERR_WORKSPACE
    assert lib.va_run(*_run_args(plan, n, ws=None)) == va.VA_ERR_WORKSPACE
    assert lib.va_run(*_run_args(plan, n, ws=ctypes.c_void_p(0x10010))) == va.VA_ERR_INVALID_ARG
    assert lib.va_run(*_run_args(plan, n, q=ctypes.c_void_p(0x10002))) == va.VA_ERR_INVALID_ARG
    assert lib.va_run(None, *_run_args(plan, n)[1:]) == va.VA_ERR_INVALID_ARG
    a = _run_args(plan, n)
    ex = (plan._h, 7) + a[1:10] + (None,) + a[10:]          # va_run_ex: stage, ..., sinks, ...
    assert lib.va_run_ex(*ex) == va.VA_ERR_INVALID_ARG


def test_plan_checks_window_and_softcap():
    for kw in (dict(window_left=-2), dict(softcap=-1.0), dict(softcap=float("nan"))):
        with pytest.raises(va.VaError) as e:
            va.Plan(**base_problem(), **kw)
        assert e.value.status == va.VA_ERR_INVALID_ARG
    assert va.Plan(**base_problem(), window_left=0, softcap=30.0).grid == 256


def test_status_strings():
    for s in range(6):
        assert va.status_str(s) and va.status_str(s) != "unknown status"
    assert va.status_str(99) == "unknown status"


def test_plan_checks_the_mla_domain():
    mla = dict(num_seqs=4, num_q_heads=16, num_kv_heads=1, max_seqlen_q=4, max_seqlen_k=4096,
               max_blocks_per_seq=256, num_blocks=1024, total_q=16, num_cus=256, head_dim=576)
    assert va.Plan(**mla, v_head_dim=512).v_head_dim == 512
    for kw, status in ((dict(v_head_dim=576), va.VA_ERR_UNSUPPORTED),
                       (dict(v_head_dim=512, num_kv_heads=2, num_q_heads=32), va.VA_ERR_UNSUPPORTED),
                       (dict(v_head_dim=512, window_left=10), va.VA_ERR_UNSUPPORTED),
                       (dict(v_head_dim=512, softcap=5.0), va.VA_ERR_UNSUPPORTED),
                       (dict(v_head_dim=512, layout="prefix_extend", page_size=1), va.VA_ERR_UNSUPPORTED),
                       (dict(v_head_dim=-1), va.VA_ERR_INVALID_ARG)):
        d = dict(mla)
        d.update(kw)
        with pytest.raises(va.VaError) as e:
            va.Plan(**d)
        assert e.value.status == status, kw
    with pytest.raises(va.VaError) as e:           # 256-wide heads with another value width
        va.Plan(**base_problem(), v_head_dim=128)
    assert e.value.status == va.VA_ERR_UNSUPPORTED


def test_workspace_is_bounded_by_the_grid_not_the_pairs():
    small = va.Plan(**base_problem())                                  # 16 pairs
    big = va.Plan(**base_problem(num_seqs=16384, num_kv_heads=4, num_q_heads=16, max_seqlen_q=1,
                                 max_seqlen_k=32, max_blocks_per_seq=2, total_q=16384))   # 65536 pairs
    assert big.grid == small.grid == 256
    # two partial slots per workgroup, plus the page prefix over the pairs
    assert big.workspace_bytes < small.workspace_bytes + 65537 * 4 + 4096
    assert big.workspace_bytes < 16 << 20


def test_binding_rejects_tensors_on_another_device():
    import torch
    va._same_device(torch.device("cpu"), torch.zeros(1), None)
    with pytest.raises(ValueError):
        va._same_device(torch.device("cpu"), torch.zeros(1), torch.empty(1, device="meta"))


def test_stream_pages_rejects_bad_arguments_before_launching():
    lib = va.library()
    P = ctypes.c_void_p
    pool, pages, sums = P(0x10000), P(0x20000), P(0x30000)     # never dereferenced: refused first
    assert lib.va_stream_pages(None, 1 << 20, pages, 10, 8, 4, sums, None) == va.VA_ERR_INVALID_ARG
    assert lib.va_stream_pages(pool, 1 << 20, None, 10, 8, 4, sums, None) == va.VA_ERR_INVALID_ARG
    assert lib.va_stream_pages(pool, 1 << 20, pages, 10, 8, 4, None, None) == va.VA_ERR_INVALID_ARG
    assert lib.va_stream_pages(pool, 1 << 20, pages, 10, 7, 4, sums, None) == va.VA_ERR_INVALID_ARG
    assert lib.va_stream_pages(pool, 1 << 20, pages, 10, 8, 0, sums, None) == va.VA_ERR_INVALID_ARG
    assert lib.va_stream_pages(pool, 4095, pages, 10, 8, 4, sums, None) == va.VA_ERR_INVALID_ARG
    assert lib.va_stream_pages(P(0x10008), 1 << 20, pages, 10, 8, 4, sums, None) == va.VA_ERR_INVALID_ARG
    assert lib.va_stream_pages(pool, 1 << 20, pages, -1, 8, 4, sums, None) == va.VA_ERR_INVALID_ARG


def test_plan_picks_the_fp8_kernel_by_pages_per_workgroup():
    """Auto choice: the one-wave-per-SIMD kernel once each workgroup streams at
    least 112 pages, the two-row-group kernel below; an explicit choice is only
    accepted for paged FP8 GQA."""
    assert va.Plan(**base_problem()).kernel == 1                          # 16 x 32768: 128 pages / WG
    assert va.Plan(**base_problem(max_seqlen_k=8192, max_blocks_per_seq=512)).kernel == 2
    assert va.Plan(**base_problem(), window_left=4095).kernel == 2        # 16 x 4100 keys read
    assert va.Plan(**base_problem(), window_left=24575).kernel == 2       # 1538 pages per sequence
    assert va.Plan(**base_problem(), window_left=28671).kernel == 1
    assert va.Plan(**base_problem(max_seqlen_k=8192, max_blocks_per_seq=512), kernel=1).kernel == 1
    assert va.Plan(**base_problem(), kernel=2).kernel == 2
    assert va.Plan(**base_problem(kv_dtype="bf16")).kernel == 0
    for kw in (dict(kernel=3), dict(kernel=-1), dict(kernel=1, kv_dtype="bf16"),
               dict(kernel=2, kv_dtype="bf16")):
        d = base_problem()
        d.update(kw)
        with pytest.raises(va.VaError) as e:
            va.Plan(**d)
        assert e.value.status == va.VA_ERR_INVALID_ARG, kw
