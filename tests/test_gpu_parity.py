"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: every element within |gpu - ref| <= 1e-2 + 1e-2*|ref|.  This is the
tolerance of the page test's assert_close (sglang PR #36330 summary page,
"Key source snippets").  In addition the relative RMS error must stay <= 5e-3.
Every test compares every output row, the full-size workloads included.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_gqa_attention_va_amd as va
import va_inputs
from gpu_util import FP8_KERNELS, as_f64, check_problem, compare, note, run, to_device, with_kernels

pytestmark = pytest.mark.gpu
KERNEL = pytest.mark.parametrize("kernel", FP8_KERNELS, ids=["k1", "k2"])


def test_fp8_dequant_all_codes_matches_oracle_decoder():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).cuda()
    got = va.fp8_to_bf16(codes).float().cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    ref = np.array([oracle.fp8_e4m3fn_to_float(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


@KERNEL
@pytest.mark.parametrize("cfg", [0, 1])
def test_tiny_configs_all_rows(cfg, kernel):
    p = va_inputs.config(cfg)
    check_problem(p, kernel=kernel)


@pytest.mark.parametrize("cfg", [0, 1])
def test_tiny_configs_unpoisoned(cfg):
    # exactly the page test's construction (identity table, no poison)
    p = va_inputs.config(cfg, poison=False)
    check_problem(p)


RAGGED = [
    # q_lens, kv_lens, Hq, Hkv, dtype, kd, vd
    ([1, 2, 3, 4, 4], [1, 17, 100, 1000, 4099], 16, 1, "fp8", 1.0, 1.0),
    ([4, 3], [33, 2050], 32, 2, "fp8", 1.5, 0.75),
    ([2, 0, 4], [47, 31, 4], 8, 1, "fp8", 1.0, 1.0),
    ([3, 1, 2, 4], [48, 15, 64, 515], 4, 1, "fp8", 0.5, 2.0),
    ([4, 2], [1024, 769], 16, 1, "bf16", 1.0, 1.0),
    ([1, 3, 2], [5000, 129, 3], 8, 2, "bf16", 1.25, 0.5),
    ([4, 4, 4, 4], [4, 5, 16, 17], 16, 4, "fp8", 1.0, 1.0),
]


@pytest.mark.parametrize("case,kernel", with_kernels(RAGGED, lambda c: c[4]))
def test_ragged_shapes_all_rows(case, kernel):
    ql, kl, hq, hkv, dt, kd, vd = case
    p = va_inputs.custom(ql, kl, hq, hkv, dt, seed=sum(kl) + hq, k_descale=kd, v_descale=vd,
                         name=f"ragged{hq}/{hkv}{dt}")
    check_problem(p, kernel=kernel)


@KERNEL
@pytest.mark.parametrize("grid", [1, 2, 7, 64, 1000])
def test_forced_grid_sizes_agree(grid, kernel):
    p = va_inputs.custom([4, 2, 3, 1], [3000, 769, 100, 40], 16, 1, "fp8", seed=42,
                         name=f"grid{grid}")
    check_problem(p, force_grid=grid, kernel=kernel)


def test_forced_grid_sizes_agree_with_each_other():
    p = va_inputs.custom([4, 2, 3], [4000, 1500, 33], 16, 2, "fp8", seed=43)
    dev = to_device(p)
    outs = [as_f64(run(p, dev=dev, force_grid=g, kernel=k)) for k in FP8_KERNELS for g in (1, 3, 16, 256)]
    for o in outs[1:]:
        compare(o, outs[0], "grid vs grid1")


def test_run_to_run_bitwise_deterministic():
    p = va_inputs.custom([4, 3, 2], [9000, 3000, 700], 16, 1, "fp8", seed=44)
    dev = to_device(p)
    for k in FP8_KERNELS:
        plan = va.Plan.for_problem(p, kernel=k)
        a = run(p, dev=dev, plan=plan).clone()
        b = run(p, dev=dev, plan=plan).clone()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_first_verify_token_with_one_key_is_exact():
    # Lk == Lq: query token 0 sees key 0 only, so out = bf16(v_descale * V[key 0])
    p = va_inputs.custom([4, 3], [4, 3], 16, 1, "fp8", seed=45, v_descale=1.5)
    out = run(p).float().cpu().numpy().reshape(p.total_q, p.num_q_heads, -1)
    V = torch.from_numpy(p.v).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(p.num_seqs):
        q0 = p.cu_seqlens_q[b]
        v0 = V[p.block_table[b, 0], 0, 0] * p.v_descale
        expect = torch.from_numpy(v0).to(torch.bfloat16).float().numpy()
        for h in range(p.num_q_heads):
            assert np.array_equal(out[q0, h], expect)


@KERNEL
def test_zero_query_gives_mean_of_visible_values(kernel):
    p = va_inputs.custom([4, 2], [3000, 77], 16, 1, "fp8", seed=46)
    p.q[:] = 0
    check_problem(p, kernel=kernel)


def test_segment_markers_expose_a_dropped_or_doubled_piece():
    # Uniform logits (Q = 0) and V zero except a marker 256.0 in dimension
    # (page index mod 256) of every key.  Each output dimension is then
    # 256 * (visible keys in pages of that residue) / (visible keys): a piece
    # of the split that went missing or was counted twice moves whole
    # dimensions by far more than the tolerance.
    p = va_inputs.custom([4, 3], [40000, 20000], 16, 1, "fp8", seed=47, poison=False)
    p.q[:] = 0
    p.v[:] = 0
    for b in range(p.num_seqs):
        for lp in range(-(-int(p.seqused_k[b]) // 16)):
            p.v[p.block_table[b, lp], :, 0, lp % 256] = 0x78      # e4m3fn 256.0
    for k in FP8_KERNELS:
        check_problem(p, kernel=k)
        check_problem(p, force_grid=37, kernel=k)


@KERNEL
@pytest.mark.parametrize("where", ["late", "first", "last"])
def test_logit_spike_far_above_the_first_keys(where, kernel):
    # One key row is 16 * sign(q) of query row (token 0, head 0): that row's
    # logit there is about 200 (natural units) above the others, far beyond the
    # FP8 kernel's accumulation headroom (64 in log2 units above the first keys
    # a row sees).  A spike after the first step makes the kernel run the
    # piece's page loop again from the new maximum; other heads see logits of
    # about +-16 from the same key.  Every row must still match the oracle.
    p = va_inputs.custom([4, 2], [6000, 3000], 16, 1, "fp8", seed=50, poison=False)
    q0 = p.q.view(np.uint16)[0, 0].astype(np.uint32) << 16
    sign = np.where(q0.view(np.float32) < 0, -1.0, 1.0)
    spike = torch.from_numpy((16.0 * sign).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    key = {"late": 5000, "first": 3, "last": 5995}[where]
    p.k[p.block_table[0, key // 16], key % 16, 0] = spike
    for grid in (0, 7):
        check_problem(p, force_grid=grid, kernel=kernel)


@KERNEL
def test_q_len_zero_rows_untouched_and_others_correct(kernel):
    p = va_inputs.custom([0, 4, 0, 2], [100, 3000, 50, 20], 8, 1, "fp8", seed=48)
    check_problem(p, kernel=kernel)


@KERNEL
def test_graph_capture_replay_matches_eager(kernel):
    p = va_inputs.custom([4, 2, 3], [5000, 800, 64], 16, 1, "fp8", seed=49)
    dev = to_device(p)
    plan = va.Plan.for_problem(p, kernel=kernel)
    ws = plan.workspace()
    eager = run(p, dev=dev, plan=plan, workspace=ws).clone()
    out = torch.empty_like(dev["q"])
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        plan.run(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cu"], dev["sk"], p.scale,
                 dev["kd"], dev["vd"], out=out, workspace=ws)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))


# ------------------------------------------- closed forms at every shape --

CLOSED_FORM_SHAPES = [
    # q_lens, kv_lens, Hq, Hkv, kv dtype: row tiles 1..4 of the FP8 kernel, a
    # bf16 cache, two kv heads; long sequences so that the split cuts them
    ([1, 2, 3, 4], [33, 5000, 20000, 70001], 16, 1, "fp8"),
    ([4, 3], [40000, 999], 8, 2, "fp8"),
    ([2, 4], [17, 30000], 16, 1, "bf16"),
]


def _visible_keys(p, b, t):
    lq = int(p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b])
    return int(p.seqused_k[b]) - lq + t + 1


@pytest.mark.parametrize("case,kernel", with_kernels(CLOSED_FORM_SHAPES, lambda c: c[4]))
def test_identical_keys_give_mean_of_visible_values(case, kernel):
    # Every key row of a sequence is the same, so every logit of a query row is
    # the same and the output is v_descale times the plain mean of the values
    # the row sees (a closed form, computed here without the oracle).  The
    # kernel's equal weights round to one bf16 value; what is left is fp32
    # summation, the fp16 partials of the split and the bf16 output.
    ql, kl, hq, hkv, dt = case
    p = va_inputs.custom(ql, kl, hq, hkv, dt, seed=60 + sum(kl), v_descale=1.25)
    rng = np.random.default_rng(61)
    for b in range(p.num_seqs):
        keys = np.arange(int(p.seqused_k[b]))
        pg, sl = p.block_table[b, keys // 16], keys % 16
        row = p.k[pg[rng.integers(len(keys))], sl[rng.integers(len(keys))]].copy()   # [Hkv, D]
        p.k[pg, sl] = row
    V = (torch.from_numpy(p.v).view(torch.float8_e4m3fn).to(torch.float64).numpy() if dt == "fp8" else
         torch.from_numpy(p.v.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy())
    G = hq // hkv
    expect = np.zeros((p.total_q, hq, 256))
    for b in range(p.num_seqs):
        q0 = int(p.cu_seqlens_q[b])
        for t in range(int(p.cu_seqlens_q[b + 1]) - q0):
            keys = np.arange(_visible_keys(p, b, t))
            vis = V[p.block_table[b, keys // 16], keys % 16]                           # [n, Hkv, D]
            mean = vis.mean(axis=0) * p.v_descale
            expect[q0 + t] = mean[np.arange(hq) // G]
    expect = expect.reshape(-1, 256)
    for grid in (0, 7, 300):
        got = as_f64(run(p, force_grid=grid, kernel=kernel))
        err = np.abs(got - expect)
        note(f"  identical keys grid {grid}: max|err|={err.max():.3e}")
        assert np.all(err <= 1e-3 + 2.0 ** -8 * np.abs(expect))


@pytest.mark.parametrize("case,kernel", with_kernels(CLOSED_FORM_SHAPES, lambda c: c[4]))
def test_constant_values_give_exactly_that_value(case, kernel):
    # V == c on every visible key: whatever the weights, the output is
    # v_descale * c.  With c = 3 and v_descale = 0.625 that is 1.875, exact in
    # bf16, and every rounding the kernel makes is far below half a bf16 step,
    # so the output must be 1.875 bit for bit.  Page tails past seqused_k keep
    # their NaN poison: a masked key that leaked into PV would show.
    ql, kl, hq, hkv, dt = case
    p = va_inputs.custom(ql, kl, hq, hkv, dt, seed=70 + sum(kl), v_descale=0.625)
    code = 0x44 if dt == "fp8" else 0x4040                     # 3.0 in e4m3fn / bf16
    for b in range(p.num_seqs):
        keys = np.arange(int(p.seqused_k[b]))
        p.v[p.block_table[b, keys // 16], keys % 16] = code
    for grid in (0, 7, 300):
        got = as_f64(run(p, force_grid=grid, kernel=kernel))
        note(f"  constant values grid {grid}: distinct outputs {np.unique(got)[:4]}")
        assert np.all(got == 1.875)


# ------------------------------------------------------- full-size workloads
#
# Every output row of the long-context, high-concurrency and shape-sweep
# workloads, at the plan's own grid (the launch configuration bench.py times),
# against the oracle.

def _both_kernels_all_rows(p):
    """Both FP8 kernels (the plan's own choice among them) against the same
    oracle rows."""
    ref, _ = oracle.attn_problem(p)
    for k in FP8_KERNELS:
        compare(as_f64(run(p, kernel=k)), ref, f"{p.name} kernel {k}")


def test_config2_long_context_all_rows():
    _both_kernels_all_rows(va_inputs.config(2))


def test_config3_high_concurrency_all_rows():
    _both_kernels_all_rows(va_inputs.config(3))


@pytest.mark.parametrize("variant", range(len(va_inputs.SWEEP_VARIANTS)),
                         ids=[f"g{g}-{d}" for g, d in va_inputs.SWEEP_VARIANTS])
def test_config4_shape_sweep_all_rows(variant):
    check_problem(va_inputs.config(4, variant))
