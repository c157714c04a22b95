"""Validate mode: the metadata rules of one call (include/va.h, va_validate).

CPU: the oracle's rule checker against hand-derived results on a small
metadata set (each rule broken on its own, padding entries and pages before a
sliding window not checked); the C ABI rejects bad arguments; VA_DEBUG makes
va_plan print the plan.
GPU (marked): the device checker equals the oracle's bit for bit on the hand
cases and on seeded random mutations; in validate mode va_run refuses invalid
metadata without launching the attention, and leaves valid calls unchanged.
No attention kernel ever runs on invalid metadata here.
"""
import ctypes

import numpy as np
import pytest

import oracle
import paged_gqa_attention_va_amd as va

# Base metadata: 3 sequences, 4 block-table entries each, 12 pool pages,
# total_q 8, max_seqlen_q 4, max_seqlen_k 64.  Entries 99 are padding.
NB, TOTAL_Q, MAX_Q, MAX_K = 12, 8, 4, 64


def base_meta():
    cu = np.array([0, 4, 6, 8], dtype=np.int32)
    sk = np.array([40, 2, 64], dtype=np.int32)
    bt = np.array([[0, 1, 2, 99], [3, 99, 99, 99], [4, 5, 6, 7]], dtype=np.int32)
    return bt, cu, sk


def mutate(cu=None, sk=None, bt=None):
    b0, c0, s0 = base_meta()
    if cu is not None:
        c0 = np.array(cu, dtype=np.int32)
    if sk is not None:
        s0 = np.array(sk, dtype=np.int32)
    for (r, c), v in (bt or {}).items():
        b0[r, c] = v
    return b0, c0, s0


# (name, metadata, window_left, expected (bits, first bad sequence)); the
# expectations are worked out by hand from the rules in include/va.h.
HAND_CASES = [
    ("valid", mutate(), -1, (0, 3)),
    ("cu0_not_zero", mutate(cu=[1, 4, 6, 8]), -1, (1, 0)),
    # b=1: cu falls (4 -> 3); b=2 then has 3 .. 8 = 5 queries > max_seqlen_q
    ("cu_falls", mutate(cu=[0, 4, 3, 8]), -1, (1 | 2, 1)),
    ("cu_past_total_q", mutate(cu=[0, 4, 6, 9]), -1, (1, 2)),
    ("q_len_gt_seqused", mutate(sk=[40, 1, 64]), -1, (8, 1)),
    ("seqused_gt_max_k", mutate(sk=[40, 2, 65]), -1, (4, 2)),
    # seqused -3: bad length, and q_len 4 > -3
    ("seqused_negative", mutate(sk=[-3, 2, 64]), -1, (4 | 8, 0)),
    ("page_eq_num_blocks", mutate(bt={(0, 2): NB}), -1, (16, 0)),
    ("page_negative", mutate(bt={(1, 0): -5}), -1, (16, 1)),
    ("padding_not_read", mutate(bt={(0, 3): -1}), -1, (0, 3)),
    # window 10 on b=0 (40 keys, 4 queries): first key 40 - 4 - 10 = 26, page 1
    ("window_skips_page0", mutate(bt={(0, 0): 999}), 10, (0, 3)),
    ("window_reads_page1", mutate(bt={(0, 1): 999}), 10, (16, 0)),
    # window 0 on b=2 (64 keys, 2 queries): first key 62, page 3
    ("window0_last_page_only", mutate(bt={(2, 2): -1}), 0, (0, 3)),
    ("two_sequences_bad", mutate(sk=[40, 1, 64], bt={(0, 0): 12}), -1, (16 | 8, 0)),
]


@pytest.mark.parametrize("name,meta,wl,expected", HAND_CASES, ids=[c[0] for c in HAND_CASES])
def test_oracle_rules_hand_cases(name, meta, wl, expected):
    bt, cu, sk = meta
    assert oracle.validate(bt, cu, sk, NB, TOTAL_Q, MAX_Q, MAX_K, window_left=wl) == expected


def test_oracle_rules_accept_generated_inputs():
    import va_inputs
    for i in (0, 1):
        p = va_inputs.config(i)
        assert oracle.validate(p.block_table, p.cu_seqlens_q, p.seqused_k, p.num_blocks, p.total_q,
                               p.max_seqlen_q, p.max_seqlen_k) == (0, p.num_seqs)
    # a q_len 0 sequence and a 0-key sequence are legal; poisoned padding is not read
    p = va_inputs.custom([0, 3, 1], [0, 33, 17], 16, 1, max_blocks_per_seq=5)
    assert oracle.validate(p.block_table, p.cu_seqlens_q, p.seqused_k, p.num_blocks, p.total_q,
                           4, 80) == (0, 3)


def test_validate_rejects_bad_arguments():
    lib = va.library()
    plan = va.Plan(num_seqs=3, num_q_heads=16, num_kv_heads=1, max_seqlen_q=MAX_Q, max_seqlen_k=MAX_K,
                   max_blocks_per_seq=4, num_blocks=NB, total_q=TOTAL_Q, num_cus=256)
    p = ctypes.c_void_p(0x10000)
    assert lib.va_validate(None, p, p, p, p, None) == va.VA_ERR_INVALID_ARG
    assert lib.va_validate(plan._h, None, p, p, p, None) == va.VA_ERR_INVALID_ARG
    assert lib.va_validate(plan._h, p, p, p, None, None) == va.VA_ERR_INVALID_ARG
    assert lib.va_validate(plan._h, p, p, p, ctypes.c_void_p(0x10002), None) == va.VA_ERR_INVALID_ARG
    assert va.status_str(va.VA_ERR_DEVICE_DATA) != "unknown status"


def test_debug_env_prints_the_plan(monkeypatch, capfd):
    kw = dict(num_seqs=3, num_q_heads=16, num_kv_heads=1, max_seqlen_q=MAX_Q, max_seqlen_k=MAX_K,
              max_blocks_per_seq=4, num_blocks=NB, total_q=TOTAL_Q, num_cus=256)
    monkeypatch.setenv("VA_DEBUG", "1")
    plan = va.Plan(**kw)
    err = capfd.readouterr().err
    assert "va_plan:" in err and f"grid={plan.grid}" in err and f"workspace={plan.workspace_bytes}" in err
    monkeypatch.setenv("VA_DEBUG", "0")
    va.Plan(**kw)
    assert "va_plan:" not in capfd.readouterr().err


# ------------------------------------------------------------------- GPU --

def random_mutation(rng, wl):
    """Seeded metadata with one to three random rule breaks (or none)."""
    bt, cu, sk = base_meta()
    for _ in range(int(rng.integers(0, 4))):
        kind = int(rng.integers(0, 5))
        b = int(rng.integers(0, 3))
        if kind == 0:
            cu[int(rng.integers(0, 4))] += int(rng.integers(-3, 4))
        elif kind == 1:
            sk[b] = int(rng.integers(-2, MAX_K + 3))
        elif kind == 2:
            bt[b, int(rng.integers(0, 4))] = int(rng.choice([-1, NB, NB + 7, 2 ** 31 - 1, -2 ** 31]))
        elif kind == 3:
            bt[b, int(rng.integers(0, 4))] = int(rng.integers(0, NB))
        else:
            sk[b] = int(rng.integers(0, 5))
    return bt, cu, sk


def _device_validate(plan, meta):
    import torch
    bt, cu, sk = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in meta)
    res = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    plan.validate(bt, cu, sk, result=res)
    torch.cuda.synchronize()
    r = res.cpu().numpy()
    return int(r[0]), int(r[1])


@pytest.mark.gpu
@pytest.mark.parametrize("wl", [-1, 0, 10, 40])
def test_gpu_validate_equals_oracle(wl):
    from gpu_util import note
    plan = va.Plan(num_seqs=3, num_q_heads=16, num_kv_heads=1, max_seqlen_q=MAX_Q, max_seqlen_k=MAX_K,
                   max_blocks_per_seq=4, num_blocks=NB, total_q=TOTAL_Q, window_left=wl)
    cases = [(n, m) for n, m, w, _ in HAND_CASES]
    rng = np.random.default_rng(100 + wl)
    cases += [(f"random{i}", random_mutation(rng, wl)) for i in range(200)]
    seen = 0
    for name, meta in cases:
        want = oracle.validate(*meta, NB, TOTAL_Q, MAX_Q, MAX_K, window_left=wl)
        got = _device_validate(plan, meta)
        assert got == want, (name, wl, meta, got, want)
        seen |= want[0]
    note(f"  window {wl}: {len(cases)} metadata sets, rule bits seen {seen:#x}")
    assert seen == 31


@pytest.mark.gpu
def test_gpu_validate_accepts_generated_inputs():
    import torch
    import va_inputs
    for p in (va_inputs.config(0), va_inputs.config(1),
              va_inputs.custom([0, 3, 1, 4], [0, 33, 17, 4096], 16, 1, window_left=100)):
        plan = va.Plan.for_problem(p)
        got = _device_validate(plan, (p.block_table, p.cu_seqlens_q, p.seqused_k))
        assert got == (0, p.num_seqs), (p.name, got)


@pytest.mark.gpu
def test_gpu_debug_mode_refuses_invalid_metadata(monkeypatch):
    import torch
    import va_inputs
    from gpu_util import to_device
    p = va_inputs.custom([4, 2, 3], [300, 40, 17], 16, 1, seed=5)
    dev = to_device(p)
    ref = va.Plan.for_problem(p).run(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cu"], dev["sk"],
                                     p.scale, dev["kd"], dev["vd"])
    monkeypatch.setenv("VA_DEBUG", "1")
    plan = va.Plan.for_problem(p)
    out = plan.run(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cu"], dev["sk"], p.scale, dev["kd"], dev["vd"])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    # q_len 2 > seqused_k 1 in sequence 1: refused, out untouched
    bad_sk = dev["sk"].clone()
    bad_sk[1] = 1
    sentinel = torch.full_like(out, 3.0)
    with pytest.raises(va.VaError) as e:
        plan.run(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cu"], bad_sk, p.scale, dev["kd"], dev["vd"],
                 out=sentinel)
    assert e.value.status == va.VA_ERR_DEVICE_DATA
    torch.cuda.synchronize()
    assert bool((sentinel == 3.0).all())
    # a page id out of range in a page the sequence reads
    bad_bt = dev["bt"].clone()
    bad_bt[2, 0] = p.num_blocks
    with pytest.raises(va.VaError) as e:
        plan.run(dev["q"], dev["k"], dev["v"], bad_bt, dev["cu"], dev["sk"], p.scale, dev["kd"], dev["vd"],
                 out=sentinel)
    assert e.value.status == va.VA_ERR_DEVICE_DATA
    torch.cuda.synchronize()
    assert bool((sentinel == 3.0).all())
