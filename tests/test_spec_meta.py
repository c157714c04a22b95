"""The draft-extend metadata conversion (kv_indptr / kv_indices -> block table,
seqused_k), the reading of the PR #30105 summary page's draft_extend_v2 path
("Key source snippets": seqused_k as the kv_indptr difference, a 2D page table
built from spec metadata).

CPU: the oracle's plain conversion is pinned by a round trip (token slots
generated from a known block table give the table back) and edge cases.
GPU (marked): the library's device conversion equals the oracle's bit for bit,
and attention through the converted table matches the oracle.
"""
import numpy as np
import pytest

import oracle
import va_inputs


def token_slots(p):
    """kv_indptr / kv_indices of problem p: every KV token's pool slot, in order."""
    B = p.num_seqs
    indptr = np.zeros(B + 1, dtype=np.int32)
    slots = []
    for b in range(B):
        n = int(p.seqused_k[b])
        indptr[b + 1] = indptr[b] + n
        j = np.arange(n)
        slots.append(p.block_table[b, j // p.page_size].astype(np.int64) * p.page_size + j % p.page_size)
    return indptr, (np.concatenate(slots) if slots else np.zeros(0)).astype(np.int32)


@pytest.mark.parametrize("kv_lens", [[1024, 769], [1, 16, 17, 0, 250], [4099, 3, 64]])
def test_round_trip_gives_the_block_table_back(kv_lens):
    p = va_inputs.custom([1] * len(kv_lens), [max(1, k) for k in kv_lens], 4, 1, "fp8", seed=len(kv_lens))
    p.seqused_k[:] = np.asarray(kv_lens, dtype=np.int32)
    indptr, idx = token_slots(p)
    bt, sk = oracle.spec_block_table(indptr, idx, 16, p.block_table.shape[1])
    assert np.array_equal(sk, p.seqused_k)
    for b, n in enumerate(kv_lens):
        used = -(-n // 16)
        assert np.array_equal(bt[b, :used], p.block_table[b, :used])
        assert np.all(bt[b, used:] == 0)


def test_page_ids_come_from_the_first_token_of_each_page():
    # sequence 0: pages 5, 2 (second partly used); sequence 1: empty; sequence 2: page 7
    idx = np.array([5 * 16 + i for i in range(16)] + [2 * 16 + i for i in range(3)] + [7 * 16], np.int32)
    indptr = np.array([0, 19, 19, 20], np.int32)
    bt, sk = oracle.spec_block_table(indptr, idx, 16, 3)
    assert sk.tolist() == [19, 0, 1]
    assert bt.tolist() == [[5, 2, 0], [0, 0, 0], [7, 0, 0]]


@pytest.mark.gpu
@pytest.mark.parametrize("case", [
    ([4, 2], [1024, 769], 16, 1, "fp8"),
    ([1, 3, 2, 4], [5000, 17, 2, 2049], 16, 1, "fp8"),
    ([3, 3], [700, 1300], 8, 2, "bf16"),
])
def test_device_conversion_and_attention_through_it(case):
    import torch
    import paged_gqa_attention_va_amd as va
    from gpu_util import as_f64, compare, run, to_device
    ql, kl, hq, hkv, dt = case
    p = va_inputs.custom(ql, kl, hq, hkv, dt, seed=sum(kl), name="draft-extend")
    indptr, idx = token_slots(p)
    mbps = p.block_table.shape[1]
    ref_bt, ref_sk = oracle.spec_block_table(indptr, idx, 16, mbps)
    bt, sk = va.spec_block_table(torch.from_numpy(indptr).cuda(), torch.from_numpy(idx).cuda(), mbps)
    torch.cuda.synchronize()
    assert np.array_equal(bt.cpu().numpy(), ref_bt) and np.array_equal(sk.cpu().numpy(), ref_sk)
    dev = to_device(p)
    dev["bt"], dev["sk"] = bt, sk                       # attention through the converted metadata
    out = as_f64(run(p, dev=dev, force_grid=64))
    ref, _ = oracle.attn_problem(p)
    compare(out, ref, p.name)


@pytest.mark.gpu
@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_graph_replay_with_new_lengths_in_place(kv_dtype):
    """Metadata conversion + attention captured once in a HIP graph, replayed
    after the lengths, block tables and pools were rewritten in place: the
    plan and the graph hold no lengths, so each replay follows the device
    data (the PR #30105 page: the seq_lens addition must stay inside the
    captured graph).  Each replay is compared with the oracle."""
    import torch
    import paged_gqa_attention_va_amd as va
    from gpu_util import as_f64, compare
    q_lens = [4, 2, 3]
    probs = [va_inputs.custom(q_lens, [5000, 800, 64], 16, 1, kv_dtype, seed=71, extra_blocks=200,
                              window_left=900 if kv_dtype == "bf16" else -1, name="graph-a"),
             va_inputs.custom(q_lens, [1200, 4000, 2049], 16, 1, kv_dtype, seed=72, extra_blocks=200,
                              window_left=900 if kv_dtype == "bf16" else -1, name="graph-b")]
    nblk = max(p.num_blocks for p in probs)
    mbps = max(p.block_table.shape[1] for p in probs)
    ntok = max(int(p.seqused_k.sum()) for p in probs)
    elt = torch.uint8 if kv_dtype == "fp8" else torch.int16
    kpool = torch.zeros((nblk, 16, 1, 256), dtype=elt, device="cuda")
    vpool = torch.zeros_like(kpool)
    q = torch.empty((sum(q_lens), 16, 256), dtype=torch.bfloat16, device="cuda")
    cu = torch.from_numpy(probs[0].cu_seqlens_q).cuda()
    indptr = torch.zeros(len(q_lens) + 1, dtype=torch.int32, device="cuda")
    indices = torch.zeros(ntok, dtype=torch.int32, device="cuda")
    kd = torch.ones(1, dtype=torch.float32, device="cuda")
    plan = va.Plan(num_seqs=3, num_q_heads=16, num_kv_heads=1, max_seqlen_q=4, max_seqlen_k=mbps * 16,
                   max_blocks_per_seq=mbps, num_blocks=nblk, total_q=sum(q_lens), kv_dtype=kv_dtype,
                   window_left=probs[0].window_left)
    ws = plan.workspace()
    out = torch.empty_like(q)

    def load(p):                                   # rewrite every input in place
        ip, idx = token_slots(p)
        kv = lambda a: torch.from_numpy(a.view(np.int16) if kv_dtype == "bf16" else a)
        kpool.zero_()
        vpool.zero_()
        kpool[:p.num_blocks].copy_(kv(p.k))
        vpool[:p.num_blocks].copy_(kv(p.v))
        q.copy_(torch.from_numpy(p.q.view(np.int16)).view(torch.bfloat16))
        indptr.copy_(torch.from_numpy(ip))
        indices[:len(idx)].copy_(torch.from_numpy(idx))
        torch.cuda.synchronize()

    kview = kpool if kv_dtype == "fp8" else kpool.view(torch.bfloat16)
    vview = vpool if kv_dtype == "fp8" else vpool.view(torch.bfloat16)
    load(probs[0])
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        bt, sk = va.spec_block_table(indptr, indices, mbps, stream=s)
        plan.run(q, kview, vview, bt, cu, sk, probs[0].scale, kd, kd, out=out, workspace=ws, stream=s)
    for rep in range(2):
        for p in probs:
            load(p)
            out.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            ref, _ = oracle.attn_problem(p)
            compare(as_f64(out), ref, f"{p.name} replay {rep}")


@pytest.mark.gpu
@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_draft_extend_metadata_into_an_mla_plan(kv_dtype):
    # The PR #30105 summary page's draft-extend path with a query/key width
    # (576) other than the value width (512): the converted block table and
    # lengths drive the absorbed-MLA plan, whose output rows are 512 wide.
    import torch
    import paged_gqa_attention_va_amd as va
    from gpu_util import as_f64, compare
    p = va_inputs.mla([4, 1, 3], [3000, 17, 700], 16, kv_dtype, seed=31, k_descale=0.8, v_descale=1.25,
                      name=f"draft-extend-mla-{kv_dtype}")
    indptr, idx = token_slots(p)
    mbps = p.block_table.shape[1]
    bt, sk = va.spec_block_table(torch.from_numpy(indptr).cuda(), torch.from_numpy(idx).cuda(), mbps)
    pool = torch.from_numpy(p.k)
    if kv_dtype == "bf16":
        pool = pool.view(torch.int16).view(torch.bfloat16)
    pool = pool.cuda()
    q = torch.from_numpy(p.q.view(np.int16)).view(torch.bfloat16).cuda()
    cu = torch.from_numpy(p.cu_seqlens_q).cuda()
    kd = torch.tensor([p.k_descale], dtype=torch.float32, device="cuda")
    vd = torch.tensor([p.v_descale], dtype=torch.float32, device="cuda")
    plan = va.Plan.for_problem(p, force_grid=32)
    out = plan.run(q, pool, pool, bt, cu, sk, p.scale, kd, vd)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (p.total_q, p.num_q_heads, va_inputs.MLA_LATENT)
    ref, _ = oracle.attn_mla_problem(p)
    compare(as_f64(out), ref, p.name)
