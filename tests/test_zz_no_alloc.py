"""va_run_noalloc, the entry point that allocates nothing, against va_run_ex
with a caller-allocated workspace: the same kernels, so the outputs must be
identical, on two calls in a row, the second with a smaller input (the
library's scratch then still holds the first call's partials).  The small
call is also checked against the oracle at the parity bar.  A plan whose
workspace exceeds the scratch is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import oracle
import paged_gqa_attention_va_amd as va
import va_inputs
from gpu_util import as_f64, compare, note, to_device

pytestmark = pytest.mark.gpu


def _both(p):
    dev = to_device(p)
    plan = va.Plan.for_problem(p)
    note(f"  {p.name}: grid={plan.grid} workspace={plan.workspace_bytes} B")
    ref = plan.run(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cu"], dev["sk"], p.scale, dev["kd"], dev["vd"],
                   sinks=dev["sinks"])
    got = plan.run_noalloc(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cu"], dev["sk"], p.scale, dev["kd"],
                           dev["vd"], sinks=dev["sinks"])
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_equals_workspace_entry_on_two_calls():
    big = va_inputs.custom([4, 3, 4, 2] * 4, [9000, 20000, 4099, 700] * 4, 16, 1, "fp8", seed=61,
                           k_descale=1.25, v_descale=0.75, name="noalloc-big")
    small = va_inputs.custom([4, 2], [1024, 769], 16, 1, "fp8", seed=62, name="noalloc-small")
    for p in (big, small):
        ref, got = _both(p)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), p.name
    compare(as_f64(got), oracle.attn_problem(small)[0], "noalloc-small vs oracle")


def test_noalloc_bf16_and_sinks():
    p = va_inputs.custom([3, 1, 2], [5000, 129, 3], 8, 2, "bf16", seed=63, sinks=[0.5] * 8, name="noalloc-bf16")
    ref, got = _both(p)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_noalloc_refuses_a_plan_beyond_its_scratch():
    p = va_inputs.custom([4, 2], [1024, 769], 16, 1, "bf16", seed=64)
    plan = va.Plan.for_problem(p, force_grid=65536)
    assert plan.workspace_bytes > 80 << 20
    dev = to_device(p)
    with pytest.raises(va.VaError) as e:
        plan.run_noalloc(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cu"], dev["sk"], p.scale, dev["kd"],
                         dev["vd"])
    assert e.value.status == va.VA_ERR_WORKSPACE
