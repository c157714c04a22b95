"""A seeded random sweep of valid calls against the fp64 oracle: every case
draws its own group size (4, 8, 16), kv heads (1, 2, 4), query lengths (0..4),
KV lengths (from one key to a few thousand, on and off page boundaries), cache
dtype, descales, and optionally a sliding window, a logit softcap and sinks; it
runs at the plan's own grid and at a small forced grid, and an FP8 case runs on
both FP8 kernels.  Same bar as test_gpu_parity.py (|gpu - ref| <= 1e-2 +
1e-2 |ref| on every element, rel-RMS <= 5e-3)."""
import numpy as np
import pytest

import va_inputs
from gpu_util import FP8_KERNELS, check_problem, kernel_for

pytestmark = pytest.mark.gpu

N_CASES = 48


def _case(i):
    rng = np.random.default_rng(1000 + i)
    G = int(rng.choice([4, 8, 16]))
    hkv = int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 7))
    q_lens = [int(x) for x in rng.integers(0, 5, size=B)]
    if max(q_lens) == 0:
        q_lens[0] = 1
    kv_lens = []
    for q in q_lens:
        kind = rng.integers(0, 4)
        k = {0: rng.integers(1, 33), 1: rng.integers(33, 700), 2: rng.integers(700, 6000),
             3: 16 * rng.integers(1, 200)}[int(kind)]
        kv_lens.append(max(int(k), q, 1))
    dt = "fp8" if rng.random() < 0.7 else "bf16"
    window = int(rng.integers(0, 600)) if rng.random() < 0.25 else -1
    softcap = float(rng.choice([0.7, 5.0, 30.0])) if rng.random() < 0.25 else 0.0
    sinks = list(rng.uniform(-3, 3, size=G * hkv)) if rng.random() < 0.25 else None
    kd = float(rng.uniform(0.5, 2.0))
    vd = float(rng.uniform(0.5, 2.0))
    return dict(q_lens=q_lens, kv_lens=kv_lens, hq=G * hkv, hkv=hkv, dt=dt, window=window, softcap=softcap,
                sinks=sinks, kd=kd, vd=vd)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case_matches_oracle(i):
    c = _case(i)
    p = va_inputs.custom(c["q_lens"], c["kv_lens"], c["hq"], c["hkv"], c["dt"], seed=2000 + i,
                         k_descale=c["kd"], v_descale=c["vd"], window_left=c["window"], softcap=c["softcap"],
                         sinks=c["sinks"], name=f"random{i}-{c['dt']}-G{c['hq'] // c['hkv']}-h{c['hkv']}")
    for grid in (0, 5):
        for k in (FP8_KERNELS if c["dt"] == "fp8" else (1,)):
            check_problem(p, force_grid=grid, kernel=kernel_for(c["dt"], k))
