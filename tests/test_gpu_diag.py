"""GPU checks of the diagnostic entry points used by bench.py: the streaming
ceiling's copy path (va_stream_pages) must really copy every listed page."""
import numpy as np
import pytest
import torch

import paged_gqa_attention_va_amd as va

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("depth", [2, 6, 10])
def test_stream_pages_copies_every_listed_page(depth):
    rng = np.random.default_rng(depth)
    n_pool, grid = 1024, 3
    pool_h = rng.integers(0, 256, size=n_pool * 4096, dtype=np.uint8)
    pages_h = np.concatenate([rng.permutation(n_pool)[:900], rng.integers(0, n_pool, 100),
                              [-5, n_pool + 7, 0, n_pool - 1]]).astype(np.int32)
    pool = torch.from_numpy(pool_h).cuda()
    pages = torch.from_numpy(pages_h).cuda()
    sums = va.stream_pages(pool, pages, depth, grid)
    torch.cuda.synchronize()
    first = pool_h.view(np.uint32)[::1024].astype(np.uint64)            # first word of every page
    clamped = np.clip(pages_h, 0, n_pool - 1)
    nw, n = grid * 4, len(pages_h)
    want = []
    for w in range(nw):
        a, b = (w * n) // nw, ((w + 1) * n) // nw
        want.append(int(first[clamped[a:b]].sum() % (1 << 32)))
    got = (sums.cpu().numpy().astype(np.int64) & 0xFFFFFFFF).tolist()
    assert got == want
