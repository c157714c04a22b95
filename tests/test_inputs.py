"""The seeded input generator: determinism, shapes and the poison recipe."""
import numpy as np

import va_inputs


def test_same_seed_same_bytes():
    a = va_inputs.custom([4, 2], [100, 37], 16, 1, "fp8", seed=5)
    b = va_inputs.custom([4, 2], [100, 37], 16, 1, "fp8", seed=5)
    c = va_inputs.custom([4, 2], [100, 37], 16, 1, "fp8", seed=6)
    for f in ("q", "k", "v", "block_table", "cu_seqlens_q", "seqused_k"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert not np.array_equal(a.q, c.q)


def test_config0_shape_follows_the_page_test():
    p = va_inputs.config(0)
    assert p.q.shape == (6, 16, 256) and p.q.dtype == np.uint16
    assert p.k.shape == (128, 16, 1, 256) and p.k.dtype == np.uint8
    assert list(p.cu_seqlens_q) == [0, 4, 6] and list(p.seqused_k) == [1024, 769]
    assert p.block_table.shape == (2, 64)
    # identity table within the used pages; poisoned (out of range) past them
    assert np.array_equal(p.block_table[0], np.arange(64))
    assert np.array_equal(p.block_table[1, :49], np.arange(64, 113))
    assert np.all(p.block_table[1, 49:] >= p.num_blocks)
    assert p.scale == np.float32(1 / 16) and p.k_descale == 1.0 and p.v_descale == 1.0


def test_config1_two_kv_heads():
    p = va_inputs.config(1)
    assert p.q.shape == (6, 32, 256) and p.k.shape == (128, 16, 2, 256)


def test_poison_covers_page_tails_and_unused_pages():
    p = va_inputs.config(0)
    last = p.block_table[1, 48]                 # 769 = 48*16 + 1 -> slot 0 valid only
    assert np.all(p.k[last, 1:] == va_inputs.FP8_NAN)
    assert np.all(p.v[last, 1:] == va_inputs.FP8_NAN)
    assert np.all(p.k[113:] == va_inputs.FP8_NAN)
    assert not np.any(p.k[last, 0] == va_inputs.FP8_NAN)


def test_unpoisoned_variant_has_no_nan_codes():
    p = va_inputs.config(0, poison=False)
    assert not np.any((p.k & 0x7F) == 0x7F)
    assert not np.any((p.v & 0x7F) == 0x7F)


def test_config3_lengths_and_descales():
    p = va_inputs.config(3, poison=False)
    assert p.num_seqs == 64 and np.all(p.q_lens == 3)
    assert p.seqused_k.min() >= 8192 and p.seqused_k.max() <= 65536
    assert 0.5 <= p.k_descale <= 2.0 and 0.5 <= p.v_descale <= 2.0
    # every page appears exactly once in the permuted table
    pages = np.ceil(p.seqused_k / 16).astype(int)
    used = np.concatenate([p.block_table[b, :pages[b]] for b in range(64)])
    assert np.array_equal(np.sort(used), np.arange(p.num_blocks))


def test_sample_rows_cover_every_sequence_boundary():
    p = va_inputs.custom([1, 3, 0, 2, 4], [20, 40, 9, 33, 70], 8, 1, "fp8", seed=4)
    rows = va_inputs.sample_rows(p, 5, seed=2)
    assert np.all(np.diff(rows) > 0) and rows[0] >= 0 and rows[-1] < p.total_q * 8
    tokens = set((rows // 8).tolist())
    cu = p.cu_seqlens_q
    for b in range(p.num_seqs):
        if cu[b + 1] > cu[b]:
            assert int(cu[b]) in tokens and int(cu[b + 1]) - 1 in tokens
    assert np.array_equal(va_inputs.sample_rows(p, 10 ** 6), np.arange(p.total_q * 8))
