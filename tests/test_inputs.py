"""Host checks of the seeded input generator (no attention arithmetic here)."""
import math

import numpy as np
import torch

from hybrid_prefill_decode_paged_amd import inputs as gen


def test_workload_sizes():
    # live pages = sum of ceil(ctx / 16) over sequences
    assert gen.config_spec(1).live_pages() == 12 + 3 + 7 + 16 + 17
    assert gen.config_spec(2).live_pages() == 256 + 64 * 256
    assert gen.config_spec(5).live_pages() == 2048 + 256 * 2048 == 526_336
    assert gen.config_spec(5).num_pages == 1 << 20
    c3 = gen.config_spec(3)
    assert len(c3.decode_ctx_len) == 128 and min(c3.decode_ctx_len) >= 4096 and max(c3.decode_ctx_len) <= 32768
    c4 = gen.config_spec(4)
    assert len(c4.decode_ctx_len) == 96 and min(c4.decode_ctx_len) >= 1024 and max(c4.decode_ctx_len) <= 32768
    assert c4.prefill_ctx_len == [512, 8704, 28512] and c4.prefill_q_len == [512] * 3
    for i in (3, 4):
        s = gen.config_spec(i)
        assert s.num_pages == s.live_pages() + s.live_pages() // 4
    # the draws are reproducible
    assert gen.config_spec(3).decode_ctx_len == c3.decode_ctx_len


def test_block_tables_are_disjoint_and_in_range():
    for i in (1, 2, 3, 4):
        s = gen.config_spec(i)
        bt = gen.block_tables_for(s)
        used = []
        for row, c in zip(bt, s.seq_ctx()):
            n = -(-c // 16)
            used.append(row[:n])
            assert np.all(row[n:] == gen.UNUSED_PAGE_ID)
        used = np.concatenate(used)
        assert used.min() >= 0 and used.max() < s.num_pages
        assert len(np.unique(used)) == len(used)


def test_config1_layout_and_determinism():
    s = gen.config_spec(1)
    b1, b2 = gen.make_batch(s), gen.make_batch(s)
    assert torch.equal(b1.q, b2.q) and torch.equal(b1.k_pool, b2.k_pool) and torch.equal(b1.v_pool, b2.v_pool)
    assert tuple(b1.q.shape) == (64 + 4, 4, 64)
    assert tuple(b1.k_pool.shape) == (64, 4, 16, 16, 4)
    assert tuple(b1.v_pool.shape) == (64, 4, 64, 16)
    assert list(b1.prefill_q_start) == [0, 64]


def test_outlier_rows_exact_count():
    s = gen.reduced_spec(4, n_decode=4, ctx_div=64)
    base = gen.make_batch(gen.replace(s, k_outlier_frac=0.0))
    b = gen.make_batch(s)
    n_rows = sum(s.seq_ctx()) * s.num_kv_heads
    kr0, kr1 = gen.k_rows_view(base.k_pool).float(), gen.k_rows_view(b.k_pool).float()
    changed = (kr0 != kr1).flatten(3).any(-1)              # [P, Hkv, 16]
    assert int(changed.sum()) == math.floor(0.01 * n_rows)
    ratio = kr1[changed] / kr0[changed]
    assert torch.all((ratio == 8.0) | (kr0[changed] == 0))
