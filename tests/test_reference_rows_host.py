"""The full-size GPU checks compute their reference one sequence at a time (each sequence's pages
renumbered into a one-sequence problem, on a pool of threads).  On the CPU: that plumbing gives
the rows of the oracle on the whole batch (to fp64 rounding: BLAS may block a subset of rows
differently), for bf16, fp32 and FP8 caches, and the rows it
picks are the first and last row of every prefill tile and every k-th decode row."""
import numpy as np
import pytest

from hybrid_prefill_decode_paged_amd import inputs as gen

from helpers import checked_rows, problem, reference_rows


@pytest.mark.parametrize("dtype", ["bf16", "fp32", "fp8"])
def test_per_sequence_reference_equals_the_batch_oracle(dtype):
    spec = gen.custom_spec(dtype, Hq=8, Hkv=2, D=64, prefill=[(70, 300), (5, 5), (33, 100)],
                           decode=[1, 17, 600, 33, 250], seed=3)
    b = gen.make_batch(spec, "cpu")
    per_seq = checked_rows(b, tile_queries=16, decode_every=2)
    rows, want = reference_rows(b, per_seq, workers=4)
    full = problem(b).full_output()
    np.testing.assert_allclose(want, full[rows], rtol=1e-12, atol=1e-14)


def test_checked_rows_are_tile_edges_and_every_kth_decode():
    spec = gen.custom_spec("bf16", Hq=4, Hkv=1, D=64, prefill=[(70, 300), (5, 5)],
                           decode=[10] * 9, seed=1)
    b = gen.make_batch(spec, "cpu")
    per_seq = checked_rows(b, tile_queries=32, decode_every=4)
    assert per_seq[0] == (0, [0, 31, 32, 63, 64, 69])
    assert per_seq[1] == (1, [70, 74])
    assert [r for _, (r,) in per_seq[2:]] == [75 + d for d in (0, 4, 8)]
