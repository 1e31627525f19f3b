"""GPU check of the measured cost table: every bucket of a small grid runs on the fused path with
no device error and a finite output and matches the fp64 oracle on its sampled rows (so it is
validated, with its errors recorded), its timings are positive and ordered (max >= median), its
signals are the host's for that bucket, and lookups round batches up to the right bucket; the
same for an FP8 cache.  A reference that disagrees, or none, leaves every bucket unvalidated and
lookups empty."""
import sys

import pytest
import torch

from hybrid_prefill_decode_paged_amd import binding as B
from hybrid_prefill_decode_paged_amd.cost_table import CostTable, bucket_batch, calibrate

from helpers import bucket_reference

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def test_small_grid_calibrates_and_looks_up():
    print("[gpu-test] cost table 8/2/128 bf16, 2x1x2x2 grid", flush=True)
    sys.stdout.flush()
    t = calibrate(8, 2, 128, "bf16", [0, 64], [1024], [0, 8], [512, 2048], steps=3, reference=bucket_reference)
    keys = [e.key() for e in t.entries]
    assert keys == sorted(keys) and len(keys) == 5        # (0,0,8,512) ... (64,1024,8,2048)
    for e in t.entries:
        assert e.validated, e
        assert e.max_abs_err <= 2e-2 and e.mean_abs_err <= 2e-3
        assert 0 < e.kernel_us_p50 <= e.kernel_us_max and 0 < e.step_us_p50 <= e.step_us_max
        q_start, p_ctx, d_ctx = bucket_batch(*e.key())
        meta = B.BatchMeta(q_start, p_ctx, d_ctx, 128, 1 << 16)
        sig = B.batch_signals(B.make_config(8, 2, 128), meta, 256, 2)
        assert sig["roofline_us"] == e.signals["roofline_us"] or abs(sig["roofline_us"] - e.signals["roofline_us"]) < 1e-9
    hit = t.lookup(30, 900, 5, 600)
    assert hit is not None and hit.key() == (64, 1024, 8, 2048)
    assert t.lookup(0, 0, 8, 400).key() == (0, 0, 8, 512)
    assert t.lookup(65, 100, 0, 0) is None
    assert t.lookup(10, 100, 0, 0).key() == (64, 1024, 0, 0)
    assert CostTable.from_json(t.to_json()).lookup(30, 900, 5, 600).key() == (64, 1024, 8, 2048)


def test_fp8_cache_grid_is_validated():
    """The same calibration for an FP8 E4M3 cache (per-slab scales that are not powers of two):
    every bucket validated against the oracle's decoded cache at the bf16 tolerance."""
    print("[gpu-test] cost table 8/2/128 fp8, 2x1x2x1 grid", flush=True)
    sys.stdout.flush()
    t = calibrate(8, 2, 128, "fp8", [0, 64], [1024], [0, 8], [2048], steps=2, reference=bucket_reference)
    assert t.dtype == "fp8" and len(t.entries) == 3
    for e in t.entries:
        assert e.validated, e
        assert e.max_abs_err <= 2e-2 and e.mean_abs_err <= 2e-3
    assert t.lookup(30, 900, 5, 600).key() == (64, 1024, 8, 2048)


def test_buckets_that_disagree_with_the_reference_are_not_validated():
    print("[gpu-test] cost table with a disagreeing reference and with none", flush=True)
    sys.stdout.flush()
    t = calibrate(8, 2, 128, "bf16", [64], [1024], [8], [512], steps=1, reference=lambda run: (0.5, 0.1))
    assert len(t.entries) == 1 and not t.entries[0].validated and t.entries[0].max_abs_err == 0.5
    assert t.lookup(64, 1024, 8, 512) is None
    t = calibrate(8, 2, 128, "bf16", [64], [1024], [8], [512], steps=1)
    assert not t.entries[0].validated and t.entries[0].max_abs_err is None
