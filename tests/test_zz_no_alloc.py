"""pod_attn_run_noalloc (workspace from the library's fixed per-GPU scratch, nothing allocated)
against pod_attn_run with a workspace of its own, through the C ABI: two calls in a row, the
second on a smaller batch (the scratch keeps the first call's contents), in every mode, bitwise
equal and within the bf16 tolerance of the fp64 oracle; plus the rejected calls."""
import sys

import pytest
import torch

from hybrid_prefill_decode_paged_amd import binding as B
from hybrid_prefill_decode_paged_amd import inputs as gen

from helpers import check_close, problem, run_library, to_f64

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


@pytest.mark.parametrize("mode", ["fused", "separate", "streams"])
def test_noalloc_matches_run_on_two_calls_in_a_row(mode):
    big = gen.custom_spec("bf16", Hq=32, Hkv=8, D=128, prefill=[(300, 5000), (40, 41)],
                          decode=[9000, 3000, 17, 700], seed=61)
    small = gen.custom_spec("bf16", Hq=32, Hkv=8, D=128, prefill=[(20, 100)], decode=[33, 1], seed=62)
    h = B.PodAttention(32, 8, 128, "bf16", mode, decode_split_tokens=512, prefill_split_cap=4)
    for name, spec in (("larger", big), ("smaller", small)):
        b = gen.make_batch(spec, "cuda")
        meta = B.BatchMeta.from_batch(b)
        _say(f"noalloc mode={mode} {name} batch")
        ref, _, _ = run_library(b, handle=h)
        assert h.stats()["num_combine_groups"] > 0 or name == "smaller"
        out = torch.full_like(b.q, float("nan"))
        h.run_noalloc(b.q, b.k_pool, b.v_pool, b.block_tables, meta, out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{mode}/{name}: differs from pod_attn_run"
        check_close(to_f64(out), problem(b).full_output(), "bf16", f"noalloc/{mode}/{name}")


def test_noalloc_fp32_matches_run():
    spec = gen.custom_spec("fp32", Hq=8, Hkv=4, D=64, prefill=[(90, 1300)], decode=[2, 400, 1900], seed=63)
    b = gen.make_batch(spec, "cuda")
    h = B.PodAttention(8, 4, 64, "fp32", "fused", decode_split_tokens=128)
    _say("noalloc fp32")
    ref, _, _ = run_library(b, handle=h)
    out = torch.full_like(b.q, float("nan"))
    h.run_noalloc(b.q, b.k_pool, b.v_pool, b.block_tables, B.BatchMeta.from_batch(b), out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_noalloc_rejects_a_batch_beyond_the_scratch_and_fp8():
    """140 decodes at 16K with 128-token splits need ~280 MiB of split partials: rejected before any
    launch, with the scratch size in the message; an FP8 handle needs its scales.  A normal call on
    the same handle still works afterwards."""
    n = 140
    h = B.PodAttention(32, 8, 128, "bf16", "fused", decode_split_tokens=128)
    meta = B.BatchMeta([0], [], [16384] * n, 1024, 1)
    assert h.workspace_size(meta) > B.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(n, 32, 128, dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros(8 * 16 * 128, dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros(n, 1024, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    _say("noalloc oversized batch")
    with pytest.raises(B.PodAttnError) as e:
        h.run_noalloc(q, pool, pool, bt, meta, out)
    assert e.value.status == -3 and "scratch" in str(e.value)
    spec = gen.custom_spec("bf16", Hq=32, Hkv=8, D=128, prefill=[(16, 40)], decode=[50], seed=64)
    b = gen.make_batch(spec, "cuda")
    ref, _, _ = run_library(b, handle=h)
    got = torch.full_like(b.q, float("nan"))
    h.run_noalloc(b.q, b.k_pool, b.v_pool, b.block_tables, B.BatchMeta.from_batch(b), got)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    hf = B.PodAttention(32, 32, 128, "fp8", "fused")
    fb = gen.custom_spec("fp8", Hq=32, Hkv=32, D=128, prefill=[(16, 40)], decode=[50], seed=65)
    fbb = gen.make_batch(fb, "cuda")
    with pytest.raises(B.PodAttnError) as e:
        hf.run_noalloc(fbb.q, fbb.k_pool, fbb.v_pool, fbb.block_tables, B.BatchMeta.from_batch(fbb),
                       torch.empty_like(fbb.q))
    assert e.value.status == -1


@pytest.mark.parametrize("mode", ["fused", "separate", "streams"])
def test_noalloc_random_sequence_matches_run(mode):
    """Twelve seeded random batches in a row on one handle, larger and smaller in turn, with and
    without splits: every call bitwise equal to pod_attn_run, so nothing the scratch keeps from
    the call before leaks into the next."""
    import random
    rng = random.Random(7300 + ["fused", "separate", "streams"].index(mode))
    h = B.PodAttention(16, 4, 128, "bf16", mode, decode_split_tokens=rng.choice([256, 512]), prefill_split_cap=4)
    for i in range(12):
        pre = [(rng.choice([1, 3, 17, 128, 129, 300]), 0) for _ in range(rng.randint(0, 2))]
        pre = [(L, L + rng.choice([0, 15, 700, 4000])) for L, _ in pre]
        dec = [rng.choice([1, 16, 17, 255, 1000, 6000]) for _ in range(rng.randint(0 if pre else 1, 5))]
        spec = gen.custom_spec("bf16", Hq=16, Hkv=4, D=128, prefill=pre, decode=dec, seed=7400 + i)
        b = gen.make_batch(spec, "cuda")
        meta = B.BatchMeta.from_batch(b)
        _say(f"noalloc sequence mode={mode} call {i}: prefill={pre} decode={dec}")
        ref, _, _ = run_library(b, handle=h)
        out = torch.full_like(b.q, float("nan"))
        h.run_noalloc(b.q, b.k_pool, b.v_pool, b.block_tables, meta, out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{mode}/call {i}: differs from pod_attn_run"
