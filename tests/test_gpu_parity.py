"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded
inputs, element by element, in every launch mode; plus the bit-exact and structural checks
(gather, page permutation, unused-slot NaNs, claim counts, determinism, bad page ids)."""
import sys

import numpy as np
import pytest
import torch

from hybrid_prefill_decode_paged_amd import binding as B
from hybrid_prefill_decode_paged_amd import inputs as gen
from oracle import attention as orc

from helpers import check_close, check_rows, checked_rows, problem, reference_rows, run_library, to_f64

pytestmark = pytest.mark.gpu
MODES = ["fused", "separate", "streams"]


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def _full_check(b, mode, what, **kw):
    _say(f"{what} mode={mode} {kw}")
    out, h, ws = run_library(b, mode=mode, **kw)
    want = problem(b).full_output()
    err = check_close(to_f64(out), want, b.spec.dtype, f"{what}/{mode}")
    return out, h, ws, err


@pytest.mark.parametrize("mode", MODES)
def test_config1_fp32_all_modes(mode):
    b = gen.make_batch(gen.config_spec(1), "cuda")
    _full_check(b, mode, "cfg1")


SMALL = [
    # (dtype, Hq, Hkv, D, prefill (q_len, ctx) pairs, decode ctx list)
    ("bf16", 4, 4, 128, [(64, 192)], [37, 100, 256, 257]),
    ("bf16", 8, 2, 128, [(100, 100), (33, 290), (1, 17)], [1, 15, 16, 17, 600]),
    ("bf16", 16, 2, 64, [(130, 700)], [2000, 31, 5]),
    ("bf16", 16, 1, 128, [(40, 1000), (17, 17)], [1, 4097]),
    ("bf16", 6, 2, 128, [(77, 200)], [999, 64]),
    ("fp32", 8, 4, 128, [(50, 130)], [300, 1]),
    ("fp32", 4, 1, 64, [(200, 480)], [77, 1025]),
    ("bf16", 4, 2, 128, [], [4096, 1000, 3]),
    ("bf16", 4, 2, 128, [(256, 3000), (0, 10)], []),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("mode", MODES)
def test_small_batches_all_modes(case, mode):
    dt, hq, hkv, d, pre, dec = SMALL[case]
    spec = gen.custom_spec(dt, Hq=hq, Hkv=hkv, D=d, prefill=pre, decode=dec, seed=100 + case)
    b = gen.make_batch(spec, "cuda")
    _full_check(b, mode, f"small{case}")


def test_prefill_heavy_batch_with_long_decode_splits():
    """A batch whose prefill share outweighs its decode share: fused handles plan longer decode
    splits (about one item per workgroup slot) than separate ones; both match the oracle on
    every output element."""
    spec = gen.custom_spec("bf16", Hq=8, Hkv=2, D=128, prefill=[(1024, 8192)],
                           decode=[20000, 15000, 9000, 30000, 12000, 25000, 4000, 33000], seed=31)
    b = gen.make_batch(spec, "cuda")
    splits = {}
    for mode in ("fused", "separate"):
        _, h, _, _ = _full_check(b, mode, "prefill-heavy")
        splits[mode] = h.stats()["decode_split_tokens"]
    assert splits["fused"] > splits["separate"], splits


@pytest.mark.parametrize("mode", MODES)
def test_forced_splits_use_the_combine(mode):
    """Short split lengths force multi-split prefill tiles and decode sequences, so the
    log-sum-exp combine (in-kernel last arriver, or the combine kernel) is exercised."""
    spec = gen.custom_spec("bf16", Hq=8, Hkv=2, D=128, prefill=[(150, 1500), (64, 64)],
                           decode=[1, 129, 700, 3000], seed=7)
    b = gen.make_batch(spec, "cuda")
    _, h, _, _ = _full_check(b, mode, "splits", decode_split_tokens=128, prefill_split_cap=16)
    st = h.stats()
    assert st["decode_max_splits"] > 1 and st["num_combine_groups"] > 0


def test_nan_in_unused_slots_changes_nothing():
    spec = gen.custom_spec("bf16", Hq=8, Hkv=2, D=128, prefill=[(45, 301)], decode=[17, 33, 250], seed=3)
    for mode in MODES:
        b = gen.make_batch(spec, "cuda")
        _say(f"nan-poison mode={mode}")
        ref, _, _ = run_library(b, mode=mode)
        gen.poison_unused(b, float("nan"))
        out, _, _ = run_library(b, mode=mode)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_permuted_and_identity_tables_bitwise_equal():
    spec = gen.custom_spec("bf16", Hq=8, Hkv=2, D=128, prefill=[(70, 500)], decode=[900, 31], seed=5,
                           identity_pages=True)
    b = gen.make_batch(spec, "cuda")
    perm = torch.randperm(spec.num_pages, generator=torch.Generator().manual_seed(0))
    b2 = gen.HybridBatch(**{**b.__dict__})
    b2.k_pool = torch.empty_like(b.k_pool)
    b2.v_pool = torch.empty_like(b.v_pool)
    b2.k_pool[perm.cuda()] = b.k_pool
    b2.v_pool[perm.cuda()] = b.v_pool
    bt2 = b.block_tables_host.copy()
    used = bt2 != gen.UNUSED_PAGE_ID
    bt2[used] = perm.numpy()[bt2[used]]
    b2.block_tables_host = bt2
    b2.block_tables = torch.from_numpy(bt2).cuda()
    for mode in MODES:
        _say(f"permuted-vs-identity mode={mode}")
        o1, _, _ = run_library(b, mode=mode)
        o2, _, _ = run_library(b2, mode=mode)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp32", 64), ("bf16", 64)])
def test_gather_is_bit_exact(dtype, D):
    spec = gen.custom_spec(dtype, Hq=4, Hkv=2, D=D, prefill=[(10, 77)], decode=[1, 16, 33, 300], seed=9)
    b = gen.make_batch(spec, "cuda")
    h = B.PodAttention(4, 2, D, dtype)
    meta = B.BatchMeta.from_batch(b)
    prob = problem(b)
    for seq, ctx in enumerate(spec.seq_ctx()):
        for which, pool in ((0, b.k_pool), (1, b.v_pool)):
            _say(f"gather {dtype} D={D} seq={seq} which={which}")
            out = torch.empty(ctx, 2, D, dtype=spec.torch_dtype, device="cuda")
            h.gather_kv(pool, which, b.block_tables, seq, ctx, meta, out)
            torch.cuda.synchronize()
            got = out.cpu()
            for g in range(2):
                K, V = orc.gather_kv(prob.k_pool, prob.v_pool, b.block_tables_host[seq], ctx, g, dtype)
                want = K if which == 0 else V
                np.testing.assert_array_equal(got[:, g].to(torch.float64).numpy(), want)


def test_gather_reports_an_out_of_pool_page():
    """pod_attn_gather_kv with a status word: an entry outside the pool is not read (its 16 tokens
    come out as zeros), the bad-page bit is set, and every other token equals the oracle's
    gather; a clean row leaves the word at 0."""
    spec = gen.custom_spec("bf16", Hq=4, Hkv=2, D=128, prefill=[(10, 77)], decode=[50], seed=9)
    b = gen.make_batch(spec, "cuda")
    h = B.PodAttention(4, 2, 128, "bf16")
    meta = B.BatchMeta.from_batch(b)
    prob = problem(b)
    bt = b.block_tables_host.copy()
    bt[0, 2] = spec.num_pages + 9                     # tokens 32 .. 47 of sequence 0
    bt_dev = torch.from_numpy(bt).cuda()
    for which, pool in ((0, b.k_pool), (1, b.v_pool)):
        _say(f"gather bad page which={which}")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        out = torch.full((77, 2, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        h.gather_kv(pool, which, bt_dev, 0, 77, meta, out, device_status=status)
        torch.cuda.synchronize()
        assert int(status.item()) & B.DEVICE_ERR_BAD_PAGE
        got = out.cpu().to(torch.float64).numpy()
        assert np.all(got[32:48] == 0.0)
        for g in range(2):
            K, V = orc.gather_kv(prob.k_pool, prob.v_pool, b.block_tables_host[0], 77, g, "bf16")
            want = K if which == 0 else V
            np.testing.assert_array_equal(np.delete(got[:, g], range(32, 48), axis=0),
                                          np.delete(want, range(32, 48), axis=0))
        status.zero_()
        h.gather_kv(pool, which, b.block_tables, 1, 50, meta, out[:50], device_status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0


def test_run_diagnostics_and_cumulative_counts(monkeypatch):
    """Per-handle counts of fused-path runs and of each fallback reason; after a run, the per-CU
    claim balance (every item claimed once, counted on the CU that ran it), the kernel time and
    the achieved rates; then a forced fallback (POD_ATTN_MODE) and a batch with no prefill."""
    spec = gen.custom_spec("bf16", Hq=8, Hkv=2, D=128, prefill=[(300, 2000)], decode=list(range(100, 3000, 97)),
                           seed=14)
    b = gen.make_batch(spec, "cuda")
    _say("diagnostics: fused run")
    out, h, ws = run_library(b, mode="fused")
    st = h.stats()
    assert st["runs"] == 1 and st["runs_fused_path"] == 1 and st["fallback_runs"] == [1, 0, 0, 0, 0]
    assert st["timed_run"] == 1 and st["kernel_us"] > 0
    assert abs(st["achieved_gbps"] - st["algorithmic_bytes"] / (st["kernel_us"] * 1e-6) / 1e9) < 1e-6 * st["achieved_gbps"]
    d = h.run_diagnostics(ws)
    assert d["status_word"] == 0 and d["run"] == 1 and d["timed_run"] == 1
    assert d["prefill_items"] == d["planned_prefill_items"] == st["num_prefill_items"] > 0
    assert d["decode_items"] == d["planned_decode_items"] == st["num_decode_items"] > 0
    assert d["cus_prefill"] > 0 and d["cus_decode"] > 0 and d["cus_any"] <= st["num_cus"]
    assert d["cus_both"] <= min(d["cus_prefill"], d["cus_decode"])
    assert 0.0 <= d["min_prefill_share"] <= d["mean_prefill_share"] <= d["max_prefill_share"] <= 1.0
    assert abs(d["prefill_decode_ratio"] - d["prefill_items"] / d["decode_items"]) < 1e-12
    assert d["kernel_us"] == st["kernel_us"]
    _say("diagnostics: decode-only batch")
    dspec = gen.custom_spec("bf16", Hq=8, Hkv=2, D=128, prefill=[], decode=[500, 3000], seed=15)
    db = gen.make_batch(dspec, "cuda")
    run_library(db, handle=h)
    st = h.stats()
    assert st["runs"] == 2 and st["runs_fused_path"] == 1
    assert st["fallback_runs"][B.FALLBACK["no_prefill"]] == 1 and st["fallback_reason"] == B.FALLBACK["no_prefill"]
    _say("diagnostics: forced fallback")
    monkeypatch.setenv("POD_ATTN_MODE", "separate")       # read when a handle is created
    out2, h2, ws2 = run_library(b, mode="fused")
    st2 = h2.stats()
    assert st2["mode_used"] == B.MODES["separate"] and st2["fallback_runs"][B.FALLBACK["env"]] == 1
    assert st2["runs_fused_path"] == 0
    d2 = h2.run_diagnostics(ws2)
    assert d2["prefill_items"] == st2["num_prefill_items"] and d2["decode_items"] == st2["num_decode_items"]
    assert d2["kernel_us"] > 0


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("fp32", 128)])
@pytest.mark.parametrize("mode", MODES)
def test_forced_splits_other_shapes(dtype, D, mode):
    spec = gen.custom_spec(dtype, Hq=8, Hkv=4, D=D, prefill=[(90, 1300), (16, 40)],
                           decode=[2, 400, 1900], seed=8)
    b = gen.make_batch(spec, "cuda")
    _, h, _, _ = _full_check(b, mode, f"splits-{dtype}-{D}", decode_split_tokens=128, prefill_split_cap=16)
    assert h.stats()["decode_max_splits"] > 1


@pytest.mark.parametrize("mode", ["fused", "separate"])
def test_decode_at_the_split_limit(mode):
    """A 64K-token decode with 512-token splits needs the largest split count (128), the size
    the combine tables are laid out for."""
    spec = gen.custom_spec("bf16", Hq=4, Hkv=2, D=128, prefill=[(32, 700)], decode=[65536, 300], seed=9)
    b = gen.make_batch(spec, "cuda")
    _, h, _, _ = _full_check(b, mode, "max-splits", decode_split_tokens=512)
    assert h.stats()["decode_max_splits"] == 128


@pytest.mark.parametrize("direction", ["rising", "falling"])
@pytest.mark.parametrize("mode", ["fused", "separate"])
def test_running_max_moves_by_large_steps(direction, mode):
    """K rows scaled by 2^(t/64) along every sequence (rising), or by its mirror (falling): the
    running maximum of the online softmax jumps by far more than 2^8 over and over (rising) or
    is set by the first keys and never moves (falling).  Both must match the oracle."""
    spec = gen.custom_spec("bf16", Hq=8, Hkv=2, D=128, prefill=[(200, 900), (64, 64)],
                           decode=[700, 1000, 33], seed=31)
    b = gen.make_batch(spec, "cuda")
    kr = gen.k_rows_view(b.k_pool)                 # [page, head, slot, D/x, x]
    for si, ctx in enumerate(spec.seq_ctx()):
        row = b.block_tables_host[si]
        for t0 in range(0, ctx, 16):
            page, n = int(row[t0 // 16]), min(16, ctx - t0)
            t = torch.arange(t0, t0 + n, device="cuda", dtype=torch.float32)
            f = torch.exp2(t / 64) if direction == "rising" else torch.exp2((ctx - 1 - t) / 64)
            kr[page, :, :n] = (kr[page, :, :n].float() * f.view(1, n, 1, 1)).to(kr.dtype)
    _full_check(b, mode, f"rescale-{direction}")


@pytest.mark.parametrize("mode", MODES)
def test_every_item_claimed_exactly_once(mode):
    spec = gen.custom_spec("bf16", Hq=8, Hkv=2, D=128, prefill=[(300, 2000), (50, 60)],
                           decode=list(range(1, 3000, 97)), seed=12)
    b = gen.make_batch(spec, "cuda")
    _say(f"claims mode={mode}")
    out, h, ws = run_library(b, mode=mode, flags=B.FLAG_DEBUG_CLAIMS, decode_split_tokens=256)
    st = h.stats()
    n = st["num_prefill_items"] + st["num_decode_items"]
    status, claims, per_cu = h.read_device_status(ws, n_items_cap=n, cu_cap=1024)
    assert status == 0
    assert len(claims) == n and np.all(claims == 1), np.unique(claims, return_counts=True)
    pf, dc = per_cu
    assert pf.sum() == st["num_prefill_items"] and dc.sum() == st["num_decode_items"]


@pytest.mark.parametrize("mode", ["fused", "separate"])
def test_trace_records_every_item(mode):
    """POD_ATTN_FLAG_TRACE: one timeline record per item, ends after starts, CU slots in range,
    kinds in item order, output unchanged by tracing.  Fused: prefill and decode items overlap in
    time (the two kinds share the machine).  Separate: every prefill item ends before the first
    decode item starts (one stream, prefill kernel first)."""
    spec = gen.custom_spec("bf16", Hq=8, Hkv=2, D=128, prefill=[(600, 9000), (200, 4000)],
                           decode=[3000 + 131 * i for i in range(40)], seed=21)
    b = gen.make_batch(spec, "cuda")
    _say(f"trace mode={mode}")
    ref, _, _ = run_library(b, mode=mode)
    out, h, ws = run_library(b, mode=mode, flags=B.FLAG_TRACE)
    assert torch.equal(out, ref)
    st = h.stats()
    npf, ndc = st["num_prefill_items"], st["num_decode_items"]
    rec = h.read_trace(ws).astype(np.int64)
    assert rec.shape == (npf + ndc, 4)
    t0 = rec[:, 0]
    dur = (rec[:, 1] - t0) % (1 << 32)
    assert np.all(dur < (1 << 31)), "an item ends before it starts"
    assert np.all(rec[:, 2] < 1024)
    assert np.all(rec[:npf, 3] == 0) and np.all(rec[npf:, 3] == 1)
    start = (t0 - t0.min()) % (1 << 32)
    end = start + dur
    pf, dc = slice(0, npf), slice(npf, npf + ndc)
    if mode == "fused":
        assert end[pf].max() > start[dc].min() and end[dc].max() > start[pf].min(), "kinds never overlapped"
    else:
        assert end[pf].max() <= start[dc].min()


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_run_to_run_bitwise_determinism(mode, dtype):
    spec = gen.custom_spec(dtype, Hq=32, Hkv=8, D=128, prefill=[(256, 2000)],
                           decode=[3000, 1500, 700, 40], seed=21)
    b = gen.make_batch(spec, "cuda")
    _say(f"determinism mode={mode} {dtype}")
    o1, h, ws = run_library(b, mode=mode, decode_split_tokens=256)
    o2 = torch.empty_like(o1)
    run_library(b, handle=h, out=o2, workspace=ws)
    o3 = torch.empty_like(o1)
    run_library(b, handle=h, out=o3, workspace=ws)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))


def test_out_of_pool_page_id_is_reported_not_read():
    """A used block-table entry outside the pool is never dereferenced: the kernels flag it in
    the workspace status word and treat that page as holding no keys."""
    spec = gen.custom_spec("bf16", Hq=4, Hkv=2, D=128, prefill=[(16, 64)], decode=[40, 20], seed=4)
    b = gen.make_batch(spec, "cuda")
    bt = b.block_tables_host.copy()
    bt[2, 1] = spec.num_pages + 1000            # row 2 = second decode (ctx 20): its second page
    b.block_tables_host = bt
    b.block_tables = torch.from_numpy(bt).cuda()
    for mode in MODES:
        _say(f"bad-page mode={mode}")
        out, h, ws = run_library(b, mode=mode)
        status, _, _ = h.read_device_status(ws)
        assert status & B.DEVICE_ERR_BAD_PAGE
        # sequences without a bad entry are unaffected
        prob = problem(b)
        want = np.stack([prob.sequence_output(s) for s in (0,)])[0]
        check_close(to_f64(out[:16]), want, "bf16", "bad-page/clean rows")
        assert not torch.isnan(out[16:]).any()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("split_cap", [0, 4])
def test_out_of_pool_entry_inside_a_prefill_chunk(dtype, split_cap):
    """A bad entry inside a prefill chunk's cached prefix: the chunk's rows equal attention with
    that page's 16 keys left out (the oracle's scores with those columns at -inf), every other
    sequence is unaffected, and the status word reports it."""
    spec = gen.custom_spec(dtype, Hq=8, Hkv=2, D=128, prefill=[(150, 1500), (20, 300)],
                           decode=[700], seed=12)
    b = gen.make_batch(spec, "cuda")
    prob = problem(b)                           # built from the clean table
    bad_pg = 10                                 # tokens 160 .. 175 of sequence 0
    bt = b.block_tables_host.copy()
    bt[0, bad_pg] = spec.num_pages + 77
    b.block_tables = torch.from_numpy(bt).cuda()
    for mode in MODES:
        _say(f"bad entry in a chunk dtype={dtype} split_cap={split_cap} mode={mode}")
        kw = {"prefill_split_cap": split_cap} if split_cap else {}
        out, h, ws = run_library(b, mode=mode, **kw)
        status, _, _ = h.read_device_status(ws)
        assert status & B.DEVICE_ERR_BAD_PAGE
        rows = prob.seq_rows(0)
        pos = np.array([prob.row_info(int(r))[1] for r in rows])
        want = np.empty((len(rows), spec.num_q_heads, spec.head_dim))
        for hh in range(spec.num_q_heads):
            K, V = prob.kv(0, prob.kv_head_of(hh), 1500)
            S = orc.masked_scores(prob.q_f64(rows, hh), pos, K, prob.scale)
            S[:, 16 * bad_pg: 16 * bad_pg + 16] = -np.inf
            want[:, hh] = orc.softmax_rows(S) @ V
        check_close(to_f64(out[rows]), want, dtype, f"bad-chunk/{dtype}/{mode}")
        for s in (1, 2):
            r = prob.seq_rows(s)
            check_close(to_f64(out[r]), prob.sequence_output(s), dtype, f"bad-chunk/clean seq {s}/{mode}")


def test_empty_batch_is_a_no_op():
    h = B.PodAttention(4, 2, 128, "bf16")
    meta = B.BatchMeta([0], [], [], 1, 1)
    q = torch.zeros(1, 4, 128, dtype=torch.bfloat16, device="cuda")
    h.run(q, q, q, torch.zeros(1, 1, dtype=torch.int32, device="cuda"), meta, q, None)
    torch.cuda.synchronize()


def test_workspace_too_small_is_rejected():
    spec = gen.custom_spec("bf16", Hq=4, Hkv=2, D=128, prefill=[(16, 64)], decode=[40], seed=4)
    b = gen.make_batch(spec, "cuda")
    h = B.PodAttention(4, 2, 128, "bf16")
    meta = B.BatchMeta.from_batch(b)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.PodAttnError) as e:
        h.run(b.q, b.k_pool, b.v_pool, b.block_tables, meta, torch.empty_like(b.q), ws)
    assert e.value.status == -3


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_million_token_contexts(dtype):
    """Contexts far past the measured workloads' 32K: a decode over 2^20 keys (a block-table row
    of 65,536 pages, split at most 128 ways) and a 64-row chunk at 300,000 keys, beside a
    17-key decode; every output element against the oracle, fused and separate."""
    spec = gen.custom_spec(dtype, Hq=8, Hkv=1, D=128, prefill=[(64, 300000)], decode=[1 << 20, 17], seed=77)
    _say(f"million-token contexts {dtype}: {spec.num_pages} pages")
    b = gen.make_batch(spec, "cuda")
    want = problem(b).full_output()
    for mode in ("fused", "separate"):
        _say(f"million-token contexts {dtype} mode={mode}")
        out, h, ws = run_library(b, mode=mode)
        check_close(to_f64(out), want, dtype, f"million/{dtype}/{mode}")
        st = h.stats()
        assert 1 < st["decode_max_splits"] <= 128 and st["prefill_max_splits"] <= 128, st
        h.close()
        del ws
    del b
    torch.cuda.empty_cache()


def test_thousands_of_short_sequences():
    """4,000 decodes of 1 to 300 keys beside three prefill chunks: far more sequences than
    workgroup slots, most of them a single partial page; every output element against the
    oracle in every mode."""
    rng = np.random.Generator(np.random.PCG64(88))
    dec = rng.integers(1, 300, size=4000, endpoint=True).tolist()
    spec = gen.custom_spec("bf16", Hq=8, Hkv=2, D=64, prefill=[(100, 100), (37, 5000), (300, 1200)],
                           decode=dec, seed=88)
    b = gen.make_batch(spec, "cuda")
    want = problem(b).full_output()
    for mode in MODES:
        _say(f"4000 short sequences mode={mode}")
        out, h, ws = run_library(b, mode=mode)
        check_close(to_f64(out), want, "bf16", f"many-seqs/{mode}")
        h.close()


# ------------------------------------------------------------------ full-size workloads
# Every mode against the fp64 oracle at the workloads' full sizes, in the launch configuration
# the bench times: every decode row (every 8th of the 256 long-context ones) and the first and
# last row of every prefill tile, all query heads; and every output row written.
FULL_DECODE_EVERY = {2: 1, 3: 1, 4: 1, 5: 8}


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_full_size_workloads_every_mode(idx):
    spec = gen.config_spec(idx)
    _say(f"cfg{idx}: generating {spec.num_pages} pages")
    b = gen.make_batch(spec, "cuda")
    outs, tq = {}, None
    for mode in MODES:
        _say(f"cfg{idx} mode={mode}")
        out, h, ws = run_library(b, mode=mode)
        outs[mode] = out
        tq = h.stats()["prefill_tile_queries"]
        del ws
    per_seq = checked_rows(b, tq, FULL_DECODE_EVERY[idx])
    _say(f"cfg{idx}: oracle on {sum(len(r) for _, r in per_seq)} rows x {spec.num_q_heads} heads")
    rows, want = reference_rows(b, per_seq)
    for mode in MODES:
        check_rows(outs[mode], rows, want, "bf16", f"cfg{idx}/{mode}")
    del outs, b
    torch.cuda.empty_cache()
