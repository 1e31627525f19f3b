"""GPU parity of the FP8 (OCP E4M3) cache with per-(page, KV head) scales: the gather moves codes
bit-exactly and the kernels' E4M3 -> bf16 conversion matches torch's float8_e4m3fn on every code;
attention over the scaled codes matches the oracle (which decodes the same codes by the format's
definition) in every mode, with splits, with NaN codes in unused slots, and at full size."""
import sys

import numpy as np
import pytest
import torch

from hybrid_prefill_decode_paged_amd import binding as B
from hybrid_prefill_decode_paged_amd import inputs as gen

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


@pytest.mark.parametrize("D", [64, 128])
def test_gather_codes_and_conversion(D):
    spec = gen.custom_spec("fp8", Hq=4, Hkv=2, D=D, prefill=[(10, 77)], decode=[1, 16, 33], seed=50)
    b = gen.make_batch(spec, "cuda")
    # every code at least once: overwrite the first page of sequence 0 with all 256 codes
    pg = int(b.block_tables_host[0][0])
    codes = torch.arange(256, dtype=torch.uint8, device="cuda").repeat(2 * 16 * D // 256 + 1)
    b.k_pool[pg].view(-1).copy_(codes[: b.k_pool[pg].numel()])
    b.v_pool[pg].view(-1).copy_(codes[7: 7 + b.v_pool[pg].numel()])
    h = B.PodAttention(4, 2, D, "fp8")
    meta = B.BatchMeta.from_batch(b)
    for seq, ctx in enumerate(spec.seq_ctx()):
        for which, pool in ((0, b.k_pool), (1, b.v_pool)):
            _say(f"fp8 gather D={D} seq={seq} which={which}")
            raw = torch.empty(ctx, 2, D, dtype=torch.uint8, device="cuda")
            h.gather_kv(pool, which, b.block_tables, seq, ctx, meta, raw)
            dec = torch.empty(ctx, 2, D, dtype=torch.bfloat16, device="cuda")
            h.gather_kv(pool, which + 2, b.block_tables, seq, ctx, meta, dec)
            torch.cuda.synchronize()
            # codes: the pool read through the layout of the ABI header
            rows = gen.k_rows_view(pool) if which == 0 else gen.v_rows_view(pool)
            pages = torch.as_tensor(b.block_tables_host[seq][: -(-ctx // 16)].astype(np.int64), device="cuda")
            if which == 1:
                want = rows[pages].permute(0, 2, 1, 3).reshape(-1, 2, D)[:ctx]
            else:
                want = rows[pages].permute(0, 2, 1, 3, 4).reshape(-1, 2, D)[:ctx]
            assert torch.equal(raw, want)
            conv = raw.view(torch.float8_e4m3fn).to(torch.bfloat16)
            nan = torch.isnan(conv)                     # NaN codes: any NaN (payloads differ)
            assert torch.equal(torch.isnan(dec), nan)
            assert torch.equal(dec.view(torch.int16)[~nan], conv.view(torch.int16)[~nan])


FP8_CASES = [
    # (Hq, Hkv, D, prefill (q_len, ctx) pairs, decode ctx list)
    (8, 2, 128, [(64, 192), (4, 300), (37, 37)], [1, 17, 256, 1000]),
    (32, 8, 128, [(130, 2000)], [4096, 5, 33]),
    (16, 2, 64, [(100, 700), (2, 2000)], [999, 64]),
    (4, 4, 128, [(200, 3000)], []),
    (8, 1, 128, [], [4097, 3, 600]),
]


@pytest.mark.parametrize("case", range(len(FP8_CASES)))
@pytest.mark.parametrize("mode", MODES)
def test_fp8_matches_the_oracle(case, mode):
    hq, hkv, d, pre, dec = FP8_CASES[case]
    spec = gen.custom_spec("fp8", Hq=hq, Hkv=hkv, D=d, prefill=pre, decode=dec, seed=60 + case)
    b = gen.make_batch(spec, "cuda")
    gen.poison_unused(b)                    # NaN codes in every slot no live token owns
    _say(f"fp8 case={case} mode={mode}")
    out, _, _ = run_library(b, mode=mode)
    check_close(to_f64(out), problem(b).full_output(), "fp8", f"fp8-{case}/{mode}")


@pytest.mark.parametrize("mode", MODES)
def test_fp8_with_splits(mode):
    spec = gen.custom_spec("fp8", Hq=8, Hkv=2, D=128, prefill=[(150, 9000), (3, 600)],
                           decode=[129, 700, 3000], seed=70)
    b = gen.make_batch(spec, "cuda")
    _say(f"fp8 splits mode={mode}")
    out, h, _ = run_library(b, mode=mode, decode_split_tokens=128, prefill_split_cap=16)
    assert h.stats()["decode_max_splits"] > 1 and h.stats()["prefill_max_splits"] > 1
    check_close(to_f64(out), problem(b).full_output(), "fp8", f"fp8-splits/{mode}")


@pytest.mark.parametrize("mode", MODES)
def test_fp8_general_scales(mode):
    """Scales that are not powers of two: each (page, KV head) scale multiplied by a factor drawn
    from [0.6, 1.5], which keeps the values' law; the scaled scores and the scaled probabilities
    are then rounded, and a scale applied to the wrong page, head or side of the product shows."""
    spec = gen.custom_spec("fp8", Hq=8, Hkv=2, D=128, prefill=[(150, 1500), (40, 900), (3, 70)],
                           decode=[1, 37, 900, 2500], seed=73)
    b = gen.make_batch(spec, "cuda")
    gen.poison_unused(b)
    rng = np.random.Generator(np.random.PCG64(730))
    for t in (b.k_scale, b.v_scale):
        t.mul_(torch.from_numpy(rng.uniform(0.6, 1.5, size=tuple(t.shape)).astype(np.float32)).to(t.device))
    _say(f"fp8 general scales mode={mode}")
    out, _, _ = run_library(b, mode=mode, decode_split_tokens=256, prefill_split_cap=4)
    check_close(to_f64(out), problem(b).full_output(), "fp8", f"fp8-scales/{mode}")


@pytest.mark.parametrize("mode", MODES)
def test_fp8_scales_outside_the_usual_range(mode):
    """Page scales a quantiser would not produce -- zero, negative and 1.3 * 2^-70 -- on about a
    fifth of the pages, K and V drawn apart: the prefill tile multiplies such a scale into its
    page's bf16 values when it converts them (instead of folding it into the exponent), the
    decode path multiplies scores and probabilities by it; both against the oracle on every
    output element.  (Scales above 2^64 take the same path; they make every softmax one-hot
    with outputs too large for an absolute tolerance, so they are not drawn here.)"""
    spec = gen.custom_spec("fp8", Hq=8, Hkv=2, D=128, prefill=[(150, 1500), (40, 900), (3, 70)],
                           decode=[1, 37, 900, 2500], seed=74)
    b = gen.make_batch(spec, "cuda")
    gen.poison_unused(b)
    rng = np.random.Generator(np.random.PCG64(740))
    odd = np.array([0.0, -0.75, 1.3 * 2.0 ** -70], dtype=np.float32)
    for t in (b.k_scale, b.v_scale):
        sc = t.cpu().numpy()
        pick = rng.random(sc.shape) < 0.2
        sc[pick] = odd[rng.integers(0, len(odd), size=int(pick.sum()))]
        t.copy_(torch.from_numpy(sc))
    _say(f"fp8 scales outside the usual range mode={mode}")
    out, _, _ = run_library(b, mode=mode, decode_split_tokens=256, prefill_split_cap=4)
    check_close(to_f64(out), problem(b).full_output(), "fp8", f"fp8-odd-scales/{mode}")


def test_fp8_entry_points_reject_what_they_cannot_do():
    spec = gen.custom_spec("fp8", Hq=4, Hkv=2, D=128, prefill=[(8, 40)], decode=[9], seed=71)
    b = gen.make_batch(spec, "cuda")
    h = B.PodAttention(4, 2, 128, "fp8")
    meta = B.BatchMeta.from_batch(b)
    ws = torch.empty(h.workspace_size(meta), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(b.q)
    with pytest.raises(B.PodAttnError) as e:
        h.run(b.q, b.k_pool, b.v_pool, b.block_tables, meta, out, ws)
    assert e.value.status == -1
    kn = torch.zeros(spec.total_q, 2, 128, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.PodAttnError) as e:
        h.run_append(b.q, kn, kn, b.k_pool, b.v_pool, b.block_tables, meta, out, ws)
    assert e.value.status == -2
    hb = B.PodAttention(4, 2, 128, "bf16")
    with pytest.raises(B.PodAttnError) as e:
        hb.run_scaled(b.q, b.q, b.q, b.k_scale, b.v_scale, b.block_tables, meta, out, ws)
    assert e.value.status == -1


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_fp8_workload_full_size(cfg):
    """The FP8 variants of the full-size workloads in every mode against the oracle (codes
    decoded from the format's definition, times their page's scale): the first and last row of
    every prefill tile and every 4th decode row (every 16th of the long-context ones), all heads."""
    spec = gen.fp8_spec(cfg)
    _say(f"fp8 cfg{cfg}: generating {spec.num_pages} pages")
    b = gen.make_batch(spec, "cuda")
    outs, tq = {}, None
    for mode in MODES:
        _say(f"fp8 cfg{cfg} mode={mode}")
        out, h, _ = run_library(b, mode=mode)
        outs[mode] = out
        tq = h.stats()["prefill_tile_queries"]
    per_seq = checked_rows(b, tq, 16 if cfg == 5 else 4)
    _say(f"fp8 cfg{cfg}: oracle on {sum(len(r) for _, r in per_seq)} rows")
    rows, want = reference_rows(b, per_seq)
    for mode in MODES:
        check_rows(outs[mode], rows, want, "fp8", f"fp8-cfg{cfg}/{mode}")
    del outs, b
    torch.cuda.empty_cache()
