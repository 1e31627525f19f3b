"""Randomized parity sweep: seeded random hybrid batches against the fp64 oracle on the whole
output.  Each case draws a dtype (bf16, fp32, or the FP8 cache with scales that are not powers
of two), head_dim, KV heads, group size, prefill chunks (lengths and offsets around tile, page and split
edges), decode contexts (page edges), a mode, and sometimes forced decode splits or a prefill
split cap; unused cache slots hold NaN.  Fusion must not change the result (POD-Attention
digest, "Virtual CTAs and per-SM balance"), whatever the shape.
"""
import random

import numpy as np
import pytest
import torch

from hybrid_prefill_decode_paged_amd import binding as B
from hybrid_prefill_decode_paged_amd import inputs as gen
from helpers import check_close, problem, run_library, to_f64

pytestmark = pytest.mark.gpu

CASES_PER_CHUNK = 30


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def _draw(rng: random.Random):
    dtype = rng.choice(["bf16", "bf16", "fp8", "fp32"])
    D = rng.choice([64, 128])
    hkv = rng.choice([1, 2, 4])
    G = rng.choice([1, 2, 4, 8, 16])
    npf = rng.randint(0, 3)
    pre = []
    for _ in range(npf):
        L = rng.choice([1, 2, 3, 5, 17, 64, 127, 128, 129, 200, 300])
        off = rng.choice([0, 0, 1, 15, 16, 63, 500, 1000, 3000])
        pre.append((L, L + off))
    ndc = rng.randint(0 if npf else 1, 6)
    dec = [rng.choice([1, 2, 15, 16, 17, 100, 255, 256, 257, 1000, 2047, 5000]) for _ in range(ndc)]
    mode = rng.choice(["fused", "separate", "streams"])
    kw = {}
    if rng.random() < 0.4:
        kw["decode_split_tokens"] = rng.choice([128, 256, 512])
    if rng.random() < 0.4:
        kw["prefill_split_cap"] = rng.choice([1, 2, 4, 16])
    seed = rng.randint(1, 10**6)
    return dtype, D, hkv, hkv * G, pre, dec, mode, kw, seed


@pytest.mark.parametrize("chunk", range(4))
def test_random_batches_match_the_oracle(chunk):
    rng = random.Random(20261203 + chunk)
    for i in range(CASES_PER_CHUNK):
        dtype, D, hkv, hq, pre, dec, mode, kw, seed = _draw(rng)
        what = (f"chunk {chunk} case {i}: {dtype} Hq={hq} Hkv={hkv} D={D} prefill={pre} decode={dec} "
                f"mode={mode} {kw} seed={seed}")
        print(what, flush=True)
        spec = gen.custom_spec(dtype, Hq=hq, Hkv=hkv, D=D, prefill=pre, decode=dec, seed=seed)
        b = gen.make_batch(spec, "cuda")
        gen.poison_unused(b)
        if dtype == "fp8":
            g = np.random.Generator(np.random.PCG64(seed))
            for t in (b.k_scale, b.v_scale):
                t.mul_(torch.from_numpy(g.uniform(0.6, 1.5, size=tuple(t.shape)).astype(np.float32)).to(t.device))
        out, h, _ = run_library(b, mode=mode, **kw)
        torch.cuda.synchronize()
        check_close(to_f64(out), problem(b).full_output(), dtype, what)
        h.close()


@pytest.mark.parametrize("chunk", range(2))
def test_random_appends_match_the_oracle(chunk):
    """The same draw through pod_attn_run_append (bf16 and fp32 caches; writing FP8 is not
    built): the new tokens' K/V land bit-exactly where the oracle's append puts them, no other
    cache byte changes, and the output over the updated cache matches the oracle."""
    from oracle import attention as orc

    def raw(t, dt):
        t = t.cpu()
        return t.view(torch.int16).numpy().copy() if dt == "bf16" else t.numpy().copy()

    rng = random.Random(20261204 + chunk)
    for i in range(CASES_PER_CHUNK):
        dtype, D, hkv, hq, pre, dec, mode, kw, seed = _draw(rng)
        if dtype == "fp8":
            dtype = "bf16"
        what = (f"append chunk {chunk} case {i}: {dtype} Hq={hq} Hkv={hkv} D={D} prefill={pre} "
                f"decode={dec} mode={mode} {kw} seed={seed}")
        print(what, flush=True)
        spec = gen.custom_spec(dtype, Hq=hq, Hkv=hkv, D=D, prefill=pre, decode=dec, seed=seed)
        b = gen.make_batch(spec, "cuda")
        rows = orc.row_positions(b.prefill_q_start, b.prefill_ctx_len, b.decode_ctx_len)
        k_new, v_new = gen.new_tokens(spec, seed + 1, "cuda")
        kr, vr = gen.k_rows_view(b.k_pool), gen.v_rows_view(b.v_pool)
        for s, pos in rows:                      # a slot the append misses shows as NaN
            p = int(b.block_tables_host[s][pos // 16])
            kr[p, :, pos % 16] = float("nan")
            vr[p, :, pos % 16] = float("nan")
        want_k, want_v = raw(b.k_pool, dtype), raw(b.v_pool, dtype)
        orc.append_tokens(want_k, want_v, b.block_tables_host, rows, raw(k_new, dtype), raw(v_new, dtype))
        h = B.PodAttention(hq, hkv, D, dtype, mode, scale=spec.softmax_scale, **kw)
        meta = B.BatchMeta.from_batch(b)
        ws = torch.empty(h.workspace_size(meta), dtype=torch.uint8, device="cuda")
        out = torch.full_like(b.q, float("nan"))
        h.run_append(b.q, k_new, v_new, b.k_pool, b.v_pool, b.block_tables, meta, out, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(raw(b.k_pool, dtype), want_k, err_msg=what)
        np.testing.assert_array_equal(raw(b.v_pool, dtype), want_v, err_msg=what)
        check_close(to_f64(out), problem(b).full_output(), dtype, what)
        h.close()
