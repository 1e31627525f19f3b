"""Seeded fuzzing of the host planner and validator through pod_attn_plan_inspect (no GPU).

Valid batches: random heads, head_dim, cache dtype, mode, CU count and workgroups per CU, split
knobs, prefill chunks (lengths and offsets on tile, page and split edges, small-q extends,
empty chunks) and decode contexts; every plan must cover each (row, KV head, key) exactly once,
with contiguous split ranges and non-overlapping partial slots (the same checker as the
workload plans).

Invalid batches: one field of a valid batch or config broken at a time (negative or zero
lengths, a chunk longer than its context, unordered row starts, contexts beyond the block
table, an empty pool, bad head counts, head_dim or split knobs); each must come back as an
error status with a message, never as a plan or a crash.
"""
import random
from types import SimpleNamespace

import numpy as np
import pytest

from hybrid_prefill_decode_paged_amd import binding as B
from test_abi_host import _check_coverage

INV, UNS = -1, -2


def _valid(rng: random.Random):
    hkv = rng.choice([1, 2, 4, 8])
    G = rng.choice([1, 2, 3, 4, 8, 16])
    D = rng.choice([64, 128])
    dtype = rng.choice(["bf16", "fp32", "fp8"])
    mode = rng.choice(["fused", "separate", "streams"])
    pq, pc = [], []
    for _ in range(rng.randint(0, 4)):
        L = rng.choice([0, 1, 2, 3, 4, 15, 16, 17, 127, 128, 129, 512, 1000])
        off = rng.choice([0, 1, 15, 16, 4095, 4096, 4097, 20000, 40000])
        pq.append(L)
        pc.append(L + off)
    dc = [rng.choice([1, 2, 15, 16, 17, 4096, 4097, 8191, 8192, 32768, 70000])
          for _ in range(rng.randint(0 if pq else 1, 40))]
    ctxs = pc + dc
    stride = max(1, max(-(-c // 16) for c in ctxs) if ctxs else 1) + rng.choice([0, 0, 3])
    cfg_kw = dict(decode_split_tokens=rng.choice([0, 0, 128, 640, 8192]),
                  prefill_split_cap=rng.choice([0, 0, 1, 3, 16, 128]),
                  extend_max_q=rng.choice([0, 0, -1, 1, 16]))
    num_cus = rng.choice([1, 7, 64, 256, 304])
    wgs = rng.choice([1, 2, 3, 4])
    return hkv, G, D, dtype, mode, pq, pc, dc, stride, cfg_kw, num_cus, wgs


def _meta(pq, pc, dc, stride, pages=1 << 20):
    qs = np.concatenate([[0], np.cumsum(pq)]).astype(np.int32)
    return B.BatchMeta(qs, np.asarray(pc, np.int32), np.asarray(dc, np.int32), stride, pages)


@pytest.mark.parametrize("chunk", range(4))
def test_random_valid_plans_cover_everything_once(chunk):
    rng = random.Random(31000 + chunk)
    for i in range(100):
        hkv, G, D, dtype, mode, pq, pc, dc, stride, cfg_kw, num_cus, wgs = _valid(rng)
        cfg = B.make_config(hkv * G, hkv, D, dtype, mode, **cfg_kw)
        items, st = B.plan_inspect(cfg, _meta(pq, pc, dc, stride), num_cus, wgs)
        spec = SimpleNamespace(num_kv_heads=hkv, prefill_q_len=pq, prefill_ctx_len=pc,
                               num_prefill=len(pq), num_decode=len(dc), decode_ctx_len=dc)
        try:
            _check_coverage(spec, items, G)
        except AssertionError as e:
            raise AssertionError(f"case {chunk}/{i}: Hkv={hkv} G={G} D={D} {dtype} {mode} {cfg_kw} "
                                 f"cus={num_cus}x{wgs} prefill={list(zip(pq, pc))} decode={dc}: {e}")
        assert st["num_prefill_items"] + st["num_decode_items"] == len(items)


def _broken(rng: random.Random):
    """A valid small batch with exactly one thing broken, and the status it must produce."""
    pq, pc, dc, stride, pages = [8, 3], [20, 3], [5, 33], 4, 100
    hq, hkv, D, cfg_kw = 4, 2, 128, {}
    kind = rng.randrange(14)
    if kind == 0:
        pc = [5, 3]                                    # a chunk longer than its context
    elif kind == 1:
        dc = [0, 5]                                    # decode context 0
    elif kind == 2:
        dc = [5, -7]                                   # negative context
    elif kind == 3:
        pq = [-2, 3]                                   # negative chunk length
    elif kind == 4:
        dc = [5, 16 * stride + 1]                      # beyond the block table row
    elif kind == 5:
        pc = [20, 16 * stride + 4]
        pq = [8, 4]
    elif kind == 6:
        stride = 0
    elif kind == 7:
        pages = 0
    elif kind == 8:
        hq, hkv = 6, 4                                 # Hq % Hkv != 0
    elif kind == 9:
        D = rng.choice([0, 32, 96, 256])               # unsupported head_dim
        return pq, pc, dc, stride, pages, hq, hkv, D, cfg_kw, UNS
    elif kind == 10:
        hq, hkv = 64, 2                                # group 32 > 16
        return pq, pc, dc, stride, pages, hq, hkv, D, cfg_kw, UNS
    elif kind == 11:
        cfg_kw = dict(decode_split_tokens=rng.choice([1, 100, 127, -128]))
    elif kind == 12:
        cfg_kw = dict(prefill_split_cap=-1)
    else:
        hkv = 0
    return pq, pc, dc, stride, pages, hq, hkv, D, cfg_kw, INV


def test_random_broken_batches_are_rejected():
    rng = random.Random(32000)
    for i in range(300):
        pq, pc, dc, stride, pages, hq, hkv, D, cfg_kw, want = _broken(rng)
        qs = np.concatenate([[0], np.cumsum(pq)]).astype(np.int32)
        meta = B.BatchMeta(qs, np.asarray(pc, np.int32), np.asarray(dc, np.int32), stride, pages)
        cfg = B.make_config(hq, hkv, D, rng.choice(["bf16", "fp32", "fp8"]), rng.choice(["fused", "separate"]),
                            **cfg_kw)
        with pytest.raises(B.PodAttnError) as e:
            B.plan_inspect(cfg, meta, 256, 2)
        assert e.value.status in (INV, UNS), (i, e.value.status, str(e.value))
        if want == UNS:
            assert e.value.status == UNS, (i, str(e.value))
        assert len(str(e.value)) > len("ERR_INVALID_ARG: "), i
