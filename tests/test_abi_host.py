"""Host-side checks of the C ABI (no GPU): the library loads and exports every declared
function, the planner covers every (query row, head, visible key) exactly once, the
validator rejects bad metadata with the documented status codes, and a host model of the
fused kernel's claim policy terminates with every item claimed once."""
import heapq
from dataclasses import replace

import numpy as np
import pytest
import torch

from hybrid_prefill_decode_paged_amd import binding as B
from hybrid_prefill_decode_paged_amd import inputs as gen


def test_library_exports_every_declared_function():
    lib = B.load()
    names = B.header_functions()
    assert len(names) >= 9, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/pod_attn.h but not exported"


def test_binding_structures_match_the_header_layout(tmp_path):
    """Every ctypes structure of the binding has the size and field offsets that a C compiler
    gives the header's structure (gcc on include/pod_attn.h)."""
    import ctypes
    import os
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    structs = {"pod_attn_config": B.Config, "pod_attn_batch": B.Batch, "pod_attn_stats": B.Stats,
               "pod_attn_signals": B.Signals, "pod_attn_run_diag": B.RunDiag}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "pod_attn.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(B.HEADER))
    subprocess.run(["gcc", "-I", inc, str(src), "-o", str(exe)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        parts = line.split()
        got[tuple(parts[:-1])] = int(parts[-1])
    for cname, cls in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert got[(cname, f)] == getattr(cls, f).offset, (cname, f)


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_create_without_device_reports_no_device():
    with pytest.raises(B.PodAttnError) as e:
        B.PodAttention(4, 4, 64, "fp32")
    assert e.value.status == -5


def _meta(spec):
    bt = gen.block_tables_for(spec)
    qs = np.zeros(spec.num_prefill + 1, np.int32)
    qs[1:] = np.cumsum(spec.prefill_q_len)
    return B.BatchMeta(qs, spec.prefill_ctx_len, spec.decode_ctx_len, bt.shape[1], spec.num_pages)


def _check_coverage(spec, items, G):
    """Every (row, head) covered by exactly one group; the group's key ranges tile [0, kv_len)
    with kv_len = last query position + 1 >= every row's position + 1."""
    Hkv = spec.num_kv_heads
    qs = np.concatenate([[0], np.cumsum(spec.prefill_q_len)]).astype(int)
    P = int(qs[-1])
    covered = np.zeros((P + spec.num_decode, Hkv), dtype=np.int64)
    groups = {}
    for it in items:
        seq, q_row, n_q, q_pos, g, a, z, grp, split, slot, kind = it[:11]
        key = (kind, q_row, g)
        groups.setdefault(key, []).append((split, a, z, n_q, q_pos, grp, slot, seq))
    for (kind, q_row, g), parts in groups.items():
        parts.sort()
        assert len(parts) <= 128, "at most 128 KV splits per group"
        n_q, q_pos, seq = parts[0][3], parts[0][4], parts[0][7]
        assert [p[0] for p in parts] == list(range(len(parts)))
        assert parts[0][1] == 0
        for x, y in zip(parts[:-1], parts[1:]):
            assert x[2] == y[1], "split ranges must be contiguous"
        kv_len = parts[-1][2]
        assert kv_len == q_pos + n_q
        assert all(p[2] > p[1] for p in parts)
        if len(parts) == 1:
            assert parts[0][5] == -1
        else:
            assert len({p[5] for p in parts}) == 1 and parts[0][5] >= 0
        covered[q_row:q_row + n_q, g] += 1
        if q_row < P:                         # a prefill chunk's rows: tile (kind 0) or small-q extend (kind 1)
            i = int(np.searchsorted(qs, q_row, side="right") - 1)
            assert seq == i and q_row + n_q <= qs[i + 1]
            L, ctx = spec.prefill_q_len[i], spec.prefill_ctx_len[i]
            assert q_pos == ctx - L + (q_row - qs[i])
            if kind == 1:
                assert n_q == L and n_q * G <= 16
        else:
            assert kind == 1
            i = q_row - P
            assert seq == spec.num_prefill + i and n_q == 1
            assert kv_len == spec.decode_ctx_len[i]
    assert np.all(covered == 1)
    # partial slots of split groups never overlap
    slots = []
    for it in items:
        if it[7] >= 0:
            ncols = it[2] * G
            slots.append((int(it[9]), int(it[9]) + ncols))
    slots.sort()
    for (a0, a1), (b0, b1) in zip(slots[:-1], slots[1:]):
        assert a1 <= b0


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("mode", ["fused", "separate", "streams"])
def test_plan_covers_every_row_head_key_once(idx, mode):
    spec = gen.config_spec(idx)
    cfg = B.make_config(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.dtype, mode)
    items, st = B.plan_inspect(cfg, _meta(spec), 256, 2)
    assert st["num_prefill_items"] + st["num_decode_items"] == len(items)
    _check_coverage(spec, items, spec.num_q_heads // spec.num_kv_heads)


def _prefill_splits(spec, mode, cus=256):
    cfg = B.make_config(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.dtype, mode)
    items, st = B.plan_inspect(cfg, _meta(spec), cus, 2)
    return st["prefill_max_splits"], st["num_prefill_items"]


def test_prefill_splits_follow_the_decode_share():
    """Tiles beside a longer decode stream (fused and two-stream plans of a batch that is not
    prefill-heavy) are cut into pieces of about the prefill share's keys over the CUs; separate
    plans and prefill-heavy batches keep pieces of at least 4096 keys (at most 8 per tile)."""
    w3, w4, w5 = gen.config_spec(3), gen.config_spec(4), gen.config_spec(5)
    # Llama-3-8B-shaped (decode-heavy): 64 tiles x 8 KV heads, ~15.4K keys each -> ~31K keys a
    # piece over 256 CUs: unsplit; separate: 16384 / 4096 = 4 pieces.
    assert _prefill_splits(w3, "fused") == (1, 512)
    assert _prefill_splits(w3, "streams") == (1, 512)
    assert _prefill_splits(w3, "separate") == (4, 2048)
    # long-context (decode-heavy): 128 tiles of ~32.5K keys -> ~16.3K a piece: 2 pieces
    assert _prefill_splits(w5, "fused") == (2, 256)
    assert _prefill_splits(w5, "separate") == (8, 1024)
    # on fewer CUs a piece is longer: 64 CUs -> ~65K keys a piece, every tile whole
    assert _prefill_splits(w5, "fused", cus=64)[0] == 1
    # Yi-6B-shaped (prefill-heavy by the planner's estimate): the 4096-key floor in every mode
    for mode in ("fused", "streams", "separate"):
        assert _prefill_splits(w4, mode) == (7, 1408)
    # FP8 halves the decode bytes: the Llama-3-8B-shaped batch becomes prefill-heavy
    assert _prefill_splits(gen.fp8_spec(3), "fused") == (4, 2048)
    # no decode work: the floor
    only = gen.custom_spec("bf16", Hq=32, Hkv=8, D=128, prefill=[(2048, 16384)], decode=[])
    assert _prefill_splits(only, "fused")[0] == 4


@pytest.mark.parametrize("G,D,split,cap", [(1, 128, 0, 0), (2, 64, 128, 1), (3, 128, 256, 3),
                                           (8, 64, 512, 0), (16, 128, 0, 2), (1, 64, 128, 128)])
def test_plan_ragged_batches(G, D, split, cap):
    rng = np.random.default_rng(G * 100 + D)
    pre = [(int(L), int(L + o)) for L, o in zip(rng.integers(1, 300, 5), rng.integers(0, 3000, 5))]
    pre.append((0, 17))                       # an empty chunk
    dec = rng.integers(1, 5000, 9).tolist() + [1, 16, 17]
    spec = gen.custom_spec("bf16", Hq=2 * G, Hkv=2, D=D, prefill=pre, decode=dec)
    cfg = B.make_config(2 * G, 2, D, "bf16", decode_split_tokens=split, prefill_split_cap=cap)
    items, st = B.plan_inspect(cfg, _meta(spec), 80, 2)
    _check_coverage(spec, items, G)
    if cap:
        assert st["prefill_max_splits"] <= cap
    if split:
        assert st["decode_split_tokens"] == split


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_decode_split_length_follows_the_share_balance(idx):
    """Fused plans of a batch whose prefill share is about as long as its decode share (the
    Yi-6B-shaped one) cut decode sequences into about one item per workgroup slot; decode-heavy
    batches, and every separate-mode plan, plan about one item per decode wave."""
    spec = gen.config_spec(idx)
    meta = _meta(spec)
    slots = 256 * 2
    tok = sum(spec.decode_ctx_len) * spec.num_kv_heads
    for mode in ("fused", "separate"):
        cfg = B.make_config(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.dtype, mode)
        _, st = B.plan_inspect(cfg, meta, 256, 2)
        per_wave = -(-tok // (slots * 4))
        expect = -(-min(32768, max(256, per_wave)) // 128) * 128
        if mode == "fused" and idx == 4:
            expect = -(-min(32768, max(256, -(-tok // slots))) // 128) * 128
        assert st["decode_split_tokens"] == expect, (idx, mode)
    cfg = B.make_config(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.dtype, "fused")
    _, st = B.plan_inspect(cfg, meta, 256, 2)
    if idx == 4:
        assert st["num_decode_items"] <= 2 * slots
    else:
        assert st["num_decode_items"] >= 4 * slots


def test_decode_items_fill_the_grid_for_every_cache():
    """Decode items hold the same number of tokens for the FP8 and the bf16 cache on the same
    batch, so a batch too small to be capped by its sequences still has about one item per
    decode wave with an FP8 cache (here 32 decodes at 4K: 2048 items on 256 CUs x 2 x 4 waves).
    The prefill-heavy fused plan (here the FP8 Llama-3-8B-shaped batch, whose halved decode
    bytes make it prefill-heavy) stops at 5120-token splits with an FP8 cache (8192 with bf16)."""
    small = gen.custom_spec("bf16", Hq=32, Hkv=8, D=128, prefill=[], decode=[4096] * 32, seed=1)
    for bf, f8 in ((gen.config_spec(2), gen.fp8_spec(2)), (gen.config_spec(5), gen.fp8_spec(5)),
                   (small, replace(small, dtype="fp8"))):
        st = {}
        for spec in (bf, f8):
            for mode in ("fused", "separate"):
                cfg = B.make_config(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.dtype, mode)
                _, s_ = B.plan_inspect(cfg, _meta(spec), 256, 2)
                st[spec.dtype, mode] = (s_["decode_split_tokens"], s_["num_decode_items"])
        assert st["fp8", "fused"] == st["bf16", "fused"] and st["fp8", "separate"] == st["bf16", "separate"], st
    assert st["fp8", "fused"][1] == 2048, st
    spec = gen.fp8_spec(3)
    cfg = B.make_config(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.dtype, "fused")
    items, s_ = B.plan_inspect(cfg, _meta(spec), 256, 2)
    assert s_["decode_split_tokens"] == 5120
    _check_coverage(spec, items, spec.num_q_heads // spec.num_kv_heads)


@pytest.mark.parametrize("idx,tapered", [(2, False), (3, True), (5, False)])
def test_decode_tail_taper(idx, tapered):
    """Decode items are claimed in queue order (longest sequences first).  When sequence lengths
    vary, the pieces claimed last take a quarter of the split length, about two short items per
    wave of the grid; batches of equal sequences keep one split length.  Either way every key of
    every decode piece is covered once."""
    spec = gen.config_spec(idx)
    cfg = B.make_config(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.dtype, "fused")
    items, st = B.plan_inspect(cfg, _meta(spec), 256, 2)
    _check_coverage(spec, items, spec.num_q_heads // spec.num_kv_heads)
    dec = items[items[:, 10] == 1]
    lengths = dec[:, 6] - dec[:, 5]
    target = st["decode_split_tokens"]
    short = dec[(lengths <= target // 4) & (dec[:, 2] == 1)]
    if not tapered:
        assert np.all(lengths <= target) and len(short) == 0
        return
    tail = max(512, target // 4)
    # the short items form the end of the queue, and they hold about two per wave of the grid
    first_short = int(np.flatnonzero((lengths <= tail))[0])
    assert np.all(lengths[first_short:] <= tail)
    assert np.all(lengths[:first_short] > tail)
    waves = 256 * 2 * 4
    assert 1.5 * waves <= len(dec) - first_short <= 3 * waves


@pytest.mark.parametrize("G", [1, 3, 4, 8, 16])
def test_small_chunks_take_the_decode_path(G):
    """Chunks whose rows x G fit one 16-column block (at most 16 rows, the default) become one
    decode-path item group each; longer chunks stay prefill tiles; extend_max_q = -1 keeps every
    chunk on the tile path and extend_max_q = 2 caps the rows."""
    pre = [(1, 9), (2, 300), (5, 40), (16, 16), (17, 900), (3, 3)]
    spec = gen.custom_spec("bf16", Hq=2 * G, Hkv=2, D=128, prefill=pre, decode=[7, 4000])
    qs = np.concatenate([[0], np.cumsum(spec.prefill_q_len)])
    for emax, cap in ((0, 16), (2, 2)):
        items, st = B.plan_inspect(B.make_config(2 * G, 2, 128, extend_max_q=emax), _meta(spec), 80, 2)
        _check_coverage(spec, items, G)
        small = [L <= cap and L * G <= 16 for L, _ in pre]
        assert st["num_small_extends"] == sum(small)
        for i, (L, _) in enumerate(pre):
            rows = items[(items[:, 1] >= qs[i]) & (items[:, 1] < qs[i + 1])]
            assert set(rows[:, 10].tolist()) == ({1} if small[i] else {0})
            if small[i]:
                assert set(rows[:, 2].tolist()) == {L} and set(rows[:, 1].tolist()) == {qs[i]}
    items, st = B.plan_inspect(B.make_config(2 * G, 2, 128, extend_max_q=-1), _meta(spec), 80, 2)
    _check_coverage(spec, items, G)
    assert st["num_small_extends"] == 0
    assert set(items[items[:, 1] < qs[-1]][:, 10].tolist()) == {0}


def test_longest_first_order():
    spec = gen.config_spec(4)
    cfg = B.make_config(32, 4, 128)
    items, _ = B.plan_inspect(cfg, _meta(spec), 256, 2)
    pf = items[items[:, 10] == 0]
    work = [(it[6] - it[5]) for it in pf[:: max(1, 1)]]
    # descriptors are ordered by tile work; the first item belongs to the longest chunk
    assert pf[0][3] + pf[0][2] == max(spec.prefill_ctx_len)
    dc = items[items[:, 10] == 1]
    kv = [int(it[3]) + 1 for it in dc]
    assert kv[0] == max(spec.decode_ctx_len)
    assert len(work) == len(pf)


def _expect(status, **batch_kw):
    cfg_kw = batch_kw.pop("cfg", {})
    base = dict(num_q_heads=4, num_kv_heads=2, head_dim=128, dtype="bf16")
    base.update(cfg_kw)
    cfg = B.make_config(**base)
    m = dict(prefill_q_start=[0, 8], prefill_ctx_len=[20], decode_ctx_len=[5, 33],
             block_table_stride=4, num_pages_in_pool=100)
    m.update(batch_kw)
    meta = B.BatchMeta(**m)
    with pytest.raises(B.PodAttnError) as e:
        B.plan_inspect(cfg, meta, 256, 2)
    assert e.value.status == status, str(e.value)
    assert len(str(e.value)) > len("ERR_INVALID_ARG: ")


def test_validator_rejects_bad_metadata():
    INV, UNS = -1, -2
    _expect(INV, cfg=dict(num_q_heads=6, num_kv_heads=4))          # Hq % Hkv != 0
    _expect(UNS, cfg=dict(head_dim=96))                             # head_dim not 64/128
    _expect(UNS, cfg=dict(num_q_heads=64, num_kv_heads=2))          # group 32 > 16
    _expect(INV, prefill_q_start=[0, 30])                           # q_len > ctx
    _expect(INV, prefill_q_start=[3, 8])                            # q_start[0] != 0
    _expect(INV, decode_ctx_len=[0, 5])                             # decode ctx 0
    _expect(INV, decode_ctx_len=[5, 65])                            # ctx > stride*16
    _expect(INV, block_table_stride=0)
    _expect(INV, num_pages_in_pool=0)
    _expect(INV, cfg=dict(decode_split_tokens=100))                 # not a multiple of 128
    cfg = B.make_config(4, 2, 128)
    cfg.page_size = 32
    with pytest.raises(B.PodAttnError) as e:
        B.plan_inspect(cfg, B.BatchMeta([0], [], [4], 1, 4), 256, 2)
    assert e.value.status == UNS


def test_empty_batch_plans_nothing():
    cfg = B.make_config(4, 2, 128)
    items, st = B.plan_inspect(cfg, B.BatchMeta([0], [], [], 1, 1), 256, 2)
    assert len(items) == 0 and st["num_decode_items"] == 0


# ------------------------------------------------------------------ claim-policy model
def simulate_fused(n_pf, n_dc, pf_time, dc_time, num_cus, wgs, cap, seed=0):
    """Event simulation of the fused kernel's scheduler: each workgroup picks a role (prefill
    only while its CU holds fewer than `cap` prefill-role workgroups, unless decode is drained),
    claims items of that kind until the counter passes the end, then re-picks; returns the
    claim log and the finish time."""
    rng = np.random.default_rng(seed)
    counters = [0, 0]
    n_items = [n_pf, n_dc]
    active = [0] * num_cus
    claimed = [[], []]
    events = []
    state = {}
    t_end = 0.0
    for wg in range(num_cus * wgs):
        cu = wg % num_cus
        state[wg] = dict(cu=cu, pf_open=n_pf > 0, dc_open=n_dc > 0, role=None, counted=False)
        heapq.heappush(events, (rng.uniform(0, 1e-3), wg))
    while events:
        t, wg = heapq.heappop(events)
        s = state[wg]
        t_end = max(t_end, t)
        if s["role"] is not None:
            i = counters[s["role"]]
            counters[s["role"]] += 1
            if i < n_items[s["role"]]:
                claimed[s["role"]].append(i)
                dt = (pf_time if s["role"] == 0 else dc_time) * rng.uniform(0.8, 1.2)
                heapq.heappush(events, (t + dt, wg))
                continue
            if s["role"] == 0:
                s["pf_open"] = False
                if s["counted"]:
                    active[s["cu"]] -= 1
                    s["counted"] = False
            else:
                s["dc_open"] = False
            s["role"] = None
        role = None
        if s["pf_open"] and s["dc_open"]:
            if active[s["cu"]] < cap:
                active[s["cu"]] += 1
                s["counted"] = True
                role = 0
            else:
                role = 1
        elif s["dc_open"]:
            role = 1
        elif s["pf_open"]:
            role = 0
        if role is None:
            continue
        assert not (role == 0 and s["dc_open"] and active[s["cu"]] > cap)
        s["role"] = role
        heapq.heappush(events, (t, wg))
    return claimed, t_end, active


@pytest.mark.parametrize("n_pf,n_dc", [(0, 500), (300, 0), (256, 4096), (2000, 64), (1, 1)])
def test_claim_policy_terminates_and_claims_each_item_once(n_pf, n_dc):
    claimed, t, active = simulate_fused(n_pf, n_dc, 5.0, 1.0, num_cus=64, wgs=2, cap=1)
    assert sorted(claimed[0]) == list(range(n_pf))
    assert sorted(claimed[1]) == list(range(n_dc))
    assert all(a == 0 for a in active)
    assert np.isfinite(t)


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_prefill_queues_hold_whole_key_range_groups(idx):
    """Prefill items are dealt to the 8 per-XCD claim queues in whole groups (same chunk, KV
    head and key range), the queues are contiguous in item order, the tiles of a chunk share
    their split boundaries, and no queue carries much more key work than the average."""
    spec = gen.config_spec(idx)
    cfg = B.make_config(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.dtype)
    items, _ = B.plan_inspect(cfg, _meta(spec), 256, 2)
    pf = items[items[:, 10] == 0]
    q = pf[:, 11]
    assert np.all(np.diff(q) >= 0) and q.min() >= 0 and q.max() < 8
    owner, work = {}, np.zeros(8)
    bounds = {}
    for it in pf:
        seq, n_q, head, a, z, queue = int(it[0]), int(it[2]), int(it[4]), int(it[5]), int(it[6]), int(it[11])
        key = (seq, head, a)
        assert owner.setdefault(key, queue) == queue, "a key-range group spans two queues"
        bounds.setdefault(seq, set()).add(a)
        work[queue] += (z - a) * n_q
    for seq, starts in bounds.items():
        st = sorted(starts)
        if len(st) > 1:
            assert len({y - x for x, y in zip(st[:-1], st[1:])}) == 1, "tiles of a chunk share split boundaries"
    assert work.max() <= 1.35 * work.mean(), work


# ------------------------------------------------------------------ scheduler signals, cost table
@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5, -2, -5])
def test_batch_signals_match_the_algorithmic_work(idx):
    """pod_attn_batch_signals' per-share FLOPs and bytes add up to the whole-batch algorithmic work
    computed independently in bench.py, and its roofline time is that work at MI355X's peaks
    (negative: the workload with an FP8 cache)."""
    import bench
    spec = gen.config_spec(idx) if idx > 0 else gen.fp8_spec(-idx)
    sig = B.batch_signals(B.make_config(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.dtype),
                          _meta(spec), 256, 2)
    w = bench.algorithmic_work(spec)
    assert sig["prefill_bytes"] + sig["decode_bytes"] == w["bytes"]
    assert sig["prefill_flops"] + sig["decode_flops"] == w["flops"]
    peak = bench.PEAK_MFMA["fp32" if spec.dtype == "fp32" else "bf16"]
    roof = max(w["flops"] / peak, w["bytes"] / bench.PEAK_HBM) * 1e6
    assert abs(sig["roofline_us"] - roof) <= 1e-9 * roof
    assert sig["lds_bytes_per_wg"] == 65536 and sig["grid_wgs"] == 512   # FP8 tiles are bf16 in LDS
    assert sig["fallback_reason"] == 0


def test_batch_signals_put_small_extends_in_the_decode_share():
    spec = gen.custom_spec("bf16", Hq=8, Hkv=2, D=128, prefill=[(4, 1000), (300, 300)], decode=[])
    cfg = B.make_config(8, 2, 128)
    sig = B.batch_signals(cfg, _meta(spec), 256, 2)
    assert sig["small_extends"] == 1 and sig["decode_items"] > 0 and sig["prefill_items"] > 0
    elem, kv_tok, qo_row = 2, 2 * 2 * 128 * 2, 2 * 8 * 128 * 2
    assert sig["decode_bytes"] == 1000 * kv_tok + 4 * qo_row + 4 * 63
    assert sig["prefill_bytes"] == 300 * kv_tok + 300 * qo_row + 4 * 19
    assert sig["decode_flops"] == 4 * 128 * 8 * (4 * 996 + 10)
    sig2 = B.batch_signals(B.make_config(8, 2, 128, extend_max_q=-1), _meta(spec), 256, 2)
    assert sig2["small_extends"] == 0 and sig2["fallback_reason"] == 2     # prefill only
    assert sig2["prefill_flops"] == sig["prefill_flops"] + sig["decode_flops"]


def test_cost_table_lookup_rounds_up_to_a_validated_bucket():
    from hybrid_prefill_decode_paged_amd.cost_table import CostTable, Entry
    mk = lambda L, C, n, Dc, us, ok=True: Entry(L, C, n, Dc, us, us, us, us, ok)
    grid = [(L, C, n, Dc) for L in (0, 512, 1024) for C in ((0,) if L == 0 else (4096, 16384))
            for n in (0, 64, 128) for Dc in ((0,) if n == 0 else (4096, 16384)) if L or n]
    us = lambda L, C, n, Dc: 1.0 + L * C / 1e4 + n * Dc / 1e3
    t = CostTable([32, 8, 128], "bf16", [mk(*g, us(*g), ok=(g != (1024, 4096, 64, 4096))) for g in grid])
    assert t.lookup(100, 2000, 10, 3000).key() == (512, 4096, 64, 4096)
    assert t.lookup(512, 4096, 64, 5000).key() == (512, 4096, 64, 16384)
    assert t.lookup(0, 0, 30, 4000).key() == (0, 0, 64, 4096)       # decode-only bucket
    assert t.lookup(600, 9000, 0, 0).key() == (1024, 16384, 0, 0)    # prefill-only bucket
    assert t.lookup(700, 4096, 64, 4096) is None                     # that bucket failed validation
    assert t.lookup(2048, 4096, 1, 1) is None                        # outside the table: admission says no
    assert t.lookup(512, 20000, 0, 0) is None
    t2 = CostTable.from_json(t.to_json())
    assert [e.key() for e in t2.entries] == [e.key() for e in t.entries]
