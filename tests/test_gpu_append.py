"""GPU parity of the KV append (pod_attn_run_append): the new tokens' K/V land bit-exactly in the
slots the oracle's append writes, no other cache byte changes, and the attention output over
the updated cache matches the oracle, in every launch mode."""
import sys

import numpy as np
import pytest
import torch

from hybrid_prefill_decode_paged_amd import binding as B
from hybrid_prefill_decode_paged_amd import inputs as gen
from oracle import attention as orc

from helpers import check_close, check_rows, checked_rows, problem, reference_rows, to_f64

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


def _raw(t: torch.Tensor, dtype: str) -> np.ndarray:
    t = t.cpu()
    return t.view(torch.int16).numpy().copy() if dtype == "bf16" else t.numpy().copy()


def _rows(b):
    return orc.row_positions(b.prefill_q_start, b.prefill_ctx_len, b.decode_ctx_len)


def _poison_new_slots(b, rows, value=float("nan")):
    """Overwrite the slots the append must fill, so that a slot it misses shows."""
    kr, vr = gen.k_rows_view(b.k_pool), gen.v_rows_view(b.v_pool)
    for s, pos in rows:
        p = int(b.block_tables_host[s][pos // 16])
        kr[p, :, pos % 16] = value
        vr[p, :, pos % 16] = value


def _run_append(b, k_new, v_new, mode, **kw):
    s = b.spec
    h = B.PodAttention(s.num_q_heads, s.num_kv_heads, s.head_dim, s.dtype, mode, scale=s.softmax_scale, **kw)
    meta = B.BatchMeta.from_batch(b)
    ws = torch.empty(h.workspace_size(meta), dtype=torch.uint8, device="cuda")
    out = torch.full_like(b.q, float("nan"))
    h.run_append(b.q, k_new, v_new, b.k_pool, b.v_pool, b.block_tables, meta, out, ws)
    torch.cuda.synchronize()
    return out, h, ws


APPEND_CASES = [
    # (dtype, Hq, Hkv, D, prefill (q_len, ctx) pairs, decode ctx list): chunks starting and
    # ending inside pages, a chunk of one page exactly, decodes at slot 0, 15 and inside a page
    ("bf16", 8, 2, 128, [(37, 301), (16, 32), (1, 1)], [1, 16, 17, 33, 600]),
    ("bf16", 16, 4, 64, [(100, 1000)], [15, 2000, 64]),
    ("fp32", 8, 4, 128, [(50, 130)], [300, 1, 17]),
    ("fp32", 4, 1, 64, [(21, 21), (0, 9)], [77, 1025]),
    ("bf16", 32, 32, 128, [(40, 97)], [5, 48]),
    ("bf16", 4, 2, 128, [], [4096, 1000, 3]),
]


@pytest.mark.parametrize("case", range(len(APPEND_CASES)))
@pytest.mark.parametrize("mode", MODES)
def test_append_then_attend(case, mode):
    dt, hq, hkv, d, pre, dec = APPEND_CASES[case]
    spec = gen.custom_spec(dt, Hq=hq, Hkv=hkv, D=d, prefill=pre, decode=dec, seed=200 + case)
    b = gen.make_batch(spec, "cuda")
    rows = _rows(b)
    k_new, v_new = gen.new_tokens(spec, 300 + case, "cuda")
    _poison_new_slots(b, rows)
    want_k, want_v = _raw(b.k_pool, dt), _raw(b.v_pool, dt)
    orc.append_tokens(want_k, want_v, b.block_tables_host, rows, _raw(k_new, dt), _raw(v_new, dt))
    _say(f"append case={case} mode={mode} rows={len(rows)}")
    out, h, _ = _run_append(b, k_new, v_new, mode)
    np.testing.assert_array_equal(_raw(b.k_pool, dt), want_k)
    np.testing.assert_array_equal(_raw(b.v_pool, dt), want_v)
    assert h.stats()["num_append_units"] > 0
    check_close(to_f64(out), problem(b).full_output(), dt, f"append{case}/{mode}")


@pytest.mark.parametrize("mode", MODES)
def test_append_with_forced_splits(mode):
    """Many split items per sequence wait on the same append units (fused mode)."""
    spec = gen.custom_spec("bf16", Hq=8, Hkv=2, D=128, prefill=[(150, 1500), (64, 64)],
                           decode=[1, 129, 700, 3000], seed=17)
    b = gen.make_batch(spec, "cuda")
    rows = _rows(b)
    k_new, v_new = gen.new_tokens(spec, 18, "cuda")
    _poison_new_slots(b, rows)
    want_k, want_v = _raw(b.k_pool, "bf16"), _raw(b.v_pool, "bf16")
    orc.append_tokens(want_k, want_v, b.block_tables_host, rows, _raw(k_new, "bf16"), _raw(v_new, "bf16"))
    _say(f"append forced splits mode={mode}")
    out, h, _ = _run_append(b, k_new, v_new, mode, decode_split_tokens=128, prefill_split_cap=16)
    assert h.stats()["decode_max_splits"] > 1
    np.testing.assert_array_equal(_raw(b.k_pool, "bf16"), want_k)
    np.testing.assert_array_equal(_raw(b.v_pool, "bf16"), want_v)
    check_close(to_f64(out), problem(b).full_output(), "bf16", f"append-splits/{mode}")


def _pool_rows(b, rows):
    """The cache's current K/V at the rows' positions, [rows, Hkv, D] (device)."""
    kr, vr = gen.k_rows_view(b.k_pool), gen.v_rows_view(b.v_pool)
    pages = torch.tensor([int(b.block_tables_host[s][p // 16]) for s, p in rows], device="cuda")
    slots = torch.tensor([p % 16 for _, p in rows], device="cuda")
    k = kr[pages, :, slots].reshape(len(rows), b.spec.num_kv_heads, -1).contiguous()
    v = vr[pages, :, slots].contiguous()
    return k, v


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_append_full_size(cfg):
    """Full-size workloads, fused mode as the bench times it: appending each row's own cached
    token changes no output bit relative to pod_attn_run; then fresh tokens are appended, the
    new slots are checked bitwise, and the first and last row of every prefill tile and every
    8th decode row (all heads) against the oracle on the updated cache."""
    spec = gen.config_spec(cfg)
    b = gen.make_batch(spec, "cuda")
    rows = _rows(b)
    s = spec
    h = B.PodAttention(s.num_q_heads, s.num_kv_heads, s.head_dim, s.dtype, "fused", scale=s.softmax_scale)
    meta = B.BatchMeta.from_batch(b)
    ws = torch.empty(h.workspace_size(meta), dtype=torch.uint8, device="cuda")
    _say(f"append full size cfg={cfg}: same tokens")
    ref = torch.full_like(b.q, float("nan"))
    h.run(b.q, b.k_pool, b.v_pool, b.block_tables, meta, ref, ws)
    k_same, v_same = _pool_rows(b, rows)
    out = torch.full_like(b.q, float("nan"))
    h.run_append(b.q, k_same, v_same, b.k_pool, b.v_pool, b.block_tables, meta, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    _say(f"append full size cfg={cfg}: new tokens")
    k_new, v_new = gen.new_tokens(spec, 1000 + cfg, "cuda")
    h.run_append(b.q, k_new, v_new, b.k_pool, b.v_pool, b.block_tables, meta, out, ws)
    torch.cuda.synchronize()
    k_got, v_got = _pool_rows(b, rows)
    assert torch.equal(k_got.view(torch.int16), k_new.view(torch.int16))
    assert torch.equal(v_got.view(torch.int16), v_new.view(torch.int16))
    per_seq = checked_rows(b, h.stats()["prefill_tile_queries"], 8)
    _say(f"append full size cfg={cfg}: oracle on {sum(len(r) for _, r in per_seq)} rows")
    rr, want = reference_rows(b, per_seq)
    check_rows(out, rr, want, "bf16", f"append-full{cfg}")


def test_append_bad_page_is_reported_not_written():
    spec = gen.custom_spec("bf16", Hq=4, Hkv=2, D=128, prefill=[(20, 40)], decode=[33], seed=23)
    b = gen.make_batch(spec, "cuda")
    bt = b.block_tables_host.copy()
    bt[1, 2] = spec.num_pages + 5                       # the decode's last page: outside the pool
    b.block_tables_host = bt
    b.block_tables = torch.from_numpy(bt).cuda()
    k_before, v_before = _raw(b.k_pool, "bf16"), _raw(b.v_pool, "bf16")
    k_new, v_new = gen.new_tokens(spec, 24, "cuda")
    for mode in MODES:
        _say(f"append bad page mode={mode}")
        _, h, ws = _run_append(b, k_new, v_new, mode)
        status, _, _ = h.read_device_status(ws)
        assert status & B.DEVICE_ERR_BAD_PAGE
    # the prefill rows were written; the decode row's slot lies in no page of the pool
    rows = _rows(b)
    want_k, want_v = k_before, v_before
    orc.append_tokens(want_k, want_v, bt, rows[:-1], _raw(k_new, "bf16")[:-1], _raw(v_new, "bf16")[:-1])
    np.testing.assert_array_equal(_raw(b.k_pool, "bf16"), want_k)
    np.testing.assert_array_equal(_raw(b.v_pool, "bf16"), want_v)
