"""Pins for the fp64 oracle: each check is fixed by the pages' definitions or by mathematics,
not by re-running the oracle's own formula.  A plausible mistake in the oracle (dropped scale,
off-by-one causal diagonal, wrong GQA head, wrong page slot, transposed operand, wrong sign in
the rescale) fails at least one test here."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as orc
from hybrid_prefill_decode_paged_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.txt")


def _problem(b: gen.HybridBatch) -> orc.HybridProblem:
    s = b.spec
    qraw = b.q.view(torch.int16).numpy() if s.dtype == "bf16" else b.q.numpy()
    kraw = b.k_pool.view(torch.int16).numpy() if s.dtype == "bf16" else b.k_pool.numpy()
    vraw = b.v_pool.view(torch.int16).numpy() if s.dtype == "bf16" else b.v_pool.numpy()
    return orc.HybridProblem(qraw, kraw, vraw, b.block_tables_host, b.prefill_q_start,
                             b.prefill_ctx_len, b.decode_ctx_len, s.num_q_heads,
                             s.num_kv_heads, s.dtype, s.softmax_scale)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ------------------------------------------------------------------ golden, hand-worked
def _golden_cases():
    cases, cur = [], None
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        tok = line.split()
        if tok[0] == "case":
            cur = {"name": tok[1], "k": {}, "v": {}, "checks": []}
        elif tok[0] == "scale":
            cur["scale"] = float(tok[1])
        elif tok[0] == "q":
            cur["q"] = np.array([float(t) for t in tok[1:]])
        elif tok[0] in ("k", "v"):
            cur[tok[0]][int(tok[1])] = np.array([float(t) for t in tok[2:]])
        elif tok[0] == "pos":
            cur["checks"].append((int(tok[1]), np.array([float(t) for t in tok[3:]])))
        elif tok[0] == "end":
            cases.append(cur)
    return cases


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden_hand_worked(case):
    n = len(case["k"])
    K = np.stack([case["k"][j] for j in range(n)])
    V = np.stack([case["v"][j] for j in range(n)])
    for pos, want in case["checks"]:
        got = orc.attend(case["q"][None], np.array([pos]), K, V, case["scale"])[0]
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
        got_on = orc.attend_online(case["q"], pos, K, V, case["scale"])
        np.testing.assert_allclose(got_on, want, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ softmax invariants
def test_softmax_rows_sum_to_one_and_mask_is_exact_zero():
    rng = np.random.default_rng(0)
    for ctx in (1, 2, 15, 16, 17, 33, 70):
        q = _rand(rng, 5, 8)
        K = _rand(rng, ctx, 8) * 3
        V = _rand(rng, ctx, 8)
        pos = np.sort(rng.integers(0, ctx, size=5))
        _, P = orc.attend(q, pos, K, V, 0.7, return_probs=True)
        assert np.all(np.abs(P.sum(axis=1) - 1.0) <= 1e-12)
        for i, p in enumerate(pos):
            assert np.all(P[i, p + 1:] == 0.0)      # keys after the query: weight exactly 0
            assert np.all(P[i, : p + 1] > 0.0)      # itself and earlier keys: all visible
            assert np.count_nonzero(P[i]) == p + 1  # inclusive diagonal


def test_visibility_pattern_of_mixed_batch():
    """The mixed batch of the Week-6 lecture ("한 스텝에 여러 종류의 request 섞기"): two
    decodes, an extend chunk of 8 over an existing prefix, a fresh prefill of 4.  Visible key
    counts per row follow from the extend/decode definitions: decode row -> ctx keys; extend
    row k of a chunk over prefix p -> p + k + 1; prefill row k -> k + 1."""
    rng = np.random.default_rng(1)
    D = 8
    seqs = [("decode", 23, 1), ("decode", 7, 1), ("extend", 5 + 8, 8), ("prefill", 4, 4)]
    want = [23, 7] + [5 + k + 1 for k in range(8)] + [k + 1 for k in range(4)]
    got = []
    for kind, ctx, L in seqs:
        K, V = _rand(rng, ctx, D), _rand(rng, ctx, D)
        pos = np.arange(ctx - L, ctx)
        _, P = orc.attend(_rand(rng, L, D), pos, K, V, 0.3, return_probs=True)
        got += [int(np.count_nonzero(r)) for r in P]
    assert len(got) == 14 and got == want


# ------------------------------------------------------------------ closed forms
@pytest.mark.parametrize("ctx", [1, 5, 16, 17, 40])
def test_closed_form_zero_keys_gives_prefix_mean(ctx):
    rng = np.random.default_rng(ctx)
    D = 6
    V = _rand(rng, ctx, D)
    K = np.zeros((ctx, D))
    q = _rand(rng, ctx, D)
    out = orc.attend(q, np.arange(ctx), K, V, 0.9)
    for i in range(ctx):
        np.testing.assert_allclose(out[i], V[: i + 1].mean(axis=0), rtol=0, atol=1e-13)


def test_closed_form_ramp_values():
    """K = 0 and V_j = j e_1: out_i = (0 + 1 + ... + i)/(i + 1) e_1 = i/2 e_1."""
    ctx, D = 50, 4
    V = np.zeros((ctx, D))
    V[:, 0] = np.arange(ctx)
    out = orc.attend(np.ones((ctx, D)), np.arange(ctx), np.zeros((ctx, D)), V, 1.0)
    np.testing.assert_allclose(out[:, 0], np.arange(ctx) / 2.0, rtol=0, atol=1e-12)
    assert np.all(out[:, 1:] == 0)


def test_closed_form_constant_values_and_single_key():
    rng = np.random.default_rng(2)
    q, K = _rand(rng, 3, 7), _rand(rng, 9, 7) * 4
    c = _rand(rng, 7)
    out = orc.attend(q, np.array([8, 3, 0]), K, np.tile(c, (9, 1)), 0.4)
    np.testing.assert_allclose(out, np.tile(c, (3, 1)), rtol=0, atol=1e-13)
    V = _rand(rng, 1, 7)
    out1 = orc.attend(q, np.array([0, 0, 0]), K[:1], V, 0.4)
    np.testing.assert_array_equal(out1, np.tile(V[0], (3, 1)))


def test_closed_form_dominant_key():
    """One key aligned with the query and scaled up wins: out -> v_j.  Also catches a sign
    error in the scale or in the max subtraction (the softmax would pick the anti-aligned key)."""
    rng = np.random.default_rng(3)
    D, ctx = 16, 30
    q = _rand(rng, D)
    q /= np.linalg.norm(q)
    K = _rand(rng, ctx, D) * 0.1
    V = _rand(rng, ctx, D)
    K[11] = 400.0 * q
    K[12] = -400.0 * q
    out = orc.attend(q[None], np.array([ctx - 1]), K, V, 1.0)[0]
    np.testing.assert_allclose(out, V[11], rtol=0, atol=1e-12)


def test_scale_is_one_over_sqrt_d_by_default():
    """Switching on the scale changes the answer as the closed form predicts: with two keys
    and q.k = (0, a), weights are (1, e^{a s})/(1 + e^{a s}); s = 1/sqrt(D) by default."""
    D = 64
    q = np.zeros(D); q[0] = 1.0
    K = np.zeros((2, D)); K[1, 0] = 8.0
    V = np.array([[1.0] + [0.0] * (D - 1), [0.0, 1.0] + [0.0] * (D - 2)])
    qraw = q.astype(np.float32).reshape(1, 1, D)
    kp = np.zeros((1, 1, D // 4, 16, 4), np.float32)
    vp = np.zeros((1, 1, D, 16), np.float32)
    for t in range(2):
        kp[0, 0, :, t, :] = K[t].reshape(D // 4, 4)
        vp[0, 0, :, t] = V[t]
    prob = orc.HybridProblem(qraw, kp, vp, np.zeros((1, 1), np.int32), [0], [], [2], 1, 1, "fp32")
    out = prob.full_output()[0, 0]
    w1 = math.exp(8.0 / 8.0) / (1 + math.exp(8.0 / 8.0))
    np.testing.assert_allclose(out[:2], [1 - w1, w1], rtol=0, atol=1e-12)


# ------------------------------------------------------------------ online / split == direct
@pytest.mark.parametrize("seed", range(6))
def test_online_blockwise_split_equal_direct(seed):
    rng = np.random.default_rng(100 + seed)
    ctx = int(rng.integers(1, 71))
    D = int(rng.choice([4, 8, 16]))
    n = int(rng.integers(1, min(ctx, 9) + 1))
    pos = np.arange(ctx - n, ctx)
    q, K, V = _rand(rng, n, D), _rand(rng, ctx, D) * 2.5, _rand(rng, ctx, D)
    K[rng.integers(0, ctx)] *= 8.0                      # a row that forces rescaling
    s = 1 / math.sqrt(D)
    ref = orc.attend(q, pos, K, V, s)
    scale_ref = np.maximum(np.abs(ref), 1.0)
    for i in range(n):
        on = orc.attend_online(q[i], int(pos[i]), K, V, s)
        assert np.all(np.abs(on - ref[i]) <= 1e-12 * scale_ref[i])
    for blk in (1, 3, 16, 17, 32):
        bw = orc.attend_blockwise(q, pos, K, V, s, blk)
        assert np.all(np.abs(bw - ref) <= 1e-12 * scale_ref)
    for cuts in ([0, ctx], [0, 16, 32, ctx], [0, 1, ctx], [0, 17, 33, ctx]):
        cuts = sorted(set(min(c, ctx) for c in cuts))
        parts = orc.split_partials(q, pos, K, V, s, cuts)
        cm = orc.combine_partials(parts)
        assert np.all(np.abs(cm - ref) <= 1e-12 * scale_ref)


def test_split_with_empty_ranges_has_zero_weight():
    """A split whose keys all lie after the query (causal) has lse = -inf and weight 0."""
    rng = np.random.default_rng(7)
    ctx, D = 48, 8
    q, K, V = _rand(rng, 2, D), _rand(rng, ctx, D), _rand(rng, ctx, D)
    pos = np.array([5, 20])
    parts = orc.split_partials(q, pos, K, V, 0.5, [0, 16, 32, 48])
    assert parts[1][1][0] == -np.inf and parts[2][1][0] == -np.inf and parts[2][1][1] == -np.inf
    np.testing.assert_allclose(orc.combine_partials(parts), orc.attend(q, pos, K, V, 0.5),
                               rtol=0, atol=1e-12)


# ------------------------------------------------------------------ paging
def _scatter_contiguous(spec, K_seq, V_seq, table):
    """Test-side scatter, written from the ABI header's layout description:
    K element (page, head, token-slot t, d) at [page, head, d // x, t, d % x];
    V element (page, head, t, d) at [page, head, d, t]."""
    x = spec.chunk_elems
    D = spec.head_dim
    P = spec.num_pages
    kp = np.full((P, spec.num_kv_heads, D // x, 16, x), np.nan, dtype=np.float32)
    vp = np.full((P, spec.num_kv_heads, D, 16), np.nan, dtype=np.float32)
    for s, (Ks, Vs) in enumerate(zip(K_seq, V_seq)):
        for g in range(spec.num_kv_heads):
            for t in range(Ks.shape[1]):
                page, slot = table[s][t // 16], t % 16
                for d in range(D):
                    kp[page, g, d // x, slot, d % x] = Ks[g, t, d]
                    vp[page, g, d, slot] = Vs[g, t, d]
    return kp, vp


def test_paged_equals_contiguous_bitwise():
    """The same tokens under a permuted table and under an identity table give bitwise-equal
    oracle outputs; the gather returns exactly the rows that were scattered, for every token."""
    spec = gen.custom_spec("fp32", Hq=4, Hkv=2, D=16, prefill=((5, 21), (3, 3)),
                           decode=(1, 16, 17, 33), seed=5, pool_slack=7)
    rng = np.random.default_rng(5)
    ctx = spec.seq_ctx()
    K_seq = [rng.standard_normal((2, c, 16)).astype(np.float32) for c in ctx]
    V_seq = [rng.standard_normal((2, c, 16)).astype(np.float32) for c in ctx]
    q = rng.standard_normal((spec.total_q, 4, 16)).astype(np.float32)
    outs = []
    for ident in (False, True):
        sp = gen.replace(spec, identity_pages=ident)
        bt = gen.block_tables_for(sp)
        kp, vp = _scatter_contiguous(sp, K_seq, V_seq, bt)
        for s, c in enumerate(ctx):
            for g in range(2):
                Kg, Vg = orc.gather_kv(kp, vp, bt[s], c, g, "fp32")
                np.testing.assert_array_equal(Kg, K_seq[s][g].astype(np.float64))
                np.testing.assert_array_equal(Vg, V_seq[s][g].astype(np.float64))
                for t in (0, c - 1, c // 2):
                    kt, vt = orc.gather_kv_token(kp, vp, bt[s], t, g, "fp32")
                    np.testing.assert_array_equal(kt, Kg[t])
                    np.testing.assert_array_equal(vt, Vg[t])
        q_start = np.array([0, 5, 8], np.int32)
        prob = orc.HybridProblem(q, kp, vp, bt, q_start, spec.prefill_ctx_len,
                                 spec.decode_ctx_len, 4, 2, "fp32")
        outs.append(prob.full_output())
    assert not np.isnan(outs[0]).any()
    np.testing.assert_array_equal(outs[0], outs[1])


# ------------------------------------------------------------------ KV append
def test_row_positions_follow_the_mixed_batch_rows():
    """Chunks (L=3, ctx=10), (L=0, ctx=4), (L=2, ctx=2) and decodes at ctx 5 and 1: rows are the
    chunks' last L positions in order, then one row per decode at ctx-1."""
    rows = orc.row_positions([0, 3, 3, 5], [10, 4, 2], [5, 1])
    assert rows == [(0, 7), (0, 8), (0, 9), (2, 0), (2, 1), (3, 4), (4, 0)]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_append_writes_exactly_the_new_rows(dtype):
    """The cache holds every sequence's tokens before this step's rows; appending the rows'
    new K/V gives, bitwise, the pools that the test-side scatter (written from the header's
    layout text) produces for the whole sequences, including the untouched NaN slots, and the
    gather at each row's position returns that row's new K/V."""
    spec = gen.custom_spec("fp32", Hq=4, Hkv=2, D=16, prefill=((5, 21), (3, 3), (0, 7)),
                           decode=(1, 16, 17, 33), seed=15, pool_slack=6)
    rng = np.random.default_rng(15)
    ctx = spec.seq_ctx()
    bt = gen.block_tables_for(spec)
    K_seq = [rng.standard_normal((2, c, 16)).astype(np.float32) for c in ctx]
    V_seq = [rng.standard_normal((2, c, 16)).astype(np.float32) for c in ctx]
    q_start = np.concatenate([[0], np.cumsum(spec.prefill_q_len)]).astype(np.int32)
    rows = orc.row_positions(q_start, spec.prefill_ctx_len, spec.decode_ctx_len)
    new_pos = {(s, pos) for s, pos in rows}
    old_K = [K.copy() for K in K_seq]
    old_V = [V.copy() for V in V_seq]
    for s, c in enumerate(ctx):                  # the cache before the step: new positions absent
        for t in range(c):
            if (s, t) in new_pos:
                old_K[s][:, t] = np.nan
                old_V[s][:, t] = np.nan
    want_k, want_v = _scatter_contiguous(spec, K_seq, V_seq, bt)
    kp, vp = _scatter_contiguous(spec, old_K, old_V, bt)
    k_new = np.stack([K_seq[s][:, pos] for s, pos in rows])
    v_new = np.stack([V_seq[s][:, pos] for s, pos in rows])
    if dtype == "bf16":                          # raw 16-bit patterns: the append moves bits
        to16 = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)
        want_k, want_v, kp, vp = map(to16, (want_k, want_v, kp, vp))
        k_new, v_new = to16(k_new), to16(v_new)
    orc.append_tokens(kp, vp, bt, rows, k_new, v_new)
    np.testing.assert_array_equal(kp, want_k)
    np.testing.assert_array_equal(vp, want_v)
    for r, (s, pos) in enumerate(rows):
        for g in range(2):
            kt, vt = orc.gather_kv_token(kp, vp, bt[s], pos, g, dtype)
            np.testing.assert_array_equal(kt, orc.to_f64(k_new[r, g], dtype))
            np.testing.assert_array_equal(vt, orc.to_f64(v_new[r, g], dtype))


def test_bf16_decoding_matches_torch():
    x = torch.randn(4096, dtype=torch.float32).to(torch.bfloat16)
    x[:4] = torch.tensor([0.0, -0.0, float("inf"), 1e-40]).to(torch.bfloat16)
    ref = x.to(torch.float64).numpy()
    got = orc.bf16_bits_to_f64(x.view(torch.int16).numpy())
    np.testing.assert_array_equal(got, ref)


# ------------------------------------------------------------------ causal / unused slots
def test_future_keys_and_unused_slots_do_not_matter():
    spec = gen.custom_spec("fp32", Hq=2, Hkv=1, D=16, prefill=((6, 29),), decode=(18,), seed=9)
    b = gen.make_batch(spec)
    p0 = _problem(b)
    ref = p0.full_output()
    gen.poison_unused(b, float("nan"))
    p1 = _problem(b)
    np.testing.assert_array_equal(p1.full_output(), ref)
    # overwrite the last key of the prefill sequence (after every query but the last)
    kr = gen.k_rows_view(b.k_pool)
    page = int(b.block_tables_host[0, 28 // 16])
    kr[page, 0, 28 % 16] = 1e6
    p2 = _problem(b)
    out2 = p2.full_output()
    np.testing.assert_array_equal(out2[:5], ref[:5])        # positions 23..27 do not see key 28
    assert not np.array_equal(out2[5], ref[5])              # position 28 does


# ------------------------------------------------------------------ library cross-check
def _sdpa_reference(prob: orc.HybridProblem):
    """torch CPU float64 SDPA with an explicit boolean mask and K/V heads expanded by
    repeat_interleave(G): a library routine independent of the oracle's code."""
    outs = {}
    n_seq = prob.n_pre + len(prob.d_ctx)
    for s in range(n_seq):
        rows = prob.seq_rows(s)
        _, _, ctx = prob.row_info(int(rows[0]))
        pos = torch.tensor([prob.row_info(int(r))[1] for r in rows])
        Ks, Vs = [], []
        for g in range(prob.Hkv):
            K, V = prob.kv(s, g, ctx)
            Ks.append(torch.from_numpy(K)); Vs.append(torch.from_numpy(V))
        K = torch.stack(Ks).repeat_interleave(prob.G, dim=0)       # [Hq, ctx, D]
        V = torch.stack(Vs).repeat_interleave(prob.G, dim=0)
        Q = torch.from_numpy(np.stack([prob.q_f64(rows, h) for h in range(prob.Hq)]))
        mask = torch.arange(ctx)[None, :] <= pos[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(
            Q, K, V, attn_mask=mask, scale=prob.scale)
        outs[s] = o.permute(1, 0, 2).numpy()
    return outs


@pytest.mark.parametrize("which", ["cfg1", "cfg2-reduced", "cfg3-reduced", "cfg4-reduced"])
def test_cross_check_against_torch_sdpa(which):
    if which == "cfg1":
        spec = gen.config_spec(1)
    elif which == "cfg2-reduced":
        spec = gen.reduced_spec(2, n_decode=3, ctx_div=16)
    elif which == "cfg3-reduced":
        spec = gen.reduced_spec(3, n_decode=3, ctx_div=64)
    else:
        spec = gen.reduced_spec(4, n_decode=3, ctx_div=32)
    b = gen.make_batch(spec)
    prob = _problem(b)
    sd = _sdpa_reference(prob)
    for s, o in sd.items():
        rows = prob.seq_rows(s)
        mine = prob.sequence_output(s)
        np.testing.assert_allclose(mine, o, rtol=1e-10, atol=1e-12)
    # the one-row-at-a-time sampled path agrees with the per-sequence path (BLAS may sum
    # a single row in another order, hence 1e-13 rather than bitwise)
    pairs = [(0, 0), (prob.n_pre_rows - 1, prob.Hq - 1), (prob.n_pre_rows, 1)]
    got = prob.sampled_output(pairs)
    full = prob.full_output()
    for i, (r, h) in enumerate(pairs):
        np.testing.assert_allclose(got[i], full[r, h], rtol=0, atol=1e-13)


def test_gqa_mapping_is_contiguous_groups():
    """With Hq = 4, Hkv = 2: heads 0,1 read KV head 0 and heads 2,3 read KV head 1.  Setting
    KV head 1's values to a constant makes heads 2,3 output exactly that constant."""
    spec = gen.custom_spec("fp32", Hq=4, Hkv=2, D=16, prefill=((4, 20),), decode=(9,), seed=4)
    b = gen.make_batch(spec)
    b.v_pool[:, 1] = 0.25
    out = _problem(b).full_output()
    np.testing.assert_allclose(out[:, 2:], 0.25, rtol=0, atol=1e-15)
    assert np.abs(out[:, :2] - 0.25).max() > 0.1


# ------------------------------------------------------------------ FP8 (E4M3) cache
def test_e4m3_decodes_every_code():
    """All 256 codes against torch's float8_e4m3fn widening (a library routine for the same OCP
    format), plus values fixed by the format: 1.0, the largest finite value 448, the smallest
    normal 2^-6 and subnormal 2^-9, signed zero, and NaN at S.1111.111."""
    codes = np.arange(256, dtype=np.uint8)
    got = orc.e4m3_to_f64(codes)
    want = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok], want[ok])
    assert np.isnan(got).sum() == 2 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert got[0x38] == 1.0 and got[0xB8] == -1.0 and got[0x7E] == 448.0
    assert got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9 and got[0x07] == 7 * 2.0 ** -9
    assert got[0x00] == 0.0 and np.signbit(got[0x80]) and got[0x3C] == 1.5


def _fp8_paged(rng, Hkv, D, ctx, n_pages, perm):
    """Random E4M3 codes for one sequence's K and V ([Hkv, ctx, D], codes 0..0x7E and their
    negatives, no NaN) scattered by the header's layout (x = 16), and per-(page, head) scales."""
    mag = rng.integers(0, 0x7F, size=(2, Hkv, ctx, D)).astype(np.uint8)
    sgn = (rng.integers(0, 2, size=mag.shape) << 7).astype(np.uint8)
    codes = mag | sgn
    kp = np.zeros((n_pages, Hkv, D // 16, 16, 16), np.uint8)
    vp = np.zeros((n_pages, Hkv, D, 16), np.uint8)
    for g in range(Hkv):
        for t in range(ctx):
            page, slot = perm[t // 16], t % 16
            for d in range(D):
                kp[page, g, d // 16, slot, d % 16] = codes[0, g, t, d]
                vp[page, g, d, slot] = codes[1, g, t, d]
    ks = np.exp2(rng.integers(-4, 3, size=(n_pages, Hkv))).astype(np.float32)
    vs = np.exp2(rng.integers(-4, 3, size=(n_pages, Hkv))).astype(np.float32) * 0.75
    return codes, kp, vp, ks, vs


def test_fp8_scaled_gather_equals_decoded_rows_times_page_scale():
    rng = np.random.default_rng(31)
    Hkv, D, ctx, P = 2, 32, 45, 7
    perm = rng.permutation(P)
    codes, kp, vp, ks, vs = _fp8_paged(rng, Hkv, D, ctx, P, perm)
    for g in range(Hkv):
        K, V = orc.gather_kv(kp, vp, perm, ctx, g, "fp8", ks, vs)
        for t in range(ctx):
            page = perm[t // 16]
            np.testing.assert_array_equal(K[t], orc.e4m3_to_f64(codes[0, g, t]) * float(ks[page, g]))
            np.testing.assert_array_equal(V[t], orc.e4m3_to_f64(codes[1, g, t]) * float(vs[page, g]))
        k1, v1 = orc.gather_kv_token(kp, vp, perm, ctx - 1, g, "fp8")     # unscaled brute force
        np.testing.assert_array_equal(k1, orc.e4m3_to_f64(codes[0, g, ctx - 1]))
        np.testing.assert_array_equal(v1, orc.e4m3_to_f64(codes[1, g, ctx - 1]))


def test_fp8_scales_act_on_scores_and_on_values():
    """A K scale c applied to every page is the softmax scale times c; a V scale c applied to
    every page multiplies the output by c."""
    rng = np.random.default_rng(32)
    Hkv, D, ctx, P = 1, 32, 40, 3
    perm = np.arange(P)
    codes, kp, vp, _, _ = _fp8_paged(rng, Hkv, D, ctx, P, perm)
    q = rng.standard_normal((2, 2, D)).astype(np.float32)
    one = np.ones((P, Hkv), np.float32)
    mk = lambda ks, vs, sc: orc.HybridProblem(q, kp, vp, perm[None, :], [0, 2], [ctx], [], 2, 1, "fp32",
                                              sc, kv_dtype="fp8", k_scale=ks, v_scale=vs).full_output()
    base = mk(one, one, 0.125)
    np.testing.assert_allclose(mk(one * 4.0, one, 0.125), mk(one, one, 0.5), rtol=1e-12, atol=0)
    np.testing.assert_allclose(mk(one, one * 0.375, 0.125), base * 0.375, rtol=1e-12, atol=0)
    # and a mixed-scale cache equals attention over the decoded, scaled rows
    ks = np.array([[0.5], [2.0], [0.25]], np.float32)
    vs = np.array([[4.0], [1.0], [0.125]], np.float32)
    K = orc.e4m3_to_f64(codes[0, 0]) * np.repeat(ks[:, 0], 16)[:ctx, None]
    V = orc.e4m3_to_f64(codes[1, 0]) * np.repeat(vs[:, 0], 16)[:ctx, None]
    want = orc.attend(q[:, 0].astype(np.float64), np.array([ctx - 2, ctx - 1]), K, V, 0.125)
    np.testing.assert_allclose(mk(ks, vs, 0.125)[:, 0], want, rtol=1e-12, atol=1e-15)
