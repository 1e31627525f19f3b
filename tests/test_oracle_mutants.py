"""Planted mistakes in the oracle, on the CPU: every mutant below replaces one oracle function
with a plausible wrong version, and at least one pin in test_oracle_pins.py must fail while it
is in place.  The mutants cover a dropped term, a wrong sign, a wrong index and a transposed
operand in each step of the definition: scores, causal mask, softmax, output product, GQA head,
paged gather (page, slot, K and V layouts), row positions, append slot, online and split-KV
rescaling, combine weights, bf16 widening and E4M3 decoding.  The oracle's file is never
changed; a mutant lives only inside its test.
"""
import math
from unittest import mock

import numpy as np
import pytest

import test_oracle_pins as pins
from oracle import attention as orc

_attend = orc.attend
_masked = orc.masked_scores
_softmax = orc.softmax_rows
_gather = orc.gather_kv
_rowpos = orc.row_positions
_e4m3 = orc.e4m3_to_f64


def _pin_calls():
    calls = []
    for name in sorted(dir(pins)):
        if not name.startswith("test_"):
            continue
        fn = getattr(pins, name)
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            calls.append((name, fn, {}))
            continue
        assert len(marks) == 1, name
        argname, values = marks[0].args[:2]
        calls.extend((name, fn, {argname: v}) for v in values)
    return calls


def _failing_pins():
    failed = []
    for name, fn, kw in _pin_calls():
        try:
            with np.errstate(all="ignore"):
                fn(**kw)
        except Exception:              # an assertion, or the mutant breaking a later step
            failed.append(name)
    return sorted(set(failed))


# ---------------------------------------------------------------- the mutants
def _causal_strict(qs, pos, K, scale):             # key j visible only when j < pos
    S = (qs @ K.T) * scale
    j = np.arange(K.shape[0])[None, :]
    return np.where(j < pos[:, None], S, -np.inf)


def _causal_one_late(qs, pos, K, scale):           # one future key leaks in
    S = (qs @ K.T) * scale
    j = np.arange(K.shape[0])[None, :]
    return np.where(j <= pos[:, None] + 1, S, -np.inf)


def _no_scale(qs, pos, K, scale):
    return _masked(qs, pos, K, 1.0)


def _softmax_wrong_axis(S):
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    return E / E.sum(axis=0, keepdims=True)


def _softmax_sign(S):
    m = S.max(axis=1, keepdims=True)
    E = np.exp(m - S)
    E = np.where(np.isfinite(S), E, 0.0)
    return E / E.sum(axis=1, keepdims=True)


def _attend_kv_swapped(qs, pos, K, V, scale, return_probs=False):
    return _attend(qs, pos, V, K, scale, return_probs)


def _attend_unnormalised(qs, pos, K, V, scale, return_probs=False):
    S = orc.masked_scores(qs, pos, K, scale)
    E = np.exp(S - S.max(axis=1, keepdims=True))
    out = E @ V
    return (out, E) if return_probs else out


def _gather_variant(k_layout=(0, 2, 1, 3), v_layout=(0, 2, 1), page_shift=0):
    def gather(k_pool, v_pool, table_row, ctx, kv_head, dtype, k_scale=None, v_scale=None):
        n_pages = -(-ctx // orc.PAGE)
        row = np.asarray(table_row, dtype=np.int64)
        pages = row[np.minimum(np.arange(n_pages) + page_shift, len(row) - 1)]
        kp = np.asarray(k_pool[pages])[:, kv_head]
        vp = np.asarray(v_pool[pages])[:, kv_head]
        n, nchunk, _, x = kp.shape
        K = orc.to_f64(kp, dtype).transpose(*k_layout).reshape(n * orc.PAGE, nchunk * x)
        V = orc.to_f64(vp, dtype).transpose(*v_layout).reshape(n * orc.PAGE, nchunk * x)
        if k_scale is not None:
            K = K * np.repeat(np.asarray(k_scale, dtype=np.float64)[pages, kv_head], orc.PAGE)[:, None]
            V = V * np.repeat(np.asarray(v_scale, dtype=np.float64)[pages, kv_head], orc.PAGE)[:, None]
        return K[:ctx], V[:ctx]
    return gather


def _gather_token_slot_off(k_pool, v_pool, table_row, t, kv_head, dtype):
    return _gather_token(k_pool, v_pool, table_row, min(t + 1, t | (orc.PAGE - 1)), kv_head, dtype)


_gather_token = orc.gather_kv_token


def _rowpos_one_late(prefill_q_start, prefill_ctx_len, decode_ctx_len):
    return [(s, p + 1) for s, p in _rowpos(prefill_q_start, prefill_ctx_len, decode_ctx_len)]


def _append_slot_off(k_pool, v_pool, block_tables, rows, k_new, v_new):
    shifted = [(s, p + 1 if (p + 1) % orc.PAGE else p) for s, p in rows]
    Hkv, D = k_new.shape[1], k_new.shape[2]
    x = k_pool.shape[-1]
    for r, (s, pos) in enumerate(shifted):
        page = int(block_tables[s][pos // orc.PAGE])
        slot = pos % orc.PAGE
        for g in range(Hkv):
            for d in range(D):
                k_pool[page, g, d // x, slot, d % x] = k_new[r, g, d]
                v_pool[page, g, d, slot] = v_new[r, g, d]


def _online_rescale_sign(q, pos, K, V, scale):
    m, d, o = -math.inf, 0.0, np.zeros(V.shape[1])
    for j in range(min(pos + 1, K.shape[0])):
        x = scale * float(q @ K[j])
        m_new = max(m, x)
        r = math.exp(m_new - m) if m != -math.inf else 0.0
        e = math.exp(x - m_new)
        d = d * r + e
        o = o * r + e * V[j]
        m = m_new
    return o / d


def _combine_sign(parts):
    lses = np.stack([p[1] for p in parts])
    M = lses.max(axis=0)
    w = np.where(np.isfinite(lses), np.exp(M[None, :] - lses), 0.0)
    num = sum(w[s][:, None] * parts[s][0] for s in range(len(parts)))
    return num / w.sum(axis=0)[:, None]


def _bf16_shift15(bits):
    u = np.asarray(bits).view(np.uint16).astype(np.uint32) << 15
    return u.view(np.float32).astype(np.float64)


def _e4m3_bias8(codes):
    return _e4m3(codes) / 2.0


def _e4m3_subnormal_scale(codes):
    c = np.asarray(codes).astype(np.uint8).astype(np.int64)
    out = _e4m3(codes)
    return np.where(((c >> 3) & 15) == 0, out / 2.0, out)


MUTANTS = {
    "causal mask excludes the diagonal": [("masked_scores", _causal_strict)],
    "causal mask admits the next key": [("masked_scores", _causal_one_late)],
    "softmax scale dropped": [("masked_scores", _no_scale)],
    "softmax normalised over the wrong axis": [("softmax_rows", _softmax_wrong_axis)],
    "softmax exponent sign flipped": [("softmax_rows", _softmax_sign)],
    "K and V swapped in the output product": [("attend", _attend_kv_swapped)],
    "output not divided by the row sum": [("attend", _attend_unnormalised)],
    "K layout transposed (dims and slots)": [("gather_kv", _gather_variant(k_layout=(0, 2, 3, 1)))],
    "V layout transposed (dims and slots)": [("gather_kv", _gather_variant(v_layout=(0, 1, 2)))],
    "block table read one page late": [("gather_kv", _gather_variant(page_shift=1))],
    "token gather one slot late": [("gather_kv_token", _gather_token_slot_off)],
    "row positions one late": [("row_positions", _rowpos_one_late)],
    "append writes the next slot": [("append_tokens", _append_slot_off)],
    "online rescale sign flipped": [("attend_online", _online_rescale_sign)],
    "split combine weight sign flipped": [("combine_partials", _combine_sign)],
    "bf16 widened by 15 bits": [("bf16_bits_to_f64", _bf16_shift15)],
    "E4M3 exponent bias 8": [("e4m3_to_f64", _e4m3_bias8)],
    "E4M3 subnormals at 2^-7": [("e4m3_to_f64", _e4m3_subnormal_scale)],
}


def test_unmutated_oracle_passes_every_pin():
    assert _failing_pins() == []


def test_wrong_gqa_head_is_caught():
    with mock.patch.object(orc.HybridProblem, "kv_head_of", lambda self, h: h % self.Hkv):
        failed = _failing_pins()
    print("GQA head h % Hkv caught by", failed)
    assert failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    patches = [mock.patch.object(orc, attr, fn) for attr, fn in MUTANTS[name]]
    for p in patches:
        p.start()
    try:
        failed = _failing_pins()
    finally:
        for p in patches:
            p.stop()
    print(f"{name}: caught by {failed}")
    assert failed, f"no pin fails with the mutant '{name}'"
