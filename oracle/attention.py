"""Plain CPU oracle for hybrid-batch (chunked prefill + decode) paged attention, in float64.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline
leg import this module.  The library (hybrid_prefill_decode_paged_amd and its native code)
never imports or calls it, and it imports nothing from the library.

Sources (web pages; section names as printed on them):
  [W6]  "Week 6: Beyond PyTorch: Custom Kernel과 vLLM" (PyTorch KR core-SIG lecture)
  [W4]  "LLMSO - W4 - Optimization & Frameworks" (seojhoon.tistory.com)
  [POD] Silicon & Systems digest "POD-Attention hybrid batching"

What is computed (the plain definition; fusion does not change the mathematics -- [POD],
section "Virtual CTAs and per-SM balance"):
  * attention(Q,K,V) = softmax(Q K^T * scale) V        -- [W6] "Attention에 적용하기", the
    Attention(Q,K,V) equation; scale = 1/sqrt(d_k) unless given.
  * causal: a token attends to itself and earlier tokens -- [W6] "Non-Causal vs. Causal
    Attention".  Positions are absolute: a prefill (extend) chunk of L tokens whose context is
    ctx holds positions ctx-L .. ctx-1 and attends to the cached prefix plus the earlier tokens
    of its own chunk; a decode token is an extend of one token, at position ctx-1 -- [W6]
    "한 스텝에 여러 종류의 request 섞기".  The chunk's own K/V are already in the cache, which
    is append-only -- [W6] "KV Cache".
  * safe softmax: subtract the row maximum before exponentiating -- [W6] "Safe softmax".
  * paging: logical block t//16 of a sequence maps through its block table to a physical
    page, slot t%16 -- [W6] "PagedAttention"; [W4] "PagedAttention -- 메모리 단편화를 없애는
    커널".
  * GQA: query head h reads KV head floor(h / (Hq/Hkv)) (contiguous groups) -- [W4] "KV 헤드
    줄이기 -- MHA -> GQA -> MQA -> MLA" (group-wise sharing; the grouping order is our reading).

Variants used only to check invariants (they must equal the direct form):
  * online softmax, one key at a time, with running max m, running denominator d' and an
    un-normalised running output o', each rescaled by exp(m_old - m_new), divided by d' once at
    the end -- [W6] "FlashAttention의 single-pass 트릭"; [W4] "FlashAttention -- I/O를 줄이는
    방향" (running max m and sum l, rescale by exp(m_old - m_new)).
  * split-KV: partial attention per chunk of keys, then a combine by each chunk's max and sum
    (log-sum-exp) -- [W4] "FlashDecoding -- decode 단계의 병렬성 확보".

Buffer formats follow the C ABI header: K pool [P][Hkv][D/x][16][x] (x = 16 bytes / element
size), V pool [P][Hkv][D][16]; bf16 arrays arrive as raw 16-bit patterns.

FP8 cache ([W6] "KV Cache": the cache can be kept in a low-precision format such as FP8 to cut
its size and the bytes every decode step reads; [W4] "1-3. 모델 압축": the scale granularity is
an implementation choice to check).  Reading taken: OCP FP8 E4M3 codes (sign, 4 exponent bits
with bias 7, 3 mantissa bits; no infinities, S.1111.111 is NaN) and one float32 scale per
(page, KV head) for K and one for V; a cache element's value is decode(code) * scale.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Sequence, Tuple

import numpy as np

PAGE = 16


# ----------------------------------------------------------------------------------------
# element decoding
# ----------------------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 is the top half of an IEEE binary32; widening is exact."""
    u = np.asarray(bits).view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3: exponent field e (bias 7) and mantissa m; e = 0 is subnormal (m/8 * 2^-6);
    e = 15 with m = 7 is NaN (the format has no infinities)."""
    c = np.asarray(codes).astype(np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if dtype == "fp32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "fp8":
        return e4m3_to_f64(raw)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------------------
# paged KV gather
# ----------------------------------------------------------------------------------------
def gather_kv_token(k_pool, v_pool, table_row, t: int, kv_head: int, dtype: str):
    """Brute force: K and V rows of logical token t of one sequence, read through its block
    table.  k_pool is indexable as [page, head, d//x, slot, d%x], v_pool as [page, head, d, slot]."""
    page = int(table_row[t // PAGE])
    slot = t % PAGE
    kp = np.asarray(k_pool[page])          # [Hkv, D/x, 16, x]
    vp = np.asarray(v_pool[page])          # [Hkv, D, 16]
    nchunk, x = kp.shape[1], kp.shape[3]
    D = nchunk * x
    k = np.empty(D, dtype=np.float64)
    v = np.empty(D, dtype=np.float64)
    for d in range(D):
        k[d] = to_f64(kp[kv_head, d // x, slot, d % x:d % x + 1], dtype)[0]
        v[d] = to_f64(vp[kv_head, d, slot:slot + 1], dtype)[0]
    return k, v


def gather_kv(k_pool, v_pool, table_row, ctx: int, kv_head: int, dtype: str, k_scale=None, v_scale=None):
    """K, V in [ctx, D] float64 for one sequence and KV head (whole pages fetched, then the
    slots past ctx dropped).  Same result as gather_kv_token for every t < ctx.  With scales
    ([page][KV head] arrays, FP8 cache) every row is multiplied by its page's scale."""
    n_pages = -(-ctx // PAGE)
    pages = np.asarray(table_row[:n_pages], dtype=np.int64)
    kp = np.asarray(k_pool[pages])[:, kv_head]          # [n, D/x, 16, x]
    vp = np.asarray(v_pool[pages])[:, kv_head]          # [n, D, 16]
    n, nchunk, _, x = kp.shape
    K = to_f64(kp, dtype).transpose(0, 2, 1, 3).reshape(n * PAGE, nchunk * x)
    V = to_f64(vp, dtype).transpose(0, 2, 1).reshape(n * PAGE, nchunk * x)
    if k_scale is not None:
        K = K * np.repeat(np.asarray(k_scale, dtype=np.float64)[pages, kv_head], PAGE)[:, None]
        V = V * np.repeat(np.asarray(v_scale, dtype=np.float64)[pages, kv_head], PAGE)[:, None]
    return K[:ctx], V[:ctx]


# ----------------------------------------------------------------------------------------
# KV append: the step before attention in every iteration
# ----------------------------------------------------------------------------------------
def row_positions(prefill_q_start, prefill_ctx_len, decode_ctx_len) -> List[Tuple[int, int]]:
    """(sequence, absolute position) of every query row, in row order.  Prefill chunk i's L rows
    sit at positions ctx_i-L .. ctx_i-1; decode i is the sequence after the prefill sequences,
    its one row at position ctx_i-1 ([W6] "한 스텝에 여러 종류의 request 섞기": a decode is an
    extend of one token)."""
    out = []
    n_pf = len(prefill_ctx_len)
    for i in range(n_pf):
        L = int(prefill_q_start[i + 1]) - int(prefill_q_start[i])
        ctx = int(prefill_ctx_len[i])
        out += [(i, ctx - L + j) for j in range(L)]
    out += [(n_pf + i, int(c) - 1) for i, c in enumerate(decode_ctx_len)]
    return out


def append_tokens(k_pool, v_pool, block_tables, rows, k_new, v_new) -> None:
    """Write every row's new K and V (raw elements, [rows][Hkv][D]) into the slot its position
    falls in, in place: page = table[seq][pos // 16], slot = pos % 16 ([W6] "PagedAttention":
    a logical block maps to a physical page; [W6] "KV Cache": the cache grows by appending the
    new tokens' keys and values).  k_pool is [page, head, d//x, slot, d%x], v_pool
    [page, head, d, slot].  Plain loops."""
    Hkv, D = k_new.shape[1], k_new.shape[2]
    x = k_pool.shape[-1]
    for r, (s, pos) in enumerate(rows):
        page = int(block_tables[s][pos // PAGE])
        slot = pos % PAGE
        for g in range(Hkv):
            for d in range(D):
                k_pool[page, g, d // x, slot, d % x] = k_new[r, g, d]
                v_pool[page, g, d, slot] = v_new[r, g, d]


# ----------------------------------------------------------------------------------------
# attention, direct form
# ----------------------------------------------------------------------------------------
def masked_scores(qs: np.ndarray, pos: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """x_ij = scale * <q_i, k_j>, and -inf where key j lies after query position pos_i."""
    S = (qs @ K.T) * scale
    j = np.arange(K.shape[0])[None, :]
    return np.where(j <= pos[:, None], S, -np.inf)


def softmax_rows(S: np.ndarray) -> np.ndarray:
    """Safe softmax over each row: exp(x - max x) / sum exp(x - max x)."""
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    return E / E.sum(axis=1, keepdims=True)


def attend(qs: np.ndarray, pos: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
           return_probs: bool = False):
    """Explicit Q K^T, causal mask by absolute position, full safe softmax, then P V."""
    P = softmax_rows(masked_scores(qs, pos, K, scale))
    out = P @ V
    return (out, P) if return_probs else out


# ----------------------------------------------------------------------------------------
# invariant-check variants
# ----------------------------------------------------------------------------------------
def attend_online(q: np.ndarray, pos: int, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """One query, one key at a time: m_0=-inf, d'_0=0, o'_0=0; for each visible key j
    m_j = max(m_{j-1}, x_j), d'_j = d'_{j-1} e^{m_{j-1}-m_j} + e^{x_j-m_j},
    o'_j = o'_{j-1} e^{m_{j-1}-m_j} + e^{x_j-m_j} v_j; result o'_N / d'_N."""
    m, d, o = -math.inf, 0.0, np.zeros(V.shape[1])
    for j in range(min(pos + 1, K.shape[0])):
        x = scale * float(q @ K[j])
        m_new = max(m, x)
        r = math.exp(m - m_new) if m != -math.inf else 0.0
        e = math.exp(x - m_new)
        d = d * r + e
        o = o * r + e * V[j]
        m = m_new
    return o / d


def attend_blockwise(qs, pos, K, V, scale, block: int) -> np.ndarray:
    """The same recurrence applied to blocks of keys: per block, rowmax, rescale of the
    running sum and output by exp(m_old - m_new), then the block's contribution."""
    n, D = qs.shape[0], V.shape[1]
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    o = np.zeros((n, D))
    for a in range(0, K.shape[0], block):
        S = _masked_scores_offset(qs, pos, K[a:a + block], scale, a)
        m_new = np.maximum(m, S.max(axis=1))
        safe = np.where(np.isfinite(m_new), m_new, 0.0)
        r = np.where(np.isfinite(m), np.exp(m - safe), 0.0)
        E = np.exp(S - safe[:, None])
        l = l * r + E.sum(axis=1)
        o = o * r[:, None] + E @ V[a:a + block]
        m = m_new
    return o / l[:, None]


def _masked_scores_offset(qs, pos, Kb, scale, a):
    S = (qs @ Kb.T) * scale
    j = a + np.arange(Kb.shape[0])[None, :]
    return np.where(j <= pos[:, None], S, -np.inf)


def split_partials(qs, pos, K, V, scale, bounds: Sequence[int]) -> List[Tuple[np.ndarray, np.ndarray]]:
    """Per key range [bounds[i], bounds[i+1]): the normalised partial output o_s and its
    log-sum-exp lse_s = m_s + ln l_s (-inf, with o_s = 0, when the range has no visible key)."""
    parts = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        S = _masked_scores_offset(qs, pos, K[a:b], scale, a)
        m = S.max(axis=1) if b > a else np.full(qs.shape[0], -np.inf)
        safe = np.where(np.isfinite(m), m, 0.0)
        E = np.exp(S - safe[:, None])
        l = E.sum(axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            o = np.where(l[:, None] > 0, (E @ V[a:b]) / l[:, None], 0.0)
            lse = np.where(l > 0, m + np.log(l), -np.inf)
        parts.append((o, lse))
    return parts


def combine_partials(parts: Sequence[Tuple[np.ndarray, np.ndarray]]) -> np.ndarray:
    """out = sum_s w_s o_s / sum_s w_s with w_s = exp(lse_s - max_s lse_s); empty splits
    (lse = -inf) weigh zero."""
    lses = np.stack([p[1] for p in parts])              # [S, n]
    M = lses.max(axis=0)
    w = np.exp(lses - M[None, :])                       # exp(-inf) = 0
    num = sum(w[s][:, None] * parts[s][0] for s in range(len(parts)))
    return num / w.sum(axis=0)[:, None]


# ----------------------------------------------------------------------------------------
# the hybrid batch
# ----------------------------------------------------------------------------------------
class HybridProblem:
    """A hybrid batch as plain arrays.

    q: [total_q, Hq, D] raw (bf16 bits or float32); k_pool, v_pool: anything indexable by an
    integer page array along axis 0 in the ABI formats; block_tables: int [n_seq, stride].
    """

    def __init__(self, q, k_pool, v_pool, block_tables, prefill_q_start, prefill_ctx_len,
                 decode_ctx_len, num_q_heads, num_kv_heads, dtype, scale=None, kv_dtype=None,
                 k_scale=None, v_scale=None):
        self.q = q
        self.kv_dtype = kv_dtype or dtype                  # "fp8": q is bf16, the cache FP8 with scales
        self.k_scale, self.v_scale = k_scale, v_scale
        self.k_pool, self.v_pool = k_pool, v_pool
        self.bt = np.asarray(block_tables)
        self.q_start = np.asarray(prefill_q_start, dtype=np.int64)
        self.p_ctx = np.asarray(prefill_ctx_len, dtype=np.int64)
        self.d_ctx = np.asarray(decode_ctx_len, dtype=np.int64)
        self.Hq, self.Hkv, self.dtype = int(num_q_heads), int(num_kv_heads), dtype
        self.D = np.asarray(q).shape[2]
        self.scale = float(scale) if scale else 1.0 / math.sqrt(self.D)
        self.G = self.Hq // self.Hkv
        self.n_pre = len(self.p_ctx)
        self.n_pre_rows = int(self.q_start[-1]) if self.n_pre else 0

    def kv_head_of(self, h: int) -> int:
        return h // self.G

    def row_info(self, r: int):
        """(sequence index into the block table, absolute position, context) of q row r."""
        if r < self.n_pre_rows:
            s = int(np.searchsorted(self.q_start, r, side="right") - 1)
            L = int(self.q_start[s + 1] - self.q_start[s])
            ctx = int(self.p_ctx[s])
            return s, ctx - L + (r - int(self.q_start[s])), ctx
        i = r - self.n_pre_rows
        ctx = int(self.d_ctx[i])
        return self.n_pre + i, ctx - 1, ctx

    def seq_rows(self, s: int) -> np.ndarray:
        if s < self.n_pre:
            return np.arange(self.q_start[s], self.q_start[s + 1])
        return np.array([self.n_pre_rows + (s - self.n_pre)])

    def q_f64(self, rows, h) -> np.ndarray:
        return to_f64(np.asarray(self.q)[rows, h], self.dtype)

    def kv(self, s: int, g: int, ctx: int):
        return gather_kv(self.k_pool, self.v_pool, self.bt[s], ctx, g, self.kv_dtype, self.k_scale, self.v_scale)

    def sequence_output(self, s: int, heads: Iterable[int] | None = None) -> np.ndarray:
        """Reference output for every row of sequence s: [rows, len(heads), D]."""
        return self.rows_output(s, self.seq_rows(s), heads)

    def rows_output(self, s: int, rows, heads: Iterable[int] | None = None) -> np.ndarray:
        """Reference output for the given q rows (all of sequence s): [rows, len(heads), D]."""
        rows = np.asarray(rows, dtype=np.int64)
        if len(rows) == 0:
            return np.zeros((0, self.Hq, self.D))
        _, _, ctx = self.row_info(int(rows[0]))
        pos = np.array([self.row_info(int(r))[1] for r in rows])
        heads = list(range(self.Hq)) if heads is None else list(heads)
        out = np.empty((len(rows), len(heads), self.D))
        cache = {}
        for j, h in enumerate(heads):
            g = self.kv_head_of(h)
            if g not in cache:
                cache[g] = self.kv(s, g, ctx)
            K, V = cache[g]
            out[:, j] = attend(self.q_f64(rows, h), pos, K, V, self.scale)
        return out

    def full_output(self) -> np.ndarray:
        total = self.n_pre_rows + len(self.d_ctx)
        out = np.empty((total, self.Hq, self.D))
        for s in range(self.n_pre + len(self.d_ctx)):
            rows = self.seq_rows(s)
            if len(rows):
                out[rows] = self.sequence_output(s)
        return out

    def sampled_output(self, pairs: Sequence[Tuple[int, int]]) -> np.ndarray:
        """Reference rows for a list of (q row, head) pairs, computed one by one."""
        res = np.empty((len(pairs), self.D))
        cache = {}
        for i, (r, h) in enumerate(pairs):
            s, pos, ctx = self.row_info(int(r))
            g = self.kv_head_of(int(h))
            key = (s, g)
            if key not in cache:
                if len(cache) > 8:
                    cache.clear()
                cache[key] = self.kv(s, g, ctx)
            K, V = cache[key]
            res[i] = attend(self.q_f64([int(r)], int(h)), np.array([pos]), K, V, self.scale)[0]
        return res
