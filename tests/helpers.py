"""Shared test plumbing: run the library on a generated batch, build the oracle problem from the
same input buffers, and compare with the stated tolerances."""
from __future__ import annotations

from collections import deque
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from hybrid_prefill_decode_paged_amd import binding
from hybrid_prefill_decode_paged_amd import inputs as gen
from oracle import attention as orc

# Tolerances: bf16 inputs with fp32 accumulation: max abs <= 2e-2 and mean abs <= 2e-3;
# fp32 inputs: max abs <= 1e-5.  FP8 cache (bf16 q/out): the bf16 bar -- the oracle decodes the
# same codes and scales, so the difference is the bf16 rounding of q, P*scale and out.
TOL = {"bf16": (2e-2, 2e-3), "fp32": (1e-5, 1e-5), "fp8": (2e-2, 2e-3)}


class DevicePages:
    """Indexable view of a device pool for the oracle: pool[pages] copies only those pages."""

    def __init__(self, t: torch.Tensor, dtype: str):
        self.t, self.dtype = t, dtype

    def __getitem__(self, idx):
        if isinstance(idx, (int, np.integer)):
            sel = self.t[int(idx)]
        else:
            sel = self.t[torch.as_tensor(np.asarray(idx, dtype=np.int64), device=self.t.device)]
        sel = sel.cpu()
        return sel.view(torch.int16).numpy() if self.dtype == "bf16" else sel.numpy()


def problem(b: gen.HybridBatch) -> orc.HybridProblem:
    s = b.spec
    q = b.q.cpu()
    qraw = q.view(torch.int16).numpy() if q.dtype == torch.bfloat16 else q.numpy()
    if s.dtype == "fp8":
        return orc.HybridProblem(qraw, DevicePages(b.k_pool, "fp8"), DevicePages(b.v_pool, "fp8"),
                                 b.block_tables_host, b.prefill_q_start, b.prefill_ctx_len, b.decode_ctx_len,
                                 s.num_q_heads, s.num_kv_heads, "bf16", s.softmax_scale, kv_dtype="fp8",
                                 k_scale=b.k_scale.cpu().numpy(), v_scale=b.v_scale.cpu().numpy())
    if b.k_pool.is_cuda:
        kp, vp = DevicePages(b.k_pool, s.dtype), DevicePages(b.v_pool, s.dtype)
    else:
        kp = b.k_pool.view(torch.int16).numpy() if s.dtype == "bf16" else b.k_pool.numpy()
        vp = b.v_pool.view(torch.int16).numpy() if s.dtype == "bf16" else b.v_pool.numpy()
    return orc.HybridProblem(qraw, kp, vp, b.block_tables_host, b.prefill_q_start, b.prefill_ctx_len,
                             b.decode_ctx_len, s.num_q_heads, s.num_kv_heads, s.dtype, s.softmax_scale)


def run_library(b: gen.HybridBatch, mode="fused", flags=0, handle=None, out=None, workspace=None, **kw):
    s = b.spec
    h = handle or binding.PodAttention(s.num_q_heads, s.num_kv_heads, s.head_dim, s.dtype, mode,
                                       scale=s.softmax_scale, flags=flags, **kw)
    meta = binding.BatchMeta.from_batch(b)
    ws_bytes = h.workspace_size(meta)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=b.q.device)
    if out is None:
        out = torch.full_like(b.q, float("nan"))
    if s.dtype == "fp8":
        h.run_scaled(b.q, b.k_pool, b.v_pool, b.k_scale, b.v_scale, b.block_tables, meta, out, workspace)
    else:
        h.run(b.q, b.k_pool, b.v_pool, b.block_tables, meta, out, workspace)
    torch.cuda.synchronize()
    return out, h, workspace


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def check_close(got: np.ndarray, want: np.ndarray, dtype: str, what: str = ""):
    max_tol, mean_tol = TOL[dtype]
    assert not np.isnan(got).any(), f"{what}: NaN in output"
    err = np.abs(got - want)
    assert err.max() <= max_tol, f"{what}: max abs err {err.max():.3g} > {max_tol}"
    assert err.mean() <= mean_tol, f"{what}: mean abs err {err.mean():.3g} > {mean_tol}"
    return float(err.max()), float(err.mean())


def sample_pairs(b: gen.HybridBatch, n_prefill: int, n_decode: int, seed: int = 0):
    """Sampled (q row, head) pairs: first/last prefill rows of each chunk, random others, and
    random decode rows (always the first and last decode)."""
    rng = np.random.default_rng(seed)
    s = b.spec
    pairs = []
    qs = b.prefill_q_start
    for i in range(s.num_prefill):
        a, z = int(qs[i]), int(qs[i + 1])
        if z > a:
            rows = {a, z - 1} | set(rng.integers(a, z, size=n_prefill).tolist())
            pairs += [(r, int(rng.integers(0, s.num_q_heads))) for r in sorted(rows)]
    P = int(qs[-1]) if s.num_prefill else 0
    if s.num_decode:
        rows = {P, P + s.num_decode - 1} | set((P + rng.integers(0, s.num_decode, size=n_decode)).tolist())
        pairs += [(r, int(rng.integers(0, s.num_q_heads))) for r in sorted(rows)]
    return pairs


# ------------------------------------------------------------------ full-size reference rows
class HostPages:
    """One sequence's pages already copied to the host, indexable like a pool by page arrays.  A
    repeat of the last page array returns the same host array without a copy: the oracle reads
    the sequence's pages once per KV head."""

    def __init__(self, a: np.ndarray):
        self.a, self._idx, self._val = a, None, None

    def __getitem__(self, idx):
        arr = np.asarray(idx, dtype=np.int64)
        if self._idx is not None and self._idx.shape == arr.shape and np.array_equal(self._idx, arr):
            return self._val
        self._idx, self._val = arr.copy(), self.a[arr]
        return self._val


def _raw_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    t = t.cpu()
    return t.view(torch.int16).numpy() if dtype == "bf16" else t.numpy()


def checked_rows(b: gen.HybridBatch, tile_queries: int, decode_every: int = 1):
    """The rows a full-size check compares, per sequence: the first and last row of every prefill
    tile (tiles of tile_queries rows from each chunk's first row) and every decode_every-th decode
    row (the last decode always).  Returns [(sequence, [q rows])]."""
    s = b.spec
    qs = b.prefill_q_start
    per_seq = []
    for i in range(s.num_prefill):
        a, z = int(qs[i]), int(qs[i + 1])
        rows = set()
        for t in range(a, z, tile_queries):
            rows.update((t, min(t + tile_queries, z) - 1))
        if rows:
            per_seq.append((i, sorted(rows)))
    P = int(qs[-1]) if s.num_prefill else 0
    dec = list(range(0, s.num_decode, decode_every))
    if s.num_decode and dec[-1] != s.num_decode - 1:
        dec.append(s.num_decode - 1)
    per_seq += [(s.num_prefill + d, [P + d]) for d in dec]
    return per_seq


def _sequence_reference(b: gen.HybridBatch, s: int, rows, kp, vp, ksc, vsc, qraw):
    """The oracle on one sequence alone: a one-sequence problem over the sequence's own pages
    (renumbered 0..n-1), giving [len(rows), Hq, D] for the given q rows of the batch."""
    spec = b.spec
    qs = b.prefill_q_start
    n = kp.shape[0]
    bt = np.arange(n, dtype=np.int32)[None, :]
    q_dtype = "bf16" if spec.dtype == "fp8" else spec.dtype
    kw = dict(kv_dtype="fp8", k_scale=ksc, v_scale=vsc) if spec.dtype == "fp8" else {}
    if s < spec.num_prefill:
        a, z = int(qs[s]), int(qs[s + 1])
        prob = orc.HybridProblem(qraw[a:z], HostPages(kp), HostPages(vp), bt, [0, z - a],
                                 [int(b.prefill_ctx_len[s])], [], spec.num_q_heads, spec.num_kv_heads,
                                 q_dtype, spec.softmax_scale, **kw)
        return prob.rows_output(0, [r - a for r in rows])
    (r,) = rows
    prob = orc.HybridProblem(qraw[r:r + 1], HostPages(kp), HostPages(vp), bt, [0], [],
                             [int(b.decode_ctx_len[s - spec.num_prefill])], spec.num_q_heads,
                             spec.num_kv_heads, q_dtype, spec.softmax_scale, **kw)
    return prob.sequence_output(0)


def reference_rows(b: gen.HybridBatch, per_seq, workers: int = 8):
    """Oracle output of the rows of checked_rows(): each sequence's pages are copied from the
    device to the host on this thread, and its fp64 reference is computed on a pool of threads
    (at most 2 * workers sequences held on the host at once).  Returns (rows, [rows, Hq, D])."""
    spec = b.spec
    q = b.q.cpu()
    qraw = q.view(torch.int16).numpy() if q.dtype == torch.bfloat16 else q.numpy()
    ctxs = spec.seq_ctx()
    rows, parts = [], []
    with ThreadPoolExecutor(workers) as ex:
        pending = deque()
        for s, rr in per_seq:
            n = -(-int(ctxs[s]) // gen.PAGE_SIZE)
            pages = torch.as_tensor(b.block_tables_host[s, :n].astype(np.int64), device=b.k_pool.device)
            kp = _raw_host(b.k_pool[pages], spec.dtype)
            vp = _raw_host(b.v_pool[pages], spec.dtype)
            ksc = b.k_scale[pages].cpu().numpy() if spec.dtype == "fp8" else None
            vsc = b.v_scale[pages].cpu().numpy() if spec.dtype == "fp8" else None
            pending.append(ex.submit(_sequence_reference, b, s, rr, kp, vp, ksc, vsc, qraw))
            rows += rr
            while len(pending) > 2 * workers:
                parts.append(pending.popleft().result())
        while pending:
            parts.append(pending.popleft().result())
    return np.asarray(rows, dtype=np.int64), np.concatenate(parts)


def check_rows(out: torch.Tensor, rows: np.ndarray, want: np.ndarray, dtype: str, what: str):
    """Compare out[rows] (all heads) with the reference rows; every row of out must be written."""
    assert not torch.isnan(out).any(), f"{what}: NaN (an unwritten row?) in the output"
    got = out[torch.as_tensor(rows, device=out.device)].to(torch.float64).cpu().numpy()
    return check_close(got, want, dtype, what)


def bucket_reference(run):
    """Reference checker for cost_table.calibrate: the fp64 oracle on the bucket's sampled rows
    (all heads), returning the (max, mean) absolute error of the library's output there."""
    q = run.q.cpu()
    qraw = q.view(torch.int16).numpy() if q.dtype == torch.bfloat16 else q.numpy()
    meta = (run.block_tables_host, run.prefill_q_start, run.prefill_ctx_len, run.decode_ctx_len,
            run.num_q_heads, run.num_kv_heads)
    if run.dtype == "fp8":
        prob = orc.HybridProblem(qraw, DevicePages(run.k_pool, "fp8"), DevicePages(run.v_pool, "fp8"), *meta,
                                 "bf16", run.scale, kv_dtype="fp8", k_scale=run.k_scale.cpu().numpy(),
                                 v_scale=run.v_scale.cpu().numpy())
    else:
        prob = orc.HybridProblem(qraw, DevicePages(run.k_pool, run.dtype), DevicePages(run.v_pool, run.dtype), *meta,
                                 run.dtype, run.scale)
    errs = []
    for r in run.rows:
        s, _, _ = prob.row_info(int(r))
        want = prob.rows_output(s, [int(r)])[0]
        got = run.out[int(r)].to(torch.float64).cpu().numpy()
        errs.append(np.abs(got - want).ravel())
    e = np.concatenate(errs)
    return float(e.max()), float(e.mean())
