"""Shared test plumbing: run the library on a generated batch, build the oracle problem from the
same input buffers, and compare with the stated tolerances."""
from __future__ import annotations

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
