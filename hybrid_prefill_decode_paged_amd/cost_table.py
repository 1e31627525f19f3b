"""Measured cost table for an outer scheduler.

The POD-Attention digest (Silicon & Systems, "POD-Attention hybrid batching", section "Resource
characteristics as scheduling inputs") asks for online signals that stay simple: the batches
cannot all be measured ahead of time, so prefill chunks and decode groups are put into buckets,
and the kernel publishes a small set of validated combinations with their latencies for the
scheduler to choose from; section "Predictable latency and diagnostics" adds that the limits
should follow tail latency and that shapes outside the validated set belong to admission
control.

``calibrate`` runs one fused step per bucket -- a prefill chunk of ``chunk_len`` rows whose
context is ``chunk_ctx``, plus ``n_decode`` decodes at context ``decode_ctx`` -- on synthetic
data in this library's buffer formats, ``steps`` times, and records the step's wall time (median
and maximum), the fused kernel's own time, and the batch's signals (``pod_attn_batch_signals``).
A bucket is validated when its runs took the fused path, reported no device error, wrote a
finite output, and its output matched an independent reference within the library's stated
tolerance (bf16 and the FP8 cache: max abs 2e-2, mean abs 2e-3; fp32: 1e-5) on the sampled rows of
``checked_rows`` (every head of the first and last prefill row and of the first and last decode
row).  The reference is the caller's (``calibrate(reference=...)``): this module computes no
attention itself, and a table calibrated without one publishes no validated bucket.  ``CostTable.lookup`` rounds each axis of a batch up to the table's next grid
value (as a static-shape backend pads a batch to its bucket, [W6] "Batching의 비용은 bucket
크기로 정해진다") and returns None outside the table or for a bucket that failed validation.
"""
from __future__ import annotations

import json
import statistics
from dataclasses import asdict, dataclass, field
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

from . import binding

PAGE = 16


@dataclass
class Entry:
    chunk_len: int
    chunk_ctx: int
    n_decode: int
    decode_ctx: int
    step_us_p50: float
    step_us_max: float
    kernel_us_p50: float
    kernel_us_max: float
    validated: bool
    signals: Dict[str, float] = field(default_factory=dict)
    max_abs_err: Optional[float] = None     # against the reference, over the sampled rows
    mean_abs_err: Optional[float] = None

    def key(self):
        return (self.chunk_len, self.chunk_ctx, self.n_decode, self.decode_ctx)


@dataclass
class CostTable:
    heads_q_kv_dim: List[int]
    dtype: str
    entries: List[Entry]

    def lookup(self, chunk_len: int, chunk_ctx: int, n_decode: int, decode_ctx: int) -> Optional[Entry]:
        """The bucket the batch pads to: each axis rounded up to the next grid value of the table
        (a chunk of 0 rows has no context, no decodes no decode context).  None when an axis is
        past the grid or the bucket was not validated."""
        def up(v, values):
            c = [x for x in sorted(set(values)) if x >= v]
            return c[0] if c else None
        L = up(chunk_len, [e.chunk_len for e in self.entries])
        n = up(n_decode, [e.n_decode for e in self.entries])
        if L is None or n is None:
            return None
        C = up(chunk_ctx, [e.chunk_ctx for e in self.entries if e.chunk_len]) if L else 0
        Dc = up(decode_ctx, [e.decode_ctx for e in self.entries if e.n_decode]) if n else 0
        if C is None or Dc is None:
            return None
        for e in self.entries:
            if e.key() == (L, C, n, Dc):
                return e if e.validated else None
        return None

    def to_json(self) -> str:
        return json.dumps({"heads_q_kv_dim": self.heads_q_kv_dim, "dtype": self.dtype,
                           "entries": [asdict(e) for e in self.entries]}, indent=1)

    @staticmethod
    def from_json(text: str) -> "CostTable":
        d = json.loads(text)
        return CostTable(d["heads_q_kv_dim"], d["dtype"], [Entry(**e) for e in d["entries"]])


def bucket_batch(chunk_len: int, chunk_ctx: int, n_decode: int, decode_ctx: int):
    """Host metadata of one bucket's batch: (prefill_q_start, prefill_ctx_len, decode_ctx_len)."""
    if chunk_len > 0:
        q_start, p_ctx = [0, chunk_len], [chunk_ctx]
    else:
        q_start, p_ctx = [0], []
    return np.asarray(q_start, np.int32), np.asarray(p_ctx, np.int32), np.full(n_decode, decode_ctx, np.int32)


TOLERANCE = {"bf16": (2e-2, 2e-3), "fp8": (2e-2, 2e-3), "fp32": (1e-5, 1e-5)}   # (max abs, mean abs) of a validated bucket


@dataclass
class BucketRun:
    """What a reference checker gets for one bucket: the inputs in the C ABI's formats (device
    tensors and host metadata), the library's output, and the q rows to compare (all heads)."""
    q: object
    k_pool: object
    v_pool: object
    block_tables_host: np.ndarray
    prefill_q_start: np.ndarray
    prefill_ctx_len: np.ndarray
    decode_ctx_len: np.ndarray
    num_q_heads: int
    num_kv_heads: int
    dtype: str
    scale: float
    out: object
    rows: List[int]
    k_scale: object = None      # FP8 cache: float32 [pages, Hkv] scale of each K slab
    v_scale: object = None


def checked_rows(chunk_len: int, n_decode: int) -> List[int]:
    """q rows a bucket is validated on: the first and last prefill row, the first and last decode."""
    rows = sorted({0, chunk_len - 1}) if chunk_len > 0 else []
    if n_decode:
        rows += sorted({chunk_len, chunk_len + n_decode - 1})
    return rows


def calibrate(num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: str,
              chunk_lens: Sequence[int], chunk_ctxs: Sequence[int], decode_counts: Sequence[int],
              decode_ctxs: Sequence[int], steps: int = 5, warmup: int = 1, seed: int = 0,
              reference: Optional[Callable[[BucketRun], "tuple[float, float]"]] = None) -> CostTable:
    """Measure every bucket of the grid in fused mode on the current GPU (see the module text).
    ``reference(run)`` returns the (max, mean) absolute error of ``run.out`` on ``run.rows``
    against an independent reference; without it no bucket is validated."""
    import torch

    fp8 = dtype == "fp8"
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16     # q and out (bf16 beside an FP8 cache)
    x = 16 // {"bf16": 2, "fp32": 4, "fp8": 1}[dtype]               # elements per 16-byte K chunk
    grid = [(L, C if L else 0, n, Dc if n else 0) for L in chunk_lens for C in chunk_ctxs
            for n in decode_counts for Dc in decode_ctxs if (L == 0 or C >= L)]
    grid = sorted(set(g for g in grid if g[0] or g[2]))
    # one pool and one q buffer sized for the largest bucket, drawn once
    max_pages = max(-(-g[1] // PAGE) + g[2] * -(-g[3] // PAGE) for g in grid) if grid else 1
    max_rows = max(g[0] + g[2] for g in grid) if grid else 1
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    q = (torch.randn(max_rows, num_q_heads, head_dim, generator=gen, device="cuda") * 0.5).to(tdt)
    k_scale = v_scale = None
    if fp8:
        # one scale per (page, KV head) slab, uniform in [0.5, 2); the slab holds the E4M3 codes
        # (round to nearest even) of N(0,1) * 0.5 / scale
        k_scale = torch.rand(max_pages, num_kv_heads, generator=gen, device="cuda") * 1.5 + 0.5
        v_scale = torch.rand(max_pages, num_kv_heads, generator=gen, device="cuda") * 1.5 + 0.5
        k_pool = (torch.randn(max_pages, num_kv_heads, head_dim // x, PAGE, x, generator=gen, device="cuda") * 0.5
                  / k_scale[:, :, None, None, None]).to(torch.float8_e4m3fn).view(torch.uint8)
        v_pool = (torch.randn(max_pages, num_kv_heads, head_dim, PAGE, generator=gen, device="cuda") * 0.5
                  / v_scale[:, :, None, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    else:
        k_pool = (torch.randn(max_pages, num_kv_heads, head_dim // x, PAGE, x, generator=gen, device="cuda") * 0.5).to(tdt)
        v_pool = (torch.randn(max_pages, num_kv_heads, head_dim, PAGE, generator=gen, device="cuda") * 0.5).to(tdt)

    def run(qv, bt_dev, meta, out, ws):
        if fp8:
            h.run_scaled(qv, k_pool, v_pool, k_scale, v_scale, bt_dev, meta, out, ws)
        else:
            h.run(qv, k_pool, v_pool, bt_dev, meta, out, ws)
    perm = np.random.Generator(np.random.PCG64(seed)).permutation(max_pages).astype(np.int32)
    h = binding.PodAttention(num_q_heads, num_kv_heads, head_dim, dtype, "fused")
    stream = torch.cuda.current_stream()
    entries = []
    for L, C, n, Dc in grid:
        q_start, p_ctx, d_ctx = bucket_batch(L, C, n, Dc)
        ctx = list(p_ctx) + list(d_ctx)
        npg = [-(-c // PAGE) for c in ctx]
        stride = max(npg)
        bt = np.zeros((len(ctx), stride), np.int32)
        pos = 0
        for s, m in enumerate(npg):
            bt[s, :m] = perm[pos:pos + m]
            pos += m
        meta = binding.BatchMeta(q_start, p_ctx, d_ctx, stride, max_pages)
        bt_dev = torch.from_numpy(bt).cuda()
        rows = L + n
        qv = q[:rows].contiguous()
        out = torch.empty_like(qv)
        ws = torch.empty(h.workspace_size(meta), dtype=torch.uint8, device="cuda")
        for _ in range(warmup):
            run(qv, bt_dev, meta, out, ws)
        torch.cuda.synchronize()
        walls, kerns = [], []
        for _ in range(steps):
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ka, kz = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ka.record(stream)
            kz.record(stream)
            torch.cuda.synchronize()
            a.record(stream)
            h.set_kernel_events(ka, kz)
            run(qv, bt_dev, meta, out, ws)
            z.record(stream)
            torch.cuda.synchronize()
            walls.append(a.elapsed_time(z) * 1e3)
            kerns.append(ka.elapsed_time(kz) * 1e3)
        st = h.stats()
        status, _, _ = h.read_device_status(ws)
        ok = st["mode_used"] == binding.MODES["fused"] and status == 0 and bool(torch.isfinite(out).all())
        max_err = mean_err = None
        if reference is not None:
            max_err, mean_err = reference(BucketRun(qv, k_pool, v_pool, bt, q_start, p_ctx, d_ctx, num_q_heads,
                                                    num_kv_heads, dtype, h.cfg.scale if h.cfg.scale > 0
                                                    else 1.0 / head_dim ** 0.5, out, checked_rows(L, n),
                                                    k_scale, v_scale))
            max_err, mean_err = float(max_err), float(mean_err)
        tol = TOLERANCE[dtype]
        ok = ok and max_err is not None and max_err <= tol[0] and mean_err <= tol[1]
        sig = binding.batch_signals(h.cfg, meta, st["num_cus"], st["wgs_per_cu"])
        entries.append(Entry(L, C, n, Dc, round(statistics.median(walls), 2), round(max(walls), 2),
                             round(statistics.median(kerns), 2), round(max(kerns), 2), ok,
                             {k: sig[k] for k in ("prefill_items", "decode_items", "lds_bytes_per_wg",
                                                  "prefill_flops", "decode_bytes", "intensity", "roofline_us")},
                             max_err, mean_err))
        del ws, out, bt_dev
    h.close()
    return CostTable([num_q_heads, num_kv_heads, head_dim], dtype, entries)


if __name__ == "__main__":
    import argparse
    import sys

    ap = argparse.ArgumentParser(description="measure a cost table on the current GPU and print it as JSON "
                                             "(timings only: without a reference no bucket is validated)")
    ap.add_argument("--heads", default="32,8,128", help="Hq,Hkv,D")
    ap.add_argument("--dtype", default="bf16")
    ap.add_argument("--chunk-lens", default="0,512,1024,2048")
    ap.add_argument("--chunk-ctxs", default="4096,16384")
    ap.add_argument("--decode-counts", default="0,32,64,128")
    ap.add_argument("--decode-ctxs", default="4096,16384,32768")
    ap.add_argument("--steps", type=int, default=5)
    a = ap.parse_args()
    ints = lambda s: [int(v) for v in s.split(",")]
    hq, hkv, d = ints(a.heads)
    t = calibrate(hq, hkv, d, a.dtype, ints(a.chunk_lens), ints(a.chunk_ctxs), ints(a.decode_counts),
                  ints(a.decode_ctxs), steps=a.steps)
    sys.stdout.write(t.to_json() + "\n")
