"""Seeded synthetic inputs for hybrid prefill/decode paged attention.

This module draws random numbers and places them in the buffer formats that the C ABI
(``include/pod_attn.h``) documents.  It computes nothing of attention: no products, no
softmax, no masking.  Both the oracle-side tests and the GPU path consume what it makes.

Workloads (the five batches the library is measured on) stand in for the long-context
Llama-2-7B / Llama-3-8B / Yi-6B serving traces that the POD-Attention digest (Silicon &
Systems, "POD-Attention hybrid batching", section "Benefit grows with long context")
evaluates on; those traces are not available, so every value here is synthetic.

Buffer formats (from the ABI header):
  q, out      [total_q][Hq][D], prefill rows first (chunk by chunk), then one row per decode
  k_pool      [num_pages][Hkv][D/x][16][x]   with x = 16 bytes / element size (8 bf16, 4 fp32)
  v_pool      [num_pages][Hkv][D][16]
  block table int32 [n_seq][stride]; row s lists the physical pages of sequence s in order;
              prefill sequences first, then decode sequences.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np
import torch

PAGE_SIZE = 16
# Unused block-table entries hold this out-of-range id; the kernels must never read them.
UNUSED_PAGE_ID = 0x3FFFFFF0


@dataclass
class BatchSpec:
    name: str
    dtype: str                      # "bf16", "fp32", or "fp8" (E4M3 cache with per-(page, head) scales, bf16 q)
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    prefill_q_len: List[int]
    prefill_ctx_len: List[int]
    decode_ctx_len: List[int]
    num_pages: int
    seed: int
    value_scale: float = 1.0        # values are N(0,1) * value_scale before the dtype cast
    k_outlier_frac: float = 0.0     # fraction of live K rows multiplied by k_outlier_mult
    k_outlier_mult: float = 8.0
    scale: Optional[float] = None   # softmax scale; None means 1/sqrt(head_dim)
    identity_pages: bool = False    # pages taken in order 0,1,2,... instead of a permutation
    extra: dict = field(default_factory=dict)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        """Bytes of one cache element."""
        return {"bf16": 2, "fp32": 4, "fp8": 1}[self.dtype]

    @property
    def q_elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    @property
    def chunk_elems(self) -> int:
        return 16 // self.elem_bytes

    @property
    def torch_dtype(self):
        """Element type of q and out (and of the cache, except for "fp8")."""
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    @property
    def cache_torch_dtype(self):
        return torch.uint8 if self.dtype == "fp8" else self.torch_dtype

    @property
    def num_prefill(self) -> int:
        return len(self.prefill_q_len)

    @property
    def num_decode(self) -> int:
        return len(self.decode_ctx_len)

    @property
    def total_q(self) -> int:
        return int(sum(self.prefill_q_len)) + self.num_decode

    def seq_ctx(self) -> List[int]:
        return list(self.prefill_ctx_len) + list(self.decode_ctx_len)

    def live_pages(self) -> int:
        return int(sum(-(-c // PAGE_SIZE) for c in self.seq_ctx()))


def _live_plus_quarter(ctx: List[int]) -> int:
    live = sum(-(-c // PAGE_SIZE) for c in ctx)
    return live + live // 4


def config_spec(idx: int) -> BatchSpec:
    """The five measured workloads (1-based index), as concrete seeded batches."""
    if idx == 1:
        return BatchSpec("tiny-fp32", "fp32", 4, 4, 64, [64], [192], [37, 100, 256, 257],
                         num_pages=64, seed=1, value_scale=1.0)
    if idx == 2:
        return BatchSpec("llama2-7b-mha", "bf16", 32, 32, 128, [1024], [4096], [4096] * 64,
                         num_pages=40960, seed=2, value_scale=0.5)
    if idx == 3:
        rng = np.random.Generator(np.random.PCG64(3))
        dec = rng.integers(4096, 32768, size=128, endpoint=True).tolist()
        ctx = [16384] + dec
        return BatchSpec("llama3-8b-gqa", "bf16", 32, 8, 128, [2048], [16384], dec,
                         num_pages=_live_plus_quarter(ctx), seed=3, value_scale=0.5)
    if idx == 4:
        rng = np.random.Generator(np.random.PCG64(4))
        raw = np.exp(rng.normal(math.log(8192.0), 1.0, size=96))
        dec = np.clip(np.rint(raw), 1024, 32768).astype(np.int64).tolist()
        pre_ctx = [512, 8192 + 512, 28000 + 512]
        return BatchSpec("yi-6b-gqa8", "bf16", 32, 4, 128, [512, 512, 512], pre_ctx, dec,
                         num_pages=_live_plus_quarter(pre_ctx + dec), seed=4, value_scale=0.5,
                         k_outlier_frac=0.01)
    if idx == 5:
        return BatchSpec("llama3-8b-long", "bf16", 32, 8, 128, [512], [32768], [32768] * 256,
                         num_pages=1 << 20, seed=5, value_scale=0.5)
    raise ValueError(f"no workload {idx}")


def fp8_spec(idx: int) -> BatchSpec:
    """Workload idx (2..5) with its cache in FP8 E4M3 with per-(page, KV head) scales and bf16 q;
    the Yi-6B-shaped workload's K outlier rows are left out (the scales are per slab)."""
    base = config_spec(idx)
    if base.dtype != "bf16":
        raise ValueError("the FP8 variants are of the bf16 workloads")
    return replace(base, name=base.name + "-fp8", dtype="fp8", k_outlier_frac=0.0)


def spec_verify_spec(n_extend: int = 4) -> BatchSpec:
    """A speculative-verification step on the Llama-3-8B-shaped workload: its 2048-token chunk at
    offset 14336, and each of its 128 decode sequences extending by ``n_extend`` tokens instead of
    one (the sequence's context as drawn for that workload, the extend's rows at its end)."""
    base = config_spec(3)
    dec = [int(c) for c in base.decode_ctx_len]
    pq = [2048] + [n_extend] * len(dec)
    pc = [16384] + dec
    return BatchSpec(f"llama3-8b-specverify{n_extend}", "bf16", 32, 8, 128, pq, pc, [],
                     num_pages=_live_plus_quarter(pc), seed=6, value_scale=0.5)


def reduced_spec(idx: int, n_decode: int, ctx_div: int, seed: Optional[int] = None) -> BatchSpec:
    """A smaller batch with the same heads, dims, dtype and value law as workload ``idx``:
    the first ``n_decode`` decodes, every context (and prefill offset) divided by ``ctx_div``."""
    base = config_spec(idx)
    pq, pc = [], []
    for L, c in zip(base.prefill_q_len, base.prefill_ctx_len):
        off = (c - L) // ctx_div
        Lr = max(1, L // ctx_div)
        pq.append(Lr)
        pc.append(off + Lr)
    dec = [max(1, c // ctx_div) for c in base.decode_ctx_len[:n_decode]]
    live = sum(-(-c // PAGE_SIZE) for c in pc + dec)
    return replace(base, name=f"{base.name}/r{n_decode}x{ctx_div}", prefill_q_len=pq,
                   prefill_ctx_len=pc, decode_ctx_len=dec, num_pages=live + live // 4 + 3,
                   seed=base.seed if seed is None else seed)


@dataclass
class HybridBatch:
    spec: BatchSpec
    q: torch.Tensor                 # [total_q, Hq, D]
    k_pool: torch.Tensor            # [P, Hkv, D/x, 16, x]
    v_pool: torch.Tensor            # [P, Hkv, D, 16]
    block_tables: torch.Tensor      # int32 [n_seq, stride] (same device as the pools)
    block_tables_host: np.ndarray   # int32 copy on the host
    prefill_q_start: np.ndarray     # int32 [num_prefill + 1]
    prefill_ctx_len: np.ndarray     # int32 [num_prefill]
    decode_ctx_len: np.ndarray      # int32 [num_decode]
    k_scale: Optional[torch.Tensor] = None   # fp8: float32 [P, Hkv], scale of each K slab
    v_scale: Optional[torch.Tensor] = None   # fp8: float32 [P, Hkv], scale of each V slab

    @property
    def device(self):
        return self.q.device


def block_tables_for(spec: BatchSpec) -> np.ndarray:
    """Physical pages for every sequence, taken consecutively from a seeded permutation of
    the pool (or in order when ``identity_pages``); unused entries hold UNUSED_PAGE_ID."""
    ctx = spec.seq_ctx()
    npages = [-(-c // PAGE_SIZE) for c in ctx]
    stride = max(npages) if npages else 1
    if spec.identity_pages:
        perm = np.arange(spec.num_pages, dtype=np.int64)
    else:
        perm = np.random.Generator(np.random.PCG64(spec.seed)).permutation(spec.num_pages)
    if sum(npages) > spec.num_pages:
        raise ValueError("pool too small for the live pages")
    bt = np.full((len(ctx), stride), UNUSED_PAGE_ID, dtype=np.int32)
    pos = 0
    for s, n in enumerate(npages):
        bt[s, :n] = perm[pos:pos + n]
        pos += n
    return bt


def k_rows_view(k_pool: torch.Tensor) -> torch.Tensor:
    """[P, Hkv, 16, D/x, x] view of a K pool: index [page, head, slot] gives one token's row."""
    return k_pool.permute(0, 1, 3, 2, 4)


def v_rows_view(v_pool: torch.Tensor) -> torch.Tensor:
    """[P, Hkv, 16, D] view of a V pool: index [page, head, slot] gives one token's row."""
    return v_pool.permute(0, 1, 3, 2)


def _fill_normal(t: torch.Tensor, gen: torch.Generator, scale: float, chunk_elems: int):
    flat = t.view(-1)
    n = flat.numel()
    for a in range(0, n, chunk_elems):
        b = min(n, a + chunk_elems)
        x = torch.randn(b - a, generator=gen, device=t.device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        flat[a:b].copy_(x)          # float32 -> bf16 copy rounds to nearest even


def make_batch(spec: BatchSpec, device="cpu", chunk_elems: int = 1 << 28) -> HybridBatch:
    """Draw the batch: q, then the whole K pool, then the whole V pool, from one torch
    generator seeded with ``spec.seed``; block tables from numpy PCG64(seed)."""
    device = torch.device(device)
    H, Hk, D, x = spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.chunk_elems
    gen = torch.Generator(device=device)
    gen.manual_seed(spec.seed)
    q = torch.empty(spec.total_q, H, D, dtype=spec.torch_dtype, device=device)
    k_pool = torch.empty(spec.num_pages, Hk, D // x, PAGE_SIZE, x, dtype=spec.cache_torch_dtype, device=device)
    v_pool = torch.empty(spec.num_pages, Hk, D, PAGE_SIZE, dtype=spec.cache_torch_dtype, device=device)
    _fill_normal(q, gen, spec.value_scale, chunk_elems)
    k_scale = v_scale = None
    if spec.dtype == "fp8":
        k_scale, v_scale = _fill_fp8(spec, k_pool, v_pool, gen, chunk_elems)
    else:
        _fill_normal(k_pool, gen, spec.value_scale, chunk_elems)
        _fill_normal(v_pool, gen, spec.value_scale, chunk_elems)

    bt = block_tables_for(spec)
    if spec.k_outlier_frac > 0:
        if spec.dtype == "fp8":
            raise ValueError("K outlier rows are drawn for bf16/fp32 caches only")
        _scale_k_outliers(spec, k_pool, bt)

    q_start = np.zeros(spec.num_prefill + 1, dtype=np.int32)
    q_start[1:] = np.cumsum(np.asarray(spec.prefill_q_len, dtype=np.int64))
    return HybridBatch(
        spec=spec, q=q, k_pool=k_pool, v_pool=v_pool,
        block_tables=torch.from_numpy(bt).to(device),
        block_tables_host=bt,
        prefill_q_start=q_start,
        prefill_ctx_len=np.asarray(spec.prefill_ctx_len, dtype=np.int32),
        decode_ctx_len=np.asarray(spec.decode_ctx_len, dtype=np.int32),
        k_scale=k_scale, v_scale=v_scale,
    )


def _fill_fp8(spec: BatchSpec, k_pool: torch.Tensor, v_pool: torch.Tensor, gen: torch.Generator,
              chunk_elems: int):
    """FP8 cache: one scale per (page, KV head) slab for K and for V, powers of two 2^-3 .. 2^0
    drawn by numpy PCG64(seed + 2); each slab holds N(0,1) * value_scale / its scale, converted to
    OCP E4M3 codes by torch's float8_e4m3fn cast (round to nearest even), K pool then V pool."""
    P, Hk = spec.num_pages, spec.num_kv_heads
    rng = np.random.Generator(np.random.PCG64(spec.seed + 2))
    dev = k_pool.device
    k_scale = torch.from_numpy(np.exp2(rng.integers(-3, 1, size=(P, Hk))).astype(np.float32)).to(dev)
    v_scale = torch.from_numpy(np.exp2(rng.integers(-3, 1, size=(P, Hk))).astype(np.float32)).to(dev)
    slab = PAGE_SIZE * spec.head_dim
    step = max(1, chunk_elems // (Hk * slab))
    for pool, scale in ((k_pool, k_scale), (v_pool, v_scale)):
        flat = pool.view(P, Hk, slab)
        for a in range(0, P, step):
            b = min(P, a + step)
            x = torch.randn((b - a) * Hk * slab, generator=gen, device=dev, dtype=torch.float32)
            x = x.view(b - a, Hk, slab) * spec.value_scale / scale[a:b, :, None]
            flat[a:b].copy_(x.to(torch.float8_e4m3fn).view(torch.uint8))
    return k_scale, v_scale


def _scale_k_outliers(spec: BatchSpec, k_pool: torch.Tensor, bt: np.ndarray):
    """Multiply exactly floor(frac * N) of the N live K rows (one row = one token's
    D-vector for one KV head) by ``k_outlier_mult``; rows drawn without replacement."""
    ctx = spec.seq_ctx()
    Hk = spec.num_kv_heads
    n_rows = int(sum(ctx)) * Hk
    n_pick = int(math.floor(spec.k_outlier_frac * n_rows))
    if n_pick == 0:
        return
    rng = np.random.Generator(np.random.PCG64(spec.seed + 1_000_003))
    pick = rng.choice(n_rows, size=n_pick, replace=False)
    # row index r = (global_token * Hk + head); global tokens enumerate sequences in order
    starts = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int64)
    tok = pick // Hk
    head = pick % Hk
    seq = np.searchsorted(starts, tok, side="right") - 1
    t = tok - starts[seq]
    page = bt[seq, t // PAGE_SIZE].astype(np.int64)
    slot = t % PAGE_SIZE
    rows = k_rows_view(k_pool)
    dev = k_pool.device
    pi = torch.from_numpy(page).to(dev)
    hi = torch.from_numpy(head).to(dev)
    si = torch.from_numpy(slot).to(dev)
    rows[pi, hi, si] = rows[pi, hi, si] * spec.k_outlier_mult


def poison_unused(batch: HybridBatch, value=float("nan")):
    """Fill every pool slot that no live token of the batch owns with ``value`` (NaN by
    default): whole unused pages and the slots past ``ctx`` in each sequence's last page."""
    spec = batch.spec
    bt = batch.block_tables_host
    used = np.zeros(spec.num_pages, dtype=bool)
    for s, c in enumerate(spec.seq_ctx()):
        used[bt[s, : -(-c // PAGE_SIZE)]] = True
    if spec.dtype == "fp8":
        value = 0x7F                        # an E4M3 NaN code
    unused = torch.from_numpy(np.nonzero(~used)[0]).to(batch.k_pool.device)
    if unused.numel():
        batch.k_pool[unused] = value
        batch.v_pool[unused] = value
    kr, vr = k_rows_view(batch.k_pool), v_rows_view(batch.v_pool)
    for s, c in enumerate(spec.seq_ctx()):
        if c % PAGE_SIZE:
            p = int(bt[s, (c - 1) // PAGE_SIZE])
            kr[p, :, c % PAGE_SIZE:] = value
            vr[p, :, c % PAGE_SIZE:] = value


def custom_spec(dtype="bf16", Hq=4, Hkv=2, D=128, prefill=((16, 40),), decode=(37,),
                seed=11, pool_slack=5, **kw) -> BatchSpec:
    """A small batch for tests: ``prefill`` holds (q_len, ctx) pairs, ``decode`` contexts."""
    pq = [int(a) for a, _ in prefill]
    pc = [int(b) for _, b in prefill]
    dec = [int(c) for c in decode]
    live = sum(-(-c // PAGE_SIZE) for c in pc + dec)
    return BatchSpec(f"custom-{dtype}-{Hq}-{Hkv}-{D}", dtype, Hq, Hkv, D, pq, pc, dec,
                     num_pages=max(1, live + pool_slack), seed=seed,
                     value_scale=kw.pop("value_scale", 1.0 if dtype == "fp32" else 0.5), **kw)


def new_tokens(spec: BatchSpec, seed: int, device="cpu"):
    """The step's new keys and values, k_new and v_new [total_q, Hkv, D] in the batch's dtype
    (rows in query-row order), drawn N(0,1) * value_scale from a torch generator seeded with
    ``seed`` (k_new first, then v_new)."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    shape = (spec.total_q, spec.num_kv_heads, spec.head_dim)
    k_new = torch.empty(shape, dtype=spec.torch_dtype, device=device)
    v_new = torch.empty(shape, dtype=spec.torch_dtype, device=device)
    _fill_normal(k_new, gen, spec.value_scale, 1 << 28)
    _fill_normal(v_new, gen, spec.value_scale, 1 << 28)
    return k_new, v_new
