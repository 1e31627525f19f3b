"""ctypes binding of libpod_attn.so: argument marshalling only, same names as the C ABI.

Every step of the attention runs in the library's HIP kernels; nothing here computes.  If the
library is missing, ``load()`` raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
import re
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpod_attn.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "pod_attn.h")

BF16, FP32, FP8_E4M3 = 0, 1, 2
DTYPES = {"bf16": BF16, "fp32": FP32, "fp8": FP8_E4M3}
MODE_FUSED, MODE_SEPARATE, MODE_STREAMS = 0, 1, 2
MODES = {"fused": MODE_FUSED, "separate": MODE_SEPARATE, "streams": MODE_STREAMS}
FLAG_DEBUG_CLAIMS = 1
FLAG_TRACE = 2
DEVICE_ERR_BAD_PAGE = 1
FALLBACK = {"none": 0, "no_prefill": 1, "no_decode": 2, "occupancy": 3, "env": 4}

STATUS = {0: "OK", -1: "ERR_INVALID_ARG", -2: "ERR_UNSUPPORTED", -3: "ERR_WORKSPACE",
          -4: "ERR_HIP", -5: "ERR_NO_DEVICE"}


class PodAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Config(C.Structure):
    _fields_ = [("num_q_heads", C.c_int), ("num_kv_heads", C.c_int), ("head_dim", C.c_int),
                ("page_size", C.c_int), ("dtype", C.c_int), ("mode", C.c_int), ("scale", C.c_float),
                ("decode_split_tokens", C.c_int), ("prefill_split_cap", C.c_int),
                ("wgs_per_cu", C.c_int), ("flags", C.c_int), ("extend_max_q", C.c_int)]


class Batch(C.Structure):
    _fields_ = [("num_prefill", C.c_int), ("prefill_q_start", C.POINTER(C.c_int32)),
                ("prefill_ctx_len", C.POINTER(C.c_int32)), ("num_decode", C.c_int),
                ("decode_ctx_len", C.POINTER(C.c_int32)), ("block_table_stride", C.c_int),
                ("num_pages_in_pool", C.c_int)]


class Stats(C.Structure):
    _fields_ = [(n, C.c_int) for n in (
        "mode_requested", "mode_used", "fallback_reason", "num_prefill_items", "num_decode_items",
        "num_combine_groups", "prefill_tile_cols", "prefill_tile_queries", "prefill_kv_tile",
        "prefill_max_splits", "decode_split_tokens", "decode_max_splits", "grid_wgs", "wgs_per_cu",
        "num_cus", "lds_bytes_per_wg", "vgprs_per_lane")] + [
        ("workspace_bytes", C.c_size_t), ("host_plan_us", C.c_double), ("prefill_wg_budget", C.c_int),
        ("num_append_units", C.c_int), ("num_small_extends", C.c_int),
        ("runs", C.c_uint64), ("runs_fused_path", C.c_uint64), ("fallback_runs", C.c_uint64 * 5),
        ("algorithmic_bytes", C.c_double), ("algorithmic_flops", C.c_double), ("timed_run", C.c_uint64),
        ("kernel_us", C.c_double), ("achieved_gbps", C.c_double), ("achieved_tflops", C.c_double)]

    def as_dict(self):
        d = {n: getattr(self, n) for n, _ in self._fields_}
        d["fallback_runs"] = list(self.fallback_runs)
        return d


class RunDiag(C.Structure):
    _fields_ = [(n, C.c_int) for n in (
        "status_word", "planned_prefill_items", "planned_decode_items", "prefill_items", "decode_items",
        "cus_any", "cus_prefill", "cus_decode", "cus_both", "max_prefill_per_cu", "max_decode_per_cu")] + [
        (n, C.c_double) for n in ("prefill_decode_ratio", "mean_prefill_share", "min_prefill_share",
                                  "max_prefill_share")] + [
        ("run", C.c_uint64), ("timed_run", C.c_uint64)] + [
        (n, C.c_double) for n in ("kernel_us", "achieved_gbps", "achieved_tflops")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class Signals(C.Structure):
    _fields_ = [(n, C.c_int) for n in (
        "prefill_items", "decode_items", "combine_groups", "small_extends", "grid_wgs",
        "lds_bytes_per_wg", "fallback_reason")] + [("workspace_bytes", C.c_size_t)] + [
        (n, C.c_double) for n in ("prefill_flops", "decode_flops", "prefill_bytes", "decode_bytes",
                                  "intensity", "roofline_us")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None


def load(path: str = LIB_PATH):
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is missing: build it with `python -m hybrid_prefill_decode_paged_amd.build`")
    lib = C.CDLL(path)
    P, I, VP = C.POINTER, C.c_int, C.c_void_p
    lib.pod_attn_create.argtypes = [P(Config), P(VP)]
    lib.pod_attn_workspace_size.argtypes = [VP, P(Batch), P(C.c_size_t)]
    lib.pod_attn_run.argtypes = [VP, VP, VP, VP, VP, P(Batch), VP, VP, C.c_size_t, VP]
    lib.pod_attn_run_append.argtypes = [VP, VP, VP, VP, VP, VP, VP, P(Batch), VP, VP, C.c_size_t, VP]
    lib.pod_attn_run_scaled.argtypes = [VP, VP, VP, VP, VP, VP, VP, P(Batch), VP, VP, C.c_size_t, VP]
    lib.pod_attn_run_noalloc.argtypes = [VP, VP, VP, VP, VP, P(Batch), VP, VP]
    lib.pod_attn_get_stats.argtypes = [VP, P(Stats)]
    lib.pod_attn_gather_kv.argtypes = [VP, VP, I, VP, I, I, P(Batch), VP, VP, VP]
    lib.pod_attn_read_run_diagnostics.argtypes = [VP, VP, VP, P(RunDiag)]
    lib.pod_attn_read_device_status.argtypes = [VP, VP, VP, P(C.c_int32), P(C.c_int32), I, P(I),
                                                P(C.c_int32), P(C.c_int32), I]
    lib.pod_attn_plan_inspect.argtypes = [P(Config), P(Batch), I, I, P(C.c_int32), I, P(I), P(Stats)]
    lib.pod_attn_read_trace.argtypes = [VP, VP, VP, P(C.c_uint32), I, P(I)]
    lib.pod_attn_set_kernel_events.argtypes = [VP, VP, VP]
    lib.pod_attn_batch_signals.argtypes = [P(Config), P(Batch), I, I, C.c_double, C.c_double, P(Signals)]
    lib.pod_attn_probe_hbm_read.argtypes = [VP, C.c_size_t, VP, VP]
    lib.pod_attn_probe_mfma.argtypes = [I, VP, P(C.c_double), VP]
    lib.pod_attn_last_error.restype = C.c_char_p
    lib.pod_attn_destroy.argtypes = [VP]
    lib.pod_attn_destroy.restype = None
    for name in ("pod_attn_create", "pod_attn_workspace_size", "pod_attn_run", "pod_attn_run_append",
                 "pod_attn_run_scaled", "pod_attn_get_stats",
                 "pod_attn_gather_kv", "pod_attn_read_device_status", "pod_attn_plan_inspect", "pod_attn_read_trace",
                 "pod_attn_set_kernel_events", "pod_attn_batch_signals", "pod_attn_probe_hbm_read",
                 "pod_attn_probe_mfma", "pod_attn_read_run_diagnostics", "pod_attn_run_noalloc"):
        getattr(lib, name).restype = C.c_int
    _lib = lib
    return lib


def header_functions(header: str = HEADER):
    """Names of the functions include/pod_attn.h declares."""
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:pod_attn_status|void|const char\*)\s+(pod_attn_\w+)\s*\(",
                                 text, flags=re.M)))


def _check(status: int):
    if status != 0:
        msg = load().pod_attn_last_error()
        raise PodAttnError(status, msg.decode() if msg else "")


def make_config(num_q_heads, num_kv_heads, head_dim, dtype="bf16", mode="fused", scale=0.0,
                decode_split_tokens=0, prefill_split_cap=0, wgs_per_cu=0, flags=0, extend_max_q=0) -> Config:
    return Config(num_q_heads, num_kv_heads, head_dim, 16, DTYPES[dtype] if isinstance(dtype, str) else int(dtype),
                  MODES[mode] if isinstance(mode, str) else int(mode), float(scale),
                  int(decode_split_tokens), int(prefill_split_cap), int(wgs_per_cu), int(flags),
                  int(extend_max_q))


class BatchMeta:
    """Host metadata of one batch, kept alive while the C structure points into it."""

    def __init__(self, prefill_q_start, prefill_ctx_len, decode_ctx_len, block_table_stride,
                 num_pages_in_pool):
        self.q_start = np.ascontiguousarray(prefill_q_start, dtype=np.int32)
        self.p_ctx = np.ascontiguousarray(prefill_ctx_len, dtype=np.int32)
        self.d_ctx = np.ascontiguousarray(decode_ctx_len, dtype=np.int32)
        if len(self.q_start) == 0:
            self.q_start = np.zeros(1, dtype=np.int32)
        ptr = lambda a: a.ctypes.data_as(C.POINTER(C.c_int32))
        self.c = Batch(len(self.p_ctx), ptr(self.q_start), ptr(self.p_ctx), len(self.d_ctx),
                       ptr(self.d_ctx), int(block_table_stride), int(num_pages_in_pool))

    @property
    def total_q(self):
        return int(self.q_start[len(self.p_ctx)]) + len(self.d_ctx)

    @classmethod
    def from_batch(cls, b):
        return cls(b.prefill_q_start, b.prefill_ctx_len, b.decode_ctx_len,
                   b.block_tables_host.shape[1], b.spec.num_pages)


def plan_inspect(cfg: Config, meta: BatchMeta, num_cus: int, wgs_per_cu: int):
    """Host-only planning (no GPU): (items [n, 16] int32, stats dict)."""
    lib = load()
    n = C.c_int(0)
    st = Stats()
    _check(lib.pod_attn_plan_inspect(C.byref(cfg), C.byref(meta.c), num_cus, wgs_per_cu, None, 0,
                                     C.byref(n), C.byref(st)))
    items = np.zeros((max(1, n.value), 16), dtype=np.int32)
    _check(lib.pod_attn_plan_inspect(C.byref(cfg), C.byref(meta.c), num_cus, wgs_per_cu,
                                     items.ctypes.data_as(C.POINTER(C.c_int32)), n.value,
                                     C.byref(n), None))
    return items[: n.value], st.as_dict()


PROBE_WGS = 4096          # workgroups of either probe (pod_attn_probe_*)
NOALLOC_SCRATCH_BYTES = 256 << 20   # pod_attn_run_noalloc's per-GPU scratch


def probe_hbm_read(buf, sink, stream=None) -> None:
    """pod_attn_probe_hbm_read: one streaming read of the device tensor buf; sink is a device
    uint32 (int32) tensor of PROBE_WGS elements receiving per-workgroup XORs of the words read."""
    _check(load().pod_attn_probe_hbm_read(_ptr(buf), int(buf.numel() * buf.element_size()), _ptr(sink),
                                          _stream_handle(stream)))


def probe_mfma(iters: int, sink, stream=None) -> float:
    """pod_attn_probe_mfma: dense bf16 MFMA work; sink is a device float tensor of 4*PROBE_WGS
    elements (each receives 8*iters).  Returns the FLOPs performed."""
    flops = C.c_double(0.0)
    _check(load().pod_attn_probe_mfma(int(iters), _ptr(sink), C.byref(flops), _stream_handle(stream)))
    return flops.value


def batch_signals(cfg: Config, meta: BatchMeta, num_cus: int, wgs_per_cu: int, peak_gbps: float = 0.0,
                  peak_tflops: float = 0.0) -> dict:
    """Host-only scheduler signals of a batch (pod_attn_batch_signals): work items, LDS, per-share
    FLOPs and bytes, intensity and the roofline time at the given peaks (0: MI355X's)."""
    out = Signals()
    _check(load().pod_attn_batch_signals(C.byref(cfg), C.byref(meta.c), int(num_cus), int(wgs_per_cu),
                                         float(peak_gbps), float(peak_tflops), C.byref(out)))
    return out.as_dict()


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


class PodAttention:
    """One library handle (one head configuration) on the current HIP device."""

    def __init__(self, num_q_heads, num_kv_heads, head_dim, dtype="bf16", mode="fused", scale=0.0,
                 decode_split_tokens=0, prefill_split_cap=0, wgs_per_cu=0, flags=0, extend_max_q=0):
        self.lib = load()
        self.cfg = make_config(num_q_heads, num_kv_heads, head_dim, dtype, mode, scale,
                               decode_split_tokens, prefill_split_cap, wgs_per_cu, flags, extend_max_q)
        h = C.c_void_p()
        _check(self.lib.pod_attn_create(C.byref(self.cfg), C.byref(h)))
        self.h = h
        self.dtype = dtype

    def close(self):
        if getattr(self, "h", None):
            self.lib.pod_attn_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_size(self, meta: BatchMeta) -> int:
        n = C.c_size_t(0)
        _check(self.lib.pod_attn_workspace_size(self.h, C.byref(meta.c), C.byref(n)))
        return n.value

    def check_buffers(self, q, k_cache, v_cache, block_tables, meta: BatchMeta, out):
        """Host-side shape checks of the caller's tensors against what the kernels will read."""
        c = self.cfg
        q_elem = 4 if c.dtype == FP32 else 2
        kv_elem = {BF16: 2, FP32: 4, FP8_E4M3: 1}[c.dtype]
        want_q = meta.total_q * c.num_q_heads * c.head_dim
        pool = meta.c.num_pages_in_pool * c.num_kv_heads * 16 * c.head_dim
        n_seq = len(meta.p_ctx) + len(meta.d_ctx)
        for name, t, n, elem in (("q", q, want_q, q_elem), ("out", out, want_q, q_elem),
                                 ("k_cache", k_cache, pool, kv_elem), ("v_cache", v_cache, pool, kv_elem)):
            if t.element_size() != elem or t.numel() < n or not t.is_contiguous():
                raise PodAttnError(-1, f"{name}: need a contiguous tensor of >= {n} {elem}-byte elements, "
                                       f"got {tuple(t.shape)} {t.dtype}")
        if block_tables.element_size() != 4 or block_tables.numel() < n_seq * meta.c.block_table_stride \
                or not block_tables.is_contiguous():
            raise PodAttnError(-1, f"block_tables: need >= {n_seq}x{meta.c.block_table_stride} int32")

    def run(self, q, k_cache, v_cache, block_tables, meta: BatchMeta, out, workspace, stream=None):
        """pod_attn_run on device tensors; asynchronous on ``stream`` (default: torch's current)."""
        if meta.total_q:
            self.check_buffers(q, k_cache, v_cache, block_tables, meta, out)
        _check(self.lib.pod_attn_run(self.h, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                     C.byref(meta.c), _ptr(out), _ptr(workspace),
                                     0 if workspace is None else workspace.numel() * workspace.element_size(),
                                     _stream_handle(stream)))
        return out

    def run_noalloc(self, q, k_cache, v_cache, block_tables, meta: BatchMeta, out, stream=None):
        """pod_attn_run_noalloc: pod_attn_run with the library's fixed per-GPU scratch as the workspace."""
        if meta.total_q:
            self.check_buffers(q, k_cache, v_cache, block_tables, meta, out)
        _check(self.lib.pod_attn_run_noalloc(self.h, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                             C.byref(meta.c), _ptr(out), _stream_handle(stream)))
        return out

    def run_scaled(self, q, k_cache, v_cache, k_scale, v_scale, block_tables, meta: BatchMeta, out, workspace,
                   stream=None):
        """pod_attn_run_scaled (FP8_E4M3 handles): k_scale / v_scale are float32 [pages, Hkv]."""
        if meta.total_q:
            self.check_buffers(q, k_cache, v_cache, block_tables, meta, out)
            want = meta.c.num_pages_in_pool * self.cfg.num_kv_heads
            for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
                if t.element_size() != 4 or t.numel() < want or not t.is_contiguous():
                    raise PodAttnError(-1, f"{name}: need a contiguous float32 tensor of >= {want} elements")
        _check(self.lib.pod_attn_run_scaled(self.h, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                            _ptr(v_scale), _ptr(block_tables), C.byref(meta.c), _ptr(out),
                                            _ptr(workspace),
                                            0 if workspace is None else workspace.numel() * workspace.element_size(),
                                            _stream_handle(stream)))
        return out

    def run_append(self, q, k_new, v_new, k_cache, v_cache, block_tables, meta: BatchMeta, out, workspace,
                   stream=None):
        """pod_attn_run_append on device tensors: writes row r's k_new/v_new [total_q, Hkv, D] into the
        cache at the row's position, then computes attention over the updated cache."""
        if meta.total_q:
            self.check_buffers(q, k_cache, v_cache, block_tables, meta, out)
            c = self.cfg
            want = meta.total_q * c.num_kv_heads * c.head_dim
            for name, t in (("k_new", k_new), ("v_new", v_new)):
                if t.element_size() != k_cache.element_size() or t.numel() < want or not t.is_contiguous():
                    raise PodAttnError(-1, f"{name}: need a contiguous tensor of >= {want} elements of the "
                                           f"cache's type, got {tuple(t.shape)} {t.dtype}")
        _check(self.lib.pod_attn_run_append(self.h, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                            _ptr(block_tables), C.byref(meta.c), _ptr(out), _ptr(workspace),
                                            0 if workspace is None else workspace.numel() * workspace.element_size(),
                                            _stream_handle(stream)))
        return out

    def set_kernel_events(self, ev_start, ev_end):
        """Arm the one-shot profiling events (torch.cuda.Event objects) for the next run."""
        _check(self.lib.pod_attn_set_kernel_events(self.h, C.c_void_p(ev_start.cuda_event),
                                                   C.c_void_p(ev_end.cuda_event)))

    def stats(self) -> dict:
        st = Stats()
        _check(self.lib.pod_attn_get_stats(self.h, C.byref(st)))
        return st.as_dict()

    def gather_kv(self, cache, which: int, block_tables, seq: int, ctx: int, meta: BatchMeta, out, stream=None,
                  device_status=None):
        """pod_attn_gather_kv; device_status (a device int32 tensor, optional) receives the bad-page bit."""
        _check(self.lib.pod_attn_gather_kv(self.h, _ptr(cache), int(which), _ptr(block_tables), int(seq),
                                           int(ctx), C.byref(meta.c), _ptr(out), _ptr(device_status),
                                           _stream_handle(stream)))
        return out

    def run_diagnostics(self, workspace, stream=None) -> dict:
        """pod_attn_read_run_diagnostics: synchronises and reads the last run's per-CU claim balance,
        status word and kernel time."""
        d = RunDiag()
        _check(self.lib.pod_attn_read_run_diagnostics(self.h, _ptr(workspace), _stream_handle(stream), C.byref(d)))
        return d.as_dict()

    def read_trace(self, workspace, stream=None) -> np.ndarray:
        """Per-item timeline of the last run (handle created with FLAG_TRACE): uint32 [n, 4] rows
        {start, end, cu_slot, kind} (100 MHz clock), prefill items first."""
        n = C.c_int(0)
        _check(self.lib.pod_attn_read_trace(self.h, _ptr(workspace), _stream_handle(stream), None, 0, C.byref(n)))
        rec = np.zeros((max(1, n.value), 4), dtype=np.uint32)
        _check(self.lib.pod_attn_read_trace(self.h, _ptr(workspace), _stream_handle(stream),
                                            rec.ctypes.data_as(C.POINTER(C.c_uint32)), n.value, C.byref(n)))
        return rec[: n.value]

    def read_device_status(self, workspace, n_items_cap: int = 0, cu_cap: int = 0, stream=None):
        """(status_word, claims[n] or None, (prefill_per_cu, decode_per_cu) or None)."""
        status = C.c_int32(0)
        n = C.c_int(0)
        claims = np.zeros(max(1, n_items_cap), dtype=np.int32)
        pf = np.zeros(max(1, cu_cap), dtype=np.int32)
        dc = np.zeros(max(1, cu_cap), dtype=np.int32)
        ip = lambda a: a.ctypes.data_as(C.POINTER(C.c_int32))
        _check(self.lib.pod_attn_read_device_status(
            self.h, _ptr(workspace), _stream_handle(stream), C.byref(status),
            ip(claims) if n_items_cap else None, n_items_cap, C.byref(n),
            ip(pf) if cu_cap else None, ip(dc) if cu_cap else None, cu_cap))
        return (status.value, claims[: min(n.value, n_items_cap)] if n_items_cap else None,
                (pf[:cu_cap], dc[:cu_cap]) if cu_cap else None)
