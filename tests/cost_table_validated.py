"""Publish a validated cost table: cost_table.calibrate on the current GPU with the fp64 oracle as
the reference (every head of the first and last prefill row and of the first and last decode row
of each bucket), written as a markdown summary.  Needs a GPU; not a pytest module.

    python tests/cost_table_validated.py OUT.md [--heads 32,8,128] [--steps 5]
"""
import argparse
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

from hybrid_prefill_decode_paged_amd.cost_table import calibrate  # noqa: E402

from helpers import bucket_reference  # noqa: E402


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("out")
    ap.add_argument("--heads", default="32,8,128")
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
                  ints(a.decode_ctxs), steps=a.steps, reference=bucket_reference)
    n_ok = sum(e.validated for e in t.entries)
    cmd = "python tests/cost_table_validated.py " + " ".join(sys.argv[1:])
    lines = [f"# Measured cost table: {hq} query / {hkv} KV heads, head_dim {d}, {a.dtype}, fused mode, one MI355X", "",
             f"Command: `{cmd}` (chunk lengths {a.chunk_lens}; chunk contexts {a.chunk_ctxs}; decode counts "
             f"{a.decode_counts}; decode contexts {a.decode_ctxs}). Each bucket is one prefill chunk of `chunk` rows "
             f"whose context is `chunk ctx`, plus `decodes` decodes at `decode ctx`, run {a.steps} times one step at "
             "a time (synchronised); `step` = wall time of the whole call (planning, plan upload, kernels), "
             "`kernel` = the fused kernel's events, `roofline` = pod_attn_batch_signals at MI355X peaks, "
             "`frac` = roofline / kernel. A bucket is validated when it ran on the fused path with status word 0 "
             "and a finite output, and every head of its first and last prefill row and first and last decode row "
             "matched the fp64 oracle within max abs 2e-2 and mean abs 2e-3 (`max err`, `mean err`).", "",
             f"{n_ok} of {len(t.entries)} buckets validated.", "",
             "| chunk | chunk ctx | decodes | decode ctx | step p50 µs | step max µs | kernel p50 µs | roofline µs "
             "| frac | max err | mean err | validated |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for e in t.entries:
        roof = e.signals["roofline_us"]
        lines.append(f"| {e.chunk_len} | {e.chunk_ctx} | {e.n_decode} | {e.decode_ctx} | {e.step_us_p50} | "
                     f"{e.step_us_max} | {e.kernel_us_p50} | {roof:.1f} | {roof / e.kernel_us_p50:.2f} | "
                     f"{e.max_abs_err:.2e} | {e.mean_abs_err:.2e} | {'yes' if e.validated else 'NO'} |")
    open(a.out, "w").write("\n".join(lines) + "\n")
    print(f"{n_ok}/{len(t.entries)} buckets validated -> {a.out}", flush=True)


if __name__ == "__main__":
    main()
