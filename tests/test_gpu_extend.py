"""GPU parity of small-q extends: prefill chunks whose rows x G fit one 16-column block run on
the decode path (a decode is an extend of one token) with a causal limit per column; compared
element by element with the oracle in every mode, with and without KV splits, and against the
same batch planned on the prefill-tile path."""
import sys

import numpy as np
import pytest
import torch

from hybrid_prefill_decode_paged_amd import binding as B
from hybrid_prefill_decode_paged_amd import inputs as gen

from helpers import check_close, check_rows, checked_rows, problem, reference_rows, run_library, to_f64

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


EXTEND_CASES = [
    # (dtype, Hq, Hkv, D, prefill (q_len, ctx) pairs, decode ctx list)
    ("bf16", 8, 2, 128, [(4, 300), (2, 2), (3, 17), (16, 700)], [33, 1000]),        # G=4: up to 4 rows
    ("bf16", 4, 4, 128, [(16, 16), (9, 4100), (2, 35)], [1, 64]),                   # G=1: up to 16 rows
    ("bf16", 16, 2, 64, [(5, 129), (2, 2000), (1, 1)], [700]),                      # G=8: up to 2 rows
    ("bf16", 16, 1, 128, [(3, 50), (1, 300)], [17, 2]),                             # G=16: one row
    ("fp32", 6, 2, 128, [(5, 97), (4, 4), (6, 80)], [300]),                         # G=3: up to 5 rows
    ("fp32", 4, 1, 64, [(4, 600), (100, 400)], [77]),                               # one chunk stays a tile
    ("bf16", 32, 8, 128, [(2, 8192), (2, 5000), (1, 31)], []),                      # extends only
]


@pytest.mark.parametrize("case", range(len(EXTEND_CASES)))
@pytest.mark.parametrize("mode", MODES)
def test_small_q_extends_match_the_oracle(case, mode):
    dt, hq, hkv, d, pre, dec = EXTEND_CASES[case]
    spec = gen.custom_spec(dt, Hq=hq, Hkv=hkv, D=d, prefill=pre, decode=dec, seed=400 + case)
    b = gen.make_batch(spec, "cuda")
    _say(f"extend case={case} mode={mode}")
    out, h, _ = run_library(b, mode=mode)
    st = h.stats()
    assert st["num_small_extends"] == sum(1 for L, _ in pre if 0 < L and L * (hq // hkv) <= 16)
    check_close(to_f64(out), problem(b).full_output(), dt, f"extend{case}/{mode}")


@pytest.mark.parametrize("mode", MODES)
def test_small_q_extends_with_splits(mode):
    """Short splits give the extend pieces several KV splits, so their partials (n_q*G columns
    per split) go through the log-sum-exp merge."""
    spec = gen.custom_spec("bf16", Hq=8, Hkv=2, D=128, prefill=[(4, 1500), (3, 700), (200, 900)],
                           decode=[129, 3000], seed=410)
    b = gen.make_batch(spec, "cuda")
    _say(f"extend splits mode={mode}")
    out, h, _ = run_library(b, mode=mode, decode_split_tokens=128)
    st = h.stats()
    assert st["decode_max_splits"] > 1 and st["num_small_extends"] == 2
    check_close(to_f64(out), problem(b).full_output(), "bf16", f"extend-splits/{mode}")


def test_decode_path_and_tile_path_agree():
    spec = gen.custom_spec("bf16", Hq=16, Hkv=4, D=128, prefill=[(4, 3000), (2, 900), (3, 64)],
                           decode=[500], seed=411)
    b = gen.make_batch(spec, "cuda")
    _say("extend vs tile path")
    o1, h1, _ = run_library(b, mode="fused")
    o2, h2, _ = run_library(b, mode="fused", extend_max_q=-1)
    assert h1.stats()["num_small_extends"] == 3 and h2.stats()["num_small_extends"] == 0
    want = problem(b).full_output()
    check_close(to_f64(o1), want, "bf16", "extend path")
    check_close(to_f64(o2), want, "bf16", "tile path")
    assert np.abs(to_f64(o1) - to_f64(o2)).max() <= 2e-2


@pytest.mark.parametrize("mode", MODES)
def test_speculative_verify_batch_full_size(mode):
    """A Llama-3-8B-shaped verification step at full size in every mode: 128 sequences each
    extending by 4 tokens (4 x G = 16 columns) at contexts of 4K-32K, plus one 2048-token chunk.
    Against the oracle: the first and last row of every tile of the chunk and all 4 rows of every
    4th extend, all heads; every output row written."""
    spec = gen.spec_verify_spec(4)
    b = gen.make_batch(spec, "cuda")
    _say(f"speculative verify full size mode={mode}")
    out, h, _ = run_library(b, mode=mode)
    st = h.stats()
    assert st["num_small_extends"] == 128
    per_seq = checked_rows(b, st["prefill_tile_queries"])
    chunk, extends = per_seq[0], per_seq[1:129]
    per_seq = [chunk] + [(s, list(range(r[0], r[-1] + 1))) for s, r in extends[::4]]
    rows, want = reference_rows(b, per_seq)
    check_rows(out, rows, want, "bf16", f"spec-verify/{mode}")
