"""GPU checks of the measurement probes through the C ABI: the HBM read probe reads every byte of
its buffer (the XOR of its per-workgroup results equals the XOR of the buffer's words, computed on
the host), and the MFMA probe's chains give exactly 4 * iters per wave; invalid arguments are
rejected before any launch."""
import sys

import numpy as np
import pytest
import torch

from hybrid_prefill_decode_paged_amd import binding as B

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


@pytest.mark.parametrize("n16", [1, 63, 4096 * 256, 4096 * 256 * 3 + 17])
def test_hbm_read_probe_reads_every_word(n16):
    _say(f"hbm read probe n16={n16}")
    g = torch.Generator(device="cuda")
    g.manual_seed(n16)
    buf = torch.randint(-2**31, 2**31 - 1, (n16 * 4,), dtype=torch.int32, device="cuda", generator=g)
    sink = torch.zeros(B.PROBE_WGS, dtype=torch.int32, device="cuda")
    B.probe_hbm_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32))
    assert got == want


def _xor_all(t):
    """XOR of every 32-bit word of an int32 device tensor, by halving on the device."""
    t = t.flatten()
    while t.numel() > 1:
        h = t.numel() // 2
        r = t[:h] ^ t[h:2 * h]
        t = torch.cat([r, t[2 * h:]]) if t.numel() % 2 else r
    return int(t.item()) & 0xFFFFFFFF


def test_hbm_read_probe_reads_every_word_with_several_blocks_per_wave():
    """Every wave of the 4096 x 4 grid reads two or three 16 KiB blocks, the last one partial for
    some waves: the two-blocks-in-flight loop and its tail."""
    n16 = 4096 * 4 * 1024 * 2 + 4096 * 4 * 512 + 5
    _say(f"hbm read probe n16={n16}")
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    buf = torch.randint(-2**31, 2**31 - 1, (n16 * 4,), dtype=torch.int32, device="cuda", generator=g)
    sink = torch.zeros(B.PROBE_WGS, dtype=torch.int32, device="cuda")
    B.probe_hbm_read(buf, sink)
    torch.cuda.synchronize()
    assert _xor_all(sink) == _xor_all(buf)


@pytest.mark.parametrize("iters", [1, 5, 1000])
def test_mfma_probe_result_is_exact(iters):
    _say(f"mfma probe iters={iters}")
    sink = torch.full((4 * B.PROBE_WGS,), -1.0, dtype=torch.float32, device="cuda")
    flops = B.probe_mfma(iters, sink)
    torch.cuda.synchronize()
    assert torch.all(sink == 8.0 * iters)
    assert flops == B.PROBE_WGS * 4 * 8 * iters * 2 * 32 * 32 * 16


def test_probes_reject_bad_arguments():
    buf = torch.zeros(64, dtype=torch.int32, device="cuda")
    sink = torch.zeros(B.PROBE_WGS, dtype=torch.int32, device="cuda")
    with pytest.raises(B.PodAttnError):
        B.probe_hbm_read(buf[1:4], sink)               # 12 bytes: not a multiple of 16
    with pytest.raises(B.PodAttnError):
        B.probe_mfma(0, sink)
