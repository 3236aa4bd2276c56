"""The measurement probes the bench's measured peaks come from: their outputs are the
values their definitions fix (so the work they are timed on is really done)."""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_amd as M

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("code,v", [(0x38, 1.0), (0x40, 2.0), (0xB8, -1.0), (0x30, 0.5)])
def test_probe_mfma_fp8_values(code, v):
    iters = 100
    print(f"probe_mfma code=0x{code:02x} iters={iters}", flush=True)
    out = M.moe_probe_mfma_fp8(6, iters, code)
    torch.cuda.synchronize()
    # four accumulators x four values per lane, each iters * 128 products of v * v
    expect = 2048.0 * iters * v * v
    assert out.shape == (6 * 512,)
    assert torch.all(out == expect), (out.min().item(), out.max().item(), expect)


@pytest.mark.parametrize("words,n_blocks", [(4 * 250001, 37), (64, 4096), (1 << 22, 1024)])
def test_probe_hbm_read_xor(words, n_blocks):
    print(f"probe_read words={words} blocks={n_blocks}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(words)
    host = torch.randint(-2**31, 2**31 - 1, (words,), dtype=torch.int32, generator=g)
    buf = host.cuda()
    out = M.moe_probe_hbm_read(buf, n_blocks)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want
