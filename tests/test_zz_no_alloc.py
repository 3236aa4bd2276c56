"""The allocation-free router entry point (static device scratch) against moe_route with
a caller workspace: identical outputs, bit for bit, on two calls in a row (the second
smaller); and the static scratch covers every shape's partial logits."""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_amd as M
import synth
from gpu_util import dev, note, to_np

SCRATCH = 32 << 20


def _case(T, d, E, k, seed):
    x = synth.normal((T, d), seed, "x", dtype=torch.bfloat16).to(dev())
    w = synth.normal((E, d), seed, "w_gate_router", std=d ** -0.5, dtype=torch.bfloat16).to(dev())
    b = synth.uniform((E,), -0.01, 0.01, seed, "bias").to(dev())
    return x, w, b


@pytest.mark.gpu
def test_route_noalloc_matches_route():
    # the prefill shape fills the 32 MiB scratch exactly (8 planes of 4096 x 256 fp32);
    # the second, smaller call reuses the scratch the first one left behind
    for T, d, E, k, seed in ((4096, 7168, 256, 8, 1), (300, 2048, 64, 6, 2)):
        note(f"route noalloc T={T} d={d} E={E} k={k}")
        assert M.moe_route_workspace_size(T, d, E) <= SCRATCH
        x, w, b = _case(T, d, E, k, seed)
        i0, w0, l0 = M.moe_route(x, w, b, k)
        for renorm in (False, True):
            i1, w1, l1 = M.moe_route_noalloc(x, w, b, k, renorm=renorm)
            i2, w2, l2 = M.moe_route(x, w, b, k, renorm=renorm)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(to_np(l1), to_np(l2))
            np.testing.assert_array_equal(to_np(i1), to_np(i2))
            np.testing.assert_array_equal(to_np(w1).view(np.uint32), to_np(w2).view(np.uint32))
        np.testing.assert_array_equal(to_np(l0), to_np(l1))


def test_route_scratch_covers_every_shape():
    """The router splits its logit product over at most ~256 workgroups of 128 tokens x 256
    experts, so the partial planes never exceed 256 x 128 x 256 fp32 = 32 MiB: the static
    scratch holds them for every accepted shape (its size check never has to refuse)."""
    worst = 0
    for T in (1, 77, 128, 300, 1024, 4096, 8192, 16384, 65536):
        for E in (1, 8, 64, 256, 300, 520, 1024):
            for d in (128, 512, 2048, 7168, 16384):
                worst = max(worst, M.moe_route_workspace_size(T, d, E))
    assert 0 < worst <= SCRATCH, worst
