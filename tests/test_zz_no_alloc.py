"""mq_linear_noalloc, the entry point for callers that cannot allocate: its
output must equal mq_linear's (same kernels, same split of K, same order of
the partial sums) on consecutive calls that use the library's workspace
array, the second with a smaller input, and stay within the oracle's bound."""
import numpy as np
import pytest

import oracle
from bit_gemm_amd import synth
from tests.gpu_util import check_linear, require_gpu, to_dev

# (N, K, rho, M): both split K across workgroups (few 256-row output tiles),
# so the partial sums go through the workspace; the second call is smaller
CASES = [(14336, 4096, 0.005, 64), (4096, 4096, 0.005, 40)]


@pytest.mark.gpu
def test_noalloc_equals_mq_linear_on_consecutive_calls():
    mq = require_gpu()
    import torch
    for idx, (N, K, rho, M) in enumerate(CASES):
        print(f"noalloc case {idx}: N={N} K={K} rho={rho} M={M}", flush=True)
        W16 = synth.weight(N, K, synth.seed_of(70, idx, 0), synth.seed_of(70, idx, 2), "columns", 8)
        X16 = synth.activations(M, K, synth.seed_of(70, idx, 1))
        p = mq.mq_pack(to_dev(W16), 128, rho)
        X = to_dev(X16)
        ref = mq.mq_linear(X, p)
        Y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        mq.mq_linear_noalloc(X, p, Y)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), ref.view(torch.int16)), f"case {idx}: differs from mq_linear"
        if N * K <= 4096 * 4096:   # the oracle packs this one in seconds
            Wt = oracle.dequant(oracle.pack(W16, 128, rho))
            check_linear(Y.cpu().numpy(), X16, Wt, f"noalloc case {idx}")
        p.free()


@pytest.mark.gpu
def test_noalloc_decode_and_errors():
    mq = require_gpu()
    import torch
    W16 = synth.weight(256, 512, synth.seed_of(71, 0, 0), synth.seed_of(71, 0, 2), "uniform")
    p = mq.mq_pack(to_dev(W16), 64, 0.01)
    for M in (3, 16, 17):   # the decode kernels (no workspace) and the GEMM
        X = to_dev(synth.activations(M, 512, synth.seed_of(71, M, 1)))
        ref = mq.mq_linear(X, p)
        Y = torch.empty_like(ref)
        mq.mq_linear_noalloc(X, p, Y)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), ref.view(torch.int16)), M
    import ctypes
    X = to_dev(synth.activations(4, 512, 1))
    xp = ctypes.c_void_p(X.data_ptr())
    assert mq.lib.mq_linear_noalloc(xp, 0, p.handle, xp, None) == -1                       # M = 0
    assert mq.lib.mq_linear_noalloc(ctypes.c_void_p(X.data_ptr() + 2), 4, p.handle, xp, None) == -1   # misaligned X
    p.free()
    assert mq.lib.mq_linear_noalloc(xp, 4, ctypes.c_void_p(0xDEADBEE0), xp, None) == -6   # not a live handle
