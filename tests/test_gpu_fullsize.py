"""The seeded workloads at their full sizes, in the launch configuration the
benchmark times, against the CPU oracle:

* the 70B-shaped MLP (W 28672x8192, rho 1 %): mq_pack bit-exact, and the
  prefill GEMM at M = 512 and 2048 on every output (the oracle's float64
  product, a chunk of token rows at a time);
* the seven linears of one 4096-hidden transformer block at M = 16, run back
  to back on one stream: packing bit-exact and every output checked;
* the residual sweep at 14336x4096 (outlier placement x density): packing
  bit-exact, and the linear at M = 1, 64 and 512 (sampled at 512).

The oracle packs each layer itself (expected values come only from oracle/).
The prefill layer needs about 9 GB of host memory and 30 s of CPU time.
"""
import numpy as np
import pytest

import oracle
from bit_gemm_amd import synth
from tests.gpu_util import assert_canonical_equal, check_linear, gpu_canonical, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mq():
    return require_gpu()


def _sampled_check(mq, p, X16, Wt, kernel, what, n_feat=192, n_tok=6, seed=0):
    """Run the kernel on all of X, then compare every token at n_feat output
    features (always including the first and last 16) and every feature at
    n_tok tokens (always including the first and last) with the oracle."""
    import torch
    M, N = X16.shape[0], Wt.shape[0]
    Y = mq.mq_linear_with(to_dev(X16), p, kernel)
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    rng = np.random.default_rng(seed)
    feats = np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N),
                                      rng.choice(N, min(N, n_feat), replace=False)]))
    toks = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, n_tok), replace=False)]))
    check_linear(Y[:, feats], X16, Wt[feats], f"{what} features {feats.size} x all tokens")
    check_linear(Y[toks, :], X16[toks], Wt, f"{what} tokens {toks.tolist()} x all features")


def _full_check(mq, p, X16, Wt, kernel, what, chunk=256):
    """Run the kernel on all of X and compare every output with the oracle,
    token rows in chunks (the float64 products of a chunk at a time)."""
    import torch
    Y = mq.mq_linear_with(to_dev(X16), p, kernel)
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    for m0 in range(0, X16.shape[0], chunk):
        check_linear(Y[m0:m0 + chunk], X16[m0:m0 + chunk], Wt, f"{what} tokens {m0}..{m0 + chunk - 1}")


@pytest.mark.timeout(900)
def test_prefill_layer_full_size(mq):
    wl = synth.WORKLOADS["prefill-28672x8192"]
    layer = wl.layers[0]
    print(f"[full size] {wl.name}: pack", flush=True)
    W = layer.W()
    p, got = gpu_canonical(mq, W, layer.group, layer.rho)
    ref = oracle.pack(W, layer.group, layer.rho)
    del W
    assert p.nnz == ref["nnz"] == oracle.budget(layer.rho, layer.N, layer.K)
    assert_canonical_equal(got, ref)
    del got
    Wt = oracle.dequant(ref)
    del ref
    for M in wl.batch:
        print(f"[full size] {wl.name}: GEMM M={M}, every output", flush=True)
        _full_check(mq, p, layer.X(M), Wt, mq.KERNEL_GEMM, f"{wl.name} M={M}")
    p.free()


@pytest.mark.timeout(600)
def test_transformer_block_linears_back_to_back(mq):
    import torch
    wl = synth.WORKLOADS["block-4096h"]
    M = wl.batch[0]
    packed, refs, xs = [], [], []
    for layer in wl.layers:
        print(f"[full size] {wl.name}/{layer.name} {layer.N}x{layer.K}: pack", flush=True)
        W = layer.W()
        p, got = gpu_canonical(mq, W, layer.group, layer.rho)
        ref = oracle.pack(W, layer.group, layer.rho)
        assert_canonical_equal(got, ref)
        packed.append(p)
        refs.append(oracle.dequant(ref))
        xs.append(layer.X(M))
    # the seven launches back to back on one stream, one synchronisation
    ys = [mq.mq_linear(to_dev(x), p) for x, p in zip(xs, packed)]
    torch.cuda.synchronize()
    for layer, y, x, Wt in zip(wl.layers, ys, xs, refs):
        check_linear(y.cpu().numpy(), x, Wt, f"{wl.name}/{layer.name} M={M}")
    for p in packed:
        p.free()


SWEEP = [(mode, rho) for mode, _ in synth.SWEEP_MODES for rho in synth.SWEEP_RHOS]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("mode,rho", SWEEP)
def test_residual_sweep_layer(mq, mode, rho):
    layer = synth.sweep_layer(mode, rho)
    print(f"[full size] sweep {mode} rho={rho}: pack", flush=True)
    W = layer.W()
    p, got = gpu_canonical(mq, W, layer.group, layer.rho)
    ref = oracle.pack(W, layer.group, layer.rho)
    assert p.nnz == ref["nnz"]
    assert_canonical_equal(got, ref)
    Wt = oracle.dequant(ref)
    for M in synth.SWEEP_BATCH:
        print(f"[full size] sweep {mode} rho={rho}: linear M={M}", flush=True)
        X = layer.X(M)
        if M <= 64:
            y = mq.mq_linear(to_dev(X), p).cpu().numpy()
            check_linear(y, X, Wt, f"sweep {mode} rho={rho} M={M}")
        else:
            _sampled_check(mq, p, X, Wt, mq.KERNEL_AUTO, f"sweep {mode} rho={rho} M={M}", n_feat=128, seed=M)
    p.free()
