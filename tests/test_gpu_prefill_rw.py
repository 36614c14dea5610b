"""The register-weight prefill kernel (long token batches, at least ~one
round of 256 x 256 output tiles) against the float64 oracle on the identical
dequantised weights: |Y - Y64| <= 2e-3 * sum|x||w~| + 1e-5 on every output.
Shapes with ragged feature and token tails, all three group sizes, and a K
that spans several stages."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import check_linear, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mq():
    return require_gpu()


def _layer(N, K, seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, rng.choice(K, 3, replace=False)] *= 20
    return W.astype(np.float16)


# (N, K, G, M): N = 4000 leaves the last feature tile 160 rows (10 row blocks)
# and M = 3300 the last token tile 228 tokens; 16 x 13 tiles each
CASES = [(4096, 256, 128, 3328), (4000, 384, 64, 3300), (4096, 512, 32, 3200)]


@pytest.mark.parametrize("N,K,G,M", CASES)
def test_prefill_register_weights_every_output(mq, N, K, G, M):
    W = _layer(N, K, seed=N + K + G)
    p = mq.mq_pack(to_dev(W), G, 0.0)
    Wt = oracle.dequant(oracle.pack(W, G, 0.0))
    X = np.random.default_rng(M).standard_normal((M, K)).astype(np.float16)
    print(f"[prefill rw] N={N} K={K} G={G} M={M}", flush=True)
    Y = mq.mq_linear_with(to_dev(X), p, mq.KERNEL_GEMM).cpu().numpy()
    check_linear(Y, X, Wt, f"prefill rw N={N} K={K} G={G} M={M}")
    # deterministic
    Y2 = mq.mq_linear_with(to_dev(X), p, mq.KERNEL_GEMM).cpu().numpy()
    assert np.array_equal(Y.view(np.uint16), Y2.view(np.uint16))
