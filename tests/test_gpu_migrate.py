"""Outlier migration on the GPU (mq_smooth_weights / mq_smooth_activations)
against the CPU oracle (oracle/migrate.py): the exponents and the scaled
weights and activations bit-exact, and the whole path -- migrate, pack,
fused linear on the smoothed activations -- within |Y - Y64| <= 2e-3 *
sum|x^||w~| + 1e-5 of the float64 oracle on the oracle's own packing of W^."""
import numpy as np
import pytest

import oracle
from oracle import migrate as om
from tests.gpu_util import check_linear, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mq():
    return require_gpu()


def _wx(N, K, M, seed, hot=4):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, rng.choice(K, 3, replace=False)] *= 20
    X = rng.standard_normal((M, K)).astype(np.float32)
    X[:, rng.choice(K, hot, replace=False)] *= 50
    return W.astype(np.float16), X.astype(np.float16)


@pytest.mark.parametrize("N,K,M", [(16, 128, 4), (37, 384, 9), (300, 4096, 16), (5, 8256, 3)])
def test_smoothing_bit_exact(mq, N, K, M):
    W, X = _wx(N, K, M, N + K)
    ax = np.abs(X.astype(np.float32)).max(axis=0)
    ax[::7] = 0.0                               # channels without activations keep e = 0
    Wh, e = mq.mq_smooth_weights(to_dev(W), to_dev(ax))
    Wr, er = om.migrate(W, ax)
    assert np.array_equal(e.cpu().numpy(), er)
    assert np.array_equal(Wh.cpu().numpy().view(np.uint16), Wr.view(np.uint16))
    Xh = mq.mq_smooth_activations(to_dev(X), e).cpu().numpy()
    assert np.array_equal(Xh.view(np.uint16), om.smooth_activations(X, er).view(np.uint16))


def test_subnormals_and_in_place(mq):
    # tiny weights pushed below the normal range round half to even, as the oracle
    K = 64
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((8, K)) * 2.0 ** -12).astype(np.float16)
    ax = np.full(K, 2.0 ** -20, dtype=np.float32)   # pulls e strongly negative
    Wd = to_dev(W)
    Wh, e = mq.mq_smooth_weights(Wd, to_dev(ax))
    Wr, er = om.migrate(W, ax)
    assert np.array_equal(e.cpu().numpy(), er) and er.min() < -2
    assert np.array_equal(Wh.cpu().numpy().view(np.uint16), Wr.view(np.uint16))
    # in place: W_out = W
    import ctypes
    ed = e.clone()
    axd = to_dev(ax)
    assert mq.lib.mq_smooth_weights(ctypes.c_void_p(Wd.data_ptr()), 8, K, ctypes.c_void_p(axd.data_ptr()),
                                    ctypes.c_void_p(Wd.data_ptr()), ctypes.c_void_p(ed.data_ptr()), None) == 0
    assert np.array_equal(Wd.cpu().numpy().view(np.uint16), Wr.view(np.uint16))


@pytest.mark.parametrize("rho", [0.0, 0.01])
def test_migrated_layer_end_to_end(mq, rho):
    N, K = 256, 4096
    W, Xcal = _wx(N, K, 64, 7)
    ax = np.abs(Xcal.astype(np.float32)).max(axis=0)
    Wh, e = mq.mq_smooth_weights(to_dev(W), to_dev(ax))
    p = mq.mq_pack(Wh, 128, rho)
    Wr, er = om.migrate(W, ax)
    Wt = oracle.dequant(oracle.pack(Wr, 128, rho))
    for M in (1, 16, 64):
        X = np.random.default_rng(M).standard_normal((M, K)).astype(np.float32)
        X[:, np.argsort(-ax)[:4]] *= 50
        X = X.astype(np.float16)
        Xh = mq.mq_smooth_activations(to_dev(X), e)
        Y = mq.mq_linear(Xh, p).cpu().numpy()
        check_linear(Y, om.smooth_activations(X, er), Wt, f"migrated rho={rho} M={M}")


def test_bad_activation_maxima(mq):
    W, X = _wx(16, 128, 2, 3)
    ax = np.abs(X.astype(np.float32)).max(axis=0)
    ax[5] = -1.0
    with pytest.raises(mq.MQError) as ei:
        mq.mq_smooth_weights(to_dev(W), to_dev(ax))
    assert ei.value.code == -1
    ax[5] = np.inf
    with pytest.raises(mq.MQError):
        mq.mq_smooth_weights(to_dev(W), to_dev(ax))
