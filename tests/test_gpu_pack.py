"""GPU packer vs the CPU oracle: canonical arrays must match bit for bit."""
import numpy as np
import pytest

import oracle
from bit_gemm_amd import synth
from tests.gpu_util import assert_canonical_equal, gpu_canonical, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mq():
    return require_gpu()


def _matrix(kind, N, K, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
        W[:, rng.choice(K, max(1, K // 64), replace=False)] *= 20
    elif kind == "ties":
        W = rng.choice(np.array([0.0, 0.25, -0.25, 0.3, 0.31, 1.0, -2.0]), size=(N, K)).astype(np.float16)
    elif kind == "grid":
        W = (rng.integers(-40, 41, size=(N, K)) / 16.0).astype(np.float16)
    elif kind == "tiny":          # subnormal scales and clamped codes
        W = (rng.standard_normal((N, K)) * 3e-7).astype(np.float16)
    elif kind == "wide":          # large magnitudes, still below the fp16 overflow guard
        W = (rng.standard_normal((N, K)) * 3000).astype(np.float16)
    else:
        raise ValueError(kind)
    return W


CASES = [
    (16, 128, 128, 0.05, "normal"),
    (17, 96, 32, 0.1, "normal"),         # ragged rows, K below one tile
    (33, 192, 64, 0.3, "ties"),
    (5, 64, 32, 1.0, "normal"),
    (40, 256, 128, 0.0, "normal"),
    (48, 384, 128, 0.02, "grid"),
    (100, 640, 32, 0.01, "ties"),
    (31, 4224, 128, 0.004, "normal"),    # two 4096-column windows, ragged tile
    (64, 512, 64, 0.2, "tiny"),
    (24, 256, 128, 0.1, "wide"),
    (3, 65536, 128, 0.001, "normal"),    # widest K the column index allows
]


@pytest.mark.parametrize("N,K,G,rho,kind", CASES)
def test_pack_matches_oracle_bit_exact(mq, N, K, G, rho, kind):
    print(f"[pack parity] N={N} K={K} G={G} rho={rho} kind={kind}", flush=True)
    W = _matrix(kind, N, K, seed=N * 1000 + K)
    p, got = gpu_canonical(mq, W, G, rho)
    ref = oracle.pack(W, G, rho)
    assert p.nnz == ref["nnz"]
    assert_canonical_equal(got, ref)


def test_pack_hand_example(mq):
    """The packing derived by hand in tests/golden/hand_2x64_g32.json, every
    array of it, and the oracle's pack of the same matrix."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "hand_2x64_g32.json")) as fh:
        g = json.load(fh)
    W = np.zeros((g["N"], g["K"]), dtype=np.float16)
    for i, j, v in g["W_nonzero"]:
        W[i, j] = v
    rho = g["rho_num"] / g["rho_den"]
    p, got = gpu_canonical(mq, W, g["G"], rho)
    ex = g["expected"]
    assert got["scales"].view(np.uint16).tolist() == ex["scales_fp16_bits"]
    assert [bytes(r).hex() for r in got["codes"]] == ex["codes_hex"]
    assert p.nnz == ex["nnz"]
    assert got["row_ptr"].tolist() == ex["row_ptr"]
    assert got["col"].view(np.uint16).tolist() == ex["col"]
    assert got["rscale"].view(np.uint32).tolist() == ex["rscale_fp32_bits"]
    assert got["rcodes"].tolist() == ex["rcodes"]
    assert_canonical_equal(got, oracle.pack(W, g["G"], rho))


@pytest.mark.parametrize("name", ["tiny-1024x1024", "decode-11008x4096"])
def test_pack_workload_layers_bit_exact(mq, name):
    layer = synth.WORKLOADS[name].layers[0]
    print(f"[pack parity] workload {name} N={layer.N} K={layer.K} rho={layer.rho}", flush=True)
    W = layer.W()
    p, got = gpu_canonical(mq, W, layer.group, layer.rho)
    ref = oracle.pack(W, layer.group, layer.rho)
    assert p.nnz == ref["nnz"] == oracle.budget(layer.rho, layer.N, layer.K)
    assert_canonical_equal(got, ref)
    # device bytes over the plain handle (which reserves the same room for
    # the row blocks' padding entries): the canonical CSR (2.5 B per entry)
    # and the two tile-ordered streams the kernels read (4 B per entry each),
    # 1.10 x the plain handle on the decode layer at rho = 0.5 %
    plain = mq.mq_pack(to_dev(W), layer.group, 0.0)
    extra = p.device_bytes - plain.device_bytes
    assert extra <= 10.5 * p.nnz + 64, (extra, p.nnz)
    if name == "decode-11008x4096":
        assert p.device_bytes / plain.device_bytes <= 1.105
    plain.free()


def test_pack_is_deterministic(mq):
    W = synth.WORKLOADS["tiny-1024x1024"].layers[0].W()
    _, a = gpu_canonical(mq, W, 128, 0.05)
    _, b = gpu_canonical(mq, W, 128, 0.05)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_tiled_layout_round_trips_to_canonical(mq):
    """The kernels' tile layout and residual stream hold exactly the canonical
    codes and entries (with the documented nibble order and corrections)."""
    N, K, G, rho = 37, 4224, 64, 0.01
    W = _matrix("normal", N, K, 7)
    p, got = gpu_canonical(mq, W, G, rho)
    ref = oracle.pack(W, G, rho)
    t = {k: v.cpu().numpy() for k, v in mq.mq_export_tiled(p).items()}
    Nb, Kt = -(-N // 16), -(-K // 128)
    tiles = t["tiles"].reshape(Nb, Kt, 64, 4, 4)          # [rb, kt, lane, dword, byte]
    words = tiles.view(np.uint32).reshape(Nb, Kt, 64, 4)
    q = ref["q"].astype(np.int16)
    for i in range(N):
        rb, r = divmod(i, 16)
        for j in range(0, K, 7):
            kt, rem = divmod(j, 128)
            t4, rem32 = divmod(rem, 32)          # dword t4 holds columns 32 t4 + 8 g + c
            g, c = divmod(rem32, 8)
            nib = int((words[rb, kt, r + 16 * g, t4] >> (4 * ((c >> 1) + 4 * (c & 1)))) & 0xF)
            assert nib - 8 == q[i, j]
    # stream: same entries as the CSR, grouped by (row block, tile)
    tp = t["tile_ptr"].astype(np.int64)
    ent = t["entries"].view(np.uint32)
    assert tp[0] == 0 and tp[-1] == ent.size
    for rb in range(Nb):            # whole 32-entry chunks per row block
        assert (tp[(rb + 1) * Kt] - tp[rb * Kt]) % 32 == 0
    sel_pos = {int(v): n for n, v in enumerate(ref["sel"].tolist())}
    sr = ref["sr"].astype(np.float64)
    qr = ref["qr"].astype(np.float64)
    seen = set()
    for rb in range(Nb):
        for kt in range(Kt):
            seg = ent[tp[rb * Kt + kt]:tp[rb * Kt + kt + 1]]
            keys = []
            real = seg[:len(seg)]
            if kt == Kt - 1:         # the row block's zero padding sits at its end
                nz = len(seg)
                while nz > 0 and seg[nz - 1] == 0:
                    nz -= 1
                real = seg[:nz]
            for e in real.tolist():
                r, jl, dbits = (e >> 12) & 15, e & 0xFFF, e >> 16
                i = 16 * rb + r
                j = (kt * 128 // 4096) * 4096 + jl
                assert j // 128 == kt
                keys.append((i, j))
                # the stored value is the residual sr * qr rounded to fp16
                val = sr[i] * qr[sel_pos[i * K + j]]
                delta = float(np.array([dbits], np.uint16).view(np.float16)[0])
                assert delta == float(np.float16(val)) or abs(delta - val) <= 2 ** -11 * abs(val) + 2 ** -24
                seen.add(i * K + j)
            assert keys == sorted(keys)
    assert seen == set(ref["sel"].tolist())


def test_pack_rejects_nonfinite_and_overflowing_scales(mq):
    W = _matrix("normal", 16, 128, 3)
    W[3, 5] = np.inf
    with pytest.raises(mq.MQError) as ei:
        mq.mq_pack(__import__("tests.gpu_util", fromlist=["to_dev"]).to_dev(W), 128, 0.1)
    assert ei.value.code == -3
    W = _matrix("normal", 16, 128, 3)
    W[2, 7] = np.float16(65504.0)          # fp16(65504/7) = 9360 and 7 * 9360 overflows fp16
    with pytest.raises(mq.MQError) as ei:
        mq.mq_pack(__import__("tests.gpu_util", fromlist=["to_dev"]).to_dev(W), 128, 0.1)
    assert ei.value.code == -2
