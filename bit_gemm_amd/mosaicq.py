"""Python binding of include/mosaicq.h (ctypes).

Argument marshalling only: every step of packing and of the fused linear runs
in the HIP library. torch tensors supply device memory and the current HIP
stream. Importing this module fails loudly when the library is not built --
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmosaicq.so")

MQ_OK = 0
STATUS = {
    0: "MQ_OK", -1: "MQ_ERR_INVALID_ARG", -2: "MQ_ERR_UNSUPPORTED", -3: "MQ_ERR_NONFINITE",
    -4: "MQ_ERR_OUT_OF_MEMORY", -5: "MQ_ERR_DEVICE", -6: "MQ_ERR_BAD_HANDLE",
}
KERNEL_AUTO, KERNEL_GEMV, KERNEL_GEMM = 0, 1, 2
GEMV_MAX_M = 64

EXPORTED = ("mq_pack", "mq_linear", "mq_linear_with", "mq_linear_noalloc", "mq_residual_add", "mq_packed_info",
            "mq_export_canonical", "mq_export_tiled", "mq_pack_blocks", "mq_block_count", "mq_export_blocks",
            "mq_smooth_weights", "mq_smooth_activations", "mq_quantize_activations", "mq_linear_a4",
            "mq_stream_read", "mq_concat", "mq_decode_a4", "mq_linear_group", "mq_free",
            "mq_status_string")


class MQError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built (run `python -m bit_gemm_amd.build`)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.mq_pack.argtypes = [vp, i64, i64, i32, ctypes.c_double, vp, ctypes.POINTER(vp)]
    lib.mq_pack.restype = ctypes.c_int
    lib.mq_linear.argtypes = [vp, i64, vp, vp, vp]
    lib.mq_linear.restype = ctypes.c_int
    lib.mq_linear_with.argtypes = [vp, i64, vp, vp, vp, i32]
    lib.mq_linear_with.restype = ctypes.c_int
    lib.mq_linear_noalloc.argtypes = [vp, i64, vp, vp, vp]
    lib.mq_linear_noalloc.restype = ctypes.c_int
    lib.mq_residual_add.argtypes = [vp, i64, vp, vp, vp]
    lib.mq_residual_add.restype = ctypes.c_int
    lib.mq_packed_info.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i32),
                                   ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_size_t)]
    lib.mq_packed_info.restype = ctypes.c_int
    lib.mq_export_canonical.argtypes = [vp] * 8
    lib.mq_export_canonical.restype = ctypes.c_int
    lib.mq_export_tiled.argtypes = [vp] * 5
    lib.mq_export_tiled.restype = ctypes.c_int
    lib.mq_pack_blocks.argtypes = [vp, i64, i64, i32, ctypes.c_double, vp, vp, ctypes.POINTER(vp)]
    lib.mq_pack_blocks.restype = ctypes.c_int
    lib.mq_block_count.argtypes = [vp, ctypes.POINTER(i64)]
    lib.mq_block_count.restype = ctypes.c_int
    lib.mq_export_blocks.argtypes = [vp] * 5
    lib.mq_export_blocks.restype = ctypes.c_int
    lib.mq_smooth_weights.argtypes = [vp, i64, i64, vp, vp, vp, vp]
    lib.mq_smooth_weights.restype = ctypes.c_int
    lib.mq_smooth_activations.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.mq_smooth_activations.restype = ctypes.c_int
    lib.mq_quantize_activations.argtypes = [vp, i64, i64, i32, vp, vp, vp]
    lib.mq_quantize_activations.restype = ctypes.c_int
    lib.mq_linear_a4.argtypes = [vp, vp, i64, vp, vp, vp]
    lib.mq_linear_a4.restype = ctypes.c_int
    lib.mq_stream_read.argtypes = [vp, i64, i32, vp, vp]
    lib.mq_stream_read.restype = ctypes.c_int
    lib.mq_decode_a4.argtypes = [vp, i64, vp, vp, vp]
    lib.mq_decode_a4.restype = ctypes.c_int
    lib.mq_concat.argtypes = [ctypes.POINTER(vp), i32, vp, ctypes.POINTER(vp)]
    lib.mq_concat.restype = ctypes.c_int
    lib.mq_linear_group.argtypes = [ctypes.POINTER(vp), i64, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, vp]
    lib.mq_linear_group.restype = ctypes.c_int
    lib.mq_free.argtypes = [vp]
    lib.mq_free.restype = None
    lib.mq_status_string.argtypes = [ctypes.c_int]
    lib.mq_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


def mq_status_string(code: int) -> str:
    return lib.mq_status_string(int(code)).decode()


def _check(code: int, where: str):
    if code != MQ_OK:
        raise MQError(code, where)


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev_fp16(t, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float16:
        raise TypeError(f"{name} must be a float16 tensor on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


_deferred = []   # handles released while a stream capture was running, freed at the next release


def _capturing() -> bool:
    try:
        import torch
        return torch.cuda.is_available() and torch.cuda.is_current_stream_capturing()
    except Exception:
        return False


def _release(h) -> None:
    """mq_free, except while the current stream is being captured into a HIP
    graph: freeing device memory then would invalidate the capture (a handle
    collected by the garbage collector mid-capture does exactly that), so the
    handle waits for the next release outside a capture."""
    if _capturing():
        _deferred.append(h)
        return
    while _deferred:
        lib.mq_free(_deferred.pop())
    lib.mq_free(h)


class Packed:
    """A packed layer (owns the library handle; freed with free() or on GC)."""

    def __init__(self, handle: ctypes.c_void_p, N: int, K: int, G: int, rho: float):
        self._h = handle
        self.N, self.K, self.G, self.rho = N, K, G, rho
        info = mq_packed_info(self)
        self.nnz = info["nnz"]
        self.device_bytes = info["bytes"]

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise MQError(-6, "packed layer already freed")
        return self._h

    def canonical_bytes(self) -> int:
        """Bytes of the canonical format: codes, fp16 scales, CSR residual."""
        return (self.N * self.K // 2 + 2 * self.N * (self.K // self.G) + 4 * (self.N + 1)
                + 2 * self.nnz + (self.nnz + 1) // 2 + 4 * self.N)

    def free(self):
        if self._h is not None:
            _release(self._h)
            self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def mq_pack(W, group_size: int = 128, residual_density: float = 0.0, stream=None) -> Packed:
    """Pack an fp16 [N, K] device tensor (see mq_pack in include/mosaicq.h)."""
    ptr = _dev_fp16(W, "W")
    if W.dim() != 2:
        raise ValueError("W must be 2-D [N, K]")
    N, K = W.shape
    out = ctypes.c_void_p()
    _check(lib.mq_pack(ptr, N, K, group_size, float(residual_density), _stream_handle(stream),
                       ctypes.byref(out)), "mq_pack")
    return Packed(out, N, K, group_size, float(residual_density))


def mq_concat(parts, stream=None) -> Packed:
    """One handle for several packed layers that read the same input, their
    rows stacked in order (see mq_concat in include/mosaicq.h); the parts
    stay owned by the caller."""
    parts = list(parts)
    arr = (ctypes.c_void_p * len(parts))(*[p.handle for p in parts])
    out = ctypes.c_void_p()
    _check(lib.mq_concat(arr, len(parts), _stream_handle(stream), ctypes.byref(out)), "mq_concat")
    N = sum(p.N for p in parts)
    info_nnz = sum(p.nnz for p in parts)
    return Packed(out, N, parts[0].K, parts[0].G, info_nnz / float(N * parts[0].K))


def mq_pack_blocks(W, group_size: int, block_fraction: float, h, stream=None) -> Packed:
    """Pack with a block-wise residual chosen by the Hessian-guided score (see
    mq_pack_blocks in include/mosaicq.h); h: float32 [K] device tensor."""
    import torch
    ptr = _dev_fp16(W, "W")
    if W.dim() != 2:
        raise ValueError("W must be 2-D [N, K]")
    N, K = W.shape
    if not isinstance(h, torch.Tensor) or not h.is_cuda or h.dtype != torch.float32 or tuple(h.shape) != (K,):
        raise TypeError(f"h must be a float32 [{K}] tensor on the GPU")
    h = h.contiguous()
    out = ctypes.c_void_p()
    _check(lib.mq_pack_blocks(ptr, N, K, group_size, float(block_fraction), ctypes.c_void_p(h.data_ptr()),
                              _stream_handle(stream), ctypes.byref(out)), "mq_pack_blocks")
    p = Packed(out, N, K, group_size, float(block_fraction))
    nb = ctypes.c_int64()
    _check(lib.mq_block_count(p.handle, ctypes.byref(nb)), "mq_block_count")
    p.nblk = nb.value
    return p


def export_blocks(packed: Packed, stream=None) -> dict:
    """The block residual of a handle from mq_pack_blocks as host numpy arrays
    (blk [B], rscale [B, 16], rcodes [B, 16, 64]); synchronises."""
    import torch
    nb = ctypes.c_int64()
    _check(lib.mq_block_count(packed.handle, ctypes.byref(nb)), "mq_block_count")
    B = max(nb.value, 0)
    out = {"blk": torch.empty(max(B, 1), dtype=torch.int32, device="cuda"),
           "rscale": torch.empty((max(B, 1), 16), dtype=torch.float32, device="cuda"),
           "rcodes": torch.empty((max(B, 1), 16, 64), dtype=torch.uint8, device="cuda")}
    _check(lib.mq_export_blocks(packed.handle, *[ctypes.c_void_p(out[k].data_ptr()) for k in
                                                 ("blk", "rscale", "rcodes")], _stream_handle(stream)),
           "mq_export_blocks")
    torch.cuda.synchronize()
    return {k: v.cpu().numpy()[:B] for k, v in out.items()}


def mq_smooth_weights(W, amax_x, stream=None):
    """(W^, e): activation outliers moved into W (see mq_smooth_weights in
    include/mosaicq.h); amax_x: float32 [K] device tensor."""
    import torch
    ptr = _dev_fp16(W, "W")
    N, K = W.shape
    if not isinstance(amax_x, torch.Tensor) or not amax_x.is_cuda or amax_x.dtype != torch.float32 \
            or tuple(amax_x.shape) != (K,):
        raise TypeError(f"amax_x must be a float32 [{K}] tensor on the GPU")
    amax_x = amax_x.contiguous()
    Wh = torch.empty_like(W)
    e = torch.empty(K, dtype=torch.int32, device=W.device)
    _check(lib.mq_smooth_weights(ptr, N, K, ctypes.c_void_p(amax_x.data_ptr()), ctypes.c_void_p(Wh.data_ptr()),
                                 ctypes.c_void_p(e.data_ptr()), _stream_handle(stream)), "mq_smooth_weights")
    return Wh, e


def mq_smooth_activations(X, e, out=None, stream=None):
    """X^ = X 2^-e for the weights from mq_smooth_weights (enqueued, no sync)."""
    import torch
    xp = _dev_fp16(X, "X")
    M, K = X.shape
    if e.dtype != torch.int32 or tuple(e.shape) != (K,) or not e.is_cuda:
        raise TypeError(f"e must be an int32 [{K}] tensor on the GPU")
    out = torch.empty_like(X) if out is None else out
    _check(lib.mq_smooth_activations(xp, M, K, ctypes.c_void_p(e.data_ptr()), _dev_fp16(out, "out"),
                                     _stream_handle(stream)), "mq_smooth_activations")
    return out


def mq_quantize_activations(X, G: int, xq=None, xmeta=None, stream=None):
    """4-bit activation codes of X for mq_linear_a4 (enqueued, no sync).
    Returns (xq uint8 [M, Kp], xmeta int32 [M, Kp / G]), Kp = 128 ceil(K / 128):
    e4m3 codes in tile order, and fp16 scale bits | code sum << 16."""
    import torch
    xp = _dev_fp16(X, "X")
    if X.dim() != 2:
        raise ValueError("X must be [M, K]")
    M, K = X.shape
    Kp = -(-K // 128) * 128
    if xq is None:
        xq = torch.empty((M, Kp), dtype=torch.uint8, device=X.device)
    if xmeta is None:
        xmeta = torch.empty((M, Kp // G), dtype=torch.int32, device=X.device)
    if xq.dtype != torch.uint8 or tuple(xq.shape) != (M, Kp) or not xq.is_contiguous():
        raise TypeError(f"xq must be a contiguous uint8 [{M}, {Kp}] tensor")
    if xmeta.dtype != torch.int32 or tuple(xmeta.shape) != (M, Kp // G) or not xmeta.is_contiguous():
        raise TypeError(f"xmeta must be a contiguous int32 [{M}, {Kp // G}] tensor")
    _check(lib.mq_quantize_activations(xp, M, K, int(G), ctypes.c_void_p(xq.data_ptr()),
                                       ctypes.c_void_p(xmeta.data_ptr()), _stream_handle(stream)),
           "mq_quantize_activations")
    return xq, xmeta


def mq_linear_a4(xq, xmeta, packed: Packed, Y=None, stream=None):
    """Y = X^ (deq(base) + deq(residual))^T from the 4-bit activation codes of
    mq_quantize_activations (enqueued, no sync)."""
    import torch
    M = xq.shape[0]
    Kp = -(-packed.K // 128) * 128
    if xq.dtype != torch.uint8 or tuple(xq.shape) != (M, Kp) or not xq.is_contiguous():
        raise TypeError(f"xq must be a contiguous uint8 [M, {Kp}] tensor")
    if xmeta.dtype != torch.int32 or tuple(xmeta.shape) != (M, Kp // packed.G) or not xmeta.is_contiguous():
        raise TypeError(f"xmeta must be a contiguous int32 [M, {Kp // packed.G}] tensor")
    if Y is None:
        Y = torch.empty((M, packed.N), dtype=torch.float16, device=xq.device)
    yp = _dev_fp16(Y, "Y")
    if tuple(Y.shape) != (M, packed.N):
        raise ValueError(f"Y must be [{M}, {packed.N}]")
    _check(lib.mq_linear_a4(ctypes.c_void_p(xq.data_ptr()), ctypes.c_void_p(xmeta.data_ptr()), M, packed.handle,
                            yp, _stream_handle(stream)), "mq_linear_a4")
    return Y


def mq_decode_a4(X, packed: Packed, Y=None, stream=None):
    """W4A4 decode (up to 2 tokens) in one kernel that quantizes X itself:
    equal to mq_linear_a4(*mq_quantize_activations(X, G), packed) (enqueued,
    no sync)."""
    import torch
    xp = _dev_fp16(X, "X")
    if X.dim() != 2 or X.shape[1] != packed.K:
        raise ValueError(f"X must be [M, {packed.K}]")
    M = X.shape[0]
    if Y is None:
        Y = torch.empty((M, packed.N), dtype=torch.float16, device=X.device)
    yp = _dev_fp16(Y, "Y")
    if tuple(Y.shape) != (M, packed.N):
        raise ValueError(f"Y must be [{M}, {packed.N}]")
    _check(lib.mq_decode_a4(xp, M, packed.handle, yp, _stream_handle(stream)), "mq_decode_a4")
    return Y


def mq_linear_with(X, packed: Packed, kernel: int = KERNEL_AUTO, Y=None, stream=None):
    """Y = X (deq(base) + deq(residual))^T, enqueued on `stream` (no sync)."""
    import torch
    xp = _dev_fp16(X, "X")
    if X.dim() != 2 or X.shape[1] != packed.K:
        raise ValueError(f"X must be [M, {packed.K}]")
    M = X.shape[0]
    if Y is None:
        Y = torch.empty((M, packed.N), dtype=torch.float16, device=X.device)
    yp = _dev_fp16(Y, "Y")
    if tuple(Y.shape) != (M, packed.N):
        raise ValueError(f"Y must be [{M}, {packed.N}]")
    _check(lib.mq_linear_with(xp, M, packed.handle, yp, _stream_handle(stream), int(kernel)), "mq_linear")
    return Y


def mq_linear(X, packed: Packed, Y=None, stream=None):
    return mq_linear_with(X, packed, KERNEL_AUTO, Y, stream)


def mq_linear_noalloc(X, packed: Packed, Y, stream=None):
    """mq_linear without any device allocation (see mq_linear_noalloc in
    include/mosaicq.h): Y must be given. Enqueued on `stream` (no sync)."""
    xp = _dev_fp16(X, "X")
    if X.dim() != 2 or X.shape[1] != packed.K:
        raise ValueError(f"X must be [M, {packed.K}]")
    M = X.shape[0]
    yp = _dev_fp16(Y, "Y")
    if tuple(Y.shape) != (M, packed.N):
        raise ValueError(f"Y must be [{M}, {packed.N}]")
    _check(lib.mq_linear_noalloc(xp, M, packed.handle, yp, _stream_handle(stream)), "mq_linear_noalloc")
    return Y


def mq_linear_group(Xs, packs, Ys=None, stream=None):
    """mq_linear of several layers with their own inputs (one token count),
    one kernel launch when they can share it (see mq_linear_group in
    include/mosaicq.h). Returns the outputs; enqueued on `stream` (no sync)."""
    import torch
    Xs, packs = list(Xs), list(packs)
    if len(Xs) != len(packs) or not packs:
        raise ValueError("one input per layer, at least one layer")
    xps = [_dev_fp16(X, "X") for X in Xs]
    M = Xs[0].shape[0] if Xs[0].dim() == 2 else -1
    for X, p in zip(Xs, packs):
        if X.dim() != 2 or tuple(X.shape) != (M, p.K):
            raise ValueError(f"every X must be [{M}, K] of its layer (K = {p.K})")
    if Ys is None:
        Ys = [torch.empty((M, p.N), dtype=torch.float16, device=Xs[0].device) for p in packs]
    Ys = list(Ys)
    if len(Ys) != len(packs):
        raise ValueError("one output per layer")
    yps = []
    for Y, p in zip(Ys, packs):
        yps.append(_dev_fp16(Y, "Y"))
        if tuple(Y.shape) != (M, p.N):
            raise ValueError(f"every Y must be [{M}, N] of its layer (N = {p.N})")
    n = len(packs)
    xa = (ctypes.c_void_p * n)(*xps)
    ha = (ctypes.c_void_p * n)(*[p.handle for p in packs])
    ya = (ctypes.c_void_p * n)(*yps)
    _check(lib.mq_linear_group(xa, M, ha, ya, n, _stream_handle(stream)), "mq_linear_group")
    return Ys


def mq_residual_add(X, packed: Packed, Y, stream=None):
    """Y <- Y + X R^T with the separate residual kernel (the unfused
    comparison), enqueued on `stream` (no sync). Y is updated in place."""
    xp = _dev_fp16(X, "X")
    if X.dim() != 2 or X.shape[1] != packed.K:
        raise ValueError(f"X must be [M, {packed.K}]")
    M = X.shape[0]
    yp = _dev_fp16(Y, "Y")
    if tuple(Y.shape) != (M, packed.N):
        raise ValueError(f"Y must be [{M}, {packed.N}]")
    _check(lib.mq_residual_add(xp, M, packed.handle, yp, _stream_handle(stream)), "mq_residual_add")
    return Y


def mq_stream_read(src, workgroups: int, sink, stream=None):
    """Read every byte of the device tensor `src` once (measurement helper;
    see mq_stream_read in include/mosaicq.h); sink: int32 [workgroups]."""
    import torch
    if not isinstance(src, torch.Tensor) or not src.is_cuda or not src.is_contiguous():
        raise TypeError("src must be a contiguous GPU tensor")
    if sink.dtype != torch.int32 or sink.numel() < workgroups or not sink.is_cuda:
        raise TypeError(f"sink must be an int32 GPU tensor of at least {workgroups} elements")
    nbytes = src.numel() * src.element_size()
    _check(lib.mq_stream_read(ctypes.c_void_p(src.data_ptr()), nbytes, int(workgroups),
                              ctypes.c_void_p(sink.data_ptr()), _stream_handle(stream)), "mq_stream_read")


def mq_packed_info(packed: Packed) -> dict:
    N, K, nnz = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    G, nbytes = ctypes.c_int32(), ctypes.c_size_t()
    _check(lib.mq_packed_info(packed.handle, ctypes.byref(N), ctypes.byref(K), ctypes.byref(G),
                              ctypes.byref(nnz), ctypes.byref(nbytes)), "mq_packed_info")
    return {"N": N.value, "K": K.value, "G": G.value, "nnz": nnz.value, "bytes": nbytes.value}


def mq_export_canonical(packed: Packed, stream=None, residual: bool = True) -> dict:
    """Canonical arrays as device tensors (synchronises the stream); with
    residual=False only the base codes and scales (all a handle from
    mq_pack_blocks exports here)."""
    import torch
    dev = torch.device("cuda", torch.cuda.current_device())
    N, K, G, nnz = packed.N, packed.K, packed.G, packed.nnz
    out = {
        "codes": torch.empty((N, K // 2), dtype=torch.uint8, device=dev),
        "scales": torch.empty((N, K // G), dtype=torch.float16, device=dev),
    }
    names = ("codes", "scales", "row_ptr", "col", "rcodes", "rscale")
    if residual:
        out.update({
            "row_ptr": torch.empty(N + 1, dtype=torch.int32, device=dev),
            "col": torch.empty(max(nnz, 1), dtype=torch.int16, device=dev),
            "rcodes": torch.empty(max((nnz + 1) // 2, 1), dtype=torch.uint8, device=dev),
            "rscale": torch.empty(N, dtype=torch.float32, device=dev),
        })
    s = _stream_handle(stream)
    _check(lib.mq_export_canonical(packed.handle, *[ctypes.c_void_p(out[k].data_ptr()) if k in out else None
                                                    for k in names], s), "mq_export_canonical")
    torch.cuda.synchronize()
    if residual:
        out["col"] = out["col"][:nnz]
        out["rcodes"] = out["rcodes"][:(nnz + 1) // 2]
    return out


def mq_export_tiled(packed: Packed, stream=None) -> dict:
    """Device layout read by the kernels (synchronises the stream)."""
    import torch
    dev = torch.device("cuda", torch.cuda.current_device())
    Nb = -(-packed.N // 16)
    Kt = -(-packed.K // 128)
    tiles = torch.empty((Nb, Kt, 64, 16), dtype=torch.uint8, device=dev)
    tile_ptr = torch.empty(Nb * Kt + 1, dtype=torch.int32, device=dev)
    s = _stream_handle(stream)
    _check(lib.mq_export_tiled(packed.handle, ctypes.c_void_p(tiles.data_ptr()),
                               ctypes.c_void_p(tile_ptr.data_ptr()), None, s), "mq_export_tiled")
    torch.cuda.synchronize()
    nstream = int(tile_ptr[-1].item())
    entries = torch.empty(max(nstream, 1), dtype=torch.int32, device=dev)
    _check(lib.mq_export_tiled(packed.handle, None, None, ctypes.c_void_p(entries.data_ptr()), s),
           "mq_export_tiled")
    torch.cuda.synchronize()
    return {"tiles": tiles, "tile_ptr": tile_ptr, "entries": entries[:nstream]}
