"""MI355X (gfx950) fused dense 4-bit base + sparse 4-bit residual linear layer.

The HIP library (libmosaicq.so, built by ``python -m bit_gemm_amd.build``) is
the product; ``bit_gemm_amd.mosaicq`` is its thin ctypes binding and
``bit_gemm_amd.synth`` draws the seeded synthetic inputs.
"""

_BINDING = ("mq_pack", "mq_linear", "mq_linear_with", "mq_packed_info", "mq_export_canonical",
            "mq_export_tiled", "mq_status_string", "Packed", "MQError")


def __getattr__(name):
    if name in _BINDING:
        from . import mosaicq
        return getattr(mosaicq, name)
    raise AttributeError(name)
