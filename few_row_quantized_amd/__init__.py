"""few_row_quantized_amd: few-row (M = 1..16) quantized GEMV for AMD Instinct MI355X (gfx950).

y[M,N] = x[M,K] . dequant(W[N,K])^T with 4-bit or 2-bit affine group-quantized
weights (fp16 scale and bias per row and group), bf16 activations and fp32
output.  All arithmetic runs in hand-written HIP kernels inside libqgemv.so;
the Python layer (``few_row_quantized_amd.qgemv``) only marshals arguments.

Submodules:
  qgemv      ctypes binding of the C ABI declared in include/qgemv.h
  synth      seeded synthetic inputs (no product arithmetic)
  accounting byte / flop counts for bandwidth figures
  build      compiles libqgemv.so with hipcc for gfx950
"""

__all__ = ["qgemv", "synth", "accounting", "build"]


def __getattr__(name):
    # Lazy submodule import, so `import few_row_quantized_amd.synth` works on a
    # host without the built library.
    import importlib
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
