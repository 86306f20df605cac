"""IO-aware exact attention for AMD Instinct MI355X (gfx950).

The compute lives in ``libfa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/fa.h``); ``io_aware_exact_amd.fa`` is the thin ctypes
binding.  Importing this package loads nothing; the library is opened on the
first call and a missing library is an error, never a silent fallback.
"""

__all__ = ["attention", "attention_varlen", "attention_decode", "attention_fp8"]


def __getattr__(name):
    if name in __all__:
        from . import fa
        return getattr(fa, name)
    raise AttributeError(name)
