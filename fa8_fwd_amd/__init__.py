"""MI355X-native FP8 (E4M3) attention forward.

The compute path is the C-ABI library ``libfa8.so`` (hand-written gfx950 HIP kernels); this
package is a thin ctypes binding over it (argument marshalling only) plus the seeded input
generators in ``fa8_fwd_amd.inputs``. The binding is imported lazily so that the input
generators stay usable on machines without the built library or a GPU; every compute entry
point raises if the library is missing.
"""

__all__ = ["prefill", "decode_splitkv", "combine", "decode", "check_params", "decode_num_splits",
           "decode_workspace_bytes", "lib_path", "FA8Error"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
