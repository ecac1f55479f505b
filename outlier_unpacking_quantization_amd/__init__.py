"""IM-Unpack exact low bit-width integer GEMM path for AMD MI355X (gfx950).

The compute path is the HIP library ``libimunpack.so`` (C ABI in
``include/imunpack.h``); ``binding`` marshals torch tensors into it and
``workloads`` draws the seeded synthetic operands.  The binding (and torch)
is imported on first use of one of its names.
"""
_BINDING = ("quantize_rtn", "plan_unpack", "unpack", "unpacked_gemm", "imunpack_matmul", "params",
            "Matrix", "ImunpackError", "Workspace", "Stats", "Plan", "version")


def __getattr__(name):
    if name in _BINDING:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
