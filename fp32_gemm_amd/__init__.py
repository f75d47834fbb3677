"""fp32_gemm_amd -- single-precision GEMM for one AMD Instinct MI355X (gfx950).

C = alpha * A @ B + beta * C on row-major fp32 matrices, computed by the
hand-written HIP kernels of ``libfp32_gemm_amd.so`` behind a C ABI
(``include/fp32_gemm.h``).  The Python side only marshals arguments; PyTorch
supplies device memory and streams.

The binding is loaded on first use of an API name, so ``fp32_gemm_amd.inputs``
can be imported on a machine where the library has not been built.
"""
_API = ("sgemm", "sgemm_ex", "sgemm_raw", "plan", "num_configs", "config_info", "configs",
        "status_string", "device_check", "SgemmError", "library_path", "check_tuple",
        "simulate_tuple", "exported_symbols", "tile_order", "ladder")


def __getattr__(name):
    if name == "binding" or name in _API:
        import importlib
        binding = importlib.import_module(__name__ + ".binding")
        return binding if name == "binding" else getattr(binding, name)
    raise AttributeError(name)


__all__ = list(_API)
