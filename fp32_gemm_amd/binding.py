"""ctypes binding of libfp32_gemm_amd.so (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
only checks tensor metadata, turns tensors into (pointer, leading dimension)
pairs and maps status codes to exceptions.  There is no fallback: if the
library is missing, importing this module raises.

torch is imported before the library is opened so that the library binds to
the HIP runtime torch has already loaded (both carry the same soname), which
makes torch's device pointers and stream handles valid for the library.
"""
from __future__ import annotations

import ctypes
import json
import os
import re

import torch  # noqa: F401  -- must load torch's HIP runtime first (see above)

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libfp32_gemm_amd.so")
_RESOURCES = os.path.join(_PKG, "_build", "resources.json")

if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is not built; run `python -m fp32_gemm_amd.build` (hipcc, gfx950)")

_lib = ctypes.CDLL(_LIB_PATH)

_i64, _i32, _f32, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p


class _Config(ctypes.Structure):
    _fields_ = [(n, _i32) for n in (
        "id", "path", "BM", "BN", "BK", "WM", "WN", "WNITER", "TM", "TN", "NT", "swz", "opt",
        "WMITER", "WSUBM", "WSUBN", "acc_per_lane", "lds_bytes", "vgpr_estimate")]


class _Plan(ctypes.Structure):
    _fields_ = [("cfg_id", _i32), ("vector_variant", _i32), ("grid", _i64), ("block", _i32),
                ("tiles_full", _i32), ("splits", _i32), ("slots", _i64)]


class _Attr(ctypes.Structure):
    _fields_ = [("num_regs", _i32), ("scratch_bytes", _i32), ("lds_bytes", _i32),
                ("max_threads", _i32)]


class _SimReport(ctypes.Structure):
    _fields_ = [("failed_check", _i32), ("store_a_ways", _i32), ("store_b_ways", _i32),
                ("read_a_ways", _i32), ("read_b_ways", _i32), ("dma_read_a_ways", _i32),
                ("dma_read_b_ways", _i32)]


_SIGS = {
    "sgemm": ([_i64, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _f32, _vp, _i64], ctypes.c_int),
    "sgemm_ex": ([_i64, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _f32, _vp, _i64, _vp, _i32],
                 ctypes.c_int),
    "sgemm_ladder": ([_i32, _i64, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _f32, _vp, _i64, _vp],
                     ctypes.c_int),
    "sgemm_num_configs": ([], ctypes.c_int),
    "sgemm_config_info": ([_i32, ctypes.POINTER(_Config)], ctypes.c_int),
    "sgemm_plan": ([_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i32,
                    ctypes.POINTER(_Plan)], ctypes.c_int),
    "sgemm_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "sgemm_last_hip_error": ([], ctypes.c_int),
    "sgemm_device_check": ([], ctypes.c_int),
    "sgemm_kernel_attributes": ([_i32, _i32, ctypes.POINTER(_Attr)], ctypes.c_int),
    "sgemm_check_tuple": ([ctypes.POINTER(_i32), _i32], ctypes.c_int),
    "sgemm_tile_order": ([_i64, _i64, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i32), _i64],
                         _i64),
    "sgemm_simulate_tuple": ([ctypes.POINTER(_i32), _i32, ctypes.POINTER(_SimReport)],
                             ctypes.c_int),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

PATHS = {0: "valu", 1: "mfma32", 2: "mfma16"}
TUPLE_FIELDS = ("BM", "BN", "BK", "WM", "WN", "WNITER", "TM", "TN", "NT", "path", "swz", "opt")


class SgemmError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        msg = _lib.sgemm_status_string(status).decode()
        if status == 4:
            msg += f" (hipError_t {_lib.sgemm_last_hip_error()})"
        super().__init__(f"sgemm status {status}: {msg}")


def library_path() -> str:
    return _LIB_PATH


def exported_symbols():
    """Names declared in include/fp32_gemm.h that the library must export."""
    return sorted(_SIGS)


def status_string(status: int) -> str:
    return _lib.sgemm_status_string(status).decode()


def device_check() -> int:
    return _lib.sgemm_device_check()


def num_configs() -> int:
    return _lib.sgemm_num_configs()


def config_info(cfg_id: int) -> dict:
    c = _Config()
    rc = _lib.sgemm_config_info(cfg_id, ctypes.byref(c))
    if rc != 0:
        raise SgemmError(rc)
    d = {f: getattr(c, f) for f, _ in _Config._fields_}
    d["tuple"] = tuple(d[f] for f in TUPLE_FIELDS)
    d["path_name"] = PATHS[d["path"]]
    return d


def _kernel_resources():
    """Compiler resource report per tuple and kernel, if the build left one:
    keys (tuple, "vec") and (tuple, "scalar")."""
    if not os.path.exists(_RESOURCES):
        return {}
    with open(_RESOURCES) as f:
        raw = json.load(f)
    out = {}
    pat = re.compile(r"TileCfgILi" + r"ELi".join([r"(\d+)"] * 12) + r"EEE(?:Lb(\d))?")
    for name, v in raw.items():
        m = pat.search(name)
        if m:
            g = tuple(int(x) for x in m.groups()[:12])
            # The hybrid kernels (the scalar variant of direct-LDS matrix-core
            # tuples) take no variant flag.
            kind = "scalar" if "hyb" in name or m.group(13) == "0" else "vec"
            out[(g, kind)] = v
    return out


def configs():
    """All compiled configurations, with the compiler's resource report."""
    res = _kernel_resources()
    out = []
    for i in range(num_configs()):
        d = config_info(i)
        d["resources_vec"] = res.get((d["tuple"], "vec"))
        d["resources_scalar"] = res.get((d["tuple"], "scalar"))
        out.append(d)
    return out


def kernel_attributes(cfg_id: int, vector_variant: int = 1) -> dict:
    """Runtime attributes of a compiled kernel: vector_variant 1 the float4
    kernel, 0 the scalar variant's."""
    a = _Attr()
    rc = _lib.sgemm_kernel_attributes(cfg_id, int(vector_variant), ctypes.byref(a))
    if rc != 0:
        raise SgemmError(rc)
    return {f: getattr(a, f) for f, _ in _Attr._fields_}


def _tuple12(tup):
    tup = tuple(tup)
    return (_i32 * 12)(*(tup + (0,) * (12 - len(tup))))


def check_tuple(tup, target: str = "gfx950") -> int:
    """Checker reason code; an 11-element tuple means opt = 0."""
    arr = _tuple12(tup)
    return _lib.sgemm_check_tuple(arr, {"gfx950": 0, "page": 1}[target])


def simulate_tuple(tup, banks: int = 32) -> dict:
    arr = _tuple12(tup)
    r = _SimReport()
    rc = _lib.sgemm_simulate_tuple(arr, banks, ctypes.byref(r))
    d = {f: getattr(r, f) for f, _ in _SimReport._fields_}
    d["status"] = rc
    return d


def tile_order(M, N, cfg_id):
    """(rows, cols) output tile of each workgroup id, as lists."""
    n = _lib.sgemm_tile_order(M, N, cfg_id, None, None, 0)
    if n < 0:
        raise ValueError("bad arguments")
    r, c = (_i32 * n)(), (_i32 * n)()
    _lib.sgemm_tile_order(M, N, cfg_id, r, c, n)
    return list(r), list(c)


def sgemm_raw(M, N, K, alpha, A_ptr, lda, B_ptr, ldb, beta, C_ptr, ldc, stream=None, cfg_id=-1):
    """Direct call of sgemm_ex on raw device pointers; returns the status."""
    return _lib.sgemm_ex(M, N, K, alpha, A_ptr, lda, B_ptr, ldb, beta, C_ptr, ldc,
                         stream, cfg_id)


def plan(M, N, K, A_ptr, lda, B_ptr, ldb, C_ptr, ldc, cfg_id=-1) -> dict:
    p = _Plan()
    rc = _lib.sgemm_plan(M, N, K, A_ptr, lda, B_ptr, ldb, C_ptr, ldc, cfg_id, ctypes.byref(p))
    if rc != 0:
        raise SgemmError(rc)
    return {f: getattr(p, f) for f, _ in _Plan._fields_}


def _operand(t, name):
    """(data pointer, leading dimension) of a 2-D float32 GPU tensor with unit
    column stride; raises on anything else."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype is not torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    shape = t.shape
    if len(shape) != 2:
        raise ValueError(f"{name} must be 2-D")
    rows, cols = shape
    s0, s1 = t.stride()
    if cols > 1 and s1 != 1:
        raise ValueError(f"{name} must have unit column stride (row-major)")
    if rows > 1 and cols > 0 and s0 < cols:
        # Expanded or otherwise overlapping rows: no leading dimension
        # describes them, and the kernels would read past the storage.
        raise ValueError(f"{name}: rows overlap (row stride {s0} < {cols} columns)")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    ld = s0 if rows > 1 else cols
    return t.data_ptr(), (ld if ld > 1 else 1)


# The raw handle of torch's current stream on a device, without building a
# Stream object (which costs more than the rest of a call); the public route
# where this build of torch lacks it.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(dev, stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    if _raw_stream is not None:
        return _raw_stream(dev.index if dev.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(dev).cuda_stream


def sgemm_ex(A, B, C, alpha=1.0, beta=0.0, stream=None, cfg_id=-1):
    """C <- alpha * A @ B + beta * C in place, for float32 GPU tensors.

    A is M x K, B is K x N, C is M x N, each row-major with unit column stride
    (a row slice of a wider buffer is fine: its row stride is the leading
    dimension).  The call is asynchronous on `stream` (default: torch's
    current stream on C's device).  Returns C.
    """
    a, lda = _operand(A, "A")
    b, ldb = _operand(B, "B")
    c, ldc = _operand(C, "C")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or C.shape != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    dev = C.device
    if A.device != dev or B.device != dev:
        raise ValueError("A, B and C must be on the same device")
    handle = _stream_handle(dev, stream)
    if dev.index is None or dev.index == torch.cuda.current_device():
        rc = _lib.sgemm_ex(M, N, K, alpha, a, lda, b, ldb, beta, c, ldc, handle, cfg_id)
    else:
        with torch.cuda.device(dev):
            rc = _lib.sgemm_ex(M, N, K, alpha, a, lda, b, ldb, beta, c, ldc, handle, cfg_id)
    if rc != 0:
        raise SgemmError(rc)
    return C


def ladder(rung, A, B, C, alpha=1.0, beta=0.0, stream=None):
    """C <- alpha * A @ B + beta * C with the kernel of ladder rung 1-4."""
    a, lda = _operand(A, "A")
    b, ldb = _operand(B, "B")
    c, ldc = _operand(C, "C")
    M, K = A.shape
    N = B.shape[1]
    if B.shape[0] != K or tuple(C.shape) != (M, N):
        raise ValueError("shape mismatch")
    if not (A.device == B.device == C.device):
        raise ValueError("A, B and C must be on the same device")
    if stream is None:
        stream = torch.cuda.current_stream(C.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    with torch.cuda.device(C.device):
        rc = _lib.sgemm_ladder(rung, M, N, K, alpha, a, lda, b, ldb, beta, c, ldc, handle)
    if rc != 0:
        raise SgemmError(rc)
    return C


def sgemm(A, B, C, alpha=1.0, beta=0.0):
    """Tuned-dispatch SGEMM on torch's current stream (see :func:`sgemm_ex`)."""
    return sgemm_ex(A, B, C, alpha, beta)
