"""Python binding of the batch-invariant GEMM library (libinvariant_matmul.so).

Argument marshalling only: every step of the product runs in the library's
HIP kernels.  PyTorch supplies device memory and streams.  The calls mirror
the C ABI in include/invariant_matmul.h:

    plan = gemm_plan(M, N, K, "f16")                  # pure host call
    gemm_run(plan, A, B, C)                           # C = A @ B
    gemm_splitk_run(plan, A, B, C, workspace)         # split-K path
    plan = gemm_plan_ex2(M, N, K, "f16", "f16", flags=PLAN_B_TRANSPOSED)
    gemm_run(plan, A, W, C, bias=b)                   # C = A @ W.T + b

A, B, C, workspace are CUDA(HIP) tensors (or raw device addresses as ints);
``stream`` defaults to torch's current stream on the operands' device.  There
is no fallback: if the shared library is missing, importing it raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "GemmError", "Plan", "PlanInfo", "gemm_plan", "gemm_plan_ex", "gemm_plan_ex2",
    "gemm_plan_info", "gemm_workspace_size", "gemm_plan_tile_of", "gemm_run", "gemm_splitk_run",
    "gemm_splitk_run_noalloc", "NOALLOC_WORKSPACE_BYTES",
    "gemm_plan_destroy", "gemm_status_string", "gemm_last_hip_error", "mm", "out_torch_dtype",
    "lib", "LIB_PATH",
    "DTYPE", "TILE", "STATUS", "EXPORTED_SYMBOLS", "PLAN_B_TRANSPOSED", "PLAN_PERSISTENT",
    "PLAN_TILE_BY_M", "PLAN_FP8_FP32_ACCUM",
    "OzakiPlan", "ozaki_plan", "ozaki_plan_info", "ozaki_workspace_size", "ozaki_split",
    "ozaki_multiply", "ozaki_run", "ozaki_mm",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libinvariant_matmul.so")

STATUS = {0: "GEMM_OK", 1: "GEMM_ERR_INVALID_VALUE", 2: "GEMM_ERR_UNSUPPORTED",
          3: "GEMM_ERR_WORKSPACE", 4: "GEMM_ERR_HIP"}
DTYPE = {"f16": 0, "bf16": 1, "e4m3": 2, "e5m2": 3, "f32": 4, "i8": 5}
TILE = {"default": 0, "256x256": 1, "128x128": 2, "32x128": 3, "256x256_rs": 4, "32x256": 5,
        "64x256": 6, "128x256": 7, "32x64": 8, "64x64": 9, "32x32": 10}
PLAN_B_TRANSPOSED = 1
PLAN_PERSISTENT = 2
PLAN_TILE_BY_M = 4
PLAN_FP8_FP32_ACCUM = 8  # fp8 widened to fp16: the fp32 bound for every K (DMA tiles only)
# GEMM_NOALLOC_WORKSPACE_BYTES: the largest workspace gemm_splitk_run_noalloc serves
NOALLOC_WORKSPACE_BYTES = 64 << 20
EXPORTED_SYMBOLS = (
    "gemm_plan", "gemm_plan_ex", "gemm_plan_ex2", "gemm_plan_info", "gemm_workspace_size",
    "gemm_plan_tile_of", "gemm_run", "gemm_run_bias", "gemm_splitk_run", "gemm_splitk_run_bias",
    "gemm_plan_destroy", "gemm_status_string", "gemm_last_hip_error", "gemm_splitk_run_noalloc",
    "ozaki_plan", "ozaki_plan_info", "ozaki_workspace_size", "ozaki_split", "ozaki_multiply",
    "ozaki_run", "ozaki_plan_destroy",
)


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = STATUS.get(status, f"status {status}")
        msg = f"{where}: {name}"
        if status == 4:
            msg += f" (hip error {lib().gemm_last_hip_error()})"
        super().__init__(msg)


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32), ("tile", ctypes.c_int32),
        ("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32), ("block_k", ctypes.c_int32),
        ("mfma_m", ctypes.c_int32), ("mfma_n", ctypes.c_int32), ("mfma_k", ctypes.c_int32),
        ("waves", ctypes.c_int32), ("group_m", ctypes.c_int32), ("split_k", ctypes.c_int32),
        ("k_per_split", ctypes.c_int64), ("tiles_m", ctypes.c_int64), ("tiles_n", ctypes.c_int64),
        ("grid_run", ctypes.c_int64), ("grid_splitk", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_uint64), ("scale_a", ctypes.c_float),
        ("scale_b", ctypes.c_float), ("run_tile", ctypes.c_int32),
        ("run_block_m", ctypes.c_int32), ("run_block_n", ctypes.c_int32),
        ("run_waves", ctypes.c_int32), ("run_tiles_m", ctypes.c_int64),
        ("run_tiles_n", ctypes.c_int64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class OzakiPlanInfo(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("type2", ctypes.c_int32), ("rho", ctypes.c_int32), ("bits", ctypes.c_int32),
        ("delta", ctypes.c_int32), ("slices", ctypes.c_int32), ("d", ctypes.c_int32),
        ("pairs", ctypes.c_int32), ("chunk", ctypes.c_int64), ("tile_m", ctypes.c_int32),
        ("tile_n", ctypes.c_int32),
        ("k_pad", ctypes.c_int64), ("n_pad", ctypes.c_int64), ("grid", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_uint64), ("a_slices_offset", ctypes.c_uint64),
        ("b_slices_offset", ctypes.c_uint64), ("a_exp_offset", ctypes.c_uint64),
        ("b_exp_offset", ctypes.c_uint64), ("scratch_offset", ctypes.c_uint64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded shared library (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m invariant_matmul_amd.build` "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_float
        pp = ctypes.POINTER(ctypes.c_void_p)
        L.gemm_plan.argtypes = [i64, i64, i64, i32, pp]
        L.gemm_plan_ex.argtypes = [i64, i64, i64, i32, i32, i32, i32, f32, f32, pp]
        L.gemm_plan_ex2.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32, f32, f32,
                                    ctypes.c_uint, pp]
        L.gemm_plan_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
        L.gemm_workspace_size.argtypes = [vp]
        L.gemm_workspace_size.restype = ctypes.c_size_t
        p64 = ctypes.POINTER(ctypes.c_int64)
        L.gemm_plan_tile_of.argtypes = [vp, i64, p64, p64, p64]
        L.gemm_run.argtypes = [vp, vp, vp, vp, vp]
        L.gemm_run_bias.argtypes = [vp, vp, vp, vp, vp, vp]
        L.gemm_splitk_run.argtypes = [vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.gemm_splitk_run_bias.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.gemm_splitk_run_noalloc.argtypes = [vp, vp, vp, vp, vp]
        L.gemm_plan_destroy.argtypes = [vp]
        L.gemm_plan_destroy.restype = None
        L.gemm_status_string.argtypes = [i32]
        L.gemm_status_string.restype = ctypes.c_char_p
        L.gemm_last_hip_error.argtypes = []
        sz = ctypes.c_size_t
        L.ozaki_plan.argtypes = [i64, i64, i64, i32, i32, i32, i64, pp]
        L.ozaki_plan_info.argtypes = [vp, ctypes.POINTER(OzakiPlanInfo)]
        L.ozaki_workspace_size.argtypes = [vp]
        L.ozaki_workspace_size.restype = sz
        L.ozaki_split.argtypes = [vp, i32, vp, vp, sz, vp]
        L.ozaki_multiply.argtypes = [vp, vp, sz, vp, vp]
        L.ozaki_run.argtypes = [vp, vp, vp, vp, vp, sz, vp]
        L.ozaki_plan_destroy.argtypes = [vp]
        L.ozaki_plan_destroy.restype = None
        for f in ("gemm_plan", "gemm_plan_ex", "gemm_plan_ex2", "gemm_plan_info",
                  "gemm_plan_tile_of", "gemm_run", "gemm_run_bias", "gemm_splitk_run",
                  "gemm_splitk_run_bias", "gemm_splitk_run_noalloc", "gemm_last_hip_error", "ozaki_plan", "ozaki_plan_info",
                  "ozaki_split", "ozaki_multiply", "ozaki_run"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _dtype_code(dt) -> int:
    if isinstance(dt, int):
        return dt
    if isinstance(dt, str):
        return DTYPE[dt]
    import torch
    m = {torch.float16: 0, torch.bfloat16: 1, torch.float8_e4m3fn: 2, torch.float8_e5m2: 3,
         torch.float32: 4}
    return m[dt]


class Plan:
    """Owns a gemm_plan_t; destroyed with the object."""

    def __init__(self, handle: int):
        self.handle = handle
        self._lib = lib()

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h:
            self._lib.gemm_plan_destroy(h)

    @property
    def info(self) -> dict:
        return gemm_plan_info(self)

    @property
    def workspace_bytes(self) -> int:
        return gemm_workspace_size(self)


def _check(status: int, where: str):
    if status != 0:
        raise GemmError(status, where)


def gemm_plan(M: int, N: int, K: int, dtype) -> Plan:
    h = ctypes.c_void_p()
    _check(lib().gemm_plan(M, N, K, _dtype_code(dtype), ctypes.byref(h)), "gemm_plan")
    return Plan(h.value)


def gemm_plan_ex(M: int, N: int, K: int, dtype, out_dtype="f32", split_k: int = 0,
                 group_m: int = 0, tile="default", scale_a: float = 1.0,
                 scale_b: float = 1.0) -> Plan:
    """Plan with explicit options.  An explicit tile is a gemm_plan_ex2 option
    (the C call gemm_plan_ex has none), so a tile other than "default" plans
    through gemm_plan_ex2 with no flags."""
    h = ctypes.c_void_p()
    t = TILE[tile] if isinstance(tile, str) else int(tile)
    if t == TILE["default"]:
        _check(lib().gemm_plan_ex(M, N, K, _dtype_code(dtype), _dtype_code(out_dtype), split_k,
                                  group_m, scale_a, scale_b, ctypes.byref(h)), "gemm_plan_ex")
    else:
        _check(lib().gemm_plan_ex2(M, N, K, _dtype_code(dtype), _dtype_code(out_dtype), split_k,
                                   group_m, t, scale_a, scale_b, 0, ctypes.byref(h)),
               "gemm_plan_ex2")
    return Plan(h.value)


def gemm_plan_ex2(M: int, N: int, K: int, dtype, out_dtype="f32", split_k: int = 0,
                  group_m: int = 0, tile="default", scale_a: float = 1.0, scale_b: float = 1.0,
                  flags: int = 0) -> Plan:
    h = ctypes.c_void_p()
    t = TILE[tile] if isinstance(tile, str) else int(tile)
    _check(lib().gemm_plan_ex2(M, N, K, _dtype_code(dtype), _dtype_code(out_dtype), split_k,
                               group_m, t, scale_a, scale_b, int(flags), ctypes.byref(h)),
           "gemm_plan_ex2")
    return Plan(h.value)


def gemm_plan_info(plan: Plan) -> dict:
    info = PlanInfo()
    _check(lib().gemm_plan_info(plan.handle, ctypes.byref(info)), "gemm_plan_info")
    return info.as_dict()


def gemm_workspace_size(plan: Plan) -> int:
    return int(lib().gemm_workspace_size(plan.handle))


def gemm_plan_tile_of(plan: Plan, workgroup: int):
    s, m, n = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().gemm_plan_tile_of(plan.handle, workgroup, ctypes.byref(s), ctypes.byref(m),
                                   ctypes.byref(n)), "gemm_plan_tile_of")
    return s.value, m.value, n.value


def _addr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else int(stream.cuda_stream)
    for t in tensors:
        if t is not None and not isinstance(t, int) and t.is_cuda:
            import torch
            return int(torch.cuda.current_stream(t.device).cuda_stream)
    return 0


def _check_device(t, name):
    """A tensor operand must live on the current CUDA (HIP) device: the kernels
    run there and would take a memory fault on a host or foreign address."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor, got one on {t.device}")
    import torch
    cur = torch.cuda.current_device()
    if t.device.index != cur:
        raise ValueError(f"{name} is on {t.device}, but the current device is cuda:{cur}")


def _check_tensor(t, name, dtype_code, numel):
    if t is None or isinstance(t, int):
        return
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if _dtype_code(t.dtype) != dtype_code:
        raise ValueError(f"{name} has dtype {t.dtype}, plan expects code {dtype_code}")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, plan expects {numel}")
    _check_device(t, name)


def _check_operands(plan: Plan, A, B, C, bias=None):
    i = gemm_plan_info(plan)
    _check_tensor(A, "A", i["in_dtype"], i["M"] * i["K"])
    _check_tensor(B, "B", i["in_dtype"], i["K"] * i["N"])
    _check_tensor(C, "C", i["out_dtype"], i["M"] * i["N"])
    _check_tensor(bias, "bias", DTYPE["f32"], i["N"])


def gemm_run(plan: Plan, A, B, C, stream=None, bias=None) -> None:
    """C = A @ B (+ bias, an fp32 vector of N) in one pass."""
    _check_operands(plan, A, B, C, bias)
    _check(lib().gemm_run_bias(plan.handle, _addr(A), _addr(B), _addr(bias), _addr(C),
                               _stream(stream, A, B, C)), "gemm_run")


def gemm_splitk_run(plan: Plan, A, B, C, workspace, stream=None, workspace_bytes=None,
                    bias=None) -> None:
    """C = A @ B (+ bias) through the split-K workspace and the reduction kernel."""
    _check_operands(plan, A, B, C, bias)
    _check_ws_device(workspace)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else (
            workspace.numel() * workspace.element_size())
    _check(lib().gemm_splitk_run_bias(plan.handle, _addr(A), _addr(B), _addr(bias), _addr(C),
                                      _addr(workspace), int(workspace_bytes),
                                      _stream(stream, A, B, C)), "gemm_splitk_run")


def gemm_splitk_run_noalloc(plan: Plan, A, B, C, stream=None) -> None:
    """C = A @ B through the split-K path with the workspace taken from the
    library's own device array (no allocation by the call); the plan's
    workspace must fit in NOALLOC_WORKSPACE_BYTES.  Calls that overlap on one
    GPU share that array and race."""
    _check_operands(plan, A, B, C)
    need = gemm_workspace_size(plan)
    if need > NOALLOC_WORKSPACE_BYTES:
        raise GemmError(3, f"gemm_splitk_run_noalloc: the plan needs a workspace of {need} "
                           f"bytes, more than the library's {NOALLOC_WORKSPACE_BYTES}")
    _check(lib().gemm_splitk_run_noalloc(plan.handle, _addr(A), _addr(B), _addr(C),
                                         _stream(stream, A, B, C)), "gemm_splitk_run_noalloc")


def gemm_plan_destroy(plan: Plan) -> None:
    h, plan.handle = plan.handle, None
    if h:
        lib().gemm_plan_destroy(h)


def gemm_status_string(status: int) -> str:
    return lib().gemm_status_string(status).decode()


def gemm_last_hip_error() -> int:
    return int(lib().gemm_last_hip_error())


def out_torch_dtype(code: int):
    """The torch dtype of an output dtype code (GEMM_F32, GEMM_BF16, GEMM_F16)."""
    import torch
    table = {DTYPE["f32"]: torch.float32, DTYPE["bf16"]: torch.bfloat16,
             DTYPE["f16"]: torch.float16}
    if code not in table:
        raise ValueError(f"output dtype code {code} is not one of f32, bf16, f16")
    return table[code]


def mm(A, B, out_dtype=None, split_k=None, plan: Plan | None = None, stream=None):
    """C = A @ B through the library, allocating C (and a workspace) with torch.

    split_k=None uses gemm_run; an int (0 = the plan's default) uses the split-K
    path.  The plan is made from (N, K, dtype) options only, never from M.
    """
    import torch
    _check_device(A, "A")
    _check_device(B, "B")
    M, K = A.shape
    N = B.shape[1]
    if plan is None:
        od = out_dtype if out_dtype is not None else (
            "bf16" if A.dtype in (torch.float8_e4m3fn, torch.float8_e5m2) else "f32")
        plan = gemm_plan_ex(M, N, K, A.dtype, od, split_k=split_k or 0)
    info = gemm_plan_info(plan)
    C = torch.empty((M, N), dtype=out_torch_dtype(info["out_dtype"]), device=A.device)
    if split_k is None:
        gemm_run(plan, A, B, C, stream)
    else:
        ws = torch.empty(max(1, gemm_workspace_size(plan) // 4), dtype=torch.float32,
                         device=A.device)
        gemm_splitk_run(plan, A, B, C, ws, stream)
    return C


# ---- Ozaki-scheme fp64 product ------------------------------------------------

class OzakiPlan:
    """Owns an ozaki_plan_t; destroyed with the object."""

    def __init__(self, handle: int):
        self.handle = handle
        self._lib = lib()

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h:
            self._lib.ozaki_plan_destroy(h)

    @property
    def info(self) -> dict:
        return ozaki_plan_info(self)


def ozaki_plan(M: int, N: int, K: int, type2="bf16", slices: int = 0, d: int = 0,
               chunk: int = 0) -> OzakiPlan:
    """Plan C = A @ B in fp64 by the Ozaki scheme with Type2 slices ("bf16",
    "e4m3" or "i8"); slices / d / chunk = 0 take the library's defaults."""
    h = ctypes.c_void_p()
    _check(lib().ozaki_plan(M, N, K, _dtype_code(type2), int(slices), int(d), int(chunk),
                            ctypes.byref(h)), "ozaki_plan")
    return OzakiPlan(h.value)


def ozaki_plan_info(plan: OzakiPlan) -> dict:
    info = OzakiPlanInfo()
    _check(lib().ozaki_plan_info(plan.handle, ctypes.byref(info)), "ozaki_plan_info")
    return info.as_dict()


def ozaki_workspace_size(plan: OzakiPlan) -> int:
    return int(lib().ozaki_workspace_size(plan.handle))


def _check_ws_device(workspace):
    if workspace is not None and not isinstance(workspace, int):
        _check_device(workspace, "workspace")


def _ws_bytes(workspace, workspace_bytes):
    if workspace_bytes is not None:
        return int(workspace_bytes)
    if workspace is None or isinstance(workspace, int):
        return 0
    return workspace.numel() * workspace.element_size()


def _check_f64(t, name, numel):
    if t is None or isinstance(t, int):
        return
    import torch
    if t.dtype != torch.float64 or not t.is_contiguous() or t.numel() != numel:
        raise ValueError(f"{name} must be a contiguous float64 tensor of {numel} elements")
    _check_device(t, name)


def ozaki_split(plan: OzakiPlan, operand: int, x, workspace, stream=None,
                workspace_bytes=None) -> None:
    """Slices and exponents of A (operand 0, [M, K]) or B (1, [K, N]) into the workspace."""
    i = ozaki_plan_info(plan)
    _check_f64(x, "x", i["M"] * i["K"] if operand == 0 else i["K"] * i["N"])
    _check_ws_device(workspace)
    _check(lib().ozaki_split(plan.handle, int(operand), _addr(x), _addr(workspace),
                             _ws_bytes(workspace, workspace_bytes), _stream(stream, x, workspace)),
           "ozaki_split")


def ozaki_multiply(plan: OzakiPlan, workspace, C, stream=None, workspace_bytes=None) -> None:
    """The slice-pair product from a workspace filled by ozaki_split of A and B."""
    i = ozaki_plan_info(plan)
    _check_f64(C, "C", i["M"] * i["N"])
    _check_ws_device(workspace)
    _check(lib().ozaki_multiply(plan.handle, _addr(workspace), _ws_bytes(workspace, workspace_bytes),
                                _addr(C), _stream(stream, C, workspace)), "ozaki_multiply")


def ozaki_run(plan: OzakiPlan, A, B, C, workspace, stream=None, workspace_bytes=None) -> None:
    """C = A @ B (fp64) by the Ozaki scheme: split A, split B, multiply."""
    i = ozaki_plan_info(plan)
    _check_f64(A, "A", i["M"] * i["K"])
    _check_f64(B, "B", i["K"] * i["N"])
    _check_f64(C, "C", i["M"] * i["N"])
    _check_ws_device(workspace)
    _check(lib().ozaki_run(plan.handle, _addr(A), _addr(B), _addr(C), _addr(workspace),
                           _ws_bytes(workspace, workspace_bytes), _stream(stream, A, B, C)),
           "ozaki_run")


def ozaki_mm(A, B, type2="bf16", slices: int = 0, d: int = 0, chunk: int = 0, stream=None):
    """C = A @ B for fp64 CUDA tensors, allocating C and the workspace with torch."""
    import torch
    _check_device(A, "A")
    _check_device(B, "B")
    M, K = A.shape
    N = B.shape[1]
    plan = ozaki_plan(M, N, K, type2, slices, d, chunk)
    ws = torch.empty(max(1, ozaki_workspace_size(plan)), dtype=torch.uint8, device=A.device)
    C = torch.empty((M, N), dtype=torch.float64, device=A.device)
    ozaki_run(plan, A.contiguous(), B.contiguous(), C, ws, stream)
    return C
