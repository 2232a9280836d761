"""Python binding of libtsgemm (include/tsgemm.h): argument marshalling only.

Every computation runs in the library's HIP kernels; PyTorch only provides
device memory and the stream.  Importing works without a GPU (plan creation and
validation are host-only); running needs the built library and a gfx950 GPU,
and fails loudly otherwise.

Names follow the C ABI: ``create`` -> :class:`Plan`, ``Plan.run``,
``Plan.run_traced``, ``Plan.run_mx``, ``Plan.run_mx_traced``,
``Plan.dump_schedule``, ``Plan.schedule_host``, ``Plan.info``, ``last_error``.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from . import _build

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtsgemm.so")

FP16 = 1
BF16 = 2
MXFP8 = 3   # E4M3 elements + E8M0 scales per 32 along K, bf16 output
OK, EINVAL, EUNSUPPORTED, EHIP, ENOMEM = 0, -1, -2, -3, -4

# every symbol the header declares
EXPORTS = (
    "tsgemm_create", "tsgemm_set_num_workgroups", "tsgemm_set_waves", "tsgemm_set_schedule", "tsgemm_set_epilogue",
    "tsgemm_set_xcd_remap", "tsgemm_set_l2_prefetch", "tsgemm_run",
    "tsgemm_run_traced", "tsgemm_run_mx", "tsgemm_run_mx_traced", "tsgemm_mx_packed_scale_bytes",
    "tsgemm_mx_pack_scales", "tsgemm_run_mx_packed", "tsgemm_num_tiles", "tsgemm_num_workgroups", "tsgemm_plan_info",
    "tsgemm_dump_schedule", "tsgemm_schedule_host", "tsgemm_destroy", "tsgemm_last_error",
    "tsgemm_last_error_code", "tsgemm_launch_info", "tsgemm_run_mx_noalloc", "tsgemm_worker_numbering",
)


class TsgemmError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"tsgemm error {code}: {msg}")
        self.code = code


class Info(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("block_M", ctypes.c_int32), ("block_N", ctypes.c_int32), ("block_K", ctypes.c_int32),
        ("group_size", ctypes.c_int32), ("num_stages", ctypes.c_int32),
        ("lds_slots", ctypes.c_int32), ("stage_bytes", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
        ("m_blocks", ctypes.c_int64), ("n_blocks", ctypes.c_int64), ("k_blocks", ctypes.c_int64),
        ("num_tiles", ctypes.c_int64),
        ("num_workgroups", ctypes.c_int32), ("waves", ctypes.c_int32),
        ("threads_per_workgroup", ctypes.c_int32), ("xcd_remap", ctypes.c_int32),
        ("cluster_size", ctypes.c_int32), ("column_major", ctypes.c_int32),
        ("store_block_N", ctypes.c_int32), ("l2_prefetch", ctypes.c_int32),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def load(path: str | None = None):
    """Load libtsgemm.so (built by __graft_entry__.build()); raises if absent.
    The environment variable TSGEMM_LIB names another build of the library
    (for instance one compiled with different -D switches) to load instead."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("TSGEMM_LIB") or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with __graft_entry__.build() "
                           "(persistent_tile_scheduled_amd._build.build_library())")
    lib = ctypes.CDLL(p)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.tsgemm_create.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32, i32]
    lib.tsgemm_create.restype = vp
    lib.tsgemm_set_num_workgroups.argtypes = [vp, i32]
    lib.tsgemm_set_num_workgroups.restype = i32
    lib.tsgemm_set_waves.argtypes = [vp, i32]
    lib.tsgemm_set_waves.restype = i32
    lib.tsgemm_set_schedule.argtypes = [vp, i32, i32]
    lib.tsgemm_set_schedule.restype = i32
    lib.tsgemm_set_epilogue.argtypes = [vp, i32]
    lib.tsgemm_set_epilogue.restype = i32
    lib.tsgemm_set_xcd_remap.argtypes = [vp, i32]
    lib.tsgemm_set_xcd_remap.restype = i32
    lib.tsgemm_set_l2_prefetch.argtypes = [vp, i32]
    lib.tsgemm_set_l2_prefetch.restype = i32
    lib.tsgemm_run.argtypes = [vp, vp, vp, vp, vp]
    lib.tsgemm_run.restype = i32
    lib.tsgemm_run_traced.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.tsgemm_run_traced.restype = i32
    lib.tsgemm_run_mx.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.tsgemm_run_mx.restype = i32
    lib.tsgemm_run_mx_traced.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
    lib.tsgemm_run_mx_traced.restype = i32
    lib.tsgemm_mx_packed_scale_bytes.argtypes = [vp, i32]
    lib.tsgemm_mx_packed_scale_bytes.restype = i64
    lib.tsgemm_mx_pack_scales.argtypes = [vp, i32, vp, vp, vp]
    lib.tsgemm_mx_pack_scales.restype = i32
    lib.tsgemm_run_mx_packed.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.tsgemm_run_mx_packed.restype = i32
    lib.tsgemm_run_mx_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.tsgemm_run_mx_noalloc.restype = i32
    lib.tsgemm_num_tiles.argtypes = [vp]
    lib.tsgemm_num_tiles.restype = i64
    lib.tsgemm_num_workgroups.argtypes = [vp]
    lib.tsgemm_num_workgroups.restype = i32
    lib.tsgemm_plan_info.argtypes = [vp, ctypes.POINTER(Info)]
    lib.tsgemm_plan_info.restype = i32
    lib.tsgemm_dump_schedule.argtypes = [vp, i32p]
    lib.tsgemm_dump_schedule.restype = i32
    lib.tsgemm_schedule_host.argtypes = [vp, i32, i32p]
    lib.tsgemm_schedule_host.restype = i32
    lib.tsgemm_destroy.argtypes = [vp]
    lib.tsgemm_destroy.restype = None
    lib.tsgemm_last_error.argtypes = []
    lib.tsgemm_last_error.restype = ctypes.c_char_p
    lib.tsgemm_last_error_code.argtypes = []
    lib.tsgemm_last_error_code.restype = i32
    lib.tsgemm_launch_info.argtypes = [vp, i32p, i32p, i32p]
    lib.tsgemm_launch_info.restype = i32
    lib.tsgemm_worker_numbering.argtypes = [i32, i32, i32, i32p]
    lib.tsgemm_worker_numbering.restype = i32
    if path is None:
        _lib = lib
    return lib


def last_error() -> str:
    return load().tsgemm_last_error().decode()


def _check(rc: int) -> int:
    if rc < 0:
        raise TsgemmError(rc, last_error())
    return rc


_DTYPES = {"fp16": FP16, "bf16": BF16, "mxfp8": MXFP8, FP16: FP16, BF16: BF16, MXFP8: MXFP8}


class Plan:
    """A validated problem (tsgemm_create).  Immutable once configured."""

    def __init__(self, M: int, N: int, K: int, dtype, block_M: int, block_N: int, block_K: int,
                 group_size: int, num_stages: int, num_workgroups: int = 0, xcd_remap: bool = True,
                 waves: int = 0, column_major: bool = False, cluster_size: int = 1, store_block_N: int = 0,
                 l2_prefetch: bool | None = None):
        lib = load()
        self._lib = lib
        dt = _DTYPES.get(dtype)
        if dt is None:
            import torch
            dt = {torch.float16: FP16, torch.bfloat16: BF16}.get(dtype, 0)
        h = lib.tsgemm_create(M, N, K, dt, block_M, block_N, block_K, group_size, num_stages)
        if not h:
            raise TsgemmError(lib.tsgemm_last_error_code(), last_error())
        self._h = ctypes.c_void_p(h)
        self.M, self.N, self.K, self.dtype = M, N, K, dt
        if num_workgroups:
            _check(lib.tsgemm_set_num_workgroups(self._h, num_workgroups))
        _check(lib.tsgemm_set_xcd_remap(self._h, 1 if xcd_remap else 0))
        if waves:
            _check(lib.tsgemm_set_waves(self._h, waves))
        if column_major or cluster_size != 1:
            _check(lib.tsgemm_set_schedule(self._h, 1 if column_major else 0, cluster_size))
        if store_block_N:
            _check(lib.tsgemm_set_epilogue(self._h, store_block_N))
        if l2_prefetch is not None:
            _check(lib.tsgemm_set_l2_prefetch(self._h, 1 if l2_prefetch else 0))

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.tsgemm_destroy(h)
            self._h = None

    # -- queries -------------------------------------------------------------
    @property
    def num_tiles(self) -> int:
        return _check(self._lib.tsgemm_num_tiles(self._h))

    @property
    def num_workgroups(self) -> int:
        return _check(self._lib.tsgemm_num_workgroups(self._h))

    def info(self) -> dict:
        inf = Info()
        _check(self._lib.tsgemm_plan_info(self._h, ctypes.byref(inf)))
        return inf.as_dict()

    # -- schedule ------------------------------------------------------------
    def schedule_host(self, num_workgroups: int) -> np.ndarray:
        out = np.empty((self.num_tiles, 4), dtype=np.int32)
        _check(self._lib.tsgemm_schedule_host(self._h, num_workgroups,
                                              out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
        return out

    def dump_schedule(self) -> np.ndarray:
        out = np.empty((self.num_tiles, 4), dtype=np.int32)
        _check(self._lib.tsgemm_dump_schedule(self._h, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
        return out

    def launch_info(self) -> dict:
        """tsgemm_launch_info: the grid a run uses on the current device."""
        P, it, x = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.tsgemm_launch_info(self._h, ctypes.byref(P), ctypes.byref(it), ctypes.byref(x)))
        return {"num_workgroups": P.value, "max_iters": it.value, "num_xcds": x.value}

    def trace_rows(self) -> int:
        """Rows (of 4 int32) a traced run may write: P * max_iters."""
        P, it = ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.tsgemm_launch_info(self._h, ctypes.byref(P), ctypes.byref(it), None))
        return P.value * it.value

    def _check_trace(self, trace):
        import torch
        if trace.dtype != torch.int32 or not trace.is_cuda or not trace.is_contiguous():
            raise ValueError("trace must be a contiguous int32 CUDA tensor")
        need = 4 * self.trace_rows()
        if trace.numel() < need:
            raise ValueError(f"trace holds {trace.numel()} int32, the run may write {need}")
        return trace.data_ptr()

    # -- run -----------------------------------------------------------------
    def _args(self, A, B, C):
        import torch
        if self.dtype == MXFP8:
            raise ValueError("an MXFP8 plan runs with run_mx")
        want = torch.float16 if self.dtype == FP16 else torch.bfloat16
        for name, t, shape in (("A", A, (self.M, self.K)), ("B", B, (self.K, self.N)), ("C", C, (self.M, self.N))):
            if t.dtype != want or tuple(t.shape) != shape or not t.is_contiguous() or not t.is_cuda:
                raise ValueError(f"{name} must be a contiguous {want} CUDA tensor of shape {shape}")
        return A.data_ptr(), B.data_ptr(), C.data_ptr()

    def run(self, A, B, C, stream=None) -> None:
        """C = A @ B on `stream` (a torch.cuda.Stream; default: torch's current stream)."""
        import torch
        a, b, c = self._args(A, B, C)
        s = (stream or torch.cuda.current_stream(C.device)).cuda_stream
        _check(self._lib.tsgemm_run(self._h, a, b, c, s))

    def run_traced(self, A, B, C, trace, stream=None) -> None:
        import torch
        a, b, c = self._args(A, B, C)
        t = self._check_trace(trace)
        s = (stream or torch.cuda.current_stream(C.device)).cuda_stream
        _check(self._lib.tsgemm_run_traced(self._h, a, b, c, s, t))

    def _mx_args(self, A, SFA, B, SFB, C):
        import torch
        if self.dtype != MXFP8:
            raise ValueError("run_mx needs a plan created with dtype 'mxfp8'")
        M, N, K = self.M, self.N, self.K
        out = []
        for name, t, shape in (("A", A, (M, K)), ("SFA", SFA, (M, K // 32)),
                               ("B", B, (N, K)), ("SFB", SFB, (N, K // 32))):
            if t.element_size() != 1 or t.dtype == torch.bool or tuple(t.shape) != shape \
                    or not t.is_contiguous() or not t.is_cuda:
                raise ValueError(f"{name} must be a contiguous 1-byte CUDA tensor of shape {shape}")
            out.append(t.data_ptr())
        if C.dtype != torch.bfloat16 or tuple(C.shape) != (M, N) or not C.is_contiguous() or not C.is_cuda:
            raise ValueError(f"C must be a contiguous torch.bfloat16 CUDA tensor of shape {(M, N)}")
        return out + [C.data_ptr()]

    def run_mx(self, A, SFA, B, SFB, C, stream=None) -> None:
        """Block-scaled FP8 product (tsgemm_run_mx): A[M,K], B[N,K] E4M3 codes,
        SFA[M,K/32], SFB[N,K/32] E8M0 codes (any 1-byte dtype), C[M,N] bf16."""
        import torch
        a, sa, b, sb, c = self._mx_args(A, SFA, B, SFB, C)
        s = (stream or torch.cuda.current_stream(C.device)).cuda_stream
        _check(self._lib.tsgemm_run_mx(self._h, a, sa, b, sb, c, s))

    def run_mx_noalloc(self, A, SFA, B, SFB, C, stream=None) -> None:
        """tsgemm_run_mx_noalloc: run_mx through the packed-scale kernel with the
        packed scales in the library's static workspace (allocates nothing)."""
        import torch
        a, sa, b, sb, c = self._mx_args(A, SFA, B, SFB, C)
        s = (stream or torch.cuda.current_stream(C.device)).cuda_stream
        _check(self._lib.tsgemm_run_mx_noalloc(self._h, a, sa, b, sb, c, s))

    def mx_packed_scale_bytes(self, operand: int) -> int:
        """Bytes of the packed scale array of operand 0 (SFA) or 1 (SFB)."""
        return _check(self._lib.tsgemm_mx_packed_scale_bytes(self._h, operand))

    def mx_pack_scales(self, SF, SFP, operand: int, stream=None) -> None:
        """tsgemm_mx_pack_scales: SF [rows, K/32] (1-byte, CUDA) -> SFP (1-byte CUDA tensor of
        mx_packed_scale_bytes(operand) bytes)."""
        import torch
        rows = self.M if operand == 0 else self.N
        if SF.element_size() != 1 or tuple(SF.shape) != (rows, self.K // 32) or not SF.is_contiguous() \
                or not SF.is_cuda:
            raise ValueError(f"SF must be a contiguous 1-byte CUDA tensor of shape {(rows, self.K // 32)}")
        need = self.mx_packed_scale_bytes(operand)
        if SFP.element_size() != 1 or SFP.numel() != need or not SFP.is_contiguous() or not SFP.is_cuda:
            raise ValueError(f"SFP must be a contiguous 1-byte CUDA tensor of {need} bytes")
        s = (stream or torch.cuda.current_stream(SFP.device)).cuda_stream
        _check(self._lib.tsgemm_mx_pack_scales(self._h, operand, SF.data_ptr(), SFP.data_ptr(), s))

    def run_mx_packed(self, A, SFAP, B, SFBP, C, stream=None) -> None:
        """tsgemm_run_mx_packed: as run_mx with scales from mx_pack_scales."""
        import torch
        if self.dtype != MXFP8:
            raise ValueError("run_mx_packed needs a plan created with dtype 'mxfp8'")
        for name, t, shape in (("A", A, (self.M, self.K)), ("B", B, (self.N, self.K))):
            if t.element_size() != 1 or tuple(t.shape) != shape or not t.is_contiguous() or not t.is_cuda:
                raise ValueError(f"{name} must be a contiguous 1-byte CUDA tensor of shape {shape}")
        for name, t, op in (("SFAP", SFAP, 0), ("SFBP", SFBP, 1)):
            need = self.mx_packed_scale_bytes(op)
            if t.element_size() != 1 or t.numel() != need or not t.is_contiguous() or not t.is_cuda:
                raise ValueError(f"{name} must be a contiguous 1-byte CUDA tensor of {need} bytes")
        if C.dtype != torch.bfloat16 or tuple(C.shape) != (self.M, self.N) or not C.is_contiguous() or not C.is_cuda:
            raise ValueError(f"C must be a contiguous torch.bfloat16 CUDA tensor of shape {(self.M, self.N)}")
        s = (stream or torch.cuda.current_stream(C.device)).cuda_stream
        _check(self._lib.tsgemm_run_mx_packed(self._h, A.data_ptr(), SFAP.data_ptr(), B.data_ptr(),
                                              SFBP.data_ptr(), C.data_ptr(), s))

    def run_mx_traced(self, A, SFA, B, SFB, C, trace, stream=None) -> None:
        import torch
        a, sa, b, sb, c = self._mx_args(A, SFA, B, SFB, C)
        t = self._check_trace(trace)
        s = (stream or torch.cuda.current_stream(C.device)).cuda_stream
        _check(self._lib.tsgemm_run_mx_traced(self._h, a, sa, b, sb, c, s, t))


def worker_numbering(num_workgroups: int, num_xcds: int, num_active: int) -> np.ndarray:
    """tsgemm_worker_numbering: the worker id of every workgroup."""
    out = np.empty(num_workgroups, dtype=np.int32)
    _check(load().tsgemm_worker_numbering(num_workgroups, num_xcds, num_active,
                                          out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
    return out


def matmul(A, B, block_M=256, block_N=256, block_K=64, group_size=8, num_stages=3):
    """Convenience: C = A @ B with a fresh plan (allocates C with torch)."""
    import torch
    M, K = A.shape
    N = B.shape[1]
    plan = Plan(M, N, K, A.dtype, block_M, block_N, block_K, group_size, num_stages)
    C = torch.empty((M, N), dtype=A.dtype, device=A.device)
    plan.run(A, B, C)
    return C
