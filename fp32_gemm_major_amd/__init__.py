"""MI355X (gfx950) FP32 GEMM: Python binding of the C ABI in include/sgemm.h.

C = alpha * A * B + beta * C for row-major FP32 operands ("GEMM 优化之路",
problem statement), and the same product with bfloat16 or float16 A and B and
FP32 C (the gsyq.cn guide, section 5.1).  Every step runs in the HIP library ``libsgemm.so``; this
module only marshals arguments.  PyTorch provides device memory and streams.
There is no fallback: if the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (load torch's HIP runtime before the library)

from .build import LIBRARY

SGEMM_OK = 0
SGEMM_ERR_HANDLE = -1
SGEMM_ERR_SIZE = -2
SGEMM_ERR_LD = -3
SGEMM_ERR_NULL = -4
SGEMM_ERR_HIP = -5
SGEMM_ERR_DEVICE = -6
SGEMM_ERR_VALUE = -7
SGEMM_ERR_ALIAS = -8
SGEMM_ERR_UNSUPPORTED = -9
SGEMM_ERR_SCRATCH = -10
SGEMM_SCRATCH_BYTES = 16 << 20

SGEMM_OP_N = 0
SGEMM_OP_T = 1

SGEMM_VARIANT_AUTO = 0
SGEMM_VARIANT_MFMA = 1
SGEMM_VARIANT_VALU = 2

SGEMM_MODE_ALIGNED = 0
SGEMM_MODE_EDGE = 1
SGEMM_MODE_GUARDED = 2

SGEMM_DTYPE_BF16 = 1
SGEMM_DTYPE_F16 = 2
SGEMM_DTYPE_FP8_E4M3 = 3
SGEMM_DTYPE_FP8_E5M2 = 4

SGEMM_SCHEDULE_TILES = 0
SGEMM_SCHEDULE_STREAM_K = 1
SGEMM_SCHEDULE_SMALL_M = 2

EXPORTED = [
    "sgemm_create", "sgemm_run", "sgemm_run_ex", "sgemm_destroy", "sgemm_validate",
    "sgemm_validate_ex", "sgemm_plan_ex",
    "sgemm_status_string", "sgemm_num_kernels", "sgemm_kernel_name",
    "sgemm_kernel_info", "sgemm_plan", "sgemm_select_kernel", "sgemm_tile_coords",
    "sgemm_set_variant", "sgemm_set_kernel", "sgemm_diag_mfma_chain",
    "sgemm_set_workspace", "sgemm_workspace_size", "sgemm_plan_handle",
    "sgemm_kernel_schedule", "sgemm_run_lowp", "sgemm_validate_lowp",
    "sgemm_lowp_num_kernels", "sgemm_lowp_kernel_name", "sgemm_lowp_kernel_info",
    "sgemm_lowp_select_kernel", "sgemm_set_lowp_kernel", "sgemm_diag_mfma_chain_lowp",
    "sgemm_diag_run_clocked", "sgemm_diag_wall_clock_khz", "sgemm_run_ex_noalloc",
    "sgemm_lowp_kernel_schedule", "sgemm_lowp_plan_handle",
]


class SgemmError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


_lib = None


def _bind(lib):
    i, f, p = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    ip = ctypes.POINTER(ctypes.c_int)
    lib.sgemm_create.argtypes = [ctypes.POINTER(p)]
    lib.sgemm_run.argtypes = [p, i, i, i, f, p, i, p, i, f, p, i, p]
    lib.sgemm_run_ex.argtypes = [p, i, i, i, i, i, f, p, i, p, i, f, p, i, p]
    lib.sgemm_run_ex_noalloc.argtypes = lib.sgemm_run_ex.argtypes
    lib.sgemm_validate_ex.argtypes = [i, i, i, i, i, p, i, p, i, f, p, i]
    lib.sgemm_plan_ex.argtypes = [i, i, i, i, i, i, p, i, p, i, p, i, ip, ip]
    lib.sgemm_destroy.argtypes = [p]
    lib.sgemm_validate.argtypes = [i, i, i, p, i, p, i, f, p, i]
    lib.sgemm_status_string.argtypes = [i]
    lib.sgemm_status_string.restype = ctypes.c_char_p
    lib.sgemm_num_kernels.argtypes = []
    lib.sgemm_kernel_name.argtypes = [i]
    lib.sgemm_kernel_name.restype = ctypes.c_char_p
    lib.sgemm_kernel_info.argtypes = [i, ip, ip, ip, ip, ip, ip, ip, ip]
    lib.sgemm_select_kernel.argtypes = [i, i, i, i, p, i, p, i, p, i]
    lib.sgemm_plan.argtypes = [i, i, i, i, p, i, p, i, p, i, ip, ip]
    lib.sgemm_tile_coords.argtypes = [i, i, i, i, ip, ip]
    lib.sgemm_tile_coords.restype = None
    lib.sgemm_set_variant.argtypes = [p, i]
    lib.sgemm_set_kernel.argtypes = [p, i]
    lib.sgemm_diag_mfma_chain.argtypes = [i, i, p, p]
    lib.sgemm_set_workspace.argtypes = [p, p, ctypes.c_size_t]
    lib.sgemm_workspace_size.argtypes = [p, ctypes.POINTER(ctypes.c_size_t)]
    lib.sgemm_plan_handle.argtypes = [p, i, i, i, i, i, p, i, p, i, p, i, ip, ip]
    lib.sgemm_kernel_schedule.argtypes = [i]
    lib.sgemm_run_lowp.argtypes = [p, i, i, i, i, i, i, f, p, i, p, i, f, p, i, p]
    lib.sgemm_validate_lowp.argtypes = [i, i, i, i, i, i, p, i, p, i, f, p, i]
    lib.sgemm_lowp_num_kernels.argtypes = []
    lib.sgemm_lowp_kernel_name.argtypes = [i]
    lib.sgemm_lowp_kernel_name.restype = ctypes.c_char_p
    lib.sgemm_lowp_kernel_info.argtypes = [i, ip, ip, ip, ip, ip, ip, ip, ip]
    lib.sgemm_lowp_select_kernel.argtypes = [i, i, i, i, i, i, p, i, p, i, p, i]
    lib.sgemm_set_lowp_kernel.argtypes = [p, i]
    lib.sgemm_diag_mfma_chain_lowp.argtypes = [i, i, i, p, p]
    lib.sgemm_lowp_kernel_schedule.argtypes = [i]
    lib.sgemm_lowp_plan_handle.argtypes = [p, i, i, i, i, i, i, p, i, p, i, p, i, ip, ip]
    lib.sgemm_diag_run_clocked.argtypes = [p, i, i, i, i, i, f, p, i, p, i, f, p, i, p, i, p]
    lib.sgemm_diag_wall_clock_khz.argtypes = [ip]
    for name in ("sgemm_lowp_kernel_schedule", "sgemm_lowp_plan_handle",
                 "sgemm_diag_run_clocked", "sgemm_diag_wall_clock_khz", "sgemm_run_ex_noalloc",
                 "sgemm_run_lowp", "sgemm_diag_mfma_chain_lowp", "sgemm_validate_lowp", "sgemm_lowp_num_kernels",
                 "sgemm_lowp_kernel_info", "sgemm_lowp_select_kernel",
                 "sgemm_set_lowp_kernel"):
        getattr(lib, name).restype = i
    for name in ("sgemm_create", "sgemm_run", "sgemm_destroy", "sgemm_validate",
                 "sgemm_num_kernels", "sgemm_kernel_info", "sgemm_select_kernel",
                 "sgemm_plan", "sgemm_diag_mfma_chain", "sgemm_run_ex",
                 "sgemm_validate_ex", "sgemm_plan_ex",
                 "sgemm_set_variant", "sgemm_set_kernel", "sgemm_set_workspace",
                 "sgemm_workspace_size", "sgemm_plan_handle", "sgemm_kernel_schedule"):
        getattr(lib, name).restype = i
    return lib


def library(path: str = LIBRARY):
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is missing: build it with `python -m fp32_gemm_major_amd.build`"
                " (or __graft_entry__.build()); there is no fallback path")
        _lib = _bind(ctypes.CDLL(path))
    return _lib


def _check(status: int, what: str) -> int:
    if status < 0:
        raise SgemmError(status, what)
    return status


# ---- the C ABI, name for name -------------------------------------------------

def sgemm_create() -> int:
    h = ctypes.c_void_p()
    _check(library().sgemm_create(ctypes.byref(h)), "sgemm_create")
    return h.value


def sgemm_run(h, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    """Enqueue on ``stream`` (an int hipStream_t); A, B, C are device addresses."""
    return _check(library().sgemm_run(h, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                      ldc, stream), "sgemm_run")


def sgemm_run_ex(h, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                 stream=0) -> int:
    """sgemm_run with operand storage flags (SGEMM_OP_N / SGEMM_OP_T)."""
    return _check(library().sgemm_run_ex(h, transa, transb, M, N, K, alpha, A, lda,
                                         B, ldb, beta, C, ldc, stream),
                  "sgemm_run_ex")


def sgemm_run_ex_noalloc(h, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C,
                         ldc, stream=0) -> int:
    """sgemm_run_ex with the library's fixed scratch buffer in place of the
    handle's workspace (no device allocation anywhere in the call); A, B, C
    are device addresses."""
    return _check(library().sgemm_run_ex_noalloc(h, transa, transb, M, N, K, alpha, A,
                                                 lda, B, ldb, beta, C, ldc, stream),
                  "sgemm_run_ex_noalloc")


def sgemm_run_lowp(h, dtype, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C,
                   ldc, stream=0) -> int:
    """The product with 16-bit A and B (SGEMM_DTYPE_BF16 / SGEMM_DTYPE_F16) or
    8-bit A and B (SGEMM_DTYPE_FP8_E4M3 / SGEMM_DTYPE_FP8_E5M2), any storage,
    and FP32 C; A, B, C are device addresses."""
    return _check(library().sgemm_run_lowp(h, dtype, transa, transb, M, N, K, alpha,
                                           A, lda, B, ldb, beta, C, ldc, stream),
                  "sgemm_run_lowp")


def sgemm_validate_lowp(dtype, transa, transb, M, N, K, A, lda, B, ldb, beta, C,
                        ldc) -> int:
    return library().sgemm_validate_lowp(dtype, transa, transb, M, N, K, A, lda, B,
                                         ldb, beta, C, ldc)


def sgemm_lowp_num_kernels() -> int:
    return library().sgemm_lowp_num_kernels()


def sgemm_lowp_kernel_name(kernel_id: int):
    s = library().sgemm_lowp_kernel_name(kernel_id)
    return s.decode() if s is not None else None


def sgemm_lowp_kernel_schedule(kernel_id: int) -> int:
    return _check(library().sgemm_lowp_kernel_schedule(kernel_id),
                  "sgemm_lowp_kernel_schedule")


def sgemm_lowp_plan_handle(h, dtype, transa, transb, M, N, K, A, lda, B, ldb, C, ldc):
    """(kernel id, K splits) of the launch sgemm_run_lowp makes on handle h."""
    kid, splits = ctypes.c_int(), ctypes.c_int()
    _check(library().sgemm_lowp_plan_handle(h, dtype, transa, transb, M, N, K, A, lda, B,
                                            ldb, C, ldc, ctypes.byref(kid),
                                            ctypes.byref(splits)),
           "sgemm_lowp_plan_handle")
    return kid.value, splits.value


def sgemm_lowp_kernel_info(kernel_id: int) -> dict:
    vals = [ctypes.c_int() for _ in range(8)]
    _check(library().sgemm_lowp_kernel_info(kernel_id, *[ctypes.byref(v) for v in vals]),
           "sgemm_lowp_kernel_info")
    keys = ("dtype", "bm", "bn", "bk", "threads", "mode", "transa", "transb")
    d = {k: v.value for k, v in zip(keys, vals)}
    d["schedule"] = sgemm_lowp_kernel_schedule(kernel_id)
    d["name"] = sgemm_lowp_kernel_name(kernel_id)
    d["id"] = kernel_id
    return d


def sgemm_lowp_select_kernel(dtype, transa, transb, M, N, K, A, lda, B, ldb, C,
                             ldc) -> int:
    return library().sgemm_lowp_select_kernel(dtype, transa, transb, M, N, K, A, lda,
                                              B, ldb, C, ldc)


def sgemm_set_lowp_kernel(h, kernel_id: int) -> int:
    return _check(library().sgemm_set_lowp_kernel(h, kernel_id), "sgemm_set_lowp_kernel")


def sgemm_destroy(h) -> int:
    return library().sgemm_destroy(h)


def sgemm_set_workspace(h, ptr, nbytes) -> int:
    """Device memory (address, bytes) for stream-K partial tiles; 0, 0 removes it."""
    return _check(library().sgemm_set_workspace(h, ptr or None, nbytes),
                  "sgemm_set_workspace")


def sgemm_workspace_size(h) -> int:
    n = ctypes.c_size_t()
    _check(library().sgemm_workspace_size(h, ctypes.byref(n)), "sgemm_workspace_size")
    return n.value


def sgemm_plan_handle(h, M, N, K, A, lda, B, ldb, C, ldc, transa=0, transb=0):
    """The launches sgemm_run_ex makes on handle h: [(kernel, first column,
    columns), ...]."""
    ks = (ctypes.c_int * 2)()
    n_split = ctypes.c_int()
    n = _check(library().sgemm_plan_handle(h, transa, transb, M, N, K, A, lda, B, ldb,
                                           C, ldc, ks, ctypes.byref(n_split)),
               "sgemm_plan_handle")
    if n == 0:
        return []
    if n == 1:
        return [(ks[0], 0, N)]
    return [(ks[0], 0, n_split.value), (ks[1], n_split.value, N - n_split.value)]


def sgemm_kernel_schedule(kernel_id: int) -> int:
    return _check(library().sgemm_kernel_schedule(kernel_id), "sgemm_kernel_schedule")


def sgemm_validate(M, N, K, A, lda, B, ldb, beta, C, ldc) -> int:
    return library().sgemm_validate(M, N, K, A, lda, B, ldb, beta, C, ldc)


def sgemm_validate_ex(transa, transb, M, N, K, A, lda, B, ldb, beta, C, ldc) -> int:
    return library().sgemm_validate_ex(transa, transb, M, N, K, A, lda, B, ldb, beta,
                                       C, ldc)


def sgemm_status_string(status: int) -> str:
    return library().sgemm_status_string(status).decode()


status_string = sgemm_status_string


def sgemm_num_kernels() -> int:
    return library().sgemm_num_kernels()


def sgemm_kernel_name(kernel_id: int):
    s = library().sgemm_kernel_name(kernel_id)
    return s.decode() if s is not None else None


def sgemm_kernel_info(kernel_id: int) -> dict:
    vals = [ctypes.c_int() for _ in range(8)]
    _check(library().sgemm_kernel_info(kernel_id, *[ctypes.byref(v) for v in vals]),
           "sgemm_kernel_info")
    keys = ("variant", "bm", "bn", "bk", "threads", "mode", "transa", "transb")
    d = {k: v.value for k, v in zip(keys, vals)}
    d["schedule"] = sgemm_kernel_schedule(kernel_id)
    d["name"] = sgemm_kernel_name(kernel_id)
    d["id"] = kernel_id
    return d


def sgemm_select_kernel(variant, M, N, K, A, lda, B, ldb, C, ldc) -> int:
    return library().sgemm_select_kernel(variant, M, N, K, A, lda, B, ldb, C, ldc)


def sgemm_plan(variant, M, N, K, A, lda, B, ldb, C, ldc, transa=0, transb=0):
    """Launches sgemm_run(_ex) would make: a list of (kernel id, first column, columns)."""
    kernels = (ctypes.c_int * 2)()
    split = ctypes.c_int()
    n = _check(library().sgemm_plan_ex(variant, transa, transb, M, N, K, A, lda, B,
                                       ldb, C, ldc, kernels, ctypes.byref(split)),
               "sgemm_plan")
    if n == 1:
        return [(kernels[0], 0, N)]
    return [(kernels[0], 0, split.value), (kernels[1], split.value, N - split.value)]


def sgemm_tile_coords(wg, nwg, tiles_m, tiles_n):
    tm, tn = ctypes.c_int(), ctypes.c_int()
    library().sgemm_tile_coords(wg, nwg, tiles_m, tiles_n, ctypes.byref(tm),
                                ctypes.byref(tn))
    return tm.value, tn.value


def sgemm_set_variant(h, variant: int) -> int:
    return _check(library().sgemm_set_variant(h, variant), "sgemm_set_variant")


def sgemm_set_kernel(h, kernel_id: int) -> int:
    return _check(library().sgemm_set_kernel(h, kernel_id), "sgemm_set_kernel")


def sgemm_diag_mfma_chain(workgroups, iterations, out, stream=0) -> int:
    return _check(library().sgemm_diag_mfma_chain(workgroups, iterations, out, stream),
                  "sgemm_diag_mfma_chain")


CHAIN_FLOPS_PER_WAVE_ITER = 8 * 2 * 32 * 32 * 2  # eight 32x32x2 MFMAs


def sgemm_diag_mfma_chain_lowp(dtype, workgroups, iterations, out, stream=0) -> int:
    return _check(library().sgemm_diag_mfma_chain_lowp(dtype, workgroups, iterations,
                                                       out, stream),
                  "sgemm_diag_mfma_chain_lowp")


def sgemm_diag_run_clocked(h, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C,
                           ldc, stamps, stamp_slots, stream=0) -> int:
    """sgemm_run_ex that also stores per-workgroup clock stamps; returns the
    number of workgroups stamped."""
    return _check(library().sgemm_diag_run_clocked(h, transa, transb, M, N, K, alpha, A,
                                                   lda, B, ldb, beta, C, ldc, stamps,
                                                   stamp_slots, stream),
                  "sgemm_diag_run_clocked")


def sgemm_diag_wall_clock_khz() -> int:
    khz = ctypes.c_int()
    _check(library().sgemm_diag_wall_clock_khz(ctypes.byref(khz)),
           "sgemm_diag_wall_clock_khz")
    return khz.value


def clock_from_stamps(stamps, workgroups, wall_khz):
    """(median shader clock in GHz over the workgroups, the launch's span in
    microseconds from the first start to the last end) from the stamps of
    sgemm_diag_run_clocked (a CPU int64 tensor or array of 4 per workgroup)."""
    t = torch.as_tensor(stamps).view(-1, 4)[:workgroups].double()
    cycles, ticks = t[:, 1] - t[:, 0], t[:, 3] - t[:, 2]
    ok = ticks > 0
    ghz = float((cycles[ok] / ticks[ok]).median()) * wall_khz * 1e3 / 1e9
    span_us = float(t[:, 3].max() - t[:, 2].min()) / (wall_khz * 1e3) * 1e6
    return ghz, span_us


CHAIN16_FLOPS_PER_WAVE_ITER = 8 * 2 * 32 * 32 * 16  # eight 32x32x16 MFMAs
CHAIN8_FLOPS_PER_WAVE_ITER = 8 * 2 * 32 * 32 * 64  # eight 32x32x64 MFMAs


def mfma_chain_tflops(workgroups=1024, iterations=4096, reps=3, dtype=None):
    """Sustained MFMA TFLOP/s of the device (best of ``reps`` timed runs):
    FP32 32x32x2 by default, or the 16-bit 32x32x16 instruction of ``dtype``
    (SGEMM_DTYPE_BF16 / SGEMM_DTYPE_F16), or the 8-bit 32x32x64 one
    (SGEMM_DTYPE_FP8_E4M3 / SGEMM_DTYPE_FP8_E5M2)."""
    out = torch.empty(workgroups * 256, device="cuda")
    stream = torch.cuda.current_stream()

    def run():
        if dtype is None:
            sgemm_diag_mfma_chain(workgroups, iterations, out.data_ptr(),
                                  stream.cuda_stream)
        else:
            sgemm_diag_mfma_chain_lowp(dtype, workgroups, iterations, out.data_ptr(),
                                       stream.cuda_stream)
    run()
    best = None
    for _ in range(reps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        run()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e)
        best = ms if best is None else min(best, ms)
    per = (CHAIN_FLOPS_PER_WAVE_ITER if dtype is None else
           CHAIN8_FLOPS_PER_WAVE_ITER if dtype >= SGEMM_DTYPE_FP8_E4M3 else
           CHAIN16_FLOPS_PER_WAVE_ITER)
    flops = per * iterations * workgroups * 4
    return flops / (best * 1e-3) / 1e12


# ---- torch-tensor convenience ------------------------------------------------

class Handle:
    """Owns one sgemm handle; usable as a context manager.

    With ``workspace=True`` (the default) it also owns a device tensor of
    sgemm_workspace_size bytes, set as the handle's stream-K workspace, so
    stream-K plans are available.  Calls through one Handle share it: use
    separate Handles for calls that may overlap on different streams."""

    def __init__(self, variant: int = SGEMM_VARIANT_AUTO, kernel: int = -1,
                 workspace: bool = True):
        self.h = sgemm_create()
        self.workspace = None
        self._stamps = None
        if variant != SGEMM_VARIANT_AUTO:
            sgemm_set_variant(self.h, variant)
        if kernel >= 0:
            sgemm_set_kernel(self.h, kernel)
        if workspace:
            self.set_workspace(sgemm_workspace_size(self.h))

    def set_workspace(self, nbytes: int):
        """Give the handle a fresh workspace of ``nbytes`` (0: none)."""
        sgemm_set_workspace(self.h, 0, 0)
        self.workspace = None
        if nbytes:
            self.workspace = torch.empty((nbytes + 3) // 4, dtype=torch.float32,
                                         device="cuda")
            sgemm_set_workspace(self.h, self.workspace.data_ptr(), nbytes)

    def plan(self, M, N, K, A, lda, B, ldb, C, ldc, transa=False, transb=False):
        return sgemm_plan_handle(self.h, M, N, K, A, lda, B, ldb, C, ldc,
                                 int(bool(transa)), int(bool(transb)))

    def close(self):
        if self.h:
            sgemm_destroy(self.h)
            self.h = None
        self.workspace = None
        self._stamps = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_variant(self, variant: int):
        sgemm_set_variant(self.h, variant)

    def set_kernel(self, kernel_id: int):
        sgemm_set_kernel(self.h, kernel_id)

    def gemm(self, A, B, C, alpha=1.0, beta=0.0, M=None, N=None, K=None,
             lda=None, ldb=None, ldc=None, stream=None, transa=False, transb=False):
        """C[:M, :N] = alpha * op(A) @ op(B) + beta * C on ``stream``.

        A, B, C are float32 CUDA tensors.  op(A) is A, or A^T when ``transa``
        (A stored K x M); op(B) likewise (B stored N x K when ``transb``).
        2-D tensors with unit column stride give their sizes and leading
        dimensions; 1-D buffers need explicit sizes and leading dimensions.
        ``stream`` defaults to torch's current stream.  Returns immediately
        (the work is queued on the stream).
        """
        for name, t in (("A", A), ("B", B), ("C", C)):
            if t.dtype != torch.float32 or not t.is_cuda:
                raise TypeError(f"{name} must be a float32 CUDA tensor")
            if t.dim() == 2 and t.numel() and t.stride(1) != 1:
                raise ValueError(f"{name} must be row-major (unit column stride)")
        M, N, K, lda, ldb, ldc = _shapes(A, B, C, M, N, K, lda, ldb, ldc, transa,
                                         transb)
        if stream is None:
            stream = torch.cuda.current_stream(C.device).cuda_stream
        elif isinstance(stream, torch.cuda.Stream):
            stream = stream.cuda_stream
        return sgemm_run_ex(self.h, int(bool(transa)), int(bool(transb)), M, N, K,
                            float(alpha), A.data_ptr(), lda, B.data_ptr(), ldb,
                            float(beta), C.data_ptr(), ldc, stream)


    def gemm_stamped(self, A, B, C, stamps, alpha=1.0, beta=0.0, M=None, N=None, K=None,
                     lda=None, ldb=None, ldc=None, transa=False, transb=False):
        """``gemm`` through sgemm_diag_run_clocked: the product kernel also
        writes its clock stamps into ``stamps`` (an int64 CUDA tensor of
        4 per workgroup).  Returns the number of workgroups stamped without
        waiting; ``clock_from_stamps`` turns the stamps into a clock once the
        stream has finished the call."""
        for name, t in (("A", A), ("B", B), ("C", C)):
            if t.dtype != torch.float32 or not t.is_cuda:
                raise TypeError(f"{name} must be a float32 CUDA tensor")
        if stamps.dtype != torch.int64 or not stamps.is_cuda or not stamps.is_contiguous():
            raise TypeError("stamps must be a contiguous int64 CUDA tensor")
        M, N, K, lda, ldb, ldc = _shapes(A, B, C, M, N, K, lda, ldb, ldc, transa,
                                         transb)
        return sgemm_diag_run_clocked(self.h, int(bool(transa)), int(bool(transb)), M, N, K,
                                      float(alpha), A.data_ptr(), lda, B.data_ptr(), ldb,
                                      float(beta), C.data_ptr(), ldc, stamps.data_ptr(),
                                      stamps.numel() // 4,
                                      torch.cuda.current_stream(C.device).cuda_stream)

    def gemm_clocked(self, A, B, C, alpha=1.0, beta=0.0, **kw):
        """``gemm_stamped`` into a buffer of the handle's, then wait: returns
        (shader clock in GHz, the launch's span in microseconds) of that call,
        from the product kernel's own clock stamps."""
        if self._stamps is None:
            self._stamps = torch.zeros(4 * 65536, dtype=torch.int64, device="cuda")
        n = self.gemm_stamped(A, B, C, self._stamps, alpha, beta, **kw)
        return clock_from_stamps(self._stamps[: 4 * n].cpu(), n, sgemm_diag_wall_clock_khz())

    def set_lowp_kernel(self, kernel_id: int):
        sgemm_set_lowp_kernel(self.h, kernel_id)

    def gemm_lowp(self, A, B, C, alpha=1.0, beta=0.0, M=None, N=None, K=None,
                  lda=None, ldb=None, ldc=None, stream=None, transa=False,
                  transb=False):
        """C[:M, :N] = alpha * op(A) @ op(B) + beta * C with A and B bfloat16,
        float16, float8_e4m3fn or float8_e5m2 CUDA tensors (both the same
        format, any storage) and C a float32 CUDA tensor; shapes, leading
        dimensions and ``stream`` as in ``gemm``."""
        formats = {torch.bfloat16: SGEMM_DTYPE_BF16, torch.float16: SGEMM_DTYPE_F16,
                   torch.float8_e4m3fn: SGEMM_DTYPE_FP8_E4M3,
                   torch.float8_e5m2: SGEMM_DTYPE_FP8_E5M2}
        if A.dtype != B.dtype or A.dtype not in formats:
            raise TypeError("A and B must have one format: bfloat16, float16, "
                            "float8_e4m3fn or float8_e5m2")
        for name, t in (("A", A), ("B", B), ("C", C)):
            if not t.is_cuda:
                raise TypeError(f"{name} must be a CUDA tensor")
            if t.dim() == 2 and t.numel() and t.stride(1) != 1:
                raise ValueError(f"{name} must be row-major (unit column stride)")
        if C.dtype != torch.float32:
            raise TypeError("C must be a float32 CUDA tensor")
        M, N, K, lda, ldb, ldc = _shapes(A, B, C, M, N, K, lda, ldb, ldc, transa,
                                         transb)
        if stream is None:
            stream = torch.cuda.current_stream(C.device).cuda_stream
        elif isinstance(stream, torch.cuda.Stream):
            stream = stream.cuda_stream
        return sgemm_run_lowp(self.h, formats[A.dtype], int(bool(transa)),
                              int(bool(transb)), M, N, K, float(alpha), A.data_ptr(),
                              lda, B.data_ptr(), ldb, float(beta), C.data_ptr(), ldc,
                              stream)


def _span(rows, cols, ld):
    """Elements from the first to the last one a rows x cols window at
    leading dimension ``ld`` touches (0 for an empty window)."""
    return 0 if rows <= 0 or cols <= 0 else (rows - 1) * ld + cols


def _elements_from_pointer(t):
    """Elements of the tensor's storage from its data pointer to the end: the
    most any window starting at ``t.data_ptr()`` may span."""
    return t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()


def _shapes(A, B, C, M, N, K, lda, ldb, ldc, transa, transb):
    """Sizes and leading dimensions from 2-D tensors where not given, checked
    against the tensors: a 2-D operand must hold its stored window (A: M x K,
    or K x M when ``transa``; B: K x N, or N x K when ``transb``; C: M x N),
    2-D A and B must agree on K unless K is given, and every operand's window
    must fit in its storage from the data pointer on.  Raises ValueError
    otherwise, before anything reaches the device."""
    k_from = {}
    if A.dim() == 2:
        ra, ca = A.shape
        M = (ca if transa else ra) if M is None else M
        k_from["A"] = ra if transa else ca
        lda = max(A.stride(0), 1) if lda is None else lda
    if B.dim() == 2:
        rb, cb = B.shape
        k_from["B"] = cb if transb else rb
        N = (rb if transb else cb) if N is None else N
        ldb = max(B.stride(0), 1) if ldb is None else ldb
    if K is None:
        if len(set(k_from.values())) > 1:
            raise ValueError(f"A and B disagree on K: {k_from['A']} (A) and "
                             f"{k_from['B']} (B)")
        K = next(iter(k_from.values()), None)
    if C.dim() == 2:
        ldc = max(C.stride(0), 1) if ldc is None else ldc
    if None in (M, N, K, lda, ldb, ldc):
        raise ValueError("sizes and leading dimensions are needed for 1-D buffers")
    check_extents(A, B, C, M, N, K, lda, ldb, ldc, transa, transb)
    return M, N, K, lda, ldb, ldc


def check_extents(A, B, C, M, N, K, lda, ldb, ldc, transa, transb):
    """Raise ValueError if a tensor cannot hold the window the call would read
    or write (see ``_shapes``).  Negative sizes and short leading dimensions
    are left to the library's own checks, which return a status."""
    if min(M, N, K) < 0:
        return
    touched = M > 0 and N > 0
    stored = (("A", A, K if transa else M, M if transa else K, lda, touched and K > 0),
              ("B", B, N if transb else K, K if transb else N, ldb, touched and K > 0),
              ("C", C, M, N, ldc, touched))
    for name, t, rows, cols, ld, used in stored:
        if not used:
            continue
        if t.dim() == 2 and (rows > t.shape[0] or cols > t.shape[1]):
            raise ValueError(f"{name}: a {rows} x {cols} window does not fit its "
                             f"{t.shape[0]} x {t.shape[1]} tensor")
        need, have = _span(rows, cols, ld), _elements_from_pointer(t)
        if need > have:
            raise ValueError(f"{name}: the {rows} x {cols} window at leading dimension "
                             f"{ld} spans {need} elements, the tensor holds {have}")


def kernel_table() -> list:
    return [sgemm_kernel_info(i) for i in range(sgemm_num_kernels())]


def lowp_kernel_table() -> list:
    return [sgemm_lowp_kernel_info(i) for i in range(sgemm_lowp_num_kernels())]
