"""Thin Python binding of the C ABI in ``include/qlora_nf4.h``.

Functions carry the same names as the C entry points and only marshal
arguments: torch supplies device memory and the current HIP stream, every
step of the computation runs in the library's HIP kernels.  There is no CPU
or PyTorch fallback: if ``libqlora_nf4.so`` is missing or a call fails, an
exception is raised.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqlora_nf4.so")
# the same library built with QN_PROFILE_HOOK (qn_profile_kernel active)
PROF_LIB_PATH = os.path.join(_PKG, "libqlora_nf4_prof.so")
_use_prof = False

QN_OK, QN_EINVAL, QN_EWORKSPACE, QN_EHIP, QN_ENONFINITE = 0, -1, -2, -3, -4
QN_ESYNC = -5
QN_F32, QN_BF16 = 0, 1
QN_FWD, QN_BWD, QN_FWD_DROPOUT = 0, 1, 2
QN_BLOCK, QN_GROUP, QN_MAX_RANK = 64, 256, 256

# Every symbol the header declares (tests check the library exports them).
EXPORTS = ("nf4_codebook", "nf4_quantize", "nf4_dequantize",
           "nf4_dequantize_batch", "nf4_merge",
           "qn_codebook", "qn_quantize", "qn_dequantize",
           "qn_adamw8_step", "qn_adamw8_staging_bytes", "qn_adamw8_paged_step",
           "qlora_linear_fwd_dropout", "qlora_linear_bwd_dropout",
           "qlora_workspace_bytes", "qlora_linear_fwd", "qlora_linear_bwd",
           "qn_strerror", "qn_profile_kernel", "qlora_linear_fwd_noalloc",
           "qlora_fwd_batch_workspace_bytes", "qlora_linear_fwd_batch")
QN_FWD_BATCH_MAX = 8
QN_DEQUANT_BATCH_MAX = 16
QN_CODE_NF4, QN_CODE_FP4, QN_CODE_INT4 = 0, 1, 2
QN_CONST_DQ8, QN_CONST_FP32, QN_CONST_CENTERED = 0, 1, 2
QN_ADAMW_BLOCK = 256
QN_NOALLOC_SCRATCH_BYTES = 32 << 20


class _NF4Struct(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("qabs", ctypes.c_void_p),
                ("gscale", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64)]


class _QStruct(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("consts", ctypes.c_void_p),
                ("gscale", ctypes.c_void_p), ("gmean", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("code", ctypes.c_int32), ("consts_mode", ctypes.c_int32)]


class _AdamHP(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double),
                ("grad_scale", ctypes.c_double)]


class _Adam8State(ctypes.Structure):
    _fields_ = [("m_codes", ctypes.c_void_p), ("m_scale", ctypes.c_void_p),
                ("r_codes", ctypes.c_void_p), ("r_scale", ctypes.c_void_p)]


class _FwdJob(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("M", ctypes.c_int64),
                ("w", ctypes.POINTER(_NF4Struct)), ("A", ctypes.c_void_p),
                ("B", ctypes.c_void_p), ("r", ctypes.c_int32),
                ("alpha", ctypes.c_float), ("y", ctypes.c_void_p),
                ("y_dtype", ctypes.c_int32), ("t_save", ctypes.c_void_p)]


class _Dropout(ctypes.Structure):
    _fields_ = [("p", ctypes.c_double), ("seed", ctypes.c_uint64)]


_lib = None


def use_profiling_build() -> None:
    """Load the profiling variant (libqlora_nf4_prof.so, whose
    qn_profile_kernel records per-launch HIP events) instead of the default
    library.  Must be called before the first call into the library."""
    global _use_prof
    if _lib is not None and not _use_prof:
        raise RuntimeError("the default library is already loaded")
    _use_prof = True


def lib_path() -> str:
    return PROF_LIB_PATH if _use_prof else LIB_PATH


def lib() -> ctypes.CDLL:
    """Load the HIP library once; raise if it has not been built.

    torch is imported first: PyTorch ships its own HIP runtime, and the
    library's dependency on the HIP runtime must resolve to that one (which
    owns the streams and memory the calls receive).  Loaded before torch,
    the library would bind the system runtime, and its launches on torch's
    streams would fail."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m "
            "bit_nf4_quantized_14_amd.build` (hipcc, gfx950)")
    import torch  # noqa: F401  (binds torch's HIP runtime first)
    L = ctypes.CDLL(path)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    sp = ctypes.POINTER(_NF4Struct)
    L.nf4_codebook.argtypes = [vp, vp]
    L.nf4_codebook.restype = ctypes.c_int
    L.nf4_quantize.argtypes = [vp, sp, vp, vp]
    L.nf4_quantize.restype = ctypes.c_int
    L.nf4_dequantize.argtypes = [sp, vp, vp]
    L.nf4_dequantize.restype = ctypes.c_int
    L.nf4_dequantize_batch.argtypes = [sp, ctypes.POINTER(vp), i32, vp]
    L.nf4_dequantize_batch.restype = ctypes.c_int
    L.nf4_merge.argtypes = [sp, vp, vp, i32, f32, vp, vp]
    L.nf4_merge.restype = ctypes.c_int
    qp = ctypes.POINTER(_QStruct)
    L.qn_codebook.argtypes = [i32, vp, vp]
    L.qn_codebook.restype = ctypes.c_int
    L.qn_quantize.argtypes = [vp, qp, vp, vp]
    L.qn_quantize.restype = ctypes.c_int
    L.qn_dequantize.argtypes = [qp, vp, vp]
    L.qn_dequantize.restype = ctypes.c_int
    hpp, stp = ctypes.POINTER(_AdamHP), ctypes.POINTER(_Adam8State)
    L.qn_adamw8_step.argtypes = [vp, vp, i64, stp, hpp, i64, vp]
    L.qn_adamw8_step.restype = ctypes.c_int
    L.qn_adamw8_staging_bytes.argtypes = [i64]
    L.qn_adamw8_staging_bytes.restype = ctypes.c_size_t
    L.qn_adamw8_paged_step.argtypes = [vp, vp, i64, stp, vp, ctypes.c_size_t,
                                       i64, hpp, i64, vp, vp, vp]
    L.qn_adamw8_paged_step.restype = ctypes.c_int
    L.qlora_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
    L.qlora_workspace_bytes.restype = ctypes.c_size_t
    L.qlora_linear_fwd.argtypes = [vp, i64, sp, vp, vp, i32, f32, vp, i32, vp,
                                   vp, ctypes.c_size_t, vp]
    L.qlora_linear_fwd.restype = ctypes.c_int
    L.qlora_linear_bwd.argtypes = [vp, vp, i64, sp, vp, vp, i32, f32, vp, vp,
                                   i32, vp, vp, vp, ctypes.c_size_t, vp]
    L.qlora_linear_bwd.restype = ctypes.c_int
    dp = ctypes.POINTER(_Dropout)
    L.qlora_linear_fwd_dropout.argtypes = [vp, i64, sp, vp, vp, i32, f32, vp,
                                           i32, vp, dp, vp, ctypes.c_size_t, vp]
    L.qlora_linear_fwd_dropout.restype = ctypes.c_int
    L.qlora_linear_bwd_dropout.argtypes = [vp, vp, i64, sp, vp, vp, i32, f32,
                                           vp, vp, i32, vp, vp, dp, vp,
                                           ctypes.c_size_t, vp]
    L.qlora_linear_bwd_dropout.restype = ctypes.c_int
    jp = ctypes.POINTER(_FwdJob)
    L.qlora_fwd_batch_workspace_bytes.argtypes = [jp, i32]
    L.qlora_fwd_batch_workspace_bytes.restype = ctypes.c_size_t
    L.qlora_linear_fwd_batch.argtypes = [jp, i32, vp, ctypes.c_size_t, vp]
    L.qlora_linear_fwd_batch.restype = ctypes.c_int
    L.qlora_linear_fwd_noalloc.argtypes = [vp, i64, sp, vp, vp, i32, f32, vp,
                                           i32, vp, vp]
    L.qlora_linear_fwd_noalloc.restype = ctypes.c_int
    L.qn_profile_kernel.argtypes = [ctypes.c_char_p, vp, vp, i32]
    L.qn_profile_kernel.restype = ctypes.c_int
    L.qn_strerror.argtypes = [ctypes.c_int]
    L.qn_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


def qn_strerror(code: int) -> str:
    return lib().qn_strerror(int(code)).decode()


class QNError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn}: {qn_strerror(code)} ({code})")
        self.code = code


def _check(fn: str, code: int) -> None:
    if code != QN_OK:
        raise QNError(fn, code)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


@dataclass
class NF4Tensor:
    """Device buffers of an NF4 + double-quantized weight (see nf4_tensor in
    the header): packed codes, 8-bit block codes, fp32 group scales."""
    packed: "object"
    qabs: "object"
    gscale: "object"
    rows: int
    cols: int

    @property
    def numel(self) -> int:
        return self.rows * self.cols

    @staticmethod
    def sizes(rows: int, cols: int):
        numel = rows * cols
        nb = -(-numel // QN_BLOCK)
        return (numel + 1) // 2, nb, -(-nb // QN_GROUP)

    @classmethod
    def empty(cls, rows: int, cols: int, device="cuda"):
        import torch
        npk, nb, ng = cls.sizes(rows, cols)
        return cls(torch.empty(npk, dtype=torch.uint8, device=device),
                   torch.empty(nb, dtype=torch.uint8, device=device),
                   torch.empty(ng, dtype=torch.float32, device=device),
                   rows, cols)

    def as_struct(self) -> _NF4Struct:
        return _NF4Struct(self.packed.data_ptr(), self.qabs.data_ptr(),
                          self.gscale.data_ptr(), self.rows, self.cols)


def nf4_codebook():
    """(levels float32[16], thresholds float32[15]) from the library."""
    lv = np.zeros(16, dtype=np.float32)
    th = np.zeros(15, dtype=np.float32)
    _check("nf4_codebook", lib().nf4_codebook(lv.ctypes.data, th.ctypes.data))
    return lv, th


def nf4_quantize(w, out: NF4Tensor | None = None, status=None, stream=None):
    """Quantize a device fp32 weight [rows, cols]; returns the NF4Tensor."""
    rows, cols = (w.shape[0], w.shape[1]) if w.dim() == 2 else (1, w.numel())
    if out is None:
        out = NF4Tensor.empty(rows, cols, device=w.device)
    st = out.as_struct()
    _check("nf4_quantize", lib().nf4_quantize(_ptr(w), ctypes.byref(st),
                                              _ptr(status), _stream(stream)))
    return out


def nf4_dequantize(w: NF4Tensor, out=None, stream=None):
    """Dequantize to a bf16 device tensor [rows, cols]."""
    import torch
    if out is None:
        out = torch.empty((w.rows, w.cols), dtype=torch.bfloat16,
                          device=w.packed.device)
    st = w.as_struct()
    _check("nf4_dequantize", lib().nf4_dequantize(ctypes.byref(st), _ptr(out),
                                                  _stream(stream)))
    return out


def nf4_dequantize_batch(ws, outs=None, stream=None):
    """Dequantize several NF4 tensors in one launch; returns the bf16
    outputs (allocated when `outs` is None)."""
    import torch
    ws = list(ws)
    if outs is None:
        outs = [torch.empty((w.rows, w.cols), dtype=torch.bfloat16,
                            device=w.packed.device) for w in ws]
    structs = (_NF4Struct * len(ws))(*[w.as_struct() for w in ws])
    ptrs = (ctypes.c_void_p * len(ws))(*[_ptr(o) for o in outs])
    _check("nf4_dequantize_batch", lib().nf4_dequantize_batch(
        structs, ptrs, len(ws), _stream(stream)))
    return outs


def nf4_merge(w: NF4Tensor, A, B, r: int, alpha: float, out=None,
              stream=None):
    """Dense bf16 [rows, cols] = bf16(W' + (alpha / r) B A)."""
    import torch
    if out is None:
        out = torch.empty((w.rows, w.cols), dtype=torch.bfloat16,
                          device=w.packed.device)
    st = w.as_struct()
    _check("nf4_merge", lib().nf4_merge(ctypes.byref(st), _ptr(A), _ptr(B),
                                        int(r), float(alpha), _ptr(out),
                                        _stream(stream)))
    return out


@dataclass
class QTensor:
    """Device buffers of a codec-variant weight (see qn_qtensor in the
    header): packed codes, per-block constants (uint8, float32 or int8 by
    consts_mode), per-group scale and mean (empty where unused)."""
    packed: "object"
    consts: "object"
    gscale: "object"
    gmean: "object"
    rows: int
    cols: int
    code: int
    consts_mode: int

    @property
    def numel(self) -> int:
        return self.rows * self.cols

    @classmethod
    def empty(cls, rows: int, cols: int, code: int, consts_mode: int,
              device="cuda"):
        import torch
        npk, nb, ng = NF4Tensor.sizes(rows, cols)
        cdt = {QN_CONST_DQ8: torch.uint8, QN_CONST_FP32: torch.float32,
               QN_CONST_CENTERED: torch.int8}[consts_mode]
        has_scale = consts_mode != QN_CONST_FP32
        has_mean = consts_mode == QN_CONST_CENTERED
        return cls(torch.empty(npk, dtype=torch.uint8, device=device),
                   torch.empty(nb, dtype=cdt, device=device),
                   torch.empty(ng if has_scale else 0, dtype=torch.float32, device=device),
                   torch.empty(ng if has_mean else 0, dtype=torch.float32, device=device),
                   rows, cols, code, consts_mode)

    def as_struct(self) -> _QStruct:
        def p(t):
            return t.data_ptr() if t is not None and t.numel() > 0 else None
        return _QStruct(self.packed.data_ptr(), p(self.consts), p(self.gscale),
                        p(self.gmean), self.rows, self.cols, self.code,
                        self.consts_mode)


def qn_codebook(code: int):
    """(levels float32[16], thresholds float32[15]) of a QN_CODE_* table."""
    lv = np.zeros(16, dtype=np.float32)
    th = np.zeros(15, dtype=np.float32)
    _check("qn_codebook", lib().qn_codebook(int(code), lv.ctypes.data,
                                            th.ctypes.data))
    return lv, th


def qn_quantize(w, code: int, consts_mode: int, out: QTensor | None = None,
                status=None, stream=None):
    """Quantize a device fp32 weight into a variant format; returns it."""
    rows, cols = (w.shape[0], w.shape[1]) if w.dim() == 2 else (1, w.numel())
    if out is None:
        out = QTensor.empty(rows, cols, code, consts_mode, device=w.device)
    st = out.as_struct()
    _check("qn_quantize", lib().qn_quantize(_ptr(w), ctypes.byref(st),
                                            _ptr(status), _stream(stream)))
    return out


def qn_dequantize(w: QTensor, out=None, stream=None):
    """bf16 device tensor [rows, cols] of a variant-format weight."""
    import torch
    if out is None:
        out = torch.empty((w.rows, w.cols), dtype=torch.bfloat16,
                          device=w.packed.device)
    st = w.as_struct()
    _check("qn_dequantize", lib().qn_dequantize(ctypes.byref(st), _ptr(out),
                                                _stream(stream)))
    return out


@dataclass
class AdamW8State:
    """8-bit AdamW state of n parameters (see qn_adamw8_state in the header):
    E4M3 codes of m and sqrt(v), one fp32 scale each per 256 elements.
    Device tensors, or pinned host tensors for the paged step."""
    m_codes: "object"
    m_scale: "object"
    r_codes: "object"
    r_scale: "object"

    @classmethod
    def zeros(cls, n: int, device="cuda", pin_memory=False):
        import torch
        nb = -(-n // QN_ADAMW_BLOCK)
        kw = dict(device=device) if not pin_memory else dict(pin_memory=True)
        return cls(torch.zeros(n, dtype=torch.uint8, **kw),
                   torch.zeros(nb, dtype=torch.float32, **kw),
                   torch.zeros(n, dtype=torch.uint8, **kw),
                   torch.zeros(nb, dtype=torch.float32, **kw))

    def as_struct(self) -> _Adam8State:
        return _Adam8State(self.m_codes.data_ptr(), self.m_scale.data_ptr(),
                           self.r_codes.data_ptr(), self.r_scale.data_ptr())


def _hparams(lr, beta1, beta2, eps, weight_decay, grad_scale) -> _AdamHP:
    return _AdamHP(float(lr), float(beta1), float(beta2), float(eps),
                   float(weight_decay), float(grad_scale))


def qn_adamw8_step(p, g, state: AdamW8State, step: int, lr=2e-4, beta1=0.9,
                   beta2=0.999, eps=1e-8, weight_decay=0.0, grad_scale=1.0,
                   stream=None):
    """One 8-bit AdamW step on bf16 parameters p (in place) with fp32
    gradients g and a device-resident state."""
    hp = _hparams(lr, beta1, beta2, eps, weight_decay, grad_scale)
    st = state.as_struct()
    _check("qn_adamw8_step", lib().qn_adamw8_step(
        _ptr(p), _ptr(g), p.numel(), ctypes.byref(st), ctypes.byref(hp),
        int(step), _stream(stream)))


def qn_adamw8_staging_bytes(chunk: int) -> int:
    return int(lib().qn_adamw8_staging_bytes(int(chunk)))


def qn_adamw8_paged_step(p, g, host_state: AdamW8State, staging, chunk: int,
                         step: int, lr=2e-4, beta1=0.9, beta2=0.999,
                         eps=1e-8, weight_decay=0.0, grad_scale=1.0,
                         stream=None, h2d_stream=None, d2h_stream=None):
    """The same step with the state in pinned host memory, paged through
    the device `staging` buffer in pages of `chunk` elements."""
    hp = _hparams(lr, beta1, beta2, eps, weight_decay, grad_scale)
    st = host_state.as_struct()
    cs = _stream(stream)
    hs = None if h2d_stream is None else getattr(h2d_stream, "cuda_stream", h2d_stream)
    ds = None if d2h_stream is None else getattr(d2h_stream, "cuda_stream", d2h_stream)
    _check("qn_adamw8_paged_step", lib().qn_adamw8_paged_step(
        _ptr(p), _ptr(g), p.numel(), ctypes.byref(st), _ptr(staging),
        staging.numel() * staging.element_size(), int(chunk),
        ctypes.byref(hp), int(step), cs, hs, ds))


def qlora_workspace_bytes(M: int, N: int, K: int, r: int, which: int) -> int:
    return int(lib().qlora_workspace_bytes(M, N, K, r, which))


def qlora_linear_fwd(x, w: NF4Tensor, A, B, r: int, alpha: float, y=None,
                     y_dtype: int = QN_F32, t_save=None, ws=None,
                     stream=None):
    """Fused forward; returns (y, t_save)."""
    import torch
    M = x.shape[0]
    dev = x.device
    if y is None:
        y = torch.empty((M, w.rows), device=dev,
                        dtype=torch.float32 if y_dtype == QN_F32 else torch.bfloat16)
    if t_save is None:
        t_save = torch.empty((M, r), device=dev, dtype=torch.float32)
    need = qlora_workspace_bytes(M, w.rows, w.cols, r, QN_FWD)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    st = w.as_struct()
    _check("qlora_linear_fwd", lib().qlora_linear_fwd(
        _ptr(x), M, ctypes.byref(st), _ptr(A), _ptr(B), r, float(alpha),
        _ptr(y), y_dtype, _ptr(t_save), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))
    return y, t_save


class FwdBatch:
    """Descriptors of a qlora_linear_fwd_batch call, kept alive with the
    tensors they point to.  jobs: sequence of (x, w, A, B, r, alpha, y,
    y_dtype, t_save) with y / t_save None to allocate them."""

    def __init__(self, jobs):
        import torch
        self.keep, self.outs = [], []
        arr = (_FwdJob * len(jobs))()
        for i, (x, w, A, B, r, alpha, y, y_dtype, t_save) in enumerate(jobs):
            M = x.shape[0]
            if y is None:
                y = torch.empty((M, w.rows), device=x.device,
                                dtype=torch.float32 if y_dtype == QN_F32
                                else torch.bfloat16)
            if t_save is None:
                t_save = torch.empty((M, r), device=x.device, dtype=torch.float32)
            st = w.as_struct()
            self.keep += [x, A, B, y, t_save, st]
            self.outs.append((y, t_save))
            arr[i] = _FwdJob(_ptr(x), M, ctypes.pointer(st), _ptr(A), _ptr(B), r,
                             float(alpha), _ptr(y), y_dtype, _ptr(t_save))
        self.arr, self.count = arr, len(jobs)
        self.ws_bytes = lib().qlora_fwd_batch_workspace_bytes(arr, self.count)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8,
                              device=jobs[0][0].device)


def qlora_fwd_batch_workspace_bytes(batch: FwdBatch) -> int:
    return int(lib().qlora_fwd_batch_workspace_bytes(batch.arr, batch.count))


def qlora_linear_fwd_batch(batch: FwdBatch, stream=None):
    """Batched skinny forward (every job M <= 16); returns [(y, t_save)]."""
    _check("qlora_linear_fwd_batch", lib().qlora_linear_fwd_batch(
        batch.arr, batch.count, _ptr(batch.ws),
        batch.ws.numel() * batch.ws.element_size(), _stream(stream)))
    return batch.outs


def qlora_linear_fwd_noalloc(x, w: NF4Tensor, A, B, r: int, alpha: float,
                             y=None, y_dtype: int = QN_F32, t_save=None,
                             stream=None):
    """Fused forward with the library's own per-GPU scratch array as its
    workspace (no workspace argument); returns (y, t_save).  Calls on one
    GPU share the array: do not overlap them."""
    import torch
    M = x.shape[0]
    dev = x.device
    if y is None:
        y = torch.empty((M, w.rows), device=dev,
                        dtype=torch.float32 if y_dtype == QN_F32 else torch.bfloat16)
    if t_save is None:
        t_save = torch.empty((M, r), device=dev, dtype=torch.float32)
    st = w.as_struct()
    _check("qlora_linear_fwd_noalloc", lib().qlora_linear_fwd_noalloc(
        _ptr(x), M, ctypes.byref(st), _ptr(A), _ptr(B), r, float(alpha),
        _ptr(y), y_dtype, _ptr(t_save), _stream(stream)))
    return y, t_save


def qlora_linear_bwd(dy, x, w: NF4Tensor, A, B, r: int, alpha: float,
                     t_saved, dx=None, dx_dtype: int = QN_F32, dA=None,
                     dB=None, ws=None, stream=None):
    """Fused backward; returns (dx, dA, dB)."""
    import torch
    M = x.shape[0]
    dev = x.device
    if dx is None:
        dx = torch.empty((M, w.cols), device=dev,
                         dtype=torch.float32 if dx_dtype == QN_F32 else torch.bfloat16)
    if dA is None:
        dA = torch.empty((r, w.cols), device=dev, dtype=torch.float32)
    if dB is None:
        dB = torch.empty((w.rows, r), device=dev, dtype=torch.float32)
    if ws is None:
        ws = torch.empty(max(1, qlora_workspace_bytes(M, w.rows, w.cols, r, QN_BWD)),
                         dtype=torch.uint8, device=dev)
    st = w.as_struct()
    _check("qlora_linear_bwd", lib().qlora_linear_bwd(
        _ptr(dy), _ptr(x), M, ctypes.byref(st), _ptr(A), _ptr(B), r,
        float(alpha), _ptr(t_saved), _ptr(dx), dx_dtype, _ptr(dA), _ptr(dB),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return dx, dA, dB


def qlora_linear_fwd_dropout(x, w: NF4Tensor, A, B, r: int, alpha: float,
                             p: float, seed: int, y=None,
                             y_dtype: int = QN_F32, t_save=None, ws=None,
                             stream=None):
    """Fused forward with LoRA dropout (probability p, 64-bit seed) on the
    adapter input; returns (y, t_save)."""
    import torch
    M = x.shape[0]
    dev = x.device
    if y is None:
        y = torch.empty((M, w.rows), device=dev,
                        dtype=torch.float32 if y_dtype == QN_F32 else torch.bfloat16)
    if t_save is None:
        t_save = torch.empty((M, r), device=dev, dtype=torch.float32)
    if ws is None:
        ws = torch.empty(max(1, qlora_workspace_bytes(M, w.rows, w.cols, r,
                                                      QN_FWD_DROPOUT)),
                         dtype=torch.uint8, device=dev)
    st = w.as_struct()
    d = _Dropout(float(p), int(seed) & 0xFFFFFFFFFFFFFFFF)
    _check("qlora_linear_fwd_dropout", lib().qlora_linear_fwd_dropout(
        _ptr(x), M, ctypes.byref(st), _ptr(A), _ptr(B), r, float(alpha),
        _ptr(y), y_dtype, _ptr(t_save), ctypes.byref(d), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))
    return y, t_save


def qlora_linear_bwd_dropout(dy, x, w: NF4Tensor, A, B, r: int, alpha: float,
                             t_saved, p: float, seed: int, dx=None,
                             dx_dtype: int = QN_F32, dA=None, dB=None,
                             ws=None, stream=None):
    """Fused backward with the forward's dropout mask; returns (dx, dA, dB)."""
    import torch
    M = x.shape[0]
    dev = x.device
    if dx is None:
        dx = torch.empty((M, w.cols), device=dev,
                         dtype=torch.float32 if dx_dtype == QN_F32 else torch.bfloat16)
    if dA is None:
        dA = torch.empty((r, w.cols), device=dev, dtype=torch.float32)
    if dB is None:
        dB = torch.empty((w.rows, r), device=dev, dtype=torch.float32)
    if ws is None:
        ws = torch.empty(max(1, qlora_workspace_bytes(M, w.rows, w.cols, r, QN_BWD)),
                         dtype=torch.uint8, device=dev)
    st = w.as_struct()
    d = _Dropout(float(p), int(seed) & 0xFFFFFFFFFFFFFFFF)
    _check("qlora_linear_bwd_dropout", lib().qlora_linear_bwd_dropout(
        _ptr(dy), _ptr(x), M, ctypes.byref(st), _ptr(A), _ptr(B), r,
        float(alpha), _ptr(t_saved), _ptr(dx), dx_dtype, _ptr(dA), _ptr(dB),
        ctypes.byref(d), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))
    return dx, dA, dB


def qn_profile_kernel(name: str | None, starts=None, stops=None) -> int:
    """Arm (or with name=None disarm) per-launch event timing of one internal
    kernel.  ``starts``/``stops`` are lists of torch.cuda.Event created with
    enable_timing=True; returns the number of launches recorded before this
    call re-armed or disarmed."""
    if name is None:
        return int(lib().qn_profile_kernel(None, None, None, 0))
    import torch
    n = len(starts)
    assert len(stops) == n
    for e in list(starts) + list(stops):
        if not e.cuda_event:           # torch creates the event on first record
            e.record()
    torch.cuda.synchronize()
    if not all(e.cuda_event for e in list(starts) + list(stops)):
        raise RuntimeError("qn_profile_kernel: event handles are not created")
    arr_t = ctypes.c_void_p * max(n, 1)
    a = arr_t(*[e.cuda_event for e in starts])
    b = arr_t(*[e.cuda_event for e in stops])
    _profile_keepalive[:] = [a, b, starts, stops]
    rc = int(lib().qn_profile_kernel(name.encode(), a, b, n))
    if rc < 0:
        raise QNError("qn_profile_kernel", rc)
    return rc


_profile_keepalive: list = []
