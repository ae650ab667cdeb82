"""ctypes binding of libheadloss.so (include/headloss.h).

Argument marshalling only: every step of the loss runs in the HIP kernels
behind ``hl_forward_backward``. PyTorch supplies device memory and the
current stream. There is no fallback: if the library is not built, loading
fails with an error.
"""

from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libheadloss.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "headloss.h")

# status codes
HL_OK = 0
HL_ERR_INVALID_ARG = 1
HL_ERR_MISSING_INPUT = 2
HL_ERR_UNSUPPORTED = 3
HL_ERR_WORKSPACE = 4
HL_ERR_HIP = 5

HL_F32 = 0
HL_BF16 = 1
HL_F16 = 2

CE = 1 << 0
ZLOSS = 1 << 1
FKL = 1 << 2
RKL = 1 << 3
GRPO = 1 << 4
ENTROPY = 1 << 5
FDCE = 1 << 6
GSPO = 1 << 7
ACCUMULATE = 1 << 16
HINTON = 1 << 17

SLOTS = ("CE", "Z", "DISTILL", "GRPO", "NEWLOGP", "RATIO", "CLIPFRAC",
         "KL_OLD_NEW", "ADV_MEAN", "ENTROPY", "TOTAL", "N_VALID", "N_BADLABEL")
NUM_SCALARS = len(SLOTS)
ROW_COLS = ("CE", "Z", "DISTILL", "GRPO", "NEWLOGP", "RATIO", "CLIPPED", "K3",
            "ADV", "ENTROPY", "VALID", "PAD")


class Weights(ctypes.Structure):
    _fields_ = [("ce", ctypes.c_float), ("z", ctypes.c_float),
                ("distill", ctypes.c_float), ("grpo", ctypes.c_float),
                ("grad_scale", ctypes.c_float), ("divisor", ctypes.c_float)]


class HeadLossError(RuntimeError):
    def __init__(self, where: str, status: int):
        self.status = status
        detail = ""
        if status == HL_ERR_HIP:
            detail = " - " + load_library().hl_last_error().decode()
        super().__init__(f"{where}: {status_str(status)} (status {status}){detail}")


_lib = None


def exported_functions_in_header(path: str = HEADER_PATH) -> list[str]:
    """Names of the functions include/headloss.h declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hl_[a-z_]+)\s*\(", text)))


def load_library(path: str | None = None):
    """Load libheadloss.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m lm_head_vocab_amd.build` "
            "(there is no CPU fallback)")
    # One HIP runtime per process: PyTorch ships its own libamdhip64.so.7.
    # Loading torch first makes the library's libamdhip64.so.7 dependency
    # resolve to that already-loaded runtime instead of a second copy (two
    # runtimes in one process cannot both open the device).
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    vp, i64, u32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float
    lib.hl_plan.argtypes = [ctypes.POINTER(vp), i64, ctypes.c_int, u32,
                            ctypes.POINTER(Weights), f32, f32, f32, f32]
    lib.hl_plan.restype = ctypes.c_int
    lib.hl_plan_destroy.argtypes = [vp]
    lib.hl_plan_destroy.restype = None
    lib.hl_workspace_bytes.argtypes = [vp, i64]
    lib.hl_workspace_bytes.restype = ctypes.c_size_t
    lib.hl_plan_set_workspace.argtypes = [vp, vp, ctypes.c_size_t]
    lib.hl_plan_set_workspace.restype = ctypes.c_int
    lib.hl_forward_backward.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.hl_forward_backward.restype = ctypes.c_int
    lib.hl_forward_backward_segments.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp]
    lib.hl_forward_backward_segments.restype = ctypes.c_int
    lib.hl_forward_backward_noalloc.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp]
    lib.hl_forward_backward_noalloc.restype = ctypes.c_int
    lib.hl_row_values.argtypes = [vp]
    lib.hl_row_values.restype = vp
    lib.hl_plan_set_chunks.argtypes = [vp, ctypes.c_int]
    lib.hl_plan_set_chunks.restype = ctypes.c_int
    lib.hl_plan_set_variant.argtypes = [vp, ctypes.c_int, ctypes.c_int]
    lib.hl_plan_set_variant.restype = ctypes.c_int
    lib.hl_plan_describe.argtypes = [vp, ctypes.POINTER(ctypes.c_int),
                                     ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    lib.hl_plan_describe.restype = ctypes.c_int
    lib.hl_plan_set_timing_events.argtypes = [vp, vp, vp]
    lib.hl_plan_set_timing_events.restype = ctypes.c_int
    lib.hl_plan_set_exchange_test.argtypes = [vp, u32, i64, ctypes.c_int]
    lib.hl_plan_set_exchange_test.restype = ctypes.c_int
    lib.hl_last_error.argtypes = []
    lib.hl_last_error.restype = ctypes.c_char_p
    lib.hl_status_str.argtypes = [ctypes.c_int]
    lib.hl_status_str.restype = ctypes.c_char_p
    lib.hl_stream_ceiling.argtypes = [vp, vp, vp, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp,
                                      ctypes.POINTER(ctypes.c_float)]
    lib.hl_stream_ceiling.restype = ctypes.c_int
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().hl_status_str(status).decode()


def _check(where: str, status: int):
    if status != HL_OK:
        raise HeadLossError(where, status)


def _torch():
    import torch
    return torch


def _dtype_code(dtype) -> int:
    torch = _torch()
    if dtype in (torch.float32, "f32", "float32"):
        return HL_F32
    if dtype in (torch.bfloat16, "bf16", "bfloat16"):
        return HL_BF16
    if dtype in (torch.float16, "f16", "float16"):
        return HL_F16
    raise ValueError(f"unsupported dtype {dtype!r}: use float32, bfloat16 or float16")


class Plan:
    """A validated loss set (``hl_plan``) bound to one vocabulary size.

    Calling the plan runs ``hl_forward_backward`` (``hl_forward_backward_segments``
    when ``seq_offsets`` is given) on the current stream of the logits' device
    and returns the device float32[13] scalar tensor.
    """

    def __init__(self, V: int, dtype, flags: int, *, ce: float = 1.0, z: float = 0.0,
                 distill: float = 0.0, grpo: float = 0.0, grad_scale: float = 1.0,
                 divisor: float = 0.0, temperature: float = 1.0, eps: float = 0.2,
                 logit_scale: float = 1.0, softcap: float = 0.0, chunks: int = 0):
        lib = load_library()
        self._lib = lib
        self.V = int(V)
        self.dtype_code = _dtype_code(dtype)
        self.flags = int(flags)
        self.weights = Weights(ce, z, distill, grpo, grad_scale, divisor)
        h = ctypes.c_void_p()
        _check("hl_plan", lib.hl_plan(ctypes.byref(h), self.V, self.dtype_code, self.flags,
                                      ctypes.byref(self.weights), temperature, eps,
                                      logit_scale, softcap))
        self._h = h
        self._ws = None
        self._scalars = None
        self._events = None
        if chunks:
            self.set_chunks(chunks)

    # -- plan queries -------------------------------------------------------
    def set_chunks(self, chunks: int):
        _check("hl_plan_set_chunks", self._lib.hl_plan_set_chunks(self._h, int(chunks)))
        self._ws = None   # layout depends on the chunk count

    def set_variant(self, chunks: int, block: int = 0):
        _check("hl_plan_set_variant", self._lib.hl_plan_set_variant(self._h, int(chunks), int(block)))
        self._ws = None

    def describe(self) -> dict:
        c, b, n = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        _check("hl_plan_describe", self._lib.hl_plan_describe(
            self._h, ctypes.byref(c), ctypes.byref(b), ctypes.byref(n)))
        return {"chunks": c.value, "block": b.value, "vec_per_thread": n.value}

    def workspace_bytes(self, n_rows: int) -> int:
        return int(self._lib.hl_workspace_bytes(self._h, int(n_rows)))

    def set_timing_events(self, before, after):
        """Record torch.cuda.Events around the fused kernel of later calls."""
        self._events = (before, after)
        self._lib.hl_plan_set_timing_events(
            self._h, ctypes.c_void_p(before.cuda_event if before is not None else 0),
            ctypes.c_void_p(after.cuda_event if after is not None else 0))

    def set_exchange_test(self, spin_limit: int = 1 << 20, withhold_row: int = -1, withhold_chunk: int = -1):
        """Failure-handling hook of the split-vocab wait (hl_plan_set_exchange_test)."""
        _check("hl_plan_set_exchange_test", self._lib.hl_plan_set_exchange_test(
            self._h, int(spin_limit), int(withhold_row), int(withhold_chunk)))

    # -- the call -----------------------------------------------------------
    def set_workspace(self, ws):
        """Use a caller's uint8 device tensor as the workspace (hl_plan_set_workspace);
        several plans may share one (their calls must not overlap)."""
        self._ws = ws
        _check("hl_plan_set_workspace", self._lib.hl_plan_set_workspace(
            self._h, ctypes.c_void_p(ws.data_ptr()), ws.numel()))

    def _ensure_workspace(self, n_rows: int, device):
        torch = _torch()
        need = max(self.workspace_bytes(n_rows), 256)
        if self._ws is None or self._ws.numel() < need or self._ws.device != device:
            self._ws = torch.empty(need, dtype=torch.uint8, device=device)
            _check("hl_plan_set_workspace", self._lib.hl_plan_set_workspace(
                self._h, ctypes.c_void_p(self._ws.data_ptr()), self._ws.numel()))

    def _ptr(self, t, name, dtype=None, shape=None):
        if t is None:
            return None
        torch = _torch()
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        del torch
        return ctypes.c_void_p(t.data_ptr())

    def __call__(self, logits, labels=None, mask=None, teacher=None, old_logprobs=None,
                 advantages=None, grad=None, scalars=None, stream=None, seq_offsets=None,
                 noalloc=False):
        """noalloc: run hl_forward_backward_noalloc (the library's static
        per-GPU workspace; no device allocation by the call itself)."""
        torch = _torch()
        if logits.dim() != 2 or logits.shape[1] != self.V:
            raise ValueError(f"logits must be [N, {self.V}], got {tuple(logits.shape)}")
        n = logits.shape[0]
        dt = {HL_F32: torch.float32, HL_BF16: torch.bfloat16, HL_F16: torch.float16}[self.dtype_code]
        dev = logits.device
        if mask is not None and mask.dtype == torch.bool:
            mask = mask.view(torch.uint8)
        args = (
            self._ptr(logits, "logits", dt, (n, self.V)),
            self._ptr(labels, "labels", torch.int64, (n,)),
            self._ptr(mask, "mask", torch.uint8, (n,)),
            self._ptr(teacher, "teacher", dt, (n, self.V)),
            self._ptr(old_logprobs, "old_logprobs", torch.float32, (n,)),
            self._ptr(advantages, "advantages", torch.float32, (n,)),
            self._ptr(grad, "grad", dt, (n, self.V)),
        )
        if scalars is None:
            scalars = torch.empty(NUM_SCALARS, dtype=torch.float32, device=dev)
        sp = self._ptr(scalars, "scalars", torch.float32, (NUM_SCALARS,))
        if stream is None:
            stream = torch.cuda.current_stream(dev)
        if noalloc:
            op, n_seg = None, 0
            if seq_offsets is not None:
                if seq_offsets.dim() != 1 or seq_offsets.numel() < 1:
                    raise ValueError("seq_offsets must be a 1-D int32 tensor of n_segments + 1 offsets")
                op, n_seg = self._ptr(seq_offsets, "seq_offsets", torch.int32), seq_offsets.numel() - 1
            st = self._lib.hl_forward_backward_noalloc(
                self._h, n, *args[:6], op, n_seg, args[6], sp, ctypes.c_void_p(stream.cuda_stream))
            _check("hl_forward_backward_noalloc", st)
            self._last_rows = n
            self._last_static = True
            return scalars
        self._ensure_workspace(n, dev)
        self._last_static = False
        if seq_offsets is None:
            st = self._lib.hl_forward_backward(self._h, n, *args, sp, ctypes.c_void_p(stream.cuda_stream))
            _check("hl_forward_backward", st)
        else:
            if seq_offsets.dim() != 1 or seq_offsets.numel() < 1:
                raise ValueError("seq_offsets must be a 1-D int32 tensor of n_segments + 1 offsets")
            op = self._ptr(seq_offsets, "seq_offsets", torch.int32)
            st = self._lib.hl_forward_backward_segments(
                self._h, n, *args[:6], op, seq_offsets.numel() - 1, args[6], sp,
                ctypes.c_void_p(stream.cuda_stream))
            _check("hl_forward_backward_segments", st)
        self._last_rows = n
        return scalars

    def row_values(self):
        """float32 [n_rows, 12] view of the per-row values of the last call."""
        torch = _torch()
        ptr = self._lib.hl_row_values(self._h)
        if getattr(self, "_last_static", False):
            raise RuntimeError("the last call used the static workspace (hl_forward_backward_noalloc); "
                               "its per-row values are at the device pointer hl_row_values returns")
        if not ptr or self._ws is None:
            raise RuntimeError("no call has been made with this plan yet")
        off = ptr - self._ws.data_ptr()
        n = self._last_rows
        nbytes = n * len(ROW_COLS) * 4
        return self._ws[off:off + nbytes].view(torch.float32).view(n, len(ROW_COLS))

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.hl_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def stream_ceiling(read0, read1, write, block: int, vec_per_thread: int, reps: int = 5) -> float:
    """hl_stream_ceiling on the current stream: milliseconds per launch of the
    data-movement-only kernel over tensors of write's size (read1 may be None)."""
    torch = _torch()
    lib = load_library()
    nbytes = write.numel() * write.element_size()
    for t in (read0, read1):
        if t is not None and t.numel() * t.element_size() < nbytes:
            raise ValueError("every read tensor must hold at least as many bytes as write")
    ms = ctypes.c_float(0.0)
    stream = torch.cuda.current_stream(write.device).cuda_stream
    _check("hl_stream_ceiling", lib.hl_stream_ceiling(
        ctypes.c_void_p(read0.data_ptr()), ctypes.c_void_p(read1.data_ptr() if read1 is not None else 0),
        ctypes.c_void_p(write.data_ptr()), nbytes, block, vec_per_thread, reps, ctypes.c_void_p(stream),
        ctypes.byref(ms)))
    return float(ms.value)


def scalars_dict(scalars) -> dict:
    vals = scalars.detach().float().cpu().tolist()
    return dict(zip(SLOTS, vals))
