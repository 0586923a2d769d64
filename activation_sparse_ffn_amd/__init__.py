"""Predictor-gated bank-wise sparse SwiGLU FFN forward on AMD MI355X.

A thin ctypes binding over libsparse_ffn.so (include/sparse_ffn.h). Every
step of the forward runs in the library's HIP kernels; this module only
marshals torch tensors (device memory) and the current HIP stream into the
C calls. There is no fallback: without the built library or a GPU the calls
raise.

    ffn = SparseFFN(W_g, W_u, W_d, A, B, bias=None, keep=16, gate="pred")
    y = ffn(x)                                  # x [T, d] on the GPU
    y, mask, logits = ffn(x, return_mask=True, return_logits=True)
    mask, ids = bank_topk(logits, keep=16, return_ids=True)

The layer is the FFN block of "Continual LLM Upcycling: A Predictor-Gated
Bank-Wise Sparsity Training Recipe for Dense-to-Sparse LLMs" (gist.science
technical summary, Methodologie > 1. Architectuur).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["SparseFFN", "bank_topk", "library_path", "load_library", "SparseFFNError",
           "SFFN_OK", "SFFN_ERR_INVALID_ARG", "SFFN_ERR_UNSUPPORTED", "SFFN_ERR_WORKSPACE",
           "SFFN_ERR_HIP", "Config", "EXPORTED_SYMBOLS"]

_PKG = os.path.dirname(os.path.abspath(__file__))

SFFN_OK, SFFN_ERR_INVALID_ARG, SFFN_ERR_UNSUPPORTED, SFFN_ERR_WORKSPACE, SFFN_ERR_HIP = range(5)
SFFN_F32, SFFN_BF16 = 0, 1
GATES = {"pred": 0, "silu": 1, "amplitude": 2}

EXPORTED_SYMBOLS = (
    "sparse_ffn_packed_size", "sparse_ffn_create", "sparse_ffn_workspace_size",
    "sparse_ffn_forward", "bank_topk", "sparse_ffn_destroy", "sparse_ffn_status_string",
    "sparse_ffn_last_error", "sparse_ffn_set_stage_events", "sparse_ffn_stage_name",
    "sparse_ffn_backward_workspace_size", "sparse_ffn_backward", "sparse_ffn_forward_noalloc",
)
SFFN_STAGES = 5
SFFN_FLAG_BACKWARD = 1


class SparseFFNError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"status {status}: {detail}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("d_i", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("bank", ctypes.c_int32), ("keep", ctypes.c_int32), ("dtype", ctypes.c_int),
                ("gate", ctypes.c_int), ("flags", ctypes.c_int32)]


def library_path() -> str:
    return os.environ.get("SFFN_LIBRARY", os.path.join(_PKG, "libsparse_ffn.so"))


_LIB = None


def load_library():
    """Load libsparse_ffn.so and declare its signatures (raises if absent)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m activation_sparse_ffn_amd.build`")
    lib = ctypes.CDLL(path)
    P, S, I64, I32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_int32
    st = ctypes.c_int
    lib.sparse_ffn_packed_size.argtypes = [ctypes.POINTER(Config)]
    lib.sparse_ffn_packed_size.restype = S
    lib.sparse_ffn_create.argtypes = [ctypes.POINTER(Config), P, P, P, P, P, P, P, S, P,
                                      ctypes.POINTER(P)]
    lib.sparse_ffn_create.restype = st
    lib.sparse_ffn_workspace_size.argtypes = [P, I64]
    lib.sparse_ffn_workspace_size.restype = S
    lib.sparse_ffn_forward.argtypes = [P, P, I64, P, P, P, P, S, P]
    lib.sparse_ffn_forward.restype = st
    lib.bank_topk.argtypes = [P, I64, I32, I32, P, P, P]
    lib.bank_topk.restype = st
    lib.sparse_ffn_destroy.argtypes = [P]
    lib.sparse_ffn_destroy.restype = None
    lib.sparse_ffn_status_string.argtypes = [st]
    lib.sparse_ffn_status_string.restype = ctypes.c_char_p
    lib.sparse_ffn_last_error.argtypes = []
    lib.sparse_ffn_last_error.restype = ctypes.c_char_p
    lib.sparse_ffn_set_stage_events.argtypes = [P, ctypes.POINTER(P), I32]
    lib.sparse_ffn_set_stage_events.restype = st
    lib.sparse_ffn_stage_name.argtypes = [P, I64, I32]
    lib.sparse_ffn_stage_name.restype = ctypes.c_char_p
    lib.sparse_ffn_backward_workspace_size.argtypes = [P, I64]
    lib.sparse_ffn_backward_workspace_size.restype = S
    lib.sparse_ffn_backward.argtypes = [P, P, P, P, I64, ctypes.c_float, P, P, P, P, P, P, P, P, S, P]
    lib.sparse_ffn_backward.restype = st
    lib.sparse_ffn_forward_noalloc.argtypes = [P, P, I64, P, P, P, P]
    lib.sparse_ffn_forward_noalloc.restype = st
    _LIB = lib
    return lib


def _check(lib, status: int):
    if status != SFFN_OK:
        detail = lib.sparse_ffn_last_error().decode()
        name = lib.sparse_ffn_status_string(status).decode()
        raise SparseFFNError(status, f"{name}: {detail}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_gpu(*ts: torch.Tensor):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


def _need_buffer(t: torch.Tensor, name: str, shape, dtype, device: torch.device):
    """A caller-supplied output or scratch tensor: shape, dtype, device and
    contiguity are checked before its address reaches the library, which
    writes through it without knowing its extent."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the layer on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def bank_topk(logits: torch.Tensor, keep: int = 16, return_ids: bool = False,
              mask_out: Optional[torch.Tensor] = None, ids_out: Optional[torch.Tensor] = None):
    """Bank-wise hard top-k over fp32 logits [T, d_i] (banks of 64).

    Returns the mask as int64 [T, d_i/64] (the uint64 bit pattern; bit i of
    word (t, b) is channel 64 b + i) and, if asked, the kept channel ids as
    int16 [T, d_i/64 * keep] (uint16 bit pattern, ascending per token).
    """
    lib = load_library()
    _need_gpu(logits)
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise ValueError("logits must be a 2-D float32 tensor")
    T, d_i = logits.shape
    nb = d_i // 64
    if mask_out is None:
        mask_out = torch.empty((T, nb), dtype=torch.int64, device=logits.device)
    else:
        _need_buffer(mask_out, "mask_out", (T, nb), torch.int64, logits.device)
    if return_ids and ids_out is None:
        ids_out = torch.empty((T, nb * keep), dtype=torch.int16, device=logits.device)
    elif return_ids:
        _need_buffer(ids_out, "ids_out", (T, nb * keep), torch.int16, logits.device)
    _check(lib, lib.bank_topk(_ptr(logits), T, d_i, keep, _ptr(mask_out),
                              _ptr(ids_out) if return_ids else None, _stream(logits.device)))
    return (mask_out, ids_out) if return_ids else mask_out


class SparseFFN:
    """One predictor-gated sparse SwiGLU FFN layer, packed on the GPU.

    Weights use nn.Linear layout: W_g, W_u [d_i, d]; W_d [d, d_i];
    A [rank, d]; B [d_i, rank]; bias fp32 [d_i] or None. All bf16 or all
    fp32, contiguous, on one GPU. The weights are copied into a packed
    buffer the object owns; the originals may be dropped afterwards.
    """

    def __init__(self, W_g, W_u, W_d, A=None, B=None, bias=None, keep: int = 16, gate: str = "pred",
                 for_backward: bool = False):
        """gate: "pred" (sigmoid of the predictor logit), "silu" (sigmoid of
        u) or "amplitude" (the Dense-4x post-hoc baseline: no predictor, the
        mask ranks |SiLU(u) v|; A and B may then be None). for_backward: keep
        W_g^T and W_u^T in the packed buffer (SFFN_FLAG_BACKWARD) so that
        backward() does not transpose them on every call."""
        self._lib = load_library()
        if gate not in GATES:
            raise ValueError("gate must be 'pred', 'silu' or 'amplitude'")
        if (A is None or B is None) and gate != "amplitude":
            raise ValueError("the predictor weights A and B are needed unless gate='amplitude'")
        _need_gpu(*(t for t in (W_g, W_u, W_d, A, B, bias) if t is not None))
        dt = W_g.dtype
        if dt not in (torch.bfloat16, torch.float32):
            raise ValueError("weights must be bfloat16 or float32")
        if any(t.dtype != dt for t in (W_u, W_d, A, B) if t is not None):
            raise ValueError("all weights must share one dtype")
        if bias is not None and bias.dtype != torch.float32:
            raise ValueError("bias must be float32")
        d_i, d = W_g.shape
        rank = A.shape[0] if A is not None else 32
        if W_u.shape != (d_i, d) or W_d.shape != (d, d_i) \
                or (A is not None and A.shape != (rank, d)) or (B is not None and B.shape != (d_i, rank)) \
                or (bias is not None and bias.shape != (d_i,)):
            raise ValueError("inconsistent weight shapes")
        self.device = W_g.device
        self.dtype = dt
        self.cfg = Config(d, d_i, rank, 64, keep, SFFN_BF16 if dt == torch.bfloat16 else SFFN_F32,
                          GATES[gate], SFFN_FLAG_BACKWARD if for_backward else 0)
        size = self._lib.sparse_ffn_packed_size(ctypes.byref(self.cfg))
        if size == 0:
            _check(self._lib, SFFN_ERR_INVALID_ARG)
        self.packed = torch.empty(size, dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        _check(self._lib, self._lib.sparse_ffn_create(
            ctypes.byref(self.cfg), _ptr(W_g), _ptr(W_u), _ptr(W_d), _ptr(A), _ptr(B), _ptr(bias),
            _ptr(self.packed), size, _stream(self.device), ctypes.byref(h)))
        self._h = h
        self._ws = {}
        self.has_bias = bias is not None

    @property
    def d(self):
        return self.cfg.d

    @property
    def d_i(self):
        return self.cfg.d_i

    def workspace_size(self, T: int) -> int:
        return int(self._lib.sparse_ffn_workspace_size(self._h, T))

    def workspace(self, T: int) -> torch.Tensor:
        """A workspace tensor for T tokens on the current stream (cached per
        stream, grown on demand). Forwards on different streams never share
        one, and a grown workspace replaces the old one only on its own
        stream, where torch's allocator reuses the freed block after the work
        already queued there."""
        need = self.workspace_size(T)
        key = torch.cuda.current_stream(self.device).cuda_stream
        ws = self._ws.get(key)
        if ws is None or ws.numel() < need:
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
            self._ws[key] = ws
        return ws

    def forward(self, x: torch.Tensor, return_mask: bool = False, return_logits: bool = False,
                y: Optional[torch.Tensor] = None, mask: Optional[torch.Tensor] = None,
                logits: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
        _need_gpu(x)
        if x.dtype != self.dtype or x.dim() != 2 or x.shape[1] != self.d:
            raise ValueError(f"x must be [T, {self.d}] {self.dtype}")
        T = x.shape[0]
        if x.device != self.device:
            raise ValueError(f"x is on {x.device}, the layer on {self.device}")
        if y is None:
            y = torch.empty_like(x)
        else:
            _need_buffer(y, "y", (T, self.d), self.dtype, self.device)
        if return_mask and mask is None:
            mask = torch.empty((T, self.d_i // 64), dtype=torch.int64, device=self.device)
        elif mask is not None:
            _need_buffer(mask, "mask", (T, self.d_i // 64), torch.int64, self.device)
        if return_logits and logits is None:
            logits = torch.empty((T, self.d_i), dtype=torch.float32, device=self.device)
        elif logits is not None:
            _need_buffer(logits, "logits", (T, self.d_i), torch.float32, self.device)
        if workspace is not None:
            _need_buffer(workspace, "workspace", None, torch.uint8, self.device)
            if workspace.dim() != 1:
                raise ValueError("workspace must be a 1-D uint8 tensor")
        ws = workspace if workspace is not None else self.workspace(T)
        _check(self._lib, self._lib.sparse_ffn_forward(
            self._h, _ptr(x), T, _ptr(y), _ptr(mask) if return_mask or mask is not None else None,
            _ptr(logits) if return_logits or logits is not None else None, _ptr(ws), ws.numel(),
            _stream(self.device)))
        out = [y]
        if return_mask:
            out.append(mask)
        if return_logits:
            out.append(logits)
        return out[0] if len(out) == 1 else tuple(out)

    __call__ = forward

    def backward(self, x: torch.Tensor, g_y: torch.Tensor, mask: torch.Tensor, tau: float = 1.0,
                 workspace: Optional[torch.Tensor] = None) -> dict:
        """Gradients of sum(y * g_y) for a forward of x that returned `mask`
        (bf16 layers; predictor or silu gate). The top-k's derivative is the
        soft surrogate sigmoid((p - theta) / tau) around each bank's
        threshold; tau = float("inf") leaves it out. Returns fp32 tensors
        "x", "A", "B", "bias" (None without a bias), "W_g", "W_u", "W_d"."""
        _need_gpu(x, g_y, mask)
        if x.dtype != self.dtype or g_y.dtype != self.dtype or x.shape != g_y.shape or x.dim() != 2 \
                or x.shape[1] != self.d:
            raise ValueError(f"x and g_y must be [T, {self.d}] {self.dtype}")
        T = x.shape[0]
        if mask.shape != (T, self.d_i // 64) or mask.dtype != torch.int64:
            raise ValueError("mask must be the forward's [T, d_i / 64] int64 mask")
        f32 = dict(dtype=torch.float32, device=self.device)
        r = self.cfg.rank
        out = {"x": torch.empty((T, self.d), **f32), "A": torch.empty((r, self.d), **f32),
               "B": torch.empty((self.d_i, r), **f32), "W_g": torch.empty((self.d_i, self.d), **f32),
               "W_u": torch.empty((self.d_i, self.d), **f32), "W_d": torch.empty((self.d, self.d_i), **f32),
               "bias": torch.empty(self.d_i, **f32) if self.has_bias else None}
        need = int(self._lib.sparse_ffn_backward_workspace_size(self._h, T))
        if workspace is not None:
            _need_buffer(workspace, "workspace", None, torch.uint8, self.device)
        ws = workspace if workspace is not None else torch.empty(max(need, 256), dtype=torch.uint8,
                                                                   device=self.device)
        _check(self._lib, self._lib.sparse_ffn_backward(
            self._h, _ptr(x), _ptr(g_y), _ptr(mask), T, ctypes.c_float(tau), _ptr(out["x"]), _ptr(out["A"]),
            _ptr(out["B"]), _ptr(out["bias"]), _ptr(out["W_g"]), _ptr(out["W_u"]), _ptr(out["W_d"]),
            _ptr(ws), ws.numel(), _stream(self.device)))
        return out

    def set_stage_events(self, events):
        """Attach 2 * SFFN_STAGES raw hipEvent_t handles (ints): the start and
        stop events of each kernel stage of later forwards; None detaches."""
        if events is None:
            _check(self._lib, self._lib.sparse_ffn_set_stage_events(self._h, None, 0))
            return
        arr = (ctypes.c_void_p * len(events))(*events)
        self._events_keepalive = arr
        _check(self._lib, self._lib.sparse_ffn_set_stage_events(self._h, arr, len(events)))

    def stage_names(self, T: int):
        return [self._lib.sparse_ffn_stage_name(self._h, T, i).decode() for i in range(SFFN_STAGES)]

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.sparse_ffn_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
