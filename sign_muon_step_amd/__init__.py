"""Python binding of the MI355X Sign-Muon step library (``libsignmuon.so``).

Argument marshalling only: torch tensors are passed to the C ABI of
``include/signmuon.h`` as device pointers, with the current torch stream.
Every step of the optimizer runs in the library's HIP kernels. If the
library is not built, every call raises: there is no other code path.

The function names are those of the C ABI. ``Matrix`` describes one weight
matrix with its per-worker buffers; ``Params`` the step's hyper-parameters.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsignmuon.so")

F32, BF16 = 0, 1
ABI_VERSION = 4
# device bytes of the static scratch behind signmuon_step_noalloc
STATIC_SCRATCH_BYTES = 128 << 20

STATUS = {0: "SIGNMUON_OK", -1: "SIGNMUON_EINVAL", -2: "SIGNMUON_EDTYPE", -3: "SIGNMUON_EALIGN",
          -4: "SIGNMUON_EWORKSPACE", -5: "SIGNMUON_EHIP", -6: "SIGNMUON_ERANGE",
          -7: "SIGNMUON_ESCRATCH"}


class SignmuonError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"{STATUS.get(status, status)}: {text}")
        self.status = status


class _Matrix(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("grad", ctypes.c_void_p),
                ("momentum", ctypes.c_void_p), ("polar_out", ctypes.c_void_p),
                ("packed", ctypes.c_void_p), ("weight", ctypes.c_void_p),
                ("vote_out", ctypes.c_void_p), ("signs_i8", ctypes.c_void_p)]


class _Params(ctypes.Structure):
    _fields_ = [("workers", ctypes.c_int32), ("beta", ctypes.c_float), ("eta", ctypes.c_float),
                ("ns_iters", ctypes.c_int32), ("post_polar_iters", ctypes.c_int32),
                ("grad_dtype", ctypes.c_int), ("mom_dtype", ctypes.c_int),
                ("ns_dtype", ctypes.c_int), ("norm", ctypes.c_int32),
                ("power_iters", ctypes.c_int32), ("payload", ctypes.c_int32)]


class _Trace(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)), ("capacity", ctypes.c_int32),
                ("kinds", ctypes.POINTER(ctypes.c_int32)), ("launches", ctypes.c_int32)]


KERNEL_KINDS = {1: "momentum", 2: "scales", 3: "ns_gram", 4: "ns_product", 5: "sign_pack",
                6: "vote_update", 7: "aux", 8: "power", 9: "vote_update_int8"}
NORM_FROBENIUS, NORM_SPECTRAL = 0, 1
PAYLOAD_BITS, PAYLOAD_INT8 = 0, 1

_lib = None


def library() -> ctypes.CDLL:
    """Load ``libsignmuon.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run sign_muon_step_amd/build.py "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    mp, pp = ctypes.POINTER(_Matrix), ctypes.POINTER(_Params)
    lib.signmuon_momentum_ns.restype = ctypes.c_int
    lib.signmuon_momentum_ns.argtypes = [mp, i32, pp, vp, ctypes.c_size_t, vp]
    lib.signmuon_step.restype = ctypes.c_int
    lib.signmuon_step.argtypes = [mp, i32, pp, vp, ctypes.c_size_t, vp]
    lib.signmuon_step_noalloc.restype = ctypes.c_int
    lib.signmuon_step_noalloc.argtypes = [mp, i32, pp, vp]
    lib.signmuon_muon_step.restype = ctypes.c_int
    lib.signmuon_muon_step.argtypes = [mp, i32, pp, vp, ctypes.c_size_t, vp]
    lib.signmuon_step_traced.restype = ctypes.c_int
    lib.signmuon_step_traced.argtypes = [mp, i32, pp, vp, ctypes.c_size_t, vp, ctypes.POINTER(_Trace)]
    lib.signmuon_sign_pack.restype = ctypes.c_int
    lib.signmuon_sign_pack.argtypes = [vp, ctypes.c_int, i64, i32, vp, vp]
    lib.signmuon_vote_update.restype = ctypes.c_int
    lib.signmuon_vote_update.argtypes = [vp, i32, i64, vp, ctypes.c_float, vp, vp]
    lib.signmuon_sign_int8.restype = ctypes.c_int
    lib.signmuon_sign_int8.argtypes = [vp, ctypes.c_int, i64, i32, vp, vp]
    lib.signmuon_vote_update_int8.restype = ctypes.c_int
    lib.signmuon_vote_update_int8.argtypes = [vp, i32, i64, vp, ctypes.c_float, vp, vp]
    lib.signmuon_packed_words.restype = ctypes.c_size_t
    lib.signmuon_packed_words.argtypes = [i64]
    lib.signmuon_workspace_bytes.restype = ctypes.c_size_t
    lib.signmuon_workspace_bytes.argtypes = [mp, i32, pp]
    lib.signmuon_strerror.restype = ctypes.c_char_p
    lib.signmuon_strerror.argtypes = [ctypes.c_int]
    lib.signmuon_abi_version.restype = ctypes.c_int
    lib.signmuon_abi_version.argtypes = []
    if lib.signmuon_abi_version() != ABI_VERSION:
        raise RuntimeError("libsignmuon.so ABI version mismatch")
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise SignmuonError(status, library().signmuon_strerror(status).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"tensors passed to the library must be in GPU memory (device {t.device})")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


@dataclass
class Matrix:
    """One R x C weight matrix and its buffers (see signmuon_matrix).

    grad, momentum, polar_out: [Mw][R][C]; packed: [Mw][packed_words] int64
    (bit pattern of the uint64 words); weight: [R][C] fp32; vote_out: [R][C]
    int8; signs_i8: [Mw][R][C] int8 (int8 payload). Optional fields may be
    None.
    """
    grad: torch.Tensor
    momentum: torch.Tensor
    packed: Optional[torch.Tensor] = None
    weight: Optional[torch.Tensor] = None
    polar_out: Optional[torch.Tensor] = None
    vote_out: Optional[torch.Tensor] = None
    signs_i8: Optional[torch.Tensor] = None

    @property
    def shape(self):
        return tuple(self.grad.shape[-2:])


@dataclass
class Params:
    workers: int
    beta: float = 0.9
    eta: float = 1e-3
    ns_iters: int = 1
    post_polar_iters: int = 0
    grad_dtype: int = F32
    mom_dtype: int = F32
    ns_dtype: int = F32
    norm: int = NORM_FROBENIUS
    power_iters: int = 0
    payload: int = PAYLOAD_BITS


_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}


def _expect(t: Optional[torch.Tensor], name: str, dtypes, numel: int) -> None:
    """Element type, element count and contiguity of one buffer the library
    reads or writes through a raw pointer (a short buffer would be accessed
    out of bounds by the kernels)."""
    if t is None:
        return
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {' or '.join(map(str, dtypes))}")
    if t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _buffers(m: Matrix):
    return [("grad", m.grad), ("momentum", m.momentum), ("polar_out", m.polar_out),
            ("packed", m.packed), ("weight", m.weight), ("vote_out", m.vote_out),
            ("signs_i8", m.signs_i8)]


def _validate(mats: Sequence[Matrix], params: Params) -> None:
    """Every buffer of every matrix has the type and size the step assumes,
    then every buffer is in GPU memory (a host pointer would fault)."""
    mw = params.workers
    for i, m in enumerate(mats):
        R, C = m.shape
        n = R * C
        tag = f"matrix {i} ({R}x{C})"
        _expect(m.grad, f"{tag} grad", (_TORCH_DTYPE.get(params.grad_dtype),), mw * n)
        _expect(m.momentum, f"{tag} momentum", (_TORCH_DTYPE.get(params.mom_dtype),), mw * n)
        _expect(m.polar_out, f"{tag} polar_out", (torch.float32,), mw * n)
        _expect(m.packed, f"{tag} packed", (torch.int64,), mw * ((n + 63) // 64))
        _expect(m.weight, f"{tag} weight", (torch.float32,), n)
        _expect(m.vote_out, f"{tag} vote_out", (torch.int8,), n)
        _expect(m.signs_i8, f"{tag} signs_i8", (torch.int8,), mw * n)
    for i, m in enumerate(mats):
        for name, t in _buffers(m):
            if t is not None and t.device.type != "cuda":
                raise ValueError(f"matrix {i} {name}: must be in GPU memory (device {t.device})")


def _marshal(mats: Sequence[Matrix], params: Params):
    _validate(mats, params)
    arr = (_Matrix * len(mats))()
    for i, m in enumerate(mats):
        R, C = m.shape
        arr[i] = _Matrix(R, C, _ptr(m.grad), _ptr(m.momentum), _ptr(m.polar_out), _ptr(m.packed),
                         _ptr(m.weight), _ptr(m.vote_out), _ptr(m.signs_i8))
    p = _Params(params.workers, params.beta, params.eta, params.ns_iters,
                params.post_polar_iters, params.grad_dtype, params.mom_dtype, params.ns_dtype,
                params.norm, params.power_iters, params.payload)
    return arr, p


def signmuon_packed_words(n: int) -> int:
    return int(library().signmuon_packed_words(n))


def signmuon_workspace_bytes(mats: Sequence[Matrix], params: Params) -> int:
    arr, p = _marshal(mats, params)
    return int(library().signmuon_workspace_bytes(arr, len(mats), ctypes.byref(p)))


def signmuon_strerror(status: int) -> str:
    return library().signmuon_strerror(status).decode()


def signmuon_abi_version() -> int:
    return int(library().signmuon_abi_version())


def signmuon_momentum_ns(mats: Sequence[Matrix], params: Params, workspace: Optional[torch.Tensor],
                         stream=None) -> None:
    arr, p = _marshal(mats, params)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().signmuon_momentum_ns(arr, len(mats), ctypes.byref(p), _ptr(workspace), nbytes,
                                          _stream(stream)))


def signmuon_step(mats: Sequence[Matrix], params: Params, workspace: Optional[torch.Tensor],
                  stream=None) -> None:
    arr, p = _marshal(mats, params)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().signmuon_step(arr, len(mats), ctypes.byref(p), _ptr(workspace), nbytes,
                                   _stream(stream)))


def signmuon_step_noalloc(mats: Sequence[Matrix], params: Params, stream=None) -> None:
    """signmuon_step with the library's static device scratch as workspace
    (no allocation anywhere); raises SignmuonError (SIGNMUON_ESCRATCH) when
    the step needs more than STATIC_SCRATCH_BYTES."""
    arr, p = _marshal(mats, params)
    _check(library().signmuon_step_noalloc(arr, len(mats), ctypes.byref(p), _stream(stream)))


def signmuon_muon_step(mats: Sequence[Matrix], params: Params, workspace: Optional[torch.Tensor],
                       stream=None) -> None:
    arr, p = _marshal(mats, params)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().signmuon_muon_step(arr, len(mats), ctypes.byref(p), _ptr(workspace), nbytes,
                                        _stream(stream)))


class Trace:
    """Per-launch timing events for signmuon_step_traced. ``events`` are raw
    hipEvent_t handles created by the caller (capacity = len(events))."""

    def __init__(self, events: Sequence[int]):
        self.capacity = len(events)
        self._events = (ctypes.c_void_p * self.capacity)(*events)
        self._kinds = (ctypes.c_int32 * max(1, self.capacity - 1))()
        self.struct = _Trace(self._events, self.capacity, self._kinds, 0)

    @property
    def launches(self) -> int:
        return int(self.struct.launches)

    def kinds(self):
        n = min(self.launches, self.capacity - 1)
        return [int(self._kinds[i]) for i in range(n)]


def signmuon_step_traced(mats: Sequence[Matrix], params: Params, workspace: Optional[torch.Tensor],
                         trace: Optional[Trace], stream=None) -> None:
    arr, p = _marshal(mats, params)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().signmuon_step_traced(arr, len(mats), ctypes.byref(p), _ptr(workspace), nbytes,
                                          _stream(stream),
                                          ctypes.byref(trace.struct) if trace else None))


class Prepared:
    """The matrices, parameters and workspace of repeated calls, checked and
    marshalled once: each call then only crosses the C ABI. The tensors are
    kept alive by this object and must stay the same buffers (their
    contents may change between calls, e.g. new gradients)."""

    def __init__(self, mats: Sequence[Matrix], params: Params, workspace: Optional[torch.Tensor]):
        self.arr, self.p = _marshal(mats, params)
        self.n = len(mats)
        self.ws = _ptr(workspace)
        self.nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        # the tensors themselves: a field of a Matrix reassigned later must not
        # free a buffer whose pointer is marshalled here
        self._keep = ([t for m in mats for _, t in _buffers(m) if t is not None], workspace)

    def _args(self, stream):
        return self.arr, self.n, ctypes.byref(self.p), self.ws, self.nbytes, _stream(stream)

    def step(self, stream=None) -> None:
        _check(library().signmuon_step(*self._args(stream)))

    def step_traced(self, trace: Optional[Trace], stream=None) -> None:
        _check(library().signmuon_step_traced(*self._args(stream),
                                              ctypes.byref(trace.struct) if trace else None))

    def momentum_ns(self, stream=None) -> None:
        _check(library().signmuon_momentum_ns(*self._args(stream)))

    def muon_step(self, stream=None) -> None:
        _check(library().signmuon_muon_step(*self._args(stream)))


def _expect_room(t: Optional[torch.Tensor], name: str, dtypes, numel: int) -> None:
    """For the single-stage calls: element type, and at least `numel` elements
    (the kernels touch exactly that many; a shorter buffer would be accessed
    out of bounds). Sizes are checked only for a valid n and worker count; the
    library rejects the others."""
    if t is None:
        return
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {' or '.join(map(str, dtypes))}")
    if numel > 0 and t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, at least {numel} needed")


def _words(n: int) -> int:
    return (n + 63) // 64 if n > 0 else 0


def signmuon_sign_pack(u: torch.Tensor, n: int, workers: int, packed: torch.Tensor,
                       stream=None) -> None:
    k = workers if workers > 0 else 0
    _expect_room(u, "u", (torch.float32, torch.bfloat16), k * max(n, 0))
    _expect_room(packed, "packed", (torch.int64,), k * _words(n))
    _check(library().signmuon_sign_pack(_ptr(u), _dtype_code(u), n, workers, _ptr(packed),
                                        _stream(stream)))


def signmuon_vote_update(packed: torch.Tensor, workers: int, n: int, weight: Optional[torch.Tensor],
                         eta: float, vote_out: Optional[torch.Tensor] = None, stream=None) -> None:
    k = workers if workers > 0 else 0
    _expect_room(packed, "packed", (torch.int64,), k * _words(n))
    _expect_room(weight, "weight", (torch.float32,), max(n, 0))
    _expect_room(vote_out, "vote_out", (torch.int8,), max(n, 0))
    _check(library().signmuon_vote_update(_ptr(packed), workers, n, _ptr(weight), eta,
                                          _ptr(vote_out), _stream(stream)))


def signmuon_sign_int8(u: torch.Tensor, n: int, workers: int, signs: torch.Tensor,
                       stream=None) -> None:
    k = workers if workers > 0 else 0
    _expect_room(u, "u", (torch.float32, torch.bfloat16), k * max(n, 0))
    _expect_room(signs, "signs", (torch.int8,), k * max(n, 0))
    _check(library().signmuon_sign_int8(_ptr(u), _dtype_code(u), n, workers, _ptr(signs),
                                        _stream(stream)))


def signmuon_vote_update_int8(signs: torch.Tensor, workers: int, n: int,
                              weight: Optional[torch.Tensor], eta: float,
                              vote_out: Optional[torch.Tensor] = None, stream=None) -> None:
    k = workers if workers > 0 else 0
    _expect_room(signs, "signs", (torch.int8,), k * max(n, 0))
    _expect_room(weight, "weight", (torch.float32,), max(n, 0))
    _expect_room(vote_out, "vote_out", (torch.int8,), max(n, 0))
    _check(library().signmuon_vote_update_int8(_ptr(signs), workers, n, _ptr(weight), eta,
                                               _ptr(vote_out), _stream(stream)))


def dtype_code(t: torch.dtype) -> int:
    return {torch.float32: F32, torch.bfloat16: BF16}[t]


def workspace_tensor(mats: Sequence[Matrix], params: Params, device) -> Optional[torch.Tensor]:
    """Allocate (with torch) the device workspace the library asks for."""
    nbytes = signmuon_workspace_bytes(mats, params)
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)
