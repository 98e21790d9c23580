"""Helpers for the GPU parity tests: host <-> device copies, running the
library on seeded inputs, and comparison statistics. Imports nothing from the
oracle; the tests call both sides."""
import sys

import numpy as np
import torch

import sign_muon_step_amd as sm

DEV = torch.device("cuda:0")


def announce(msg: str) -> None:
    sys.__stderr__.write(msg + "\n")
    sys.__stderr__.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    if a.dtype == np.uint64:
        return torch.from_numpy(a.view(np.int64)).to(DEV)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.int64:
        return t.cpu().numpy().view(np.uint64)
    return t.cpu().numpy()


def dtype_of(name: str):
    return {"f32": (np.float32, torch.float32, sm.F32),
            "bf16": (np.uint16, torch.bfloat16, sm.BF16)}[name]


def make_matrix(g: np.ndarray, m: np.ndarray, w: np.ndarray = None, *, polar=True, vote=True,
                packed=True) -> sm.Matrix:
    mw, R, C = g.shape
    return sm.Matrix(
        grad=to_dev(g), momentum=to_dev(m),
        packed=torch.zeros((mw, sm.signmuon_packed_words(R * C)), dtype=torch.int64, device=DEV)
        if packed else None,
        weight=to_dev(w) if w is not None else None,
        polar_out=torch.zeros((mw, R, C), dtype=torch.float32, device=DEV) if polar else None,
        vote_out=torch.zeros((R, C), dtype=torch.int8, device=DEV) if vote else None)


def traced_step_kinds(mats, params: sm.Params, capacity: int = 256):
    """Run signmuon_step_traced once; the kernel kind of each launch, in order
    (names from sm.KERNEL_KINDS)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    events = []
    for _ in range(capacity):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        events.append(e.value)
    try:
        tr = sm.Trace(events)
        sm.signmuon_step_traced(mats, params, sm.workspace_tensor(mats, params, DEV), tr)
        torch.cuda.synchronize()
        assert tr.launches < capacity
        return [sm.KERNEL_KINDS[k] for k in tr.kinds()]
    finally:
        for e in events:
            hip.hipEventDestroy(e)


def run(entry: str, mats, params: sm.Params):
    ws = sm.workspace_tensor(mats, params, DEV)
    getattr(sm, entry)(mats, params, ws)
    torch.cuda.synchronize()


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    a = a.astype(np.float64)
    b = b.astype(np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def sign_stats(u_gpu: np.ndarray, u_ref: np.ndarray):
    """Fraction of sign agreement over entries with |U| >= 1e-6 max|U| (the
    rest may take either sign within rounding), and the disagreeing count."""
    thresh = 1e-6 * float(np.abs(u_ref).max()) if u_ref.size else 0.0
    keep = np.abs(u_ref) >= thresh
    same = (u_gpu >= 0) == (u_ref >= 0)
    n = int(keep.sum())
    bad = int((~same & keep).sum())
    return (1.0 if n == 0 else 1.0 - bad / n), bad, n


def bit_sign_stats(packed_words: np.ndarray, u_ref: np.ndarray):
    """sign_stats for packed bits (LSB-first words, bit 1 = +1) against a
    reference U: agreement over the entries with |U| >= 1e-6 max|U|."""
    n = u_ref.size
    bits = np.unpackbits(packed_words.view(np.uint8), bitorder="little")[:n].astype(bool)
    ref = u_ref.ravel()
    keep = np.abs(ref) >= 1e-6 * float(np.abs(ref).max())
    bad = int((bits != (ref >= 0))[keep].sum())
    cnt = int(keep.sum())
    return (1.0 if cnt == 0 else 1.0 - bad / cnt), bad, cnt
