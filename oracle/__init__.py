"""CPU oracle for the Sign-Muon optimizer step -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package. The GPU library (``sign_muon_step_amd``) never
imports it, and it never imports the GPU library.

This module only marshals numpy arrays into the plain C oracle
(``signmuon_oracle.c``); every step of the arithmetic happens there. bf16
arrays are numpy ``uint16`` arrays holding raw bf16 bit patterns.

Method source: the technical summary of "SignMuon: Communication-Efficient
Distributed Muon Optimization" (gist.science, paper 2605.16311), cited by
section in the C file.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16, F64 = 0, 1, 2

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    i64, i32, f32, f64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_double
    vp = ctypes.c_void_p
    lib.orc_bf16_from_f32.restype = ctypes.c_uint16
    lib.orc_bf16_from_f32.argtypes = [f32]
    lib.orc_bf16_to_f32.restype = f32
    lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_round_array.argtypes = [i64, vp, vp]
    lib.orc_momentum.argtypes = [i64, f32, vp, ctypes.c_int, vp, ctypes.c_int]
    lib.orc_normalise.restype = f64
    lib.orc_normalise.argtypes = [i64, vp, ctypes.c_int, vp]
    lib.orc_newton_schulz.restype = ctypes.c_int
    lib.orc_newton_schulz.argtypes = [i64, i64, vp, ctypes.c_int, ctypes.c_int, vp]
    lib.orc_newton_schulz_a0.restype = ctypes.c_int
    lib.orc_newton_schulz_a0.argtypes = [i64, i64, vp, vp, ctypes.c_int, ctypes.c_int, vp]
    lib.orc_power_lambda.restype = f64
    lib.orc_power_lambda.argtypes = [i64, vp, ctypes.c_int]
    lib.orc_spectral_x0_a0.restype = f64
    lib.orc_spectral_x0_a0.argtypes = [i64, i64, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
    lib.orc_step_matrix_norm.restype = ctypes.c_int
    lib.orc_step_matrix_norm.argtypes = [i64, i64, i32, f32, f32, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, vp, vp, vp, vp, vp, vp]
    lib.orc_muon_step_matrix.restype = ctypes.c_int
    lib.orc_muon_step_matrix.argtypes = [i64, i64, f32, f32, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         vp, vp, vp, vp]
    lib.orc_ns1_entries.restype = ctypes.c_int
    lib.orc_ns1_entries.argtypes = [i64, i64, vp, ctypes.c_int, i64, vp, vp, vp]
    lib.orc_sign_pack.argtypes = [i64, vp, ctypes.c_int, vp]
    lib.orc_packed_words.restype = i64
    lib.orc_packed_words.argtypes = [i64]
    lib.orc_vote_update.argtypes = [i64, i32, vp, vp, f32, vp]
    lib.orc_sign_int8.argtypes = [i64, vp, ctypes.c_int, vp]
    lib.orc_vote_update_int8.argtypes = [i64, i32, vp, vp, f32, vp]
    lib.orc_post_polar.restype = i64
    lib.orc_post_polar.argtypes = [i64, i64, vp, ctypes.c_int, ctypes.c_int, vp, f32]
    lib.orc_step_matrix.restype = ctypes.c_int
    lib.orc_step_matrix.argtypes = [i64, i64, i32, f32, f32, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    vp, vp, vp, vp, vp, vp]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported oracle storage dtype {a.dtype}")


def _c(a, dtype=None):
    a = np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))
    return a


# -- storage ---------------------------------------------------------------
def bf16_from_f32(x):
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().orc_bf16_round_array(x.size, _ptr(x), _ptr(out))
    return out


def bf16_to_f32(h):
    """bf16 bit patterns (uint16) -> fp32 values (exact)."""
    h = _c(h, np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


# -- O1..O8 ------------------------------------------------------------------
def momentum(g, m, beta):
    """O1, in place on ``m`` (float32 or bf16-as-uint16): m <- fmaf(beta, m, g)."""
    assert m.flags.c_contiguous and g.size == m.size
    g = _c(g)
    _load().orc_momentum(m.size, beta, _ptr(g), _dtype_code(g), _ptr(m), _dtype_code(m))
    return m


def normalise(m):
    """O2: returns (nu, x0) with x0 = m / ||m||_F in fp64 (0 when nu = 0)."""
    m = _c(m)
    x0 = np.empty(m.shape, np.float64)
    nu = _load().orc_normalise(m.size, _ptr(m), _dtype_code(m), _ptr(x0))
    return nu, x0


def newton_schulz(x0, k, ns_dtype):
    """O3: k cubic Newton-Schulz iterations on the R x C fp64 array ``x0``."""
    x0 = _c(x0, np.float64)
    R, C = x0.shape
    u = np.empty_like(x0)
    rc = _load().orc_newton_schulz(R, C, _ptr(x0), k, ns_dtype, _ptr(u))
    if rc != 0:
        raise MemoryError("oracle newton_schulz")
    return u


NORM_FROB, NORM_SPECTRAL = 0, 1


def newton_schulz_a0(x0, a0, k, ns_dtype):
    """O3 with the first iteration's Gram matrix a0 (r x r, already rounded)."""
    x0 = _c(x0, np.float64)
    a0 = _c(a0, np.float64)
    R, C = x0.shape
    r = min(R, C)
    assert a0.shape == (r, r)
    u = np.empty_like(x0)
    if _load().orc_newton_schulz_a0(R, C, _ptr(x0), _ptr(a0), k, ns_dtype, _ptr(u)) != 0:
        raise MemoryError("oracle newton_schulz_a0")
    return u


def power_lambda(a, p):
    """Spectral normalisation: p power-iteration steps on the symmetric a
    from the all-ones vector; the last ||A v||."""
    a = _c(a, np.float64)
    lam = _load().orc_power_lambda(a.shape[0], _ptr(a), p)
    if lam < 0:
        raise MemoryError("oracle power_lambda")
    return float(lam)


def spectral_x0_a0(m, ns_dtype, p):
    """Spectral normalisation of one stored R x C momentum: (lambda, x0, a0)."""
    m = _c(m)
    R, C = m.shape
    r = min(R, C)
    x0 = np.empty((R, C), np.float64)
    a0 = np.empty((r, r), np.float64)
    lam = _load().orc_spectral_x0_a0(R, C, _ptr(m), _dtype_code(m), ns_dtype, p, _ptr(x0), _ptr(a0))
    if lam < 0:
        raise MemoryError("oracle spectral_x0_a0")
    return float(lam), x0, a0


def ns1_entries(x0, ns_dtype, rows, cols):
    """O3 with k = 1, evaluated only at the (rows[t], cols[t]) entries."""
    x0 = _c(x0, np.float64)
    R, C = x0.shape
    rows = _c(rows, np.int64)
    cols = _c(cols, np.int64)
    assert rows.shape == cols.shape
    assert (rows >= 0).all() and (rows < R).all() and (cols >= 0).all() and (cols < C).all()
    out = np.empty(rows.shape, np.float64)
    rc = _load().orc_ns1_entries(R, C, _ptr(x0), ns_dtype, rows.size, _ptr(rows), _ptr(cols),
                                 _ptr(out))
    if rc != 0:
        raise MemoryError("oracle ns1_entries")
    return out


def packed_words(n):
    return int(_load().orc_packed_words(n))


def sign_pack(u):
    """O4+O5: uint64 words of (u >= 0), LSB-first over the flat index."""
    u = _c(u)
    words = np.empty(packed_words(u.size), np.uint64)
    _load().orc_sign_pack(u.size, _ptr(u), _dtype_code(u), _ptr(words))
    return words


def vote_update(packed, w, eta, want_vote=True):
    """O6+O7: packed is [mw][words]; W (float32) is updated in place.
    Returns the vote S-bar as int8 when ``want_vote``."""
    packed = _c(packed, np.uint64)
    mw = packed.shape[0]
    assert w.dtype == np.float32 and w.flags.c_contiguous
    assert packed.shape[1] == packed_words(w.size)
    vote = np.empty(w.shape, np.int8) if want_vote else None
    _load().orc_vote_update(w.size, mw, _ptr(packed), _ptr(w), eta, _ptr(vote))
    return vote


def sign_int8(u):
    """Int8 payload: +1 where u >= 0, -1 elsewhere (the packed bits' rule)."""
    u = _c(u)
    out = np.empty(u.shape, np.int8)
    _load().orc_sign_int8(u.size, _ptr(u), _dtype_code(u), _ptr(out))
    return out


def vote_update_int8(signs, w, eta, want_vote=True):
    """Int8 payload vote: signs is [mw][n] int8; the vote is the sign of the
    integer sum over workers; W (float32) is updated in place."""
    signs = _c(signs, np.int8)
    mw = signs.shape[0]
    assert w.dtype == np.float32 and w.flags.c_contiguous
    assert signs.reshape(mw, -1).shape[1] == w.size
    vote = np.empty(w.shape, np.int8) if want_vote else None
    _load().orc_vote_update_int8(w.size, mw, _ptr(signs), _ptr(w), eta, _ptr(vote))
    return vote


def post_polar(vote, w, eta, k, ns_dtype):
    """O8: W <- fmaf(-eta, NS_k(V/||V||_F), W) in place; returns nnz(V)."""
    vote = _c(vote, np.int8)
    R, C = vote.shape
    assert w.dtype == np.float32 and w.size == vote.size and w.flags.c_contiguous
    nnz = _load().orc_post_polar(R, C, _ptr(vote), k, ns_dtype, _ptr(w), eta)
    if nnz < 0:
        raise MemoryError("oracle post_polar")
    return int(nnz)


def step_matrix(g, m, w, beta, eta, k, ns_dtype, post_k=0, want_u=False, norm=0, power_iters=0):
    """One full step for one R x C matrix and all workers.

    g: [mw][R][C] float32 (or bf16 uint16); m: [mw][R][C] float32 or uint16,
    updated in place; w: [R][C] float32, updated in place.
    Returns (packed [mw][words] uint64, vote int8 [R][C], u fp64 or None).
    """
    assert m.flags.c_contiguous and w.flags.c_contiguous and w.dtype == np.float32
    g = _c(g)
    mw, R, C = m.shape
    assert g.shape == m.shape and w.shape == (R, C)
    packed = np.empty((mw, packed_words(R * C)), np.uint64)
    vote = np.empty((R, C), np.int8)
    u = np.empty((mw, R, C), np.float64) if want_u else None
    rc = _load().orc_step_matrix_norm(R, C, mw, beta, eta, k, post_k, _dtype_code(g),
                                      _dtype_code(m), ns_dtype, norm, power_iters, _ptr(g), _ptr(m),
                                      _ptr(u), _ptr(packed), _ptr(w), _ptr(vote))
    if rc != 0:
        raise MemoryError("oracle step_matrix")
    return packed, vote, u


def muon_step_matrix(g, m, w, beta, eta, k, ns_dtype, norm=0, power_iters=0, want_u=False):
    """Full-precision Muon step for one worker: g, m are [R][C] (m updated in
    place), w [R][C] float32 updated in place. Returns U (fp64) or None."""
    assert m.flags.c_contiguous and w.flags.c_contiguous and w.dtype == np.float32
    g = _c(g)
    R, C = m.shape
    assert g.shape == m.shape == w.shape
    u = np.empty((R, C), np.float64) if want_u else None
    rc = _load().orc_muon_step_matrix(R, C, beta, eta, k, _dtype_code(g), _dtype_code(m), ns_dtype,
                                      norm, power_iters, _ptr(g), _ptr(m), _ptr(u), _ptr(w))
    if rc != 0:
        raise MemoryError("oracle muon_step_matrix")
    return u
