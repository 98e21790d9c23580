"""Host-side checks of the C ABI: the library loads, exports every function
include/signmuon.h declares, and rejects bad arguments before any launch
(these calls never reach the GPU, so they run without one)."""
import ctypes
import os
import re

import pytest

import sign_muon_step_amd as sm
import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "signmuon.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(signmuon_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sm.LIB_PATH):
        from sign_muon_step_amd import build
        build.build()
    return sm.library()


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("signmuon_momentum_ns", "signmuon_sign_pack", "signmuon_vote_update", "signmuon_step"):
        assert n in names


def test_library_exports_every_declared_function(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_host_helpers(lib):
    assert sm.signmuon_abi_version() == sm.ABI_VERSION
    assert [sm.signmuon_packed_words(n) for n in (0, 1, 63, 64, 65, 128)] == [0, 1, 1, 1, 2, 2]
    for st in (0, -1, -2, -3, -4, -5, -6, 7):
        assert isinstance(sm.signmuon_strerror(st), str)


def _fake(R, C, mw, *, aligned=True, polar=False, vote=False):
    """A matrix descriptor with fake (never dereferenced) device addresses."""
    base = 0x7f0000000000 if aligned else 0x7f0000000004
    m = sm._Matrix(R, C, base, base + 0x100000, base + 0x200000 if polar else None,
                   base + 0x300000, base + 0x400000, base + 0x500000 if vote else None)
    return m


def _call(fn, mats, params, ws=0x7f1000000000, ws_bytes=1 << 40):
    arr = (sm._Matrix * len(mats))(*mats)
    p = sm._Params(params.workers, params.beta, params.eta, params.ns_iters,
                   params.post_polar_iters, params.grad_dtype, params.mom_dtype, params.ns_dtype,
                   params.norm, params.power_iters, params.payload)
    return fn(arr, len(mats), ctypes.byref(p), ws, ws_bytes, None)


def test_workspace_bytes_cover_the_gram_buffers(lib):
    wl = synthetic.WORKLOADS["gpt2s_mw8_k1"]
    mats = [sm.Matrix(grad=None, momentum=None) for _ in wl.shapes]
    arr = (sm._Matrix * len(wl.shapes))(*[sm._Matrix(R, C, None, None, None, None, None, None)
                                          for R, C in wl.shapes])
    p = sm._Params(8, 0.9, 1e-3, 1, 0, sm.F32, sm.BF16, sm.BF16)
    nbytes = lib.signmuon_workspace_bytes(arr, len(mats), ctypes.byref(p))
    gram = sum(8 * min(R, C) ** 2 * 2 for R, C in wl.shapes)
    assert gram <= nbytes <= gram + (64 << 20)
    p5 = sm._Params(8, 0.9, 1e-3, 5, 0, sm.F32, sm.BF16, sm.BF16)
    nb5 = lib.signmuon_workspace_bytes(arr, len(mats), ctypes.byref(p5))
    assert nb5 >= nbytes + 2 * 8 * wl.params * 2  # two iterate buffers
    bad = sm._Params(0, 0.9, 1e-3, 1, 0, sm.F32, sm.BF16, sm.BF16)
    assert lib.signmuon_workspace_bytes(arr, len(mats), ctypes.byref(bad)) == 0


P = sm.Params(workers=4, ns_iters=1)


@pytest.mark.parametrize("fn", ["signmuon_step", "signmuon_momentum_ns"])
def test_argument_errors_return_before_launch(lib, fn):
    f = getattr(lib, fn)
    polar = fn == "signmuon_momentum_ns"
    ok = _fake(64, 64, 4, polar=polar)
    assert _call(f, [_fake(0, 64, 4, polar=polar)], P) == -1
    assert _call(f, [ok], sm.Params(workers=0)) == -1
    assert _call(f, [ok], sm.Params(workers=4, ns_iters=-1)) == -1
    assert _call(f, [ok], sm.Params(workers=4, beta=float("nan"))) == -1
    assert _call(f, [ok], sm.Params(workers=4, eta=float("inf"))) == -1
    assert _call(f, [ok], sm.Params(workers=4, mom_dtype=sm.BF16, ns_dtype=sm.F32)) == -2
    assert _call(f, [ok], sm.Params(workers=4, grad_dtype=7)) == -2
    assert _call(f, [ok], sm.Params(workers=256)) == -6
    assert _call(f, [_fake(1 << 21, 2, 4, polar=polar)], P) == -6
    assert _call(f, [_fake(64, 64, 4, aligned=False, polar=polar)], P) == -3
    assert _call(f, [ok], P, ws=0, ws_bytes=0) == -4
    assert _call(f, [ok], P, ws_bytes=16) == -4
    arr = (sm._Matrix * 1)(ok)
    assert f(arr, 0, ctypes.byref(sm._Params(4, 0.9, 1e-3, 1, 0, 0, 0, 0)), 0, 0, None) == -1
    assert f(None, 1, None, 0, 0, None) == -1


def test_step_requires_packed_and_weight(lib):
    m = _fake(64, 64, 4)
    m.packed = None
    assert _call(lib.signmuon_step, [m], P) == -1
    m = _fake(64, 64, 4)
    m.weight = None
    assert _call(lib.signmuon_step, [m], P) == -1


def test_momentum_ns_requires_polar_out(lib):
    assert _call(lib.signmuon_momentum_ns, [_fake(64, 64, 4, polar=False)], P) == -1


def test_sign_pack_and_vote_argument_errors(lib):
    a = 0x7f0000000000
    assert lib.signmuon_sign_pack(None, 0, 10, 1, a, None) == -1
    assert lib.signmuon_sign_pack(a, 0, 0, 1, a, None) == -1
    assert lib.signmuon_sign_pack(a, 0, 10, 0, a, None) == -1
    assert lib.signmuon_sign_pack(a, 5, 10, 1, a, None) == -2
    assert lib.signmuon_sign_pack(a + 4, 0, 10, 1, a, None) == -3
    assert lib.signmuon_vote_update(None, 3, 10, a, 1e-3, None, None) == -1
    assert lib.signmuon_vote_update(a, 3, 10, None, 1e-3, None, None) == -1
    assert lib.signmuon_vote_update(a, 0, 10, a, 1e-3, None, None) == -1
    assert lib.signmuon_vote_update(a, 3, 10, a, float("nan"), None, None) == -1
    assert lib.signmuon_vote_update(a, 256, 10, a, 1e-3, None, None) == -6
    assert lib.signmuon_vote_update(a, 3, 10, a + 8, 1e-3, None, None) == -3


def test_int8_payload_argument_errors(lib):
    a = 0x7f0000000000
    assert lib.signmuon_sign_int8(None, 0, 10, 1, a, None) == -1
    assert lib.signmuon_sign_int8(a, 0, 10, 1, None, None) == -1
    assert lib.signmuon_sign_int8(a, 0, 0, 1, a, None) == -1
    assert lib.signmuon_sign_int8(a, 0, 10, 0, a, None) == -1
    assert lib.signmuon_sign_int8(a, 7, 10, 1, a, None) == -2
    assert lib.signmuon_sign_int8(a, 0, 10, 1, a + 1, None) == -3
    assert lib.signmuon_sign_int8(a, 0, 10, 256, a, None) == -6
    assert lib.signmuon_vote_update_int8(None, 3, 10, a, 1e-3, None, None) == -1
    assert lib.signmuon_vote_update_int8(a, 3, 10, None, 1e-3, None, None) == -1
    assert lib.signmuon_vote_update_int8(a, 0, 10, a, 1e-3, None, None) == -1
    assert lib.signmuon_vote_update_int8(a, 3, 10, a, float("inf"), None, None) == -1
    assert lib.signmuon_vote_update_int8(a, 256, 10, a, 1e-3, None, None) == -6
    assert lib.signmuon_vote_update_int8(a + 2, 3, 10, a, 1e-3, None, None) == -3
    assert lib.signmuon_vote_update_int8(a, 3, 10, a, 1e-3, a + 4, None) == -3


def test_step_int8_payload_argument_errors(lib):
    """payload must be BITS or INT8; INT8 needs signs_i8 (16-byte aligned),
    not packed, and does not combine with the post-vote polar step."""
    i8 = sm.Params(workers=4, payload=sm.PAYLOAD_INT8)
    assert _call(lib.signmuon_step, [_fake(64, 64, 4)], sm.Params(workers=4, payload=2)) == -1
    assert _call(lib.signmuon_step, [_fake(64, 64, 4)], sm.Params(workers=4, payload=-1)) == -1
    m = _fake(64, 64, 4)  # no signs_i8
    assert _call(lib.signmuon_step, [m], i8) == -1
    m = _fake(64, 64, 4)
    m.signs_i8 = 0x7f0000600000 + 8
    assert _call(lib.signmuon_step, [m], i8) == -3
    m = _fake(64, 64, 4)
    m.signs_i8 = 0x7f0000600000
    m.packed = None
    assert _call(lib.signmuon_step, [m], sm.Params(workers=4, payload=sm.PAYLOAD_INT8,
                                                   post_polar_iters=1)) == -1
    m.weight = None
    assert _call(lib.signmuon_step, [m], i8) == -1
    # the packed payload still needs packed
    m = _fake(64, 64, 4)
    m.packed = None
    m.signs_i8 = 0x7f0000600000
    assert _call(lib.signmuon_step, [m], sm.Params(workers=4)) == -1


def test_int8_payload_needs_no_more_workspace(lib):
    arr = (sm._Matrix * 2)(sm._Matrix(300, 700, None, None, None, None, None, None),
                           sm._Matrix(130, 70, None, None, None, None, None, None))
    bits = sm._Params(4, 0.9, 1e-3, 1, 0, sm.F32, sm.BF16, sm.BF16, 0, 0, sm.PAYLOAD_BITS)
    i8 = sm._Params(4, 0.9, 1e-3, 1, 0, sm.F32, sm.BF16, sm.BF16, 0, 0, sm.PAYLOAD_INT8)
    # the int8 payload is written by the last product itself: no fp32 U scratch
    # for the shape whose columns are not a multiple of 64
    assert 0 < lib.signmuon_workspace_bytes(arr, 2, ctypes.byref(i8)) < \
        lib.signmuon_workspace_bytes(arr, 2, ctypes.byref(bits))


@pytest.mark.parametrize("fn", ["signmuon_step", "signmuon_momentum_ns"])
def test_spectral_argument_errors(lib, fn):
    f = getattr(lib, fn)
    polar = fn == "signmuon_momentum_ns"
    ok = _fake(64, 64, 4, polar=polar)
    assert _call(f, [ok], sm.Params(workers=4, norm=2)) == -1
    assert _call(f, [ok], sm.Params(workers=4, norm=sm.NORM_SPECTRAL, power_iters=0)) == -1
    assert _call(f, [ok], sm.Params(workers=4, norm=sm.NORM_SPECTRAL, power_iters=1001)) == -6
    big = _fake(8200, 8200, 1, polar=polar)
    assert _call(f, [big], sm.Params(workers=1, norm=sm.NORM_SPECTRAL, power_iters=4)) == -6


def test_spectral_workspace_adds_power_vectors(lib):
    arr = (sm._Matrix * 1)(sm._Matrix(300, 700, None, None, None, None, None, None))
    frob = sm._Params(4, 0.9, 1e-3, 0, 0, sm.F32, sm.F32, sm.F32, sm.NORM_FROBENIUS, 0)
    spec = sm._Params(4, 0.9, 1e-3, 0, 0, sm.F32, sm.F32, sm.F32, sm.NORM_SPECTRAL, 3)
    nf = lib.signmuon_workspace_bytes(arr, 1, ctypes.byref(frob))
    ns = lib.signmuon_workspace_bytes(arr, 1, ctypes.byref(spec))
    # k = 0 with spectral scaling still needs the Gram matrix and the power vectors
    assert ns >= nf + 4 * 300 * 300 * 4 + 2 * 4 * 300 * 4


def test_muon_step_argument_errors(lib):
    one = _fake(64, 64, 1)
    assert _call(lib.signmuon_muon_step, [one], sm.Params(workers=2, ns_iters=1)) == -1
    assert _call(lib.signmuon_muon_step, [one], sm.Params(workers=1, ns_iters=0)) == -1
    assert _call(lib.signmuon_muon_step, [one], sm.Params(workers=1, ns_iters=1,
                                                          post_polar_iters=1)) == -1
    no_w = _fake(64, 64, 1)
    no_w.weight = None
    assert _call(lib.signmuon_muon_step, [no_w], sm.Params(workers=1, ns_iters=1)) == -1
    assert _call(lib.signmuon_muon_step, [_fake(64, 64, 1, aligned=False)],
                 sm.Params(workers=1, ns_iters=1)) == -3
