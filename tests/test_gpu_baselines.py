"""GPU parity of the comparison steps: the full-precision Muon step
(signmuon_muon_step, one worker, no sign) and majority-vote signum with
momentum (signmuon_step with ns_iters = 0), against the CPU oracle.

Bar: Muon's U within 1e-5 (fp32) / 2e-2 (bf16) relative Frobenius error and
W = fmaf(-eta, U, W) exactly on the GPU's own U; signum bit-exact (momentum,
packed signs, vote, W)."""
import numpy as np
import pytest
import torch

import oracle
import sign_muon_step_amd as sm
import synthetic
from gpu_util import DEV, announce, dtype_of, make_matrix, rel_fro, run, to_dev, to_host

pytestmark = pytest.mark.gpu

NS_TOL = {"f32": 1e-5, "bf16": 2e-2}
ORC_DT = {"f32": oracle.F32, "bf16": oracle.BF16}


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(f"[gpu-test] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def fmaf32(a: np.float32, b: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Correctly rounded fp32 a*b + c. The fp64 product of two fp32 values is
    exact; the fp64 sum s and its rounding error e (two-sum) hold a*b + c
    exactly, so rounding s to fp32 is right except when s sits exactly on a
    midpoint between two fp32 values, where the sign of e decides."""
    p = np.float64(a) * b.astype(np.float64)
    c64 = c.astype(np.float64)
    s = p + c64
    bb = s - p
    e = (p - (s - bb)) + (c64 - bb)
    out = s.astype(np.float32)
    above = out.astype(np.float64) > s
    lo = np.where(above, np.nextafter(out, np.float32(-np.inf)), out)
    hi = np.where(above, out, np.nextafter(out, np.float32(np.inf)))
    mid = (lo.astype(np.float64) + hi.astype(np.float64)) / 2
    on_mid = s == mid
    return np.where(on_mid & (e > 0), hi, np.where(on_mid & (e < 0), lo, out)).astype(np.float32)


MUON_CASES = [("f32", s, k, n) for s in [(256, 256), (300, 700), (700, 300)] for k in (1, 3)
              for n in ("frobenius", "spectral")] + \
             [("bf16", s, k, n) for s in [(384, 1024), (1024, 384), (768, 768)] for k in (1, 3)
              for n in ("frobenius", "spectral")]


@pytest.mark.parametrize("ns,shape,k,norm", MUON_CASES)
def test_muon_step_parity(ns, shape, k, norm):
    R, C = shape
    g = synthetic.random_matrix(61, (1, R, C), 1e-3, "normal")
    m0 = np.zeros((1, R, C), np.float32 if ns == "f32" else np.uint16)
    w0 = synthetic.random_matrix(62, (R, C), 0.02, "normal")
    eta = np.float32(1e-2)
    spectral = norm == "spectral"
    code = dtype_of(ns)[2]
    p = sm.Params(workers=1, beta=0.9, eta=float(eta), ns_iters=k, mom_dtype=code, ns_dtype=code,
                  norm=sm.NORM_SPECTRAL if spectral else sm.NORM_FROBENIUS,
                  power_iters=6 if spectral else 0)
    mat = make_matrix(g, m0, w0, polar=True, vote=False, packed=False)
    run("signmuon_muon_step", [mat], p)
    u = to_host(mat.polar_out)[0]
    w = to_host(mat.weight)
    np.testing.assert_array_equal(w, fmaf32(-eta, u, w0))
    m_ref = m0[0].copy()
    w_ref = w0.copy()
    u_ref = oracle.muon_step_matrix(g[0], m_ref, w_ref, 0.9, float(eta), k, ORC_DT[ns],
                                    norm=oracle.NORM_SPECTRAL if spectral else oracle.NORM_FROB,
                                    power_iters=6 if spectral else 0, want_u=True)
    np.testing.assert_array_equal(to_host(mat.momentum)[0], m_ref)
    err = rel_fro(u, u_ref)
    announce(f"    rel err {err:.2e}")
    assert err < NS_TOL[ns]
    # the update moves W by eta U: the deviation from the oracle's W is eta times U's
    assert np.abs(w - w_ref).max() <= float(eta) * np.abs(u - u_ref).max() * 1.001 + 1e-7


def test_muon_step_without_polar_out_moves_w_the_same():
    R, C = 300, 520
    g = synthetic.random_matrix(63, (1, R, C), 1.0, "normal")
    w0 = synthetic.random_matrix(64, (R, C), 0.02, "normal")
    p = sm.Params(workers=1, beta=0.9, eta=1e-3, ns_iters=2)
    a = make_matrix(g, np.zeros((1, R, C), np.float32), w0, polar=True, vote=False, packed=False)
    b = make_matrix(g, np.zeros((1, R, C), np.float32), w0, polar=False, vote=False, packed=False)
    run("signmuon_muon_step", [a], p)
    run("signmuon_muon_step", [b], p)
    np.testing.assert_array_equal(to_host(a.weight), to_host(b.weight))


@pytest.mark.parametrize("mom", ["f32", "bf16"])
@pytest.mark.parametrize("mw", [1, 4, 7])
def test_majority_vote_signum_is_the_k0_step(mom, mw):
    """k = 0: each worker's sign of its momentum, the majority vote, the
    update -- bit-exact against the oracle (no Newton-Schulz rounding)."""
    R, C = 192, 320
    g = np.stack([synthetic.random_matrix(70 + i, (R, C), 1e-3, "normal") for i in range(mw)])
    m0 = np.zeros((mw, R, C), np.float32 if mom == "f32" else np.uint16)
    w0 = synthetic.random_matrix(80, (R, C), 0.02, "normal")
    code = dtype_of(mom)[2]
    mat = make_matrix(g, m0, w0)
    run("signmuon_step", [mat], sm.Params(workers=mw, beta=0.9, eta=1e-3, ns_iters=0,
                                          mom_dtype=code, ns_dtype=code))
    w_ref = w0.copy()
    m_ref = m0.copy()
    packed, vote, _ = oracle.step_matrix(g, m_ref, w_ref, 0.9, 1e-3, 0, ORC_DT[mom])
    np.testing.assert_array_equal(to_host(mat.momentum), m_ref)
    np.testing.assert_array_equal(to_host(mat.packed), packed)
    np.testing.assert_array_equal(to_host(mat.vote_out), vote)
    np.testing.assert_array_equal(to_host(mat.weight), w_ref)


@pytest.mark.parametrize("mom", ["f32", "bf16"])
@pytest.mark.parametrize("mw", [1, 4, 8])
def test_signum_signs_packed_by_the_momentum_kernel(mom, mw):
    """k = 0 with no U output: the momentum kernel packs the signs of the
    stored M itself (n % 64 == 0); the other matrices in the same call take
    the separate pack of s * M (n % 8 == 0 but not 64: the 16-byte-piece
    kernel; n % 8 != 0: the per-chunk kernel). Two steps; degenerate workers
    next to ordinary ones: a zero gradient (U = 0: every bit 1), a NaN and an
    Inf entry (||M||_F is not finite, s = 0: U = 0 * M, +1 for finite entries
    and -1 for the NaN and Inf) in the first and the last matrix, and an
    extreme dynamic range (one entry near 1e38 next to -1e-10 ones, whose
    U = M / ||M||_F is about -1e-48) in a matrix the momentum kernel packs.
    Momentum, packed signs, vote and W bit-exact against the oracle's whole
    step."""
    shapes = [(192, 320), (64, 576), (37, 53), (40, 52)]
    np_m, _, code = dtype_of(mom)
    rng = np.random.default_rng(90 + mw)
    host = []
    for j, (R, C) in enumerate(shapes):
        g = np.stack([synthetic.random_matrix(900 + 10 * j + i, (R, C), 1e-3, "normal") for i in range(mw)])
        if j in (0, 3) and mw >= 4:
            g[1] = 0.0
            g[2].ravel()[rng.integers(R * C)] = np.nan
            g[3, 5, 7] = -np.inf
        if j == 1 and mw >= 4:
            g[1] = -1e-10
            g[1, 3, 3] = 1e38
        host.append((g, synthetic.random_matrix(950 + j, (R, C), 0.02, "normal")))
    mats = [make_matrix(g, np.zeros(g.shape, np_m), w, polar=False) for g, w in host]
    m_ref = [np.zeros(g.shape, np_m) for g, _ in host]
    w_ref = [w.copy() for _, w in host]
    p = sm.Params(workers=mw, beta=0.9, eta=1e-3, ns_iters=0, mom_dtype=code, ns_dtype=code)
    ws = sm.workspace_tensor(mats, p, DEV)
    for t in range(2):
        if t == 1:  # new gradients, same degenerate pattern's finite workers
            for j, (g, _) in enumerate(host):
                mats[j].grad.copy_(to_dev(g * np.float32(0.5)))
                host[j] = (g * np.float32(0.5), host[j][1])
        sm.signmuon_step(mats, p, ws)
        torch.cuda.synchronize()
        for j, (g, _) in enumerate(host):
            packed, vote, _ = oracle.step_matrix(g, m_ref[j], w_ref[j], 0.9, 1e-3, 0, ORC_DT[mom])
            np.testing.assert_array_equal(to_host(mats[j].momentum), m_ref[j], err_msg=f"M {j} step {t}")
            np.testing.assert_array_equal(to_host(mats[j].packed), packed, err_msg=f"packed {j} step {t}")
            np.testing.assert_array_equal(to_host(mats[j].vote_out), vote, err_msg=f"vote {j} step {t}")
            np.testing.assert_array_equal(to_host(mats[j].weight), w_ref[j], err_msg=f"W {j} step {t}")
