"""GPU parity of spectral normalisation (signmuon_params.norm =
SIGNMUON_NORM_SPECTRAL) against the CPU oracle on the same seeded inputs.

Bar: the polar factor within 1e-5 (fp32) / 2e-2 (bf16) relative Frobenius
error, signs agreeing on >= 99.9% of the entries with |U| >= 1e-6 max|U|;
momentum, packed signs given U, vote and update bit-exact. The power
iteration runs in fp32 on the GPU and in fp64 in the oracle, which the
tolerance covers."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import sign_muon_step_amd as sm
import synthetic
from gpu_util import (DEV, announce, dtype_of, make_matrix, rel_fro, run, sign_stats, to_dev, to_host,
                      traced_step_kinds)

pytestmark = pytest.mark.gpu

NS_TOL = {"f32": 1e-5, "bf16": 2e-2}
ORC_DT = {"f32": oracle.F32, "bf16": oracle.BF16}
POOL = ThreadPoolExecutor(max_workers=12)


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(f"[gpu-test] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def grads(seed, mw, R, C, scale=1.0):
    return np.stack([synthetic.random_matrix(seed * 1000 + i, (R, C), scale, "normal")
                     for i in range(mw)])


def params(mw, k, ns, p):
    code = dtype_of(ns)[2]
    return sm.Params(workers=mw, beta=0.9, eta=1e-3, ns_iters=k, mom_dtype=code, ns_dtype=code,
                     norm=sm.NORM_SPECTRAL, power_iters=p)


def oracle_u(m_after, k, ns, p):
    def one(mm):
        _, x0, a0 = oracle.spectral_x0_a0(mm, ORC_DT[ns], p)
        return oracle.newton_schulz_a0(x0, a0, k, ORC_DT[ns])
    return np.stack(list(POOL.map(one, list(m_after))))


def momentum_after(g, ns):
    m = np.zeros(g.shape, np.float32 if ns == "f32" else np.uint16)
    oracle.momentum(g, m, 0.9)
    return m


@pytest.mark.parametrize("ns", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(64, 200), (200, 64), (300, 300)])
@pytest.mark.parametrize("p", [1, 4])
def test_spectral_k0_is_m_over_sigma_hat(ns, shape, p):
    R, C = shape
    mw = 3
    g = grads(41, mw, R, C)
    m0 = np.zeros(g.shape, np.float32 if ns == "f32" else np.uint16)
    mat = make_matrix(g, m0, polar=True, vote=False, packed=False)
    run("signmuon_momentum_ns", [mat], params(mw, 0, ns, p))
    m_ref = momentum_after(g, ns)
    np.testing.assert_array_equal(to_host(mat.momentum), m_ref)
    u = to_host(mat.polar_out)
    for w in range(mw):
        _, x0, _ = oracle.spectral_x0_a0(m_ref[w], ORC_DT[ns], p)
        assert rel_fro(u[w], x0) < 1e-5


NS_CASES = ([("f32", s, k, p) for s in [(256, 256), (300, 700), (700, 300), (64, 576)]
             for k, p in [(1, 1), (1, 6), (3, 4)]]
            + [("bf16", s, k, p) for s in [(384, 1024), (1024, 384), (300, 704), (256, 256)]
               for k, p in [(1, 2), (1, 8), (3, 5)]])


@pytest.mark.parametrize("ns,shape,k,p", NS_CASES)
def test_spectral_newton_schulz_parity(ns, shape, k, p):
    R, C = shape
    mw = 2
    g = grads(43 + k + p, mw, R, C)
    m0 = np.zeros(g.shape, np.float32 if ns == "f32" else np.uint16)
    mat = make_matrix(g, m0, polar=True, vote=False, packed=False)
    run("signmuon_momentum_ns", [mat], params(mw, k, ns, p))
    u_ref = oracle_u(momentum_after(g, ns), k, ns, p)
    u = to_host(mat.polar_out)
    for w in range(mw):
        err = rel_fro(u[w], u_ref[w])
        agree, bad, n = sign_stats(u[w], u_ref[w])
        announce(f"    worker {w}: rel err {err:.2e}, sign agreement {agree:.6f} ({bad} of {n} differ)")
        assert err < NS_TOL[ns]
        assert agree >= 0.999


@pytest.mark.parametrize("ns", ["f32", "bf16"])
def test_spectral_step_vote_and_update(ns):
    mw, R, C = 5, 128, 320
    g = grads(47, mw, R, C)
    m0 = np.zeros(g.shape, np.float32 if ns == "f32" else np.uint16)
    w0 = synthetic.random_matrix(48, (R, C), 0.02, "normal")
    mat = make_matrix(g, m0, w0)
    run("signmuon_step", [mat], params(mw, 2, ns, 5))
    u = to_host(mat.polar_out)
    packed = to_host(mat.packed)
    for w in range(mw):
        np.testing.assert_array_equal(packed[w], oracle.sign_pack(u[w]))
    w_ref = w0.copy()
    vote_ref = oracle.vote_update(packed, w_ref.ravel(), 1e-3)
    np.testing.assert_array_equal(to_host(mat.vote_out).ravel(), vote_ref)
    np.testing.assert_array_equal(to_host(mat.weight), w_ref)
    u_ref = oracle_u(momentum_after(g, ns), 2, ns, 5)
    for w in range(mw):
        assert rel_fro(u[w], u_ref[w]) < NS_TOL[ns]


def test_spectral_zero_momentum_gives_all_plus_signs():
    mw, R, C = 2, 64, 128
    g = np.zeros((mw, R, C), np.float32)
    for k in (0, 2):
        mat = make_matrix(g, np.zeros((mw, R, C), np.float32), np.zeros((R, C), np.float32))
        run("signmuon_step", [mat], params(mw, k, "f32", 3))
        assert not to_host(mat.polar_out).any()
        assert (to_host(mat.packed) == np.uint64(0xFFFFFFFFFFFFFFFF)).all()


def test_spectral_gpt2_shape_full_size():
    """768 x 3072 (GPT-2 small MLP) in bf16 with 8 power steps; two workers
    checked against the full oracle."""
    R, C, mw, k, p = 768, 3072, 2, 1, 8
    g = grads(49, mw, R, C, 1e-3)
    m0 = np.zeros(g.shape, np.uint16)
    mat = make_matrix(g, m0, polar=True, vote=False, packed=False)
    run("signmuon_momentum_ns", [mat], params(mw, k, "bf16", p))
    u_ref = oracle_u(momentum_after(g, "bf16"), k, "bf16", p)
    u = to_host(mat.polar_out)
    for w in range(mw):
        err = rel_fro(u[w], u_ref[w])
        agree, bad, n = sign_stats(u[w], u_ref[w])
        announce(f"    worker {w}: rel err {err:.2e}, sign agreement {agree:.6f} ({bad} of {n} differ)")
        assert err < NS_TOL["bf16"]
        assert agree >= 0.999


@pytest.mark.parametrize("ns", ["f32", "bf16"])
@pytest.mark.parametrize("k", [0, 1])
def test_spectral_power_iteration_in_one_launch(ns, k):
    """A batch of at least half a device of (matrix, worker) units, every r a
    multiple of 8 and at most 1016 (bf16) or 504 (fp32), takes the power
    iteration with one
    workgroup per unit: all p steps and the scales in a single launch, the
    steps reading the upper part of A only (A stays unscaled; the first
    product applies s^2 to its accumulators). U of
    the first and last worker of each distinct shape against the oracle; the
    packed signs of every worker equal those of its stored U."""
    shapes = [(64, 200), (200, 64), (128, 320), (256, 256), (200, 448), (448, 200)] * 4
    mw, p = 8, 4
    np_m = np.float32 if ns == "f32" else np.uint16
    g = [grads(60 + j, mw, R, C) for j, (R, C) in enumerate(shapes)]
    mats = [make_matrix(g[j], np.zeros(g[j].shape, np_m), np.zeros(s_, np.float32))
            for j, s_ in enumerate(shapes)]
    kinds = traced_step_kinds(mats, params(mw, k, ns, p))
    announce(f"  {len(shapes)} matrices x {mw} workers, k = {k}: launches {kinds}")
    assert kinds.count("power") == 1
    for j in range(len(shapes)):
        u, packed = to_host(mats[j].polar_out), to_host(mats[j].packed)
        for w in range(mw):
            np.testing.assert_array_equal(packed[w], oracle.sign_pack(u[w]))
    for j in range(6):
        m_ref = momentum_after(g[j], ns)
        np.testing.assert_array_equal(to_host(mats[j].momentum), m_ref)
        u = to_host(mats[j].polar_out)
        for w in (0, mw - 1):
            if k == 0:
                ref = oracle.spectral_x0_a0(m_ref[w], ORC_DT[ns], p)[1]
                tol = 1e-5
            else:
                ref = oracle_u(m_ref[w:w + 1], k, ns, p)[0]
                tol = NS_TOL[ns]
            err = rel_fro(u[w], ref)
            announce(f"    {shapes[j]} worker {w}: rel err {err:.2e} (bound {tol:.0e})")
            assert err < tol


@pytest.mark.parametrize("ns", ["f32", "bf16"])
def test_spectral_one_launch_at_its_widest(ns):
    """The one-launch power iteration at r up to its limit (1016 in bf16, 504
    in fp32), where a pair of row groups spreads over two chunks per lane,
    and at r = 768 (the GPT-2 shapes): 16 matrices x 8 workers, k = 1. U of
    the first and last worker of each distinct shape against the oracle."""
    shapes = ([(768, 1536), (1016, 1016), (1536, 768), (512, 600)] if ns == "bf16"
              else [(504, 504), (256, 512), (480, 256), (264, 256)])
    mw, p, k = 8, 6, 1
    np_m = np.float32 if ns == "f32" else np.uint16
    g = list(POOL.map(lambda j: grads(90 + j, mw, *shapes[j]), range(len(shapes))))
    mats = [make_matrix(g[j % 4], np.zeros(g[j % 4].shape, np_m), np.zeros(shapes[j % 4], np.float32))
            for j in range(16)]
    kinds = traced_step_kinds(mats, params(mw, k, ns, p))
    announce(f"  16 matrices x {mw} workers, k = {k}: launches {kinds}")
    assert kinds.count("power") == 1
    for j in range(4):
        m_ref = momentum_after(g[j], ns)
        for jj in (j, j + 12):
            np.testing.assert_array_equal(to_host(mats[jj].momentum), m_ref)
        u, u_last = to_host(mats[j].polar_out), to_host(mats[j + 12].polar_out)
        np.testing.assert_array_equal(u, u_last)
        refs = oracle_u(m_ref[[0, mw - 1]], k, ns, p)
        for w, ref in zip((0, mw - 1), refs):
            err = rel_fro(u[w], ref)
            announce(f"    {shapes[j]} worker {w}: rel err {err:.2e} (bound {NS_TOL[ns]:.0e})")
            assert err < NS_TOL[ns]
