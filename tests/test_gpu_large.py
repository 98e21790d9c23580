"""Full-size GPU checks of the two larger workloads: GPT-2 small shapes with 16
workers, 5 Newton-Schulz iterations and Student-t(3) gradients (with and
without the post-vote polar step), and a large transformer block (4 x
4096x4096, 4096x11008, 11008x4096) with 16 workers.

At these sizes the oracle cannot run every whole matrix, so the checks are
the ones that hold at any size, plus whole-matrix or sampled oracle values
where the oracle is fast enough:
  - momentum bit-exact on sampled rows of two workers (oracle O1);
  - the packed bits equal the signs of the GPU's own U (oracle O4+O5);
  - the vote and W bit-exact against the oracle's vote of the GPU's packed
    signs (O6+O7), over every entry of every matrix;
  - ||U||_2 <= 1 (the spectral-norm bound of the Newton-Schulz iterate, up to
    bf16 rounding), by power iteration on the host;
  - GPT-2 shapes: U of one 768 x 768 matrix against the oracle's full k = 5
    iteration, and the post-vote polar step's W against the oracle's;
  - block shapes: sampled entries of U at k = 1 against the oracle's
    per-entry k = 1 formula, for the 4096 x 11008 and 11008 x 4096 matrices."""
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import sign_muon_step_amd as sm
import synthetic
from gpu_util import DEV, announce, rel_fro, sign_stats, to_dev, to_host

pytestmark = pytest.mark.gpu

POOL = ThreadPoolExecutor(max_workers=16)


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(f"[gpu-test] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def spectral_norm(u: np.ndarray, iters: int = 40) -> float:
    """Largest singular value of u by power iteration on u^T u (fp64)."""
    u = u.astype(np.float64)
    v = np.ones(u.shape[1]) / np.sqrt(u.shape[1])
    s = 0.0
    for _ in range(iters):
        w = u.T @ (u @ v)
        n = np.linalg.norm(w)
        if n == 0:
            return 0.0
        v = w / n
        s = np.sqrt(n)
    return float(s)


def upload_gradients(wl, keep):
    """Device gradients of every matrix, drawn per (matrix, worker) from the
    seeded generator; the host keeps the (matrix, worker) arrays in keep."""
    dev = [torch.empty((wl.workers,) + tuple(s), dtype=torch.float32, device=DEV) for s in wl.shapes]
    host = {}

    def one(jm):
        j, m = jm
        return jm, synthetic.gradient(wl, j, m, 0)

    jobs = [(j, m) for j in range(len(wl.shapes)) for m in range(wl.workers)]
    for (j, m), g in POOL.map(one, jobs):
        dev[j][m].copy_(torch.from_numpy(g))
        if (j, m) in keep:
            host[(j, m)] = g
    torch.cuda.synchronize()
    return dev, host


def run_step(wl, grads, k, polar_for=(), post=0):
    mats = []
    for j, (R, C) in enumerate(wl.shapes):
        mats.append(sm.Matrix(
            grad=grads[j], momentum=torch.zeros((wl.workers, R, C), dtype=torch.bfloat16, device=DEV),
            packed=torch.zeros((wl.workers, sm.signmuon_packed_words(R * C)), dtype=torch.int64,
                               device=DEV),
            weight=to_dev(synthetic.initial_weight(wl, j)),
            polar_out=torch.zeros((wl.workers, R, C), dtype=torch.float32, device=DEV)
            if j in polar_for else None,
            vote_out=torch.zeros((R, C), dtype=torch.int8, device=DEV)))
    params = sm.Params(workers=wl.workers, beta=wl.beta, eta=wl.eta, ns_iters=k,
                       post_polar_iters=post, mom_dtype=sm.BF16, ns_dtype=sm.BF16)
    ws = sm.workspace_tensor(mats, params, DEV)
    announce(f"  launching {wl.name}: k = {k}, post-polar {post}")
    sm.signmuon_step(mats, params, ws)
    torch.cuda.synchronize()
    del ws
    return mats


def check_momentum_rows(wl, mats, host, rng):
    for (j, m), g in host.items():
        R, C = wl.shapes[j]
        rows = np.sort(rng.choice(R, 8, replace=False))
        m_ref = np.zeros((8, C), np.uint16)
        oracle.momentum(np.ascontiguousarray(g[rows]), m_ref, wl.beta)
        got = to_host(mats[j].momentum[m][torch.from_numpy(rows).to(DEV)])
        np.testing.assert_array_equal(got, m_ref, err_msg=f"momentum {j} worker {m}")


def check_vote_all(wl, mats):
    for j, mat in enumerate(mats):
        packed = to_host(mat.packed)
        w_ref = synthetic.initial_weight(wl, j).copy()
        vote = oracle.vote_update(packed, w_ref, wl.eta)
        np.testing.assert_array_equal(to_host(mat.vote_out), vote, err_msg=f"vote {j}")
        np.testing.assert_array_equal(to_host(mat.weight), w_ref, err_msg=f"W {j}")


def test_gpt2_shapes_mw16_k5_full_size():
    wl = synthetic.WORKLOADS["gpt2s_mw16_k5_t3"]
    keep = {(1, 0), (1, wl.workers - 1), (2, 0), (3, wl.workers - 1)}
    grads, host = upload_gradients(wl, keep)
    mats = run_step(wl, grads, wl.ns_iters, polar_for=(0, 1, 2, 3))
    rng = np.random.default_rng(5)
    check_momentum_rows(wl, mats, host, rng)
    for j in (0, 1, 2, 3):
        u = to_host(mats[j].polar_out)
        packed = to_host(mats[j].packed)
        for w in (0, wl.workers - 1):
            np.testing.assert_array_equal(packed[w], oracle.sign_pack(u[w]), err_msg=f"pack {j} {w}")
            norm2 = spectral_norm(u[w])
            announce(f"  {wl.shapes[j]} worker {w}: ||U||_2 = {norm2:.5f}")
            assert norm2 <= 1.02
    # one whole 768 x 768 matrix against the oracle's five iterations
    m_ref = np.zeros((768, 768), np.uint16)
    oracle.momentum(host[(1, 0)], m_ref, wl.beta)
    _, x0 = oracle.normalise(m_ref)
    u_ref = oracle.newton_schulz(x0, wl.ns_iters, oracle.BF16)
    u0 = to_host(mats[1].polar_out)[0]
    err = rel_fro(u0, u_ref)
    agree, bad, n = sign_stats(u0, u_ref)
    announce(f"  768x768 worker 0, k = 5: rel err {err:.2e}, sign agreement {agree:.6f} "
             f"({bad} of {n} differ)")
    assert err < 2e-2 and agree >= 0.999
    check_vote_all(wl, mats)  # 16 workers: even, so ties vote 0


def test_gpt2_shapes_mw16_k5_post_polar_full_size():
    wl = synthetic.WORKLOADS["gpt2s_mw16_k5_t3_postpolar"]
    grads, _ = upload_gradients(wl, set())
    mats = run_step(wl, grads, wl.ns_iters, post=wl.post_polar_iters)
    for j, mat in enumerate(mats):
        packed = to_host(mat.packed)
        w_tmp = synthetic.initial_weight(wl, j).copy()
        vote = oracle.vote_update(packed, w_tmp, wl.eta)  # the vote of the GPU's own signs
        np.testing.assert_array_equal(to_host(mat.vote_out), vote, err_msg=f"vote {j}")
        if j == 1:  # a 768 x 768 matrix: the oracle's polar step on that vote
            w0 = synthetic.initial_weight(wl, j)
            w_ref = w0.copy()
            nnz = oracle.post_polar(vote, w_ref, wl.eta, wl.post_polar_iters, oracle.BF16)
            assert nnz > 0
            y_gpu = (to_host(mat.weight).astype(np.float64) - w0) / -wl.eta
            y_ref = (w_ref.astype(np.float64) - w0) / -wl.eta
            err = rel_fro(y_gpu, y_ref)
            announce(f"  post-polar 768x768: rel err of Y {err:.2e}")
            assert err <= 2e-2 + 1e-4


def test_block4096_full_size():
    wl = synthetic.WORKLOADS["block4096_mw16_k5"]
    mw = wl.workers
    keep = {(0, 0), (4, 0), (4, mw - 1), (5, 0), (5, mw - 1)}
    t0 = time.perf_counter()
    grads, host = upload_gradients(wl, keep)
    announce(f"  gradients drawn and uploaded in {time.perf_counter() - t0:.1f} s")
    rng = np.random.default_rng(6)
    # k = 1 first: sampled entries of U against the oracle's per-entry formula
    t0 = time.perf_counter()
    mats = run_step(wl, grads, 1, polar_for=(4, 5))
    check_momentum_rows(wl, mats, host, rng)
    announce(f"  k = 1 step and momentum rows in {time.perf_counter() - t0:.1f} s")
    t0 = time.perf_counter()
    for j in (4, 5):
        R, C = wl.shapes[j]
        u = mats[j].polar_out
        for w in (0, mw - 1):
            m_ref = np.zeros((R, C), np.uint16)
            oracle.momentum(host[(j, w)], m_ref, wl.beta)
            _, x0 = oracle.normalise(m_ref)
            ri = rng.integers(0, R, 16)
            ci = rng.integers(0, C, 16)
            ref = oracle.ns1_entries(x0, oracle.BF16, ri, ci)
            got = to_host(u[w][torch.from_numpy(ri).to(DEV), torch.from_numpy(ci).to(DEV)])
            rms = float(torch.sqrt(torch.mean(u[w].double() ** 2)).item())
            dev_rel = np.abs(got.astype(np.float64) - ref).max() / rms
            announce(f"  {wl.shapes[j]} worker {w}, k = 1: max|dU|/rms(U) = {dev_rel:.3e}")
            assert dev_rel <= 2e-2
        packed = to_host(mats[j].packed)
        for w in (0, mw - 1):
            np.testing.assert_array_equal(packed[w], oracle.sign_pack(to_host(u[w])))
    announce(f"  sampled k = 1 entries and packed bits in {time.perf_counter() - t0:.1f} s")
    del mats
    t0 = time.perf_counter()
    # the workload itself: k = 5
    mats = run_step(wl, grads, wl.ns_iters, polar_for=(0,))
    check_momentum_rows(wl, mats, host, rng)
    u = to_host(mats[0].polar_out[0])
    np.testing.assert_array_equal(to_host(mats[0].packed)[0], oracle.sign_pack(u))
    norm2 = spectral_norm(u)
    announce(f"  4096x4096 worker 0, k = 5: ||U||_2 = {norm2:.5f} "
             f"({time.perf_counter() - t0:.1f} s with the k = 5 step)")
    assert norm2 <= 1.02
    t0 = time.perf_counter()
    check_vote_all(wl, mats)
    announce(f"  vote and W of every matrix in {time.perf_counter() - t0:.1f} s")
