"""GPU parity of the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bar: momentum, pack, vote and update bit-exact (pack/vote/update given the
same sign inputs); the Newton-Schulz factor within 1e-5 (fp32) / 2e-2 (bf16)
relative Frobenius error; signs agree on >= 99.9% of the entries with
|U| >= 1e-6 max|U|, every residual disagreement reported.
"""
import json
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import sign_muon_step_amd as sm
import synthetic
from gpu_util import (DEV, announce, bit_sign_stats, dtype_of, make_matrix, rel_fro, run, sign_stats,
                      to_dev, to_host)

pytestmark = pytest.mark.gpu

NS_TOL = {"f32": 1e-5, "bf16": 2e-2}
ORC_DT = {"f32": oracle.F32, "bf16": oracle.BF16}
POOL = ThreadPoolExecutor(max_workers=12)


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(f"[gpu-test] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def grads(seed, mw, R, C, scale=1.0, dist="normal"):
    return np.stack([synthetic.random_matrix(seed * 1000 + i, (R, C), scale, dist)
                     for i in range(mw)])


def zeros_m(mw, R, C, mom):
    return np.zeros((mw, R, C), np.float32 if mom == "f32" else np.uint16)


def oracle_u(m_after, k, ns):
    """fp64 U of each worker from the stored momentum (oracle O2 + O3)."""
    def one(mm):
        _, x0 = oracle.normalise(mm)
        return oracle.newton_schulz(x0, k, ORC_DT[ns])
    return np.stack(list(POOL.map(one, list(m_after))))


# ---------------------------------------------------------------------------
# momentum (bit-exact) and the k = 0 polar output U = M / ||M||_F
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("gdt,mom", [("f32", "f32"), ("f32", "bf16"), ("bf16", "bf16"),
                                     ("bf16", "f32")])
@pytest.mark.parametrize("shape", [(37, 53), (256, 256), (1, 9), (700, 300)])
def test_momentum_bitexact_two_steps(gdt, mom, shape):
    R, C = shape
    mw = 3
    m_host = zeros_m(mw, R, C, mom)
    m_dev = to_dev(m_host)
    for step in range(2):
        g = grads(10 + step, mw, R, C)
        if gdt == "bf16":
            g = oracle.bf16_from_f32(g)
        mat = sm.Matrix(grad=to_dev(g), momentum=m_dev,
                        polar_out=torch.zeros((mw, R, C), dtype=torch.float32, device=DEV))
        run("signmuon_momentum_ns", [mat],
            sm.Params(workers=mw, beta=0.9, ns_iters=0, grad_dtype=dtype_of(gdt)[2],
                      mom_dtype=dtype_of(mom)[2], ns_dtype=dtype_of(mom)[2]))
        oracle.momentum(g, m_host, 0.9)
        np.testing.assert_array_equal(to_host(m_dev), m_host)
        u = to_host(mat.polar_out)
        for w in range(mw):
            _, x0 = oracle.normalise(m_host[w])
            assert rel_fro(u[w], x0) < 1e-6


def test_zero_gradient_gives_all_plus_signs():
    """M = 0 has no direction: U = 0 and every packed bit is 1 (+1)."""
    mw, R, C = 2, 64, 128
    g = np.zeros((mw, R, C), np.float32)
    for k in (0, 1, 3):
        mat = make_matrix(g, zeros_m(mw, R, C, "f32"), np.zeros((R, C), np.float32))
        run("signmuon_step", [mat], sm.Params(workers=mw, ns_iters=k))
        assert not to_host(mat.polar_out).any()
        assert (to_host(mat.packed) == np.uint64(0xFFFFFFFFFFFFFFFF)).all()
        assert (to_host(mat.vote_out) == 1).all()


# ---------------------------------------------------------------------------
# sign + pack (bit-exact)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("udt", ["f32", "bf16"])
@pytest.mark.parametrize("n,workers", [(1, 1), (63, 2), (64, 1), (65, 3), (4097, 2), (100003, 5),
                                       (2048 * 33 + 7, 1),
                                       # n % 8 == 0: the 16-byte-piece kernel, words staged in LDS;
                                       # one chunk, a partial last word, several blocks (8192 fp32 /
                                       # 16384 bf16 entries each) with a partial last block
                                       (8, 3), (72, 2), (8192 + 24, 2), (16384 * 3 + 8, 2), (100000, 3)])
def test_sign_pack_bitexact(udt, n, workers):
    rng = np.random.default_rng(n)
    u = rng.standard_normal((workers, n)).astype(np.float32)
    u.ravel()[rng.integers(0, u.size, max(1, u.size // 50))] = 0.0
    u.ravel()[rng.integers(0, u.size, max(1, u.size // 50))] = -0.0
    u.ravel()[rng.integers(0, u.size, max(1, u.size // 97))] = np.nan
    if udt == "bf16":
        u = oracle.bf16_from_f32(u)
    nw = sm.signmuon_packed_words(n)
    packed = torch.full((workers, nw), -1, dtype=torch.int64, device=DEV)
    sm.signmuon_sign_pack(to_dev(u), n, workers, packed)
    torch.cuda.synchronize()
    got = to_host(packed)
    for w in range(workers):
        np.testing.assert_array_equal(got[w], oracle.sign_pack(u[w]))


def test_sign_pack_golden_vectors(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "pack_vectors.json")))
    for case in spec["cases"]:
        vals = []
        for v, cnt in case["runs"]:
            x = {"nan": np.nan, "-0": -0.0}.get(v, v) if isinstance(v, str) else float(v)
            vals += [x] * cnt
        u = np.array(vals, np.float32)[None, :]
        packed = torch.zeros((1, sm.signmuon_packed_words(u.size)), dtype=torch.int64, device=DEV)
        sm.signmuon_sign_pack(to_dev(u), u.size, 1, packed)
        torch.cuda.synchronize()
        expect = np.array([int(h, 16) for h in case["expected_words_hex"]], np.uint64)
        np.testing.assert_array_equal(to_host(packed)[0], expect, err_msg=case["name"])


# ---------------------------------------------------------------------------
# vote + update (bit-exact)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mw", [1, 2, 3, 4, 5, 8, 10, 15, 16, 17, 31, 64, 255])
@pytest.mark.parametrize("n", [1, 100, 4096, 4096 * 4 + 37, 300001])
def test_vote_update_bitexact(mw, n):
    rng = np.random.default_rng(mw * 7 + n)
    nw = (n + 63) // 64
    bits = rng.integers(0, 2, (mw, nw * 64), dtype=np.uint8)
    bits[:, n:] = 0
    packed = np.packbits(bits, axis=1, bitorder="little").view(np.uint64).reshape(mw, nw)
    w0 = rng.standard_normal(n).astype(np.float32) * np.float32(0.02)
    eta = 1e-3
    w_dev = to_dev(w0)
    vote_dev = torch.zeros(n, dtype=torch.int8, device=DEV)
    sm.signmuon_vote_update(to_dev(packed), mw, n, w_dev, eta, vote_dev)
    torch.cuda.synchronize()
    w_ref = w0.copy()
    vote_ref = oracle.vote_update(packed, w_ref, eta)
    np.testing.assert_array_equal(to_host(vote_dev), vote_ref)
    np.testing.assert_array_equal(to_host(w_dev), w_ref)


def test_vote_only_and_update_only():
    rng = np.random.default_rng(5)
    mw, n = 6, 5000
    nw = (n + 63) // 64
    bits = rng.integers(0, 2, (mw, nw * 64), dtype=np.uint8)
    bits[:, n:] = 0
    packed = np.packbits(bits, axis=1, bitorder="little").view(np.uint64).reshape(mw, nw)
    w0 = rng.standard_normal(n).astype(np.float32)
    w_ref = w0.copy()
    vote_ref = oracle.vote_update(packed, w_ref, 0.5)
    vote_dev = torch.zeros(n, dtype=torch.int8, device=DEV)
    sm.signmuon_vote_update(to_dev(packed), mw, n, None, 0.5, vote_dev)
    w_dev = to_dev(w0)
    sm.signmuon_vote_update(to_dev(packed), mw, n, w_dev, 0.5, None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(vote_dev), vote_ref)
    np.testing.assert_array_equal(to_host(w_dev), w_ref)


def test_vote_worked_example_from_pages(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "vote_worked_example.json")))
    for case in spec["cases"]:
        mw, plus = case["workers"], case["plus_votes"]
        packed = np.zeros((mw, 1), np.uint64)
        packed[:plus, 0] = 1
        w = to_dev(np.zeros(1, np.float32))
        vote = torch.zeros(1, dtype=torch.int8, device=DEV)
        sm.signmuon_vote_update(to_dev(packed), mw, 1, w, 1.0, vote)
        torch.cuda.synchronize()
        assert int(to_host(vote)[0]) == case["expected_vote"]
        assert float(to_host(w)[0]) == -float(case["expected_vote"])


# ---------------------------------------------------------------------------
# Newton-Schulz factor (tolerance + sign agreement)
# ---------------------------------------------------------------------------
NS_CASES = ([("f32", s, k) for s in [(256, 256), (300, 700), (700, 300), (64, 576), (513, 260),
                                      (130, 258), (1, 300), (300, 1), (1, 1)] for k in (1, 2, 5)]
            + [("bf16", s, k) for s in [(768, 768), (384, 1024), (1024, 384), (300, 704),
                                       (704, 300), (256, 520), (200, 333)] for k in (1, 2, 5)])


@pytest.mark.parametrize("ns,shape,k", NS_CASES)
def test_newton_schulz_parity(ns, shape, k):
    R, C = shape
    mw = 2
    g = grads(77 + R + C, mw, R, C, 1e-3)
    m_host = zeros_m(mw, R, C, ns)
    mat = sm.Matrix(grad=to_dev(g), momentum=to_dev(m_host),
                    polar_out=torch.zeros((mw, R, C), dtype=torch.float32, device=DEV))
    run("signmuon_momentum_ns", [mat],
        sm.Params(workers=mw, ns_iters=k, mom_dtype=dtype_of(ns)[2], ns_dtype=dtype_of(ns)[2]))
    oracle.momentum(g, m_host, 0.9)
    np.testing.assert_array_equal(to_host(mat.momentum), m_host)
    u_ref = oracle_u(m_host, k, ns)
    u = to_host(mat.polar_out)
    for w in range(mw):
        err = rel_fro(u[w], u_ref[w])
        agree, bad, cnt = sign_stats(u[w], u_ref[w])
        announce(f"  {ns} {shape} k={k} worker {w}: rel_fro={err:.3e} sign agreement "
                 f"{agree:.6f} ({bad} of {cnt} differ)")
        assert err <= NS_TOL[ns]
        assert agree >= 0.999


@pytest.mark.parametrize("ns", ["f32", "bf16"])
def test_newton_schulz_grouped_launch_matches_single(ns):
    """Several matrices and workers in one call give the same bits as each
    matrix alone (no cross-talk between the tiles of a grouped launch)."""
    shapes = [(256, 512), (512, 256), (96, 96), (300, 704)]
    mw, k = 3, 2
    gs = [grads(200 + i, mw, R, C, 1e-3) for i, (R, C) in enumerate(shapes)]
    params = sm.Params(workers=mw, ns_iters=k, mom_dtype=dtype_of(ns)[2], ns_dtype=dtype_of(ns)[2])
    together = [make_matrix(g, zeros_m(mw, *g.shape[1:], ns), np.zeros(g.shape[1:], np.float32))
                for g in gs]
    run("signmuon_step", together, params)
    for g, t in zip(gs, together):
        alone = make_matrix(g, zeros_m(mw, *g.shape[1:], ns), np.zeros(g.shape[1:], np.float32))
        run("signmuon_step", [alone], params)
        np.testing.assert_array_equal(to_host(alone.polar_out), to_host(t.polar_out))
        np.testing.assert_array_equal(to_host(alone.packed), to_host(t.packed))
        np.testing.assert_array_equal(to_host(alone.weight), to_host(t.weight))


# ---------------------------------------------------------------------------
# whole step on the small workloads
# ---------------------------------------------------------------------------
def check_step(wl: synthetic.Workload, steps=1, matrices=None, label=""):
    idx = list(range(len(wl.shapes))) if matrices is None else matrices
    mom_np, _, mom_code = dtype_of(wl.mom_dtype)
    ns_code = dtype_of(wl.ns_dtype)[2]
    params = sm.Params(workers=wl.workers, beta=wl.beta, eta=wl.eta, ns_iters=wl.ns_iters,
                       post_polar_iters=wl.post_polar_iters, mom_dtype=mom_code, ns_dtype=ns_code)
    host = {j: (np.zeros((wl.workers,) + wl.shapes[j], mom_np), synthetic.initial_weight(wl, j))
            for j in idx}
    dev = {j: (to_dev(host[j][0]), to_dev(host[j][1])) for j in idx}
    for t in range(steps):
        gs = dict(zip(idx, POOL.map(lambda j: synthetic.gradients(wl, j, t), idx)))
        mats = []
        for j in idx:
            R, C = wl.shapes[j]
            mats.append(sm.Matrix(
                grad=to_dev(gs[j]), momentum=dev[j][0], weight=dev[j][1],
                packed=torch.zeros((wl.workers, sm.signmuon_packed_words(R * C)), dtype=torch.int64,
                                   device=DEV),
                polar_out=torch.zeros((wl.workers, R, C), dtype=torch.float32, device=DEV),
                vote_out=torch.zeros((R, C), dtype=torch.int8, device=DEV)))
        run("signmuon_step", mats, params)
        for j, mat in zip(idx, mats):
            m_host, w_host = host[j]
            oracle.momentum(gs[j], m_host, wl.beta)
            np.testing.assert_array_equal(to_host(mat.momentum), m_host, err_msg=f"M {j} step {t}")
            u = to_host(mat.polar_out)
            u_ref = oracle_u(m_host, wl.ns_iters, wl.ns_dtype)
            packed = to_host(mat.packed)
            for w in range(wl.workers):
                np.testing.assert_array_equal(packed[w], oracle.sign_pack(u[w]),
                                              err_msg=f"pack {j} worker {w}")
                err = rel_fro(u[w], u_ref[w])
                agree, bad, cnt = sign_stats(u[w], u_ref[w])
                announce(f"  {label} step {t} matrix {j} {wl.shapes[j]} worker {w}: rel_fro={err:.3e}"
                         f" sign agreement {agree:.6f} ({bad} of {cnt} differ)")
                assert err <= NS_TOL[wl.ns_dtype]
                assert agree >= 0.999
            # vote + update given the GPU's packed signs: bit-exact
            vote = oracle.vote_update(packed, w_host, wl.eta)
            np.testing.assert_array_equal(to_host(mat.vote_out), vote, err_msg=f"vote {j}")
            np.testing.assert_array_equal(to_host(mat.weight), w_host, err_msg=f"W {j}")


def test_step_square256_workload():
    check_step(synthetic.WORKLOADS["square256_mw4_k1"], steps=3, label="square256")


def test_step_resnet50_four_shapes_k1():
    check_step(synthetic.WORKLOADS["resnet50_4shapes_mw4_k1"], steps=2, label="resnet50 k1")


def test_step_resnet50_k5_small_shapes():
    check_step(synthetic.WORKLOADS["resnet50_4shapes_mw4_k5"], steps=1, matrices=[0, 1],
               label="resnet50 k5")


def test_step_resnet50_k5_large_shapes():
    """The two larger conv shapes (512 x 4608, 2048 x 512) at k = 5 in fp32."""
    check_step(synthetic.WORKLOADS["resnet50_4shapes_mw4_k5"], steps=1, matrices=[2, 3],
               label="resnet50 k5 large")


def test_step_resnet50_all_convs_subset():
    """Ragged shapes (64 x 147: no fused pack) next to regular ones."""
    check_step(synthetic.WORKLOADS["resnet50_all_convs_mw4_k1"], steps=1,
               matrices=[0, 1, 2, 3, 5, 8], label="resnet50 all")


def test_step_resnet50_every_conv():
    """All 53 ResNet-50 conv weights (23.5M parameters, 4 workers, k = 1, fp32),
    the ragged ones (C % 64 != 0: no fused pack) included."""
    check_step(synthetic.WORKLOADS["resnet50_all_convs_mw4_k1"], steps=1, label="resnet50 all 53")


def test_step_gpt2_shapes_mw16_k5_one_layer():
    """Student-t gradients, 16 workers (ties), 5 iterations, bf16: one layer."""
    check_step(synthetic.WORKLOADS["gpt2s_mw16_k5_t3"].with_(workers=4), steps=1,
               matrices=[1], label="gpt2 k5")


def test_step_is_deterministic():
    wl = synthetic.WORKLOADS["gpt2s_mw8_k1"]
    shapes = [(768, 768), (3072, 768)]
    outs = []
    for _ in range(2):
        mats = []
        for j, (R, C) in enumerate(shapes):
            g = grads(300 + j, 4, R, C, 1e-3)
            mats.append(make_matrix(g, zeros_m(4, R, C, "bf16"), np.zeros((R, C), np.float32)))
        run("signmuon_step", mats, sm.Params(workers=4, ns_iters=2, mom_dtype=sm.BF16,
                                             ns_dtype=sm.BF16))
        outs.append([(to_host(m.polar_out), to_host(m.packed), to_host(m.weight)) for m in mats])
    for a, b in zip(*outs):
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)
    del wl


# ---------------------------------------------------------------------------
# optional post-vote polar step
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("ns", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(256, 512), (512, 256), (100, 130)])
def test_post_polar_step(ns, shape):
    R, C = shape
    mw, k, kp, eta = 4, 1, 2, 1e-3
    g = grads(400 + R, mw, R, C, 1e-3, "student_t3")
    w0 = synthetic.random_matrix(401, (R, C), 0.02)
    mat = make_matrix(g, zeros_m(mw, R, C, ns), w0)
    run("signmuon_step", [mat], sm.Params(workers=mw, ns_iters=k, post_polar_iters=kp,
                                          mom_dtype=dtype_of(ns)[2], ns_dtype=dtype_of(ns)[2]))
    packed = to_host(mat.packed)
    w_tmp = w0.copy()
    vote = oracle.vote_update(packed, w_tmp, eta)  # the vote of the GPU's own signs
    np.testing.assert_array_equal(to_host(mat.vote_out), vote)
    w_ref = w0.copy()
    nnz = oracle.post_polar(vote, w_ref, eta, kp, ORC_DT[ns])
    assert nnz > 0
    y_gpu = (to_host(mat.weight).astype(np.float64) - w0) / -eta
    y_ref = (w_ref.astype(np.float64) - w0) / -eta
    err = rel_fro(y_gpu, y_ref)
    announce(f"  post-polar {ns} {shape}: rel_fro(Y) = {err:.3e}")
    assert err <= NS_TOL[ns] + 1e-4  # W's own fp32 rounding adds ~|W| ulp / eta


# ---------------------------------------------------------------------------
# the GPT-2 small workload at full size (84.9M parameters, 8 workers)
# ---------------------------------------------------------------------------
def gpt2_state(wl, polar_for=()):
    """Device buffers of the benchmarked workload: as bench.py passes them
    (packed signs and W; no U, no vote output), plus fp32 U for the matrices
    in polar_for."""
    mw = wl.workers
    return [sm.Matrix(
        grad=torch.empty((mw, R, C), dtype=torch.float32, device=DEV),
        momentum=torch.zeros((mw, R, C), dtype=torch.bfloat16, device=DEV),
        weight=to_dev(synthetic.initial_weight(wl, j)),
        packed=torch.zeros((mw, sm.signmuon_packed_words(R * C)), dtype=torch.int64, device=DEV),
        polar_out=torch.zeros((mw, R, C), dtype=torch.float32, device=DEV) if j in polar_for else None,
        vote_out=None) for j, (R, C) in enumerate(wl.shapes)]


def test_gpt2_small_full_size_bench_launches():
    """Two consecutive steps of the benchmarked workload at full size (the
    momentum carries over), in the launch configuration bench.py times: no
    U output anywhere, so every final product takes the persistent walk with
    the signs packed from its accumulators. A second state on the same
    gradients stores U for the first layer's four shapes (one tile per
    block). Each step:
      - momentum bit-exact for every matrix and worker;
      - the benchmarked run's packed signs equal the stored-U run's, word
        for word, for every matrix, and W follows from them bit-exactly
        (the oracle's vote of those buffers);
      - for workers 0 and 7 of the first layer, the whole U against the
        oracle's full Newton-Schulz: relative Frobenius error <= 2e-2, and
        the benchmarked run's bits agree with the oracle's signs on >=
        99.9% of the entries with |U| >= 1e-6 max|U| (every residual
        disagreement reported)."""
    wl = synthetic.WORKLOADS["gpt2s_mw8_k1"]
    mw = wl.workers
    idx = list(range(len(wl.shapes)))
    layer0 = (0, 1, 2, 3)
    w_host = [synthetic.initial_weight(wl, j) for j in idx]
    m_host = {j: np.zeros((mw,) + wl.shapes[j], np.uint16) for j in idx}
    bench_mats, stored = gpt2_state(wl), gpt2_state(wl, polar_for=layer0)
    params = sm.Params(workers=mw, beta=wl.beta, eta=wl.eta, ns_iters=wl.ns_iters,
                       mom_dtype=sm.BF16, ns_dtype=sm.BF16)
    ws_b = sm.workspace_tensor(bench_mats, params, DEV)
    ws_s = sm.workspace_tensor(stored, params, DEV)
    for t in range(2):
        gs = list(POOL.map(lambda j: synthetic.gradients(wl, j, t), idx))
        for j in idx:
            bench_mats[j].grad.copy_(torch.from_numpy(gs[j]))
            stored[j].grad.copy_(bench_mats[j].grad)
            oracle.momentum(gs[j], m_host[j], wl.beta)
        # the oracle's whole U of the checked (matrix, worker) pairs, on the
        # host while the GPU runs
        cases = [(j, w) for j in layer0 for w in (0, mw - 1)]
        futs = {c: POOL.submit(lambda jw: oracle.newton_schulz(
            oracle.normalise(m_host[jw[0]][jw[1]])[1], wl.ns_iters, oracle.BF16), c) for c in cases}
        announce(f"  full-size step {t}: launching the benchmarked configuration")
        sm.signmuon_step(bench_mats, params, ws_b)
        announce(f"  full-size step {t}: launching with U stored for layer 0")
        sm.signmuon_step(stored, params, ws_s)
        torch.cuda.synchronize()
        for j in idx:
            np.testing.assert_array_equal(to_host(bench_mats[j].momentum), m_host[j],
                                          err_msg=f"momentum {j} step {t}")
            packed = to_host(bench_mats[j].packed)
            np.testing.assert_array_equal(packed, to_host(stored[j].packed), err_msg=f"packed {j} step {t}")
            oracle.vote_update(packed, w_host[j], wl.eta, want_vote=False)
            np.testing.assert_array_equal(to_host(bench_mats[j].weight), w_host[j], err_msg=f"W {j} step {t}")
            np.testing.assert_array_equal(to_host(stored[j].weight), w_host[j], err_msg=f"W {j} step {t}")
        for (j, w), fut in futs.items():
            u_ref = fut.result()
            u = to_host(stored[j].polar_out[w])
            packed = to_host(bench_mats[j].packed)[w]
            np.testing.assert_array_equal(to_host(stored[j].packed)[w], oracle.sign_pack(u))
            err = rel_fro(u, u_ref)
            agree, bad, cnt = bit_sign_stats(packed, u_ref)
            announce(f"  gpt2 full step {t} matrix {j} {wl.shapes[j]} worker {w}: rel_fro={err:.3e}, "
                     f"benchmarked bits vs oracle signs {agree:.6f} ({bad} of {cnt} differ)")
            assert err <= NS_TOL["bf16"]
            assert agree >= 0.999


@pytest.mark.parametrize("ns", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(768, 3072), (3072, 768), (300, 640), (640, 300), (256, 1024)])
def test_pack_without_polar_out_matches(ns, shape):
    """With polar_out NULL the last product packs signs straight from its
    accumulators; the bits must equal those packed from the stored U (same
    accumulators) and agree with the oracle's signs."""
    R, C = shape
    mw, k = 3, 1
    g = grads(900 + R, mw, R, C, 1e-3)
    params = sm.Params(workers=mw, ns_iters=k, mom_dtype=dtype_of(ns)[2], ns_dtype=dtype_of(ns)[2])
    with_u = make_matrix(g, zeros_m(mw, R, C, ns), np.zeros((R, C), np.float32))
    without_u = make_matrix(g, zeros_m(mw, R, C, ns), np.zeros((R, C), np.float32), polar=False)
    run("signmuon_step", [with_u], params)
    run("signmuon_step", [without_u], params)
    np.testing.assert_array_equal(to_host(without_u.packed), to_host(with_u.packed))
    np.testing.assert_array_equal(to_host(without_u.weight), to_host(with_u.weight))
    m_host = zeros_m(mw, R, C, ns)
    oracle.momentum(g, m_host, 0.9)
    u_ref = oracle_u(m_host, k, ns)
    bits = np.unpackbits(to_host(without_u.packed).view(np.uint8), axis=1, bitorder="little")[:, :R * C]
    for w in range(mw):
        ref = (u_ref[w].ravel() >= 0)
        keep = np.abs(u_ref[w].ravel()) >= 1e-6 * np.abs(u_ref[w]).max()
        agree = np.mean((bits[w].astype(bool) == ref)[keep])
        announce(f"  pack without U {ns} {shape} worker {w}: sign agreement {agree:.6f}")
        assert agree >= 0.999
