"""GPU parity of the int8 payload (signmuon_sign_int8, signmuon_vote_update_int8)
against the CPU oracle, and its equality with the packed-bit vote.

Bar: bit-exact (signs, vote, W bits)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import sign_muon_step_amd as sm
import synthetic
from gpu_util import DEV, announce, make_matrix, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(f"[gpu-test] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def special_u(rng, shape):
    u = rng.standard_normal(shape).astype(np.float32)
    flat = u.ravel()
    flat[rng.integers(0, u.size, max(1, u.size // 50))] = 0.0
    flat[rng.integers(0, u.size, max(1, u.size // 50))] = -0.0
    flat[rng.integers(0, u.size, max(1, u.size // 97))] = np.nan
    return u


@pytest.mark.parametrize("udt", ["f32", "bf16"])
@pytest.mark.parametrize("n,workers", [(1, 1), (15, 2), (16, 1), (17, 3), (4097, 2), (100003, 5),
                                       (4096 * 33 + 16, 4)])
def test_sign_int8_bitexact(udt, n, workers):
    rng = np.random.default_rng(n + workers)
    u = special_u(rng, (workers, n))
    if udt == "bf16":
        u = oracle.bf16_from_f32(u)
    signs = torch.zeros((workers, n), dtype=torch.int8, device=DEV)
    sm.signmuon_sign_int8(to_dev(u), n, workers, signs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(signs), oracle.sign_int8(u))


@pytest.mark.parametrize("values", ["pm1", "any"])
@pytest.mark.parametrize("mw", [1, 2, 3, 4, 5, 8, 10, 16, 17, 255])
@pytest.mark.parametrize("n", [1, 100, 4096, 4096 * 4 + 37, 65536 + 16])
def test_vote_update_int8_bitexact(values, mw, n):
    rng = np.random.default_rng(mw * 13 + n)
    if values == "pm1":
        signs = (2 * rng.integers(0, 2, (mw, n)) - 1).astype(np.int8)
    else:
        signs = rng.integers(-128, 128, (mw, n)).astype(np.int8)
        signs[:, :3] = 0
    w0 = rng.standard_normal(n).astype(np.float32) * np.float32(0.02)
    eta = 1e-3
    w_dev = to_dev(w0)
    vote_dev = torch.zeros(n, dtype=torch.int8, device=DEV)
    sm.signmuon_vote_update_int8(to_dev(signs), mw, n, w_dev, eta, vote_dev)
    torch.cuda.synchronize()
    w_ref = w0.copy()
    vote_ref = oracle.vote_update_int8(signs, w_ref, eta)
    np.testing.assert_array_equal(to_host(vote_dev), vote_ref)
    np.testing.assert_array_equal(to_host(w_dev).view(np.uint32), w_ref.view(np.uint32))


def test_vote_update_int8_vote_only_and_update_only():
    rng = np.random.default_rng(8)
    mw, n = 6, 5008
    signs = (2 * rng.integers(0, 2, (mw, n)) - 1).astype(np.int8)
    w0 = rng.standard_normal(n).astype(np.float32)
    w_ref = w0.copy()
    vote_ref = oracle.vote_update_int8(signs, w_ref, 0.5)
    vote_dev = torch.zeros(n, dtype=torch.int8, device=DEV)
    sm.signmuon_vote_update_int8(to_dev(signs), mw, n, None, 0.5, vote_dev)
    w_dev = to_dev(w0)
    sm.signmuon_vote_update_int8(to_dev(signs), mw, n, w_dev, 0.5, None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(vote_dev), vote_ref)
    np.testing.assert_array_equal(to_host(w_dev), w_ref)


def test_int8_vote_worked_example_from_pages(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "vote_worked_example.json")))
    for case in spec["cases"]:
        mw, plus = case["workers"], case["plus_votes"]
        signs = -np.ones((mw, 1), np.int8)
        signs[:plus, 0] = 1
        w = to_dev(np.zeros(1, np.float32))
        vote = torch.zeros(1, dtype=torch.int8, device=DEV)
        sm.signmuon_vote_update_int8(to_dev(signs), mw, 1, w, 1.0, vote)
        torch.cuda.synchronize()
        assert int(to_host(vote)[0]) == case["expected_vote"]


@pytest.mark.parametrize("mw", [3, 8, 16])
@pytest.mark.parametrize("n", [1000, 4096 * 3])
def test_int8_vote_equals_packed_vote_on_gpu(mw, n):
    """The same U through both payloads gives the same vote and W bits."""
    rng = np.random.default_rng(mw + n)
    u = to_dev(special_u(rng, (mw, n)))
    packed = torch.zeros((mw, sm.signmuon_packed_words(n)), dtype=torch.int64, device=DEV)
    signs = torch.zeros((mw, n), dtype=torch.int8, device=DEV)
    sm.signmuon_sign_pack(u, n, mw, packed)
    sm.signmuon_sign_int8(u, n, mw, signs)
    w0 = rng.standard_normal(n).astype(np.float32)
    w_a, w_b = to_dev(w0), to_dev(w0)
    v_a = torch.zeros(n, dtype=torch.int8, device=DEV)
    v_b = torch.zeros(n, dtype=torch.int8, device=DEV)
    sm.signmuon_vote_update(packed, mw, n, w_a, 1e-3, v_a)
    sm.signmuon_vote_update_int8(signs, mw, n, w_b, 1e-3, v_b)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(v_a), to_host(v_b))
    np.testing.assert_array_equal(to_host(w_a).view(np.uint32), to_host(w_b).view(np.uint32))


def test_int8_gpt2_layer_full_size():
    """One GPT-2 small layer at full size with 8 workers (the benchmarked
    configuration): the step's fused packed vote equals the int8 vote of its
    own U, and the int8 vote of every matrix equals the oracle's."""
    wl = synthetic.WORKLOADS["gpt2s_mw8_k1"]
    mats, ws = [], []
    for j in range(4):
        R, C = wl.shapes[j]
        g = synthetic.gradients(wl, j, 0)
        m = np.zeros((wl.workers, R, C), np.uint16)
        w = synthetic.initial_weight(wl, j)
        mats.append(make_matrix(g, m, w))
        ws.append(w)
    p = sm.Params(workers=wl.workers, beta=wl.beta, eta=wl.eta, ns_iters=1, mom_dtype=sm.BF16,
                  ns_dtype=sm.BF16)
    space = sm.workspace_tensor(mats, p, DEV)
    sm.signmuon_step(mats, p, space)
    torch.cuda.synchronize()
    for j, mat in enumerate(mats):
        R, C = wl.shapes[j]
        n = R * C
        signs = torch.zeros((wl.workers, n), dtype=torch.int8, device=DEV)
        sm.signmuon_sign_int8(mat.polar_out, n, wl.workers, signs)
        w_dev = to_dev(ws[j].ravel())
        vote = torch.zeros(n, dtype=torch.int8, device=DEV)
        sm.signmuon_vote_update_int8(signs, wl.workers, n, w_dev, wl.eta, vote)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(vote).reshape(R, C), to_host(mat.vote_out))
        np.testing.assert_array_equal(to_host(w_dev).reshape(R, C), to_host(mat.weight))
        w_ref = ws[j].ravel().copy()
        vote_ref = oracle.vote_update_int8(to_host(signs), w_ref, wl.eta)
        np.testing.assert_array_equal(to_host(vote), vote_ref)
        np.testing.assert_array_equal(to_host(w_dev), w_ref)
