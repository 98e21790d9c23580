"""GPU tests of the whole step with the int8 payload (signmuon_params.payload
= SIGNMUON_PAYLOAD_INT8): each worker's signs leave the last Newton-Schulz
product (or, for k = 0, the sign kernel) as int8 +1 / -1, and the vote is the
sign of their integer sum over workers.

Bar (bit-exact): on the same inputs, the int8 signs equal 2 * bit - 1 of the
packed path's bits, and the momentum, the vote and W equal the packed path's;
the int8 vote also equals the oracle's vote of the GPU's own signs
(oracle.vote_update_int8), so both sides of the comparison are pinned."""
import numpy as np
import pytest
import torch

import oracle
import sign_muon_step_amd as sm
import synthetic
from gpu_util import DEV, announce, dtype_of, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(f"[gpu-test] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def unpack_signs(packed: np.ndarray, n: int) -> np.ndarray:
    """[Mw][words] uint64 -> [Mw][n] int8 in {-1, +1} (bit j of word w is
    entry 64 w + j)."""
    bits = np.unpackbits(packed.view(np.uint8), axis=-1, bitorder="little")[..., :n]
    return (2 * bits.astype(np.int16) - 1).astype(np.int8)


def build(shapes, mw, ns, seed, int8):
    np_t, torch_t, _ = dtype_of(ns)
    mats = []
    for j, (R, C) in enumerate(shapes):
        g = np.stack([synthetic.random_matrix(seed * 100 + 10 * j + m, (R, C), 1e-3, "normal")
                      for m in range(mw)])
        w = synthetic.random_matrix(seed * 100 + 10 * j + 9, (R, C), 0.02, "normal")
        mats.append(sm.Matrix(
            grad=to_dev(g), momentum=torch.zeros((mw, R, C), dtype=torch_t, device=DEV),
            packed=None if int8 else torch.zeros((mw, sm.signmuon_packed_words(R * C)),
                                                 dtype=torch.int64, device=DEV),
            weight=to_dev(w), vote_out=torch.zeros((R, C), dtype=torch.int8, device=DEV),
            signs_i8=torch.zeros((mw, R, C), dtype=torch.int8, device=DEV) if int8 else None))
    return mats


def step(mats, mw, k, ns, payload, norm=sm.NORM_FROBENIUS, p=0, steps=1):
    code = dtype_of(ns)[2]
    params = sm.Params(workers=mw, beta=0.9, eta=1e-3, ns_iters=k, mom_dtype=code, ns_dtype=code,
                       norm=norm, power_iters=p, payload=payload)
    ws = sm.workspace_tensor(mats, params, DEV)
    for _ in range(steps):
        sm.signmuon_step(mats, params, ws)
    torch.cuda.synchronize()


def compare(shapes, mw, k, ns, seed, norm=sm.NORM_FROBENIUS, p=0, steps=1):
    bits = build(shapes, mw, ns, seed, False)
    ints = build(shapes, mw, ns, seed, True)
    step(bits, mw, k, ns, sm.PAYLOAD_BITS, norm, p, steps)
    step(ints, mw, k, ns, sm.PAYLOAD_INT8, norm, p, steps)
    for (R, C), a, b in zip(shapes, bits, ints):
        n = R * C
        signs = to_host(b.signs_i8).reshape(mw, n)
        np.testing.assert_array_equal(signs, unpack_signs(to_host(a.packed), n))
        np.testing.assert_array_equal(to_host(b.momentum), to_host(a.momentum))
        np.testing.assert_array_equal(to_host(b.vote_out), to_host(a.vote_out))
        np.testing.assert_array_equal(to_host(b.weight), to_host(a.weight))
    return bits, ints


SHAPES = [(96, 200), (200, 96), (130, 70), (64, 576), (257, 129), (33, 7), (1, 9)]


@pytest.mark.parametrize("ns", ["f32", "bf16"])
@pytest.mark.parametrize("k", [0, 1, 2])
@pytest.mark.parametrize("mw", [1, 3, 8])
def test_int8_payload_step_equals_packed_step(ns, k, mw):
    compare(SHAPES, mw, k, ns, seed=5 + k + mw)


def test_int8_payload_vote_is_the_oracle_vote_of_the_gpu_signs():
    shapes, mw = [(128, 320), (100, 36)], 5
    ints = build(shapes, mw, "bf16", 7, True)
    w0 = [to_host(m.weight).copy() for m in ints]
    step(ints, mw, 1, "bf16", sm.PAYLOAD_INT8)
    for (R, C), m, w in zip(shapes, ints, w0):
        signs = to_host(m.signs_i8).reshape(mw, R * C)
        w_ref = w.ravel().copy()
        vote = oracle.vote_update_int8(signs, w_ref, 1e-3)
        np.testing.assert_array_equal(to_host(m.vote_out).ravel(), vote)
        np.testing.assert_array_equal(to_host(m.weight).ravel(), w_ref)


def test_int8_payload_two_steps_and_spectral():
    compare([(192, 320), (320, 192)], 4, 1, "bf16", seed=11, steps=2)
    compare([(192, 320), (70, 130)], 3, 2, "f32", seed=12, norm=sm.NORM_SPECTRAL, p=3)


def test_int8_payload_more_matrices_than_one_launch_takes():
    shapes = [(16 + 8 * (j % 5), 24 + 16 * (j % 3)) for j in range(53)]
    compare(shapes, 3, 1, "bf16", seed=13)


def test_int8_payload_gpt2_layer_full_size():
    """One GPT-2 small layer's four matrices, 8 workers, in the launch
    configuration the benchmark times."""
    compare([(768, 2304), (768, 768), (768, 3072), (3072, 768)], 8, 1, "bf16", seed=17)
