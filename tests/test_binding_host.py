"""Host-side checks of the Python binding: every buffer handed to the library
is checked for element type, element count, contiguity and GPU residence
before any call, since the C ABI only sees raw pointers."""
import pytest
import torch

import sign_muon_step_amd as sm


def cpu_matrix(mw=2, R=8, C=96, **over):
    kw = dict(grad=torch.zeros((mw, R, C), dtype=torch.float32),
              momentum=torch.zeros((mw, R, C), dtype=torch.bfloat16),
              packed=torch.zeros((mw, (R * C + 63) // 64), dtype=torch.int64),
              weight=torch.zeros((R, C), dtype=torch.float32),
              vote_out=torch.zeros((R, C), dtype=torch.int8))
    kw.update(over)
    return sm.Matrix(**kw)


P = sm.Params(workers=2, mom_dtype=sm.BF16, ns_dtype=sm.BF16)


def call(m, p=P):
    sm.signmuon_step([m], p, None)


def test_gradient_of_the_wrong_type():
    with pytest.raises(TypeError, match="grad"):
        call(cpu_matrix(grad=torch.zeros((2, 8, 96), dtype=torch.bfloat16)))


def test_momentum_of_the_wrong_type_or_size():
    with pytest.raises(TypeError, match="momentum"):
        call(cpu_matrix(momentum=torch.zeros((2, 8, 96), dtype=torch.float32)))
    with pytest.raises(ValueError, match="momentum"):
        call(cpu_matrix(momentum=torch.zeros((1, 8, 96), dtype=torch.bfloat16)))


def test_packed_weight_vote_and_int8_sizes():
    with pytest.raises(ValueError, match="packed"):
        call(cpu_matrix(packed=torch.zeros((2, 11), dtype=torch.int64)))
    with pytest.raises(ValueError, match="weight"):
        call(cpu_matrix(weight=torch.zeros((8, 95), dtype=torch.float32)))
    with pytest.raises(TypeError, match="vote_out"):
        call(cpu_matrix(vote_out=torch.zeros((8, 96), dtype=torch.uint8)))
    with pytest.raises(ValueError, match="signs_i8"):
        call(cpu_matrix(signs_i8=torch.zeros((1, 8, 96), dtype=torch.int8)))


def test_non_contiguous_buffer():
    w = torch.zeros((96, 8), dtype=torch.float32).t()
    with pytest.raises(ValueError, match="contiguous"):
        call(cpu_matrix(weight=w))


def test_host_memory_is_refused():
    with pytest.raises(ValueError, match="GPU memory"):
        call(cpu_matrix())
    with pytest.raises(ValueError, match="GPU memory"):
        sm.signmuon_sign_pack(torch.zeros(64), 64, 1, torch.zeros(1, dtype=torch.int64))


def test_single_stage_calls_refuse_short_buffers():
    # checked before the library sees a pointer; the buffers are CPU tensors, so
    # a buffer that passes the size check is then refused as host memory
    u = torch.zeros(2 * 100)
    with pytest.raises(ValueError, match="packed"):
        sm.signmuon_sign_pack(u, 100, 2, torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError, match="u:"):
        sm.signmuon_sign_pack(torch.zeros(199), 100, 2, torch.zeros(4, dtype=torch.int64))
    with pytest.raises(ValueError, match="signs"):
        sm.signmuon_sign_int8(u, 100, 2, torch.zeros(199, dtype=torch.int8))
    with pytest.raises(ValueError, match="weight"):
        sm.signmuon_vote_update(torch.zeros(4, dtype=torch.int64), 2, 100, torch.zeros(99), 1e-3)
    with pytest.raises(ValueError, match="vote_out"):
        sm.signmuon_vote_update_int8(torch.zeros(200, dtype=torch.int8), 2, 100, None, 1e-3,
                                     torch.zeros(99, dtype=torch.int8))
    with pytest.raises(TypeError, match="packed"):
        sm.signmuon_vote_update(torch.zeros(4, dtype=torch.int32), 2, 100, None, 1e-3)
    with pytest.raises(ValueError, match="GPU memory"):
        sm.signmuon_sign_pack(u, 100, 2, torch.zeros(4, dtype=torch.int64))

