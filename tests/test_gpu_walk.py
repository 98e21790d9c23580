"""The final product's persistent tile walk (bf16, signs packed from the
accumulators, no U output): one workgroup per CU walks several tiles, and the
loads of each tile's last iterations fetch the next tile's first slices.

Its packed bits must equal, bit for bit, those of the one-tile-per-block
kernel that also stores U (same operands, same k order, same accumulators),
for batches with several tiles per workgroup: wide and tall matrices (two
launches), ragged tiles (R or C not a multiple of 256), the shortest k loop
the walk accepts (min(R, C) = 384: 12 slices of 32), and matrices the walk
does not take in the same call. The vote and W follow from the bits and must
match too; U itself is checked against the oracle's whole Newton-Schulz
result, and the walk's bits against the oracle's signs (entries with
|U| >= 1e-6 max|U|)."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import sign_muon_step_amd as sm
import synthetic
from gpu_util import DEV, announce, bit_sign_stats, rel_fro, to_dev, to_host

pytestmark = pytest.mark.gpu

POOL = ThreadPoolExecutor(max_workers=8)

# walk-eligible (C % 64 == 0, min(R, C) % 8 == 0, ceil(min(R, C) / 32) a
# multiple of 4 and >= 12), wide and tall, ragged and regular
WALK = [(640, 1216), (1216, 640), (384, 1024), (1024, 384), (768, 3072), (3072, 768), (768, 768)]
# not walk-eligible: k loop too short (r = 256), r % 32 leaves a slice count
# that is not a multiple of 4 (r = 520), C % 64 != 0 (no fused pack at all)
PLAIN = [(256, 1024), (520, 1088), (300, 640)]


@pytest.fixture(autouse=True)
def _name_the_case(request):
    announce(f"[gpu-test] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def build(shapes, mw, seed, polar, int8=False):
    def grad(jm):
        j, m = jm
        return synthetic.random_matrix(seed + 100 * j + m, shapes[j], 1e-3)

    mats, host = [], []
    for j, (R, C) in enumerate(shapes):
        g = np.stack(list(POOL.map(grad, [(j, m) for m in range(mw)])))
        w0 = synthetic.random_matrix(seed + 100 * j + 99, (R, C), 0.02)
        host.append((g, w0))
        mats.append(sm.Matrix(
            grad=to_dev(g), momentum=torch.zeros((mw, R, C), dtype=torch.bfloat16, device=DEV),
            packed=None if int8 else torch.zeros((mw, sm.signmuon_packed_words(R * C)), dtype=torch.int64,
                                                 device=DEV),
            weight=to_dev(w0),
            polar_out=torch.zeros((mw, R, C), dtype=torch.float32, device=DEV) if polar else None,
            vote_out=torch.zeros((R, C), dtype=torch.int8, device=DEV),
            signs_i8=torch.zeros((mw, R, C), dtype=torch.int8, device=DEV) if int8 else None))
    return mats, host


@pytest.mark.parametrize("mw,k", [(16, 1), (5, 1), (5, 2)])
def test_walk_bits_equal_stored_u_bits(mw, k):
    shapes = WALK + PLAIN
    p = sm.Params(workers=mw, beta=0.9, eta=1e-3, ns_iters=k, mom_dtype=sm.BF16, ns_dtype=sm.BF16)
    walk, host = build(shapes, mw, 7000, polar=False)
    ref, _ = build(shapes, mw, 7000, polar=True)
    announce(f"  {mw} workers, {len(shapes)} matrices, k = {k}: walk run")
    sm.signmuon_step(walk, p, sm.workspace_tensor(walk, p, DEV))
    announce("  reference run (U stored: one tile per block)")
    sm.signmuon_step(ref, p, sm.workspace_tensor(ref, p, DEV))
    torch.cuda.synchronize()
    for j, (a, b) in enumerate(zip(walk, ref)):
        np.testing.assert_array_equal(to_host(a.momentum), to_host(b.momentum), err_msg=f"M {shapes[j]}")
        pw, pr = to_host(a.packed), to_host(b.packed)
        np.testing.assert_array_equal(pw, pr, err_msg=f"packed {shapes[j]}")
        np.testing.assert_array_equal(to_host(a.vote_out), to_host(b.vote_out), err_msg=f"vote {shapes[j]}")
        np.testing.assert_array_equal(to_host(a.weight), to_host(b.weight), err_msg=f"W {shapes[j]}")
    # the stored U (reference run) of workers 0 and mw - 1 against the
    # oracle's whole Newton-Schulz result, and the walk's bits against the
    # oracle's signs (the acceptance rule: |U| >= 1e-6 max|U|)
    cases = [(j, w) for j in range(len(shapes)) for w in (0, mw - 1)]

    def oracle_u(jw):
        j, w = jw
        m_ref = np.zeros(shapes[j], np.uint16)
        oracle.momentum(host[j][0][w], m_ref, 0.9)
        return oracle.newton_schulz(oracle.normalise(m_ref)[1], k, oracle.BF16)

    for (j, w), u_ref in zip(cases, POOL.map(oracle_u, cases)):
        u = to_host(ref[j].polar_out)[w]
        err = rel_fro(u, u_ref)
        agree, bad, cnt = bit_sign_stats(to_host(walk[j].packed)[w], u_ref)
        announce(f"  {shapes[j]} worker {w}: rel_fro {err:.2e}, walk bits vs oracle signs "
                 f"{agree:.6f} ({bad} of {cnt} differ)")
        assert err <= 2e-2
        assert agree >= 0.999


@pytest.mark.parametrize("mw,k,plain", [(16, 1, 2), (5, 2, 3)])
def test_walk_bits_equal_stored_u_bits_spectral(mw, k, plain):
    """Spectral scaling (8 power steps). The Gram matrix stays unscaled and the
    first product takes the identity coefficient -3 / s^2 and multiplies its
    accumulators by s^2: in the walk a compile-time flag, in the one-tile-per-
    block product (the stored-U run) a run-time one, with the same MFMAs in
    the same order, so the packed bits, the vote and W must be equal. 16
    workers with r % 8 == 0 throughout run the one-launch power iteration;
    5 workers with a 300-row matrix run the per-step launches, and k = 2 adds
    an intermediate walk product (the next iterate) under the flag. U of
    workers 0 and mw - 1 against the oracle's spectral Newton-Schulz, and the
    walk's bits against the oracle's signs."""
    shapes = WALK + PLAIN[:plain]
    power = 8
    p = sm.Params(workers=mw, beta=0.9, eta=1e-3, ns_iters=k, mom_dtype=sm.BF16, ns_dtype=sm.BF16,
                  norm=sm.NORM_SPECTRAL, power_iters=power)
    walk, host = build(shapes, mw, 7300, polar=False)
    ref, _ = build(shapes, mw, 7300, polar=True)
    announce(f"  {mw} workers, {len(shapes)} matrices, k = {k}, spectral: walk run")
    sm.signmuon_step(walk, p, sm.workspace_tensor(walk, p, DEV))
    announce("  reference run (U stored: one tile per block)")
    sm.signmuon_step(ref, p, sm.workspace_tensor(ref, p, DEV))
    torch.cuda.synchronize()
    for j, (a, b) in enumerate(zip(walk, ref)):
        np.testing.assert_array_equal(to_host(a.momentum), to_host(b.momentum), err_msg=f"M {shapes[j]}")
        np.testing.assert_array_equal(to_host(a.packed), to_host(b.packed), err_msg=f"packed {shapes[j]}")
        np.testing.assert_array_equal(to_host(a.vote_out), to_host(b.vote_out), err_msg=f"vote {shapes[j]}")
        np.testing.assert_array_equal(to_host(a.weight), to_host(b.weight), err_msg=f"W {shapes[j]}")
    cases = [(j, w) for j in range(len(shapes)) for w in (0, mw - 1)]

    def oracle_u(jw):
        j, w = jw
        m_ref = np.zeros(shapes[j], np.uint16)
        oracle.momentum(host[j][0][w], m_ref, 0.9)
        _, x0, a0 = oracle.spectral_x0_a0(m_ref, oracle.BF16, power)
        return oracle.newton_schulz_a0(x0, a0, k, oracle.BF16)

    for (j, w), u_ref in zip(cases, POOL.map(oracle_u, cases)):
        u = to_host(ref[j].polar_out)[w]
        err = rel_fro(u, u_ref)
        agree, bad, cnt = bit_sign_stats(to_host(walk[j].packed)[w], u_ref)
        announce(f"  {shapes[j]} worker {w}: rel_fro {err:.2e}, walk bits vs oracle signs "
                 f"{agree:.6f} ({bad} of {cnt} differ)")
        assert err <= 2e-2
        assert agree >= 0.999


def test_walk_on_gpt2_small_matches_plain_kernel_over_two_steps():
    """The benchmarked batch itself (48 GPT-2 small matrices, 8 workers): two
    steps, every packed word, the vote and W equal to the stored-U run's."""
    wl = synthetic.WORKLOADS["gpt2s_mw8_k1"]
    mw = wl.workers
    p = sm.Params(workers=mw, beta=wl.beta, eta=wl.eta, ns_iters=1, mom_dtype=sm.BF16, ns_dtype=sm.BF16)

    def state(polar):
        return [sm.Matrix(
            grad=torch.empty((mw, R, C), dtype=torch.float32, device=DEV),
            momentum=torch.zeros((mw, R, C), dtype=torch.bfloat16, device=DEV),
            packed=torch.zeros((mw, sm.signmuon_packed_words(R * C)), dtype=torch.int64, device=DEV),
            weight=to_dev(synthetic.initial_weight(wl, j)),
            polar_out=torch.zeros((mw, R, C), dtype=torch.float32, device=DEV) if polar else None,
            vote_out=torch.zeros((R, C), dtype=torch.int8, device=DEV)) for j, (R, C) in enumerate(wl.shapes)]

    walk, ref = state(False), state(True)
    ws_w, ws_r = sm.workspace_tensor(walk, p, DEV), sm.workspace_tensor(ref, p, DEV)
    for t in range(2):
        for j in range(len(wl.shapes)):
            g = torch.from_numpy(synthetic.gradients(wl, j, t)).to(DEV)
            walk[j].grad.copy_(g)
            ref[j].grad.copy_(g)
        announce(f"  step {t}")
        sm.signmuon_step(walk, p, ws_w)
        sm.signmuon_step(ref, p, ws_r)
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(walk, ref)):
            np.testing.assert_array_equal(to_host(a.packed), to_host(b.packed), err_msg=f"packed {j} t {t}")
            np.testing.assert_array_equal(to_host(a.vote_out), to_host(b.vote_out), err_msg=f"vote {j} t {t}")
            np.testing.assert_array_equal(to_host(a.weight), to_host(b.weight), err_msg=f"W {j} t {t}")


def test_walk_with_more_matrices_than_one_launch_holds():
    """60 walk-eligible matrices (wide and tall): each group splits into
    launches of at most 48 matrices; bits, vote and W as with stored U."""
    shapes = [(384, 1024), (1024, 384), (640, 704)] * 20
    mw = 2
    p = sm.Params(workers=mw, beta=0.9, eta=1e-3, ns_iters=1, mom_dtype=sm.BF16, ns_dtype=sm.BF16)
    walk, _ = build(shapes, mw, 8100, polar=False)
    ref, _ = build(shapes, mw, 8100, polar=True)
    sm.signmuon_step(walk, p, sm.workspace_tensor(walk, p, DEV))
    sm.signmuon_step(ref, p, sm.workspace_tensor(ref, p, DEV))
    torch.cuda.synchronize()
    for j, (a, b) in enumerate(zip(walk, ref)):
        np.testing.assert_array_equal(to_host(a.packed), to_host(b.packed), err_msg=f"packed {j} {shapes[j]}")
        np.testing.assert_array_equal(to_host(a.weight), to_host(b.weight), err_msg=f"W {j} {shapes[j]}")


@pytest.mark.parametrize("mw,k,spectral", [(16, 1, False), (3, 2, False), (16, 1, True)])
def test_walk_int8_signs_equal_stored_u_int8_signs(mw, k, spectral):
    """The int8 payload: the walk expands each sign word into 64 bytes of
    +1 / -1; they must equal the int8 signs of the one-tile-per-block kernel
    that also stores U, and 2 bit - 1 of the oracle's signs where clear. Also
    under spectral scaling (the first product with the unscaled Gram matrix)."""
    shapes = WALK + PLAIN
    p = sm.Params(workers=mw, beta=0.9, eta=1e-3, ns_iters=k, mom_dtype=sm.BF16, ns_dtype=sm.BF16,
                  payload=sm.PAYLOAD_INT8, norm=sm.NORM_SPECTRAL if spectral else sm.NORM_FROBENIUS,
                  power_iters=6 if spectral else 0)
    walk, host = build(shapes, mw, 9100, polar=False, int8=True)
    ref, _ = build(shapes, mw, 9100, polar=True, int8=True)
    announce(f"  int8, {mw} workers, k = {k}: walk run, then stored-U run")
    sm.signmuon_step(walk, p, sm.workspace_tensor(walk, p, DEV))
    sm.signmuon_step(ref, p, sm.workspace_tensor(ref, p, DEV))
    torch.cuda.synchronize()
    for j, (a, b) in enumerate(zip(walk, ref)):
        sw = to_host(a.signs_i8)
        np.testing.assert_array_equal(sw, to_host(b.signs_i8), err_msg=f"int8 signs {shapes[j]}")
        assert set(np.unique(sw).tolist()) <= {-1, 1}
        np.testing.assert_array_equal(to_host(a.vote_out), to_host(b.vote_out), err_msg=f"vote {shapes[j]}")
        np.testing.assert_array_equal(to_host(a.weight), to_host(b.weight), err_msg=f"W {shapes[j]}")
        # U of the stored-U run decides the sign of every int8 entry
        u = to_host(b.polar_out)
        np.testing.assert_array_equal(sw, np.where(u >= 0, 1, -1).astype(np.int8), err_msg=f"rule {shapes[j]}")


@pytest.mark.parametrize("spectral", [False, True])
def test_walk_degenerate_workers_match_oracle(spectral):
    """Workers whose gradient is zero (U = 0: every sign +1), holds a NaN (U
    is NaN: every sign -1) or an Inf (s = 0, and 0 * Inf is NaN: every sign
    -1), next to ordinary workers, through the walk: every packed word of
    the degenerate workers equals the oracle's, and the whole output equals
    the stored-U kernel's. Under spectral scaling lambda is 0 or not finite
    for them, so s = s^2 = 0 and the first product's identity coefficient is
    -3."""
    shapes = [(384, 1024), (1024, 384), (768, 768)]
    mw = 3
    norm = sm.NORM_SPECTRAL if spectral else sm.NORM_FROBENIUS
    power = 5 if spectral else 0
    p = sm.Params(workers=mw, beta=0.9, eta=1e-3, ns_iters=1, mom_dtype=sm.BF16, ns_dtype=sm.BF16,
                  norm=norm, power_iters=power)
    bad = {0: (0, "zero"), 1: (1, "nan"), 2: (2, "inf")}  # matrix -> (worker, kind)
    runs = []
    for polar in (False, True):
        mats, host = build(shapes, mw, 9500, polar=polar)
        for j, (w, kind) in bad.items():
            g = host[j][0]
            if kind == "zero":
                g[w] = 0.0
            else:
                g[w].ravel()[12345 % g[w].size] = np.nan if kind == "nan" else np.inf
            mats[j].grad.copy_(torch.from_numpy(g))
        sm.signmuon_step(mats, p, sm.workspace_tensor(mats, p, DEV))
        torch.cuda.synchronize()
        runs.append((mats, host))
    (walk, host), (ref, _) = runs
    for j, (w, kind) in bad.items():
        R, C = shapes[j]
        pw = to_host(walk[j].packed)
        np.testing.assert_array_equal(pw, to_host(ref[j].packed), err_msg=f"packed {shapes[j]}")
        np.testing.assert_array_equal(to_host(walk[j].weight), to_host(ref[j].weight), err_msg=f"W {shapes[j]}")
        m = np.zeros((mw, R, C), np.uint16)
        w0 = host[j][1].copy()
        packed_ref, _, _ = oracle.step_matrix(host[j][0], m, w0, 0.9, 1e-3, 1, oracle.BF16,
                                              norm=oracle.NORM_SPECTRAL if spectral else oracle.NORM_FROB,
                                              power_iters=power)
        announce(f"  {shapes[j]} worker {w} ({kind}): GPU words {np.unique(pw[w])[:3]}, "
                 f"oracle words {np.unique(packed_ref[w])[:3]}")
        np.testing.assert_array_equal(pw[w], packed_ref[w], err_msg=f"{kind} worker")
        want = np.uint64(0xFFFFFFFFFFFFFFFF) if kind == "zero" else np.uint64(0)
        assert (pw[w] == want).all()


def test_walk_iterates_do_not_depend_on_the_batch():
    """k = 3: the intermediate products write the next iterate from the walk
    (staged through LDS beside the stage buffers). A matrix's U must be the
    same bit for bit alone (one tile per workgroup) and among 40 others
    (several tiles per workgroup, wide and tall launches), and within the
    Newton-Schulz tolerance of the oracle's."""
    mw, k = 4, 3
    target = (768, 1024)
    others = [(640, 1216), (1216, 640), (384, 1024), (1024, 384)] * 10
    p = sm.Params(workers=mw, beta=0.9, eta=1e-3, ns_iters=k, mom_dtype=sm.BF16, ns_dtype=sm.BF16)
    alone, host = build([target], mw, 9700, polar=True)
    sm.signmuon_step(alone, p, sm.workspace_tensor(alone, p, DEV))
    batch, _ = build([target] + others, mw, 9700, polar=True)  # same seeds for the target
    announce(f"  target alone, then among {len(others)} others")
    sm.signmuon_step(batch, p, sm.workspace_tensor(batch, p, DEV))
    torch.cuda.synchronize()
    u = to_host(alone[0].polar_out)
    np.testing.assert_array_equal(u, to_host(batch[0].polar_out))
    np.testing.assert_array_equal(to_host(alone[0].packed), to_host(batch[0].packed))
    m_ref = np.zeros((mw,) + target, np.uint16)
    oracle.momentum(host[0][0], m_ref, 0.9)
    _, x0 = oracle.normalise(m_ref[1])
    u_ref = oracle.newton_schulz(x0, k, oracle.BF16)
    err = np.linalg.norm(u[1] - u_ref) / np.linalg.norm(u_ref)
    announce(f"  {target} worker 1, k = {k}: rel err {err:.2e}")
    assert err <= 2e-2
