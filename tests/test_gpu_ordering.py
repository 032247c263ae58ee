"""Bit-exact ordering checks of the state API on the GPU.

Frame-level access and the clean-pass update ("Attend Locally, Remember
Linearly" technical summary, §2.2) as byte-level properties of the HIP path:
  G1 reads never change S;
  G2 a commit with alpha = 1, beta = 0 leaves S unchanged;
  G3 S_n does not depend on how many denoising reads preceded the clean pass;
  G4 two identical rollouts give identical bytes (no atomics, fixed order);
  G5 identical query rows give identical O_inter rows;
  G6 saving S at frame k and restoring it continues bit-identically.
"""
import numpy as np
import pytest

from gpu_helpers import dev, dev32, log, shape_of
from hybrid_linear_memory_amd import synth

pytestmark = pytest.mark.gpu

CASES = [synth.WORKLOADS[0], synth.WORKLOADS[1].replace(T=400, H=3, frames=4)]


def _ids(w):
    return f"{w.dtype}-H{w.H}T{w.T}D{w.D}"


def _bytes(t):
    import torch
    return t.detach().contiguous().cpu().view(-1).view(torch.uint8).numpy().copy()


def _layer(w):
    from hybrid_linear_memory_amd.layer import Arl2Layer
    return Arl2Layer(shape_of(w), *[dev(p, w.dtype) for p in synth.phi_maps(w)])


def _frame(w, f, p):
    q, k, v = synth.qkv(w, f, p)
    return dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype)


def _gates(w, f, alpha=None, beta=None):
    b, a = synth.gates(w, f)
    if alpha is not None:
        a = np.full_like(a, alpha)
    if beta is not None:
        b = np.full_like(b, beta)
    return dev32(b), dev32(a)


def _warm_state(layer, w, n=2):
    for f in range(n):
        layer.clean_pass(*_frame(w, f, w.passes - 1), *_gates(w, f))


@pytest.mark.parametrize("w", CASES, ids=_ids)
def test_g1_reads_never_write_state(w):
    import torch
    log(f"G1 {_ids(w)}")
    layer = _layer(w)
    _warm_state(layer, w)
    before = _bytes(layer.S)
    other = _bytes(layer._S[1 - layer._cur])
    for p in range(6):
        layer.read(*_frame(w, 5, p))
    torch.cuda.synchronize()
    assert np.array_equal(_bytes(layer.S), before)
    assert np.array_equal(_bytes(layer._S[1 - layer._cur]), other)


@pytest.mark.parametrize("w", CASES, ids=_ids)
def test_g2_identity_commit(w):
    log(f"G2 {_ids(w)}")
    layer = _layer(w)
    _warm_state(layer, w)
    before = _bytes(layer.S)
    layer.clean_pass(*_frame(w, 7, 0), *_gates(w, 7, alpha=1.0, beta=0.0))
    assert np.array_equal(_bytes(layer.S), before)


@pytest.mark.parametrize("w", CASES, ids=_ids)
def test_g3_state_independent_of_read_count(w):
    log(f"G3 {_ids(w)}")
    finals = []
    for n_reads in (0, 1, 4):
        layer = _layer(w)
        for f in range(3):
            for p in range(n_reads):
                layer.read(*_frame(w, f, p))
            layer.clean_pass(*_frame(w, f, w.passes - 1), *_gates(w, f))
        finals.append(_bytes(layer.S))
    assert np.array_equal(finals[0], finals[1])
    assert np.array_equal(finals[0], finals[2])


@pytest.mark.parametrize("w", CASES, ids=_ids)
def test_g4_deterministic(w):
    log(f"G4 {_ids(w)}")
    runs = []
    for _ in range(2):
        layer = _layer(w)
        outs = []
        for f in range(3):
            outs.append(_bytes(layer.read(*_frame(w, f, 0))))
            outs.append(_bytes(layer.clean_pass(*_frame(w, f, w.passes - 1), *_gates(w, f))))
        runs.append((outs, _bytes(layer.S)))
    for a, b in zip(runs[0][0], runs[1][0]):
        assert np.array_equal(a, b)
    assert np.array_equal(runs[0][1], runs[1][1])


@pytest.mark.parametrize("w", CASES, ids=_ids)
def test_g5_identical_rows_identical_inter_read(w):
    log(f"G5 {_ids(w)}")
    layer = _layer(w)
    _warm_state(layer, w)
    q, k, v = synth.qkv(w, 9, 0)
    T = w.T
    pairs = [(0, T - 1), (1, T // 2), (3, 35), (T // 3, min(T - 2, T // 3 + 64))]
    for a, b in pairs:
        q[:, :, b] = q[:, :, a]
    o_e = layer.new_output()
    o_i = layer.new_output()
    layer.read(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), o_intra=o_i, o_inter=o_e)
    oe = o_e.float().cpu().numpy()
    for a, b in pairs:
        assert np.array_equal(oe[:, :, a], oe[:, :, b]), (a, b)


@pytest.mark.parametrize("w", CASES, ids=_ids)
def test_g6_checkpoint_resume(w):
    log(f"G6 {_ids(w)}")
    full = _layer(w)
    for f in range(w.frames):
        full.clean_pass(*_frame(w, f, w.passes - 1), *_gates(w, f))
        if f == 1:
            sd = full.state_dict()
    resumed = _layer(w)
    resumed.load_state_dict(sd)
    assert resumed.frame == 2
    for f in range(2, w.frames):
        resumed.clean_pass(*_frame(w, f, w.passes - 1), *_gates(w, f))
    assert np.array_equal(_bytes(resumed.S), _bytes(full.S))


@pytest.mark.parametrize("w", CASES, ids=_ids)
def test_debug_check_refuses_non_finite_inputs(w):
    """With check_finite, a NaN or an infinity in any input of a pass raises
    before anything is launched: the state bytes, the frame index and the
    pass count stay as they were, and the next good pass runs normally."""
    import torch
    from hybrid_linear_memory_amd.layer import Arl2Layer, NonFiniteInput
    log(f"debug finiteness check {_ids(w)}")
    layer = Arl2Layer(shape_of(w), *[dev(p, w.dtype) for p in synth.phi_maps(w)],
                      check_finite=True)
    _warm_state(layer, w)
    torch.cuda.synchronize()
    before = _bytes(layer.S)
    frame, reads = layer.frame, layer.seq.reads
    q, k, v = _frame(w, 5, 0)
    beta, alpha = _gates(w, 5)
    bad_q = q.clone()
    bad_q[0, 0, 3, 1] = float("nan")
    with pytest.raises(NonFiniteInput, match="q"):
        layer.read(bad_q, k, v)
    bad_alpha = alpha.clone()
    bad_alpha[0, 0] = float("inf")
    with pytest.raises(NonFiniteInput, match="alpha"):
        layer.clean_pass(q, k, v, beta, bad_alpha)
    bad_v = v.clone()
    bad_v[0, -1, -1, -1] = float("-inf")
    with pytest.raises(NonFiniteInput, match="v"):
        layer.commit(k, bad_v, beta, alpha)
    torch.cuda.synchronize()
    assert np.array_equal(_bytes(layer.S), before)
    assert (layer.frame, layer.seq.reads) == (frame, reads)
    layer.read(q, k, v)
    layer.clean_pass(q, k, v, beta, alpha)
    assert layer.frame == frame + 1
