"""Parity of the HIP path (through the C-ABI) with the fp64 oracle.

Tolerance: max |gpu - oracle| <= 1e-4 * max|oracle| for float32 workloads and
<= 2e-2 * max|oracle| for bf16 workloads, per tensor (each output of each
compared pass, the state after every commit). Inputs come from the seeded
generator, identical on both sides (bf16 values upcast exactly by the oracle).
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import (TOL, assert_close, dev, dev32, host, lockstep_rollout, log,
                         shape_of)
from hybrid_linear_memory_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import hybrid_linear_memory_amd.arl2  # noqa: F401  (fails loudly if not built)


def _w(dtype, B, H, T, D, frames=2, n_denoise=1):
    base = synth.WORKLOADS[0] if dtype == "f32" else synth.WORKLOADS[1]
    return base.replace(B=B, H=H, T=T, D=D, frames=frames, n_denoise=n_denoise)


STEP_CASES = [
    ("f32", 1, 1, 64, 16), ("f32", 2, 3, 100, 32), ("f32", 1, 2, 37, 64), ("f32", 1, 2, 130, 128),
    ("f32", 1, 1, 1, 16),
    ("bf16", 1, 2, 200, 128), ("bf16", 2, 3, 1, 128), ("bf16", 1, 1, 37, 128),
    ("bf16", 1, 2, 100, 128), ("bf16", 1, 2, 150, 128),
    ("bf16", 1, 2, 513, 128), ("bf16", 1, 12, 1560, 128),
    ("bf16", 1, 2, 200, 64), ("bf16", 2, 1, 77, 16), ("bf16", 1, 3, 1560, 64),
    ("bf16", 1, 1, 1, 16),
]


def _ids(c):
    return "{}-B{}H{}T{}D{}".format(*c)


@pytest.mark.parametrize("case", STEP_CASES, ids=_ids)
@pytest.mark.parametrize("normalize", [False, True])
def test_feature_map(case, normalize):
    from hybrid_linear_memory_amd import arl2
    w = _w(*case)
    log(f"feature_map {_ids(case)} normalize={normalize}")
    x, _, _ = synth.qkv(w, 0, 0)
    phi = synth.phi_maps(w)[1]
    out = dev(np.zeros_like(x), w.dtype)
    arl2.feature_map(shape_of(w), dev(x, w.dtype), dev(phi, w.dtype), out, normalize)
    ref = oracle.feature_map(x, phi)
    if normalize:
        ref = oracle.l2_normalize_rows(ref)
    assert_close(host(out), ref, TOL[w.dtype], "feature map")


@pytest.mark.parametrize("case", STEP_CASES, ids=_ids)
@pytest.mark.parametrize("stress", [False, True])
def test_intra_attn(case, stress):
    from hybrid_linear_memory_amd import arl2
    w = _w(*case)
    log(f"intra_attn {_ids(case)} stress={stress}")
    q, k, v = synth.stress_qkv(w, 0, 1) if stress else synth.qkv(w, 0, 1)
    o = dev(np.zeros_like(q), w.dtype)
    arl2.intra_attn(shape_of(w), dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), o)
    ref = oracle.intra_attention(q, k, v)
    assert_close(host(o), ref, TOL[w.dtype], "o_intra")


def test_intra_attn_far_maximum():
    """Keys whose scores exceed every score of their stream's first tile by
    far more than 64 in log2 units (beyond the fixed-reference exponent range):
    the kernel must take its exact-maximum redo and still match the oracle."""
    from hybrid_linear_memory_amd import arl2
    w = _w("bf16", 1, 2, 300, 128)
    log("intra_attn far maximum")
    q, k, v = synth.qkv(w, 0, 1)
    q = synth.bf16_round(q + np.where(np.arange(128) == 0, 4.0, 0.0).astype(np.float32))
    k = k.copy()
    for t in (250, 290):             # second tiles of streams B (keys 192-255) and A (256-299)
        k[:, :, t, :] = 0.0
        k[:, :, t, 0] = 250.0
    o = dev(np.zeros_like(q), w.dtype)
    arl2.intra_attn(shape_of(w), dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), o)
    ref = oracle.intra_attention(q, k, v)
    assert_close(host(o), ref, TOL[w.dtype], "o_intra")


@pytest.mark.parametrize("case", STEP_CASES, ids=_ids)
def test_inter_read(case):
    from hybrid_linear_memory_amd import arl2
    w = _w(*case)
    log(f"inter_read {_ids(case)}")
    qp, oi, _ = synth.qkv(w, 1, 0)
    g = np.random.default_rng(5)
    S = (g.standard_normal((w.B, w.H, w.D, w.D)) * 0.05).astype(np.float32)
    o = dev(np.zeros_like(qp), w.dtype)
    arl2.inter_read(shape_of(w), dev(qp, w.dtype), dev32(S), dev(oi, w.dtype), o)
    ref = oi.astype(np.float64) + oracle.inter_read(qp, S)
    assert_close(host(o), ref, TOL[w.dtype], "o")
    # without o_intra, and in place (o == o_intra)
    o2 = dev(np.zeros_like(qp), w.dtype)
    arl2.inter_read(shape_of(w), dev(qp, w.dtype), dev32(S), None, o2)
    assert_close(host(o2), oracle.inter_read(qp, S), TOL[w.dtype], "o_inter only")
    o3 = dev(oi, w.dtype)
    arl2.inter_read(shape_of(w), dev(qp, w.dtype), dev32(S), o3, o3)
    assert_close(host(o3), ref, TOL[w.dtype], "in place")


@pytest.mark.parametrize("case", STEP_CASES, ids=_ids)
def test_state_commit(case):
    from hybrid_linear_memory_amd import arl2
    w = _w(*case)
    log(f"state_commit {_ids(case)}")
    k, v = synth.kv(w, 0, 0)                      # unit rows, cast to the activation type
    beta, alpha = synth.gates(w, 0)
    g = np.random.default_rng(6)
    S = (g.standard_normal((w.B, w.H, w.D, w.D)) * 0.05).astype(np.float32)
    Sn = dev32(np.zeros_like(S))
    sh = shape_of(w)
    ws = arl2.alloc_workspace(sh, arl2.OP_STATE_COMMIT)
    arl2.state_commit(sh, dev(k, w.dtype), dev(v, w.dtype), dev32(beta), dev32(alpha), dev32(S),
                      Sn, ws)
    ref = oracle.state_commit(k, v, beta, alpha, S)
    assert_close(host(Sn), ref, TOL[w.dtype], "S_next")


# The fused commit from the raw K, V over its token-part splits: 2 parts (513
# tokens; 3 heads x 777; 8 videos; one token), 3 (one head x 768), 4 (12 heads
# x 1560; one head x 1560, ragged parts) and 8 (one head x 4000).
COMMIT_CASES = [("bf16", 1, 2, 513, 128), ("bf16", 2, 3, 1, 128), ("bf16", 1, 3, 777, 128),
                ("bf16", 1, 1, 768, 128), ("bf16", 1, 12, 1560, 128), ("bf16", 1, 1, 1560, 128),
                ("bf16", 1, 1, 4000, 128), ("bf16", 8, 12, 200, 128)]


@pytest.mark.parametrize("case", COMMIT_CASES, ids=_ids)
def test_commit(case):
    """arl2_commit against the oracle's commit on a workspace first filled with
    arbitrary bytes (no clearing needed: the counters carry a per-call tag),
    then again on the same workspace with different inputs (every part's slot
    and the counters reused)."""
    import torch
    from hybrid_linear_memory_amd import arl2
    w = _w(*case)
    log(f"commit {_ids(case)}")
    sh = shape_of(w)
    phis = synth.phi_maps(w)
    ws = arl2.alloc_workspace(sh, arl2.OP_COMMIT)
    tg = torch.Generator(device="cuda").manual_seed(11)
    ws.copy_(torch.randint(0, 256, ws.shape, generator=tg, device="cuda", dtype=torch.int32)
             .to(torch.uint8))
    g = np.random.default_rng(9)
    for call in range(2):
        k, v = synth.kv(w, call, 0)
        beta, alpha = synth.gates(w, call)
        S = (g.standard_normal((w.B, w.H, w.D, w.D)) * 0.05).astype(np.float32)
        Sn = dev32(np.zeros_like(S))
        arl2.commit(sh, dev(k, w.dtype), dev(v, w.dtype), dev(phis[1], w.dtype),
                    dev(phis[2], w.dtype), dev32(beta), dev32(alpha), dev32(S), Sn, ws)
        assert_close(host(Sn), oracle.commit(k, v, phis[1], phis[2], beta, alpha, S),
                     TOL[w.dtype], f"S_next (call {call})")


@pytest.mark.parametrize("case", STEP_CASES, ids=_ids)
def test_clean_pass_prepared(case):
    """The one-call clean pass from a prepared map: every output and S_next
    against the oracle's read and commit, and the next frame's map."""
    import torch
    from hybrid_linear_memory_amd import arl2
    w = _w(*case)
    log(f"clean_pass_prepared {_ids(case)}")
    sh = shape_of(w)
    q, k, v = synth.qkv(w, 1, w.passes - 1)
    beta, alpha = synth.gates(w, 1)
    phis = synth.phi_maps(w)
    g = np.random.default_rng(8)
    S = (g.standard_normal((w.B, w.H, w.D, w.D)) * 0.05).astype(np.float32)
    dS, Sn = dev32(S), dev32(np.zeros_like(S))
    M = arl2.alloc_prepared(sh)
    arl2.read_prepare(sh, dev(phis[0], w.dtype), dS, M)
    o, oi, oe = (dev(np.zeros_like(q), w.dtype) for _ in range(3))
    ws = arl2.alloc_workspace(sh, arl2.OP_CLEAN_PASS_PREPARED)
    M_next = arl2.alloc_prepared(sh)
    dphi_q = dev(phis[0], w.dtype)
    arl2.clean_pass_prepared(sh, dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), M,
                             dev(phis[1], w.dtype), dev(phis[2], w.dtype), dev32(beta),
                             dev32(alpha), dS, Sn, o, oi, oe, ws, phi_q=dphi_q,
                             prepared_next=M_next)
    ref = oracle.read(q, k, v, phis[0], S)
    for name, got in (("o", o), ("o_intra", oi), ("o_inter", oe)):
        assert_close(host(got), ref[name], TOL[w.dtype], name)
    assert_close(host(Sn), oracle.commit(k, v, phis[1], phis[2], beta, alpha, S), TOL[w.dtype],
                 "S_next")
    # the next map is exactly what a separate preparation from S_next forms
    M_sep = arl2.alloc_prepared(sh)
    arl2.read_prepare(sh, dphi_q, Sn, M_sep)
    torch.cuda.synchronize()
    assert torch.equal(M_next, M_sep)


def test_rollout_tiny_fp32_all_passes():
    """Workload 0: every pass of every frame, every row, and the state."""
    w = synth.WORKLOADS[0]
    log("rollout tiny fp32")
    worst = lockstep_rollout(w, read_frames=set(range(w.frames)))
    log(f"worst relative errors {worst}")


@pytest.mark.parametrize("prepared", [True, False])
def test_rollout_clean_pass_as_two_calls(prepared):
    """The layer with its clean pass issued as a read and a commit (not the
    one-launch clean pass), with and without prepared reads."""
    w = synth.WORKLOADS[1]
    log(f"rollout, clean pass as two calls, prepared={prepared}")
    worst = lockstep_rollout(w, read_frames={0, 2}, row_sample=np.r_[0:16, w.T - 16:w.T],
                             frames=3, prepared=prepared, fused_clean=False)
    log(f"worst relative errors {worst}")


def _rows(T):
    return np.unique(np.r_[0:16, T // 2 - 8:T // 2 + 8, T - 16:T])


def test_rollout_wan13b_layer():
    """Workload 1 (1 x 12 x 128, T = 1560, 21 frames, 4 reads + clean pass):
    state after every commit; every row of every pass's outputs on frames 0,
    1, 10 and 20."""
    w = synth.WORKLOADS[1]
    log("rollout wan13b layer")
    worst = lockstep_rollout(w, read_frames={0, 1, 10, 20})
    log(f"worst relative errors {worst}")


@pytest.mark.timeout(900)
def test_rollout_wan13b_layer_clean_pass_every_frame():
    """Workload 1 with every frame's state written by the layer's one-call
    clean pass (the read and the fused commit in one launch, then the chunk
    sum that also forms the next frame's map): all 21 frames in a row, every
    row of the clean pass's outputs on every frame, the state after every
    commit; frames 0 and 20 also run their 4 denoising reads."""
    w = synth.WORKLOADS[1]
    log("rollout wan13b layer, clean pass on every frame")
    worst = lockstep_rollout(w, read_frames={0, 20}, commit_via="clean_pass")
    log(f"worst relative errors {worst}")


@pytest.mark.timeout(900)
def test_rollout_long_240_frames():
    """Workload 2: 240 consecutive frames through the layer's one-call clean
    pass; the state after every commit, the clean pass's outputs on sampled
    rows of every frame and on every row of every 20th frame and the last;
    every row of every pass of frames 0, 120 and 239 (with their denoising
    reads)."""
    w = synth.WORKLOADS[2]
    log("rollout long 240 frames")
    worst = lockstep_rollout(w, read_frames={0, 120, 239}, commit_via="clean_pass",
                             clean_rows=_rows(w.T), full_every=20)
    log(f"worst relative errors {worst}")


@pytest.mark.timeout(900)
def test_rollout_batched_streams():
    """Workload 3: 8 independent videos; every row of every pass on frames 0
    and 20, the state after every commit."""
    w = synth.WORKLOADS[3]
    log("rollout batched streams")
    worst = lockstep_rollout(w, read_frames={0, 20})
    log(f"worst relative errors {worst}")


@pytest.mark.timeout(900)
def test_rollout_large_model():
    """Workload 4: 40 heads, 81 frames; every row of every pass on frames 0,
    40 and 80, the state after every commit."""
    w = synth.WORKLOADS[4]
    log("rollout large model")
    worst = lockstep_rollout(w, read_frames={0, 40, 80})
    log(f"worst relative errors {worst}")


@pytest.mark.parametrize("D", [16, 64])
def test_rollout_bf16_small_head_dims(D):
    """bf16 activations at head dimensions 16 and 64 (the generic kernels):
    three frames through the layer, every row of every pass, the state after
    every commit, with both the one-call clean pass and the commit-only call."""
    w = synth.WORKLOADS[1].replace(H=3, D=D, T=300, frames=3, n_denoise=2)
    log(f"rollout bf16 D={D}")
    worst = lockstep_rollout(w, read_frames={0, 2})
    log(f"worst relative errors {worst}")
    worst = lockstep_rollout(w, read_frames={2}, commit_via="clean_pass")
    log(f"worst relative errors (clean pass every frame) {worst}")


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_fullkv_comparator(dtype, D):
    """The full-KV comparator equals softmax over every cached key (three
    frames in a larger cache, ragged total)."""
    import torch
    from hybrid_linear_memory_amd import arl2
    T = 300 if dtype == "bf16" else 70
    w = _w(dtype, 1, 2, T, D)
    log(f"fullkv {dtype} D={D}")
    frames = [synth.qkv(w, f, 0) for f in range(3)]
    cap = 4 * T + 5
    kc = torch.zeros((1, 2, cap, D), dtype=shape_of(w).torch_dtype, device="cuda")
    vc = torch.zeros_like(kc)
    for f, (_, k, v) in enumerate(frames):
        kc[:, :, f * T:(f + 1) * T] = dev(k, dtype)
        vc[:, :, f * T:(f + 1) * T] = dev(v, dtype)
    q = frames[2][0]
    o = dev(np.zeros_like(q), dtype)
    arl2.fullkv_attn(shape_of(w), dev(q, dtype), kc, vc, 3 * T, o)
    K = np.concatenate([f[1] for f in frames], 2)
    V = np.concatenate([f[2] for f in frames], 2)
    assert_close(host(o), oracle.fullkv_attention(q, K, V), TOL[dtype], "fullkv")


@pytest.mark.parametrize("case", [("bf16", 1, 3, 300, 128), ("f32", 2, 2, 70, 32)], ids=_ids)
def test_read_paths_agree(case):
    """The one-call read (Phi_q and S given) and the prepared read (M = Phi_q S
    formed once) both match the oracle; on the bf16 path the one-call read is
    the prepared read, so their bytes agree exactly. (The float32 one-call read
    forms Q' = Q Phi_q first, so its rounding order differs.)"""
    import torch
    from hybrid_linear_memory_amd import arl2
    w = _w(*case)
    log(f"read paths {_ids(case)}")
    sh = shape_of(w)
    q, k, v = synth.qkv(w, 2, 0)
    phi = synth.phi_maps(w)[0]
    g = np.random.default_rng(7)
    S = (g.standard_normal((w.B, w.H, w.D, w.D)) * 0.05).astype(np.float32)
    dq, dk, dv, dphi, dS = dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), dev(phi, w.dtype), dev32(S)
    o1, o2 = dev(np.zeros_like(q), w.dtype), dev(np.zeros_like(q), w.dtype)
    ws = arl2.alloc_workspace(sh, arl2.OP_READ)
    arl2.read(sh, dq, dk, dv, dphi, dS, o1, ws=ws)
    M = arl2.alloc_prepared(sh)
    arl2.read_prepare(sh, dphi, dS, M)
    wsp = arl2.alloc_workspace(sh, arl2.OP_READ_PREPARED)
    oi, oe = dev(np.zeros_like(q), w.dtype), dev(np.zeros_like(q), w.dtype)
    arl2.read_prepared(sh, dq, dk, dv, M, o2, oi, oe, ws=wsp)
    torch.cuda.synchronize()
    if w.dtype == "bf16":
        assert torch.equal(o1, o2)
    ref = oracle.read(q, k, v, phi, S)
    assert_close(host(o1), ref["o"], TOL[w.dtype], "o (one-call read)")
    assert_close(host(o2), ref["o"], TOL[w.dtype], "o")
    assert_close(host(oi), ref["o_intra"], TOL[w.dtype], "o_intra")
    assert_close(host(oe), ref["o_inter"], TOL[w.dtype], "o_inter")


def test_binding_rejects_wrong_sizes():
    """The binding checks every tensor's element count against the shape
    before calling the library (which sees only pointers): a tensor one
    element short, or a map of the wrong head count, raises without a launch."""
    import torch
    from hybrid_linear_memory_amd import arl2
    sh = arl2.Shape(1, 2, 64, 128, arl2.BF16)
    act = dict(dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((1, 2, 64, 128), **act)
    short = torch.zeros(1 * 2 * 64 * 128 - 1, **act)
    o = torch.zeros_like(q)
    with pytest.raises(ValueError, match="elements"):
        arl2.intra_attn(sh, q, short, q, o)
    phi = torch.zeros((3, 128, 128), **act)
    S = torch.zeros((1, 2, 128, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="phi_q"):
        arl2.read(sh, q, q, q, phi, S, o, ws=arl2.alloc_workspace(sh, arl2.OP_READ))
    small = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="prepared"):
        arl2.read_prepared(sh, q, q, q, small, o)
