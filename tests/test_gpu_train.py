"""Parity of the training-side calls (arl2_intra_attn_backward,
arl2_read_backward, arl2_commit_backward, arl2_state_scan and the rollout
driver) with the oracle's gradients (themselves pinned by finite differences).

Tolerance as for the forward: max |gpu - oracle| <= 1e-4 * max|oracle| for
float32 workloads and <= 2e-2 * max|oracle| for bf16 workloads, per gradient
tensor. The upstream gradients are seeded normal tensors; the forward o_intra
that the backward takes is the GPU forward's own output.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, assert_close, dev, dev32, host, log, shape_of
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


CASES = [
    ("f32", 1, 1, 64, 16), ("f32", 2, 3, 100, 32), ("f32", 1, 2, 37, 64), ("f32", 1, 2, 130, 128),
    ("f32", 1, 1, 1, 16),
    ("bf16", 2, 3, 1, 128), ("bf16", 1, 1, 37, 128), ("bf16", 1, 2, 200, 128),
    ("bf16", 1, 2, 513, 128), ("bf16", 1, 4, 1560, 128),
]


def _ids(c):
    return "{}-B{}H{}T{}D{}".format(*c)


def _grad_out(w, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return synth.bf16_round(g.standard_normal((w.B, w.H, w.T, w.D)) * scale) \
        if w.dtype == "bf16" else g.standard_normal((w.B, w.H, w.T, w.D)) * scale


def _close(got, ref, tol, name, floor=0.0):
    """assert_close, except that a gradient the mathematics makes exactly zero
    (one key: dQ = dK = 0) is held to tol times the scale of a sibling gradient."""
    if np.abs(ref).max() == 0.0:
        assert np.all(np.isfinite(got)) and np.abs(got).max() <= tol * floor, name
        return
    assert_close(got, ref, tol, name)


def _zeros(shape, dtype="f32"):
    import torch
    return torch.zeros(shape, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                       device="cuda")


def _forward(arl2, sh, w, q, k, v, with_lse):
    """o_intra, and the rows' log-sum-exp when with_lse (else None)."""
    o = _zeros((w.B, w.H, w.T, w.D), w.dtype)
    if not with_lse:
        arl2.intra_attn(sh, q, k, v, o)
        return o, None
    lse = _zeros((w.B, w.H, w.T))
    arl2.intra_attn_lse(sh, q, k, v, o, lse)
    return o, lse


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_intra_attn_lse(case):
    """The forward with the rows' log-sum-exp: o_intra identical to
    arl2_intra_attn's, lse against the oracle's (absolute: it is a logarithm;
    bf16 inputs, and the kernel's sum of bf16-rounded weights, leave ~1e-3)."""
    import torch
    from hybrid_linear_memory_amd import arl2
    w = _w(*case)
    log(f"intra_attn_lse {_ids(case)}")
    sh = shape_of(w)
    q, k, v = synth.qkv(w, 0, 1)
    dq_, dk_, dv_ = (dev(x, w.dtype) for x in (q, k, v))
    o1, _ = _forward(arl2, sh, w, dq_, dk_, dv_, False)
    o2, lse = _forward(arl2, sh, w, dq_, dk_, dv_, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    ref = oracle.attention_logsumexp(q, k)
    err = np.abs(host(lse) - ref).max()
    assert err <= (2e-2 if w.dtype == "bf16" else 1e-5), f"lse: max |err| {err:.3e}"


@pytest.mark.parametrize("case", CASES, ids=_ids)
@pytest.mark.parametrize("with_lse", [False, True])
def test_intra_attn_backward(case, with_lse):
    from hybrid_linear_memory_amd import arl2
    w = _w(*case)
    log(f"intra_attn_backward {_ids(case)} lse={with_lse}")
    sh = shape_of(w)
    q, k, v = synth.qkv(w, 0, 1)
    d_o = _grad_out(w, 20)
    dq_, dk_, dv_ = (dev(x, w.dtype) for x in (q, k, v))
    o, lse = _forward(arl2, sh, w, dq_, dk_, dv_, with_lse)
    grads = [_zeros((w.B, w.H, w.T, w.D), w.dtype) for _ in range(3)]
    ws = arl2.alloc_workspace(sh, arl2.OP_INTRA_ATTN_BACKWARD)
    arl2.intra_attn_backward(sh, dq_, dk_, dv_, o, dev(d_o, w.dtype), *grads, ws=ws, lse=lse)
    ref = oracle.intra_attention_backward(q, k, v, d_o)
    for name, got in zip(("dq", "dk", "dv"), grads):
        _close(host(got), ref[name], TOL[w.dtype], name, floor=np.abs(ref["dv"]).max())


@pytest.mark.parametrize("case", [("bf16", 1, 2, 513, 128), ("bf16", 1, 3, 256, 128)], ids=_ids)
def test_attn_backward_split_halves(case):
    """Shapes whose dK/dV key blocks are split over two query halves (the
    second half to finish adds the first's fp32 sums): identical bits over
    repeated calls on a workspace refilled with arbitrary bytes (the pair
    counters need no clearing), accumulate = 1 doubles, and the oracle agrees
    (513 tokens: 9 query stages, halves of 4 and 5)."""
    import torch
    from hybrid_linear_memory_amd import arl2
    w = _w(*case)
    log(f"attention backward split halves {_ids(case)}")
    sh = shape_of(w)
    q, k, v = synth.qkv(w, 0, 1)
    d_o = _grad_out(w, 21)
    dq_, dk_, dv_, do_ = (dev(x, w.dtype) for x in (q, k, v, d_o))
    o, lse = _forward(arl2, sh, w, dq_, dk_, dv_, True)
    ws = arl2.alloc_workspace(sh, arl2.OP_INTRA_ATTN_BACKWARD)
    runs = []
    for fill in (0xA5, 0x00, 0xFF):
        ws.fill_(fill)
        grads = [_zeros((w.B, w.H, w.T, w.D), w.dtype) for _ in range(3)]
        arl2.intra_attn_backward(sh, dq_, dk_, dv_, o, do_, *grads, ws=ws, lse=lse)
        runs.append(grads)
    torch.cuda.synchronize()
    for r in runs[1:]:
        for name, x, y in zip(("dq", "dk", "dv"), runs[0], r):
            assert torch.equal(x, y), f"{name} not reproducible"
    twice = [x.clone() for x in runs[0]]
    arl2.intra_attn_backward(sh, dq_, dk_, dv_, o, do_, *twice, accumulate=True, ws=ws, lse=lse)
    for name, x, y in zip(("dq", "dk", "dv"), runs[0], twice):
        assert_close(host(y), 2 * host(x), 1e-2, name)
    ref = oracle.intra_attention_backward(q, k, v, d_o)
    for name, got in zip(("dq", "dk", "dv"), runs[0]):
        _close(host(got), ref[name], TOL[w.dtype], name, floor=np.abs(ref["dv"]).max())


@pytest.mark.parametrize("case", [("bf16", 1, 2, 513, 128), ("bf16", 1, 4, 1560, 128)], ids=_ids)
def test_attn_backward_split_reused_workspace_new_inputs(case):
    """One workspace across attention backward calls whose inputs all differ:
    each call's gradients equal, bit for bit, those of the same inputs on a
    fresh workspace, and match the oracle. A pair merge that added sums left
    in a slot by the previous call would fail both."""
    import torch
    from hybrid_linear_memory_amd import arl2
    w = _w(*case)
    log(f"attention backward, reused workspace, new inputs {_ids(case)}")
    sh = shape_of(w)
    ws = arl2.alloc_workspace(sh, arl2.OP_INTRA_ATTN_BACKWARD)
    for call, frame in enumerate((0, 1, 2)):
        q, k, v = synth.qkv(w, frame, 1)
        d_o = _grad_out(w, 30 + frame)
        dq_, dk_, dv_, do_ = (dev(x, w.dtype) for x in (q, k, v, d_o))
        o, lse = _forward(arl2, sh, w, dq_, dk_, dv_, True)
        grads = [_zeros((w.B, w.H, w.T, w.D), w.dtype) for _ in range(3)]
        arl2.intra_attn_backward(sh, dq_, dk_, dv_, o, do_, *grads, ws=ws, lse=lse)
        fresh = arl2.alloc_workspace(sh, arl2.OP_INTRA_ATTN_BACKWARD)
        fresh.fill_(0x3C)
        again = [_zeros((w.B, w.H, w.T, w.D), w.dtype) for _ in range(3)]
        arl2.intra_attn_backward(sh, dq_, dk_, dv_, o, do_, *again, ws=fresh, lse=lse)
        torch.cuda.synchronize()
        for name, x, y in zip(("dq", "dk", "dv"), grads, again):
            assert torch.equal(x, y), f"call {call}: {name} differs from a fresh workspace"
        ref = oracle.intra_attention_backward(q, k, v, d_o)
        for name, got in zip(("dq", "dk", "dv"), grads):
            _close(host(got), ref[name], TOL[w.dtype], f"call {call} {name}",
                   floor=np.abs(ref["dv"]).max())
        del fresh


@pytest.mark.parametrize("case", CASES, ids=_ids)
@pytest.mark.parametrize("with_lse", [False, True])
def test_read_backward(case, with_lse):
    from hybrid_linear_memory_amd import arl2
    w = _w(*case)
    log(f"read_backward {_ids(case)} lse={with_lse}")
    sh = shape_of(w)
    q, k, v = synth.qkv(w, 0, 1)
    phis = synth.phi_maps(w)
    g = np.random.default_rng(21)
    S = (g.standard_normal((w.B, w.H, w.D, w.D)) * 0.05).astype(np.float32)
    d_o = _grad_out(w, 22)
    dq_, dk_, dv_ = (dev(x, w.dtype) for x in (q, k, v))
    o, lse = _forward(arl2, sh, w, dq_, dk_, dv_, with_lse)
    grads = [_zeros((w.B, w.H, w.T, w.D), w.dtype) for _ in range(3)]
    dphi = _zeros((w.H, w.D, w.D))
    dS = _zeros((w.B, w.H, w.D, w.D))
    ws = arl2.alloc_workspace(sh, arl2.OP_READ_BACKWARD)
    arl2.read_backward(sh, dq_, dk_, dv_, dev(phis[0], w.dtype), dev32(S), o, dev(d_o, w.dtype),
                       *grads, dphi, dS, ws=ws, lse=lse)
    ref = oracle.read_backward(q, k, v, phis[0], S, d_o)
    for name, got in zip(("dq", "dk", "dv", "dphi_q", "dS"), grads + [dphi, dS]):
        _close(host(got), ref[name], TOL[w.dtype], name, floor=np.abs(ref["dv"]).max())


def _commit_inputs(w, strong):
    q, k, v = synth.qkv(w, 1, w.passes - 1)
    beta, alpha = synth.gates(w, 1)
    g = np.random.default_rng(23)
    if strong:
        beta = (1.0 / (1.0 + np.exp(-g.standard_normal((w.B, w.H, w.T))))).astype(np.float32)
    S = (g.standard_normal((w.B, w.H, w.D, w.D)) * 0.05).astype(np.float32)
    G = g.standard_normal((w.B, w.H, w.D, w.D)).astype(np.float32)
    return k, v, beta, alpha, S, G


def _commit_call(arl2, w, sh, k, v, phis, beta, alpha, S, G, accumulate=False, outs=None):
    if outs is None:
        outs = [_zeros((w.B, w.H, w.T, w.D), w.dtype), _zeros((w.B, w.H, w.T, w.D), w.dtype),
                _zeros((w.H, w.D, w.D)), _zeros((w.H, w.D, w.D)), _zeros((w.B, w.H, w.T)),
                _zeros((w.B, w.H)), _zeros((w.B, w.H, w.D, w.D))]
    ws = arl2.alloc_workspace(sh, arl2.OP_COMMIT_BACKWARD)
    arl2.commit_backward(sh, dev(k, w.dtype), dev(v, w.dtype), dev(phis[1], w.dtype),
                         dev(phis[2], w.dtype), dev32(beta), dev32(alpha), dev32(S), dev32(G),
                         *outs, accumulate=accumulate, ws=ws)
    return outs


COMMIT_NAMES = ("dk", "dv", "dphi_k", "dphi_v", "dbeta", "dalpha", "dS_prev")


@pytest.mark.parametrize("case", CASES, ids=_ids)
@pytest.mark.parametrize("strong", [False, True])
def test_commit_backward(case, strong):
    from hybrid_linear_memory_amd import arl2
    w = _w(*case)
    log(f"commit_backward {_ids(case)} strong={strong}")
    sh = shape_of(w)
    k, v, beta, alpha, S, G = _commit_inputs(w, strong)
    phis = synth.phi_maps(w)
    outs = _commit_call(arl2, w, sh, k, v, phis, beta, alpha, S, G)
    ref = oracle.commit_backward(k, v, phis[1], phis[2], beta, alpha, S, G)
    for name, got in zip(COMMIT_NAMES, outs):
        assert_close(host(got), ref[name], TOL[w.dtype], name)


@pytest.mark.parametrize("case", [("f32", 2, 3, 100, 32), ("bf16", 1, 2, 200, 128)], ids=_ids)
def test_backward_accumulate_and_determinism(case):
    """accumulate = 1 adds to what the outputs hold (twice the gradient after a
    second call); accumulate = 0 overwrites; identical calls give identical
    bits."""
    import torch
    from hybrid_linear_memory_amd import arl2
    w = _w(*case)
    log(f"accumulate/determinism {_ids(case)}")
    sh = shape_of(w)
    k, v, beta, alpha, S, G = _commit_inputs(w, True)
    phis = synth.phi_maps(w)
    a = _commit_call(arl2, w, sh, k, v, phis, beta, alpha, S, G)
    b = _commit_call(arl2, w, sh, k, v, phis, beta, alpha, S, G)
    for name, x, y in zip(COMMIT_NAMES, a, b):
        assert torch.equal(x, y), f"{name} not reproducible"
    twice = _commit_call(arl2, w, sh, k, v, phis, beta, alpha, S, G, accumulate=True,
                         outs=[x.clone() for x in a])
    for name, x, y in zip(COMMIT_NAMES, a, twice):
        assert_close(host(y), 2 * host(x), 1e-2 if w.dtype == "bf16" else 1e-6, name)
    junk = [x.clone().fill_(7.0) for x in a]
    over = _commit_call(arl2, w, sh, k, v, phis, beta, alpha, S, G, accumulate=False, outs=junk)
    for name, x, y in zip(COMMIT_NAMES, a, over):
        assert torch.equal(x, y), f"{name}: accumulate=0 did not overwrite"


@pytest.mark.parametrize("dtype,B,H,T,D", [("f32", 2, 2, 70, 32), ("bf16", 1, 3, 300, 128)])
def test_state_scan(dtype, B, H, T, D):
    import torch
    from hybrid_linear_memory_amd import arl2
    w = _w(dtype, B, H, T, D, frames=3)
    log(f"state_scan {dtype} B{B}H{H}T{T}D{D}")
    sh = shape_of(w)
    phis = synth.phi_maps(w)
    ks, vs, betas, alphas = [], [], [], []
    oframes = []
    for f in range(w.frames):
        k, v = synth.kv(w, f, w.passes - 1)
        beta, alpha = synth.gates(w, f)
        ks.append(k); vs.append(v); betas.append(beta); alphas.append(alpha)
        oframes.append({"passes": [(None, k, v)], "beta": beta, "alpha": alpha})
    g = np.random.default_rng(24)
    S0 = (g.standard_normal((B, H, D, D)) * 0.05).astype(np.float32)
    states = _zeros((w.frames + 1, B, H, D, D))
    ws = arl2.alloc_workspace(sh, arl2.OP_COMMIT)
    arl2.state_scan(sh, dev(np.stack(ks), dtype), dev(np.stack(vs), dtype),
                    dev(phis[1], dtype), dev(phis[2], dtype), dev32(np.stack(betas)),
                    dev32(np.stack(alphas)), dev32(S0), states, ws)
    ref = oracle.state_scan(oframes, phis[1], phis[2], S0)
    torch.cuda.synchronize()
    assert np.array_equal(host(states[0]), S0.astype(np.float64))
    for f in range(1, w.frames + 1):
        assert_close(host(states[f]), ref[f], TOL[dtype], f"state {f}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rollout_backward(dtype):
    """Gradients through the frame recurrence (train.rollout_backward on the
    C-ABI calls) against oracle.rollout_backward: every q, k, v of every pass,
    the gates, the three maps and S_0."""
    from hybrid_linear_memory_amd import train
    w = (synth.WORKLOADS[0].replace(frames=3) if dtype == "f32" else
         synth.WORKLOADS[1].replace(H=2, T=200, frames=3, n_denoise=1))
    log(f"rollout_backward {dtype}")
    sh = shape_of(w)
    phis = synth.phi_maps(w)
    g = np.random.default_rng(25)
    S0 = (g.standard_normal((w.B, w.H, w.D, w.D)) * 0.05).astype(np.float32)
    oframes, dframes, d_out, dd_out = [], [], {}, {}
    for f in range(w.frames):
        beta, alpha = synth.gates(w, f)
        beta = beta * w.T * 0.5
        passes = [synth.qkv(w, f, p) for p in range(w.passes)]
        oframes.append({"passes": passes, "beta": beta, "alpha": alpha})
        dframes.append({"passes": [tuple(dev(x, dtype) for x in ps) for ps in passes],
                        "beta": dev32(beta), "alpha": dev32(alpha)})
        for p in range(w.passes):
            d_out[(f, p)] = _grad_out(w, 100 + 10 * f + p, 0.1)
            dd_out[(f, p)] = dev(d_out[(f, p)], dtype)
    dS_final = (g.standard_normal((w.B, w.H, w.D, w.D)) * 0.1).astype(np.float32)
    got = train.rollout_backward(sh, dframes, *(dev(p, dtype) for p in phis), dd_out,
                                 S0=dev32(S0), dS_final=dev32(dS_final))
    ref = oracle.rollout_backward(oframes, *phis, d_out, S0=S0, dS_final=dS_final)
    tol = TOL[dtype]
    for key, (dq, dk, dv) in ref["d_passes"].items():
        for name, x, y in zip(("dq", "dk", "dv"), got["d_passes"][key], (dq, dk, dv)):
            assert_close(host(x), y, tol, f"{name} {key}")
    for f in range(w.frames):
        assert_close(host(got["dbeta"][f]), ref["dbeta"][f], tol, f"dbeta {f}")
        assert_close(host(got["dalpha"][f]), ref["dalpha"][f], tol, f"dalpha {f}")
    for name in ("dphi_q", "dphi_k", "dphi_v", "dS0"):
        assert_close(host(got[name]), ref[name], tol, name)
