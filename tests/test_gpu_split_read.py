"""The split-key fused read (shapes whose query blocks leave compute units
idle: each query block's key tiles are dealt to several workgroups, whose
partial softmax results the last of them merges) matches the oracle, agrees
with the plain grid to the bf16 tolerance, and is deterministic: repeated
calls, and calls on a workspace holding arbitrary bytes, give the same bytes.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, assert_close, dev, dev32, host, log, shape_of
from hybrid_linear_memory_amd import synth

pytestmark = pytest.mark.gpu

# (B, H, T): long frames with few heads (the plain grid holds at most 128
# workgroups of 64 or 128 key tiles); a ragged last key tile and query block;
# two videos; three heads of 8192 tokens; more query blocks than compute
# units (workgroups then hold whole blocks between their first and last
# segments): 40 heads of 1560 tokens, 12 heads of 3600
CASES = [(1, 4, 4096), (1, 2, 8192), (1, 5, 4000), (2, 2, 4096), (1, 3, 8192), (1, 40, 1560),
         (1, 12, 3600)]


def _ids(c):
    return "B{}H{}T{}".format(*c)


def _setup(B, H, T, seed_frame=3):
    import torch
    from hybrid_linear_memory_amd import arl2
    w = synth.WORKLOADS[1].replace(B=B, H=H, T=T)
    sh = shape_of(w)
    q, k, v = synth.qkv(w, seed_frame, 0)
    phi = synth.phi_maps(w)[0]
    g = np.random.default_rng(11)
    S = (g.standard_normal((B, H, 128, 128)) * 0.05).astype(np.float32)
    M = arl2.alloc_prepared(sh)
    arl2.read_prepare(sh, dev(phi, "bf16"), dev32(S), M)
    torch.cuda.synchronize()
    return w, sh, (q, k, v, phi, S), M


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_split_read_matches_oracle(case):
    import torch
    from hybrid_linear_memory_amd import arl2
    w, sh, (q, k, v, phi, S), M = _setup(*case)
    log(f"split read {_ids(case)}")
    assert arl2.workspace_bytes(sh, arl2.OP_READ_PREPARED) > 0, "shape does not take the split"
    ws = arl2.alloc_workspace(sh, arl2.OP_READ_PREPARED)
    dq, dk, dv = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    o, oi, oe = (torch.empty(dq.shape, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    arl2.read_prepared(sh, dq, dk, dv, M, o, oi, oe, ws=ws)
    ref = oracle.read(q, k, v, phi, S)
    for name, t in (("o", o), ("o_intra", oi), ("o_inter", oe)):
        assert_close(host(t), ref[name], TOL["bf16"], name)
    # the plain grid (no workspace): same values up to the order of fp32 sums
    o_plain = torch.empty_like(o)
    arl2.read_prepared(sh, dq, dk, dv, M, o_plain)
    assert_close(host(o), host(o_plain), TOL["bf16"], "split vs plain grid")


@pytest.mark.parametrize("case", [(1, 4, 4096), (1, 5, 4000), (1, 40, 1560)], ids=_ids)
def test_split_read_deterministic_on_any_workspace(case):
    """Per-call counter tags: a workspace left by earlier calls, or filled
    with arbitrary bytes, needs no clearing, and every call gives the same
    bytes (the merge runs in key order, whichever segment arrives last)."""
    import torch
    from hybrid_linear_memory_amd import arl2
    w, sh, (q, k, v, _, _), M = _setup(*case)
    log(f"split read determinism {_ids(case)}")
    ws = arl2.alloc_workspace(sh, arl2.OP_READ_PREPARED)
    dq, dk, dv = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    outs = []
    for rep in range(4):
        if rep == 2:
            g = torch.Generator(device="cuda").manual_seed(5)
            ws.copy_(torch.randint(0, 256, ws.shape, generator=g, device="cuda",
                                   dtype=torch.int32).to(torch.uint8))
        o = torch.empty(dq.shape, dtype=torch.bfloat16, device="cuda")
        arl2.read_prepared(sh, dq, dk, dv, M, o, ws=ws)
        outs.append(o)
    torch.cuda.synchronize()
    for rep in range(1, 4):
        assert torch.equal(outs[0], outs[rep]), f"call {rep} differs"


@pytest.mark.parametrize("case", [(1, 4, 4096), (1, 5, 4000), (1, 40, 1560), (1, 12, 3600)],
                         ids=_ids)
def test_split_read_reused_workspace_new_inputs(case):
    """One workspace across calls whose inputs all differ (queries, keys,
    values and map): every row of each call against the oracle, and each
    call's bytes equal to those of the same inputs on a fresh workspace. A
    merge that read a slot left by the previous call (stale data from an
    earlier call in a cache) would fail both."""
    import torch
    from hybrid_linear_memory_amd import arl2
    B, H, T = case
    log(f"split read, reused workspace, new inputs {_ids(case)}")
    ws = None
    for call, frame in enumerate((3, 4, 5)):
        w, sh, (q, k, v, phi, S), M = _setup(B, H, T, seed_frame=frame)
        if ws is None:
            ws = arl2.alloc_workspace(sh, arl2.OP_READ_PREPARED)
        dq, dk, dv = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
        o, oi, oe = (torch.empty(dq.shape, dtype=torch.bfloat16, device="cuda")
                     for _ in range(3))
        arl2.read_prepared(sh, dq, dk, dv, M, o, oi, oe, ws=ws)
        fresh = arl2.alloc_workspace(sh, arl2.OP_READ_PREPARED)
        fresh.fill_(0x5A)
        o2 = torch.empty_like(o)
        arl2.read_prepared(sh, dq, dk, dv, M, o2, ws=fresh)
        torch.cuda.synchronize()
        assert torch.equal(o, o2), f"call {call}: reused workspace differs from a fresh one"
        ref = oracle.read(q, k, v, phi, S)
        for name, t in (("o", o), ("o_intra", oi), ("o_inter", oe)):
            assert_close(host(t), ref[name], TOL["bf16"], f"call {call} {name}")
        del fresh


def test_split_read_far_maximum():
    """A key far above every score of its segment's first tiles makes that
    segment take the exact-maximum redo; the merged output still matches."""
    import torch
    from hybrid_linear_memory_amd import arl2
    w, sh, (q, k, v, phi, S), M = _setup(1, 4, 4096)
    log("split read far maximum")
    q = synth.bf16_round(q + np.where(np.arange(128) == 0, 4.0, 0.0).astype(np.float32))
    k = k.copy()
    for t in (200, 1777, 3500):
        k[:, :, t, :] = 0.0
        k[:, :, t, 0] = 250.0
    ws = arl2.alloc_workspace(sh, arl2.OP_READ_PREPARED)
    o = torch.empty((1, 4, 4096, 128), dtype=torch.bfloat16, device="cuda")
    arl2.read_prepared(sh, dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), M, o, ws=ws)
    ref = oracle.read(q, k, v, phi, S)
    assert_close(host(o), ref["o"], TOL["bf16"], "o")


def test_split_read_workspace_too_small():
    import torch
    from hybrid_linear_memory_amd import arl2
    sh = arl2.Shape(1, 4, 4096, 128, arl2.BF16)
    need = arl2.workspace_bytes(sh, arl2.OP_READ_PREPARED)
    x = torch.zeros((1, 4, 4096, 128), dtype=torch.bfloat16, device="cuda")
    M = arl2.alloc_prepared(sh)
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(arl2.Arl2Error, match="workspace"):
        arl2.read_prepared(sh, x, x, x, M, torch.empty_like(x), ws=small)


def test_split_read_layer_rollout():
    """Three frames of a 4-head, 4096-token layer through Arl2Layer (whose
    denoising reads take the split-key grid): every row of every pass's
    outputs and the state after every commit against the oracle."""
    from gpu_helpers import lockstep_rollout
    from hybrid_linear_memory_amd import arl2
    w = synth.WORKLOADS[1].replace(H=4, T=4096, frames=3)
    assert arl2.workspace_bytes(shape_of(w), arl2.OP_READ_PREPARED) > 0
    log("split read layer rollout 1x4x4096")
    worst = lockstep_rollout(w, read_frames={0, 1, 2})
    log(f"worst relative errors {worst}")
