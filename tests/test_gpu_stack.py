"""A model-shaped stack of hybrid ARL2 layers and KV-cache softmax layers
against the oracle's stack (hybrid_stack_rollout): every output of every pass
of every layer, and every ARL2 layer's state after each frame. Tolerances as
in the other parity tests (1e-4 fp32, 2e-2 bf16, of max|oracle| per tensor)."""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, assert_close, dev, dev32, host, log, shape_of
from hybrid_linear_memory_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stack_matches_oracle(dtype):
    import torch
    from hybrid_linear_memory_amd.stack import HybridStack
    if dtype == "bf16":
        base = synth.WORKLOADS[1].replace(H=2, T=200, frames=3, n_denoise=2)
    else:
        base = synth.WORKLOADS[0].replace(T=40, frames=3, n_denoise=2)
    mask = [True, False, False, True]
    lws = [base.replace(seed=l + 1) for l in range(len(mask))]     # own inputs per layer
    phis = [synth.phi_maps(lw) for lw in lws]
    log(f"stack {dtype} mask={mask}")
    stack = HybridStack(shape_of(base), mask, [tuple(dev(p, dtype) for p in ph) for ph in phis],
                        max_frames=base.frames)
    layers = [{"frames": [synth.oracle_frame(lw, f) for f in range(base.frames)],
               "phis": ph} for lw, ph in zip(lws, phis)]
    ref = oracle.hybrid_stack_rollout(layers, mask)
    tol = TOL[dtype]
    for f in range(base.frames):
        for p in range(base.passes):
            inputs = [tuple(dev(x, dtype) for x in synth.qkv(lw, f, p)) for lw in lws]
            if p < base.passes - 1:
                outs = stack.read(inputs)
            else:
                gates = [tuple(dev32(g) for g in synth.gates(lw, f)) for lw in lws]
                outs = stack.clean_pass(inputs, gates)
            for l, o in enumerate(outs):
                assert_close(host(o), ref[l]["o"][(f, p)], tol, f"layer {l} frame {f} pass {p}")
        torch.cuda.synchronize()
        for l, lay in enumerate(stack.layers):
            if mask[l]:
                assert_close(host(lay.S), ref[l]["states"][f + 1], tol, f"layer {l} state {f + 1}")
    # attention state: the softmax layers' caches hold every frame, the ARL2 layers a constant
    s = shape_of(base)
    ebytes = 2 if dtype == "bf16" else 4
    cache = 2 * base.frames * base.T * base.H * base.D * ebytes
    const = 2 * base.H * base.D * base.D * 4 + 2 * base.H * base.D * base.D * ebytes
    assert stack.state_bytes() == 2 * const + 2 * cache, (stack.state_bytes(), const, cache)
