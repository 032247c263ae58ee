"""The allocation-free read (arl2_read_noalloc, for callers that cannot
allocate): its scratch is the library's fixed device array instead of a
caller workspace. Through the C ABI it must give what arl2_read gives on the
same inputs (the same kernels run: identical bytes), on two calls in a row,
the second with a smaller input, for the bf16 MFMA path and the float32 /
small-D path; a shape beyond the fixed scratch is refused before any launch.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, assert_close, dev, dev32, host, log, shape_of
from hybrid_linear_memory_amd import synth

pytestmark = pytest.mark.gpu


def _inputs(w, frame):
    q, k, v = synth.qkv(w, frame, 0)
    phi = synth.phi_maps(w)[0]
    g = np.random.default_rng(40 + frame)
    S = (g.standard_normal((w.B, w.H, w.D, w.D)) * 0.05).astype(np.float32)
    return q, k, v, phi, S


def _both(w, frame):
    import torch
    from hybrid_linear_memory_amd import arl2
    sh = shape_of(w)
    q, k, v, phi, S = _inputs(w, frame)
    dq, dk, dv, dphi, dS = (dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype),
                            dev(phi, w.dtype), dev32(S))
    outs = []
    for noalloc in (True, False):
        o, oi, oe = (torch.full(dq.shape, 7.0, dtype=dq.dtype, device="cuda") for _ in range(3))
        if noalloc:
            arl2.read_noalloc(sh, dq, dk, dv, dphi, dS, o, oi, oe)
        else:
            arl2.read(sh, dq, dk, dv, dphi, dS, o, oi, oe,
                      ws=arl2.alloc_workspace(sh, arl2.OP_READ))
        outs.append((o, oi, oe))
    torch.cuda.synchronize()
    return outs, oracle.read(q, k, v, phi, S)


# (dtype, B, H, T, D) pairs: a first call, then a smaller one
PAIRS = [
    (("bf16", 1, 3, 300, 128), ("bf16", 1, 2, 100, 128)),
    (("bf16", 1, 12, 1560, 128), ("bf16", 1, 1, 37, 128)),
    (("f32", 1, 2, 130, 64), ("f32", 1, 1, 37, 16)),
    (("bf16", 2, 3, 200, 64), ("bf16", 1, 1, 1, 16)),
]


def _w(dtype, B, H, T, D):
    base = synth.WORKLOADS[0] if dtype == "f32" else synth.WORKLOADS[1]
    return base.replace(B=B, H=H, T=T, D=D)


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: "{}-B{}H{}T{}D{}".format(*p[0]))
def test_read_noalloc_matches_read(pair):
    import torch
    for call, case in enumerate(pair):
        w = _w(*case)
        log(f"read_noalloc call {call}: {case}")
        (mine, theirs), ref = _both(w, frame=call)
        for name, x, y in zip(("o", "o_intra", "o_inter"), mine, theirs):
            assert torch.equal(x, y), f"call {call}: {name} differs from arl2_read"
            assert_close(host(x), ref[name], TOL[w.dtype], f"call {call} {name}")


def test_read_noalloc_refuses_beyond_its_scratch():
    import torch
    from hybrid_linear_memory_amd import arl2
    # bf16 D = 128 needs B*H*D*D*2 bytes of scratch for the map: 300 heads is
    # 9.8 MB, above the fixed 8 MiB
    sh = arl2.Shape(1, 300, 8, 128, arl2.BF16)
    assert 300 * 128 * 128 * 2 > arl2.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((1, 300, 8, 128), dtype=torch.bfloat16, device="cuda")
    phi = torch.zeros((300, 128, 128), dtype=torch.bfloat16, device="cuda")
    S = torch.zeros((1, 300, 128, 128), dtype=torch.float32, device="cuda")
    o = torch.full_like(x, 3.0)
    with pytest.raises(arl2.Arl2Error, match="scratch"):
        arl2.read_noalloc(sh, x, x, x, phi, S, o)
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()), "refused call wrote its output"
