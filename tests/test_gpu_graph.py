"""The layer's frame loop captured in a HIP graph (as bench.py times it) gives
exactly the results of the same calls issued eagerly, on every replay.

A graph of two frames (denoising reads, then the clean pass, which commits
and forms the next frame's map) is captured once and replayed three times,
with eager work and synchronisations between the replays; each replay
continues the rollout from the state the previous one left. An eager layer
runs the same six frames; every output and the state after every replay must
match bit for bit (same kernels, same inputs, fixed reduction order).
"""
import numpy as np
import pytest

from gpu_helpers import dev, dev32, log, shape_of
from hybrid_linear_memory_amd import synth

pytestmark = pytest.mark.gpu


# (4, 4096): the reads take the split-key grid, whose per-call counter tags
# are fixed in the graph (each replay must still leave every counter at 0)
@pytest.mark.parametrize("H,T", [(2, 300), (12, 1560), (4, 4096)])
def test_layer_graph_replays_match_eager(H, T):
    import torch
    from hybrid_linear_memory_amd.layer import Arl2Layer
    assert torch.cuda.is_available()
    w = synth.WORKLOADS[1].replace(H=H, T=T, frames=2, n_denoise=2)
    log(f"graph replay H{H} T{T}")
    sh = shape_of(w)
    phis = [dev(p, w.dtype) for p in synth.phi_maps(w)]
    frames = []
    for f in range(w.frames):
        beta, alpha = synth.gates(w, f)
        frames.append(([tuple(dev(x, w.dtype) for x in synth.qkv(w, f, p))
                        for p in range(w.passes)], dev32(beta), dev32(alpha)))
    n_out = w.frames * w.passes

    def run(layer, outs):
        i = 0
        for passes, beta, alpha in frames:
            for p, (q, k, v) in enumerate(passes):
                if p < w.passes - 1:
                    layer.read(q, k, v, o=outs[i])
                else:
                    layer.clean_pass(q, k, v, beta, alpha, o=outs[i])
                i += 1

    lg = Arl2Layer(sh, *phis)
    le = Arl2Layer(sh, *phis)
    outs_g = [lg.new_output() for _ in range(n_out)]
    outs_e = [le.new_output() for _ in range(n_out)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(lg, outs_g)                 # warm-up on the capture stream
    torch.cuda.synchronize()
    lg.reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        run(lg, outs_g)
    # two frames bring the double buffers back to where the capture began
    assert lg._cur == 0 and lg._mcur == 0
    scratch = torch.zeros(1 << 20, device="cuda")
    for rep in range(3):
        graph.replay()
        scratch.add_(1.0)                # eager work between replays
        torch.cuda.synchronize()
        run(le, outs_e)
        torch.cuda.synchronize()
        for i in range(n_out):
            assert torch.equal(outs_g[i], outs_e[i]), f"replay {rep} output {i}"
        assert torch.equal(lg.S, le.S), f"replay {rep} state"
        assert torch.equal(lg.M, le.M), f"replay {rep} prepared map"
        assert float(scratch[0]) == rep + 1.0
    assert np.isfinite(lg.S.cpu().numpy()).all()
