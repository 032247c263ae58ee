"""Training-side driver: gradients of a rollout of one ARL2 layer through the
frame recurrence, on the library's backward calls.

The summary's two-stage distillation (§2.3) fine-tunes the hybrid model end
to end; a loss on the outputs of several frames reaches each frame's read
(arl2_read_backward) and, through the state, every earlier commit
(arl2_commit_backward). Frame f's reads use S_f and its clean pass commits
S_{f+1}; with G = dL/dS_{f+1} the frames are visited backwards: the commit's
backward turns G into its share of dL/dS_f, and the frame's reads add theirs.
All gradients accumulate in place (accumulate = 1) into zeroed buffers.
"""
from __future__ import annotations

import torch

from . import arl2


def workspace(shape: arl2.Shape, device=None) -> torch.Tensor:
    """One workspace large enough for every call of the driver."""
    n = max(arl2.workspace_bytes(shape, op) for op in
            (arl2.OP_READ_BACKWARD, arl2.OP_COMMIT_BACKWARD, arl2.OP_COMMIT,
             arl2.OP_INTRA_ATTN_BACKWARD))
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device or "cuda")


def rollout_states(shape: arl2.Shape, frames, phi_k, phi_v, S0=None, ws=None, stream=None):
    """S_0..S_F committed by the frames' clean passes (frames[f]["passes"][-1]
    holds the clean pass's q, k, v)."""
    dev = frames[0]["passes"][-1][1].device
    ws = workspace(shape, dev) if ws is None else ws
    st = (shape.B, shape.H, shape.D, shape.D)
    states = [torch.zeros(st, dtype=torch.float32, device=dev) if S0 is None else S0]
    for fr in frames:
        _, kc, vc = fr["passes"][-1]
        nxt = torch.empty(st, dtype=torch.float32, device=dev)
        arl2.commit(shape, kc, vc, phi_k, phi_v, fr["beta"], fr["alpha"], states[-1], nxt, ws,
                    stream)
        states.append(nxt)
    return states


def rollout_backward(shape: arl2.Shape, frames, phi_q, phi_k, phi_v, d_outputs, S0=None,
                     dS_final=None, stream=None) -> dict:
    """Gradients of a loss whose gradient with respect to the output of pass
    p of frame f is d_outputs[(f, p)] (passes without an entry take none) and
    with respect to the final state is dS_final (default none).

    Returns "d_passes"[(f, p)] = (dq, dk, dv), "dbeta"[f], "dalpha"[f],
    "dphi_q", "dphi_k", "dphi_v" (float32 [H, D, D]) and "dS0"."""
    dev = frames[0]["passes"][-1][1].device
    ws = workspace(shape, dev)
    states = rollout_states(shape, frames, phi_k, phi_v, S0, ws, stream)
    a = shape.torch_dtype
    B, H, T, D = shape.B, shape.H, shape.T, shape.D
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"d_passes": {}, "dbeta": {}, "dalpha": {},
           "dphi_q": torch.zeros((H, D, D), **f32), "dphi_k": torch.zeros((H, D, D), **f32),
           "dphi_v": torch.zeros((H, D, D), **f32)}
    G = torch.zeros((B, H, D, D), **f32) if dS_final is None else dS_final.clone()
    G2 = torch.zeros_like(G)
    o_intra = torch.empty((B, H, T, D), dtype=a, device=dev)
    lse = torch.empty((B, H, T), **f32)
    for f in range(len(frames) - 1, -1, -1):
        fr = frames[f]
        grads = [tuple(torch.zeros((B, H, T, D), dtype=a, device=dev) for _ in range(3))
                 for _ in fr["passes"]]
        out["dbeta"][f] = torch.zeros((B, H, T), **f32)
        out["dalpha"][f] = torch.zeros((B, H), **f32)
        G2.zero_()
        _, kc, vc = fr["passes"][-1]
        _, dkc, dvc = grads[-1]
        arl2.commit_backward(shape, kc, vc, phi_k, phi_v, fr["beta"], fr["alpha"], states[f], G,
                             dkc, dvc, out["dphi_k"], out["dphi_v"], out["dbeta"][f],
                             out["dalpha"][f], G2, accumulate=True, ws=ws, stream=stream)
        for p, (q, k, v) in enumerate(fr["passes"]):
            if (f, p) not in d_outputs:
                continue
            dq, dk, dv = grads[p]
            arl2.intra_attn_lse(shape, q, k, v, o_intra, lse, stream)
            arl2.read_backward(shape, q, k, v, phi_q, states[f], o_intra, d_outputs[(f, p)], dq,
                               dk, dv, out["dphi_q"], G2, accumulate=True, ws=ws, stream=stream,
                               lse=lse)
        for p, g in enumerate(grads):
            out["d_passes"][(f, p)] = g
        G, G2 = G2, G
    out["dS0"] = G
    return out
