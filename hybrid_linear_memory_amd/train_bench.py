"""Time of the training-side calls on one layer's shapes.

    python -m hybrid_linear_memory_amd.train_bench [--B 1] [--H 12] [--T 1560] [--iters 20]

Measures, with HIP events around back-to-back calls on one stream, the
forward read (arl2_read) and commit (arl2_commit) beside their backward calls
(arl2_read_backward, arl2_commit_backward), the intra-frame attention
backward alone (arl2_intra_attn_backward), the same backward calls given the
rows' log-sum-exp by the forward (arl2_intra_attn_lse, timed too), and the
clean-state scan over 21 frames (arl2_state_scan). bf16 activations, fp32 state, seeded synthetic
inputs resident in HBM. The attention backward's algorithmic work is counted
as the five T x T x d products of its definition (S, dP, dV, dQ, dK:
10 T^2 d FLOP per head); the kernels recompute S for the log-sum-exp pass and
S, dP once more so that no accumulation crosses workgroups (16 T^2 d; 14 when
the log-sum-exp comes from the forward).
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--B", type=int, default=1)
    ap.add_argument("--H", type=int, default=12)
    ap.add_argument("--T", type=int, default=1560)
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--frames", type=int, default=21)
    args = ap.parse_args(argv)

    import torch

    from . import arl2

    assert torch.cuda.is_available(), "train_bench needs a GPU"
    sh = arl2.Shape(args.B, args.H, args.T, 128, arl2.BF16)
    B, H, T, D = sh.B, sh.H, sh.T, sh.D
    g = torch.Generator(device="cuda").manual_seed(0)

    def rnd(*s, scale=1.0, dtype=torch.bfloat16):
        return (torch.randn(*s, generator=g, device="cuda") * scale).to(dtype)

    act = (B, H, T, D)
    q, k, v, d_o = (rnd(*act) for _ in range(4))
    k = torch.nn.functional.normalize(k.float(), dim=-1).to(torch.bfloat16)
    phis = [rnd(H, D, D, scale=D ** -0.5) for _ in range(3)]
    beta = torch.sigmoid(torch.randn(B, H, T, generator=g, device="cuda")) / T
    alpha = torch.sigmoid(torch.randn(B, H, generator=g, device="cuda") * 0.5 + 3.0)
    S = rnd(B, H, D, D, scale=0.05, dtype=torch.float32)
    G = rnd(B, H, D, D, dtype=torch.float32)
    zf = dict(dtype=torch.float32, device="cuda")
    o, o_intra = torch.empty(act, dtype=torch.bfloat16, device="cuda"), torch.empty(
        act, dtype=torch.bfloat16, device="cuda")
    dq, dk, dv = (torch.zeros(act, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    dphi = [torch.zeros((H, D, D), **zf) for _ in range(3)]
    dS, dS_prev, S_next = (torch.zeros((B, H, D, D), **zf) for _ in range(3))
    dbeta, dalpha = torch.zeros((B, H, T), **zf), torch.zeros((B, H), **zf)
    ws = torch.empty(max(arl2.workspace_bytes(sh, op) for op in
                         (arl2.OP_READ, arl2.OP_COMMIT, arl2.OP_READ_BACKWARD,
                          arl2.OP_COMMIT_BACKWARD, arl2.OP_INTRA_ATTN_BACKWARD)),
                     dtype=torch.uint8, device="cuda")
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    arl2.intra_attn_lse(sh, q, k, v, o_intra, lse)

    calls = {
        "read": lambda: arl2.read(sh, q, k, v, phis[0], S, o, None, None, ws),
        "commit": lambda: arl2.commit(sh, k, v, phis[1], phis[2], beta, alpha, S, S_next, ws),
        "intra_attn_backward": lambda: arl2.intra_attn_backward(sh, q, k, v, o_intra, d_o, dq, dk,
                                                                dv, ws=ws),
        "read_backward": lambda: arl2.read_backward(sh, q, k, v, phis[0], S, o_intra, d_o, dq, dk,
                                                    dv, dphi[0], dS, ws=ws),
        # with the rows' log-sum-exp from the forward (no pass to recompute it)
        "intra_attn_lse": lambda: arl2.intra_attn_lse(sh, q, k, v, o_intra, lse),
        "intra_attn_backward_lse": lambda: arl2.intra_attn_backward(sh, q, k, v, o_intra, d_o, dq,
                                                                    dk, dv, ws=ws, lse=lse),
        "read_backward_lse": lambda: arl2.read_backward(sh, q, k, v, phis[0], S, o_intra, d_o, dq,
                                                        dk, dv, dphi[0], dS, ws=ws, lse=lse),
        "commit_backward": lambda: arl2.commit_backward(sh, k, v, phis[1], phis[2], beta, alpha, S,
                                                        G, dk, dv, dphi[1], dphi[2], dbeta,
                                                        dalpha, dS_prev, ws=ws),
    }
    res = {}
    for name, fn in calls.items():
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name + "_us"] = e0.elapsed_time(e1) * 1000.0 / args.iters
    # clean-state scan over F frames
    F = args.frames
    ks = torch.stack([k] * F).contiguous()
    vs = torch.stack([v] * F).contiguous()
    betas = torch.stack([beta] * F).contiguous()
    alphas = torch.stack([alpha] * F).contiguous()
    states = torch.empty((F + 1, B, H, D, D), **zf)
    wsc = arl2.alloc_workspace(sh, arl2.OP_COMMIT)
    for _ in range(2):
        arl2.state_scan(sh, ks, vs, phis[1], phis[2], betas, alphas, S, states, wsc)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        arl2.state_scan(sh, ks, vs, phis[1], phis[2], betas, alphas, S, states, wsc)
    e1.record()
    torch.cuda.synchronize()
    res["state_scan_us_per_frame"] = e0.elapsed_time(e1) * 1000.0 / 5 / F
    heads = B * H
    alg = 10.0 * T * T * D * heads
    res["intra_attn_backward_tflops_algorithmic"] = alg / (res["intra_attn_backward_us"] * 1e-6) / 1e12
    res["intra_attn_backward_tflops_executed"] = 1.6 * res["intra_attn_backward_tflops_algorithmic"]
    res["intra_attn_backward_frac_of_bf16_peak"] = res["intra_attn_backward_tflops_algorithmic"] / 2500.0
    res["intra_attn_backward_lse_tflops_algorithmic"] = (
        alg / (res["intra_attn_backward_lse_us"] * 1e-6) / 1e12)
    out = {"workload": f"{B} x {H} heads x 128, T={T}, bf16 activations, fp32 state", **{
        key: round(val, 3) for key, val in res.items()}}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
