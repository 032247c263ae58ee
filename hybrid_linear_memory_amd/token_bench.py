"""Frame time under token-level versus frame-level access.

    python -m hybrid_linear_memory_amd.token_bench [--B 8] [--H 12] [--T 1560]
        [--frames 21] [--reps 3]

The summary's ablation (§4) compares frame-level access (every token of frame
N reads S_{N-1}) with token-level access (each token reads the state updated by
the frame's earlier tokens) on quality; this measures what each costs on the
GPU. One step is one generated frame of one layer: the denoising reads and the
clean pass (4 + 1 passes), over B streams of H heads of 128 and T tokens,
bf16 activations, fp32 state, seeded synthetic inputs resident in HBM (a small
pool cycled over passes), beta = sigmoid(N(0,1)) / T, alpha = sigmoid(N(3,0.5)).

Frame-level access runs the library's fast path (prepared reads, one-launch
clean pass); token-level access runs arl2_token_read / arl2_token_clean_pass
(feature maps, intra-frame attention, per-chunk triangular solve, sequential
chunk scan). Prints one JSON line per access mode and the ratio.
"""
from __future__ import annotations

import argparse
import json


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--B", type=int, default=8)
    ap.add_argument("--H", type=int, default=12)
    ap.add_argument("--T", type=int, default=1560)
    ap.add_argument("--frames", type=int, default=21, help="frames per timed rollout")
    ap.add_argument("--reps", type=int, default=3, help="timed rollouts (best is reported)")
    ap.add_argument("--n-denoise", type=int, default=4)
    ap.add_argument("--pool", type=int, default=6)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one 1 GiB device-to-device copy (a known-size reference "
                         "for rocprofv3 FETCH_SIZE / WRITE_SIZE runs)")
    args = ap.parse_args(argv)

    import torch

    from . import arl2
    from .layer import Arl2Layer

    assert torch.cuda.is_available(), "token_bench needs a GPU"
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    shape = arl2.Shape(args.B, args.H, args.T, 128, arl2.BF16)
    dims = (shape.B, shape.H, shape.T, shape.D)
    g = torch.Generator(device="cuda").manual_seed(0)

    def rnd(*s, scale=1.0):
        return (torch.randn(*s, generator=g, device="cuda") * scale).to(torch.bfloat16)

    pool = [tuple(rnd(*dims) for _ in range(3)) for _ in range(args.pool)]
    phis = [rnd(shape.H, shape.D, shape.D, scale=shape.D ** -0.5) for _ in range(3)]
    beta = torch.sigmoid(torch.randn(shape.B, shape.H, shape.T, generator=g, device="cuda")) / shape.T
    alpha = torch.sigmoid(torch.randn(shape.B, shape.H, generator=g, device="cuda") * 0.5 + 3.0)
    passes = args.n_denoise + 1
    results = {}
    for access in ("frame", "token"):
        layer = Arl2Layer(shape, *phis, n_denoise=args.n_denoise, access=access)
        o = layer.new_output()
        step = [0]

        def frame():
            for p in range(passes):
                q, k, v = pool[(step[0] + p) % len(pool)]
                if p < passes - 1:
                    layer.read(q, k, v, o=o, beta=beta if access == "token" else None)
                else:
                    layer.clean_pass(q, k, v, beta, alpha, o=o)
            step[0] += 1

        for _ in range(3):
            frame()
        best = None
        for _ in range(args.reps):
            layer.reset()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(args.frames):
                frame()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.frames
            best = ms if best is None else min(best, ms)
        results[access] = best
        line = {"access": access, "workload": f"{shape.B}x{shape.H} heads x 128, T={shape.T}",
                "passes_per_frame": passes, "ms_per_frame": round(best, 4),
                "frames_per_s": round(1000.0 / best, 2),
                "tokens_per_s": round(1000.0 / best * shape.B * shape.T, 0)}
        print(json.dumps(line), flush=True)
        del layer
    print(json.dumps({"token_over_frame_time": round(results["token"] / results["frame"], 3)}),
          flush=True)


if __name__ == "__main__":
    main()
