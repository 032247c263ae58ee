"""Time and attention-state memory of a 30-layer stack against video length.

    python -m hybrid_linear_memory_amd.stack_bench [--fractions 0,0.5,0.75,1]
        [--video-frames 81,161,321,641,921] [--layers 30] [--reps 2]

The stack (``stack.HybridStack``) has the attention shape of the model the
summary evaluates (1.3B, 30 attention layers, 12 heads of 128, 1560 tokens per
latent frame; §4) with a fraction of its layers replaced by ARL2 layers, spread
evenly; the others keep softmax attention over a KV cache. A step is one
generated latent frame: 4 denoising passes and the clean pass through every
layer. For each video length the softmax layers' caches are positioned at the
number of latent frames already generated, 1 + (video frames - 1) / 4 (the
4x temporal compression of the model's VAE; 81 video frames = 21 latent
frames), and the time of one frame is measured there; the attention state is
what the layers hold at that point (caches plus the ARL2 layers' fixed state).

Inputs are seeded synthetic tensors resident in HBM (a small pool cycled over
layers and passes); the softmax layers share one cache buffer, which leaves
their work unchanged (the memory column counts one cache per layer). Only
attention is measured: no projections, MLPs or VAE. Prints one JSON line per
(fraction, length) and a table.
"""
from __future__ import annotations

import argparse
import json
import sys
import time


def _mask(fraction: float, n_layers: int):
    return [int((l + 1) * fraction) > int(l * fraction) for l in range(n_layers)]


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--fractions", default="0,0.5,0.75,1")
    ap.add_argument("--video-frames", default="81,161,321,641,921")
    ap.add_argument("--layers", type=int, default=30)
    ap.add_argument("--reps", type=int, default=2, help="timed frames per point")
    ap.add_argument("--pool", type=int, default=6, help="distinct resident input sets")
    args = ap.parse_args(argv)

    import torch

    from . import arl2
    from .stack import HybridStack

    assert torch.cuda.is_available(), "stack_bench needs a GPU"
    fractions = [float(x) for x in args.fractions.split(",")]
    videos = [int(x) for x in args.video_frames.split(",")]
    latents = [1 + (v - 1) // 4 for v in videos]
    shape = arl2.Shape(1, 12, 1560, 128, arl2.BF16)
    g = torch.Generator(device="cuda").manual_seed(0)
    dims = (shape.B, shape.H, shape.T, shape.D)

    def rnd(*s, scale=1.0, dtype=torch.bfloat16):
        return (torch.randn(*s, generator=g, device="cuda") * scale).to(dtype)

    pool = [tuple(rnd(*dims) for _ in range(3)) for _ in range(args.pool)]
    beta = torch.sigmoid(torch.randn(shape.B, shape.H, shape.T, generator=g, device="cuda")) / shape.T
    alpha = torch.sigmoid(torch.randn(shape.B, shape.H, generator=g, device="cuda") * 0.5 + 3.0)
    rows = []
    for frac in fractions:
        mask = _mask(frac, args.layers)
        phis = [tuple(rnd(shape.H, shape.D, shape.D, scale=shape.D ** -0.5) for _ in range(3))
                if m else None for m in mask]
        stack = HybridStack(shape, mask, phis, max_frames=max(latents) + 1, shared_cache=True)
        gates = [(beta, alpha)] * args.layers
        softmax_layers = [lay for lay, m in zip(stack.layers, mask) if not m]
        passes = 5

        def one_frame(n):
            for lay in softmax_layers:
                lay.frame = n
            for p in range(passes):
                inputs = [pool[(l + p) % len(pool)] for l in range(args.layers)]
                if p < passes - 1:
                    stack.read(inputs)
                else:
                    stack.clean_pass(inputs, gates)

        for v, n in zip(videos, latents):
            print(f"[stack] fraction {frac} video frames {v} (latent {n})", file=sys.stderr,
                  flush=True)
            one_frame(n)                                   # warm-up
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            w0 = time.perf_counter()
            e0.record()
            for _ in range(args.reps):
                one_frame(n)
            e1.record()
            torch.cuda.synchronize()
            wall = time.perf_counter() - w0
            ms = max(e0.elapsed_time(e1) / 1e3, wall) / args.reps * 1e3
            row = {"replaced_fraction": frac, "arl2_layers": sum(mask),
                   "softmax_layers": args.layers - sum(mask), "video_frames": v,
                   "latent_frames": n, "ms_per_latent_frame": ms,
                   "attention_state_bytes": stack.state_bytes(frames=n)}
            rows.append(row)
            print(json.dumps(row), flush=True)
        del stack
        torch.cuda.empty_cache()
    # table
    print("\n| replaced | video frames | latent frames | ms per latent frame | attention state GB |")
    print("|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['replaced_fraction']:.0%} | {r['video_frames']} | {r['latent_frames']} | "
              f"{r['ms_per_latent_frame']:.2f} | {r['attention_state_bytes'] / 1e9:.2f} |")
    return rows


if __name__ == "__main__":
    main()
