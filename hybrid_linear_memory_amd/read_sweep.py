"""Time of the denoising read (arl2_read_prepared) across shapes.

    python -m hybrid_linear_memory_amd.read_sweep [--iters 200]

For each (B, H, T) at d = 128 the fused read runs back to back on one stream
over a pool of resident inputs (at least 512 MB, so that they come from HBM),
timed with HIP events; with a workspace, so that the shapes that take the
split-key grid do. Inputs follow the synthetic workloads' recipe: Q, K, V
standard normal, keys L2-normalised row by row. Algorithmic work per launch: 4 T^2 d (Q K^T and P V) plus
2 T d^2 (Q M) FLOP per head; the fraction is of the dense bf16 MFMA peak
(2.5 PFLOP/s). One JSON line per shape.
"""
from __future__ import annotations

import argparse
import json

SHAPES = [(1, 12, 1560), (1, 12, 3600), (1, 12, 6240), (2, 12, 1560), (4, 12, 1560),
          (8, 12, 1560), (1, 40, 1560), (1, 4, 4096), (1, 2, 8192)]
PEAK = 2.5e15


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--iters", type=int, default=200)
    args = ap.parse_args(argv)

    import torch

    from . import arl2
    assert torch.cuda.is_available(), "read_sweep needs a GPU"
    for B, H, T in SHAPES:
        sh = arl2.Shape(B, H, T, 128, arl2.BF16)
        g = torch.Generator(device="cuda").manual_seed(0)
        per_set = 3 * B * H * T * 128 * 2
        n_sets = max(2, -(-(512 << 20) // per_set))
        def qkv():
            q, k, v = (torch.randn(B, H, T, 128, generator=g, device="cuda") for _ in range(3))
            k = k / k.norm(dim=-1, keepdim=True)     # keys L2-normalised per row, as generated
            return tuple(x.to(torch.bfloat16) for x in (q, k, v))

        sets = [qkv() for _ in range(n_sets)]
        M = arl2.alloc_prepared(sh)
        phi = (torch.randn(H, 128, 128, generator=g, device="cuda") * 128 ** -0.5).to(
            torch.bfloat16)
        arl2.read_prepare(sh, phi, torch.randn(B, H, 128, 128, generator=g, device="cuda") * 0.05,
                          M)
        o = torch.empty(B, H, T, 128, dtype=torch.bfloat16, device="cuda")
        ws = arl2.alloc_workspace(sh, arl2.OP_READ_PREPARED)
        split = arl2.workspace_bytes(sh, arl2.OP_READ_PREPARED) > 0
        iters = max(20, args.iters * 1560 * 12 // (T * H * B))
        # warm-up as long as the timed run (clocks settle under sustained load)
        for i in range(iters):
            arl2.read_prepared(sh, *sets[i % n_sets], M, o, ws=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(iters):
            arl2.read_prepared(sh, *sets[i % n_sets], M, o, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / iters
        flop = B * H * (4.0 * T * T * 128 + 2.0 * T * 128 * 128)
        print(json.dumps({"B": B, "H": H, "T": T, "split_key_grid": split,
                          "query_blocks": B * H * (-(-T // 128)), "us": round(us, 2),
                          "tflops": round(flop / us / 1e6, 1),
                          "frac_of_bf16_peak": round(flop / (us * 1e-6) / PEAK, 4)}), flush=True)
        del sets


if __name__ == "__main__":
    main()
