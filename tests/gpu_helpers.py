"""Shared helpers of the GPU parity tests: device transfer, tolerance checks
and a lock-step rollout that drives the HIP path and the fp64 oracle on the
same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from hybrid_linear_memory_amd import synth

TOL = {"f32": 1e-4, "bf16": 2e-2}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x, dtype_name: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    return t.to("cuda").to(dt).contiguous()


def dev32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").contiguous()


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_rel_err(got, ref) -> tuple[float, float]:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref))), float(np.max(np.abs(ref)))


def assert_close(got, ref, rel: float, name: str):
    err, scale = max_rel_err(got, ref)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert err <= rel * scale, f"{name}: max|err| {err:.3e} > {rel:g} * max|ref| {scale:.3e}"
    return err / scale if scale > 0 else 0.0


def shape_of(w: synth.Workload):
    from hybrid_linear_memory_amd import arl2
    return arl2.Shape(w.B, w.H, w.T, w.D, arl2.BF16 if w.dtype == "bf16" else arl2.F32)


def lockstep_rollout(w: synth.Workload, read_frames, row_sample=None, check_state=True,
                     frames=None, commit_via="commit", clean_rows=None, full_every=1,
                     **layer_kwargs):
    """Drive Arl2Layer and the oracle frame by frame.

    Frames in ``read_frames`` run every denoising read and the clean pass, and
    their outputs (o, o_intra, o_inter) are compared on ``row_sample`` query
    rows (all rows if None). Other frames write the state without the
    denoising reads: with ``commit_via="commit"`` through the commit-only call
    (reads never change the state, so the state trajectory is the same); with
    ``commit_via="clean_pass"`` through the layer's clean pass, whose outputs
    are compared on every row on every ``full_every``-th frame and on
    ``clean_rows`` rows (all rows if None) on the others. The state is compared
    after every commit. Returns the worst relative errors seen."""
    import torch
    from hybrid_linear_memory_amd.layer import Arl2Layer

    if commit_via not in ("commit", "clean_pass"):
        raise ValueError(commit_via)
    tol = TOL[w.dtype]
    phis = synth.phi_maps(w)
    layer = Arl2Layer(shape_of(w), *[dev(p, w.dtype) for p in phis], **layer_kwargs)
    S_ref = np.zeros((w.B, w.H, w.D, w.D))
    worst = {"S": 0.0, "o": 0.0, "o_intra": 0.0, "o_inter": 0.0}
    n_frames = w.frames if frames is None else frames

    def _compare(o, o_i, o_e, q, k, v, rows, what):
        sel = slice(None) if rows is None else np.asarray(rows)
        ref = oracle.read(q[:, :, sel], k, v, phis[0], S_ref)
        got = {"o": host(o)[:, :, sel], "o_intra": host(o_i)[:, :, sel],
               "o_inter": host(o_e)[:, :, sel]}
        for name in ("o", "o_intra", "o_inter"):
            r = assert_close(got[name], ref[name], tol, f"{what} {name}")
            worst[name] = max(worst[name], r)

    for f in range(n_frames):
        beta, alpha = synth.gates(w, f)
        if f in read_frames:
            for p in range(w.passes):
                q, k, v = synth.qkv(w, f, p)
                o_i = layer.new_output()
                o_e = layer.new_output()
                if p < w.passes - 1:
                    o = layer.read(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype),
                                   o_intra=o_i, o_inter=o_e)
                else:
                    o = layer.clean_pass(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype),
                                         dev32(beta), dev32(alpha), o_intra=o_i, o_inter=o_e)
                _compare(o, o_i, o_e, q, k, v, row_sample, f"frame {f} pass {p}")
            kc, vc = k, v                      # the clean pass's keys and values
        elif commit_via == "clean_pass":
            q, kc, vc = synth.qkv(w, f, w.passes - 1)
            o_i = layer.new_output()
            o_e = layer.new_output()
            o = layer.clean_pass(dev(q, w.dtype), dev(kc, w.dtype), dev(vc, w.dtype),
                                 dev32(beta), dev32(alpha), o_intra=o_i, o_inter=o_e)
            rows = None if f % full_every == 0 or f == n_frames - 1 else clean_rows
            _compare(o, o_i, o_e, q, kc, vc, rows, f"frame {f} clean pass")
        else:
            kc, vc = synth.kv(w, f, w.passes - 1)
            layer.commit(dev(kc, w.dtype), dev(vc, w.dtype), dev32(beta), dev32(alpha))
        S_ref = oracle.commit(kc, vc, phis[1], phis[2], beta, alpha, S_ref)
        if check_state:
            torch.cuda.synchronize()
            r = assert_close(host(layer.S), S_ref, tol, f"frame {f} state")
            worst["S"] = max(worst["S"], r)
    return worst
