"""Seeded synthetic inputs for the ARL2 hybrid attention step.

This module generates inputs only; it holds none of the method's arithmetic.
Both the HIP path (bench, tests) and the fp64 oracle consume exactly the
arrays produced here: bf16 workloads are rounded to bf16 here (round to
nearest even) and handed over as float32 arrays whose values are exactly
bf16-representable, so the GPU sees the same numbers the oracle upcasts.

Workload shapes follow the model the ARL2 pages evaluate (a 1.3B
autoregressive video diffusion model, 480p, 30x52 latent = 1560 tokens per
frame, 12 heads of 128; ARL2 summary §4): the pages measure on VBench, and
these seeded Gaussian tensors stand in for it. Five workloads:

  0 tiny_fp32    1 x 1 x 16, T=64, 8 frames, 1 read + clean pass, fp32,
                 phi = I + 0.1 N(0,1), alpha ~ sigmoid(N(2, 0.5))
  1 wan13b       1 x 12 x 128, T=1560, 21 frames, 4 reads + clean pass, bf16
  2 long         workload 1 over 240 frames (plus the full-KV comparator)
  3 batched      8 x 12 x 128, T=1560, 21 frames, bf16
  4 large        1 x 40 x 128, T=1560, 81 frames, bf16

For all: Q, K, V ~ N(0, 1) with K rows L2-normalised (in fp32, before bf16
rounding), beta = sigmoid(N(0, 1)) / T per (video, head, token), alpha per
(video, head, frame), phi ~ N(0, 1/d) dense d x d per head for the bf16
workloads. Every tensor is drawn from its own PCG64 stream keyed by
(seed, workload id, frame, pass, tensor id), so any frame regenerates alone.
"""
from __future__ import annotations

import dataclasses

import numpy as np

# tensor ids of the per-stream seeds
_Q, _K, _V, _BETA, _ALPHA, _PHI_Q, _PHI_K, _PHI_V = range(8)
_STATIC_FRAME = 1 << 20   # frame key of the per-layer (not per-frame) tensors


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    B: int
    H: int
    D: int
    T: int
    frames: int
    n_denoise: int
    dtype: str                 # "f32" or "bf16" (activations); state is fp32
    alpha_mu: float
    alpha_sigma: float
    phi_kind: str              # "identity_plus" or "gaussian"
    seed: int = 0

    @property
    def passes(self) -> int:
        return self.n_denoise + 1

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    0: Workload(0, "tiny_fp32", 1, 1, 16, 64, 8, 1, "f32", 2.0, 0.5, "identity_plus"),
    1: Workload(1, "wan13b_layer", 1, 12, 128, 1560, 21, 4, "bf16", 3.0, 0.5, "gaussian"),
    2: Workload(2, "long_rollout", 1, 12, 128, 1560, 240, 4, "bf16", 3.0, 0.5, "gaussian"),
    3: Workload(3, "batched_streams", 8, 12, 128, 1560, 21, 4, "bf16", 3.0, 0.5, "gaussian"),
    4: Workload(4, "large_model", 1, 40, 128, 1560, 81, 4, "bf16", 3.0, 0.5, "gaussian"),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32
    holding exactly bf16-representable values. Finite inputs only."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite values never carry out of 32 bits here (max 0xFF7FFFFF + 0x8000)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(x.shape)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of bf16-representable float32 values, as uint16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def rng(w: Workload, frame: int, pass_: int, tensor: int) -> np.random.Generator:
    ss = np.random.SeedSequence([w.seed, w.wid, frame, pass_, tensor])
    return np.random.Generator(np.random.PCG64(ss))


def _cast(w: Workload, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return bf16_round(x) if w.dtype == "bf16" else x


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.einsum("...i,...i->...", x, x))[..., None]
    return (x / np.maximum(n, np.float32(1e-30))).astype(np.float32)


def qkv(w: Workload, frame: int, pass_: int, rows=None):
    """Q, K, V of one pass of one frame: float32 [B, H, T, D].

    Keys are L2-normalised row by row before rounding, as the workloads
    specify. ``rows`` (optional slice or index array over T) returns only those
    query rows of Q (K and V always whole)."""
    shape = (w.B, w.H, w.T, w.D)
    q = rng(w, frame, pass_, _Q).standard_normal(shape, dtype=np.float32)
    k = rng(w, frame, pass_, _K).standard_normal(shape, dtype=np.float32)
    v = rng(w, frame, pass_, _V).standard_normal(shape, dtype=np.float32)
    k = _unit_rows(k)
    if rows is not None:
        q = q[:, :, rows, :]
    return _cast(w, q), _cast(w, k), _cast(w, v)


def kv(w: Workload, frame: int, pass_: int):
    """K, V only (the clean pass's commit inputs), float32 [B, H, T, D]."""
    shape = (w.B, w.H, w.T, w.D)
    k = rng(w, frame, pass_, _K).standard_normal(shape, dtype=np.float32)
    v = rng(w, frame, pass_, _V).standard_normal(shape, dtype=np.float32)
    return _cast(w, _unit_rows(k)), _cast(w, v)


def gates(w: Workload, frame: int):
    """beta [B, H, T] = sigmoid(N(0,1)) / T and alpha [B, H] =
    sigmoid(N(mu, sigma)), float32."""
    b = rng(w, frame, 0, _BETA).standard_normal((w.B, w.H, w.T))
    a = rng(w, frame, 0, _ALPHA).normal(w.alpha_mu, w.alpha_sigma, (w.B, w.H))
    beta = (_sigmoid(b) / w.T).astype(np.float32)
    alpha = _sigmoid(a).astype(np.float32)
    return beta, alpha


def phi_maps(w: Workload):
    """phi_q, phi_k, phi_v: float32 [H, D, D] (d_in rows, d_out columns)."""
    out = []
    for t in (_PHI_Q, _PHI_K, _PHI_V):
        g = rng(w, _STATIC_FRAME, 0, t).standard_normal((w.H, w.D, w.D))
        if w.phi_kind == "identity_plus":
            m = np.eye(w.D)[None] + 0.1 * g
        else:
            m = g / np.sqrt(w.D)
        out.append(_cast(w, m.astype(np.float32)))
    return tuple(out)


def frame_passes(w: Workload, frame: int):
    """All passes (q, k, v) of a frame; the last one is the clean pass."""
    return [qkv(w, frame, p) for p in range(w.passes)]


def oracle_frame(w: Workload, frame: int, with_reads: bool = True):
    """A frame in the form the oracle's rollout takes. With ``with_reads``
    False only the clean pass is materialised (denoising reads never change
    the state, so the state trajectory needs only the clean passes)."""
    beta, alpha = gates(w, frame)
    if with_reads:
        passes = frame_passes(w, frame)
    else:
        passes = [qkv(w, frame, w.passes - 1)]
    return {"passes": passes, "beta": beta, "alpha": alpha}


def stress_qkv(w: Workload, frame: int, pass_: int, logit_std: float = 3.0):
    """Un-normalised keys scaled so that the softmax logits have standard
    deviation ~logit_std: exercises the online-softmax rescaling that the
    unit-norm keys of the workloads (logit std ~ 1/sqrt(d)) leave untested.
    With q ~ N(0,1) and k ~ N(0, s^2) the logit q.k/sqrt(d) has std s."""
    shape = (w.B, w.H, w.T, w.D)
    q = rng(w, frame, pass_, _Q).standard_normal(shape, dtype=np.float32)
    k = rng(w, frame, pass_, _K).standard_normal(shape, dtype=np.float32)
    v = rng(w, frame, pass_, _V).standard_normal(shape, dtype=np.float32)
    k = k * np.float32(logit_std)
    return _cast(w, q), _cast(w, k), _cast(w, v)
