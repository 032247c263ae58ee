"""fp64 CPU oracle for the ARL2 hybrid attention step.

TEST INFRASTRUCTURE. This module is the slow, obviously-correct statement of
what the hybrid attention step computes. It is imported only by ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``. The
product path (``hybrid_linear_memory_amd``) never imports it, and it imports
nothing from the product path: it shares no kernel, helper, table or constant
with the HIP code. Every array is upcast to float64 on entry; bf16 inputs are
taken as the exact values the GPU sees.

Source: "Attend Locally, Remember Linearly: Linear Attention as Cross-Frame
Memory for Autoregressive Video Diffusion" (Li, Shah, Shang), technical summary
as published on gist.science in Chinese, Portuguese and French (the three agree
sentence for sentence). Cited below as "ARL2 summary" plus section:

  §2.1  Hybrid attention decomposition: intra-frame branch = the original
        bidirectional softmax over the frame's tokens with the frozen Q/K/V;
        inter-frame branch = a fixed-size recurrent state S updated by the gated
        delta rule, fed through per-head grouped 1x1 feature maps phi_q, phi_k,
        phi_v; update equation S_N = alpha_N S_{N-1} + beta_N K'_N (V'_N -
        K'_N S_{N-1}); read equation O_inter = Q'_N S_{N-1}.
  §2.2  Memory state management: frame-level access (every token of frame N
        queries the same pre-update S_{N-1}; S changes only after the whole
        frame) and the clean-pass update (denoising steps read S and never
        write it; S is written once per frame, after the final clean pass).
  §4    Ablations: per-head gating is the best trade-off; token-level access is
        worse than frame-level access.

Readings taken where the pages are silent, ambiguous or garbled (each is
applied by exactly one function below):

  A1  The update as printed lacks a transpose for a T x d key matrix. The only
      shape-consistent reading with the row-vector read Q'S is
      S_N = alpha S_{N-1} + K'^T diag(beta) (V' - K' S_{N-1}),
      i.e. the sum over tokens of beta_t k'_t^T (v'_t - k'_t S_{N-1}).
  A2  The residual uses the undecayed S_{N-1}, as printed (not alpha*S_{N-1}).
  A3  alpha is one scalar per (video, head, frame)  (per-head gating, §4).
  A4  beta is one scalar per (video, head, token): diag(beta) over the T rows.
  A5  All T rank-1 terms of a frame use the same S_{N-1} (frame-level access,
      §2.2); there is no sequential per-token update inside a frame.
  A6  K' rows are L2-normalised after phi_k: x / max(||x||_2, 1e-12). Q' is not
      normalised.
  A7  phi_x is linear, no bias: X' = X Phi_x[h], Phi stored [H, d_in, d_out].
  A8  Intra-frame softmax: scale 1/sqrt(d) unless given, no mask, raw Q, K, V.
  A9  O = O_intra + O_inter.
  A10 S_0 = 0.
  A11 The clean pass is a separate pass after the denoising reads; it also
      reads S_{N-1} and produces O, then commits.
  A12 Frames are indexed 0..F-1 here: frame f reads S_f and commits S_{f+1}.
  A13 The commit uses the clean pass's K and V.
  A15 Token-level access (the ablated alternative, §4), not defined further by
      the pages: within a pass, token t reads the state left by the tokens
      before it in the frame, S_t = S_{t-1} + beta_t k'_t^T (v'_t - k'_t
      S_{t-1}) starting from S_{N-1}, o_inter_t = q'_t S_{t-1}; denoising
      passes discard these updates, the clean pass commits
      S_N = alpha_N S_{N-1} + (S_T - S_{N-1}) (the frame's gate applied once,
      as in the frame-level update). With T = 1 it equals frame-level access.

Every function in this module is pinned by ``tests/test_oracle_pins.py``
against closed forms, invariants, exact rational worked examples and scalar
brute-force loops.
"""
from __future__ import annotations

import numpy as np

L2_EPS = 1e-12  # reading A6


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _t(x: np.ndarray) -> np.ndarray:
    """Transpose the last two axes."""
    return np.swapaxes(x, -1, -2)


def feature_map(x, phi) -> np.ndarray:
    """Per-head grouped 1x1 feature map X' = X Phi[h]  (ARL2 summary §2.1,
    "Adaptation"; reading A7).

    x: [B, H, T, d_in]; phi: [H, d_in, d_out]. Returns [B, H, T, d_out]."""
    x = _f64(x)
    phi = _f64(phi)
    return np.matmul(x, phi[None, :, :, :])


def l2_normalize_rows(x, eps: float = L2_EPS) -> np.ndarray:
    """Row-wise x / max(||x||_2, eps)  (reading A6)."""
    x = _f64(x)
    norm = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(norm, eps)


def default_scale(d: int) -> float:
    """Softmax temperature 1/sqrt(d)  (reading A8)."""
    return 1.0 / np.sqrt(float(d))


def attention_weights(q, k, scale: float | None = None) -> np.ndarray:
    """Bidirectional softmax weights over the frame's tokens, no mask
    (ARL2 summary §2.1, intra-frame branch; reading A8).

    q: [..., Tq, d], k: [..., Tk, d] -> [..., Tq, Tk]. The row maximum is
    subtracted before exp; it cancels in the ratio."""
    q = _f64(q)
    k = _f64(k)
    if scale is None:
        scale = default_scale(q.shape[-1])
    a = np.matmul(q, _t(k)) * scale
    a = a - np.max(a, axis=-1, keepdims=True)
    e = np.exp(a)
    return e / np.sum(e, axis=-1, keepdims=True)


def intra_attention(q, k, v, scale: float | None = None) -> np.ndarray:
    """O_intra = softmax(Q K^T * scale) V over one frame (ARL2 summary §2.1).

    Works row by row, so q may hold any subset of the frame's query rows."""
    return np.matmul(attention_weights(q, k, scale), _f64(v))


def inter_read(q_prime, S) -> np.ndarray:
    """O_inter = Q' S_{N-1}  (ARL2 summary §2.1, output equation).

    q_prime: [B, H, T, d_k]; S: [B, H, d_k, d_v]. S is only read."""
    return np.matmul(_f64(q_prime), _f64(S))


def read(q, k, v, phi_q, S, scale: float | None = None) -> dict:
    """One pass of the hybrid attention layer against state S (a denoising
    read, or the read half of the clean pass).

    Frame-level access (ARL2 summary §2.2): every query row uses the same S.
    Returns a dict with o, o_intra, o_inter; S is not modified."""
    o_intra = intra_attention(q, k, v, scale)
    q_prime = feature_map(q, phi_q)
    o_inter = inter_read(q_prime, S)
    return {"o": o_intra + o_inter, "o_intra": o_intra, "o_inter": o_inter}


def state_commit(k_prime, v_prime, beta, alpha, S_prev) -> np.ndarray:
    """Gated delta update of the state, applied once per frame
    (ARL2 summary §2.1 update equation; readings A1-A5).

    k_prime, v_prime: [B, H, T, d]; beta: [B, H, T]; alpha: [B, H];
    S_prev: [B, H, d_k, d_v]. Returns S_next; S_prev is not modified.

      P = K' S_prev                      prediction of V' from the old state
      R = V' - P                         residual against the undecayed state
      U = K'^T diag(beta) R              batched rank-T correction
      S_next = alpha * S_prev + U
    """
    kp = _f64(k_prime)
    vp = _f64(v_prime)
    beta = _f64(beta)
    alpha = _f64(alpha)
    S_prev = _f64(S_prev)
    P = np.matmul(kp, S_prev)
    R = vp - P
    U = np.matmul(_t(kp), beta[..., :, None] * R)
    return alpha[..., None, None] * S_prev + U


def commit_inputs(k, v, phi_k, phi_v) -> tuple[np.ndarray, np.ndarray]:
    """K' = rownorm(K Phi_k[h]), V' = V Phi_v[h]  (ARL2 summary §2.1
    "Adaptation"; readings A6, A7)."""
    k_prime = l2_normalize_rows(feature_map(k, phi_k))
    v_prime = feature_map(v, phi_v)
    return k_prime, v_prime


def commit(k, v, phi_k, phi_v, beta, alpha, S_prev) -> np.ndarray:
    """Clean-pass state write from the frame's raw K, V (ARL2 summary §2.2,
    clean-pass update; reading A13)."""
    k_prime, v_prime = commit_inputs(k, v, phi_k, phi_v)
    return state_commit(k_prime, v_prime, beta, alpha, S_prev)


def fullkv_attention(q, k_all, v_all, scale: float | None = None) -> np.ndarray:
    """The cross-frame softmax that the recurrent state replaces (ARL2 summary
    §1, growing KV cache): the current frame's queries attend over every cached
    frame's keys plus the current frame's, no mask.

    q: [B, H, Tq, d]; k_all, v_all: [B, H, n_kv, d]."""
    return intra_attention(q, k_all, v_all, scale)


def rollout(frames, phi_q, phi_k, phi_v, S0=None, scale=None,
            eval_pass=None):
    """Streaming loop of the hybrid layer over frames (ARL2 summary §2.2).

    frames: sequence; frames[f] is a dict with
        "passes": list of (q, k, v) per pass, the last being the clean pass;
        "beta": [B, H, T]; "alpha": [B, H].
    eval_pass(f, p) -> bool selects which passes' outputs are computed
    (default: all). Reads never change S, so skipping one leaves the state
    trajectory unchanged.

    Returns (outputs, states): outputs[(f, p)] = read(...) dict;
    states[f] = S_f for f = 0..F (states[0] = S_0).
    """
    first_q = frames[0]["passes"][0][0]
    B, H, _, d = np.shape(first_q)
    S = np.zeros((B, H, d, d)) if S0 is None else _f64(S0).copy()  # A10
    states = [S]
    outputs = {}
    for f, fr in enumerate(frames):
        n_pass = len(fr["passes"])
        for p, (q, k, v) in enumerate(fr["passes"]):
            if eval_pass is None or eval_pass(f, p):
                outputs[(f, p)] = read(q, k, v, phi_q, S, scale)
        _, kc, vc = fr["passes"][n_pass - 1]          # A11, A13: clean pass
        S = commit(kc, vc, phi_k, phi_v, fr["beta"], fr["alpha"], S)
        states.append(S)
    return outputs, states


def softmax_layer_rollout(frames, scale=None, eval_pass=None):
    """A softmax attention layer of the autoregressive video model, the kind
    the hybrid replaces (ARL2 summary §1: every generated block's keys and
    values join a KV cache that later blocks attend to; §3: the layers not
    replaced keep softmax attention). Every pass of frame f attends, with no
    mask, over the clean-pass keys and values of frames 0..f-1 (the cache) plus
    the pass's own; after the frame its clean-pass K and V join the cache.

    frames: as for ``rollout`` ("beta"/"alpha" unused). Returns outputs[(f, p)]
    = O [B, H, T, d] for the evaluated passes."""
    cache_k, cache_v = [], []
    outputs = {}
    for f, fr in enumerate(frames):
        n_pass = len(fr["passes"])
        for p, (q, k, v) in enumerate(fr["passes"]):
            if eval_pass is None or eval_pass(f, p):
                k_all = np.concatenate([_f64(c) for c in cache_k] + [_f64(k)], axis=2)
                v_all = np.concatenate([_f64(c) for c in cache_v] + [_f64(v)], axis=2)
                outputs[(f, p)] = fullkv_attention(q, k_all, v_all, scale)
        _, kc, vc = fr["passes"][n_pass - 1]
        cache_k.append(kc)
        cache_v.append(vc)
    return outputs


def hybrid_stack_rollout(layers, mask, scale=None, eval_pass=None):
    """A stack of attention layers in which the layers marked in ``mask`` are
    hybrid ARL2 layers (state S, ``rollout``) and the others softmax layers
    with a KV cache (``softmax_layer_rollout``); the summary's hybrid model
    replaces a fraction of a 30-layer model's attention layers (§3: 50% or 75%).
    Each layer takes its own inputs: layers[l] = {"frames": ..., "phis":
    (phi_q, phi_k, phi_v)} ("phis" unused for softmax layers).

    Returns per layer: {"o": outputs[(f, p)] -> O} and, for ARL2 layers,
    "states" (S_0..S_F)."""
    res = []
    for lay, is_arl2 in zip(layers, mask):
        if is_arl2:
            outs, states = rollout(lay["frames"], *lay["phis"], scale=scale, eval_pass=eval_pass)
            res.append({"o": {key: r["o"] for key, r in outs.items()}, "states": states})
        else:
            res.append({"o": softmax_layer_rollout(lay["frames"], scale, eval_pass)})
    return res


def token_level_read(q, k, v, phi_q, phi_k, phi_v, beta, S, scale=None) -> dict:
    """One pass under token-level access (reading A15; ARL2 summary §4 ablation):
    the intra-frame softmax as in ``read``, and an inter-frame branch in which
    token t reads the state updated by the frame's earlier tokens, in token
    order, starting from S = S_{N-1}:
        o_inter_t = q'_t S_{t-1};  S_t = S_{t-1} + beta_t k'_t^T (v'_t - k'_t S_{t-1}).
    Returns o, o_intra, o_inter and S_T (the state after the last token)."""
    q_prime = feature_map(q, phi_q)
    k_prime, v_prime = commit_inputs(k, v, phi_k, phi_v)
    beta = _f64(beta)
    St = _f64(S).copy()                               # [B, H, d, d]
    o_inter = np.zeros(q_prime.shape[:3] + (St.shape[-1],))
    for t in range(q_prime.shape[2]):
        o_inter[:, :, t] = np.einsum("bhi,bhij->bhj", q_prime[:, :, t], St)
        kt, vt = k_prime[:, :, t], v_prime[:, :, t]
        resid = vt - np.einsum("bhi,bhij->bhj", kt, St)
        St = St + beta[:, :, t, None, None] * kt[..., :, None] * resid[..., None, :]
    o_intra = intra_attention(q, k, v, scale)
    return {"o": o_intra + o_inter, "o_intra": o_intra, "o_inter": o_inter, "S_T": St}


def token_level_rollout(frames, phi_q, phi_k, phi_v, S0=None, scale=None, eval_pass=None):
    """The streaming loop under token-level access (reading A15): every pass
    runs ``token_level_read`` from S_{N-1}; the clean pass's end state commits
    S_N = alpha S_{N-1} + (S_T - S_{N-1}). Same arguments and returns as
    ``rollout``."""
    first_q = frames[0]["passes"][0][0]
    B, H, _, d = np.shape(first_q)
    S = np.zeros((B, H, d, d)) if S0 is None else _f64(S0).copy()
    states = [S]
    outputs = {}
    for f, fr in enumerate(frames):
        n_pass = len(fr["passes"])
        clean = None
        for p, (q, k, v) in enumerate(fr["passes"]):
            if p == n_pass - 1 or eval_pass is None or eval_pass(f, p):
                r = token_level_read(q, k, v, phi_q, phi_k, phi_v, fr["beta"], S, scale)
                outputs[(f, p)] = r
                if p == n_pass - 1:
                    clean = r
        alpha = _f64(fr["alpha"])[:, :, None, None]
        S = alpha * S + (clean["S_T"] - S)
        states.append(S)
    return outputs, states
