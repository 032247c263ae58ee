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
  A16 Training (the summary's §2.3 two-stage distillation fine-tunes the
      hybrid model end to end; the pages give no backward pass): the
      gradients are the exact derivatives of the forward step as read above,
      with respect to every input of a pass (q, k, v, phi_q, phi_k, phi_v,
      beta, alpha and the state). phi maps are shared by the B videos, so
      their gradients sum over videos and tokens. Below the 1e-12 floor of
      reading A6 the row map is x / 1e-12, differentiated as such.
  A17 The clean-state precompute for training (a scan over frames: the states
      S_0..S_F that the clean passes commit, computed ahead of the reads, as in
      the prefetch of clean hidden states) is ``rollout``'s commit sequence
      without its reads.

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


def attention_logsumexp(q, k, scale: float | None = None) -> np.ndarray:
    """Each query row's log-sum-exp of its scaled scores over the frame's keys,
    log sum_j exp(scale q . k_j) (natural log): the normaliser of the weights
    of attention_weights, exp(scale q . k_j - lse) = weight j (ARL2 summary
    §2.1, intra-frame branch; the quantity a backward pass reuses).

    q: [..., Tq, d], k: [..., Tk, d] -> [..., Tq]."""
    q = _f64(q)
    k = _f64(k)
    if scale is None:
        scale = default_scale(q.shape[-1])
    a = np.matmul(q, _t(k)) * scale
    m = np.max(a, axis=-1)
    return m + np.log(np.sum(np.exp(a - m[..., None]), axis=-1))


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


def intra_attention_backward(q, k, v, d_o, scale: float | None = None) -> dict:
    """Gradients of O_intra = softmax(Q K^T * scale) V (ARL2 summary §2.1
    intra-frame branch; reading A16) given dL/dO_intra = d_o:
        P = softmax(Q K^T * scale),  dV = P^T dO,  dP = dO V^T,
        dZ = P * (dP - rowsum(P * dP)),  dQ = scale dZ K,  dK = scale dZ^T Q."""
    q, k, v, d_o = _f64(q), _f64(k), _f64(v), _f64(d_o)
    if scale is None:
        scale = default_scale(q.shape[-1])
    P = attention_weights(q, k, scale)
    dP = np.matmul(d_o, _t(v))
    dZ = P * (dP - np.sum(P * dP, axis=-1, keepdims=True))
    return {"dq": scale * np.matmul(dZ, k), "dk": scale * np.matmul(_t(dZ), q),
            "dv": np.matmul(_t(P), d_o)}


def read_backward(q, k, v, phi_q, S, d_o, scale: float | None = None) -> dict:
    """Gradients of one read, O = softmax(Q K^T * scale) V + (Q Phi_q) S
    (ARL2 summary §2.1; readings A9, A16), given dL/dO = d_o. Returns dq, dk,
    dv, dphi_q (summed over videos and tokens) and dS:
        dQ' = dO S^T,  dS = Q'^T dO,  dQ += dQ' Phi_q^T,  dPhi_q = sum_b Q^T dQ'."""
    q, S, d_o = _f64(q), _f64(S), _f64(d_o)
    g = intra_attention_backward(q, k, v, d_o, scale)
    q_prime = feature_map(q, phi_q)
    dq_prime = np.matmul(d_o, _t(S))
    g["dq"] = g["dq"] + np.matmul(dq_prime, _t(_f64(phi_q))[None])
    g["dphi_q"] = np.sum(np.matmul(_t(q), dq_prime), axis=0)
    g["dS"] = np.matmul(_t(q_prime), d_o)
    return g


def commit_backward(k, v, phi_k, phi_v, beta, alpha, S_prev, dS_next) -> dict:
    """Gradients of the clean-pass commit S_next = alpha S_prev +
    K'^T diag(beta) (V' - K' S_prev), K' = rownorm(K Phi_k), V' = V Phi_v
    (ARL2 summary §2.1 update equation; readings A1-A7, A16), given
    G = dL/dS_next:
        R = V' - K' S_prev
        dalpha = <S_prev, G>,   dS_prev = alpha G - K'^T diag(beta) K' G
        dV' = diag(beta) K' G,  dbeta = rowsum((K' G) * R)
        dK' = diag(beta) (R G^T - K' G S_prev^T)
    then through the row normalisation and the maps: dK~ = (dK' - K' rowsum(K'
    * dK')) / ||K~|| (dK' / 1e-12 below the floor), dK = dK~ Phi_k^T,
    dPhi_k = sum_b K^T dK~, dV = dV' Phi_v^T, dPhi_v = sum_b V^T dV'."""
    k, v, beta, alpha = _f64(k), _f64(v), _f64(beta), _f64(alpha)
    S_prev, G = _f64(S_prev), _f64(dS_next)
    k_raw = feature_map(k, phi_k)
    norm = np.sqrt(np.sum(k_raw * k_raw, axis=-1, keepdims=True))
    k_prime = k_raw / np.maximum(norm, L2_EPS)
    v_prime = feature_map(v, phi_v)
    R = v_prime - np.matmul(k_prime, S_prev)
    KG = np.matmul(k_prime, G)
    b = beta[..., :, None]
    d_v_prime = b * KG
    d_k_prime = b * (np.matmul(R, _t(G)) - np.matmul(KG, _t(S_prev)))
    above = norm > L2_EPS
    d_k_raw = np.where(above,
                       (d_k_prime - k_prime * np.sum(k_prime * d_k_prime, axis=-1, keepdims=True))
                       / np.maximum(norm, L2_EPS),
                       d_k_prime / L2_EPS)
    return {
        "dk": np.matmul(d_k_raw, _t(_f64(phi_k))[None]),
        "dv": np.matmul(d_v_prime, _t(_f64(phi_v))[None]),
        "dphi_k": np.sum(np.matmul(_t(k), d_k_raw), axis=0),
        "dphi_v": np.sum(np.matmul(_t(v), d_v_prime), axis=0),
        "dbeta": np.sum(KG * R, axis=-1),
        "dalpha": np.sum(S_prev * G, axis=(-2, -1)),
        "dS_prev": alpha[..., None, None] * G - np.matmul(_t(k_prime), b * KG),
    }


def state_scan(frames, phi_k, phi_v, S0=None) -> list:
    """The clean-state precompute (reading A17): the states S_0..S_F that the
    frames' clean passes commit, without any read. frames as for ``rollout``
    (only the clean pass's k, v and the gates are used)."""
    _, k0, _ = frames[0]["passes"][-1]
    B, H, _, d = np.shape(k0)
    S = np.zeros((B, H, d, d)) if S0 is None else _f64(S0).copy()
    states = [S]
    for fr in frames:
        _, kc, vc = fr["passes"][-1]
        S = commit(kc, vc, phi_k, phi_v, fr["beta"], fr["alpha"], S)
        states.append(S)
    return states


def rollout_backward(frames, phi_q, phi_k, phi_v, d_outputs, S0=None, scale=None,
                     dS_final=None) -> dict:
    """Gradients of a loss on the outputs of a rollout (ARL2 summary §2.2
    streaming loop; reading A16), backpropagated through the frame recurrence.

    d_outputs[(f, p)] = dL/dO of pass p of frame f (passes without an entry
    take no gradient); dS_final = dL/dS_F (default 0). Frame f's reads use S_f
    and its commit maps S_f to S_{f+1}, so with G = dL/dS_{f+1} the frames are
    visited backwards: the commit's backward turns G into its share of
    dL/dS_f, the reads add dS = Q'^T dO. Returns "d_passes"[(f, p)] = (dq, dk,
    dv), "dbeta"[f], "dalpha"[f], dphi_q, dphi_k, dphi_v and dS0."""
    states = state_scan(frames, phi_k, phi_v, S0)
    _, k0, _ = frames[0]["passes"][-1]
    H, d = np.shape(k0)[1], np.shape(k0)[3]
    out = {"d_passes": {}, "dbeta": {}, "dalpha": {},
           "dphi_q": np.zeros((H, d, d)), "dphi_k": np.zeros((H, d, d)),
           "dphi_v": np.zeros((H, d, d))}
    G = np.zeros_like(states[-1]) if dS_final is None else _f64(dS_final).copy()
    for f in range(len(frames) - 1, -1, -1):
        fr = frames[f]
        n_pass = len(fr["passes"])
        _, kc, vc = fr["passes"][n_pass - 1]
        cb = commit_backward(kc, vc, phi_k, phi_v, fr["beta"], fr["alpha"], states[f], G)
        out["dbeta"][f] = cb["dbeta"]
        out["dalpha"][f] = cb["dalpha"]
        out["dphi_k"] += cb["dphi_k"]
        out["dphi_v"] += cb["dphi_v"]
        G = cb["dS_prev"]
        for p, (q, k, v) in enumerate(fr["passes"]):
            dq = np.zeros(np.shape(q))
            dk = np.zeros(np.shape(k))
            dv = np.zeros(np.shape(v))
            if (f, p) in d_outputs:
                rb = read_backward(q, k, v, phi_q, states[f], d_outputs[(f, p)], scale)
                dq, dk, dv = rb["dq"], dk + rb["dk"], dv + rb["dv"]
                out["dphi_q"] += rb["dphi_q"]
                G = G + rb["dS"]
            if p == n_pass - 1:
                dk = dk + cb["dk"]
                dv = dv + cb["dv"]
            out["d_passes"][(f, p)] = (dq, dk, dv)
    out["dS0"] = G
    return out


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
