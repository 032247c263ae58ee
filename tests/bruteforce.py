"""Scalar-loop restatement of the ARL2 hybrid attention step, for tiny inputs.

Independent of ``oracle/``: no numpy linear algebra, only Python floats and
explicit loops over every index, so that a transposed operand, a wrong index or
a dropped term in the oracle's matrix form shows up as a mismatch. Used only by
the oracle's pin tests.

Follows "Attend Locally, Remember Linearly" (technical summary): §2.1 read and
update equations, §2.2 frame-level access and clean-pass update, with the same
readings as the oracle (transpose on the first K', undecayed residual, alpha per
head and frame, beta per token, K' rows unit-normalised after phi_k).
"""
from __future__ import annotations

import math


def _zeros(*shape):
    if len(shape) == 1:
        return [0.0] * shape[0]
    return [_zeros(*shape[1:]) for _ in range(shape[0])]


def feature_map(x, phi):
    """x[t][i], phi[i][j] -> y[t][j] = sum_i x[t][i] phi[i][j] (one head)."""
    T, d_in, d_out = len(x), len(phi), len(phi[0])
    y = _zeros(T, d_out)
    for t in range(T):
        for j in range(d_out):
            acc = 0.0
            for i in range(d_in):
                acc += float(x[t][i]) * float(phi[i][j])
            y[t][j] = acc
    return y


def unit_rows(x, eps=1e-12):
    out = []
    for row in x:
        n = math.sqrt(sum(float(a) * float(a) for a in row))
        n = max(n, eps)
        out.append([float(a) / n for a in row])
    return out


def softmax_attention(q, k, v, scale):
    Tq, Tk, dv = len(q), len(k), len(v[0])
    out = _zeros(Tq, dv)
    for t in range(Tq):
        logits = []
        for s in range(Tk):
            dot = 0.0
            for i in range(len(q[t])):
                dot += float(q[t][i]) * float(k[s][i])
            logits.append(dot * scale)
        m = max(logits)
        w = [math.exp(a - m) for a in logits]
        z = sum(w)
        for j in range(dv):
            acc = 0.0
            for s in range(Tk):
                acc += w[s] / z * float(v[s][j])
            out[t][j] = acc
    return out


def row_times_matrix(x, S):
    T, dk, dv = len(x), len(S), len(S[0])
    y = _zeros(T, dv)
    for t in range(T):
        for j in range(dv):
            acc = 0.0
            for i in range(dk):
                acc += float(x[t][i]) * float(S[i][j])
            y[t][j] = acc
    return y


def commit_tokens(kp, vp, beta, alpha, S):
    """S_next = alpha S + sum_t beta_t k_t^T (v_t - k_t S), every rank-1 term
    against the same pre-update S (frame-level access)."""
    dk, dv = len(S), len(S[0])
    new = [[float(alpha) * float(S[i][j]) for j in range(dv)] for i in range(dk)]
    for t in range(len(kp)):
        pred = [sum(float(kp[t][i]) * float(S[i][j]) for i in range(dk)) for j in range(dv)]
        res = [float(vp[t][j]) - pred[j] for j in range(dv)]
        for i in range(dk):
            for j in range(dv):
                new[i][j] += float(beta[t]) * float(kp[t][i]) * res[j]
    return new


def rollout(frames, phi_q, phi_k, phi_v, scale):
    """One head. frames[f] = {"passes": [(q, k, v), ...], "beta": [T], "alpha": a}.
    Returns outputs[(f, p)] = {"o", "o_intra", "o_inter"} and states[0..F]."""
    d = len(phi_q)
    S = _zeros(d, d)
    states = [S]
    outputs = {}
    for f, fr in enumerate(frames):
        for p, (q, k, v) in enumerate(fr["passes"]):
            oi = softmax_attention(q, k, v, scale)
            oe = row_times_matrix(feature_map(q, phi_q), S)
            o = [[oi[t][j] + oe[t][j] for j in range(d)] for t in range(len(q))]
            outputs[(f, p)] = {"o": o, "o_intra": oi, "o_inter": oe}
        _, kc, vc = fr["passes"][-1]
        kp = unit_rows(feature_map(kc, phi_k))
        vp = feature_map(vc, phi_v)
        S = commit_tokens(kp, vp, fr["beta"], fr["alpha"], S)
        states.append(S)
    return outputs, states


def softmax_layer_rollout(frames, scale):
    """One head of a KV-cache softmax layer: each pass of frame f attends over
    the clean-pass keys/values of frames 0..f-1 followed by its own, written as
    explicit loops over the cached tokens. frames[f] = {"passes": [(q, k, v)]}.
    Returns outputs[(f, p)] = O."""
    cache_k, cache_v = [], []
    outputs = {}
    for f, fr in enumerate(frames):
        for p, (q, k, v) in enumerate(fr["passes"]):
            keys = [row for row in cache_k] + [row for row in k]
            vals = [row for row in cache_v] + [row for row in v]
            out = []
            for t in range(len(q)):
                logits = []
                for s in range(len(keys)):
                    dot = 0.0
                    for i in range(len(q[t])):
                        dot += float(q[t][i]) * float(keys[s][i])
                    logits.append(dot * scale)
                m = max(logits)
                w = [math.exp(a - m) for a in logits]
                z = sum(w)
                out.append([sum(w[s] / z * float(vals[s][j]) for s in range(len(keys)))
                            for j in range(len(vals[0]))])
            outputs[(f, p)] = out
        _, kc, vc = fr["passes"][-1]
        cache_k.extend(kc)
        cache_v.extend(vc)
    return outputs


def token_level_read(q, k, v, phi_q, phi_k, phi_v, beta, S, scale):
    """One head under token-level access: token t reads the state left by the
    earlier tokens of the frame, then updates it with its own delta-rule term.
    Returns (o_inter, S_T)."""
    qp = feature_map(q, phi_q)
    kp = unit_rows(feature_map(k, phi_k))
    vp = feature_map(v, phi_v)
    dk, dv = len(S), len(S[0])
    St = [[float(S[i][j]) for j in range(dv)] for i in range(dk)]
    o = []
    for t in range(len(qp)):
        o.append([sum(qp[t][i] * St[i][j] for i in range(dk)) for j in range(dv)])
        pred = [sum(kp[t][i] * St[i][j] for i in range(dk)) for j in range(dv)]
        for i in range(dk):
            for j in range(dv):
                St[i][j] += float(beta[t]) * kp[t][i] * (vp[t][j] - pred[j])
    return o, St
