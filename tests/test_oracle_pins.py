"""Pins of the fp64 oracle to things other than itself.

Source: "Attend Locally, Remember Linearly" technical summary (gist.science),
§2.1 (hybrid decomposition: intra-frame softmax, feature maps, update and read
equations) and §2.2 (frame-level access, clean-pass update). The pages print no
numerical example, so the pins are closed forms, invariants, hand-derived
rational examples (tests/golden/), special cases and a scalar brute-force
unroll (tests/bruteforce.py). Each test names the mistake it is meant to catch.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import bruteforce as bf
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            key, r, c = parts[0], int(parts[1]), int(parts[2])
            vals = []
            for tok in parts[3:]:
                vals.append(math.log(3.0) if tok == "ln3" else Fraction(tok))
            out[key] = (r, c, vals)
    return out


def _as_array(entry):
    r, c, vals = entry
    return np.array([float(v) for v in vals], dtype=np.float64).reshape(r, c)


def _rs(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- softmax (a2)

def test_p1_softmax_rows_sum_to_one():
    """P1: attention weights are a probability distribution per query row."""
    g = _rs(1)
    q = g.standard_normal((2, 3, 17, 8)) * 3
    k = g.standard_normal((2, 3, 29, 8)) * 3
    w = oracle.attention_weights(q, k)
    assert w.shape == (2, 3, 17, 29)
    assert np.all(w >= 0)
    np.testing.assert_allclose(w.sum(-1), 1.0, rtol=0, atol=1e-15)


def test_golden_softmax_ln3():
    """Hand-derived weights (1/4, 3/4): catches a wrong exp base, a missing
    normalisation or weights applied to the wrong value rows."""
    gd = _load_golden("softmax_ln3.txt")
    q, k, v = _as_array(gd["q"]), _as_array(gd["k"]), _as_array(gd["v"])
    w = oracle.attention_weights(q[None, None], k[None, None], scale=1.0)[0, 0]
    np.testing.assert_allclose(w, _as_array(gd["weights"]), rtol=0, atol=1e-15)
    o = oracle.intra_attention(q[None, None], k[None, None], v[None, None], scale=1.0)[0, 0]
    np.testing.assert_allclose(o, _as_array(gd["o"]), rtol=0, atol=1e-14)


def test_p2_closed_forms():
    """P2: Q = 0 gives the column mean of V; T = 1 gives V; equal keys give
    uniform weights whatever the query."""
    g = _rs(2)
    v = g.standard_normal((1, 2, 11, 4))
    k = g.standard_normal((1, 2, 11, 4))
    o = oracle.intra_attention(np.zeros((1, 2, 5, 4)), k, v)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape),
                               rtol=0, atol=1e-15)
    o1 = oracle.intra_attention(g.standard_normal((1, 2, 1, 4)), k[:, :, :1], v[:, :, :1])
    np.testing.assert_allclose(o1, v[:, :, :1], rtol=0, atol=1e-15)
    keq = np.broadcast_to(g.standard_normal((1, 2, 1, 4)), (1, 2, 11, 4))
    w = oracle.attention_weights(g.standard_normal((1, 2, 3, 4)), keq)
    np.testing.assert_allclose(w, 1.0 / 11, rtol=0, atol=1e-15)


def test_default_scale_is_inverse_sqrt_d():
    """Reading A8: temperature 1/sqrt(d). Two keys differing by a logit gap:
    the weight ratio is exp(gap / sqrt(d))."""
    d = 16
    q = np.zeros((1, 1, 1, d)); q[..., 0] = 2.0
    k = np.zeros((1, 1, 2, d)); k[..., 1, 0] = 1.5
    w = oracle.attention_weights(q, k)[0, 0, 0]
    assert w[1] / w[0] == pytest.approx(math.exp(3.0 / 4.0), rel=1e-14)


def test_p3_bruteforce_attention():
    """P3: the matrix form equals scalar loops on T <= 8 (catches K vs K^T and
    softmax over the wrong axis)."""
    g = _rs(3)
    q = g.standard_normal((6, 5)) * 2
    k = g.standard_normal((8, 5)) * 2
    v = g.standard_normal((8, 3))
    ref = bf.softmax_attention(q.tolist(), k.tolist(), v.tolist(), 0.37)
    got = oracle.intra_attention(q[None, None], k[None, None], v[None, None], 0.37)[0, 0]
    np.testing.assert_allclose(got, np.array(ref), rtol=0, atol=1e-13)


def test_softmax_shift_invariance_large_logits():
    """Adding a constant to every logit of a row leaves the weights unchanged,
    also far beyond exp's range (max subtraction)."""
    g = _rs(4)
    q = g.standard_normal((1, 1, 3, 4))
    k = g.standard_normal((1, 1, 7, 4))
    w = oracle.attention_weights(q, k, 1.0)
    shift = np.zeros((1, 1, 1, 5)); shift[..., 4] = 1.0
    q2 = np.concatenate([q, np.full((1, 1, 3, 1), 1.0)], -1)
    k2 = np.concatenate([k, np.full((1, 1, 7, 1), 900.0)], -1)
    w2 = oracle.attention_weights(q2, k2, 1.0)
    np.testing.assert_allclose(w2, w, rtol=1e-12, atol=0)


def test_logsumexp_closed_forms():
    """The rows' log-sum-exp: log 4 for the golden example's scores (0, ln 3)
    (4 = e^0 + e^ln3), log T for Q = 0, the single score for one key, and
    log T plus the common score for T equal keys; catches a base-2 or
    unscaled sum, a dropped max shift or a sum over the wrong axis."""
    gd = _load_golden("softmax_ln3.txt")
    q, k = _as_array(gd["q"]), _as_array(gd["k"])
    lse = oracle.attention_logsumexp(q[None, None], k[None, None], scale=1.0)[0, 0]
    np.testing.assert_allclose(lse, math.log(4.0), rtol=0, atol=1e-14)
    g = _rs(11)
    k = g.standard_normal((2, 3, 9, 8))
    np.testing.assert_allclose(oracle.attention_logsumexp(np.zeros((2, 3, 5, 8)), k),
                               np.log(9.0), rtol=0, atol=1e-14)
    q1, k1 = g.standard_normal((1, 2, 4, 8)), g.standard_normal((1, 2, 1, 8))
    one = (q1 @ np.swapaxes(k1, -1, -2))[..., 0] * 0.5
    np.testing.assert_allclose(oracle.attention_logsumexp(q1, k1, 0.5), one, rtol=1e-14)
    kr = np.repeat(k1, 6, axis=2)
    np.testing.assert_allclose(oracle.attention_logsumexp(q1, kr, 0.5), one + math.log(6.0),
                               rtol=0, atol=1e-13)
    # far beyond exp's range: the max shift keeps it finite and exact
    big = oracle.attention_logsumexp(np.full((1, 1, 1, 1), 30.0), np.full((1, 1, 2, 1), 40.0),
                                     1.0)
    np.testing.assert_allclose(big, 1200.0 + math.log(2.0), rtol=1e-15)


# ----------------------------------------------------------- feature maps (a1)

def test_feature_map_orientation_and_heads():
    """Reading A7: X' = X Phi[h] with Phi[h] indexed [d_in, d_out]. A unit row
    e_i picks row i of Phi[h]; each head uses its own Phi (catches Phi^T and a
    head-index mix-up)."""
    g = _rs(5)
    phi = g.standard_normal((3, 4, 4))
    x = np.zeros((2, 3, 4, 4))
    for b in range(2):
        for h in range(3):
            x[b, h] = np.eye(4)
    y = oracle.feature_map(x, phi)
    for b in range(2):
        for h in range(3):
            np.testing.assert_array_equal(y[b, h], phi[h])
    xr = g.standard_normal((1, 3, 6, 4))
    yr = oracle.feature_map(xr, phi)
    for h in range(3):
        ref = bf.feature_map(xr[0, h].tolist(), phi[h].tolist())
        np.testing.assert_allclose(yr[0, h], np.array(ref), rtol=0, atol=1e-13)


def test_l2_normalize_rows():
    """Reading A6: unit rows, direction kept, the zero row stays zero."""
    g = _rs(6)
    x = g.standard_normal((5, 7)) * 10
    x[2] = 0.0
    y = oracle.l2_normalize_rows(x)
    n = np.linalg.norm(y, axis=-1)
    np.testing.assert_allclose(np.delete(n, 2), 1.0, rtol=0, atol=1e-15)
    np.testing.assert_array_equal(y[2], 0.0)
    np.testing.assert_allclose(y[0] * np.linalg.norm(x[0]), x[0], rtol=1e-14)
    assert oracle.l2_normalize_rows(np.array([[3.0, 4.0]])).tolist() == [[0.6, 0.8]]


# ------------------------------------------------------------ commit (a5)

def test_golden_delta_rule_2x2():
    """Hand-derived rational example: catches the residual taken against
    alpha*S (reading A2), beta applied per column instead of per token, S K'
    instead of K' S, and a missing alpha*S term."""
    gd = _load_golden("delta_rule_2x2.txt")
    S = _as_array(gd["S_prev"])[None, None]
    K = _as_array(gd["K"])[None, None]
    V = _as_array(gd["V"])[None, None]
    beta = _as_array(gd["beta"])[None]            # [1, 1, T]
    alpha = _as_array(gd["alpha"])[0]             # [1, 1]
    got = oracle.state_commit(K, V, beta, alpha, S)[0, 0]
    np.testing.assert_allclose(got, _as_array(gd["S_next"]), rtol=0, atol=1e-15)
    # through the full commit with identity maps and the same (unit) keys
    eye = np.eye(2)[None]
    got2 = oracle.commit(K, V, eye, eye, beta, alpha, S)[0, 0]
    np.testing.assert_allclose(got2, _as_array(gd["S_next"]), rtol=0, atol=1e-15)


def test_p4_identity_and_pure_decay():
    """P4: alpha=1, beta=0 leaves S unchanged exactly; beta=0 gives alpha*S and
    after k frames prod(alpha)*S."""
    g = _rs(7)
    B, H, T, d = 2, 3, 9, 5
    S = g.standard_normal((B, H, d, d))
    kp = oracle.l2_normalize_rows(g.standard_normal((B, H, T, d)))
    vp = g.standard_normal((B, H, T, d))
    zero = np.zeros((B, H, T))
    out = oracle.state_commit(kp, vp, zero, np.ones((B, H)), S)
    np.testing.assert_array_equal(out, S)
    cur = S
    prod = np.ones((B, H))
    for _ in range(4):
        a = g.uniform(0.2, 0.99, (B, H))
        cur = oracle.state_commit(kp, vp, zero, a, cur)
        prod = prod * a
    np.testing.assert_allclose(cur, prod[..., None, None] * S, rtol=1e-14, atol=0)


def test_p5_exact_write_single_key():
    """P5 (delta-rule exact write): alpha=1, beta=1, one unit key k, identity
    maps: afterwards k S_n = v, whatever S_{n-1} held. Catches a wrong sign in
    the residual and the missing transpose."""
    g = _rs(8)
    d = 6
    S = g.standard_normal((1, 1, d, d))
    k = g.standard_normal((1, 1, 1, d)) * 3.0     # not unit: commit normalises
    v = g.standard_normal((1, 1, 1, d))
    eye = np.eye(d)[None]
    Sn = oracle.commit(k, v, eye, eye, np.ones((1, 1, 1)), np.ones((1, 1)), S)
    ku = k / np.linalg.norm(k)
    np.testing.assert_allclose(ku[0, 0] @ Sn[0, 0], v[0, 0], rtol=0, atol=1e-14)


def test_p6_exact_write_orthonormal_keys():
    """P6: T <= d orthonormal keys, alpha = beta = 1, identity maps:
    K' S_n = V' for every key at once (frame-level batched write)."""
    g = _rs(9)
    d, T = 8, 5
    Qm, _ = np.linalg.qr(g.standard_normal((d, d)))
    K = Qm[:T][None, None]
    V = g.standard_normal((1, 1, T, d))
    S = g.standard_normal((1, 1, d, d))
    eye = np.eye(d)[None]
    Sn = oracle.commit(K, V, eye, eye, np.ones((1, 1, T)), np.ones((1, 1)), S)
    np.testing.assert_allclose(K[0, 0] @ Sn[0, 0], V[0, 0], rtol=0, atol=1e-13)


def test_p7_token_loop_and_gram_form():
    """P7: the matrix form equals the loop of rank-1 terms against the same
    S_{n-1}, and the independent Gram form
    S_n = (alpha I - K'^T B K') S_{n-1} + K'^T B V'."""
    g = _rs(10)
    B, H, T, d = 1, 2, 7, 4
    kp = oracle.l2_normalize_rows(g.standard_normal((B, H, T, d)))
    vp = g.standard_normal((B, H, T, d))
    beta = g.uniform(0, 1, (B, H, T))
    alpha = g.uniform(0.5, 1, (B, H))
    S = g.standard_normal((B, H, d, d))
    got = oracle.state_commit(kp, vp, beta, alpha, S)
    for h in range(H):
        ref = bf.commit_tokens(kp[0, h].tolist(), vp[0, h].tolist(), beta[0, h].tolist(),
                               alpha[0, h], S[0, h].tolist())
        np.testing.assert_allclose(got[0, h], np.array(ref), rtol=0, atol=1e-13)
        Bm = np.diag(beta[0, h])
        K, V = kp[0, h], vp[0, h]
        gram = (alpha[0, h] * np.eye(d) - K.T @ Bm @ K) @ S[0, h] + K.T @ Bm @ V
        np.testing.assert_allclose(got[0, h], gram, rtol=0, atol=1e-13)


def test_p12_first_frame():
    """P12: S_0 = 0 gives S_1 = K'^T diag(beta) V' and a zero inter read."""
    g = _rs(11)
    B, H, T, d = 1, 1, 6, 4
    q = g.standard_normal((B, H, T, d))
    k = g.standard_normal((B, H, T, d))
    v = g.standard_normal((B, H, T, d))
    phis = [g.standard_normal((H, d, d)) for _ in range(3)]
    beta = g.uniform(0, 0.2, (B, H, T))
    alpha = g.uniform(0.5, 1, (B, H))
    frames = [{"passes": [(q, k, v)], "beta": beta, "alpha": alpha}]
    outs, states = oracle.rollout(frames, *phis)
    np.testing.assert_array_equal(outs[(0, 0)]["o_inter"], 0.0)
    kp, vp = oracle.commit_inputs(k, v, phis[1], phis[2])
    ref = kp[0, 0].T @ np.diag(beta[0, 0]) @ vp[0, 0]
    np.testing.assert_allclose(states[1][0, 0], ref, rtol=0, atol=1e-14)


def test_p11_stability_bound():
    """P11: with the workloads' gates (sum of beta < 1), the linear part
    A = alpha I - K'^T diag(beta) K' has eigenvalues in [alpha - sum(beta),
    alpha], and ||S|| stays bounded over a long rollout."""
    g = _rs(12)
    T, d = 64, 16
    kp = oracle.l2_normalize_rows(g.standard_normal((T, d)))
    beta = 1.0 / (1.0 + np.exp(-g.standard_normal(T))) / T
    alpha = 0.9
    A = alpha * np.eye(d) - kp.T @ np.diag(beta) @ kp
    ev = np.linalg.eigvalsh(A)
    assert ev.min() >= alpha - beta.sum() - 1e-12 and ev.max() <= alpha + 1e-12
    S = np.zeros((1, 1, d, d))
    norms = []
    for f in range(240):
        kf = oracle.l2_normalize_rows(g.standard_normal((1, 1, T, d)))
        vf = g.standard_normal((1, 1, T, d))
        bf_ = (1.0 / (1.0 + np.exp(-g.standard_normal((1, 1, T)))) / T)
        af = 1.0 / (1.0 + np.exp(-g.normal(3.0, 0.5, (1, 1))))
        S = oracle.state_commit(kf, vf, bf_, af, S)
        norms.append(np.linalg.norm(S))
    assert max(norms[120:]) < 3 * max(norms[:120]) + 1e-9
    assert np.isfinite(norms).all()


# ------------------------------------------------ read and sequencing (a3-a6)

def test_p9_frame_level_access():
    """P9: identical query rows in a frame get identical O_inter (and O) rows,
    because every row reads the same S_{N-1}."""
    g = _rs(13)
    B, H, T, d = 1, 2, 10, 8
    q = g.standard_normal((B, H, T, d))
    q[:, :, 7] = q[:, :, 2]
    k = g.standard_normal((B, H, T, d))
    v = g.standard_normal((B, H, T, d))
    S = g.standard_normal((B, H, d, d))
    phi = g.standard_normal((H, d, d))
    out = oracle.read(q, k, v, phi, S)
    np.testing.assert_allclose(out["o_inter"][:, :, 7], out["o_inter"][:, :, 2], rtol=0, atol=1e-14)
    np.testing.assert_allclose(out["o"][:, :, 7], out["o"][:, :, 2], rtol=0, atol=1e-14)
    np.testing.assert_allclose(out["o"], out["o_intra"] + out["o_inter"], rtol=0, atol=0)


def test_p10_reads_never_mutate_state():
    """P10: a read leaves S untouched, and S_n does not depend on how many
    denoising reads preceded the clean pass."""
    g = _rs(14)
    B, H, T, d = 1, 2, 6, 4
    phis = [g.standard_normal((H, d, d)) for _ in range(3)]
    S = g.standard_normal((B, H, d, d))
    S_copy = S.copy()
    oracle.read(g.standard_normal((B, H, T, d)), g.standard_normal((B, H, T, d)),
                g.standard_normal((B, H, T, d)), phis[0], S)
    np.testing.assert_array_equal(S, S_copy)

    clean = [(g.standard_normal((B, H, T, d)) for _ in range(3)) for _ in range(3)]
    clean = [tuple(c) for c in clean]
    gates_ = [(g.uniform(0, 0.1, (B, H, T)), g.uniform(0.5, 1, (B, H))) for _ in range(3)]
    finals = []
    for n_denoise in (0, 1, 4):
        frames = []
        for f in range(3):
            noisy = [tuple(g.standard_normal((B, H, T, d)) for _ in range(3))
                     for _ in range(n_denoise)]
            frames.append({"passes": noisy + [clean[f]], "beta": gates_[f][0],
                           "alpha": gates_[f][1]})
        _, states = oracle.rollout(frames, *phis)
        finals.append(states)
    for f in range(4):
        np.testing.assert_array_equal(finals[0][f], finals[1][f])
        np.testing.assert_array_equal(finals[0][f], finals[2][f])


def test_p8_bruteforce_rollout():
    """P8: the oracle's whole rollout (reads on every pass, clean-pass commits,
    frame-level access) equals explicit scalar loops on tiny inputs, with
    distinct denoise and clean inputs so that committing a noisy pass, reading
    the post-commit state, or mixing frames all fail."""
    g = _rs(15)
    B, H, T, d, F, P = 1, 2, 5, 4, 4, 3
    phis = [g.standard_normal((H, d, d)) for _ in range(3)]
    frames = []
    for f in range(F):
        passes = [tuple(g.standard_normal((B, H, T, d)) for _ in range(3)) for _ in range(P)]
        frames.append({"passes": passes, "beta": g.uniform(0, 0.3, (B, H, T)),
                       "alpha": g.uniform(0.5, 1, (B, H))})
    scale = 1.0 / math.sqrt(d)
    outs, states = oracle.rollout(frames, *phis)
    for h in range(H):
        bframes = []
        for fr in frames:
            bframes.append({
                "passes": [tuple(x[0, h].tolist() for x in p) for p in fr["passes"]],
                "beta": fr["beta"][0, h].tolist(), "alpha": float(fr["alpha"][0, h])})
        bouts, bstates = bf.rollout(bframes, phis[0][h].tolist(), phis[1][h].tolist(),
                                    phis[2][h].tolist(), scale)
        for f in range(F + 1):
            np.testing.assert_allclose(states[f][0, h], np.array(bstates[f]), rtol=0, atol=1e-12)
        for key, val in bouts.items():
            for name in ("o", "o_intra", "o_inter"):
                np.testing.assert_allclose(outs[key][name][0, h], np.array(val[name]),
                                           rtol=0, atol=1e-12)


def test_fullkv_comparator_is_softmax_over_all_keys():
    """The comparator is plain softmax attention over the concatenated keys;
    with a single frame in the cache it equals the intra-frame branch."""
    g = _rs(16)
    q = g.standard_normal((1, 1, 4, 8))
    ks = [g.standard_normal((1, 1, 6, 8)) for _ in range(3)]
    vs = [g.standard_normal((1, 1, 6, 8)) for _ in range(3)]
    o = oracle.fullkv_attention(q, np.concatenate(ks, 2), np.concatenate(vs, 2))
    ref = bf.softmax_attention(q[0, 0].tolist(), np.concatenate(ks, 2)[0, 0].tolist(),
                               np.concatenate(vs, 2)[0, 0].tolist(), 1 / math.sqrt(8))
    np.testing.assert_allclose(o[0, 0], np.array(ref), rtol=0, atol=1e-13)
    np.testing.assert_allclose(oracle.fullkv_attention(q, ks[0], vs[0]),
                               oracle.intra_attention(q, ks[0], vs[0]), rtol=0, atol=0)


def test_planted_mistakes_are_caught():
    """A mistake planted in a copy of the commit (residual against alpha*S,
    the reading the pages do not print) changes the golden example, so the
    golden pin can tell the two readings apart."""
    gd = _load_golden("delta_rule_2x2.txt")
    S = _as_array(gd["S_prev"]); K = _as_array(gd["K"]); V = _as_array(gd["V"])
    beta = _as_array(gd["beta"])[0]; alpha = float(_as_array(gd["alpha"])[0, 0])
    decay_first = alpha * S + K.T @ np.diag(beta) @ (V - K @ (alpha * S))
    assert np.abs(decay_first - _as_array(gd["S_next"])).max() > 0.1


# ------------------------------------------------- KV-cache softmax layer, stack
def _frames(g, B, H, T, d, F, P):
    frames = []
    for _ in range(F):
        passes = [tuple(g.standard_normal((B, H, T, d)) for _ in range(3)) for _ in range(P)]
        frames.append({"passes": passes, "beta": g.uniform(0, 0.3, (B, H, T)),
                       "alpha": g.uniform(0.5, 1, (B, H))})
    return frames


def test_softmax_layer_bruteforce():
    """The KV-cache layer equals scalar loops over cached tokens: only clean
    passes enter the cache, in frame order, and each pass sees its own keys
    (caching a noisy pass, skipping the current pass or reversing the cache
    order fail)."""
    g = _rs(21)
    B, H, T, d, F, P = 1, 2, 3, 4, 3, 3
    frames = _frames(g, B, H, T, d, F, P)
    outs = oracle.softmax_layer_rollout(frames)
    for h in range(H):
        bframes = [{"passes": [tuple(x[0, h].tolist() for x in p) for p in fr["passes"]]}
                   for fr in frames]
        bouts = bf.softmax_layer_rollout(bframes, 1 / math.sqrt(d))
        for key, val in bouts.items():
            np.testing.assert_allclose(outs[key][0, h], np.array(val), rtol=0, atol=1e-12)


def test_softmax_layer_first_frame_and_uniform_cache():
    """Frame 0 has an empty cache, so it is the intra-frame softmax; with all
    keys zero every weight is equal and O is the mean of the cached clean V
    rows and the pass's own V rows."""
    g = _rs(22)
    B, H, T, d, F, P = 1, 1, 4, 3, 3, 2
    frames = _frames(g, B, H, T, d, F, P)
    outs = oracle.softmax_layer_rollout(frames)
    for p, (q, k, v) in enumerate(frames[0]["passes"]):
        np.testing.assert_allclose(outs[(0, p)], oracle.intra_attention(q, k, v), rtol=0, atol=0)
    for fr in frames:
        fr["passes"] = [(q, np.zeros_like(k), v) for (q, k, v) in fr["passes"]]
    outs = oracle.softmax_layer_rollout(frames)
    clean_v = [fr["passes"][-1][2] for fr in frames]
    for f in range(F):
        for p, (_, _, v) in enumerate(frames[f]["passes"]):
            rows = np.concatenate(clean_v[:f] + [v], axis=2)
            mean = np.broadcast_to(rows.mean(axis=2, keepdims=True), outs[(f, p)].shape)
            np.testing.assert_allclose(outs[(f, p)], mean, rtol=0, atol=1e-14)


def test_hybrid_stack_composes_its_layers():
    """A stack with a mixed mask gives each layer exactly what that layer's
    own rollout gives, in layer order (swapping two layers' kinds or inputs
    fails)."""
    g = _rs(23)
    B, H, T, d, F, P = 1, 1, 3, 4, 3, 2
    layers = [{"frames": _frames(g, B, H, T, d, F, P),
               "phis": tuple(g.standard_normal((H, d, d)) for _ in range(3))} for _ in range(4)]
    mask = [True, False, False, True]
    res = oracle.hybrid_stack_rollout(layers, mask)
    for lay, is_arl2, r in zip(layers, mask, res):
        if is_arl2:
            outs, states = oracle.rollout(lay["frames"], *lay["phis"])
            for key in outs:
                np.testing.assert_array_equal(r["o"][key], outs[key]["o"])
            assert len(r["states"]) == F + 1
        else:
            ref = oracle.softmax_layer_rollout(lay["frames"])
            for key in ref:
                np.testing.assert_array_equal(r["o"][key], ref[key])
            assert "states" not in r


# ------------------------------------------------------ token-level access (A15)
def _tl_inputs(g, B, H, T, d, beta_hi=0.3):
    q, k, v = (g.standard_normal((B, H, T, d)) for _ in range(3))
    phis = [g.standard_normal((H, d, d)) / math.sqrt(d) for _ in range(3)]
    beta = g.uniform(0, beta_hi, (B, H, T))
    S = g.standard_normal((B, H, d, d)) * 0.3
    return q, k, v, phis, beta, S


def test_token_level_bruteforce():
    """Token-level read and end state equal scalar loops (reading a token's own
    update, or the pre-frame state for every token, fail)."""
    g = _rs(31)
    B, H, T, d = 1, 2, 5, 4
    q, k, v, phis, beta, S = _tl_inputs(g, B, H, T, d)
    r = oracle.token_level_read(q, k, v, *phis, beta, S)
    for h in range(H):
        o, St = bf.token_level_read(q[0, h].tolist(), k[0, h].tolist(), v[0, h].tolist(),
                                    phis[0][h].tolist(), phis[1][h].tolist(),
                                    phis[2][h].tolist(), beta[0, h].tolist(), S[0, h].tolist(),
                                    1 / math.sqrt(d))
        np.testing.assert_allclose(r["o_inter"][0, h], np.array(o), rtol=0, atol=1e-12)
        np.testing.assert_allclose(r["S_T"][0, h], np.array(St), rtol=0, atol=1e-12)


def test_token_level_chunk_closed_form():
    """The token recurrence in closed form over a chunk (the triangular-solve
    form a chunked kernel uses): U = (I + tril(diag(beta) K'K'^T, -1))^-1
    diag(beta) (V' - K' S0), O_inter = Q' S0 + tril(Q' K'^T, -1) U,
    S_T = S0 + K'^T U."""
    g = _rs(32)
    B, H, T, d = 1, 1, 7, 5
    q, k, v, phis, beta, S = _tl_inputs(g, B, H, T, d, beta_hi=0.9)
    r = oracle.token_level_read(q, k, v, *phis, beta, S)
    Qp = q[0, 0] @ phis[0][0]
    Kt = k[0, 0] @ phis[1][0]
    Kp = Kt / np.linalg.norm(Kt, axis=1, keepdims=True)
    Vp = v[0, 0] @ phis[2][0]
    b = beta[0, 0]
    A = np.eye(T) + np.tril(b[:, None] * (Kp @ Kp.T), -1)
    U = np.linalg.solve(A, b[:, None] * (Vp - Kp @ S[0, 0]))
    np.testing.assert_allclose(r["o_inter"][0, 0], Qp @ S[0, 0] + np.tril(Qp @ Kp.T, -1) @ U,
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["S_T"][0, 0], S[0, 0] + Kp.T @ U, rtol=0, atol=1e-12)


def test_token_level_reduces_to_frame_level():
    """T = 1: token-level and frame-level access coincide (read and commit).
    beta = 0: the reads coincide and the commit is pure decay. Orthonormal
    keys (phi_k = phi_v = I): the commits coincide, since no key sees another's
    update."""
    g = _rs(33)
    B, H, d = 1, 2, 4
    q, k, v, phis, beta, S = _tl_inputs(g, B, H, 1, d)
    alpha = g.uniform(0.5, 1, (B, H))
    frames = [{"passes": [(q, k, v)], "beta": beta, "alpha": alpha}]
    outs_t, st_t = oracle.token_level_rollout(frames, *phis, S0=S)
    outs_f, st_f = oracle.rollout(frames, *phis, S0=S)
    np.testing.assert_allclose(outs_t[(0, 0)]["o"], outs_f[(0, 0)]["o"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(st_t[1], st_f[1], rtol=0, atol=1e-13)
    T = 6
    q, k, v, phis, beta, S = _tl_inputs(g, B, H, T, d)
    r = oracle.token_level_read(q, k, v, *phis, np.zeros_like(beta), S)
    np.testing.assert_allclose(r["o"], oracle.read(q, k, v, phis[0], S)["o"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["S_T"], S, rtol=0, atol=0)
    eye = np.broadcast_to(np.eye(d), (H, d, d))
    korth = np.zeros((B, H, d, d))
    for h in range(H):
        korth[0, h] = np.linalg.qr(g.standard_normal((d, d)))[0].T     # orthonormal rows
    beta = g.uniform(0, 1, (B, H, d))
    alpha = g.uniform(0.5, 1, (B, H))
    frames = [{"passes": [(q[:, :, :d], korth, v[:, :, :d])], "beta": beta, "alpha": alpha}]
    _, st_t = oracle.token_level_rollout(frames, eye, eye, eye, S0=S)
    _, st_f = oracle.rollout(frames, eye, eye, eye, S0=S)
    np.testing.assert_allclose(st_t[1], st_f[1], rtol=0, atol=1e-12)


# ------------------------------------------------------ training-side gradients
# Every gradient of the oracle is pinned by central finite differences of the
# (already pinned) forward functions, in float64: for L = <W, f(x)> with a
# random W, dL/dx_i ~ (L(x + h e_i) - L(x - h e_i)) / 2h, h = 1e-6 (truncation
# O(h^2), rounding O(1e-16 / h)), checked to 1e-6 relative on every
# coordinate of tiny inputs.

def _fd_check(loss, x, grad, name, h=1e-6, rel=1e-6, coords=None):
    x = np.asarray(x, dtype=np.float64)
    grad = np.asarray(grad, dtype=np.float64)
    assert grad.shape == x.shape, name
    flat = x.reshape(-1)
    idx = range(flat.size) if coords is None else coords
    fd = []
    an = []
    for i in idx:
        old = flat[i]
        flat[i] = old + h
        lp = loss()
        flat[i] = old - h
        lm = loss()
        flat[i] = old
        fd.append((lp - lm) / (2 * h))
        an.append(grad.reshape(-1)[i])
    fd, an = np.array(fd), np.array(an)
    scale = max(np.abs(fd).max(), 1e-30)
    assert np.abs(fd - an).max() <= rel * scale, f"{name}: {np.abs(fd - an).max():.3e} vs {scale:.3e}"


def test_intra_attention_backward_finite_differences():
    g = _rs(40)
    q, k, v = (g.standard_normal((2, 2, 5, 4)) for _ in range(3))
    W = g.standard_normal((2, 2, 5, 4))
    gr = oracle.intra_attention_backward(q, k, v, W, 0.7)
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        _fd_check(lambda: np.sum(W * oracle.intra_attention(q, k, v, 0.7)), x, gr[name], name)


def test_intra_attention_backward_closed_forms():
    """One key: the weights are the constant 1, so dQ = dK = 0 and dV = sum of
    dO over queries; identical value rows make O independent of the scores,
    so dQ = dK = 0 again."""
    g = _rs(41)
    q, k, v = (g.standard_normal((1, 2, 1, 4)) for _ in range(3))
    d_o = g.standard_normal((1, 2, 1, 4))
    gr = oracle.intra_attention_backward(q, k, v, d_o)
    assert np.abs(gr["dq"]).max() == 0 and np.abs(gr["dk"]).max() == 0
    assert np.allclose(gr["dv"], d_o)
    q, k = (g.standard_normal((1, 1, 6, 4)) for _ in range(2))
    v = np.repeat(g.standard_normal((1, 1, 1, 4)), 6, axis=2)
    gr = oracle.intra_attention_backward(q, k, v, g.standard_normal((1, 1, 6, 4)))
    assert np.abs(gr["dq"]).max() < 1e-12 and np.abs(gr["dk"]).max() < 1e-12


def test_read_backward_finite_differences():
    g = _rs(42)
    q, k, v = (g.standard_normal((2, 2, 5, 4)) for _ in range(3))
    phi_q = g.standard_normal((2, 4, 4)) * 0.5
    S = g.standard_normal((2, 2, 4, 4))
    W = g.standard_normal((2, 2, 5, 4))
    gr = oracle.read_backward(q, k, v, phi_q, S, W)

    def loss():
        return np.sum(W * oracle.read(q, k, v, phi_q, S)["o"])
    for name, x in (("dq", q), ("dk", k), ("dv", v), ("dphi_q", phi_q), ("dS", S)):
        _fd_check(loss, x, gr[name], name)


def test_commit_backward_finite_differences():
    g = _rs(43)
    B, H, T, d = 2, 2, 5, 4
    k, v = (g.standard_normal((B, H, T, d)) for _ in range(2))
    phi_k, phi_v = (g.standard_normal((H, d, d)) * 0.5 for _ in range(2))
    beta = g.uniform(0.1, 0.9, (B, H, T))
    alpha = g.uniform(0.5, 1.0, (B, H))
    S = g.standard_normal((B, H, d, d))
    G = g.standard_normal((B, H, d, d))
    gr = oracle.commit_backward(k, v, phi_k, phi_v, beta, alpha, S, G)

    def loss():
        return np.sum(G * oracle.commit(k, v, phi_k, phi_v, beta, alpha, S))
    for name, x in (("dk", k), ("dv", v), ("dphi_k", phi_k), ("dphi_v", phi_v),
                    ("dbeta", beta), ("dalpha", alpha), ("dS_prev", S)):
        _fd_check(loss, x, gr[name], name)


def test_commit_backward_closed_forms():
    """beta = 0: the commit is alpha S, so dS_prev = alpha G, dalpha = <S, G>
    and no gradient reaches K, V or the maps; dbeta is then the first-order
    change of <G, S_next>: rowsum((K'G) * (V' - K'S))."""
    g = _rs(44)
    B, H, T, d = 1, 2, 4, 3
    k, v = (g.standard_normal((B, H, T, d)) for _ in range(2))
    phi_k, phi_v = (g.standard_normal((H, d, d)) for _ in range(2))
    alpha = g.uniform(0.5, 1.0, (B, H))
    S, G = (g.standard_normal((B, H, d, d)) for _ in range(2))
    gr = oracle.commit_backward(k, v, phi_k, phi_v, np.zeros((B, H, T)), alpha, S, G)
    assert np.allclose(gr["dS_prev"], alpha[..., None, None] * G)
    assert np.allclose(gr["dalpha"], np.sum(S * G, axis=(-2, -1)))
    for name in ("dk", "dv", "dphi_k", "dphi_v"):
        assert np.abs(gr[name]).max() == 0, name
    kp = oracle.l2_normalize_rows(oracle.feature_map(k, phi_k))
    vp = oracle.feature_map(v, phi_v)
    expect = np.einsum("bhti,bhij,bhtj->bht", kp, G, vp - kp @ S)
    assert np.allclose(gr["dbeta"], expect)


def test_state_scan_is_the_rollout_commit_sequence():
    g = _rs(45)
    frames = _frames(g, 1, 2, 5, 3, 3, 2)
    phis = [g.standard_normal((2, 3, 3)) for _ in range(3)]
    _, states = oracle.rollout(frames, *phis)
    scanned = oracle.state_scan(frames, phis[1], phis[2])
    assert len(scanned) == len(states)
    for a, b in zip(scanned, states):
        assert np.array_equal(a, b)


def test_rollout_backward_finite_differences():
    """Gradients through the frame recurrence: every q, k, v of every pass,
    the gates of every frame, the three maps and S_0, for a loss on every
    pass's output of a 3-frame, 2-pass rollout."""
    g = _rs(46)
    B, H, T, d, F, P = 1, 2, 4, 3, 3, 2
    frames = _frames(g, B, H, T, d, F, P)
    phis = [g.standard_normal((H, d, d)) * 0.6 for _ in range(3)]
    S0 = g.standard_normal((B, H, d, d)) * 0.3
    W = {(f, p): g.standard_normal((B, H, T, d)) for f in range(F) for p in range(P)}
    Wfin = g.standard_normal((B, H, d, d))
    gr = oracle.rollout_backward(frames, *phis, W, S0=S0, dS_final=Wfin)

    def loss():
        outs, states = oracle.rollout(frames, *phis, S0=S0)
        return sum(np.sum(W[key] * r["o"]) for key, r in outs.items()) + np.sum(Wfin * states[-1])
    for f in range(F):
        for p in range(P):
            for j, name in enumerate(("dq", "dk", "dv")):
                _fd_check(loss, frames[f]["passes"][p][j], gr["d_passes"][(f, p)][j],
                          f"{name} f{f} p{p}")
        _fd_check(loss, frames[f]["beta"], gr["dbeta"][f], f"dbeta f{f}")
        _fd_check(loss, frames[f]["alpha"], gr["dalpha"][f], f"dalpha f{f}")
    for j, name in enumerate(("dphi_q", "dphi_k", "dphi_v")):
        _fd_check(loss, phis[j], gr[name], name)
    _fd_check(loss, S0, gr["dS0"], "dS0")
