"""Focus oracle, training side: the soft-gated forward and the backward that trains only the
centroids and the projection. TEST INFRASTRUCTURE ONLY (same rules as focus_ref: imported by
tests/, __graft_entry__.smoke() and bench.py's oracle leg alone; shares no code with the HIP
library).

Pages: "Why Attend to Everything? Focus is the Key".
  (NL) Dutch technical summary (gist.science/nl), "Kerncomponenten" 1: a token is assigned to
       the groups through a soft assignment g_i, built from the affinity between the token and
       the centroids; 2: Sinkhorn normalisation is the balancing constraint during training;
       4: during training every pair is computed with soft gates.
  (ZH) Chinese technical summary (gist.science/zh), 2.1.1 (projection, similarity to the
       centroids, Sinkhorn in place of softmax), 2.1.2 (gate formula with the group affinity
       a_ij), 2.2 (only the centroids and the projection are trained; the model stays frozen).

Reading taken (the pages leave g_i and a_ij without formulas):
  * g_i is row i of the balanced Sinkhorn plan P = exp(S + u + v) after the iterations of
    focus_ref.sinkhorn_ref: the same plan whose top-k gives the hard memberships at inference.
  * a_ij = g_i . g_j - 1/2. With one-hot rows this is 1[same group] - 1/2, the hard reading of
    the gate used by focus_ref.soft_gate_ref; with soft rows it is the probability that the two
    tokens fall into the same group, centred.
  * Gate on the weight (as soft_gate_ref): far causal pairs (i - j >= window) add
    log sigmoid(lambda * a_ij) to the logit scale * q_i . k_j; near pairs add nothing.
  * Training is "frozen model": Q, K, V and the hidden states are inputs; the backward returns
    the gradients of L = sum(dO * O) (dO the caller's upstream gradient) with respect to the
    centroids C and the projection W_g, and the hidden states (for the layers below).

Every step is written in the forward's order and differentiated by hand, in fp64, with no
blocking or fusion.
"""
import math

import numpy as np

from .focus_ref import _logsumexp, _widen, scores_ref, sinkhorn_ref


# ------------------------------------------------------------------ forward pieces
def sinkhorn_iterates_ref(S, iters):
    """The potentials after every half-step: us[t-1] = u^t, vs[t] = v^t (vs[0] = 0), t = 1..T,
    from the iteration of sinkhorn_ref (row step with v^{t-1}, then column step with u^t)."""
    n, K = S.shape
    c = math.log(n / K) if n > 0 else 0.0
    vs = [np.zeros(K)]
    us = []
    for _ in range(iters):
        u = -_logsumexp(S + vs[-1][None, :], axis=1)
        v = c - _logsumexp(S + u[:, None], axis=0)
        us.append(u)
        vs.append(v)
    return us, vs


def soft_assignment_ref(hidden, w_g, centroids, iters):
    """g [n, K] = the balanced plan exp(S + u + v) (NL Kerncomponenten 1 and 2; ZH 2.1.1)."""
    S = scores_ref(hidden, w_g, centroids)
    u, v = sinkhorn_ref(S, iters)
    return np.exp(S + u[:, None] + v[None, :])


def soft_affinity_bias_ref(g, window, lam):
    """B [n, n] added to every head's logits: -inf where j > i, 0 where 0 <= i - j < window,
    log sigmoid(lam * (g_i . g_j - 1/2)) where i - j >= window (ZH 2.1.2 gate formula)."""
    g = np.asarray(g, np.float64)
    n = g.shape[0]
    a = g @ g.T - 0.5
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    far = (i - j) >= window
    B = np.where(far, -np.logaddexp(0.0, -lam * a), 0.0)
    return np.where(j <= i, B, -np.inf)


def biased_attention_ref(q, k, v, bias, scale=None):
    """out[i, h] = sum_j softmax_j(scale * q[i,h] . k[j,h/G] + bias[i, j]) v[j,h/G]; lse the
    natural log of the softmax denominator. q [n, Hq, dh], k and v [n, Hkv, dh]."""
    n, Hq, dh = q.shape
    G = Hq // k.shape[1]
    scale = 1.0 / math.sqrt(dh) if scale is None or scale <= 0 else float(scale)
    qq, kk, vv = _widen(q), _widen(k), _widen(v)
    out = np.empty((n, Hq, v.shape[2]))
    lse = np.empty((n, Hq))
    for h in range(Hq):
        s = scale * qq[:, h, :] @ kk[:, h // G, :].T + bias
        l = _logsumexp(s, axis=1)
        out[:, h, :] = np.exp(s - l[:, None]) @ vv[:, h // G, :]
        lse[:, h] = l
    return out, lse


def soft_train_forward_ref(hidden, w_g, centroids, iters, q, k, v, window, lam, scale=None):
    """The soft-gated training forward: returns (out [n, Hq, dh], lse [n, Hq], g [n, K])."""
    g = soft_assignment_ref(hidden, w_g, centroids, iters)
    out, lse = biased_attention_ref(q, k, v, soft_affinity_bias_ref(g, window, lam), scale)
    return out, lse, g


# ------------------------------------------------------------------ backward
def soft_train_backward_ref(hidden, w_g, centroids, iters, q, k, v, dout, window, lam,
                            scale=None):
    """Gradients of L = sum(dout * out) for out = soft_train_forward_ref(...)[0].

    Returns a dict with d_centroids [K, d_g], d_w_g [d, d_g], d_hidden [n, d] and the
    intermediate gradients d_plan (dL/dg, [n, K]) and d_scores (dL/dS, [n, K]).
    """
    H = np.asarray(hidden, np.float64)
    W = np.asarray(w_g, np.float64)
    C = np.asarray(centroids, np.float64)
    n, Hq, dh = q.shape
    G = Hq // k.shape[1]
    scale = 1.0 / math.sqrt(dh) if scale is None or scale <= 0 else float(scale)

    # forward, keeping what the backward needs
    Z = H @ W
    S = Z @ C.T
    us, vs = sinkhorn_iterates_ref(S, iters)
    u_last = us[-1] if iters > 0 else np.zeros(n)
    P = np.exp(S + u_last[:, None] + vs[-1][None, :])      # g
    a = P @ P.T - 0.5
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    causal = j <= i
    far = ((i - j) >= window) & causal
    B = np.where(far, -np.logaddexp(0.0, -lam * a), 0.0)
    B = np.where(causal, B, -np.inf)

    # attention: dB = sum over heads of the logit gradient P^h (dP^h - D^h)
    qq, kk, vv, do = _widen(q), _widen(k), _widen(v), _widen(dout)
    dB = np.zeros((n, n))
    for h in range(Hq):
        s = scale * qq[:, h, :] @ kk[:, h // G, :].T + B
        p = np.exp(s - _logsumexp(s, axis=1)[:, None])
        o = p @ vv[:, h // G, :]
        dp = do[:, h, :] @ vv[:, h // G, :].T
        D = np.sum(do[:, h, :] * o, axis=1)
        dB += p * (dp - D[:, None])

    # gate: d/da log sigmoid(lam a) = lam sigmoid(-lam a), on far pairs only
    dA = np.where(far, dB * lam * np.exp(-np.logaddexp(0.0, lam * a)), 0.0)
    # a = P P^T - 1/2
    dP = (dA + dA.T) @ P

    # P = exp(E), E = S + u^T + v^T
    dE = dP * P
    dS = dE.copy()
    du = dE.sum(axis=1)
    dv = dE.sum(axis=0)
    for t in range(iters, 0, -1):
        u_t, v_t, v_prev = us[t - 1], vs[t], vs[t - 1]
        # column step: v^t_c = log(n/K) - logsumexp_i(S_ic + u^t_i)
        Wc = np.exp(S + u_t[:, None] - _logsumexp(S + u_t[:, None], axis=0)[None, :])
        dS -= dv[None, :] * Wc
        du = du - Wc @ dv
        # row step: u^t_i = -logsumexp_c(S_ic + v^{t-1}_c)
        Wr = np.exp(S + v_prev[None, :] + u_t[:, None])
        dS -= du[:, None] * Wr
        dv = -(du @ Wr)     # dv^{t-1}: v^{t-1} feeds only this row step
        du = np.zeros(n)    # u^{t-1} feeds only the column step of iteration t-1
    # S = Z C^T, Z = H W
    dZ = dS @ C
    return dict(d_centroids=dS.T @ Z, d_w_g=H.T @ dZ, d_hidden=dZ @ W.T, d_plan=dP,
                d_scores=dS)


def soft_train_forward_rows_ref(g, q, k, v, window, lam, rows, scale=None):
    """soft_train_forward_ref's output on the given query rows only, from the soft assignment g
    (soft_assignment_ref): each row's gate biases are formed on their own, so long sequences can
    be checked on a sample of rows. Returns (out [len(rows), Hq, dh], lse [len(rows), Hq])."""
    g = np.asarray(g, np.float64)
    n, Hq, dh = q.shape
    G = Hq // k.shape[1]
    scale = 1.0 / math.sqrt(dh) if scale is None or scale <= 0 else float(scale)
    out = np.empty((len(rows), Hq, v.shape[2]))
    lse = np.empty((len(rows), Hq))
    for r, i in enumerate(rows):
        i = int(i)
        j = np.arange(i + 1)
        a = g[:i + 1] @ g[i] - 0.5
        bias = np.where((i - j) >= window, -np.logaddexp(0.0, -lam * a), 0.0)
        qi = _widen(q[i])
        for h in range(Hq):
            kk = _widen(k[:i + 1, h // G, :])
            s = scale * kk @ qi[h] + bias
            l = _logsumexp(s, axis=0)
            out[r, h] = np.exp(s - l) @ _widen(v[:i + 1, h // G, :])
            lse[r, h] = l
    return out, lse
