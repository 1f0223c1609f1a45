"""Focus oracle: a plain, slow, fp64 CPU statement of what the Focus inference path computes.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
bench.py may import this package. It shares no code with the HIP library and imports nothing
from it; the HIP library never imports, links or runs it.

Pages cited (all describe the method "Focus", arXiv 2604.03260):
  (ABS) "Why Attend to Everything? Focus is the Key", English abstract (arxivdaily.com).
  (NL)  Same title, Dutch technical summary (gist.science/nl), "Methodologie: Focus",
        "Kerncomponenten" items 1-4.
  (ZH)  Same title, Chinese technical summary (gist.science/zh), sections 2.1.1 (token
        grouping), 2.1.2 (gated attention, with its gate formula), 2.1.3 (top-k inference).
  (DE)  flowki-club.de blog post on Focus, section "Wie Focus funktioniert".

What the pages fix, and the reading taken where they are silent:
  * Scores: hidden states are projected into a d_g-dimensional group space and compared
    with K centroids C in R^{K x d_g} (ZH 2.1.1; NL Kerncomponenten 1). Reading: plain
    dot product S = (H W_g) C^T, no bias, norm or temperature; one W_g per layer shared
    by all heads, so memberships are per token.
  * Balance: Sinkhorn normalisation replaces softmax so that every group receives the same
    token mass (ZH 2.1.1; NL Kerncomponenten 2). Reading: log domain, unit temperature,
    u = v = 0 at the start, each iteration a row step (rows carry mass 1) then a column step
    (columns carry mass n/K), so the column masses are exact after the last iteration.
  * Membership: at inference each token belongs to its k highest-scoring groups (ZH 2.1.3;
    NL Kerncomponenten 4). Reading: scores are the balanced log-plan S + u + v (u cancels
    within a row); ties go to the lower group index; the set is reported in ascending order.
  * Pair rule: nearby tokens always attend; far tokens only if they share at least one
    group (ZH 2.1.2, 2.1.3; NL Kerncomponenten 3; DE "Wie Focus funktioniert").
    Reading: causal, key j <= query i, "nearby" means i - j < window.
  * Exact softmax over the allowed pairs (NL Kerncomponenten 3), each allowed pair once.
    Reading: scale 1/sqrt(d_head); lse is the natural log of the sum of exp(scaled logits).
  * GQA (NL Belangrijkste Bijdragen 3; ZH 3.2): query head h reads kv head h // (Hq/Hkv).
  * Asymmetric top-k (NL Resultaten, "Inferentie": each token looks at 2 of the 4 groups for
    a 2x speed-up; ZH 4 table, top-k trade-off): reading used: every key sits in its top-1
    group only, a query looks at its k groups, and a far pair is allowed when the key's group
    is one of the query's. This is what makes "2 of 4 groups" halve the far pairs.
  * Soft gate (ZH 2.1.2 formula): the printed form multiplies the logit by the gate, which
    cannot approach a hard mask; reading used: the gate multiplies the weight exp(q.k),
    i.e. adds log(sigmoid(lambda * a_ij)) to the logit of far pairs, with group affinity
    a_ij = 1[share] - 1/2. Both forms are provided; only the weight form is pinned.

Precision: inputs are taken as given (bf16 Q/K/V widened exactly); all arithmetic is fp64.
"""
import itertools
import math

import numpy as np

TIE_REL = 1e-5
# A relative gap of TIE_REL between balanced plan entries exp(b) is a log-domain gap of
# -log(1 - TIE_REL) between the balanced scores b.
TIE_LOG = -math.log1p(-TIE_REL)


# ------------------------------------------------------------------ small helpers
def _widen(x):
    """bf16 bit patterns (uint16) or floats -> float64, exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _logsumexp(x, axis):
    m = np.max(x, axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return np.squeeze(m, axis) + np.log(np.sum(np.exp(x - m), axis=axis))


# ------------------------------------------------------------------ stage A: assignment
def scores_ref(hidden, w_g, centroids, chunk=16384):
    """S[i, c] = (h_i W_g) . C_c in fp64 (ZH 2.1.1: projection, then similarity to centroids).

    Rows are independent; they are processed in chunks only to bound host memory.
    """
    w = np.asarray(w_g, np.float64)
    c = np.asarray(centroids, np.float64)
    n = hidden.shape[0]
    S = np.empty((n, c.shape[0]), np.float64)
    for r0 in range(0, n, chunk):
        z = np.asarray(hidden[r0:r0 + chunk], np.float64) @ w
        S[r0:r0 + chunk] = z @ c.T
    return S


def sinkhorn_ref(S, iters):
    """Log-domain Sinkhorn on the score matrix S [n, K] (ZH 2.1.1; NL Kerncomponenten 2).

    Returns the potentials (u [n], v [K]) such that the plan P = exp(S + u + v) has column
    sums n/K after the last column step. Each iteration: u_i = -logsumexp_c(S_ic + v_c),
    then v_c = log(n/K) - logsumexp_i(S_ic + u_i).
    """
    n, K = S.shape
    u = np.zeros(n)
    v = np.zeros(K)
    log_col_mass = math.log(n / K) if n > 0 else 0.0
    for _ in range(iters):
        u = -_logsumexp(S + v[None, :], axis=1)
        v = log_col_mass - _logsumexp(S + u[:, None], axis=0)
    return u, v


def topk_ref(b, top_k):
    """The top_k largest entries of each row of b (ZH 2.1.3), ties to the lower index.

    Returns (groups [n, top_k] int32 in ascending group order, tie [n] bool, gap [n]) where
    tie marks rows whose top_k-th and (top_k+1)-th balanced scores differ by less than
    TIE_REL relative (in the plan), i.e. TIE_LOG in the log domain.
    """
    n, K = b.shape
    order = np.argsort(-b, axis=1, kind="stable")
    groups = np.sort(order[:, :top_k], axis=1).astype(np.int32)
    if top_k < K:
        vals = np.take_along_axis(b, order[:, top_k - 1:top_k + 1], axis=1)
        gap = vals[:, 0] - vals[:, 1]
    else:
        gap = np.full(n, np.inf)
    return groups, gap < TIE_LOG, gap


def assign_ref(hidden, w_g, centroids, top_k, iters):
    """Full group assignment: scores, Sinkhorn, top-k (ZH 2.1.1 and 2.1.3)."""
    S = scores_ref(hidden, w_g, centroids)
    u, v = sinkhorn_ref(S, iters)
    b = S + v[None, :]  # u_i is constant within row i, so it does not change the ranking
    groups, tie, gap = topk_ref(b, top_k)
    return dict(S=S, u=u, v=v, groups=groups, tie=tie, gap=gap)


# ------------------------------------------------------------------ stage B: pair set
def allowed_keys_ref(i, groups, window, query_groups=None):
    """Keys j that query i may attend (ZH 2.1.2; NL Kerncomponenten 3).

    j <= i and (i - j < window or the two tokens share at least one group). The query's own
    groups default to groups[i]; `query_groups` overrides them (decode).
    """
    groups = np.asarray(groups)
    gi = groups[i] if query_groups is None else np.asarray(query_groups)
    j = np.arange(i + 1)
    local = (i - j) < window
    gj = groups[:i + 1]
    share = (gj[:, :, None] == gi[None, None, :]).any(axis=(1, 2))
    if query_groups is not None:
        share[i] = True  # the query token carries its own groups
    return j[local | share]


def owner_ref(i, j, groups, window):
    """Which pass owns allowed pair (i, j): -1 for the local window, else the lowest
    shared group; None if the pair is not allowed. Each allowed pair has exactly one owner.
    """
    if j > i:
        return None
    if i - j < window:
        return -1
    shared = set(int(g) for g in groups[i]) & set(int(g) for g in groups[j])
    return min(shared) if shared else None


def pair_count_ref(groups, window):
    """Exact number of allowed keys of every query, [n] int64, in O(n log n).

    count_i = min(i + 1, window) + #{j <= i - window : G_i and G_j intersect}; the second
    term is taken by inclusion-exclusion over the non-empty subsets of G_i, counting the
    earlier tokens whose group set contains each subset.
    """
    groups = np.asarray(groups, np.int64)
    n, k = groups.shape
    K = int(groups.max()) + 1 if n else 1
    pos = np.arange(n, dtype=np.int64)
    counts = np.minimum(pos + 1, window).astype(np.int64)
    limit = pos - window  # far keys are j <= limit
    for s in range(1, k + 1):
        sign = 1 if s % 2 == 1 else -1
        assert K ** s * (n + 1) < 2 ** 62, "subset codes overflow int64"
        combos = list(itertools.combinations(range(k), s))
        # code of every s-subset of every token's (ascending) group list
        codes = np.stack([np.zeros(n, np.int64) + sum(groups[:, c] * K ** (s - 1 - t)
                                                       for t, c in enumerate(cb))
                          for cb in combos], axis=1)  # [n, C(k,s)]
        table = np.sort((codes * (n + 1) + pos[:, None]).ravel())
        lo = np.searchsorted(table, codes * (n + 1), side="left")
        hi = np.searchsorted(table, codes * (n + 1) + np.maximum(limit, -1)[:, None], side="right")
        far = np.where(limit[:, None] >= 0, hi - lo, 0)
        counts += sign * far.sum(axis=1)
    return counts


# ------------------------------------------------------------------ stage C: attention
def attention_rows_ref(q, k, v, groups, window, scale=None, rows=None):
    """Exact masked softmax attention for the given query rows (NL Kerncomponenten 3).

    q [n, Hq, dh], k and v [n, Hkv, dh] (bf16 bit patterns or floats); groups [n, top_k].
    Returns (out [len(rows), Hq, dh], lse [len(rows), Hq]) in fp64; lse is the natural log
    of the sum over the allowed keys of exp(scale * q.k).
    """
    n, Hq, dh = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(dh) if scale is None or scale <= 0 else float(scale)
    rows = np.arange(n) if rows is None else np.asarray(rows)
    kv_of = np.arange(Hq) // G
    out = np.empty((len(rows), Hq, v.shape[2]))
    lse = np.empty((len(rows), Hq))
    for r, i in enumerate(rows):
        J = allowed_keys_ref(int(i), groups, window)
        qi = _widen(q[i])                       # [Hq, dh]
        kj = _widen(k[J])[:, kv_of, :]          # [|J|, Hq, dh]
        vj = _widen(v[J])[:, kv_of, :]
        s = scale * np.einsum("hd,jhd->hj", qi, kj)
        l = _logsumexp(s, axis=1)
        p = np.exp(s - l[:, None])
        out[r] = np.einsum("hj,jhd->hd", p, vj)
        lse[r] = l
    return out, lse


def decode_ref(q, q_groups, k_cache, v_cache, cache_len, cache_groups, window, scale=None):
    """One new token per sequence against its cache (ZH 2.1.3 inference; NL Kerncomponenten 4).

    Sequence b's query sits at position L_b - 1 of its cache (its K/V already appended) and
    carries the groups q_groups[b]; it attends keys j <= L_b - 1 under the same pair rule.
    Returns (out [B, Hq, dh], lse [B, Hq]).
    """
    B, Hq, dh = q.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(dh) if scale is None or scale <= 0 else float(scale)
    kv_of = np.arange(Hq) // G
    out = np.empty((B, Hq, v_cache.shape[3]))
    lse = np.empty((B, Hq))
    for b in range(B):
        p = int(cache_len[b]) - 1
        J = allowed_keys_ref(p, cache_groups[b], window, query_groups=q_groups[b])
        qi = _widen(q[b])
        kj = _widen(k_cache[b][J])[:, kv_of, :]
        vj = _widen(v_cache[b][J])[:, kv_of, :]
        s = scale * np.einsum("hd,jhd->hj", qi, kj)
        l = _logsumexp(s, axis=1)
        out[b] = np.einsum("hj,jhd->hd", np.exp(s - l[:, None]), vj)
        lse[b] = l
    return out, lse


# ------------------------------------------------------------------ asymmetric top-k variant
def allowed_keys_asym_ref(i, q_groups, k_group, window):
    """Keys j that query i may attend under the asymmetric top-k reading (NL Resultaten,
    "Inferentie"; ZH 4 table): j <= i and (i - j < window or k_group[j] is one of the
    query's groups q_groups[i]). k_group [n] is each token's single key group (its top-1),
    q_groups [n, k] the groups each token looks at as a query.
    """
    looked_at = np.asarray(q_groups)[i]
    j = np.arange(i + 1)
    local = (i - j) < window
    far_ok = np.isin(np.asarray(k_group).reshape(-1)[:i + 1], looked_at)
    return j[local | far_ok]


def pair_count_asym_ref(q_groups, k_group, window):
    """Exact allowed-key count of every query under the asymmetric rule, [n] int64:
    min(i + 1, window) plus, for each distinct group g the query looks at, the number of keys
    j <= i - window whose key group is g (one ascending position list per group, searched).
    """
    q_groups = np.asarray(q_groups, np.int64)
    k_group = np.asarray(k_group, np.int64).reshape(-1)
    n = q_groups.shape[0]
    pos = np.arange(n, dtype=np.int64)
    counts = np.minimum(pos + 1, window).astype(np.int64)
    members = {int(g): pos[k_group == g] for g in np.unique(k_group)}
    for i in range(n):
        limit = i - window
        if limit < 0:
            continue
        for g in set(int(x) for x in q_groups[i]):
            if g in members:
                counts[i] += int(np.searchsorted(members[g], limit, side="right"))
    return counts


def attention_rows_asym_ref(q, k, v, q_groups, k_group, window, scale=None, rows=None):
    """Exact masked softmax attention under the asymmetric top-k rule for the given query rows
    (NL Kerncomponenten 3 with the pair set of allowed_keys_asym_ref). Shapes and outputs as
    attention_rows_ref: (out [len(rows), Hq, dh], lse [len(rows), Hq]) in fp64. A row with no
    allowed key (possible only at window 0) has lse -inf and out 0.
    """
    n, Hq, dh = q.shape
    G = Hq // k.shape[1]
    scale = 1.0 / math.sqrt(dh) if scale is None or scale <= 0 else float(scale)
    rows = np.arange(n) if rows is None else np.asarray(rows)
    kv_of = np.arange(Hq) // G
    out = np.empty((len(rows), Hq, v.shape[2]))
    lse = np.empty((len(rows), Hq))
    for r, i in enumerate(rows):
        J = allowed_keys_asym_ref(int(i), q_groups, k_group, window)
        if len(J) == 0:  # window 0 and the token's key group outside its query groups
            out[r], lse[r] = 0.0, -np.inf
            continue
        qi = _widen(q[i])
        kj = _widen(k[J])[:, kv_of, :]
        vj = _widen(v[J])[:, kv_of, :]
        s = scale * np.einsum("hd,jhd->hj", qi, kj)
        l = _logsumexp(s, axis=1)
        out[r] = np.einsum("hj,jhd->hd", np.exp(s - l[:, None]), vj)
        lse[r] = l
    return out, lse


# ------------------------------------------------------------------ training-time soft gate
def _soft_gate_logits(q, k, groups, window, lam, scale, literal):
    n, Hq, dh = q.shape
    G = Hq // k.shape[1]
    scale = 1.0 / math.sqrt(dh) if scale is None or scale <= 0 else float(scale)
    kv_of = np.arange(Hq) // G
    qq = _widen(q)
    kk = _widen(k)[:, kv_of, :]
    s = scale * np.einsum("ihd,jhd->hij", qq, kk)             # [Hq, n, n]
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    local = (i - j) < window
    g = np.asarray(groups)
    share = (g[:, None, :, None] == g[None, :, None, :]).any(axis=(2, 3))
    a = share.astype(np.float64) - 0.5                         # group affinity
    log_gate = -np.logaddexp(0.0, -lam * a)                    # log sigmoid(lambda * a)
    if literal:
        s = s * np.where(local, 1.0, np.exp(log_gate))[None]
    else:
        s = s + np.where(local, 0.0, log_gate)[None]
    return np.where((j <= i)[None], s, -np.inf)


def soft_gate_ref(q, k, v, groups, window, lam, scale=None, literal=False, with_lse=False):
    """Training-time soft gate over all causal pairs (ZH 2.1.2 formula), weight reading by
    default; literal=True applies the printed form (gate multiplies the logit).
    Returns out [n, Hq, dh], and lse [n, Hq] (natural log of the sum of exp of the gated
    logits) as well when with_lse.
    """
    s = _soft_gate_logits(q, k, groups, window, lam, scale, literal)
    G = q.shape[1] // k.shape[1]
    vv = _widen(v)[:, np.arange(q.shape[1]) // G, :]
    lse = _logsumexp(s, axis=2)                                 # [Hq, n]
    p = np.exp(s - lse[:, :, None])
    out = np.einsum("hij,jhd->ihd", p, vv)
    return (out, lse.T.copy()) if with_lse else out
