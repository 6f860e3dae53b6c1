"""Plain CPU oracle for the DSA draft-and-verify path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library and imports
nothing from it.

Everything is computed in float64 with NumPy, written as the plain definition
of each step so that it can be checked against the pages by eye.  Sources
("Optimizing speculative decoding" / "GLM-5.2: Tuning MTP speculative decoding
to the limit", both longformexplainers.com):

* DSA (glossary entry in the section "IndexShare and KVShare"): a light
  indexer scores every past token with dot products, a top-k keeps the most
  relevant positions, and full attention runs over that subset only.
* IndexShare / KVShare (same section): the indexer runs on the first draft
  step only; later steps reuse its top-k indices and therefore see only
  positions whose KV the target model wrote.
* Rejection sampling (section "Rejection sampling and a loss that optimizes
  acceptance directly"): drafts are sampled from the draft distribution q and
  accepted or rejected against the target distribution p, which preserves p.
  The Kimi K3 section states that sum_x min(p(x), q(x)) is the exact per-token
  acceptance probability.

The indexer's scoring form  s_t = sum_h w_h * ReLU(q_h . k_t)  and the
residual / bonus rule of the verifier are fixed by the problem statement this
library implements; the pages only say "cheap dot products" and "the exact
protocol".  Readings of points the pages leave open are listed in each
function's docstring.

Random numbers the verifier draws are *inputs* here (u_accept, u_sample): the
oracle never generates them.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "index_scores",
    "topk",
    "attention",
    "sparse_attn",
    "dense_attn",
    "draft_block",
    "layer_block",
    "mixed_kv_sets",
    "mixed_kv_draft_block",
    "softmax",
    "icdf",
    "spec_verify_seq",
    "spec_verify",
    "greedy_verify_seq",
    "greedy_verify",
    "acceptance_probability",
    "total_variation",
]


# ----------------------------------------------------------------------------
# a1: lightning-indexer scores
# ----------------------------------------------------------------------------
def index_scores(q, w, keys, row_len):
    """Indexer score of every visible past position.

    s[r, t] = sum_h w[r, h] * max(0, sum_d q[r, h, d] * keys[t, d])   for t < row_len[r]

    DSA glossary ("IndexShare and KVShare" section): the indexer scores every
    past token with cheap dot products.  One index key per position is shared
    by all indexer heads; each head has its own query and weight.

    q: [R, H, D]   w: [R, H]   keys: [L, D] (logical order)   row_len: [R]
    Returns float64 [R, L]; entries at t >= row_len[r] are NaN (undefined).
    """
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    R, H, D = q.shape
    L = keys.shape[0]
    out = np.full((R, L), np.nan)
    for r in range(R):
        n = int(row_len[r])
        if n == 0:
            continue
        dots = q[r] @ keys[:n].T                  # [H, n]: q_h . k_t
        relu = np.maximum(dots, 0.0)              # ReLU per head
        out[r, :n] = w[r] @ relu                  # sum_h w_h * ReLU(.)
    return out


# ----------------------------------------------------------------------------
# a2: top-k selection
# ----------------------------------------------------------------------------
def topk(scores, row_len, k):
    """Top-k positions of one score row.

    DSA glossary: a top-k selection keeps the most relevant past positions.
    Readings: candidates are exactly t in [0, row_len); ordering key is
    (score descending, position ascending), so equal scores keep the lower
    position; -0.0 equals +0.0 (real-valued comparison); when k >= row_len all
    positions are kept.  The kept set is returned in ascending position order,
    padded with -1 to length k.
    """
    n = int(row_len)
    s = np.asarray(scores, dtype=np.float64)[:n]
    if np.isnan(s).any():
        raise ValueError("NaN scores are outside the defined input domain")
    t = np.arange(n)
    order = np.lexsort((t, -s))                   # primary -s, secondary t
    keep = np.sort(order[: min(k, n)])
    out = np.full(k, -1, dtype=np.int64)
    out[: keep.size] = keep
    return out


# ----------------------------------------------------------------------------
# a3: attention over a selected position set
# ----------------------------------------------------------------------------
def attention(q, K, V, positions, scale):
    """Softmax attention of every query head over the given positions.

    q: [H_q, D_qk]; K: [L, H_kv, D_qk]; V: [L, H_kv, D_v]; positions: 1-D ints.
    Query head h reads KV head g = h // (H_q // H_kv).
    o_h   = sum_t softmax_t(scale * q_h . K[t, g]) * V[t, g]
    lse_h = log sum_t exp(scale * q_h . K[t, g])
    An empty position set gives o = 0 and lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    pos = np.asarray(positions, dtype=np.int64)
    H_q = q.shape[0]
    H_kv = K.shape[1]
    D_v = V.shape[2]
    group = H_q // H_kv
    o = np.zeros((H_q, D_v))
    lse = np.full(H_q, -np.inf)
    if pos.size == 0:
        return o, lse
    for h in range(H_q):
        g = h // group
        logits = scale * (K[pos, g, :] @ q[h])    # [n]
        m = logits.max()
        e = np.exp(logits - m)
        z = e.sum()
        o[h] = (e @ V[pos, g, :]) / z
        lse[h] = m + np.log(z)
    return o, lse


def sparse_attn(q, K, V, idx, scale):
    """DSA sparse attention: full attention over the selected set only.

    DSA glossary: full attention runs over only the top-k subset.
    idx is the top-k output (-1 marks padding and is ignored); the set is what
    matters, not its order.
    """
    idx = np.asarray(idx, dtype=np.int64)
    return attention(q, K, V, idx[idx >= 0], scale)


def dense_attn(q, K, V, L, scale):
    """Ordinary attention over every visible position [0, L)."""
    return attention(q, K, V, np.arange(int(L)), scale)


def draft_block(q_index, w, keys, L, k, q_steps, K, V, scale):
    """One drafted chain with IndexShare / KVShare.

    Section "IndexShare and KVShare": the indexer (and its top-k) runs on the
    first draft step only and every later step reuses that index set, so every
    step attends only to positions [0, L) whose KV the target wrote.
    q_index: [H_I, D_I]; w: [H_I]; keys: [L_total, D_I]; q_steps: [G, H_q, D_qk].
    Returns (idx [k], outs [G, H_q, D_v], lses [G, H_q]).
    """
    s = index_scores(np.asarray(q_index)[None], np.asarray(w)[None], keys, [L])[0]
    idx = topk(s, L, k)
    outs, lses = [], []
    for qj in q_steps:
        o, lse = sparse_attn(qj, K, V, idx, scale)
        outs.append(o)
        lses.append(lse)
    return idx, np.stack(outs), np.stack(lses)


def layer_block(q_index, w, keys, L, k, q_layers, K_layers, V_layers, scale):
    """Cross-layer IndexShare: one indexer serves a block of backbone layers.

    Section "IndexShare and KVShare" (and the IndexShare glossary entry): one
    indexer is shared across every four backbone layers; the first computes
    which past tokens matter and the rest reuse its top-k.  Each layer keeps
    its own queries and KV cache.  q_layers: [n, H_q, D_qk];
    K_layers / V_layers: [n, L_total, H_kv, D].  Returns (idx, outs [n, H_q,
    D_v], lses [n, H_q]).
    """
    s = index_scores(np.asarray(q_index)[None], np.asarray(w)[None], keys, [L])[0]
    idx = topk(s, L, k)
    outs, lses = [], []
    for q, K, V in zip(q_layers, K_layers, V_layers):
        o, lse = sparse_attn(q, K, V, idx, scale)
        outs.append(o)
        lses.append(lse)
    return idx, np.stack(outs), np.stack(lses)


def mixed_kv_sets(idx, L, G):
    """Index sets of the mixed-KV drafting the same section describes for
    GLM-5.1 (kept here as a negative control): draft step j (0-based) attends
    to the step-1 selection plus the draft-written slots L .. L+j-1, whose KV
    came from the MTP layer's own hidden states.  Returns [G, len(idx) + G - 1]
    index rows padded with -1."""
    idx = np.asarray(idx, dtype=np.int64)
    rows = np.full((G, len(idx) + G - 1), -1, dtype=np.int64)
    for j in range(G):
        sel = np.concatenate([idx[idx >= 0], np.arange(L, L + j)])
        rows[j, : len(sel)] = sel
    return rows


def mixed_kv_draft_block(q_index, w, keys, L, k, q_steps, K, V, scale):
    """The mixed-KV chain: like draft_block, but step j also sees slots
    L .. L+j-1 (mixed_kv_sets).  Returns (sets, outs [G, H_q, D_v], lses)."""
    s = index_scores(np.asarray(q_index)[None], np.asarray(w)[None], keys, [L])[0]
    sets = mixed_kv_sets(topk(s, L, k), L, len(q_steps))
    outs, lses = [], []
    for qj, sj in zip(q_steps, sets):
        o, lse = sparse_attn(qj, K, V, sj, scale)
        outs.append(o)
        lses.append(lse)
    return sets, np.stack(outs), np.stack(lses)


# ----------------------------------------------------------------------------
# a4: rejection-sampling verification
# ----------------------------------------------------------------------------
def softmax(logits):
    """Probability distribution of one logit row (temperature 1)."""
    x = np.asarray(logits, dtype=np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def icdf(weights, u):
    """Inverse-CDF draw from unnormalised non-negative weights.

    Returns the smallest i with sum_{t <= i} w_t > u * sum_t w_t, scanning the
    vocabulary in ascending index order, plus the draw's float64 margin: the
    distance of u*W to the nearest cumulative boundary of the chosen index,
    relative to W (tells near-boundary draws apart from clear ones).
    """
    w = np.asarray(weights, dtype=np.float64)
    c = np.cumsum(w)
    W = c[-1]
    x = u * W
    i = int(np.searchsorted(c, x, side="right"))
    lo = c[i - 1] if i > 0 else 0.0
    margin = min(x - lo, c[i] - x) / W
    return i, margin


def spec_verify_seq(target_logits, draft_logits, drafts, u_accept, u_sample):
    """Verify one drafted chain of G tokens.

    Section "Rejection sampling and a loss that optimizes acceptance
    directly": draft tokens are sampled from q and accepted/rejected against
    p; the protocol preserves p.  Kimi K3 section: sum_x min(p, q) is the exact
    per-token acceptance probability, i.e. draft d is accepted with
    probability min(1, p(d)/q(d)).

    Readings (the pages point to a protocol whose text is not included):
      * accept d_j iff u_accept[j] * q_j(d_j) < p_j(d_j), in order j = 1..G,
        stopping at the first rejection;
      * on a rejection at j, emit a draw from norm(max(0, p_j - q_j))
        (falling back to p_j when that residual has no mass) using u_sample[j];
      * when all G drafts are accepted emit a bonus draw from p_{G+1} using
        u_sample[G];
      * draws are inverse-CDF over ascending vocabulary index (icdf).

    target_logits: [G+1, V]; draft_logits: [G, V]; drafts: [G];
    u_accept: [G]; u_sample: [G+1].
    Returns dict with n (accepted drafts), emitted ([G+1], -1 padded),
    p_draft / q_draft ([G] probabilities of the drafted tokens, NaN past the
    decision point), accept_margin ([G] relative |u*q - p| / p of each decision
    taken) and sample_margin (margin of the final draw).
    """
    tl = np.asarray(target_logits, dtype=np.float64)
    dl = np.asarray(draft_logits, dtype=np.float64)
    G = dl.shape[0]
    emitted = np.full(G + 1, -1, dtype=np.int64)
    p_d = np.full(G, np.nan)
    q_d = np.full(G, np.nan)
    acc_margin = np.full(G, np.nan)
    for j in range(G):
        p = softmax(tl[j])
        q = softmax(dl[j])
        d = int(drafts[j])
        p_d[j], q_d[j] = p[d], q[d]
        lhs = float(u_accept[j]) * q[d]
        acc_margin[j] = abs(lhs - p[d]) / max(p[d], 1e-300)
        if lhs < p[d]:
            emitted[j] = d
            continue
        resid = np.maximum(p - q, 0.0)
        if resid.sum() <= 0.0:
            resid = p
        tok, margin = icdf(resid, float(u_sample[j]))
        emitted[j] = tok
        return dict(n=j, emitted=emitted, p_draft=p_d, q_draft=q_d,
                    accept_margin=acc_margin, sample_margin=margin)
    tok, margin = icdf(softmax(tl[G]), float(u_sample[G]))
    emitted[G] = tok
    return dict(n=G, emitted=emitted, p_draft=p_d, q_draft=q_d,
                accept_margin=acc_margin, sample_margin=margin)


def spec_verify(target_logits, draft_logits, drafts, u_accept, u_sample):
    """Batched spec_verify_seq.  Shapes [B, G+1, V], [B, G, V], [B, G],
    [B, G], [B, G+1].  Returns (n [B], emitted [B, G+1], list of per-sequence
    result dicts)."""
    B = np.asarray(drafts).shape[0]
    res = [spec_verify_seq(target_logits[b], draft_logits[b], drafts[b],
                           u_accept[b], u_sample[b]) for b in range(B)]
    n = np.array([r["n"] for r in res], dtype=np.int64)
    emitted = np.stack([r["emitted"] for r in res])
    return n, emitted, res


def greedy_verify_seq(target_logits, drafts):
    """Greedy verification of one drafted chain of G tokens.

    Section "Rejection sampling and a loss that optimizes acceptance
    directly" contrasts probabilistic drafting with greedy drafting, where
    the draft is the most likely token.  Reading: d_j is accepted iff it is
    the argmax of target row j; the first mismatch emits that argmax and
    stops; a fully accepted chain emits the argmax of target row G.  argmax
    picks the lowest token id among equal maxima (numpy's argmax does; softmax
    is monotone, so the argmax of the logits is that of p).

    target_logits: [G+1, V]; drafts: [G].  Returns (n, emitted [G+1], -1 padded).
    """
    tl = np.asarray(target_logits, dtype=np.float64)
    G = tl.shape[0] - 1
    emitted = np.full(G + 1, -1, dtype=np.int64)
    for j in range(G):
        best = int(np.argmax(tl[j]))
        if int(drafts[j]) != best:
            emitted[j] = best
            return j, emitted
        emitted[j] = best
    emitted[G] = int(np.argmax(tl[G]))
    return G, emitted


def greedy_verify(target_logits, drafts):
    """Batched greedy_verify_seq: [B, G+1, V], [B, G] -> (n [B], emitted [B, G+1])."""
    out = [greedy_verify_seq(target_logits[b], drafts[b]) for b in range(np.asarray(drafts).shape[0])]
    return np.array([o[0] for o in out], dtype=np.int64), np.stack([o[1] for o in out])


def acceptance_probability(p, q):
    """Kimi K3 section: sum_x min(p(x), q(x)), the per-token acceptance
    probability of lossless speculative sampling."""
    return float(np.minimum(np.asarray(p, np.float64), np.asarray(q, np.float64)).sum())


def total_variation(p, q):
    """Total-variation distance: half the summed absolute differences
    (glossary entry in the rejection-sampling section)."""
    return 0.5 * float(np.abs(np.asarray(p, np.float64) - np.asarray(q, np.float64)).sum())
