"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: hand-worked
examples (tests/golden/), brute force on tiny inputs, a library routine that
the definition reduces to, closed forms and invariants, and statistical laws
of the verifier (acceptance probability sum_x min(p, q); emitted tokens follow
p).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy import stats

from oracle import dsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# a1 indexer
# ----------------------------------------------------------------------------
def test_index_scores_hand_example():
    g = _golden("index_scores_hand.json")
    s = O.index_scores(np.array(g["q"])[None], np.array(g["w"])[None],
                       np.array(g["keys"]), [g["row_len"]])
    np.testing.assert_array_equal(s[0], np.array(g["scores"]))


def test_index_scores_bruteforce_loops():
    rng = np.random.default_rng(11)
    R, H, D, L = 2, 3, 5, 9
    q = rng.integers(-4, 5, (R, H, D)).astype(float)
    w = rng.integers(0, 64, (R, H)) / 64.0
    keys = rng.integers(-4, 5, (L, D)).astype(float)
    row_len = [9, 4]
    s = O.index_scores(q, w, keys, row_len)
    for r in range(R):
        for t in range(L):
            if t >= row_len[r]:
                assert math.isnan(s[r, t])
                continue
            tot = 0.0
            for h in range(H):
                dot = 0.0
                for d in range(D):
                    dot += q[r, h, d] * keys[t, d]
                if dot > 0:
                    tot += w[r, h] * dot
            assert s[r, t] == tot   # integer/dyadic inputs: exact


def test_index_scores_single_head_is_relu_matmul_torch():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((1, 1, 16))
    keys = rng.standard_normal((40, 16))
    s = O.index_scores(q, np.ones((1, 1)), keys, [40])[0]
    ref = torch.relu(torch.from_numpy(keys) @ torch.from_numpy(q[0, 0])).numpy()
    np.testing.assert_allclose(s, ref, rtol=1e-13, atol=1e-13)


def test_index_scores_invariants():
    rng = np.random.default_rng(13)
    R, H, D, L = 1, 6, 8, 30
    q = rng.standard_normal((R, H, D))
    w = rng.random((R, H))
    keys = rng.standard_normal((L, D))
    s = O.index_scores(q, w, keys, [L])
    # head permutation applied to q and w together leaves s unchanged
    perm = rng.permutation(H)
    s2 = O.index_scores(q[:, perm], w[:, perm], keys, [L])
    np.testing.assert_allclose(s, s2, rtol=1e-12)
    # zero query -> zero scores
    assert np.all(O.index_scores(np.zeros_like(q), w, keys, [L]) == 0)
    # positive homogeneity in q (ReLU(c x) = c ReLU(x) for c > 0)
    np.testing.assert_allclose(O.index_scores(2.5 * q, w, keys, [L]), 2.5 * s, rtol=1e-12)
    # negating q flips which heads are active: s(q) + s(-q) = sum_h w_h |q_h.k|
    sneg = O.index_scores(-q, w, keys, [L])
    absdot = np.abs(np.einsum("hd,td->ht", q[0], keys))
    np.testing.assert_allclose(s[0] + sneg[0], w[0] @ absdot, rtol=1e-12)
    # scores are non-negative for non-negative weights
    assert np.all(s >= 0)


# ----------------------------------------------------------------------------
# a2 top-k
# ----------------------------------------------------------------------------
def test_topk_hand_example():
    g = _golden("topk_hand.json")
    s = np.array(g["scores"])
    for c in g["cases"]:
        np.testing.assert_array_equal(O.topk(s, len(s), c["k"]), c["idx"])


def _beats(s, a, b):
    """a is ranked above b: higher score, or equal score and lower position."""
    return s[a] > s[b] or (s[a] == s[b] and a < b)


@pytest.mark.parametrize("seed", range(6))
def test_topk_bruteforce_pairwise(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 14))
    k = int(rng.integers(1, 16))
    s = rng.integers(-3, 4, n).astype(float)        # many ties
    idx = O.topk(s, n, k)
    kept = [int(i) for i in idx if i >= 0]
    assert len(kept) == min(k, n)
    assert kept == sorted(kept)
    assert np.all(idx[len(kept):] == -1)
    dropped = [t for t in range(n) if t not in kept]
    for a in kept:
        for b in dropped:
            assert _beats(s, a, b)
    # exhaustive: the kept set is the unique subset of its size dominating the rest
    if n <= 10:
        winners = [c for c in itertools.combinations(range(n), min(k, n))
                   if all(_beats(s, a, b) for a in c for b in range(n) if b not in c)]
        assert winners == [tuple(kept)]


def test_topk_special_cases():
    L = 50
    np.testing.assert_array_equal(O.topk(np.full(L, 0.5), L, 7), np.arange(7))
    full = O.topk(np.random.default_rng(0).random(L), L, 64)
    np.testing.assert_array_equal(full[:L], np.arange(L))
    assert np.all(full[L:] == -1)
    # -0.0 and +0.0 are the same score: the lower position wins the tie
    s = np.array([1.0, 0.0, -0.0, -1.0])
    np.testing.assert_array_equal(O.topk(np.array([0.0, -0.0])[::-1], 2, 1), [0])
    np.testing.assert_array_equal(O.topk(s, 4, 2), [0, 1])
    # positions at or beyond row_len are never candidates
    s = np.array([0.0, 1.0, 9.0, 9.0])
    np.testing.assert_array_equal(O.topk(s, 2, 2), [0, 1])
    # empty row
    assert np.all(O.topk(np.zeros(3), 0, 4) == -1)


# ----------------------------------------------------------------------------
# a3 attention
# ----------------------------------------------------------------------------
def test_attention_hand_example():
    g = _golden("attention_hand.json")
    o, lse = O.sparse_attn(np.array(g["q"]), np.array(g["K"]), np.array(g["V"]),
                           np.array(g["idx"]), g["scale"])
    np.testing.assert_allclose(o, np.array(g["o"]), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(lse, np.array(g["lse"]), rtol=1e-14)


def _sdpa(q, K, V, pos, scale):
    """torch's scaled_dot_product_attention in float64 on the CPU, with the
    KV heads expanded to the query heads."""
    H_q = q.shape[0]
    H_kv = K.shape[1]
    Kt = torch.from_numpy(K[pos]).permute(1, 0, 2)          # [H_kv, n, D]
    Vt = torch.from_numpy(V[pos]).permute(1, 0, 2)
    Kt = Kt.repeat_interleave(H_q // H_kv, dim=0)
    Vt = Vt.repeat_interleave(H_q // H_kv, dim=0)
    qt = torch.from_numpy(q)[:, None, :]                       # [H_q, 1, D]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)
    lse = torch.logsumexp(scale * (qt @ Kt.transpose(1, 2))[:, 0, :], dim=-1)
    return o[:, 0, :].numpy(), lse.numpy()


@pytest.mark.parametrize("H_q,H_kv,Dqk,Dv", [(4, 4, 16, 16), (8, 2, 24, 16), (6, 1, 20, 12)])
def test_attention_matches_torch_sdpa(H_q, H_kv, Dqk, Dv):
    rng = np.random.default_rng(H_q * 100 + H_kv)
    L = 37
    q = rng.standard_normal((H_q, Dqk))
    K = rng.standard_normal((L, H_kv, Dqk))
    V = rng.standard_normal((L, H_kv, Dv))
    idx = np.array([3, 30, 7, 0, 22, -1, -1])
    o, lse = O.sparse_attn(q, K, V, idx, 0.3)
    o_ref, lse_ref = _sdpa(q, K, V, idx[idx >= 0], 0.3)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12)
    od, lsed = O.dense_attn(q, K, V, L, 0.3)
    o_ref, lse_ref = _sdpa(q, K, V, np.arange(L), 0.3)
    np.testing.assert_allclose(od, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lsed, lse_ref, rtol=1e-12)


def test_sparse_attention_reduces_to_dense_when_k_covers_context():
    rng = np.random.default_rng(21)
    L, H, D, I = 40, 3, 8, 4
    q_idx = rng.standard_normal((I, D))
    w = rng.random(I)
    keys = rng.standard_normal((L + 5, D))
    q = rng.standard_normal((2, H, D))
    K = rng.standard_normal((L + 5, H, D))
    V = rng.standard_normal((L + 5, H, D))
    idx, outs, lses = O.draft_block(q_idx, w, keys, L, 64, q, K, V, 0.25)
    for j in range(2):
        od, ld = O.dense_attn(q[j], K, V, L, 0.25)
        np.testing.assert_allclose(outs[j], od, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lses[j], ld, rtol=1e-12)


def test_attention_invariants():
    rng = np.random.default_rng(22)
    L, H, D = 25, 2, 6
    q = rng.standard_normal((H, D))
    K = rng.standard_normal((L, H, D))
    V = rng.standard_normal((L, H, D))
    # one selected position: output is that V row, lse its logit
    o, lse = O.sparse_attn(q, K, V, np.array([9, -1]), 0.5)
    np.testing.assert_allclose(o, V[9], rtol=1e-15)
    np.testing.assert_allclose(lse, 0.5 * np.einsum("hd,hd->h", q, K[9]), rtol=1e-14)
    # zero query: uniform weights -> mean of the selected V rows
    sel = np.array([1, 4, 17, 20])
    o, lse = O.sparse_attn(np.zeros_like(q), K, V, sel, 0.5)
    np.testing.assert_allclose(o, V[sel].mean(axis=0), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, np.log(4.0), rtol=1e-15)
    # set semantics: order of the indices does not matter
    o1, _ = O.sparse_attn(q, K, V, sel, 0.5)
    o2, _ = O.sparse_attn(q, K, V, sel[::-1], 0.5)
    np.testing.assert_allclose(o1, o2, rtol=1e-14)
    # empty selection
    o, lse = O.sparse_attn(q, K, V, np.array([-1, -1]), 0.5)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_index_share_steps_see_only_target_written_positions():
    """KVShare: with the draft-written slots poisoned (NaN), every draft step's
    output stays finite and equal to the clean run."""
    rng = np.random.default_rng(23)
    L, G, H, D, I = 30, 7, 2, 8, 2
    keys = rng.standard_normal((L + G, D))
    K = rng.standard_normal((L + G, H, D))
    V = rng.standard_normal((L + G, H, D))
    q_idx, w = rng.standard_normal((I, D)), rng.random(I)
    q = rng.standard_normal((G, H, D))
    idx, outs, _ = O.draft_block(q_idx, w, keys, L, 12, q, K, V, 0.3)
    keys_p, K_p, V_p = keys.copy(), K.copy(), V.copy()
    keys_p[L:] = np.nan
    K_p[L:] = np.nan
    V_p[L:] = np.nan
    idx_p, outs_p, _ = O.draft_block(q_idx, w, keys_p, L, 12, q, K_p, V_p, 0.3)
    np.testing.assert_array_equal(idx, idx_p)
    assert np.all(idx[idx >= 0] < L)
    assert np.all(np.isfinite(outs_p))
    np.testing.assert_array_equal(outs, outs_p)


def test_mixed_kv_control_sees_draft_written_slots():
    """Negative control (GLM-5.1 mixed KV): poisoning the draft-written slots
    leaves step 0 untouched but reaches every later step, the opposite of the
    KVShare invariant above."""
    rng = np.random.default_rng(24)
    L, G, H, D, I = 30, 7, 2, 8, 2
    keys = rng.standard_normal((L + G, D))
    K = rng.standard_normal((L + G, H, D))
    V = rng.standard_normal((L + G, H, D))
    q_idx, w = rng.standard_normal((I, D)), rng.random(I)
    q = rng.standard_normal((G, H, D))
    sets, outs, _ = O.mixed_kv_draft_block(q_idx, w, keys, L, 12, q, K, V, 0.3)
    idx, outs_share, _ = O.draft_block(q_idx, w, keys, L, 12, q, K, V, 0.3)
    for j in range(G):   # the sets: the selection plus exactly the j newest draft slots
        sel = sets[j][sets[j] >= 0]
        assert set(sel.tolist()) == set(idx[idx >= 0].tolist()) | set(range(L, L + j))
    np.testing.assert_array_equal(outs[0], outs_share[0])
    K_p, V_p = K.copy(), V.copy()
    K_p[L:] = np.nan
    V_p[L:] = np.nan
    _, outs_p, _ = O.mixed_kv_draft_block(q_idx, w, keys, L, 12, q, K_p, V_p, 0.3)
    np.testing.assert_array_equal(outs_p[0], outs[0])
    assert np.all(np.isnan(outs_p[1:]))


def test_mixed_kv_step_matches_torch_sdpa_over_union():
    rng = np.random.default_rng(25)
    L, G, H, D = 40, 5, 3, 16
    K = rng.standard_normal((L + G, H, D))
    V = rng.standard_normal((L + G, H, D))
    q = rng.standard_normal((H, D))
    idx = np.sort(rng.choice(L, 9, replace=False))
    sets = O.mixed_kv_sets(np.concatenate([idx, [-1, -1]]), L, G)
    for j in range(G):
        o, _ = O.sparse_attn(q, K, V, sets[j], 0.25)
        pos = np.concatenate([idx, np.arange(L, L + j)])
        Kt = torch.from_numpy(K[pos]).permute(1, 0, 2)[None]
        Vt = torch.from_numpy(V[pos]).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[None, :, None], Kt, Vt,
                                                               scale=0.25)[0, :, 0].numpy()
        np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_layer_block_reuses_one_selection():
    """Cross-layer IndexShare: every layer of the block uses the first
    layer's selection with its own queries and KV; a layer equals a
    stand-alone sparse attention over that selection."""
    rng = np.random.default_rng(26)
    L, n, H, D, I = 50, 4, 2, 8, 2
    keys = rng.standard_normal((L, D))
    Ks = rng.standard_normal((n, L, H, D))
    Vs = rng.standard_normal((n, L, H, D))
    qs = rng.standard_normal((n, H, D))
    q_idx, w = rng.standard_normal((I, D)), rng.random(I)
    idx, outs, _ = O.layer_block(q_idx, w, keys, L, 10, qs, Ks, Vs, 0.3)
    ref_idx = O.topk(O.index_scores(q_idx[None], w[None], keys, [L])[0], L, 10)
    np.testing.assert_array_equal(idx, ref_idx)
    for l in range(n):
        sel = idx[idx >= 0]
        Kt = torch.from_numpy(Ks[l][sel]).permute(1, 0, 2)[None]
        Vt = torch.from_numpy(Vs[l][sel]).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(qs[l])[None, :, None], Kt, Vt,
                                                               scale=0.3)[0, :, 0].numpy()
        np.testing.assert_allclose(outs[l], ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# a4 verification
# ----------------------------------------------------------------------------
def test_verify_hand_example():
    g = _golden("verify_hand.json")
    tl = np.log(np.array(g["p"]))
    dl = np.log(np.array(g["q"]))
    for c in g["cases"]:
        r = O.spec_verify_seq(tl, dl, g["draft"], c["u_accept"], c["u_sample"])
        assert r["n"] == c["n"]
        np.testing.assert_array_equal(r["emitted"], c["emitted"])
    p, q = np.array(g["p"][0]), np.array(g["q"][0])
    assert O.acceptance_probability(p, q) == pytest.approx(g["acceptance_probability"], abs=1e-15)
    assert O.total_variation(p, q) == pytest.approx(g["total_variation"], abs=1e-15)


def test_icdf_hand_and_zero_weights():
    w = np.array([1.0, 0.0, 2.0, 1.0])          # cumulative 1, 1, 3, 4
    assert O.icdf(w, 0.2)[0] == 0                # 0.8 < 1
    assert O.icdf(w, 0.25)[0] == 2               # 1.0 is not > 1: skips the zero weight
    assert O.icdf(w, 0.3)[0] == 2
    assert O.icdf(w, 0.75)[0] == 3               # 3.0 is not > 3
    assert O.icdf(w, 0.0)[0] == 0
    rng = np.random.default_rng(5)
    for _ in range(200):
        ww = rng.random(7) * (rng.random(7) < 0.5)
        if ww.sum() == 0:
            continue
        i, _ = O.icdf(ww, rng.random())
        assert ww[i] > 0


def test_acceptance_closed_form_identity():
    rng = np.random.default_rng(31)
    for _ in range(50):
        p = rng.dirichlet(np.ones(20))
        q = rng.dirichlet(np.ones(20))
        assert O.acceptance_probability(p, q) == pytest.approx(1 - O.total_variation(p, q), abs=1e-14)


def _probs(rng, V, std):
    return rng.standard_normal(V) * std


def test_accept_rate_matches_sum_min_binomial():
    """Kimi K3 section: sum_x min(p, q) is the exact acceptance probability."""
    rng = np.random.default_rng(41)
    V, M = 12, 40000
    tl = _probs(rng, V, 1.5)[None]
    dl = _probs(rng, V, 1.5)[None]
    p, q = O.softmax(tl[0]), O.softmax(dl[0])
    alpha = O.acceptance_probability(p, q)
    drafts = rng.choice(V, size=M, p=q)
    ua = rng.random(M)
    acc = 0
    for m in range(M):
        r = O.spec_verify_seq(np.vstack([tl, tl]), dl, [drafts[m]], [ua[m]], [0.5, 0.5])
        acc += r["n"]
    sigma = math.sqrt(alpha * (1 - alpha) / M)
    assert abs(acc / M - alpha) < 5 * sigma


def test_emitted_tokens_follow_target_distribution_chisquare():
    """Rejection sampling preserves the target distribution: the first emitted
    token ~ p_1, and the second (given the first draft was accepted) ~ p_2."""
    rng = np.random.default_rng(42)
    V, M, G = 10, 30000, 2
    tl = rng.standard_normal((G + 1, V)) * 1.2
    dl = rng.standard_normal((G, V)) * 1.2
    p = [O.softmax(tl[j]) for j in range(G + 1)]
    q = [O.softmax(dl[j]) for j in range(G)]
    first = np.zeros(V)
    second = np.zeros(V)
    for m in range(M):
        d = [rng.choice(V, p=q[j]) for j in range(G)]
        r = O.spec_verify_seq(tl, dl, d, rng.random(G), rng.random(G + 1))
        first[r["emitted"][0]] += 1
        if r["n"] >= 1:
            second[r["emitted"][1]] += 1
    for counts, pj in ((first, p[0]), (second, p[1])):
        exp = pj * counts.sum()
        assert exp.min() >= 5
        assert stats.chisquare(counts, exp).pvalue > 1e-3


def test_chain_length_law():
    """Independent positions: P(n >= m) = prod_{j<=m} alpha_j, so
    E[n] = sum_m prod_{j<=m} alpha_j."""
    rng = np.random.default_rng(43)
    V, M, G = 8, 20000, 4
    tl = rng.standard_normal((G + 1, V))
    dl = tl[:G] + rng.standard_normal((G, V)) * 0.8
    p = [O.softmax(tl[j]) for j in range(G)]
    q = [O.softmax(dl[j]) for j in range(G)]
    alphas = [O.acceptance_probability(p[j], q[j]) for j in range(G)]
    expected = sum(np.prod(alphas[: m + 1]) for m in range(G))
    ns = np.zeros(M)
    for m in range(M):
        d = [rng.choice(V, p=q[j]) for j in range(G)]
        ns[m] = O.spec_verify_seq(tl, dl, d, rng.random(G), rng.random(G + 1))["n"]
    se = ns.std() / math.sqrt(M)
    assert abs(ns.mean() - expected) < 5 * se


def test_verify_special_cases():
    rng = np.random.default_rng(44)
    V, G = 16, 7
    tl = rng.standard_normal((G + 1, V)) * 2
    # p = q: every draft accepted (u < 1), bonus drawn from p_{G+1}
    for _ in range(20):
        d = [int(rng.integers(V)) for _ in range(G)]
        us = rng.random(G + 1)
        r = O.spec_verify_seq(tl, tl[:G], d, rng.random(G), us)
        assert r["n"] == G
        assert list(r["emitted"][:G]) == d
        assert r["emitted"][G] == O.icdf(O.softmax(tl[G]), us[G])[0]
    # draft mass only where p = 0: always rejected, residual equals p
    tl2 = np.full((2, V), -np.inf)
    tl2[:, :8] = rng.standard_normal((2, 8))
    dl2 = np.full((1, V), -np.inf)
    dl2[0, 8:] = 0.0
    for _ in range(20):
        d = [int(rng.integers(8, V))]
        us = rng.random(2)
        r = O.spec_verify_seq(tl2, dl2, d, rng.random(1), us)
        assert r["n"] == 0
        assert r["emitted"][0] == O.icdf(O.softmax(tl2[0]), us[0])[0]
        assert r["emitted"][0] < 8
    # one-hot target: the emitted token is always its argmax
    tl3 = np.full((2, V), -np.inf)
    tl3[:, 5] = 0.0
    dl3 = rng.standard_normal((1, V))
    for _ in range(20):
        d = [int(rng.integers(V))]
        r = O.spec_verify_seq(tl3, dl3, d, rng.random(1), rng.random(2))
        assert r["emitted"][0] == 5
        assert r["n"] == (1 if d[0] == 5 else 0)


# ----------------------------------------------------------------------------
# f2 greedy verification
# ----------------------------------------------------------------------------
def _greedy_loops(tl, drafts):
    """Greedy verification with explicit loops: the first strictly larger
    logit moves the argmax, so equal maxima keep the lowest token id."""
    G = len(tl) - 1
    out = [-1] * (G + 1)

    def arg(row):
        best_i, best_v = 0, row[0]
        for i in range(1, len(row)):
            if row[i] > best_v:
                best_i, best_v = i, row[i]
        return best_i

    for j in range(G):
        a = arg(tl[j])
        out[j] = a
        if drafts[j] != a:
            return j, out
    out[G] = arg(tl[G])
    return G, out


@pytest.mark.parametrize("seed", range(6))
def test_greedy_verify_bruteforce(seed):
    rng = np.random.default_rng(900 + seed)
    G, V = (7, 15)[seed % 2], 12
    for _ in range(40):
        tl = rng.integers(-3, 4, size=(G + 1, V)).astype(np.float64)   # many ties
        best = [int(np.flatnonzero(r == r.max())[0]) for r in tl]
        # drafts agree with the argmax for a random prefix, then differ (or not)
        cut = int(rng.integers(0, G + 1))
        drafts = [best[j] if j < cut else int(rng.integers(V)) for j in range(G)]
        n, em = O.greedy_verify_seq(tl, drafts)
        n2, em2 = _greedy_loops(tl.tolist(), drafts)
        assert n == n2 and list(em) == em2
        assert n >= min(cut, G)


def test_greedy_verify_special_cases():
    tl = np.array([[0.0, 3.0, 3.0, 1.0],       # tie: lowest id (1) wins
                   [-0.0, 0.0, -1.0, -2.0],    # -0.0 == +0.0: id 0 wins
                   [5.0, 5.0, 5.0, 5.0]])      # all equal: id 0
    n, em = O.greedy_verify_seq(tl, [1, 0])
    assert n == 2 and list(em) == [1, 0, 0]
    n, em = O.greedy_verify_seq(tl, [2, 0])
    assert n == 0 and list(em) == [1, -1, -1]
    n, em = O.greedy_verify_seq(tl, [1, 3])
    assert n == 1 and list(em) == [1, 0, -1]


def test_greedy_equals_sampling_verify_for_one_hot_targets():
    """With one-hot target rows, rejection sampling (any draft logits, any
    uniforms) accepts a draft iff it is the target's argmax and resamples that
    argmax from the residual: it must coincide with greedy verification."""
    rng = np.random.default_rng(77)
    G, V = 7, 32
    for _ in range(50):
        hot = rng.integers(V, size=G + 1)
        tl = np.full((G + 1, V), -1e3)
        tl[np.arange(G + 1), hot] = 0.0   # exp(-1000) underflows: p is exactly one-hot
        dl = rng.standard_normal((G, V)) * 2
        cut = int(rng.integers(0, G + 1))
        drafts = [int(hot[j]) if j < cut else int(rng.integers(V)) for j in range(G)]
        r = O.spec_verify_seq(tl, dl, drafts, rng.random(G), rng.random(G + 1))
        n, em = O.greedy_verify_seq(tl, drafts)
        assert r["n"] == n
        assert list(r["emitted"]) == list(em)
