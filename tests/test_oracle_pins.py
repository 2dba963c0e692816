"""Pins for the CPU oracle, each against something other than the oracle itself:
values printed on the SnapKV observation-window page, exact rational
arithmetic from the page's printed exp-weight tables, closed forms, brute force
over subsets, and PyTorch CPU float64 library routines."""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import snapkv_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def weights_to_inputs(rows, placeholder, L):
    """Keys whose coordinate i is ln(w_i[j]) and queries sqrt(D) * e_i, so that
    q_i . k_j / sqrt(D) = ln w_i[j] (the page's construction)."""
    W = len(rows)
    D = W
    K = np.zeros((L, D))
    for i, row in enumerate(rows):
        for j, w in enumerate(row):
            K[j, i] = math.log(placeholder if w is None else w)
    Q = np.zeros((W, D))
    for i in range(W):
        Q[i, i] = math.sqrt(D)
    return Q, K


def exact_votes(rows, P):
    """Votes and row sums as exact rationals straight from exp-weights: row i
    sees positions j <= P + i (None marks the causal future)."""
    sums = []
    votes = [Fraction(0)] * P
    for i, row in enumerate(rows):
        vis = [Fraction(w) for w in row[: P + i + 1]]
        Z = sum(vis)
        sums.append(Z)
        for j in range(P):
            votes[j] += vis[j] / Z
    return votes, sums


def exact_pool(votes, k, pooling):
    P, r = len(votes), k // 2
    out = []
    for j in range(P):
        nb = [votes[p] for p in range(j - r, j + r + 1) if 0 <= p < P]
        out.append(sum(nb, Fraction(0)) / k if pooling == "avg" else max(nb))
    return out


def exact_top(pooled, n):
    return sorted(sorted(range(len(pooled)), key=lambda j: (-pooled[j], j))[:n])


# ------------------------------------------------------------- worked example

def worked():
    g = load("worked_example.json")
    rows = [g["exp_weight_rows"]["query_6"], g["exp_weight_rows"]["query_7"]]
    Q, K = weights_to_inputs(rows, g["masked_placeholder"], g["L"])
    V = np.array([[j, -j] for j in range(g["L"])], dtype=np.float64)
    return g, rows, Q, K, V


def test_worked_example_page_values():
    g, rows, Q, K, V = worked()
    r = O.snapkv_select(Q, K, V, g["W"], g["C"], g["kernel"], g["pooling"])
    assert r["indices"].tolist() == g["expected_indices"]
    assert r["values"].tolist() == g["expected_values"]
    np.testing.assert_array_equal(r["keys"], K[g["expected_indices"]])
    # Row sums 25 and 26 in exp-weight units: Z_i * exp(m_i).
    got = r["row_sum"] * np.exp(r["row_max"])
    np.testing.assert_allclose(got, [g["row_sums"]["query_6"], g["row_sums"]["query_7"]], rtol=1e-13)
    assert int(np.argmax(r["votes"])) == g["raw_vote_argmax"]
    assert int(np.argmax(r["pooled"])) == g["pooled_argmax"]
    # Position 4 is lifted by its neighbour 3: above position 1 after pooling
    # although its raw vote is below position 1's.
    assert r["votes"][4] < r["votes"][1] and r["pooled"][4] > r["pooled"][1]


def test_worked_example_exact_rationals():
    g, rows, Q, K, V = worked()
    P = g["L"] - g["W"]
    ev, sums = exact_votes(rows, P)
    assert sums == [25, 26]
    assert ev == [Fraction(n, 650) for n in (51, 77, 460, 508, 51, 51)]
    ep = exact_pool(ev, 3, "avg")
    assert ep == [Fraction(n, 1950) for n in (128, 588, 1045, 1019, 610, 102)]
    r = O.snapkv_select(Q, K, V, g["W"], g["C"], 3, "avg")
    np.testing.assert_allclose(r["votes"], [float(x) for x in ev], rtol=1e-14)
    np.testing.assert_allclose(r["pooled"], [float(x) for x in ep], rtol=1e-14)
    # Other widths and modes on the same page data, exact expectations.
    for k, pooling, C in [(1, "avg", 5), (3, "max", 5), (3, "max", 4), (5, "avg", 5), (5, "max", 3)]:
        expect = exact_top(exact_pool(ev, k, pooling), C - g["W"])
        r = O.snapkv_select(Q, K, V, g["W"], C, k, pooling)
        assert r["indices"].tolist() == expect + [6, 7], (k, pooling, C)
    # Specific consequences: width 1 picks {1,2,3}; max-3 with C=4 is a
    # three-way tie (2,3,4 at 508/650) resolved to the lowest indices.
    assert O.snapkv_select(Q, K, V, 2, 5, 1, "avg")["indices"].tolist() == [1, 2, 3, 6, 7]
    r = O.snapkv_select(Q, K, V, 2, 4, 3, "max")
    assert r["indices"].tolist() == [2, 3, 6, 7]
    assert r["pooled"][2] == r["pooled"][3] == r["pooled"][4]


@pytest.mark.parametrize("placeholder", [1e-6, 1.0, 1e6])
def test_worked_example_masked_entry_has_no_effect(placeholder):
    g, rows, Q, K, V = worked()
    Q2, K2 = weights_to_inputs(rows, placeholder, g["L"])
    a = O.snapkv_select(Q, K, V, 2, 5, 3, "avg")
    b = O.snapkv_select(Q2, K2, V, 2, 5, 3, "avg")
    np.testing.assert_allclose(b["votes"], a["votes"], rtol=1e-14)
    np.testing.assert_allclose(b["row_sum"] * np.exp(b["row_max"]), [25, 26], rtol=1e-13)
    assert b["indices"].tolist() == a["indices"].tolist()


# ------------------------------------------------------------- counterexample

def counter():
    g = load("counterexample.json")
    rows = [g["exp_weight_rows"]["query_2"], g["exp_weight_rows"]["query_3"]]
    Q, K = weights_to_inputs(rows, g["masked_placeholder"], g["L"])
    V = np.arange(2 * g["L"], dtype=np.float64).reshape(g["L"], 2)
    return g, rows, Q, K, V


def check_counterexample(select_fn):
    g, rows, Q, K, V = counter()
    p = g["printed"]["full_softmax"]
    r = select_fn(Q, K, V, g["W"], g["C"], 1, "avg")
    np.testing.assert_allclose(r["votes"], [p["A_vote"], p["B_vote"]], rtol=1e-12)
    pick = g["positions"][p["pick"]]
    assert r["indices"].tolist() == [pick, 2, 3]


def test_counterexample_full_softmax_picks_B():
    g, rows, Q, K, V = counter()
    # The reconstructed weights reproduce all eight printed probabilities.
    full, prefix = g["printed"]["full_softmax"], g["printed"]["prefix_only"]
    ev, _ = exact_votes(rows, 2)
    assert [float(x) for x in ev] == pytest.approx([full["A_vote"], full["B_vote"]], rel=1e-15)
    pre = [[Fraction(w) / sum(Fraction(x) for x in row[:2]) for w in row[:2]] for row in rows]
    assert [float(pre[0][0]), float(pre[1][0])] == pytest.approx(prefix["A_terms"])
    assert [float(pre[0][1]), float(pre[1][1])] == pytest.approx(prefix["B_terms"])
    check_counterexample(O.snapkv_select)
    # Per-row terms of the full softmax, against the printed ones.
    r = O.snapkv_select(Q, K, V, 2, 3, 1, "avg")
    L, P = 4, 2
    logits = O.window_logits(Q, K)
    m, Z = O.causal_row_stats(logits, P)
    probs = O.attention_probs(logits, P, m, Z)
    np.testing.assert_allclose(probs[:, 0], full["A_terms"], rtol=1e-12)
    np.testing.assert_allclose(probs[:, 1], full["B_terms"], rtol=1e-12)
    assert r["votes"][1] > r["votes"][0]


def test_negative_control_prefix_only_normalisation_is_caught(monkeypatch):
    """Plant the page's wrong variant (softmax renormalised over the prefix
    columns only) into the oracle: the counterexample pin must reject it."""
    def prefix_only(logits, P, m, Z):
        W, L = logits.shape
        probs = np.zeros((W, L))
        for i in range(W):
            w = np.exp(logits[i, :P] - logits[i, :P].max())
            probs[i, :P] = w / w.sum()
        return probs

    monkeypatch.setattr(O, "attention_probs", prefix_only)
    g, rows, Q, K, V = counter()
    r = O.snapkv_select(Q, K, V, 2, 3, 1, "avg")
    np.testing.assert_allclose(r["votes"], [1.15, 0.85], rtol=1e-12)
    assert r["indices"][0] == g["positions"]["A"]
    with pytest.raises(AssertionError):
        check_counterexample(O.snapkv_select)


def test_counterexample_avg3_is_an_exact_tie():
    g, rows, Q, K, V = counter()
    r = O.snapkv_select(Q, K, V, 2, 3, 3, "avg")
    assert r["pooled"][0] == r["pooled"][1]
    assert r["pooled"][0] == pytest.approx(1 / 3, rel=1e-15)
    assert r["indices"].tolist() == [0, 2, 3]


# ------------------------------------------------------------- handed-over row statistics

def test_worked_example_row_lse_and_votes():
    """The page's row sums 25 and 26 (in exp-weight units) are the row
    log-sum-exps ln 25 and ln 26; with them handed over, the votes are the
    page's, and so is the selection."""
    g, rows, Q, K, V = worked()
    P = g["L"] - g["W"]
    lse = O.row_log_sum_exp(O.window_logits(Q, K), P)
    np.testing.assert_allclose(lse, [math.log(25), math.log(26)], rtol=1e-14)
    r = O.snapkv_select_lse(Q, K, V, [math.log(25), math.log(26)], g["W"], g["C"], 3, "avg")
    np.testing.assert_allclose(r["votes"], [n / 650 for n in (51, 77, 460, 508, 51, 51)], rtol=1e-14)
    np.testing.assert_allclose(r["pooled"], [n / 1950 for n in (128, 588, 1045, 1019, 610, 102)], rtol=1e-14)
    assert r["indices"].tolist() == g["expected_indices"]
    assert r["values"].tolist() == g["expected_values"]


def test_counterexample_handed_over_normaliser():
    """The counterexample through handed-over statistics: the full-prompt
    normalisers (ln 100, ln 40 from the exp-weight rows) pick B with the
    printed votes; the page's wrong prefix-only normalisers (ln 10, ln 36)
    reproduce its wrong votes 1.15 / 0.85 and pick A."""
    g, rows, Q, K, V = counter()
    full, prefix = g["printed"]["full_softmax"], g["printed"]["prefix_only"]
    lse = O.row_log_sum_exp(O.window_logits(Q, K), 2)
    np.testing.assert_allclose(lse, [math.log(100), math.log(40)], rtol=1e-14)
    r = O.snapkv_select_lse(Q, K, V, lse, 2, 3, 1, "avg")
    np.testing.assert_allclose(r["votes"], [full["A_vote"], full["B_vote"]], rtol=1e-12)
    assert r["indices"].tolist() == [g["positions"][full["pick"]], 2, 3]
    r = O.snapkv_select_lse(Q, K, V, [math.log(10), math.log(36)], 2, 3, 1, "avg")
    np.testing.assert_allclose(r["votes"], [sum(prefix["A_terms"]), sum(prefix["B_terms"])], rtol=1e-12)
    assert r["indices"].tolist() == [g["positions"]["A"], 2, 3]


@pytest.mark.parametrize("L,W,D", [(17, 5, 4), (130, 32, 16)])
def test_row_lse_crosscheck_torch(L, W, D):
    """row_log_sum_exp equals PyTorch's float64 logsumexp over the causally
    masked logits, and the votes from it equal the column sums of PyTorch's
    full causal attention."""
    rng = np.random.default_rng(L * 7 + W)
    Qfull = rng.standard_normal((L, D)) * 2
    K = rng.standard_normal((L, D)) * 2
    V = rng.standard_normal((L, D))
    P = L - W
    q, k = torch.from_numpy(Qfull), torch.from_numpy(K)
    logits = ((q @ k.T) / math.sqrt(D)).masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
    ref_lse = torch.logsumexp(logits[P:], dim=-1).numpy()
    np.testing.assert_allclose(O.row_log_sum_exp(O.window_logits(Qfull[P:], K), P), ref_lse, rtol=1e-13)
    ref_votes = torch.softmax(logits, dim=-1)[P:, :P].sum(dim=0).numpy()
    r = O.snapkv_select_lse(Qfull[P:], K, V, ref_lse, W, W + 3, 1, "avg")
    np.testing.assert_allclose(r["votes"], ref_votes, rtol=1e-12)
    full = O.snapkv_select(Qfull[P:], K, V, W, W + 3, 1, "avg")
    assert r["indices"].tolist() == full["indices"].tolist()


def test_row_lse_shift_scales_rows():
    """An offset d added to row i's log-sum-exp scales that row's
    probabilities by exp(-d): the same offset on every row scales every vote,
    and the ranking does not change."""
    rng = np.random.default_rng(5)
    L, W, D = 40, 4, 8
    Q, K, V = rng.standard_normal((W, D)), rng.standard_normal((L, D)), rng.standard_normal((L, D))
    lse = O.row_log_sum_exp(O.window_logits(Q, K), L - W)
    base = O.snapkv_select_lse(Q, K, V, lse, W, 12, 3, "max")
    half = O.snapkv_select_lse(Q, K, V, lse + math.log(2), W, 12, 3, "max")
    np.testing.assert_allclose(half["votes"], base["votes"] / 2, rtol=1e-13)
    assert half["indices"].tolist() == base["indices"].tolist()
    one = O.snapkv_select_lse(Q, K, V, lse + np.array([0, 0, math.log(3), 0]), W, 12, 3, "max")
    probs = O.attention_probs(O.window_logits(Q, K), L - W, *O.causal_row_stats(O.window_logits(Q, K), L - W))
    np.testing.assert_allclose(one["votes"], base["votes"] - probs[2, : L - W] * (2 / 3), rtol=1e-12)


# ------------------------------------------------------------- grouped query heads

def test_gqa_matches_repeat_interleave_expansion():
    """Query head h reads key/value head h // G: the result equals expanding
    K and V with PyTorch's repeat_interleave over the head axis (what the
    model's key/value repetition does) and selecting per query head."""
    rng = np.random.default_rng(11)
    Hq, Hkv, L, W, D = 6, 2, 60, 4, 8
    Q = rng.standard_normal((Hq, W, D))
    K = rng.standard_normal((Hkv, L, D)) * 1.5
    V = rng.standard_normal((Hkv, L, D))
    got = O.snapkv_select_gqa(Q, K, V, W, 20, 3, "avg")
    Ke = torch.from_numpy(K).repeat_interleave(Hq // Hkv, dim=0).numpy()
    Ve = torch.from_numpy(V).repeat_interleave(Hq // Hkv, dim=0).numpy()
    ref = O.snapkv_select_heads(Q, Ke, Ve, W, 20, 3, "avg")
    for h in range(Hq):
        assert got[h]["indices"].tolist() == ref[h]["indices"].tolist()
        np.testing.assert_array_equal(got[h]["votes"], ref[h]["votes"])
        np.testing.assert_array_equal(got[h]["values"], ref[h]["values"])
    # heads of one group differ (their own queries), heads of different groups read different keys
    assert got[0]["indices"].tolist() != got[1]["indices"].tolist() or not np.array_equal(got[0]["votes"], got[1]["votes"])
    with pytest.raises(ValueError):
        O.snapkv_select_gqa(Q[:5], K, V, W, 20, 3, "avg")


def test_expanded_cache_ratio_page_example():
    """The page's GQA ledger: 32 query heads, 8 key/value heads, L = 16384,
    C = 1024 and 512 generated tokens keep 4/11 of the native cache (not the
    1/11 the sequence lengths alone suggest)."""
    assert O.expanded_cache_ratio(32, 8, 16384, 1024, 512) == pytest.approx(4 / 11, rel=1e-15)
    assert O.expanded_cache_ratio(8, 8, 16384, 1024, 512) == pytest.approx(1 / 11, rel=1e-15)


@pytest.mark.parametrize("L,C", [(40, 60), (40, 40), (40, 39), (40, 9), (9, 9)])
def test_cache_ledger_after_decode(L, C):
    """The compressed cache serves decode: after the prefill selection a head
    holds min(L, C) prompt rows (all L when the prompt is shorter than the
    budget), and g generated tokens are appended to it, so the ledger reads
    min(L, C) + g rows; a refresh that keeps J of those J + g rows returns it
    to J (SnapKV page, section "prefill still reads the full K/V; the
    compressed cache serves decode"; counter-causal page, the refresh loop).
    The expanded GQA ledger counts the same rows per query head."""
    rng = np.random.default_rng(L * 100 + C)
    W, D = 8, 4
    q, k, v = (rng.standard_normal((n, D)) for n in (W, L, L))
    out = O.snapkv_select(q, k, v, W, C, 3, "avg")
    kept = len(out["indices"])
    assert kept == min(L, C) and len(out["keys"]) == kept and len(out["values"]) == kept
    for g in (0, 1, 7, 64):
        rows = kept + g                       # decode appends one row per generated token
        assert rows == min(L, C) + g
        scores = rng.random(rows)
        J = kept
        after = O.refresh_select(scores, J, min(2, J), 0)
        assert len(after) == J                # a refresh returns the cache to J rows
        assert O.expanded_cache_ratio(32, 8, L, C, g) == pytest.approx(32 * rows / (8 * (L + g)), rel=1e-15)


# ------------------------------------------------------------- refresh selection

@pytest.mark.parametrize("seed", range(6))
def test_refresh_select_bruteforce(seed):
    """Brute force over every subset of the middle region: the kept set is
    the protected head and tail plus the flexible subset of maximum score
    sum, lexicographically smallest among equal sums (the lowest-index tie
    rule), and it always holds exactly `keep` positions."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(4, 11))
    scores = rng.integers(0, 4, size=n).astype(np.float64)  # many exact ties
    for keep in range(1, n + 1):
        for head in range(0, keep + 1):
            for tail in range(0, keep - head + 1):
                got = O.refresh_select(scores, keep, head, tail)
                assert len(got) == keep and len(set(got.tolist())) == keep
                mid = list(range(head, n - tail))
                k = keep - head - tail
                best = None
                for sub in itertools.combinations(mid, k):
                    key = (-sum(scores[j] for j in sub), sub)
                    best = key if best is None or key < best else best
                expect = sorted(list(range(head)) + list(best[1]) + list(range(n - tail, n)))
                assert got.tolist() == expect, (scores.tolist(), keep, head, tail)


def test_refresh_select_rules():
    s = np.array([5.0, 1.0, 9.0, 9.0, 2.0, 7.0])
    assert O.refresh_select(s, 6, 0, 0).tolist() == [0, 1, 2, 3, 4, 5]   # keep everything
    assert O.refresh_select(s, 3, 1, 1).tolist() == [0, 2, 5]            # ties at 9: the lower index
    assert O.refresh_select(s, 2, 1, 1).tolist() == [0, 5]               # no flexible budget
    with pytest.raises(ValueError):
        O.refresh_select(s, 2, 2, 1)
    with pytest.raises(ValueError):
        O.refresh_select(s, 7, 0, 0)


# ------------------------------------------------------------- Jacap scores

def test_jacap_sensitivity_closed_forms():
    """The page's sensitivities: probabilities (0.5, 0.5) give
    alpha (1 - alpha) = 0.25, (0.99, 0.01) give 0.0099; a key set whose
    centre logits are equal gives alpha = 1/N exactly."""
    for probs, rho in (((0.5, 0.5), 0.25), ((0.99, 0.01), 0.0099)):
        z = np.log(np.array(probs))           # logits with these probabilities
        keys = np.zeros((2, 4))
        keys[:, 0] = z * 2.0                  # mu = e_0, tau = 1, sqrt(d_k) = 2
        sc = O.jacap_scores(keys, np.eye(2), np.eye(4)[0], np.ones(4), 1.0)
        np.testing.assert_allclose(sc["alpha"], probs, rtol=1e-13)
        np.testing.assert_allclose(sc["alpha"] * (1 - sc["alpha"]), rho, rtol=1e-12)
    sc = O.jacap_scores(np.ones((5, 3)), np.eye(5, 2), np.ones(3), np.ones(3), 0.7)
    np.testing.assert_allclose(sc["alpha"], 0.2, rtol=1e-14)


def test_jacap_logit_and_curvature_closed_forms():
    """Hand-computed values: keys (2, 0, 0, 0) and 0 with mu = e_0, tau = 0.5
    and d_k = 4 give centre logits 2 / (0.5 * 2) = 2 and 0, so alpha_0 =
    e^2 / (e^2 + 1); with Lambda = (3, 5, 7, 11) the key (1, 2, 0, 0) has
    kappa = 3 + 20 = 23; w = [alpha (1 - alpha)]^2 kappa / 4."""
    keys = np.array([[2.0, 0, 0, 0], [0.0, 0, 0, 0]])
    sc = O.jacap_scores(keys, np.eye(2), np.eye(4)[0], np.array([3.0, 5, 7, 11]), 0.5)
    np.testing.assert_allclose(sc["z"], [2.0, 0.0], rtol=1e-15)
    a0 = math.exp(2) / (math.exp(2) + 1)
    np.testing.assert_allclose(sc["alpha"], [a0, 1 - a0], rtol=1e-14)
    np.testing.assert_allclose(sc["kappa"], [12.0, 0.0], rtol=1e-15)      # 3 * 2^2
    sc = O.jacap_scores(np.array([[1.0, 2, 0, 0], [0.0, 0, 0, 0]]), np.eye(2), np.zeros(4),
                        np.array([3.0, 5, 7, 11]), 1.0)
    np.testing.assert_allclose(sc["kappa"], [23.0, 0.0], rtol=1e-15)
    np.testing.assert_allclose(sc["w"], [(0.25 ** 2) * 23 / 4, 0.0], rtol=1e-14)   # equal logits: alpha = 1/2


def test_jacap_saturated_token_keeps_its_sensitivity():
    """A centre probability within 1e-20 of one still has alpha (1 - alpha)
    equal to the other tokens' mass (here e^-50 of it), not zero: two
    tokens with logits 0 and -50 give 1 - alpha_0 = e^-50 / (1 + e^-50)."""
    keys = np.zeros((2, 4))
    keys[1, 0] = -100.0                         # z = -100 / (1 * 2) = -50 with mu = e_0, tau = 1
    sc = O.jacap_scores(keys, np.eye(2), np.eye(4)[0], np.ones(4), 1.0)
    q = math.exp(-50)
    np.testing.assert_allclose(sc["alpha"], [1 / (1 + q), q / (1 + q)], rtol=1e-15)
    rho0 = (1 / (1 + q)) * (q / (1 + q))
    assert rho0 > 0
    assert sc["w"][0] == 0.0                                                        # kappa_0 = 0 (zero key)
    sc = O.jacap_scores(keys + np.array([0, 1.0, 0, 0]), np.eye(2), np.eye(4)[0], np.ones(4), 1.0)
    np.testing.assert_allclose(sc["w"][0], rho0 ** 2 * 1.0 / 4, rtol=1e-12)        # kappa_0 = 1


def jacap_toy():
    """The page's 2-D miniature: u1 = (1, 0), u2 = (0.95, 0.05), u3 = (0, 1)
    with w = (1, 1, 0.7), realised through keys whose weights come out
    exactly so (equal centre logits, kappa scaled per token)."""
    u = np.array([[1.0, 0.0], [0.95, 0.05], [0.0, 1.0]])
    want_w = np.array([1.0, 1.0, 0.7])
    N, dk = 3, 4
    a = 1.0 / N
    rho2 = (a * (1 - a)) ** 2
    kappa = want_w * dk / rho2                  # w = rho^2 kappa / d_k
    keys = np.zeros((N, dk))
    keys[:, 1] = np.sqrt(kappa)                 # Lambda = e_1: kappa = k_1^2; mu = e_0: equal logits
    return keys, u, np.eye(dk)[0], np.eye(dk)[1], want_w


def test_jacap_leverage_toy_prefers_the_spanning_pair():
    """Independent weighting prefers tokens 1 and 2; leverage discounts
    token 2 (nearly collinear with token 1) and keeps tokens 1 and 3, which
    span both axes (the page's worked miniature)."""
    keys, u, mu, lam, w = jacap_toy()
    sc = O.jacap_scores(keys, u, mu, lam, 1.0)
    np.testing.assert_allclose(sc["w"], w, rtol=1e-12)
    A = np.eye(2) + sum(w[j] * np.outer(u[j], u[j]) for j in range(3))
    np.testing.assert_allclose(sc["A"], A, rtol=1e-14)
    assert sc["r"][2] > sc["r"][0] > sc["r"][1]
    r = O.jacap_select(keys, np.arange(6.0).reshape(3, 2), u, mu, lam, 1.0, keep=2)
    assert r["indices"].tolist() == [0, 2]
    assert sorted(np.argsort(-w, kind="stable")[:2].tolist()) == [0, 1]   # plain weighting would keep 1 and 2


@pytest.mark.parametrize("seed", range(4))
def test_jacap_determinant_lemma_and_sanity(seed):
    """r_i = det(A + w_i u_i u_i^T) / det(A) - 1 (the determinant lemma the
    page derives the leverage from), checked with explicit determinants;
    the page's sanity list: A symmetric positive definite, every w >= 0,
    scores finite, retained count equal to the budget after protection."""
    rng = np.random.default_rng(seed)
    N, dk, du = 9, 6, 5
    keys = rng.standard_normal((N, dk)) * 2
    outs = rng.standard_normal((N, du))
    mu = rng.standard_normal(dk)
    lam = rng.random(dk) * 2
    sc = O.jacap_scores(keys, outs, mu, lam, 0.8)
    A = sc["A"]
    detA = np.linalg.det(A)
    for i in range(N):
        lemma = np.linalg.det(A + sc["w"][i] * np.outer(outs[i], outs[i])) / detA - 1
        np.testing.assert_allclose(sc["r"][i], lemma, rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(A, A.T, rtol=0, atol=0)
    assert np.all(np.linalg.eigvalsh(A) >= 1 - 1e-12)
    assert np.all(sc["w"] >= 0) and np.all(np.isfinite(sc["r"]))
    sel = O.jacap_select(keys, keys, outs, mu, lam, 0.8, keep=5, protect_head=1, protect_tail=2)
    assert len(sel["indices"]) == 5 and sel["indices"][0] == 0 and sel["indices"][-2:].tolist() == [7, 8]


# ------------------------------------------------------------- closed forms

@pytest.mark.parametrize("L,W", [(10, 3), (64, 8), (257, 32)])
def test_uniform_closed_form(L, W):
    """All keys equal (or all window queries zero): row i is uniform over its
    P + i + 1 visible positions, so every prefix vote is H_L - H_P."""
    rng = np.random.default_rng(L)
    D, P = 8, L - W
    s_exact = sum(Fraction(1, P + i + 1) for i in range(W))
    if (L, W) == (10, 3):
        assert s_exact == Fraction(121, 360)
    Q = rng.standard_normal((W, D))
    K = np.tile(rng.standard_normal(D), (L, 1))
    V = rng.standard_normal((L, D))
    for (q, k) in [(Q, K), (np.zeros((W, D)), rng.standard_normal((L, D)))]:
        r = O.snapkv_select(q, k, V, W, W + 1, 3, "avg")
        np.testing.assert_allclose(r["votes"], float(s_exact), rtol=1e-13)
        expect = np.full(P, float(s_exact))
        expect[0] = expect[-1] = float(s_exact) * 2 / 3
        np.testing.assert_allclose(r["pooled"], expect, rtol=1e-13)
        r = O.snapkv_select(q, k, V, W, W + 1, 5, "max")
        np.testing.assert_allclose(r["pooled"], float(s_exact), rtol=1e-13)


def test_uniform_ties_go_to_lowest_index():
    L, W, D = 40, 4, 8
    P = L - W
    rng = np.random.default_rng(7)
    Q = rng.standard_normal((W, D))
    K = np.tile(rng.standard_normal(D), (L, 1))
    V = rng.standard_normal((L, D))
    for n in (1, 5, P - 2):
        r = O.snapkv_select(Q, K, V, W, W + n, 3, "avg")
        # interior positions tie exactly; the two edges are lower (2/3)
        assert r["indices"].tolist() == list(range(1, n + 1)) + list(range(P, L))
    r = O.snapkv_select(Q, K, V, W, W + P - 1, 3, "avg")
    assert r["indices"][:P - 1].tolist() == list(range(0, P - 1))


def test_identical_keys_give_bitwise_equal_votes():
    rng = np.random.default_rng(11)
    L, W, D = 300, 16, 32
    book = rng.standard_normal((5, D))
    codes = rng.integers(0, 5, size=L)
    K = book[codes]
    Q = rng.standard_normal((W, D))
    r = O.snapkv_select(Q, K, np.zeros((L, D)), W, W + 20, 5, "avg")
    P = L - W
    for c in range(5):
        vs = r["votes"][codes[:P] == c]
        assert np.all(vs == vs[0])
    # equal neighbour multisets give bitwise-equal pooled scores
    seen = {}
    for j in range(2, P - 2):
        key = tuple(sorted(codes[j - 2:j + 3]))
        if key in seen:
            assert r["pooled"][j] == seen[key]
        seen[key] = r["pooled"][j]


# ------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", range(12))
def test_bruteforce_subsets(seed):
    """Tiny prompts from integer exp-weights: the oracle's selection must be a
    maximum-sum (C-W)-subset of the exact pooled scores, and when the maximum
    is unique, exactly that subset."""
    rng = np.random.default_rng(1000 + seed)
    W = int(rng.integers(1, 4))
    L = int(rng.integers(W + 2, W + 10))
    P = L - W
    C = int(rng.integers(W + 1, L + 1))
    k = int(rng.choice([1, 3, 5]))
    pooling = str(rng.choice(["avg", "max"]))
    rows = [[int(x) for x in rng.integers(1, 60, size=L)] for _ in range(W)]
    for i in range(W):
        for j in range(P + i + 1, L):
            rows[i][j] = None
    Q, K = weights_to_inputs(rows, 1, L)
    V = rng.standard_normal((L, W))
    r = O.snapkv_select(Q, K, V, W, C, k, pooling)
    ev, _ = exact_votes(rows, P)
    ep = exact_pool(ev, k, pooling)
    n = C - W
    subsets = list(itertools.combinations(range(P), n))
    sums = [sum((ep[j] for j in s), Fraction(0)) for s in subsets]
    best = max(sums)
    winners = [s for s, t in zip(subsets, sums) if t == best]
    got = tuple(r["indices"][:n].tolist())
    assert got in winners
    if len(winners) == 1:
        assert got == winners[0]
    assert r["indices"][n:].tolist() == list(range(P, L))


def test_bruteforce_exact_ties_lowest_index():
    """Exact ties built from identical weight columns: among all maximum-sum
    subsets the oracle returns the lexicographically smallest, i.e. the
    lowest tied indices."""
    L, W = 9, 2
    P = L - W
    col = [3, 5, 3, 5, 5, 3, 5]
    rows = [[c for c in col] + [4, None], [c for c in col] + [4, 4]]
    Q, K = weights_to_inputs(rows, 1, L)
    V = np.zeros((L, 2))
    ev, _ = exact_votes(rows, P)
    for C in range(W + 1, L):
        n = C - W
        ep = exact_pool(ev, 1, "avg")
        subsets = list(itertools.combinations(range(P), n))
        sums = [sum((ep[j] for j in s), Fraction(0)) for s in subsets]
        best = min(s for s, t in zip(subsets, sums) if t == max(sums))
        r = O.snapkv_select(Q, K, V, W, C, 1, "avg")
        assert tuple(r["indices"][:n].tolist()) == best


# ------------------------------------------------------------- libraries

@pytest.mark.parametrize("L,W,D", [(17, 5, 4), (64, 16, 8), (130, 32, 16)])
def test_full_causal_attention_crosscheck(L, W, D):
    """Votes equal the column sums, over the last W rows, of the full L x L
    causal attention that PyTorch computes in float64 (softmax over a
    triangular mask)."""
    rng = np.random.default_rng(L * 31 + W)
    Qfull = rng.standard_normal((L, D)) * 2
    K = rng.standard_normal((L, D)) * 2
    V = rng.standard_normal((L, D))
    P = L - W
    q, k = torch.from_numpy(Qfull), torch.from_numpy(K)
    logits = (q @ k.T) / math.sqrt(D)
    mask = torch.triu(torch.ones(L, L, dtype=torch.bool), diagonal=1)
    att = torch.softmax(logits.masked_fill(mask, float("-inf")), dim=-1)
    ref_votes = att[P:, :P].sum(dim=0).numpy()
    r = O.snapkv_select(Qfull[P:], K, V, W, W + 1, 1, "avg")
    np.testing.assert_allclose(r["votes"], ref_votes, rtol=1e-12, atol=1e-300)
    lse = torch.logsumexp(logits.masked_fill(mask, float("-inf"))[P:], dim=-1).numpy()
    np.testing.assert_allclose(r["row_max"] + np.log(r["row_sum"]), lse, rtol=1e-13)
    np.testing.assert_allclose(r["row_max"], logits.masked_fill(mask, float("-inf"))[P:].max(dim=-1).values.numpy(), rtol=1e-14)


@pytest.mark.parametrize("k", [1, 3, 5, 7, 9])
@pytest.mark.parametrize("P", [1, 2, 6, 50])
def test_pool_crosscheck_torch(k, P):
    rng = np.random.default_rng(k * 100 + P)
    v = rng.random(P) ** 3
    t = torch.from_numpy(v)[None, None]
    r = k // 2
    if r <= k // 2 and P >= 1:
        ref_avg = torch.nn.functional.avg_pool1d(t, k, stride=1, padding=r, count_include_pad=True)[0, 0].numpy()
        ref_max = torch.nn.functional.max_pool1d(t, k, stride=1, padding=r)[0, 0].numpy()
        np.testing.assert_allclose(O.pool1d(v, k, "avg"), ref_avg, rtol=1e-15)
        np.testing.assert_array_equal(O.pool1d(v, k, "max"), ref_max)


def test_top_prefix_matches_python_sort():
    rng = np.random.default_rng(5)
    for _ in range(50):
        P = int(rng.integers(1, 200))
        s = rng.integers(0, 6, size=P).astype(np.float64)  # many exact ties
        n = int(rng.integers(1, P + 1))
        ref = sorted(sorted(range(P), key=lambda j: (-s[j], j))[:n])
        assert O.top_prefix(s, n).tolist() == ref


# ------------------------------------------------------------- invariants

def random_case(seed, L=200, W=16, D=32):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((W, D)) * 1.5, rng.standard_normal((L, D)) * 1.5,
            rng.standard_normal((L, D)))


@pytest.mark.parametrize("seed", range(4))
def test_invariants(seed):
    Q, K, V = random_case(seed)
    W, L, D = Q.shape[0], K.shape[0], K.shape[1]
    P = L - W
    C = 60
    r = O.snapkv_select(Q, K, V, W, C, 5, "avg")
    s = r["votes"]
    assert np.all(s >= 0) and np.all(s <= W)
    # total prefix vote = sum over rows of (1 - mass on window columns)
    logits = O.window_logits(Q, K)
    m, Z = O.causal_row_stats(logits, P)
    probs = O.attention_probs(logits, P, m, Z)
    np.testing.assert_allclose(probs.sum(axis=1), 1.0, rtol=1e-13)
    assert s.sum() == pytest.approx(W - probs[:, P:].sum(), rel=1e-12)
    # joint permutation of the head dimension
    perm = np.random.default_rng(seed).permutation(D)
    r2 = O.snapkv_select(Q[:, perm], K[:, perm], V, W, C, 5, "avg")
    np.testing.assert_allclose(r2["votes"], s, rtol=1e-12)
    assert r2["indices"].tolist() == r["indices"].tolist()
    # V affects only V'
    r3 = O.snapkv_select(Q, K, V * -3 + 1, W, C, 5, "avg")
    assert r3["indices"].tolist() == r["indices"].tolist()
    np.testing.assert_array_equal(r3["values"], (V * -3 + 1)[r["indices"]])
    # max pooling dominates the raw votes; window indices; pairing
    rm = O.snapkv_select(Q, K, V, W, C, 5, "max")
    assert np.all(rm["pooled"] >= rm["votes"])
    assert r["indices"][C - W:].tolist() == list(range(P, L))
    np.testing.assert_array_equal(r["keys"], K[r["indices"]])
    np.testing.assert_array_equal(r["values"], V[r["indices"]])
    assert len(set(r["indices"].tolist())) == C


def test_heads_are_independent():
    rng = np.random.default_rng(3)
    H, L, W, D = 3, 120, 8, 16
    Q = rng.standard_normal((H, W, D)) * 2
    K = rng.standard_normal((H, L, D)) * 2
    V = rng.standard_normal((H, L, D))
    res = O.snapkv_select_heads(Q, K, V, W, 30, 3, "avg")
    perm = [2, 0, 1]
    res_p = O.snapkv_select_heads(Q[perm], K[perm], V[perm], W, 30, 3, "avg")
    for a, h in zip(res_p, perm):
        assert a["indices"].tolist() == res[h]["indices"].tolist()
    assert len({tuple(r["indices"].tolist()) for r in res}) > 1


def test_bypass_and_full_budget():
    Q, K, V = random_case(9, L=50, W=10, D=8)
    r = O.snapkv_select(Q, K, V, 10, 51, 3, "avg")
    assert r["indices"].tolist() == list(range(50))
    np.testing.assert_array_equal(r["keys"], K)
    np.testing.assert_array_equal(r["values"], V)
    r = O.snapkv_select(Q, K, V, 10, 50, 3, "avg")
    assert r["indices"].tolist() == list(range(50))
    Qw = np.random.default_rng(4).standard_normal((50, 8))
    r = O.snapkv_select(Qw, K, V, 50, 51, 3, "max")  # W == L: empty prefix, bypass
    assert r["indices"].tolist() == list(range(50))


def test_window_equals_prompt_with_budget_equal():
    # W == L and C == L is rejected? No: C must exceed W, so C = L is invalid.
    Q, K, V = random_case(2, L=20, W=20, D=4)
    with pytest.raises(ValueError):
        O.snapkv_select(Q, K, V, 20, 20, 3, "avg")


@pytest.mark.parametrize("args", [
    dict(W=0), dict(W=51), dict(C=10), dict(C=5), dict(kernel=2), dict(kernel=0),
    dict(pooling="min"), dict(W=True),
])
def test_validation_rules(args):
    Q, K, V = random_case(1, L=50, W=10, D=8)
    kw = dict(W=10, C=20, kernel=3, pooling="avg")
    kw.update(args)
    q = Q if kw["W"] in (10, True) or not isinstance(kw["W"], int) else np.zeros((max(kw["W"], 0), 8))
    with pytest.raises(ValueError):
        O.snapkv_select(q, K, V, kw["W"], kw["C"], kw["kernel"], kw["pooling"])


def test_nonfinite_rejected():
    Q, K, V = random_case(1, L=50, W=10, D=8)
    K = K.copy()
    K[3, 2] = np.inf
    with pytest.raises(ValueError):
        O.snapkv_select(Q, K, V, 10, 20, 3, "avg")
