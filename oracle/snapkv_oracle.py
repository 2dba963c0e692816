"""Plain, slow CPU oracle for SnapKV observation-window KV selection.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from the package.

Source: the web page "SnapKV: selecting the KV cache for long prompts with an
observation window" (charlestar.github.io, 2026-10-20).  Each function below
cites the section of that page it restates.  Section names are English glosses
of the page's Chinese headings:

  * "the prompt cache shrinks, the positions keep their origin" (problem setup:
    L, W, P = L - W, budget C includes the window),
  * "votes must come from the causal softmax over the full prompt",
  * "pooling spreads a peak into a neighbourhood preference",
  * "one full selection computed from Q and K" (worked example, argument rules,
    short-prompt bypass, tie rule),
  * "prefill still reads the full K/V; the compressed cache serves decode"
    (bypass when L < C).

Precision: every floating-point step runs in float64 on values that are exact
upcasts of the caller's fp32 or bf16 bits.  The page evaluates its example in
Python floats with exactly rounded sums; this oracle keeps float64 but fixes
each summation order so that equal inputs give bitwise-equal outputs (this
matters for exact vote ties):

  * logits: sum over d = 0 .. D-1 in that order,
  * row normaliser Z_i: exactly rounded (math.fsum),
  * votes: sum over window rows i = 0 .. W-1 in that order,
  * avg pooling: the in-range neighbours are summed in ascending order of
    value (a function of the multiset of neighbours only), then divided by k.

Readings taken where the page is silent (each is also listed in the design doc):
  * selected prefix indices are returned in ascending order, followed by the
    window positions P .. L-1 (the page says storage order is free for
    single-query reads; its example emits score order),
  * max pooling takes the maximum of the in-range neighbours (padding never
    wins because every vote is >= 0 and the centre is always in range),
  * for L < C the whole prompt is kept (bypass), for L == C the whole prefix
    is selected, which gives the same indices.

Pins: tests/test_oracle_pins.py checks every function here against the page's
worked example and counterexample, exact rational arithmetic, closed forms,
brute force over subsets, and PyTorch CPU float64 library routines.
"""

from __future__ import annotations

import math
from typing import Dict, List, Sequence

import numpy as np

POOLINGS = ("avg", "max")


def validate(L: int, W: int, C: int, D: int, kernel: int, pooling: str) -> None:
    """Argument rules of the page's worked selection (section "one full
    selection computed from Q and K"): positive integers, window not longer
    than the prompt, budget strictly larger than the window, odd pooling
    width, avg or max pooling, positive head dimension."""
    for name, value in (("L", L), ("W", W), ("C", C), ("D", D), ("kernel", kernel)):
        if isinstance(value, bool) or not isinstance(value, (int, np.integer)) or value <= 0:
            raise ValueError(f"{name} must be a positive integer, got {value!r}")
    if W > L:
        raise ValueError("window must not exceed the prompt length")
    if C <= W:
        raise ValueError("budget C must exceed the window W")
    if kernel % 2 != 1:
        raise ValueError("pooling kernel width must be odd")
    if pooling not in POOLINGS:
        raise ValueError("pooling must be 'avg' or 'max'")


def window_logits(qwin: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Logits of the W window queries against all L prompt keys.

    Section "votes must come from the causal softmax over the full prompt":
    l[i, j] = (q_{P+i} . k_j) / sqrt(D).  The dot product is accumulated over
    d = 0 .. D-1 in that order, in float64.
    Returns a [W, L] float64 array (no mask applied here).
    """
    qwin = np.asarray(qwin, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    W, D = qwin.shape
    L, D2 = keys.shape
    if D != D2:
        raise ValueError("query and key head dimensions differ")
    acc = np.zeros((W, L), dtype=np.float64)
    for d in range(D):
        acc += np.multiply.outer(qwin[:, d], keys[:, d])
    logits = acc / math.sqrt(D)
    if not np.all(np.isfinite(logits)):
        raise ValueError("non-finite dot product")
    return logits


def causal_row_stats(logits: np.ndarray, P: int):
    """Per window row i (query position t = P + i) over the visible positions
    j <= t, which include every prefix position and the window positions up to
    t (section "votes must come from the causal softmax over the full prompt"):
        m_i = max_j l[i, j],   Z_i = sum_j exp(l[i, j] - m_i).
    Returns (m, Z), each [W] float64.
    """
    W = logits.shape[0]
    m = np.empty(W, dtype=np.float64)
    Z = np.empty(W, dtype=np.float64)
    for i in range(W):
        visible = logits[i, : P + i + 1]
        m[i] = visible.max()
        Z[i] = math.fsum(np.exp(visible - m[i]).tolist())
    return m, Z


def attention_probs(logits: np.ndarray, P: int, m: np.ndarray, Z: np.ndarray) -> np.ndarray:
    """Full causal softmax of the window rows: alpha[i, j] = exp(l - m_i) / Z_i
    for j <= P + i and exactly 0 for the masked future positions j > P + i
    (section "votes must come from the causal softmax over the full prompt")."""
    W, L = logits.shape
    probs = np.zeros((W, L), dtype=np.float64)
    for i in range(W):
        t = P + i
        probs[i, : t + 1] = np.exp(logits[i, : t + 1] - m[i]) / Z[i]
    return probs


def prefix_votes(probs: np.ndarray, P: int) -> np.ndarray:
    """Votes s_j = sum over window rows of alpha[i, j], for prefix columns
    j < P only, summed over i = 0 .. W-1 in that order (section "votes must come
    from the causal softmax over the full prompt")."""
    s = np.zeros(P, dtype=np.float64)
    for i in range(probs.shape[0]):
        s = s + probs[i, :P]
    return s


def pool1d(votes: np.ndarray, kernel: int, pooling: str) -> np.ndarray:
    """Stride-1 1-D pooling of the prefix votes with radius r = (k-1)/2
    (section "pooling spreads a peak into a neighbourhood preference").

    avg: out-of-range neighbours count as zero and the divisor is always k
         (PyTorch's count_include_pad=True edge rule).  The in-range
         neighbours are added in ascending order of value.
    max: maximum of the in-range neighbours.
    Neighbours are taken from the prefix only; window votes do not exist.
    """
    if pooling not in POOLINGS:
        raise ValueError("pooling must be 'avg' or 'max'")
    votes = np.asarray(votes, dtype=np.float64)
    P = votes.shape[0]
    r = kernel // 2
    # nb[j, o] = votes[j - r + o] when 0 <= j - r + o < P, else padding.
    pad = 0.0 if pooling == "avg" else -np.inf
    padded = np.concatenate([np.full(r, pad), votes, np.full(r, pad)])
    nb = np.stack([padded[o:o + P] for o in range(kernel)], axis=1)
    if pooling == "max":
        return nb.max(axis=1)
    # Votes are >= 0, so the zero padding sorts first and adding it is exact:
    # the running sum equals the ascending-order sum of the in-range values.
    nb = np.sort(nb, axis=1)
    total = np.zeros(P, dtype=np.float64)
    for o in range(kernel):
        total = total + nb[:, o]
    return total / kernel


def top_prefix(pooled: np.ndarray, count: int) -> np.ndarray:
    """The `count` prefix positions ranked first by (-pooled_j, j): highest
    pooled score first, equal scores broken towards the lowest index (section
    "one full selection computed from Q and K").  Returned in ascending index
    order (reading: storage order of kept positions is free)."""
    P = pooled.shape[0]
    order = np.lexsort((np.arange(P), -pooled))
    return np.sort(order[:count])


def snapkv_select(qwin, keys, values, W: int, C: int, kernel: int = 3, pooling: str = "avg") -> Dict:
    """SnapKV observation-window selection for one (sequence, head).

    qwin: [W, D] queries of the last W prompt positions (P .. L-1),
    keys, values: [L, D].
    Returns a dict with
      indices [min(L, C)] int64: ascending selected prefix positions, then
                                 the window positions P .. L-1,
      keys, values:              rows of K and V at those indices,
      votes [P], pooled [P]:     float64 (empty when the bypass applies),
      row_max [W], row_sum [W]:  float64 m_i and Z_i (empty for the bypass).
    """
    qwin = np.asarray(qwin, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    L, D = keys.shape
    if values.shape != keys.shape or qwin.shape != (W, D):
        raise ValueError("shape mismatch between Qwin, K and V")
    validate(L, W, C, D, kernel, pooling)
    for name, x in (("Qwin", qwin), ("K", keys), ("V", values)):
        if not np.all(np.isfinite(x)):
            raise ValueError(f"{name} must be finite")
    empty = np.zeros(0, dtype=np.float64)
    if L < C:
        # Short-prompt bypass: keep every position (sections "one full
        # selection computed from Q and K" and "prefill still reads the full
        # K/V; the compressed cache serves decode").
        idx = np.arange(L, dtype=np.int64)
        return {"indices": idx, "keys": keys.copy(), "values": values.copy(),
                "votes": empty, "pooled": empty, "row_max": empty, "row_sum": empty}
    P = L - W
    logits = window_logits(qwin, keys)
    m, Z = causal_row_stats(logits, P)
    probs = attention_probs(logits, P, m, Z)
    votes = prefix_votes(probs, P)
    pooled = pool1d(votes, kernel, pooling)
    chosen = top_prefix(pooled, C - W)
    idx = np.concatenate([chosen, np.arange(P, L)]).astype(np.int64)
    return {"indices": idx, "keys": keys[idx], "values": values[idx],
            "votes": votes, "pooled": pooled, "row_max": m, "row_sum": Z}


def row_log_sum_exp(logits: np.ndarray, P: int) -> np.ndarray:
    """Natural-log log-sum-exp of each window row over its visible positions
    j <= P + i: lse_i = ln sum_j exp(l[i, j]) = m_i + ln Z_i, the log of the
    softmax denominator of row i (section "votes must come from the causal
    softmax over the full prompt").  Prefill attention forms the same causal
    softmax for every prompt query over the full K (section "prefill still
    reads the full K/V; the compressed cache serves decode"), so these are the
    normalisers of its last W rows.  Returns [W] float64."""
    m, Z = causal_row_stats(logits, P)
    return m + np.log(Z)


def snapkv_select_lse(qwin, keys, values, row_lse, W: int, C: int, kernel: int = 3,
                      pooling: str = "avg") -> Dict:
    """Selection with the row normalisers handed over as log-sum-exps.

    Same steps as snapkv_select, except that the causal softmax of window row
    i is alpha[i, j] = exp(l[i, j] - row_lse[i]) for j <= P + i (0 beyond),
    with row_lse taken as given instead of computed from K.  With the exact
    row_log_sum_exp this is snapkv_select; an error d_i in row_lse[i] scales
    row i's probabilities by exp(-d_i).
    Returns indices, keys, values, votes and pooled as snapkv_select does.
    """
    qwin = np.asarray(qwin, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    row_lse = np.asarray(row_lse, dtype=np.float64)
    L, D = keys.shape
    if values.shape != keys.shape or qwin.shape != (W, D) or row_lse.shape != (W,):
        raise ValueError("shape mismatch between Qwin, K, V and row_lse")
    validate(L, W, C, D, kernel, pooling)
    for name, x in (("Qwin", qwin), ("K", keys), ("V", values), ("row_lse", row_lse)):
        if not np.all(np.isfinite(x)):
            raise ValueError(f"{name} must be finite")
    empty = np.zeros(0, dtype=np.float64)
    if L < C:
        idx = np.arange(L, dtype=np.int64)
        return {"indices": idx, "keys": keys.copy(), "values": values.copy(), "votes": empty, "pooled": empty}
    P = L - W
    logits = window_logits(qwin, keys)
    probs = np.zeros((W, L), dtype=np.float64)
    for i in range(W):
        t = P + i
        probs[i, : t + 1] = np.exp(logits[i, : t + 1] - row_lse[i])
    votes = prefix_votes(probs, P)
    pooled = pool1d(votes, kernel, pooling)
    chosen = top_prefix(pooled, C - W)
    idx = np.concatenate([chosen, np.arange(P, L)]).astype(np.int64)
    return {"indices": idx, "keys": keys[idx], "values": values[idx], "votes": votes, "pooled": pooled}


def snapkv_select_gqa(qwin, keys, values, W: int, C: int, kernel: int = 3, pooling: str = "avg",
                      row_lse=None) -> List[Dict]:
    """Grouped-query attention: qwin [H_q, W, D] against keys/values
    [H_kv, L, D], group G = H_q / H_kv.  The integration the page describes
    expands K/V to the H_q query heads before compressing each query head on
    its own (section "under GQA the saving is not just C divided by L"), so
    query head h selects with key/value head h // G (consecutive query heads
    share one, as the repetition expands them).  row_lse: None, or [H_q, W]
    handed-over statistics (snapkv_select_lse).  Returns one result per
    query head."""
    Hq, Hkv = len(qwin), len(keys)
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError("query heads must be a positive multiple of the key/value heads")
    G = Hq // Hkv
    if row_lse is None:
        return [snapkv_select(qwin[h], keys[h // G], values[h // G], W, C, kernel, pooling) for h in range(Hq)]
    return [snapkv_select_lse(qwin[h], keys[h // G], values[h // G], row_lse[h], W, C, kernel, pooling)
            for h in range(Hq)]


def expanded_cache_ratio(q_heads: int, kv_heads: int, L: int, C: int, g: int) -> float:
    """Persistent K/V of the expanded selection (every query head keeps
    min(L, C) prompt positions plus g generated tokens) over the native
    grouped full cache (kv_heads heads of L + g positions); batch, layers,
    head dimension and element size cancel (section "under GQA the saving is
    not just C divided by L")."""
    return q_heads * (min(L, C) + g) / (kv_heads * (L + g))


def refresh_select(scores, keep: int, protect_head: int, protect_tail: int) -> np.ndarray:
    """The selection step of a periodic cache refresh over n cached tokens:
    keep exactly `keep` positions.  The first protect_head (mandatory prefix,
    attention sinks) and the last protect_tail (recent window) are reserved,
    and the flexible budget keep - protect_head - protect_tail is filled with
    the highest scores of the positions in between, equal scores going to the
    lowest index.  Web page "Signals from the future: KV cache eviction by
    counter-causal surprise", section "architecture overview: the
    inference/refresh loop" (a refresh keeps the top J of the J + h cached
    tokens); web page "Jacap: Preserving Nonlinear Information in KV-Cache
    Eviction", section "Algorithm 2: a serving-safe integration sketch"
    (protected tokens first, then the flexible budget by score) and its
    sanity checks (the kept count equals the budget).  Returned ascending
    (reading: storage order is free; ascending keeps causal order)."""
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    if not (1 <= keep <= n) or protect_head < 0 or protect_tail < 0 or protect_head + protect_tail > keep:
        raise ValueError("need 1 <= keep <= n and protected tokens that fit the budget")
    if not np.all(np.isfinite(scores)):
        raise ValueError("scores must be finite")
    flexible = keep - protect_head - protect_tail
    middle = scores[protect_head:n - protect_tail]
    picked = top_prefix(middle, flexible) + protect_head if flexible > 0 else np.zeros(0, dtype=np.int64)
    kept = np.concatenate([np.arange(protect_head), picked, np.arange(n - protect_tail, n)])
    return np.sort(kept).astype(np.int64)


def jacap_scores(keys, outs, mu_q, lambda_q, tau: float) -> Dict:
    """Jacap leverage scores of N cached tokens of one head (web page "Jacap:
    Preserving Nonlinear Information in KV-Cache Eviction", sections
    "Practical approximation" and "Algorithm 1: one eviction event"):
      z_i = k_i . mu_Q / (tau sqrt(d_k)), alpha = softmax(z) over all N,
      kappa_i = k_i^T Lambda_Q k_i (Lambda_Q diagonal, given as its diagonal),
      w_i = [alpha_i (1 - alpha_i)]^2 kappa_i / d_k,
      A = I + sum_j w_j u_j u_j^T (u_j = outs[j]: W_O v_j, or v_j),
      r_i = w_i u_i^T A^{-1} u_i, with A factored once (Cholesky) and solved.
    keys [N, d_k], outs [N, d_u]; float64 throughout.  Returns z, alpha,
    kappa, w, A and r."""
    keys = np.asarray(keys, dtype=np.float64)
    outs = np.asarray(outs, dtype=np.float64)
    mu = np.asarray(mu_q, dtype=np.float64)
    lam = np.asarray(lambda_q, dtype=np.float64)
    N, dk = keys.shape
    if outs.shape[0] != N or mu.shape != (dk,) or lam.shape != (dk,) or not tau > 0:
        raise ValueError("shape mismatch or non-positive temperature")
    if np.any(lam < 0):
        raise ValueError("Lambda_Q is a second moment: its diagonal is >= 0")
    z = np.zeros(N)
    for d in range(dk):
        z += keys[:, d] * mu[d]
    z /= tau * math.sqrt(dk)
    m = z.max()
    e = np.exp(z - m)
    total = math.fsum(e.tolist())
    alpha = e / total
    # 1 - alpha_i is the probability of the other tokens: sum_{j != i} e_j / total.
    # Formed as (total - e_i) / total except for the largest term, whose
    # complement is summed directly (total - e_i would cancel when it dominates).
    rest = total - e
    top = int(np.argmax(e))
    rest[top] = math.fsum(np.delete(e, top).tolist())
    one_minus = rest / total
    kappa = np.zeros(N)
    for d in range(dk):
        kappa += lam[d] * keys[:, d] ** 2
    w = (alpha * one_minus) ** 2 * kappa / dk
    du = outs.shape[1]
    A = np.eye(du)
    for j in range(N):
        A += w[j] * np.outer(outs[j], outs[j])
    L = np.linalg.cholesky(A)
    # A^{-1} u_i by two triangular solves with the factor.
    y = np.linalg.solve(L, outs.T)          # L y = u
    x = np.linalg.solve(L.T, y)             # L^T x = y
    r = w * np.einsum("ij,ji->i", outs, x)
    return {"z": z, "alpha": alpha, "kappa": kappa, "w": w, "A": A, "r": r}


def jacap_select(keys, values, outs, mu_q, lambda_q, tau: float, keep: int, protect_head: int = 0,
                 protect_tail: int = 0) -> Dict:
    """One Jacap eviction event for one head: protected head and tail
    reserved, the flexible budget filled with the highest leverage scores
    (web page "Jacap: Preserving Nonlinear Information in KV-Cache Eviction",
    sections "Algorithm 1: one eviction event" and "Algorithm 2: a
    serving-safe integration sketch"), keys and values gathered."""
    sc = jacap_scores(keys, outs, mu_q, lambda_q, tau)
    idx = refresh_select(sc["r"], keep, protect_head, protect_tail)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    return {"indices": idx, "keys": keys[idx], "values": values[idx], **sc}


def snapkv_select_heads(qwin, keys, values, W: int, C: int, kernel: int = 3,
                        pooling: str = "avg", heads: Sequence[int] | None = None) -> List[Dict]:
    """Independent selection per head (section "the prompt cache shrinks, the
    positions keep their origin": every layer and head chooses on its own).
    qwin [H, W, D], keys/values [H, L, D]; `heads` restricts the evaluation to a
    subset of heads (results are returned in that order)."""
    H = keys.shape[0]
    heads = range(H) if heads is None else heads
    return [snapkv_select(qwin[h], keys[h], values[h], W, C, kernel, pooling) for h in heads]
