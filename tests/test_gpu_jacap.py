"""Jacap eviction event (kvsel_jacap_select) against the float64 oracle
(web page "Jacap: Preserving Nonlinear Information in KV-Cache Eviction",
sections "Practical approximation", "Algorithm 1: one eviction event").

Scores: every r_i within a relative tolerance derived from the arithmetic
(bf16 hi + lo split of the two contractions, fp32 dots, softmax and
Cholesky), printed with the error observed.  Selection: the indices equal the
oracle's refresh selection taken on the GPU's own float32 scores (the integer
decision in the kernel's precision), and every token on which they differ from
the oracle's float64 selection lies within the score tolerance of the
oracle's cutoff.  Gather: K/V rows and token ids bit for bit."""

import math

import numpy as np
import pytest
import torch

from oracle import snapkv_oracle as O
from prompt_kv_selection_amd import workloads as WL

from parity import bits, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from prompt_kv_selection_amd import binding
    return binding


def dev_bf16(a16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(a16.view(np.int16)).cuda().view(torch.bfloat16)


def run(B, K, V, U, mu, lam, tau, keep, head, tail, tokens=None, scores=True):
    H, N, D = K.shape
    Kd, Vd, Ud = dev_bf16(K), dev_bf16(V), dev_bf16(U)
    mud, lamd = torch.from_numpy(mu).cuda(), torch.from_numpy(lam).cuda()
    idx = torch.full((H, keep), -1, dtype=torch.int32, device="cuda")
    Ko = torch.zeros((H, keep, D), dtype=torch.bfloat16, device="cuda")
    Vo = torch.zeros_like(Ko)
    tok = None if tokens is None else torch.from_numpy(tokens).cuda()
    to = None if tokens is None else torch.zeros((H, keep), dtype=torch.int32, device="cuda")
    r = torch.full((H, N), float("nan"), dtype=torch.float32, device="cuda") if scores else None
    ws = torch.empty(B.kvsel_jacap_workspace_bytes(H, N, D), dtype=torch.uint8, device="cuda")
    B.kvsel_jacap_select(Kd, Vd, Ud, mud, lamd, tau, H, N, D, "bf16", keep, head, tail, tok, idx, Ko, Vo, to, r, ws)
    status = B.kvsel_status(ws)
    torch.cuda.synchronize()
    return dict(Kd=Kd, Vd=Vd, idx=idx, Ko=Ko, Vo=Vo, tok=tok, to=to, r=r, status=status)


def tolerance(K64, U64, mu, lam, tau, sc) -> float:
    """Relative error bound of r_i: the dropped lo*lo products of the split
    (2^-16 each side), fp32 dot products over D terms feeding the logits
    (|z| error amplified twice through [alpha (1 - alpha)]^2), and the fp32
    Cholesky's backward error (a relative change of r_i of at most
    |dA|_2 since A >= I), each with a safety factor of 8."""
    D = K64.shape[1]
    u = 2.0 ** -24
    zmag = float(np.max(np.abs(K64) @ np.abs(mu.astype(np.float64)))) / (tau * math.sqrt(D))
    anorm = float(np.linalg.norm(sc["A"], 2))
    return 8.0 * (2.0 ** -15 + 4 * D * u * zmag + 2 * D * u * anorm + 4 * D * u)


CASES = [
    # heads, N, D, keep, head, tail, tau, mu_scale, separate_u
    (2, 5000, 128, 1000, 4, 64, 10.0, 1.0, False),    # several chunks and Gram slices, ragged tail
    (3, 3000, 64, 600, 4, 32, 0.3, 1.0, True),        # sharp centre softmax: A far from I
    (2, 37, 128, 10, 1, 2, 1.0, 1.0, False),          # one partial chunk
    (1, 1, 64, 1, 0, 0, 1.0, 1.0, False),             # one token: alpha = 1, w = r = 0
    (2, 9000, 128, 3000, 0, 0, 0.5, 2.0, True),       # no protected tokens
    (2, 4096, 64, 64, 32, 32, 2.0, 1.0, False),       # no flexible budget
    (2, 300, 64, 300, 0, 0, 1.0, 1.0, True),          # keep everything
    (3, 2047, 128, 1, 0, 0, 0.1, 3.0, True),          # one kept token, very sharp centre softmax
    (1, 70000, 128, 7000, 4, 64, 10.0, 1.0, False),   # one head: 32 Gram slices, segment-parallel selection
]


@pytest.mark.parametrize("case", CASES, ids=[f"h{c[0]}-N{c[1]}-D{c[2]}-k{c[3]}-p{c[4]}.{c[5]}-tau{c[6]}" for c in CASES])
def test_jacap_matches_oracle(B, case):
    H, N, D, keep, head, tail, tau, mus, sep = case
    K, V, U, mu, lam = WL.jacap_arrays(1000 + N, H, N, D, mu_scale=mus, separate_u=sep)
    rng = np.random.default_rng(N)
    tokens = rng.integers(0, 1 << 30, size=(H, N)).astype(np.int32)
    log(f"jacap {case}")
    out = run(B, K, V, U, mu, lam, tau, keep, head, tail, tokens)
    assert out["status"] == B.KVSEL_OK, B.kvsel_last_error()
    r_gpu = out["r"].cpu().numpy().astype(np.float64)
    got = out["idx"].cpu().numpy()
    worst = 0.0
    for h in range(H):
        K64 = WL.bf16_bits_to_f32(K[h]).astype(np.float64)
        U64 = WL.bf16_bits_to_f32(U[h]).astype(np.float64)
        sc = O.jacap_scores(K64, U64, mu[h], lam[h], tau)
        tol = tolerance(K64, U64, mu[h], lam[h], tau, sc)
        ref = sc["r"]
        assert np.all(np.isfinite(r_gpu[h])) and np.all(r_gpu[h] >= 0.0)
        floor = 1e-30 + 1e-7 * float(ref.max())
        err = np.abs(r_gpu[h] - ref)
        rel = err / np.maximum(np.abs(ref), floor)
        worst = max(worst, float(rel.max()))
        assert np.all(err <= tol * np.abs(ref) + floor * tol), \
            f"head {h}: max relative error {rel.max():.3e} > {tol:.3e} at token {int(rel.argmax())}"
        # The decision in the kernel's precision: identical indices.
        mine = O.refresh_select(r_gpu[h], keep, head, tail)
        np.testing.assert_array_equal(got[h], mine, err_msg=f"head {h}")
        # Against the float64 selection: differences only within the band.
        want = O.refresh_select(ref, keep, head, tail)
        diff = np.setxor1d(got[h], want)
        if diff.size:
            flex = keep - head - tail
            mid = np.sort(ref[head:N - tail])[::-1]
            cut = mid[flex - 1]
            assert np.all(np.abs(ref[diff] - cut) <= 2 * tol * cut + floor), f"head {h}: {diff[:8]}"
    log(f"  max relative score error {worst:.3e}")
    gi = out["idx"].long()
    assert torch.equal(bits(out["Ko"]), bits(torch.gather(out["Kd"], 1, gi[:, :, None].expand(H, keep, D))))
    assert torch.equal(bits(out["Vo"]), bits(torch.gather(out["Vd"], 1, gi[:, :, None].expand(H, keep, D))))
    assert torch.equal(out["to"], torch.gather(out["tok"], 1, gi))


def test_jacap_without_score_output_selects_the_same(B):
    H, N, D = 2, 3000, 128
    K, V, U, mu, lam = WL.jacap_arrays(7, H, N, D)
    a = run(B, K, V, U, mu, lam, 1.0, 500, 4, 16)
    b = run(B, K, V, U, mu, lam, 1.0, 500, 4, 16, scores=False)
    assert torch.equal(a["idx"], b["idx"])
    assert torch.equal(bits(a["Ko"]), bits(b["Ko"]))


def test_jacap_is_deterministic(B):
    H, N, D = 2, 6000, 128
    K, V, U, mu, lam = WL.jacap_arrays(8, H, N, D, mu_scale=2.0)
    a = run(B, K, V, U, mu, lam, 0.5, 1500, 4, 16)
    b = run(B, K, V, U, mu, lam, 0.5, 1500, 4, 16)
    assert torch.equal(bits(a["r"]), bits(b["r"]))
    assert torch.equal(a["idx"], b["idx"])


def test_jacap_leverage_toy(B):
    """The page's miniature example embedded in D = 64 (u_1 = e_1,
    u_2 = 0.95 e_1 + 0.05 e_2, u_3 = e_2, weights 1, 1 and about 0.7): the
    near-collinear second token scores lowest although its weight is the
    highest, so a budget of two keeps the spanning pair (tokens 0 and 2)."""
    D = 64
    K = np.zeros((1, 3, D), dtype=np.float32)
    K[0, :2, 0] = 1.0                      # mu = 0: equal logits, alpha = 1/3 for every token
    K[0, 2, 0] = math.sqrt(0.7)
    U = np.zeros((1, 3, D), dtype=np.float32)
    U[0, 0, 0] = 1.0
    U[0, 1, 0], U[0, 1, 1] = 0.95, 0.05
    U[0, 2, 1] = 1.0
    mu = np.zeros((1, D), dtype=np.float32)
    lam = np.ones((1, D), dtype=np.float32)
    lam[0, 0] = 1296.0                     # kappa / D = (9 / 2)^2 = 1 / [alpha (1 - alpha)]^2: w = (1, 1, 0.7)
    K16, U16 = WL.f32_to_bf16_bits(K), WL.f32_to_bf16_bits(U)
    out = run(B, K16, U16, U16, mu, lam, 1.0, 2, 0, 0)
    ref = O.jacap_scores(WL.bf16_bits_to_f32(K16[0]).astype(np.float64),
                         WL.bf16_bits_to_f32(U16[0]).astype(np.float64), mu[0], lam[0], 1.0)
    np.testing.assert_allclose(out["r"].cpu().numpy()[0], ref["r"], rtol=1e-4)
    assert ref["r"][1] < ref["r"][0] < ref["r"][2]
    assert out["idx"].cpu().numpy()[0].tolist() == [0, 2]


def test_jacap_non_finite_key_is_flagged(B):
    H, N, D = 2, 2000, 128
    K, V, U, mu, lam = WL.jacap_arrays(9, H, N, D)
    K[1, 777, 5] = 0x7FC0                   # a bf16 NaN
    out = run(B, K, V, U, mu, lam, 1.0, 100, 0, 0)
    assert out["status"] == B.KVSEL_ENONFINITE
    clean = run(B, K[:1].copy(), V[:1].copy(), U[:1].copy(), mu[:1].copy(), lam[:1].copy(), 1.0, 100, 0, 0)
    assert clean["status"] == B.KVSEL_OK      # the flag is cleared by the next call


def test_jacap_full_size_sampled_heads(B):
    """The measured configuration (32 heads, 32768 cached tokens, D = 128,
    keep 6554 = 20 %, 4 sink and 64 recent tokens protected, tau = 10), in
    one call; heads 0 and 31 are checked against the oracle."""
    H, N, D, keep, head, tail, tau = 32, 32768, 128, 6554, 4, 64, 10.0
    K, V, U, mu, lam = WL.jacap_arrays(11, H, N, D)
    out = run(B, K, V, U, mu, lam, tau, keep, head, tail)
    assert out["status"] == B.KVSEL_OK, B.kvsel_last_error()
    r_gpu = out["r"].cpu().numpy().astype(np.float64)
    got = out["idx"].cpu().numpy()
    for h in (0, H - 1):
        K64 = WL.bf16_bits_to_f32(K[h]).astype(np.float64)
        U64 = WL.bf16_bits_to_f32(U[h]).astype(np.float64)
        sc = O.jacap_scores(K64, U64, mu[h], lam[h], tau)
        tol = tolerance(K64, U64, mu[h], lam[h], tau, sc)
        rel = np.abs(r_gpu[h] - sc["r"]) / sc["r"]
        log(f"  head {h}: max relative score error {rel.max():.3e} (bound {tol:.3e})")
        assert rel.max() <= tol
        np.testing.assert_array_equal(got[h], O.refresh_select(r_gpu[h], keep, head, tail))
    gi = out["idx"].long()
    assert torch.equal(bits(out["Ko"]), bits(torch.gather(out["Kd"], 1, gi[:, :, None].expand(H, keep, D))))


def test_jacap_concurrent_calls_on_two_streams(B):
    """Two independent events on two streams, each with its own workspace,
    give the same bits as the same events run one after the other."""
    H, N, D = 4, 9000, 128
    evs = [WL.jacap_arrays(20 + k, H, N, D) for k in range(2)]
    seq = [run(B, *ev, 1.0, 900, 4, 32) for ev in evs]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for ev, st in zip(evs, (s1, s2)):
        K, V, U, mu, lam = ev
        o = dict(idx=torch.full((H, 900), -1, dtype=torch.int32, device="cuda"),
                 r=torch.empty((H, N), dtype=torch.float32, device="cuda"),
                 Ko=torch.empty((H, 900, D), dtype=torch.bfloat16, device="cuda"),
                 ws=torch.empty(B.kvsel_jacap_workspace_bytes(H, N, D), dtype=torch.uint8, device="cuda"),
                 inp=(dev_bf16(K), dev_bf16(V), dev_bf16(U), torch.from_numpy(mu).cuda(), torch.from_numpy(lam).cuda()))
        o["Vo"] = torch.empty_like(o["Ko"])
        outs.append(o)
    torch.cuda.synchronize()
    for o, st in zip(outs, (s1, s2)):
        Kd, Vd, Ud, mud, lamd = o["inp"]
        B.kvsel_jacap_select(Kd, Vd, Ud, mud, lamd, 1.0, H, N, D, "bf16", 900, 4, 32, None, o["idx"], o["Ko"],
                             o["Vo"], None, o["r"], o["ws"], stream=st)
    torch.cuda.synchronize()
    for o, a, st in zip(outs, seq, (s1, s2)):
        assert B.kvsel_status(o["ws"], st) == B.KVSEL_OK
        assert torch.equal(o["idx"], a["idx"])
        assert torch.equal(bits(o["r"]), bits(a["r"]))
        assert torch.equal(bits(o["Ko"]), bits(a["Ko"]))


def test_negative_second_moment_is_reported(B):
    """lambda_q is a diagonal second moment (>= 0).  A negative entry would
    make weights and scores negative and rank them wrongly: the call still
    completes, and the status names the input as out of its domain."""
    H, N, D = 2, 3000, 128
    K, V, U, mu, lam = WL.jacap_arrays(5, H, N, D, 1.0, False)
    out = run(B, K, V, U, mu, lam, 10.0, 600, 4, 32)
    assert out["status"] == B.KVSEL_OK, B.kvsel_last_error()
    lam = lam.copy()
    lam[1, 77] = -0.5
    log("jacap: negative lambda entry")
    out = run(B, K, V, U, mu, lam, 10.0, 600, 4, 32)
    assert out["status"] == B.KVSEL_EINVAL, B.kvsel_last_error()
    assert "lambda_q" in B.kvsel_last_error()
    idx = out["idx"].cpu().numpy()
    assert np.all((idx >= 0) & (idx < N))
