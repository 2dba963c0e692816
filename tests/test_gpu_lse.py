"""GPU parity of the selection with handed-over row statistics
(kvsel_select_lse / kvsel_select_varlen_lse): the oracle's snapkv_select_lse
on the same float32 log-sum-exps, the page's worked example, and agreement
with the full path fed its own row statistics.  Tolerances are stated in
tests/parity.py."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import snapkv_oracle as O
from prompt_kv_selection_amd import workloads as WL

from parity import (band_check, bits, check_gather, check_head_lse, close, log, run_select, run_select_lse,
                    single_read_covers, to_device)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from prompt_kv_selection_amd import binding
    return binding


def oracle_lse(Q, K, dtype, W, L):
    """Float32 row log-sum-exps of every head from the oracle (float64, then
    rounded once), as [H, W]."""
    out = np.empty((Q.shape[0], W), dtype=np.float32)
    for h in range(Q.shape[0]):
        logits = O.window_logits(WL.to_float64(Q[h], dtype), WL.to_float64(K[h], dtype))
        out[h] = O.row_log_sum_exp(logits, L - W).astype(np.float32)
    return out


@pytest.mark.parametrize("scoring", ["auto", "two_pass"])
def test_lse_worked_example(B, scoring):
    """The page's worked example with its row sums handed over as ln 25 and
    ln 26: the page's votes, pooled scores and selection."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    rows = [g["exp_weight_rows"]["query_6"], g["exp_weight_rows"]["query_7"]]
    L, D = g["L"], 64
    K = np.zeros((L, D), dtype=np.float32)
    for i, row in enumerate(rows):
        for j, w in enumerate(row):
            K[j, i] = math.log(g["masked_placeholder"] if w is None else w)
    Q = np.zeros((2, D), dtype=np.float32)
    Q[0, 0] = Q[1, 1] = math.sqrt(D)
    V = np.zeros((L, D), dtype=np.float32)
    V[:, 0] = np.arange(L)
    V[:, 1] = -np.arange(L)
    log(f"lse worked example scoring={scoring}")
    Qd, Kd, Vd = (to_device(x[None], "f32") for x in (Q, K, V))
    lse = torch.tensor([[math.log(25), math.log(26)]], dtype=torch.float32, device="cuda")
    out = run_select_lse(Qd, Kd, Vd, lse, L, g["W"], g["C"], g["kernel"], g["pooling"], "f32", scoring)
    assert out["idx"][0].tolist() == g["expected_indices"]
    assert out["Vo"][0, :, :2].cpu().tolist() == g["expected_values"]
    np.testing.assert_allclose(out["votes"][0], np.array([51, 77, 460, 508, 51, 51]) / 650, rtol=1e-5)
    np.testing.assert_allclose(out["pooled"][0], np.array([128, 588, 1045, 1019, 610, 102]) / 1950, rtol=1e-5)


LSE_CASES = [
    # dtype, D, H, L, W, C, kernel, pooling
    ("bf16", 128, 3, 4096, 32, 512, 5, "avg"),
    ("bf16", 128, 2, 3001, 32, 700, 5, "max"),     # ragged tile and chunk tails
    ("bf16", 128, 2, 1057, 7, 100, 3, "avg"),      # W not a multiple of 32
    ("bf16", 128, 1, 3000, 100, 900, 9, "max"),    # several row blocks (two-pass only)
    ("bf16", 64, 2, 2049, 33, 200, 3, "avg"),
    ("bf16", 64, 2, 5000, 1, 2, 5, "avg"),         # W = 1
    ("f32", 128, 2, 1500, 40, 1500, 5, "max"),     # L == C
    ("bf16", 128, 2, 300, 32, 1024, 5, "avg"),     # bypass L < C
    ("bf16", 128, 2, 20000, 32, 1024, 5, "max"),   # five selection segments
]


@pytest.mark.parametrize("scoring", ["two_pass", "single_read"])
@pytest.mark.parametrize("case", LSE_CASES, ids=[f"{c[0]}-D{c[1]}-H{c[2]}-L{c[3]}-W{c[4]}-C{c[5]}-k{c[6]}{c[7]}"
                                                 for c in LSE_CASES])
def test_lse_random_cases(B, case, scoring):
    dtype, D, H, L, W, C, kernel, pooling = case
    w = WL.Workload("case", seed=L * 13 + W, heads=H, L=L, W=W, C=C, D=D, dtype=dtype, kernel=kernel,
                    pooling=pooling, keys="spike", spike_frac=0.02 if L - W >= 50 else 0.0)
    Q, K, V = WL.layer_arrays(w)
    log(f"lse case {case} scoring={scoring}")
    Qd, Kd, Vd = to_device(Q, dtype), to_device(K, dtype), to_device(V, dtype)
    lse = oracle_lse(Q, K, dtype, W, L)
    lse_d = torch.from_numpy(lse).cuda()
    if scoring == "single_read" and not single_read_covers(dtype, D, W) and L >= C:
        with pytest.raises(B.KvselError) as ei:
            run_select_lse(Qd, Kd, Vd, lse_d, L, W, C, kernel, pooling, dtype, scoring)
        assert ei.value.code == B.KVSEL_EUNSUPPORTED
        return
    out = run_select_lse(Qd, Kd, Vd, lse_d, L, W, C, kernel, pooling, dtype, scoring)
    for h in range(H):
        ref = O.snapkv_select_lse(WL.to_float64(Q[h], dtype), WL.to_float64(K[h], dtype),
                                  WL.to_float64(V[h], dtype), lse[h].astype(np.float64), W, C, kernel, pooling)
        check_head_lse(out, h, ref, L, W, C, f"{case} head {h}")
    check_gather(out, Kd, Vd, C, L)


@pytest.mark.parametrize("scoring", ["two_pass", "single_read"])
def test_lse_agrees_with_full_path(B, scoring):
    """Fed the full path's own row statistics (lse = m + ln Z), the hand-off
    path gives the same votes within the score tolerance and a selection
    inside the same tie band."""
    dtype, D, H, L, W, C, kernel, pooling = "bf16", 128, 4, 8192, 32, 1024, 5, "max"
    w = WL.Workload("case", seed=99, heads=H, L=L, W=W, C=C, D=D, dtype=dtype, kernel=kernel, pooling=pooling,
                    keys="spike", spike_frac=0.01)
    Q, K, V = WL.layer_arrays(w)
    Qd, Kd, Vd = to_device(Q, dtype), to_device(K, dtype), to_device(V, dtype)
    log(f"lse vs full path scoring={scoring}")
    full = run_select(Qd, Kd, Vd, L, W, C, kernel, pooling, dtype, scoring)
    lse = (full["rs"][:, :, 0].astype(np.float64) + np.log(full["rs"][:, :, 1].astype(np.float64))).astype(np.float32)
    out = run_select_lse(Qd, Kd, Vd, torch.from_numpy(lse).cuda(), L, W, C, kernel, pooling, dtype, scoring)
    n = C - W
    for h in range(H):
        close(out["votes"][h], full["votes"][h], f"head {h} votes")
        close(out["pooled"][h], full["pooled"][h], f"head {h} pooled")
        band_check(out["idx"][h, :n].cpu().numpy(), full["pooled"][h].astype(np.float64), n, f"head {h}")
    check_gather(out, Kd, Vd, C, L)


def test_lse_varlen_matches_per_sequence_calls(B):
    w = WL.reduced(WL.get("ragged_b8_h32_l4k_64k"), heads=4, batch=5, L_min=900, L_max=5000)
    Q, K, V, Ls, Cs, cu = WL.ragged_arrays(w)
    Ls, Cs = list(Ls), list(Cs)
    Cs[1] = Ls[1] + 3  # one bypassed sequence
    H, W, D = w.heads, w.W, w.D
    log(f"lse varlen lengths {Ls} budgets {Cs}")
    Qd, Kd, Vd = to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
    lse = np.stack([oracle_lse(Q[b], K[H * cu[b] * D: H * cu[b + 1] * D].reshape(H, Ls[b], D), "bf16", W, Ls[b])
                    for b in range(len(Ls))])
    lse_d = torch.from_numpy(lse).cuda()
    cuC = np.concatenate([[0], np.cumsum(Cs)])
    cuP = np.concatenate([[0], np.cumsum([L - W for L in Ls])])
    ws = torch.empty(B.kvsel_varlen_workspace_bytes(cu.tolist(), Cs, H, W, D, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    idx = torch.full((H * int(cuC[-1]),), -1, dtype=torch.int32, device="cuda")
    Ko = torch.zeros((H * int(cuC[-1]), D), dtype=torch.bfloat16, device="cuda")
    Vo = torch.zeros_like(Ko)
    vt = torch.zeros((H * int(cuP[-1]),), dtype=torch.float32, device="cuda")
    B.kvsel_select_varlen_lse(Qd, Kd, Vd, lse_d, cu.tolist(), Cs, W, D, H, w.kernel, w.pooling, torch.bfloat16,
                              idx, Ko, Vo, vt, None, ws)
    torch.cuda.synchronize()
    for b, (L, C) in enumerate(zip(Ls, Cs)):
        k = Kd[H * int(cu[b]) * D: H * int(cu[b + 1]) * D].view(H, L, D)
        v = Vd[H * int(cu[b]) * D: H * int(cu[b + 1]) * D].view(H, L, D)
        single = run_select_lse(Qd[b].contiguous(), k.contiguous(), v.contiguous(), lse_d[b].contiguous(), L, W, C,
                                w.kernel, w.pooling, "bf16")
        n_out = min(L, C)
        got_idx = idx[H * int(cuC[b]): H * int(cuC[b + 1])].view(H, C)[:, :n_out]
        assert torch.equal(got_idx, single["idx"][:, :n_out]), f"sequence {b}"
        got_k = Ko[H * int(cuC[b]): H * int(cuC[b + 1])].view(H, C, D)[:, :n_out]
        assert torch.equal(bits(got_k), bits(single["Ko"][:, :n_out])), f"sequence {b} K_out"
        if L >= C:
            got_v = vt[H * int(cuP[b]): H * int(cuP[b + 1])].view(H, L - W).cpu().numpy()
            np.testing.assert_array_equal(got_v.view(np.int32), single["votes"].view(np.int32))
        if b in (0, 1):
            h = 2
            q1, k1, v1 = WL.head_arrays(w, h, seq=b)
            ref = O.snapkv_select_lse(WL.to_float64(q1, "bf16"), WL.to_float64(k1, "bf16"),
                                      WL.to_float64(v1, "bf16"), lse[b, h].astype(np.float64), W, C, w.kernel,
                                      w.pooling)
            check_head_lse(single, h, ref, L, W, C, f"lse varlen seq {b} head {h}")


@pytest.mark.slow
def test_lse_full_size_benchmark_layer(B):
    """One layer of the 32-head, L = 32768 benchmark workload through the
    hand-off path (statistics from the oracle on sampled heads, from the full
    path elsewhere), sampled heads against the oracle."""
    w = WL.get("spike_l32x_h32_l32k")
    log("lse full size: drawing inputs")
    Q, K, V = WL.layer_arrays(w, layer=0)
    Qd, Kd, Vd = to_device(Q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    full = run_select(Qd, Kd, Vd, w.L, w.W, w.C, w.kernel, w.pooling, w.dtype)
    lse = (full["rs"][:, :, 0].astype(np.float64) + np.log(full["rs"][:, :, 1].astype(np.float64))).astype(np.float32)
    sampled = (0, 21)
    for h in sampled:
        log(f"lse full size: oracle statistics of head {h}")
        logits = O.window_logits(WL.to_float64(Q[h], w.dtype), WL.to_float64(K[h], w.dtype))
        lse[h] = O.row_log_sum_exp(logits, w.L - w.W).astype(np.float32)
    del K, V
    log("lse full size: GPU call")
    out = run_select_lse(Qd, Kd, Vd, torch.from_numpy(lse).cuda(), w.L, w.W, w.C, w.kernel, w.pooling, w.dtype)
    check_gather(out, Kd, Vd, w.C, w.L)
    for h in sampled:
        log(f"lse full size: oracle head {h}")
        q, k, v = WL.head_arrays(w, h, layer=0)
        ref = O.snapkv_select_lse(WL.to_float64(q, w.dtype), WL.to_float64(k, w.dtype), WL.to_float64(v, w.dtype),
                                  lse[h].astype(np.float64), w.W, w.C, w.kernel, w.pooling)
        check_head_lse(out, h, ref, w.L, w.W, w.C, f"lse full size head {h}")
