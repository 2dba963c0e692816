"""Calls that launch no fill: single-read scoring followed by the
cooperative or split selection clears its own shared words (exchange slots,
the cooperative selection's words, header word 0) inside the scoring
kernel, and two-pass scoring clears the words of any selection (with the
histograms of the whole-row and segment selections) in its statistics
kernel.  A workspace holding any bytes, or the previous call's words, must
give the same outputs, bit for bit, as a zeroed one, on the residency path
and on the forced fallback, and report only the call's own flags."""

import numpy as np
import pytest
import torch

from oracle import snapkv_oracle as O
from prompt_kv_selection_amd import workloads as WL

from parity import SELECT, band_check, bits, close, log, run_select, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from prompt_kv_selection_amd import binding
    return binding


def run(B, w, arrs, ws, select, fallback=False, scoring="single_read"):
    Q, K, V = arrs
    H, L, D = K.shape
    B.kvsel_set_option(B.KVSEL_OPT_SCORING, B.SCORING[scoring])
    B.kvsel_set_option(B.KVSEL_OPT_SELECT, SELECT[select])
    B.kvsel_set_option(B.KVSEL_OPT_FORCE_FALLBACK, 1 if fallback else 0)
    try:
        idx = torch.full((H, w.C), -7, dtype=torch.int32, device="cuda")
        Ko = torch.zeros((H, w.C, D), dtype=torch.bfloat16, device="cuda")
        Vo = torch.zeros_like(Ko)
        vt = torch.full((H, L - w.W), float("nan"), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        B.kvsel_profile_enable(True)
        B.kvsel_select(Q, K, V, L, w.W, w.C, D, H, w.kernel, w.pooling, torch.bfloat16, idx, Ko, Vo, None, vt, None,
                       ws)
        torch.cuda.synchronize()
        launches = B.kvsel_profile_read()
        B.kvsel_profile_enable(False)
        rc = B.kvsel_status(ws)
        last, _ = B.kvsel_status_flags(ws)
    finally:
        B.kvsel_set_option(B.KVSEL_OPT_SCORING, 0)
        B.kvsel_set_option(B.KVSEL_OPT_SELECT, 0)
        B.kvsel_set_option(B.KVSEL_OPT_FORCE_FALLBACK, 0)
    return dict(rc=rc, flags=B.flag_names(last), path=B.path_names(B.kvsel_last_path()), launches=launches,
                idx=idx.cpu().numpy(), Ko=bits(Ko).cpu(), Vo=bits(Vo).cpu(), votes=vt.cpu().numpy())


def same(a, b, what):
    np.testing.assert_array_equal(a["idx"], b["idx"], err_msg=f"{what}: indices")
    assert torch.equal(a["Ko"], b["Ko"]) and torch.equal(a["Vo"], b["Vo"]), f"{what}: K/V rows"
    np.testing.assert_array_equal(a["votes"].view(np.uint32), b["votes"].view(np.uint32), err_msg=f"{what}: votes")


CASES = [
    # (scoring, select, heads, L, C, pooling width, expected selection path)
    ("single_read", "auto", 8, 20000, 1024, 5, "select_coop"),
    ("single_read", "exchange", 40, 70000, 2000, 5, "select_coop"),   # several cooperative launches
    ("single_read", "split", 8, 20000, 1024, 5, "select_split"),
    ("two_pass", "auto", 8, 20000, 1024, 5, "select_coop"),
    ("two_pass", "exchange", 40, 70000, 2000, 3, "select_coop"),
    ("two_pass", "split", 8, 20000, 1024, 7, "select_split"),
    ("two_pass", "auto", 6, 20000, 1024, 9, "select_rows"),            # width 9: the whole-row selection
    ("two_pass", "auto", 3, 50000, 2048, 9, "select_segments"),       # and the segment chain
]


@pytest.mark.parametrize("fallback", [False, True], ids=["resident", "forced_fallback"])
@pytest.mark.parametrize("scoring,select,H,L,C,kernel,path", CASES)
def test_garbage_workspace_matches_zeroed(B, scoring, select, H, L, C, kernel, path, fallback):
    w = WL.Workload("self_clear", seed=H + L, heads=H, L=L, W=32, C=C, D=128, dtype="bf16", kernel=kernel,
                    pooling="avg", keys="spike", spike_frac=0.01)
    Q, K, V = WL.layer_arrays(w)
    arrs = (to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"))
    nbytes = B.kvsel_workspace_bytes(H, L, w.W, C, w.D, torch.bfloat16)
    log(f"self-clear: {scoring} select={select} H={H} L={L} C={C} k={kernel} fallback={fallback}: zeroed workspace")
    ref = run(B, w, arrs, torch.zeros(nbytes, dtype=torch.uint8, device="cuda"), select, fallback, scoring)
    assert ref["rc"] == B.KVSEL_OK, B.kvsel_last_error()
    assert path in ref["path"] and scoring in ref["path"], ref["path"]
    assert "fill" not in ref["launches"], f"a fill was launched: {ref['launches']}"
    assert ("scoring_fallback" in ref["flags"]) == (fallback and scoring == "single_read"), ref["flags"]
    for pattern in (0xAB, 0xFF):
        log(f"self-clear: workspace filled with {pattern:#x}, then the same workspace again")
        ws = torch.full((nbytes,), pattern, dtype=torch.uint8, device="cuda")
        for rep in range(2):
            out = run(B, w, arrs, ws, select, fallback, scoring)
            assert out["rc"] == B.KVSEL_OK, (pattern, rep, B.kvsel_last_error())
            assert out["flags"] == ref["flags"], (pattern, rep, out["flags"], ref["flags"])
            same(out, ref, f"pattern {pattern:#x} call {rep}")
    # The outputs are the method's: head 0 against the oracle.
    r = O.snapkv_select(WL.to_float64(Q[0], w.dtype), WL.to_float64(K[0], w.dtype), WL.to_float64(V[0], w.dtype),
                        w.W, C, w.kernel, w.pooling)
    P, n = L - w.W, C - w.W
    close(ref["votes"][0], r["votes"], "head 0 votes")
    band_check(ref["idx"][0, :n], r["pooled"], n, "head 0")
    np.testing.assert_array_equal(ref["idx"][0, n:], np.arange(P, L))


def test_stale_error_flags_do_not_carry_over(B):
    """A call that flags a non-finite key, then a clean call on the same
    workspace: the clean call reports OK (header word 0 is cleared by its
    scoring kernel, and the flags of the scoring kernel carry the call's tag)."""
    w = WL.Workload("self_clear_flags", seed=11, heads=4, L=20000, W=32, C=1024, D=128, dtype="bf16", kernel=5,
                    pooling="avg", keys="spike", spike_frac=0.01)
    Q, K, V = WL.layer_arrays(w)
    K2 = K.copy()
    K2[2, 1234, 7] = np.uint16(0x7FC0)  # NaN
    good = (to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"))
    bad = (good[0], to_device(K2, "bf16"), good[2])
    nbytes = B.kvsel_workspace_bytes(w.heads, w.L, w.W, w.C, w.D, torch.bfloat16)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for scoring in ("single_read", "two_pass"):
        for select in ("auto", "split"):
            log(f"stale flags: NaN key, {scoring}, select={select}")
            out = run(B, w, bad, ws, select, scoring=scoring)
            assert out["rc"] == B.KVSEL_ENONFINITE, (scoring, select, B.kvsel_last_error())
            assert "fill" not in out["launches"], out["launches"]
            log(f"stale flags: clean call on the same workspace, {scoring}, select={select}")
            out = run(B, w, good, ws, select, scoring=scoring)
            assert out["rc"] == B.KVSEL_OK, (scoring, select, B.kvsel_last_error())
            assert out["flags"] == [], out["flags"]


@pytest.mark.parametrize("select", ["auto", "split"])
def test_many_sequences_on_a_garbage_workspace(B, select):
    """A ragged batch of 20 sequences runs as two launch groups (up to 16
    sequences each): each group's scoring kernel clears its own words, and
    only the first clears header word 0.  A workspace of 0xAB bytes, used
    twice, gives what per-sequence calls on zeroed workspaces give."""
    w = WL.reduced(WL.get("ragged_b8_h32_l4k_64k"), heads=2, batch=20, L_min=1500, L_max=6000)
    Q, K, V, Ls, Cs, cu = WL.ragged_arrays(w)
    Ls, Cs = list(Ls), list(Cs)
    assert all(L >= C for L, C in zip(Ls, Cs))
    H, W, D = w.heads, w.W, w.D
    Qd, Kd, Vd = to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
    cuC = np.concatenate([[0], np.cumsum(Cs)])
    nbytes = B.kvsel_varlen_workspace_bytes(cu.tolist(), Cs, H, W, D, torch.bfloat16)
    ws = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda")
    B.kvsel_set_option(B.KVSEL_OPT_SELECT, SELECT[select])
    try:
        outs = []
        for rep in range(2):
            log(f"many sequences: select={select} call {rep}")
            idx = torch.full((H * int(cuC[-1]),), -1, dtype=torch.int32, device="cuda")
            Ko = torch.zeros((H * int(cuC[-1]), D), dtype=torch.bfloat16, device="cuda")
            Vo = torch.zeros_like(Ko)
            torch.cuda.synchronize()
            B.kvsel_profile_enable(True)
            B.kvsel_select_varlen(Qd, Kd, Vd, cu.tolist(), Cs, W, D, H, w.kernel, w.pooling, torch.bfloat16, idx, Ko,
                                  Vo, None, None, None, ws)
            torch.cuda.synchronize()
            launches = B.kvsel_profile_read()
            B.kvsel_profile_enable(False)
            assert B.kvsel_status(ws) == B.KVSEL_OK, B.kvsel_last_error()
            assert "fill" not in launches, launches
            outs.append((idx.cpu().numpy(), bits(Ko).cpu(), bits(Vo).cpu()))
    finally:
        B.kvsel_set_option(B.KVSEL_OPT_SELECT, 0)
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1]) and torch.equal(outs[0][2], outs[1][2])
    idx, Ko, Vo = outs[0]
    for b in (0, 7, 15, 16, 19):  # both groups
        L, C = Ls[b], Cs[b]
        k = Kd[H * int(cu[b]) * D: H * int(cu[b + 1]) * D].view(H, L, D).contiguous()
        v = Vd[H * int(cu[b]) * D: H * int(cu[b + 1]) * D].view(H, L, D).contiguous()
        single = run_select(Qd[b].contiguous(), k, v, L, W, C, w.kernel, w.pooling, "bf16", select=select)
        got = idx[H * int(cuC[b]): H * int(cuC[b + 1])].reshape(H, C)
        np.testing.assert_array_equal(got, single["idx"].cpu().numpy(), err_msg=f"sequence {b}")
        got_k = Ko[H * int(cuC[b]): H * int(cuC[b + 1])].reshape(H, C, D)
        assert torch.equal(got_k, bits(single["Ko"]).cpu()), f"sequence {b} K_out"
    # One sequence's head against the oracle.
    b, h = 16, 1
    q1, k1, v1 = WL.head_arrays(w, h, seq=b)
    ref = O.snapkv_select(WL.to_float64(q1, "bf16"), WL.to_float64(k1, "bf16"), WL.to_float64(v1, "bf16"), W, Cs[b],
                          w.kernel, w.pooling)
    n = Cs[b] - W
    got = idx[H * int(cuC[b]): H * int(cuC[b + 1])].reshape(H, Cs[b])[h]
    band_check(got[:n], ref["pooled"], n, f"sequence {b} head {h}")
    np.testing.assert_array_equal(got[n:], np.arange(Ls[b] - W, Ls[b]))
