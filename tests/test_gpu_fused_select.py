"""The selection fused into the single-read scoring kernel (KVSEL_OPT_FUSED_SELECT).

The fused kernel runs the same votes arithmetic and the same pooling order as
the separate selection launch, so its indices, K/V rows, votes, pooled scores
and row statistics must equal the separate path's bit for bit, on every
pooling width and mode it covers, ragged chunk tails, prompts whose window
fills the last chunk, exact ties, and the handed-over statistics.  Its
residency fallback (forced from the host) merges the statistics in another
order, so it is held to the oracle under the stated tolerances instead, and
its indices must still be the top-(C-W) of its own pooled scores."""

import numpy as np
import pytest
import torch

from oracle import snapkv_oracle as O
from prompt_kv_selection_amd import workloads as WL

from parity import bits, check_gather, check_head, gpu_internal_topk, log, to_device, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from prompt_kv_selection_amd import binding
    return binding


def call(B, Qd, Kd, Vd, L, W, C, kernel, pooling, dtype, fused=True, fallback=False, lse=None):
    H, _, D = Kd.shape
    td = torch_dtype(dtype)
    B.kvsel_set_option(B.KVSEL_OPT_FUSED_SELECT, 1 if fused else 0)
    B.kvsel_set_option(B.KVSEL_OPT_FORCE_FALLBACK, 1 if fallback else 0)
    try:
        ws = torch.empty(B.kvsel_workspace_bytes(H, L, W, C, D, td), dtype=torch.uint8, device="cuda")
        ws.fill_(0x5A)  # the fused call clears what it needs itself
        out = dict(idx=torch.full((H, C), -7, dtype=torch.int32, device="cuda"),
                   Ko=torch.zeros((H, C, D), dtype=td, device="cuda"),
                   Vo=torch.zeros((H, C, D), dtype=td, device="cuda"),
                   rs=torch.full((H, W, 2), float("nan"), dtype=torch.float32, device="cuda"),
                   votes=torch.full((H, L - W), float("nan"), dtype=torch.float32, device="cuda"),
                   pooled=torch.full((H, L - W), float("nan"), dtype=torch.float32, device="cuda"))
        if lse is None:
            B.kvsel_select(Qd, Kd, Vd, L, W, C, D, H, kernel, pooling, td, out["idx"], out["Ko"], out["Vo"],
                           out["rs"], out["votes"], out["pooled"], ws)
        else:
            B.kvsel_select_lse(Qd, Kd, Vd, lse, L, W, C, D, H, kernel, pooling, td, out["idx"], out["Ko"],
                               out["Vo"], out["votes"], out["pooled"], ws)
        path = B.path_names(B.kvsel_last_path())
        rc = B.kvsel_status(ws)
        last, _ = B.kvsel_status_flags(ws)
        torch.cuda.synchronize()
    finally:
        B.kvsel_set_option(B.KVSEL_OPT_FUSED_SELECT, 0)
        B.kvsel_set_option(B.KVSEL_OPT_FORCE_FALLBACK, 0)
    assert rc == B.KVSEL_OK, B.kvsel_last_error()
    out["path"], out["flags"] = path, B.flag_names(last)
    return out


CASES = [
    # H, L, W, C, D, kernel, pooling, keys
    (4, 5000, 32, 512, 128, 5, "max", "spike"),      # ragged last chunk
    (3, 6144, 32, 700, 128, 7, "avg", "spike"),      # chunk-aligned prompt
    (2, 9000, 16, 300, 128, 3, "avg", "lognorm"),    # W < 32
    (2, 4096, 32, 4096, 128, 1, "avg", "normal"),    # L == C: the whole prefix is kept
    (2, 2047, 32, 40, 128, 5, "max", "spike"),       # few picks
    (2, 7000, 32, 800, 64, 5, "avg", "spike"),       # D = 64
    (2, 4106, 32, 900, 128, 3, "max", "spike"),      # the last chunk holds window positions only
    (2, 4128, 32, 1000, 128, 5, "avg", "lognorm"),   # P a multiple of the chunk
    (2, 20000, 32, 2048, 128, 3, "max", "codebook"), # exact ties across chunks
    (1, 600, 32, 100, 128, 7, "avg", "spike"),       # two chunks
    (32, 32768, 32, 1024, 128, 5, "max", "spike"),   # the benchmark layer
]


def inputs(case, seed_extra=0):
    H, L, W, C, D, kernel, pooling, keys = case
    w = WL.Workload("fused", seed=L * 13 + W + seed_extra, heads=H, L=L, W=W, C=C, D=D, dtype="bf16",
                    kernel=kernel, pooling=pooling, keys=keys, spike_frac=0.02)
    Q, K, V = WL.layer_arrays(w)
    return w, Q, K, V


@pytest.mark.parametrize("case", CASES, ids=[f"H{c[0]}-L{c[1]}-W{c[2]}-C{c[3]}-D{c[4]}-k{c[5]}{c[6]}-{c[7]}"
                                             for c in CASES])
def test_fused_equals_separate(B, case):
    H, L, W, C, D, kernel, pooling, keys = case
    w, Q, K, V = inputs(case)
    Qd, Kd, Vd = to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
    log(f"fused selection {case}")
    a = call(B, Qd, Kd, Vd, L, W, C, kernel, pooling, "bf16", fused=True)
    assert "select_fused" in a["path"] and "single_read" in a["path"], a["path"]
    assert not a["flags"], a["flags"]
    log(f"separate selection {case}")
    b = call(B, Qd, Kd, Vd, L, W, C, kernel, pooling, "bf16", fused=False)
    assert "select_fused" not in b["path"]
    for k in ("idx", "Ko", "Vo", "rs", "votes", "pooled"):
        assert torch.equal(bits(a[k]), bits(b[k])), f"{case}: {k} differs between the fused and separate paths"
    for h in sorted({0, H - 1}):
        ref = O.snapkv_select(WL.to_float64(Q[h], "bf16"), WL.to_float64(K[h], "bf16"),
                              WL.to_float64(V[h], "bf16"), W, C, kernel, pooling)
        check_head({**a, "votes": a["votes"].cpu().numpy(), "pooled": a["pooled"].cpu().numpy(),
                    "rs": a["rs"].cpu().numpy()}, h, ref, L, W, C, f"fused {case} head {h}")


@pytest.mark.parametrize("case", [CASES[0], CASES[5], CASES[6], CASES[8], CASES[10]],
                         ids=["ragged", "D64", "window-chunk", "ties", "layer"])
def test_fused_fallback_matches_oracle(B, case):
    """ABORT forced from the host: statistics and votes per chunk from a
    counter (two passes), then each row's selection in one workgroup."""
    H, L, W, C, D, kernel, pooling, keys = case
    w, Q, K, V = inputs(case, seed_extra=1)
    Qd, Kd, Vd = to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
    log(f"fused selection, forced fallback {case}")
    a = call(B, Qd, Kd, Vd, L, W, C, kernel, pooling, "bf16", fused=True, fallback=True)
    assert "scoring_fallback" in a["flags"], a["flags"]
    out = {**a, "votes": a["votes"].cpu().numpy(), "pooled": a["pooled"].cpu().numpy(), "rs": a["rs"].cpu().numpy()}
    n = C - W
    idx = a["idx"].cpu().numpy()
    for h in range(H):
        gpu_internal_topk(idx[h, :n], out["pooled"][h], n, f"fallback {case} head {h}")
    for h in sorted({0, H // 2, H - 1}):
        ref = O.snapkv_select(WL.to_float64(Q[h], "bf16"), WL.to_float64(K[h], "bf16"),
                              WL.to_float64(V[h], "bf16"), W, C, kernel, pooling)
        check_head(out, h, ref, L, W, C, f"fallback {case} head {h}")
    check_gather(a, Kd, Vd, C, L)


@pytest.mark.parametrize("fallback", [False, True])
def test_fused_handed_over_statistics(B, fallback):
    case = (4, 7000, 32, 600, 128, 5, "avg", "spike")
    H, L, W, C, D, kernel, pooling, keys = case
    w, Q, K, V = inputs(case, seed_extra=2)
    Qd, Kd, Vd = to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
    full = call(B, Qd, Kd, Vd, L, W, C, kernel, pooling, "bf16", fused=False)
    lse = (full["rs"][:, :, 0].double() + full["rs"][:, :, 1].double().log()).float().contiguous()
    log(f"fused selection with handed-over statistics, fallback={fallback}")
    a = call(B, Qd, Kd, Vd, L, W, C, kernel, pooling, "bf16", fused=True, fallback=fallback, lse=lse)
    b = call(B, Qd, Kd, Vd, L, W, C, kernel, pooling, "bf16", fused=False, lse=lse)
    assert "select_fused" in a["path"] and "handed_over" in a["path"]
    for k in ("idx", "Ko", "Vo", "votes", "pooled"):
        assert torch.equal(bits(a[k]), bits(b[k])), f"lse: {k} differs between the fused and separate paths"


def test_fused_ragged_batch(B):
    """Three sequences in one call: rounds run over all of them, each row
    selects on its own."""
    w = WL.Workload("fused_ragged", seed=31, heads=4, batch=3, L_min=3000, L_max=12000, W=32, D=128,
                    dtype="bf16", kernel=7, pooling="avg")
    Q, K, V, Ls, Cs, cu = WL.ragged_arrays(w)
    H, W, D = w.heads, w.W, w.D
    Qd, Kd, Vd = to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
    cuC = np.concatenate([[0], np.cumsum(Cs)])
    res = {}
    for fused in (True, False):
        B.kvsel_set_option(B.KVSEL_OPT_FUSED_SELECT, 1 if fused else 0)
        try:
            ws = torch.empty(B.kvsel_varlen_workspace_bytes(cu.tolist(), Cs, H, W, D, torch.bfloat16),
                             dtype=torch.uint8, device="cuda")
            idx = torch.full((H * int(cuC[-1]),), -1, dtype=torch.int32, device="cuda")
            Ko = torch.zeros((H * int(cuC[-1]), D), dtype=torch.bfloat16, device="cuda")
            Vo = torch.zeros_like(Ko)
            log(f"ragged batch {Ls} fused={fused}")
            B.kvsel_select_varlen(Qd, Kd, Vd, cu.tolist(), Cs, W, D, H, w.kernel, w.pooling, torch.bfloat16, idx,
                                  Ko, Vo, None, None, None, ws)
            assert ("select_fused" in B.path_names(B.kvsel_last_path())) == fused
            assert B.kvsel_status(ws) == B.KVSEL_OK, B.kvsel_last_error()
            res[fused] = (idx, Ko, Vo)
        finally:
            B.kvsel_set_option(B.KVSEL_OPT_FUSED_SELECT, 0)
    for a, b in zip(res[True], res[False]):
        assert torch.equal(bits(a), bits(b))
