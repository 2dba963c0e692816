"""Grouped-query attention (kvsel_select_gqa): each K/V head is streamed once
for its group of query heads, and every output equals, bit for bit, running
the expanded heads (K and V repeated over the head axis, as the model's
integration does) through the two-pass path; sampled heads against the
oracle; handed-over statistics."""

import numpy as np
import pytest
import torch

from oracle import snapkv_oracle as O
from prompt_kv_selection_amd import workloads as WL

from parity import bits, check_head, check_head_lse, log, run_select, to_device, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from prompt_kv_selection_amd import binding
    return binding


def gqa_call(B, Qd, Kd, Vd, Hq, Hkv, L, W, C, kernel, pooling, dtype, lse=None):
    D = Kd.shape[-1]
    td = torch_dtype(dtype)
    ws = torch.empty(B.kvsel_gqa_workspace_bytes(Hq, Hkv, L, W, C, D, td), dtype=torch.uint8, device="cuda")
    idx = torch.full((Hq, C), -7, dtype=torch.int32, device="cuda")
    Ko = torch.zeros((Hq, C, D), dtype=td, device="cuda")
    Vo = torch.zeros((Hq, C, D), dtype=td, device="cuda")
    rs = None if lse is not None else torch.full((Hq, W, 2), float("nan"), dtype=torch.float32, device="cuda")
    vt = torch.full((Hq, L - W), float("nan"), dtype=torch.float32, device="cuda")
    pl = torch.full((Hq, L - W), float("nan"), dtype=torch.float32, device="cuda")
    B.kvsel_select_gqa(Qd, Kd, Vd, lse, L, W, C, D, Hq, Hkv, kernel, pooling, td, idx, Ko, Vo, rs, vt, pl, ws)
    assert B.kvsel_status(ws) == B.KVSEL_OK, B.kvsel_last_error()
    torch.cuda.synchronize()
    return dict(idx=idx, Ko=Ko, Vo=Vo, rs=None if rs is None else rs.cpu().numpy(), votes=vt.cpu().numpy(),
                pooled=pl.cpu().numpy())


def draw(dtype, Hq, Hkv, L, W, C, D, kernel, pooling, seed):
    w = WL.Workload("gqa", seed=seed, heads=Hkv, L=L, W=W, C=C, D=D, dtype=dtype, kernel=kernel, pooling=pooling,
                    keys="spike", spike_frac=0.02)
    _, K, V = WL.layer_arrays(w)
    wq = WL.Workload("gqa_q", seed=seed + 1, heads=Hq, L=W, W=W, C=W + 1, D=D, dtype=dtype, kernel=1,
                     pooling="avg", keys="normal")
    Q, _, _ = WL.layer_arrays(wq)
    return Q, K, V


GQA_CASES = [
    # dtype, Hq, Hkv, L, W, C, D, kernel, pooling
    ("bf16", 8, 2, 5000, 32, 512, 128, 5, "max"),
    ("bf16", 4, 2, 3001, 64, 700, 128, 3, "avg"),
    ("f32", 4, 2, 2049, 32, 300, 64, 7, "avg"),
    ("bf16", 8, 2, 20000, 32, 1024, 128, 5, "max"),   # several selection segments
    ("bf16", 4, 1, 300, 32, 1024, 128, 5, "avg"),     # bypass
    ("bf16", 6, 2, 7001, 32, 800, 128, 5, "avg"),     # three row blocks per K/V head (eight-wave kernels)
    ("bf16", 3, 1, 5000, 32, 600, 64, 3, "max"),      # three row blocks, D = 64
]


@pytest.mark.parametrize("case", GQA_CASES, ids=[f"{c[0]}-Hq{c[1]}-Hkv{c[2]}-L{c[3]}-W{c[4]}-C{c[5]}" for c in GQA_CASES])
def test_gqa_equals_expanded_heads(B, case):
    dtype, Hq, Hkv, L, W, C, D, kernel, pooling = case
    Q, K, V = draw(dtype, Hq, Hkv, L, W, C, D, kernel, pooling, seed=L + Hq)
    Qd, Kd, Vd = to_device(Q, dtype), to_device(K, dtype), to_device(V, dtype)
    G = Hq // Hkv
    log(f"gqa {case}")
    got = gqa_call(B, Qd, Kd, Vd, Hq, Hkv, L, W, C, kernel, pooling, dtype)
    Ke, Ve = Kd.repeat_interleave(G, dim=0).contiguous(), Vd.repeat_interleave(G, dim=0).contiguous()
    ref = run_select(Qd, Ke, Ve, L, W, C, kernel, pooling, dtype, "two_pass")
    n_out = min(L, C)
    assert torch.equal(got["idx"][:, :n_out], ref["idx"][:, :n_out])
    assert torch.equal(bits(got["Ko"][:, :n_out]), bits(ref["Ko"][:, :n_out]))
    assert torch.equal(bits(got["Vo"][:, :n_out]), bits(ref["Vo"][:, :n_out]))
    if L >= C:
        np.testing.assert_array_equal(got["votes"].view(np.int32), ref["votes"].view(np.int32))
        np.testing.assert_array_equal(got["pooled"].view(np.int32), ref["pooled"].view(np.int32))
        np.testing.assert_array_equal(got["rs"].view(np.int32), ref["rs"].view(np.int32))
        for h in (0, Hq - 1):
            r = O.snapkv_select(WL.to_float64(Q[h], dtype), WL.to_float64(K[h // G], dtype),
                                WL.to_float64(V[h // G], dtype), W, C, kernel, pooling)
            check_head(got, h, r, L, W, C, f"gqa {case} head {h}")


def test_gqa_workgroups_walk_several_chunks(B):
    """More chunks than resident workgroups (16 K/V heads x 20 chunks of
    1024 positions): each workgroup of the eight-wave kernels scores one or
    two chunks, some of them across a K/V head boundary, with its Qwin
    re-staged for the second head.  The expanded heads' launch splits the
    chunks differently, so the statistics may differ in the last bits: heads
    are checked against the oracle instead."""
    dtype, Hq, Hkv, L, W, C, D, kernel, pooling = "bf16", 64, 16, 20000, 32, 1024, 128, 5, "max"
    Q, K, V = draw(dtype, Hq, Hkv, L, W, C, D, kernel, pooling, seed=64)
    Qd, Kd, Vd = to_device(Q, dtype), to_device(K, dtype), to_device(V, dtype)
    log("gqa, several chunks per workgroup")
    got = gqa_call(B, Qd, Kd, Vd, Hq, Hkv, L, W, C, kernel, pooling, dtype)
    G = Hq // Hkv
    for h in (0, 3, 17, 30, 33, 46, 62, 63):
        r = O.snapkv_select(WL.to_float64(Q[h], dtype), WL.to_float64(K[h // G], dtype),
                            WL.to_float64(V[h // G], dtype), W, C, kernel, pooling)
        check_head(got, h, r, L, W, C, f"gqa several chunks head {h}")


def test_gqa_oracle_heads_and_lse(B):
    dtype, Hq, Hkv, L, W, C, D, kernel, pooling = "bf16", 8, 2, 6000, 32, 600, 128, 5, "avg"
    Q, K, V = draw(dtype, Hq, Hkv, L, W, C, D, kernel, pooling, seed=77)
    Qd, Kd, Vd = to_device(Q, dtype), to_device(K, dtype), to_device(V, dtype)
    q64, k64, v64 = (WL.to_float64(x, dtype) for x in (Q, K, V))
    log("gqa oracle parity")
    got = gqa_call(B, Qd, Kd, Vd, Hq, Hkv, L, W, C, kernel, pooling, dtype)
    refs = O.snapkv_select_gqa(q64, k64, v64, W, C, kernel, pooling)
    for h in (1, 2, 5):
        check_head(got, h, refs[h], L, W, C, f"gqa head {h}")
    log("gqa handed-over statistics")
    lse = np.stack([O.row_log_sum_exp(O.window_logits(q64[h], k64[h // 4]), L - W) for h in range(Hq)]).astype(np.float32)
    got = gqa_call(B, Qd, Kd, Vd, Hq, Hkv, L, W, C, kernel, pooling, dtype, lse=torch.from_numpy(lse).cuda())
    refs = O.snapkv_select_gqa(q64, k64, v64, W, C, kernel, pooling, row_lse=lse.astype(np.float64))
    for h in (0, 3, 6):
        check_head_lse(got, h, refs[h], L, W, C, f"gqa lse head {h}")


def test_gqa_group_of_one_is_plain_select(B):
    dtype, H, L, W, C, D = "bf16", 4, 4096, 32, 512, 128
    Q, K, V = draw(dtype, H, H, L, W, C, D, 5, "max", seed=5)
    Qd, Kd, Vd = to_device(Q, dtype), to_device(K, dtype), to_device(V, dtype)
    log("gqa group of one")
    got = gqa_call(B, Qd, Kd, Vd, H, H, L, W, C, 5, "max", dtype)
    ref = run_select(Qd, Kd, Vd, L, W, C, 5, "max", dtype)
    assert torch.equal(got["idx"], ref["idx"])
    np.testing.assert_array_equal(got["votes"].view(np.int32), ref["votes"].view(np.int32))
