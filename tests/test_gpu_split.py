"""The split selection (KVSEL_SELECT_SPLIT: every workgroup of a row finds the
threshold itself and writes a share of the row's output) against the
exchange-based kernels (KVSEL_SELECT_EXCHANGE: the cooperative selection or
the per-row / segment chains) and against the oracle.

The top-(C-W) with lowest-index ties is unique, so both families must give
the same indices and K/V rows bit for bit.  Cases cover the kernel variants'
boundaries (8192, 16384, 32768 and 65535 prefix positions), every pooling
width the kernel takes, ragged batches with a bypassed sequence, grouped
heads, handed-over statistics, more workgroups per row than picks, and the
two rare branches of the threshold: the sample's window of first-digit bins
missing the boundary (spikes placed where no sample is taken), and a
boundary bin too large for LDS (the last two digits counted from
registers)."""

import numpy as np
import pytest
import torch

from oracle import snapkv_oracle as O
from prompt_kv_selection_amd import workloads as WL

from parity import bits, check_gather, check_head, log, run_select, run_select_lse, to_device, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from prompt_kv_selection_amd import binding
    return binding


def same(a, b, what):
    for key in ("idx", "Ko", "Vo"):
        assert torch.equal(bits(a[key]), bits(b[key])), f"{what}: {key} differs between the selection kernels"
    for key in ("votes", "pooled"):
        if key in a:
            np.testing.assert_array_equal(a[key].view(np.int32), b[key].view(np.int32), err_msg=f"{what}: {key}")


# dtype, D, H, L, W, C, kernel, pooling
SHAPES = [
    ("bf16", 128, 2, 8224, 32, 700, 5, "max"),     # P = 8192: the smallest variant, full
    ("bf16", 128, 2, 8225, 32, 700, 3, "avg"),     # P = 8193: the next variant, one position into it
    ("bf16", 128, 2, 16416, 32, 2048, 7, "avg"),   # P = 16384
    ("bf16", 128, 2, 16417, 32, 2048, 1, "avg"),   # P = 16385
    ("bf16", 128, 2, 32800, 32, 1024, 5, "max"),   # P = 32768
    ("bf16", 128, 1, 32801, 32, 1024, 7, "max"),   # P = 32769: 1024 threads, two staging rounds
    ("bf16", 128, 1, 65567, 32, 6000, 5, "avg"),   # P = 65535: the largest row the split selection takes
    ("bf16", 64, 3, 5000, 32, 400, 3, "max"),      # D = 64
    ("f32", 64, 2, 3000, 32, 300, 5, "avg"),       # fp32 rows (16 pieces each)
    ("f32", 128, 2, 3000, 40, 300, 7, "max"),      # fp32 D = 128 (32 pieces), W not a multiple of 32
    ("bf16", 128, 1, 6000, 32, 37, 5, "avg"),      # 5 picks over 64 workgroups: most shares empty
    ("bf16", 128, 2, 1500, 32, 1500, 5, "avg"),    # L == C: every prefix position is picked
    ("bf16", 128, 2, 300, 32, 1024, 5, "avg"),     # bypass
]


@pytest.mark.parametrize("case", SHAPES, ids=[f"{c[0]}-D{c[1]}-H{c[2]}-L{c[3]}-W{c[4]}-C{c[5]}-k{c[6]}{c[7]}"
                                              for c in SHAPES])
def test_split_matches_exchange_and_oracle(B, case):
    dtype, D, H, L, W, C, kernel, pooling = case
    w = WL.Workload("split", seed=L + 3 * C, heads=H, L=L, W=W, C=C, D=D, dtype=dtype, kernel=kernel,
                    pooling=pooling, keys="spike", spike_frac=0.02)
    Q, K, V = WL.layer_arrays(w)
    log(f"split case {case}")
    Qd, Kd, Vd = to_device(Q, dtype), to_device(K, dtype), to_device(V, dtype)
    split = run_select(Qd, Kd, Vd, L, W, C, kernel, pooling, dtype, select="split")
    if L >= C:
        assert "select_split" in split["path"], split["path"]
    exch = run_select(Qd, Kd, Vd, L, W, C, kernel, pooling, dtype, select="exchange")
    assert "select_split" not in exch["path"], exch["path"]
    same(split, exch, f"{case}")
    check_gather(split, Kd, Vd, C, L)
    h = H - 1
    ref = O.snapkv_select(WL.to_float64(Q[h], dtype), WL.to_float64(K[h], dtype), WL.to_float64(V[h], dtype),
                          W, C, kernel, pooling)
    check_head(split, h, ref, L, W, C, f"split {case} head {h}")


def test_split_uncovered_shape_is_refused(B):
    """Forcing the split selection on a row it does not take (above 65535
    prefix positions, or a pooling width above 7) is refused before any work."""
    w = WL.Workload("split_wide", seed=5, heads=1, L=3000, W=32, C=300, D=128, dtype="bf16", kernel=9,
                    pooling="avg", keys="spike", spike_frac=0.02)
    Q, K, V = WL.layer_arrays(w)
    Qd, Kd, Vd = to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
    with pytest.raises(B.KvselError) as ei:
        run_select(Qd, Kd, Vd, 3000, 32, 300, 9, "avg", "bf16", select="split")
    assert ei.value.code == B.KVSEL_EUNSUPPORTED
    auto = run_select(Qd, Kd, Vd, 3000, 32, 300, 9, "avg", "bf16")
    assert "select_split" not in auto["path"], auto["path"]


def test_split_handed_over_statistics(B):
    w = WL.Workload("split_lse", seed=11, heads=3, L=9000, W=32, C=900, D=128, dtype="bf16", kernel=5,
                    pooling="max", keys="spike", spike_frac=0.02)
    Q, K, V = WL.layer_arrays(w)
    Qd, Kd, Vd = to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
    from test_gpu_lse import oracle_lse
    lse_d = torch.from_numpy(oracle_lse(Q, K, "bf16", 32, 9000)).cuda()
    a = run_select_lse(Qd, Kd, Vd, lse_d, 9000, 32, 900, 5, "max", "bf16", select="split")
    b = run_select_lse(Qd, Kd, Vd, lse_d, 9000, 32, 900, 5, "max", "bf16", select="exchange")
    same(a, b, "handed-over statistics")


def test_split_ragged_batch(B):
    """A ragged batch (one sequence bypassed, lengths across two variants) on
    both selection families: identical outputs."""
    w = WL.reduced(WL.get("ragged_b8_h32_l4k_64k"), heads=4, batch=6, L_min=900, L_max=40000)
    Q, K, V, Ls, Cs, cu = WL.ragged_arrays(w)
    Cs = list(Cs)
    Cs[3] = int(Ls[3]) + 9
    H, W, D = w.heads, w.W, w.D
    log(f"split ragged lengths {list(Ls)} budgets {Cs}")
    Qd, Kd, Vd = to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
    cuC = int(np.sum(Cs))
    cuP = int(np.sum([L - W for L in Ls]))
    outs = []
    for sel in (1, 2):
        B.kvsel_set_option(B.KVSEL_OPT_SELECT, sel)
        try:
            ws = torch.empty(B.kvsel_varlen_workspace_bytes(cu.tolist(), Cs, H, W, D, torch.bfloat16),
                             dtype=torch.uint8, device="cuda")
            idx = torch.full((H * cuC,), -1, dtype=torch.int32, device="cuda")
            Ko = torch.zeros((H * cuC, D), dtype=torch.bfloat16, device="cuda")
            Vo = torch.zeros_like(Ko)
            pl = torch.zeros((H * cuP,), dtype=torch.float32, device="cuda")
            B.kvsel_select_varlen(Qd, Kd, Vd, cu.tolist(), Cs, W, D, H, w.kernel, w.pooling, torch.bfloat16, idx,
                                  Ko, Vo, None, None, pl, ws)
            torch.cuda.synchronize()
            assert B.kvsel_status(ws) == B.KVSEL_OK
            outs.append(dict(idx=idx, Ko=Ko, Vo=Vo, pooled=pl.cpu().numpy(),
                             path=B.path_names(B.kvsel_last_path())))
        finally:
            B.kvsel_set_option(B.KVSEL_OPT_SELECT, 0)
    assert "select_split" in outs[0]["path"] and "select_split" not in outs[1]["path"]
    same(outs[0], outs[1], "ragged batch")


def test_split_grouped_heads(B):
    from test_gpu_gqa import draw, gqa_call
    Q, K, V = draw("bf16", 8, 2, 20000, 32, 1024, 128, 5, "max", seed=77)
    Qd, Kd, Vd = to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
    outs = []
    for sel in (1, 2):
        B.kvsel_set_option(B.KVSEL_OPT_SELECT, sel)
        try:
            outs.append(gqa_call(B, Qd, Kd, Vd, 8, 2, 20000, 32, 1024, 5, "max", "bf16"))
        finally:
            B.kvsel_set_option(B.KVSEL_OPT_SELECT, 0)
    same(outs[0], outs[1], "grouped heads")


# ----------------------------------------------------------------- the threshold's branches, on given scores

def topk(B, s, count, select):
    rows, n = s.shape
    sd = torch.from_numpy(s).cuda()
    out = torch.full((rows, count), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(B.kvsel_topk_workspace_bytes(rows, n), dtype=torch.uint8, device="cuda")
    B.kvsel_set_option(B.KVSEL_OPT_SELECT, select)
    try:
        B.kvsel_topk(sd, rows, n, count, out, count, ws)
        torch.cuda.synchronize()
        path = B.path_names(B.kvsel_last_path())
    finally:
        B.kvsel_set_option(B.KVSEL_OPT_SELECT, 0)
    return out.cpu().numpy(), path


def sample_free_positions(n, kpt):
    """Positions no sample is taken from: thread t samples position
    t * kpt + kpt / 4 (odd t) or t * kpt + 3 kpt / 4 (even t)."""
    p = np.arange(n)
    u = p % kpt
    return p[(u != kpt // 4) & (u != (3 * kpt) // 4)]


@pytest.mark.parametrize("n,kpt", [(5000, 16), (12000, 32), (30000, 64), (50000, 64)])
def test_window_miss_falls_back_to_full_histogram(B, n, kpt):
    """A handful of huge scores, none of them sampled, far above the rest:
    the sample's estimate lies many bins below the boundary, the exact
    window counts see more than count keys above it, and the full histogram
    takes over.  Exactly the oracle's ranking."""
    rng = np.random.default_rng(n)
    s = rng.random((2, n)).astype(np.float32)
    count = 6
    free = sample_free_positions(n, kpt)
    for r in range(2):
        spots = rng.choice(free, size=count + 3, replace=False)
        s[r, spots] = (2.0 ** rng.integers(20, 40, size=count + 3)).astype(np.float32)
    got, path = topk(B, s, count, 1)
    assert "select_split" in path, path
    for r in range(2):
        np.testing.assert_array_equal(got[r], O.top_prefix(s[r].astype(np.float64), count))


@pytest.mark.parametrize("n,count", [(40000, 20000), (65535, 1), (65535, 65535), (34000, 33999)])
def test_boundary_bin_larger_than_lds(B, n, count):
    """Every score equal except a few (rows above 33286 positions): the
    boundary bin holds more keys than LDS takes, so its last two digits are
    counted from the keys in registers; ties go to the lowest indices."""
    rng = np.random.default_rng(n + count)
    s = np.full((2, n), 0.75, dtype=np.float32)
    s[0, rng.choice(n, size=50, replace=False)] = 0.5
    s[1, rng.choice(n, size=50, replace=False)] = 1.0
    got, path = topk(B, s, count, 1)
    assert "select_split" in path, path
    for r in range(2):
        np.testing.assert_array_equal(got[r], O.top_prefix(s[r].astype(np.float64), count))


@pytest.mark.parametrize("n", [1, 2, 31, 1000, 8192, 8193, 65535])
def test_split_topk_matches_oracle_on_dense_ties(B, n):
    rng = np.random.default_rng(3 * n)
    s = (rng.integers(0, 9, size=(3, n)) * 0.5).astype(np.float32)
    s[2] = 0.0
    for count in sorted({1, max(1, n // 7), n}):
        got, path = topk(B, s, count, 1)
        assert "select_split" in path, path
        for r in range(3):
            np.testing.assert_array_equal(got[r], O.top_prefix(s[r].astype(np.float64), count), err_msg=f"n={n} "
                                          f"count={count} row {r}")
