"""Refresh selection (kvsel_refresh): indices equal the oracle's exactly on
the same float32 scores (many exact ties), protected head and tail always
kept, exactly `keep` entries, K/V rows and token ids gathered bit for bit."""

import numpy as np
import pytest
import torch

from oracle import snapkv_oracle as O

from parity import bits, log, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from prompt_kv_selection_amd import binding
    return binding


CASES = [
    # rows, n, keep, head, tail, dtype, D
    (3, 100, 40, 4, 8, "bf16", 128),
    (3, 5000, 1200, 16, 256, "bf16", 128),
    (2, 40000, 4096, 4, 1024, "bf16", 128),   # longer than one workgroup's row: segment-parallel path
    (2, 300, 300, 0, 0, "f32", 64),           # keep everything
    (2, 500, 20, 10, 10, "bf16", 128),        # no flexible budget
    (2, 2000, 1, 0, 0, "f32", 64),
    (2, 2000, 1, 1, 0, "bf16", 64),
    (2, 2000, 5, 0, 5, "bf16", 128),
    (4, 6144, 1536, 64, 512, "bf16", 128),    # J = 1536 kept of J + h = 6144 (h = J * 3)
]


@pytest.mark.parametrize("case", CASES, ids=[f"r{c[0]}-n{c[1]}-k{c[2]}-h{c[3]}-t{c[4]}-{c[5]}-D{c[6]}" for c in CASES])
def test_refresh_matches_oracle(B, case):
    rows, n, keep, head, tail, dtype, D = case
    rng = np.random.default_rng(n + keep)
    scores = (rng.integers(0, 200, size=(rows, n)) / 16.0).astype(np.float32)  # exact ties everywhere
    td = torch_dtype(dtype)
    K = torch.randn((rows, n, D), dtype=torch.float32).to(td).cuda()
    V = torch.randn((rows, n, D), dtype=torch.float32).to(td).cuda()
    tokens = torch.from_numpy(rng.integers(0, 1 << 30, size=(rows, n)).astype(np.int32)).cuda()
    sd = torch.from_numpy(scores).cuda()
    idx = torch.full((rows, keep), -1, dtype=torch.int32, device="cuda")
    Ko = torch.zeros((rows, keep, D), dtype=td, device="cuda")
    Vo = torch.zeros_like(Ko)
    to = torch.zeros((rows, keep), dtype=torch.int32, device="cuda")
    ws = torch.empty(B.kvsel_refresh_workspace_bytes(rows, n), dtype=torch.uint8, device="cuda")
    log(f"refresh {case}")
    B.kvsel_refresh(sd, rows, n, keep, head, tail, K, V, D, td, tokens, idx, Ko, Vo, to, ws)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for r in range(rows):
        ref = O.refresh_select(scores[r].astype(np.float64), keep, head, tail)
        np.testing.assert_array_equal(got[r], ref, err_msg=f"row {r}")
    gi = idx.long()
    assert torch.equal(bits(Ko), bits(torch.gather(K, 1, gi[:, :, None].expand(rows, keep, D))))
    assert torch.equal(bits(Vo), bits(torch.gather(V, 1, gi[:, :, None].expand(rows, keep, D))))
    assert torch.equal(to, torch.gather(tokens, 1, gi))


def test_refresh_negative_zero_scores(B):
    """-0.0 scores rank with the +0.0 ones (the oracle compares values)."""
    rows, n, keep, head, tail, D = 2, 6000, 1500, 4, 64, 128
    rng = np.random.default_rng(11)
    scores = (rng.integers(0, 6, size=(rows, n)) / 4.0).astype(np.float32)
    scores[(scores == 0.0) & (rng.random((rows, n)) < 0.5)] = np.float32(-0.0)
    K = torch.randn((rows, n, D), dtype=torch.float32).to(torch.bfloat16).cuda()
    V = torch.randn((rows, n, D), dtype=torch.float32).to(torch.bfloat16).cuda()
    idx = torch.full((rows, keep), -1, dtype=torch.int32, device="cuda")
    Ko = torch.zeros((rows, keep, D), dtype=torch.bfloat16, device="cuda")
    Vo = torch.zeros_like(Ko)
    ws = torch.empty(B.kvsel_refresh_workspace_bytes(rows, n), dtype=torch.uint8, device="cuda")
    log("refresh with -0.0 scores")
    B.kvsel_refresh(torch.from_numpy(scores).cuda(), rows, n, keep, head, tail, K, V, D, torch.bfloat16, None, idx,
                    Ko, Vo, None, ws)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for r in range(rows):
        np.testing.assert_array_equal(got[r], O.refresh_select(scores[r].astype(np.float64), keep, head, tail))
