"""The cooperative selection over several launches: rows whose grid does not
fit the device at once are selected a subset of rows at a time, each launch
with its own residency handshake and status block.  AUTO takes this for rows
too long for the split selection (65536 prefix positions and more);
KVSEL_SELECT_EXCHANGE takes it wherever the single launch does not fit.

The top-(C-W) with lowest-index ties is unique, so the split selection and
the cooperative selection must agree bit for bit; heads from every launch
are checked against the oracle, including exact vote ties (keys drawn from a
16-vector codebook) and the forced residency fallback."""

import numpy as np
import pytest
import torch

from oracle import snapkv_oracle as O
from prompt_kv_selection_amd import workloads as WL

from parity import bits, check_head, log, run_select, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from prompt_kv_selection_amd import binding
    return binding


def oracle_heads(Q, K, V, heads, w, out, what):
    for h in heads:
        r = O.snapkv_select(WL.to_float64(Q[h], w.dtype), WL.to_float64(K[h], w.dtype), WL.to_float64(V[h], w.dtype),
                            w.W, w.C, w.kernel, w.pooling)
        check_head(out, h, r, w.L, w.W, w.C, f"{what} head {h}")


def test_exchange_launches_match_split(B):
    # 64 rows x 10 segments: two launches on a device that holds 512 of the
    # cooperative selection's workgroups at once.
    w = WL.Workload("coop_launches", seed=71, heads=64, L=40000, W=32, C=2000, D=128, dtype="bf16", kernel=5,
                    pooling="avg", keys="spike", spike_frac=0.01)
    Q, K, V = WL.layer_arrays(w)
    Qd, Kd, Vd = to_device(Q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    log("cooperative selection over several launches vs the split selection")
    coop = run_select(Qd, Kd, Vd, w.L, w.W, w.C, w.kernel, w.pooling, w.dtype, select="exchange")
    assert "select_coop" in coop["path"], coop["path"]
    split = run_select(Qd, Kd, Vd, w.L, w.W, w.C, w.kernel, w.pooling, w.dtype, select="split")
    for key in ("idx", "Ko", "Vo"):
        assert torch.equal(bits(coop[key]), bits(split[key])), key
    np.testing.assert_array_equal(coop["pooled"].view(np.int32), split["pooled"].view(np.int32))
    oracle_heads(Q, K, V, (0, 31, 32, 63), w, coop, "coop launches")


@pytest.mark.parametrize("W,scoring", [(64, "auto"), (32, "single_read_fallback")])
def test_long_tied_rows(B, W, scoring):
    # About 70000 prefix positions (beyond the split selection), 18 segments a
    # row, 40 rows: two launches; keys from a codebook, so votes tie exactly
    # and the threshold's first digit holds far more keys than the candidate
    # round takes.  W = 64 scores on the two-pass path; W = 32 on the
    # single-read kernel forced onto its fallback, which also forces every
    # selection launch's fallback.
    w = WL.Workload("coop_launches_tied", seed=72, heads=40, L=70000, W=W, C=3000, D=128, dtype="bf16", kernel=5,
                    pooling="avg", keys="codebook", spike_frac=0.005)
    Q, K, V = WL.layer_arrays(w)
    Qd, Kd, Vd = to_device(Q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    log(f"long tied rows, scoring {scoring}")
    out = run_select(Qd, Kd, Vd, w.L, w.W, w.C, w.kernel, w.pooling, w.dtype, scoring=scoring)
    assert "select_coop" in out["path"], out["path"]
    oracle_heads(Q, K, V, (0, 39), w, out, f"long tied rows ({scoring})")
