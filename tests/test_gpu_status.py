"""Device-side outcome of a call (kvsel_status): clean calls report OK; a
non-finite key (seen through its row normaliser on every call) or any
non-finite input (validating mode) reports KVSEL_ENONFINITE, on every scoring
path, while the call still completes with in-range indices."""

import math

import numpy as np
import pytest
import torch

from prompt_kv_selection_amd import workloads as WL

from parity import log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from prompt_kv_selection_amd import binding
    return binding


def inputs(H=2, L=5000, W=32, D=128, seed=3):
    w = WL.Workload("status", seed=seed, heads=H, L=L, W=W, C=512, D=D, dtype="bf16", kernel=5, pooling="max",
                    keys="spike", spike_frac=0.01)
    return w, WL.layer_arrays(w)


def call(B, Q, K, V, w, lse=None, scoring="auto", validate=False):
    """One selection call; returns (status code, indices)."""
    B.kvsel_set_option(B.KVSEL_OPT_SCORING, B.SCORING[scoring])
    B.kvsel_set_option(B.KVSEL_OPT_VALIDATE, 1 if validate else 0)
    try:
        H, L, D = K.shape
        ws = torch.empty(B.kvsel_workspace_bytes(H, L, w.W, w.C, D, torch.bfloat16), dtype=torch.uint8, device="cuda")
        ws.fill_(0xAB)  # the call must clear its own flags
        idx = torch.full((H, w.C), -1, dtype=torch.int32, device="cuda")
        Ko = torch.empty((H, w.C, D), dtype=torch.bfloat16, device="cuda")
        Vo = torch.empty_like(Ko)
        if lse is None:
            B.kvsel_select(Q, K, V, L, w.W, w.C, D, H, w.kernel, w.pooling, torch.bfloat16, idx, Ko, Vo, None, None,
                           None, ws)
        else:
            B.kvsel_select_lse(Q, K, V, lse, L, w.W, w.C, D, H, w.kernel, w.pooling, torch.bfloat16, idx, Ko, Vo,
                               None, None, ws)
        rc = B.kvsel_status(ws)
        torch.cuda.synchronize()
        return rc, idx.cpu().numpy()
    finally:
        B.kvsel_set_option(B.KVSEL_OPT_SCORING, 0)
        B.kvsel_set_option(B.KVSEL_OPT_VALIDATE, 0)


def nan_bits():
    return np.uint16(0x7FC0)


@pytest.mark.parametrize("scoring", ["single_read", "two_pass"])
def test_status_clean_and_nonfinite_key(B, scoring):
    w, (Q, K, V) = inputs()
    log(f"status: clean call, scoring={scoring}")
    Qd, Kd, Vd = to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
    rc, idx = call(B, Qd, Kd, Vd, w, scoring=scoring)
    assert rc == B.KVSEL_OK, B.kvsel_last_error()
    log(f"status: NaN key element, scoring={scoring}")
    K2 = K.copy()
    K2[1, 777, 5] = nan_bits()
    rc, idx = call(B, Qd, to_device(K2, "bf16"), Vd, w, scoring=scoring)
    assert rc == B.KVSEL_ENONFINITE, B.kvsel_last_error()
    P = w.L - w.W
    n = w.C - w.W
    assert np.all((idx[:, :n] >= 0) & (idx[:, :n] < P)), "indices stay in range"
    assert np.array_equal(idx[0, n:], np.arange(P, w.L))


@pytest.mark.parametrize("where", ["Q", "V"])
def test_validating_mode_flags_nonfinite_inputs(B, where):
    """A NaN in V never reaches the arithmetic, and a NaN in a window query
    could hide in a row that contributes nothing; the validating mode scans
    every element and flags both."""
    w, (Q, K, V) = inputs(seed=5)
    Qd, Kd, Vd = to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
    log(f"status: validating mode, clean inputs")
    rc, _ = call(B, Qd, Kd, Vd, w, validate=True)
    assert rc == B.KVSEL_OK, B.kvsel_last_error()
    if where == "V":
        V2 = V.copy()
        V2[0, 4000, 100] = nan_bits()
        Vd = to_device(V2, "bf16")
    else:
        Q2 = Q.copy()
        Q2[1, 3, 17] = np.uint16(0xFF80)  # -inf
        Qd = to_device(Q2, "bf16")
    log(f"status: validating mode, non-finite {where}")
    rc, _ = call(B, Qd, Kd, Vd, w, validate=True)
    assert rc == B.KVSEL_ENONFINITE, B.kvsel_last_error()
    if where == "V":
        rc, _ = call(B, Qd, Kd, Vd, w, validate=False)  # not seen without the scan
        assert rc == B.KVSEL_OK


@pytest.mark.parametrize("scoring", ["single_read", "two_pass"])
def test_status_nonfinite_lse(B, scoring):
    w, (Q, K, V) = inputs(seed=9)
    Qd, Kd, Vd = to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
    lse = torch.full((w.heads, w.W), 10.0, dtype=torch.float32, device="cuda")
    log(f"status: finite lse, scoring={scoring}")
    rc, _ = call(B, Qd, Kd, Vd, w, lse=lse, scoring=scoring)
    assert rc == B.KVSEL_OK, B.kvsel_last_error()
    lse[1, 7] = math.inf
    log(f"status: infinite lse, scoring={scoring}")
    rc, _ = call(B, Qd, Kd, Vd, w, lse=lse, scoring=scoring)
    assert rc == B.KVSEL_ENONFINITE, B.kvsel_last_error()


@pytest.mark.parametrize("H,W", [(1, 2), (3, 5), (2, 32)])
def test_validating_mode_checks_every_lse(B, H, W):
    """The validating scan reads every handed-over log-sum-exp, including a
    tail that is not a whole 16-byte unit (heads * W not a multiple of 4)."""
    w = WL.Workload("status_lse", seed=21, heads=H, L=3000, W=W, C=400, D=128, dtype="bf16", kernel=3,
                    pooling="avg", keys="normal")
    Q, K, V = WL.layer_arrays(w)
    Qd, Kd, Vd = to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
    lse = torch.full((H, W), 12.0, dtype=torch.float32, device="cuda")
    log(f"status: validating mode, finite lse H={H} W={W}")
    rc, _ = call(B, Qd, Kd, Vd, w, lse=lse, validate=True)
    assert rc == B.KVSEL_OK, B.kvsel_last_error()
    lse[H - 1, W - 1] = math.nan  # the very last element
    log(f"status: validating mode, NaN in the last lse H={H} W={W}")
    rc, _ = call(B, Qd, Kd, Vd, w, lse=lse, validate=True)
    assert rc == B.KVSEL_ENONFINITE, B.kvsel_last_error()
