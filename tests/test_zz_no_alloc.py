"""Allocation-free entry point (kvsel_select_noalloc) against kvsel_select.

The allocation-free call runs the same kernels on the library's per-device
scratch array instead of a caller's workspace, so its outputs must equal
kvsel_select's bit for bit.  Two calls in a row, the second smaller, check
that the scratch left behind by the first does not leak into the second; the
first has the benchmark layer's shape and launch configuration (32 heads,
L = 32768).  A shape whose workspace exceeds the array is rejected before any
launch."""

import numpy as np
import pytest
import torch

from oracle import snapkv_oracle as O
from prompt_kv_selection_amd import workloads as WL

from parity import band_check, bits, close, log, to_device, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from prompt_kv_selection_amd import binding
    return binding


def outputs(w, H, L, C, D):
    td = torch_dtype(w.dtype)
    return dict(idx=torch.full((H, C), -7, dtype=torch.int32, device="cuda"),
                Ko=torch.zeros((H, C, D), dtype=td, device="cuda"),
                Vo=torch.zeros((H, C, D), dtype=td, device="cuda"),
                rs=torch.full((H, w.W, 2), float("nan"), dtype=torch.float32, device="cuda"),
                votes=torch.full((H, L - w.W), float("nan"), dtype=torch.float32, device="cuda"),
                pooled=torch.full((H, L - w.W), float("nan"), dtype=torch.float32, device="cuda"))


def run_both(B, w):
    Q, K, V = WL.layer_arrays(w)
    Qd, Kd, Vd = to_device(Q, w.dtype), to_device(K, w.dtype), to_device(V, w.dtype)
    H, L, D = Kd.shape
    td = torch_dtype(w.dtype)
    ref = outputs(w, H, L, w.C, D)
    ws = torch.empty(B.kvsel_workspace_bytes(H, L, w.W, w.C, D, td), dtype=torch.uint8, device="cuda")
    B.kvsel_select(Qd, Kd, Vd, L, w.W, w.C, D, H, w.kernel, w.pooling, td, ref["idx"], ref["Ko"], ref["Vo"],
                   ref["rs"], ref["votes"], ref["pooled"], ws)
    assert B.kvsel_status(ws) == B.KVSEL_OK, B.kvsel_last_error()
    got = outputs(w, H, L, w.C, D)
    B.kvsel_select_noalloc(Qd, Kd, Vd, L, w.W, w.C, D, H, w.kernel, w.pooling, td, got["idx"], got["Ko"],
                           got["Vo"], got["rs"], got["votes"], got["pooled"])
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(bits(got[k]), bits(ref[k])), f"{w.name}: {k} differs from kvsel_select"
    return Q, K, V, got


def test_noalloc_matches_select_twice(B):
    big = WL.get("spike_l32x_h32_l32k")
    small = WL.reduced(WL.get("lognorm_h32_l16k"), L=5000, heads=4, layers=1, C=400)
    log("noalloc: 32 heads, L = 32768 (benchmark layer shape)")
    run_both(B, big)
    log("noalloc: 4 heads, L = 5000, right after the larger call")
    Q, K, V, got = run_both(B, small)
    # One head of the smaller call against the oracle as well.
    h = 2
    ref = O.snapkv_select(WL.to_float64(Q[h], small.dtype), WL.to_float64(K[h], small.dtype),
                          WL.to_float64(V[h], small.dtype), small.W, small.C, small.kernel, small.pooling)
    close(got["votes"][h].cpu().numpy(), ref["votes"], "noalloc votes")
    close(got["pooled"][h].cpu().numpy(), ref["pooled"], "noalloc pooled")
    n = small.C - small.W
    band_check(got["idx"][h, :n].cpu().numpy(), ref["pooled"], n, "noalloc selection")


def test_noalloc_rejects_shapes_beyond_the_scratch(B):
    H, L, W, C, D = 64, 131072, 64, 4096, 128
    need = B.kvsel_workspace_bytes(H, L, W, C, D, torch.bfloat16)
    assert need > B.KVSEL_NOALLOC_SCRATCH_BYTES
    t = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    idx = torch.empty(16, dtype=torch.int32, device="cuda")
    with pytest.raises(B.KvselError) as e:
        B.kvsel_select_noalloc(t, t, t, L, W, C, D, H, 5, "avg", torch.bfloat16, idx, t, t)
    assert e.value.code == B.KVSEL_EWORKSPACE
    assert "scratch" in str(e.value)
