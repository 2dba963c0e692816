"""Helpers shared by the GPU parity tests: moving generator bytes to the
device, running the HIP path through the C ABI, and comparing with the CPU
oracle under the stated tolerances.

Tolerances (votes and pooled scores within 1e-3 relative for bf16 inputs with
fp32 accumulation; selections equal except inside a 1e-3 relative band around
the oracle's boundary score; gathered K/V bit-exact):
  * votes, pooled:  |gpu - oracle| <= 1e-3 * |oracle| + 1e-30
  * row stats:      |(m + ln Z)_gpu - (m + ln Z)_oracle| <= 1e-4 * max(1, |.|)
  * selection:      with tau the oracle's (C-W)-th pooled score, the GPU set
                    has C-W distinct prefix positions, contains every j with
                    pooled_j > tau (1 + 1e-3), none with pooled_j < tau (1 - 1e-3),
                    and equals the oracle set when the band holds only exact
                    ties of tau; the window positions follow in order
  * GPU-internal:   the GPU picks are exactly the top C-W of the GPU's own
                    fp32 pooled scores, lowest index first on ties
  * K_out, V_out:   bit-equal to K[idx], V[idx]
"""

from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import snapkv_oracle as O
from prompt_kv_selection_amd import workloads as WL

REL = 1e-3
ABS = 1e-30


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(stored: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(stored).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(stored, dtype=np.float32)).cuda()


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def band_check(gpu_prefix: np.ndarray, pooled: np.ndarray, n: int, what: str = "") -> None:
    P = pooled.shape[0]
    g = np.asarray(gpu_prefix, dtype=np.int64)
    assert g.shape == (n,), (what, g.shape, n)
    assert np.all((g >= 0) & (g < P)), what
    assert len(np.unique(g)) == n, f"{what}: duplicate picks"
    assert np.all(np.diff(g) > 0), f"{what}: picks not ascending"
    order = np.lexsort((np.arange(P), -pooled))
    tau = pooled[order[n - 1]]
    sel = np.zeros(P, dtype=bool)
    sel[g] = True
    must = pooled > tau * (1 + REL)
    never = pooled < tau * (1 - REL)
    missing = np.where(must & ~sel)[0]
    extra = np.where(never & sel)[0]
    assert missing.size == 0, f"{what}: {missing.size} positions above the band not picked, e.g. {missing[:5]}"
    assert extra.size == 0, f"{what}: {extra.size} positions below the band picked, e.g. {extra[:5]}"
    band = ~must & ~never
    if np.all(pooled[band] == tau):
        expect = np.sort(order[:n])
        np.testing.assert_array_equal(g, expect, err_msg=f"{what}: exact-tie band, lowest-index rule")


def close(gpu: np.ndarray, ref: np.ndarray, what: str) -> None:
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - ref)
    lim = REL * np.abs(ref) + ABS
    bad = np.where(err > lim)[0] if err.ndim == 1 else np.argwhere(err > lim)
    assert len(bad) == 0, (f"{what}: {len(bad)} of {ref.size} outside 1e-3 rel; first {bad[:3]} "
                           f"gpu={gpu.ravel()[:3]} ref={ref.ravel()[:3]}")


def gpu_internal_topk(gpu_prefix: np.ndarray, gpu_pooled_f32: np.ndarray, n: int, what: str) -> None:
    expect = O.top_prefix(gpu_pooled_f32.astype(np.float64), n)
    np.testing.assert_array_equal(np.asarray(gpu_prefix, dtype=np.int64), expect,
                                  err_msg=f"{what}: GPU picks differ from top-n of the GPU's own scores")


SELECT = {"auto": 0, "split": 1, "exchange": 2}


def run_select(Qd, Kd, Vd, L, W, C, kernel, pooling, dtype: str, scoring: str = "auto", select: str = "auto"):
    """Run kvsel_select with every optional output; returns host numpy arrays.
    `scoring` picks the scoring path (auto, two_pass, single_read, or
    single_read_fallback: the single-read launch forced onto its two-pass
    fallback); `select` the selection kernels (auto, split, or exchange:
    the cooperative selection or the per-row / segment chains)."""
    from prompt_kv_selection_amd import binding as B
    fallback = scoring == "single_read_fallback"
    B.kvsel_set_option(B.KVSEL_OPT_SCORING, B.SCORING["single_read" if fallback else scoring])
    B.kvsel_set_option(B.KVSEL_OPT_FORCE_FALLBACK, 1 if fallback else 0)
    B.kvsel_set_option(B.KVSEL_OPT_SELECT, SELECT[select])
    try:
        return _run_select(B, Qd, Kd, Vd, L, W, C, kernel, pooling, dtype)
    finally:
        B.kvsel_set_option(B.KVSEL_OPT_SCORING, 0)
        B.kvsel_set_option(B.KVSEL_OPT_FORCE_FALLBACK, 0)
        B.kvsel_set_option(B.KVSEL_OPT_SELECT, 0)


def run_select_lse(Qd, Kd, Vd, lse_d, L, W, C, kernel, pooling, dtype: str, scoring: str = "auto",
                   select: str = "auto"):
    """Run kvsel_select_lse (row statistics handed over as lse_d [H, W]
    float32 on the device) with votes and pooled outputs; host numpy arrays."""
    from prompt_kv_selection_amd import binding as B
    H, _, D = Kd.shape
    td = torch_dtype(dtype)
    B.kvsel_set_option(B.KVSEL_OPT_SCORING, B.SCORING[scoring])
    B.kvsel_set_option(B.KVSEL_OPT_SELECT, SELECT[select])
    try:
        ws = torch.empty(B.kvsel_workspace_bytes(H, L, W, C, D, td), dtype=torch.uint8, device="cuda")
        idx = torch.full((H, C), -7, dtype=torch.int32, device="cuda")
        Ko = torch.zeros((H, C, D), dtype=td, device="cuda")
        Vo = torch.zeros((H, C, D), dtype=td, device="cuda")
        vt = torch.full((H, L - W), float("nan"), dtype=torch.float32, device="cuda")
        pl = torch.full((H, L - W), float("nan"), dtype=torch.float32, device="cuda")
        B.kvsel_select_lse(Qd, Kd, Vd, lse_d, L, W, C, D, H, kernel, pooling, td, idx, Ko, Vo, vt, pl, ws)
        torch.cuda.synchronize()
    finally:
        B.kvsel_set_option(B.KVSEL_OPT_SCORING, 0)
        B.kvsel_set_option(B.KVSEL_OPT_SELECT, 0)
    return dict(idx=idx, Ko=Ko, Vo=Vo, votes=vt.cpu().numpy(), pooled=pl.cpu().numpy())


def check_head_lse(out, h, ref, L, W, C, what):
    """Compare head h of a kvsel_select_lse result with the oracle's
    snapkv_select_lse result on the same (float32) statistics."""
    n_out = min(L, C)
    idx = out["idx"][h, :n_out].cpu().numpy()
    if L < C:
        np.testing.assert_array_equal(idx, np.arange(L), err_msg=what)
        return
    P = L - W
    close(out["votes"][h], ref["votes"], f"{what} votes")
    close(out["pooled"][h], ref["pooled"], f"{what} pooled")
    n = C - W
    band_check(idx[:n], ref["pooled"], n, what)
    gpu_internal_topk(idx[:n], out["pooled"][h], n, what)
    np.testing.assert_array_equal(idx[n:], np.arange(P, L), err_msg=f"{what} window")


def single_read_covers(dtype, D, W):
    return dtype == "bf16" and D in (64, 128) and W <= 32


def _run_select(B, Qd, Kd, Vd, L, W, C, kernel, pooling, dtype):
    H, _, D = Kd.shape
    td = torch_dtype(dtype)
    ws = torch.empty(B.kvsel_workspace_bytes(H, L, W, C, D, td), dtype=torch.uint8, device="cuda")
    idx = torch.full((H, C), -7, dtype=torch.int32, device="cuda")
    Ko = torch.zeros((H, C, D), dtype=td, device="cuda")
    Vo = torch.zeros((H, C, D), dtype=td, device="cuda")
    rs = torch.full((H, W, 2), float("nan"), dtype=torch.float32, device="cuda")
    vt = torch.full((H, L - W), float("nan"), dtype=torch.float32, device="cuda")
    pl = torch.full((H, L - W), float("nan"), dtype=torch.float32, device="cuda")
    B.kvsel_select(Qd, Kd, Vd, L, W, C, D, H, kernel, pooling, td, idx, Ko, Vo, rs, vt, pl, ws)
    torch.cuda.synchronize()
    assert B.kvsel_status(ws) == B.KVSEL_OK, B.kvsel_last_error()
    return dict(idx=idx, Ko=Ko, Vo=Vo, rs=rs.cpu().numpy(), votes=vt.cpu().numpy(), pooled=pl.cpu().numpy(),
                path=B.path_names(B.kvsel_last_path()), flags=B.flag_names(B.kvsel_status_flags(ws)[0]))


def check_head(out, h, ref, L, W, C, what, gather_rows=True):
    """Compare head h of a kvsel_select result with the oracle's result."""
    n_out = min(L, C)
    idx = out["idx"][h, :n_out].cpu().numpy()
    if L < C:
        np.testing.assert_array_equal(idx, np.arange(L), err_msg=what)
    else:
        P = L - W
        close(out["votes"][h], ref["votes"], f"{what} votes")
        close(out["pooled"][h], ref["pooled"], f"{what} pooled")
        lse_g = out["rs"][h, :, 0].astype(np.float64) + np.log(out["rs"][h, :, 1].astype(np.float64))
        lse_o = ref["row_max"] + np.log(ref["row_sum"])
        assert np.all(np.abs(lse_g - lse_o) <= 1e-4 * np.maximum(1, np.abs(lse_o))), f"{what} row stats"
        n = C - W
        band_check(idx[:n], ref["pooled"], n, what)
        gpu_internal_topk(idx[:n], out["pooled"][h], n, what)
        np.testing.assert_array_equal(idx[n:], np.arange(P, L), err_msg=f"{what} window")


def check_gather(out, Kd, Vd, C, L):
    """K_out / V_out rows are bit copies of K / V at the emitted indices."""
    n_out = min(L, C)
    idx = out["idx"][:, :n_out].long()
    H, _, D = Kd.shape
    gi = idx[:, :, None].expand(H, n_out, D)
    ek = torch.gather(Kd, 1, gi)
    ev = torch.gather(Vd, 1, gi)
    assert torch.equal(bits(out["Ko"][:, :n_out]), bits(ek)), "K_out rows differ from K[idx]"
    assert torch.equal(bits(out["Vo"][:, :n_out]), bits(ev)), "V_out rows differ from V[idx]"


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)
