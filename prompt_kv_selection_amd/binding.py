"""ctypes binding of libkvsel.so (C ABI in include/kvsel.h).

Functions carry the C names and take PyTorch tensors; they only marshal
pointers, sizes and the current HIP stream.  Every step of the selection runs
in the library's HIP kernels: there is no other implementation behind these
calls, and importing this module raises if the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvsel.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libkvsel_debug.so")  # the same library built with KVSEL_DEBUG

KVSEL_OK = 0
KVSEL_EINVAL = -1
KVSEL_EUNSUPPORTED = -2
KVSEL_EWORKSPACE = -3
KVSEL_EDEVICE = -4
KVSEL_ENONFINITE = -5
POOL = {"avg": 0, "max": 1}
DTYPE = {torch.float32: 0, torch.bfloat16: 1, "f32": 0, "bf16": 1}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m prompt_kv_selection_amd.build`")

lib = ctypes.CDLL(LIB_PATH)

_vp, _i, _sz, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)

lib.kvsel_version.restype = _i
lib.kvsel_version.argtypes = []
lib.kvsel_last_error.restype = ctypes.c_char_p
lib.kvsel_last_error.argtypes = []
lib.kvsel_status.restype = _i
lib.kvsel_status.argtypes = [_vp, _vp]
lib.kvsel_status_flags.restype = _i
lib.kvsel_status_flags.argtypes = [_vp, _vp, _i, ctypes.POINTER(ctypes.c_uint), ctypes.POINTER(ctypes.c_uint)]
lib.kvsel_last_path.restype = ctypes.c_uint
lib.kvsel_last_path.argtypes = []
FLAG = {"exchange_wait": 0x1, "lds_wait": 0x2, "select_wait": 0x4, "nonfinite": 0x8, "domain": 0x10,
        "index_range": 0x20, "scoring_fallback": 0x100, "select_fallback": 0x200}
lib.kvsel_debug_flags.restype = _i
lib.kvsel_debug_flags.argtypes = [_i]
PATH = {"single_read": 0x1, "two_pass": 0x2, "votes_only": 0x4, "handed_over": 0x8, "bypass": 0x10,
        "select_coop": 0x20, "select_rows": 0x40, "select_segments": 0x80, "select_fused": 0x100,
        "select_split": 0x200}
lib.kvsel_probe_sink_bytes.restype = _sz
lib.kvsel_probe_sink_bytes.argtypes = []
lib.kvsel_probe_stream.restype = _i
lib.kvsel_probe_stream.argtypes = [_vp, _sz, _i, _vp, _sz, _vp]
lib.kvsel_workspace_bytes.restype = _sz
lib.kvsel_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
lib.kvsel_varlen_workspace_bytes.restype = _sz
lib.kvsel_varlen_workspace_bytes.argtypes = [_i32p, _i32p, _i, _i, _i, _i, _i]
lib.kvsel_select.restype = _i
lib.kvsel_select.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i,
                             _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
lib.kvsel_select_varlen.restype = _i
lib.kvsel_select_varlen.argtypes = [_vp, _vp, _vp, _i32p, _i32p, _i, _i, _i, _i, _i, _i, _i,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
lib.kvsel_select_lse.restype = _i
lib.kvsel_select_lse.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
lib.kvsel_select_varlen_lse.restype = _i
lib.kvsel_select_varlen_lse.argtypes = [_vp, _vp, _vp, _vp, _i32p, _i32p, _i, _i, _i, _i, _i, _i, _i,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
lib.kvsel_gqa_workspace_bytes.restype = _sz
lib.kvsel_gqa_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i]
lib.kvsel_select_gqa.restype = _i
lib.kvsel_select_gqa.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
lib.kvsel_select_noalloc.restype = _i
lib.kvsel_select_noalloc.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i,
                                     _vp, _vp, _vp, _vp, _vp, _vp, _vp]
KVSEL_NOALLOC_SCRATCH_BYTES = 32 << 20
lib.kvsel_topk_workspace_bytes.restype = _sz
lib.kvsel_topk_workspace_bytes.argtypes = [_i, _i]
lib.kvsel_topk.restype = _i
lib.kvsel_topk.argtypes = [_vp, _i, _i, _i, _vp, _i, _vp, _sz, _vp]
lib.kvsel_refresh_workspace_bytes.restype = _sz
lib.kvsel_refresh_workspace_bytes.argtypes = [_i, _i]
lib.kvsel_refresh.restype = _i
lib.kvsel_refresh.argtypes = [_vp, _i, _i, _i, _i, _i, _vp, _vp, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
lib.kvsel_jacap_workspace_bytes.restype = _sz
lib.kvsel_jacap_workspace_bytes.argtypes = [_i, _i, _i]
lib.kvsel_jacap_select.restype = _i
lib.kvsel_jacap_select.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, _i, _i, _i, _i, _i, _i, _i,
                                   _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
lib.kvsel_pool1d.restype = _i
lib.kvsel_pool1d.argtypes = [_vp, _i, _i, _i, _i, _vp, _vp]
lib.kvsel_gather.restype = _i
lib.kvsel_gather.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp]


class KvselError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"kvsel error {code}: {message}")
        self.code = code


def _check(rc: int) -> None:
    if rc != KVSEL_OK:
        raise KvselError(rc, kvsel_last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _i32_array(values: Sequence[int]):
    arr = (ctypes.c_int32 * len(values))(*[int(v) for v in values])
    return arr


def kvsel_status_flags(workspace, stream=None, reset=False):
    """(last call's flags, sticky flags since the last reset) of a
    workspace; waits for the stream.  reset=True clears the sticky word."""
    last, sticky = ctypes.c_uint(0), ctypes.c_uint(0)
    _check(lib.kvsel_status_flags(_ptr(workspace), _stream(stream), 1 if reset else 0, ctypes.byref(last),
                                  ctypes.byref(sticky)))
    return last.value, sticky.value


def kvsel_probe_stream(src, mode, sink, stream=None, nbytes=None) -> None:
    """Streaming-read probe over src (a device tensor; nbytes of it)."""
    n = src.numel() * src.element_size() if nbytes is None else nbytes
    _check(lib.kvsel_probe_stream(_ptr(src), n, mode, _ptr(sink), sink.numel() * sink.element_size(),
                                  _stream(stream)))


def kvsel_probe_sink_bytes() -> int:
    return lib.kvsel_probe_sink_bytes()


def kvsel_last_path() -> int:
    return lib.kvsel_last_path()


def flag_names(flags: int):
    return [k for k, v in FLAG.items() if flags & v]


def path_names(path: int):
    return [k for k, v in PATH.items() if path & v]


def kvsel_version() -> int:
    return lib.kvsel_version()


def kvsel_last_error() -> str:
    return lib.kvsel_last_error().decode()


def kvsel_status(workspace, stream=None) -> int:
    """Device-side outcome of the last selection call that used `workspace`
    (waits for the stream): KVSEL_OK, KVSEL_ENONFINITE or KVSEL_EDEVICE."""
    return lib.kvsel_status(_ptr(workspace), _stream(stream))


def kvsel_workspace_bytes(heads: int, L: int, W: int, C: int, D: int, dtype) -> int:
    n = lib.kvsel_workspace_bytes(heads, L, W, C, D, DTYPE.get(dtype, dtype))
    if n == 0:
        raise KvselError(KVSEL_EINVAL, kvsel_last_error())
    return n


def kvsel_varlen_workspace_bytes(cu_L: Sequence[int], C: Sequence[int], heads: int, W: int, D: int, dtype) -> int:
    B = len(C)
    n = lib.kvsel_varlen_workspace_bytes(_i32_array(cu_L), _i32_array(C), B, heads, W, D, DTYPE.get(dtype, dtype))
    if n == 0:
        raise KvselError(KVSEL_EINVAL, kvsel_last_error())
    return n


def kvsel_select(Qwin, K, V, L, W, C, D, heads, kernel, pooling, dtype, indices, K_out, V_out,
                 row_stats=None, votes=None, pooled=None, workspace=None, workspace_bytes=None,
                 stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(lib.kvsel_select(_ptr(Qwin), _ptr(K), _ptr(V), L, W, C, D, heads, kernel,
                            POOL.get(pooling, pooling), DTYPE.get(dtype, dtype),
                            _ptr(indices), _ptr(K_out), _ptr(V_out), _ptr(row_stats), _ptr(votes),
                            _ptr(pooled), _ptr(workspace), ws_bytes, _stream(stream)))


def kvsel_select_noalloc(Qwin, K, V, L, W, C, D, heads, kernel, pooling, dtype, indices, K_out, V_out,
                         row_stats=None, votes=None, pooled=None, stream=None) -> None:
    """kvsel_select without a workspace: the library's per-device scratch
    array serves instead (calls on one GPU must not overlap)."""
    _check(lib.kvsel_select_noalloc(_ptr(Qwin), _ptr(K), _ptr(V), L, W, C, D, heads, kernel,
                                    POOL.get(pooling, pooling), DTYPE.get(dtype, dtype),
                                    _ptr(indices), _ptr(K_out), _ptr(V_out), _ptr(row_stats), _ptr(votes),
                                    _ptr(pooled), _stream(stream)))


def kvsel_select_varlen(Qwin, K, V, cu_L, C, W, D, heads, kernel, pooling, dtype, indices, K_out, V_out,
                        row_stats=None, votes=None, pooled=None, workspace=None, workspace_bytes=None,
                        stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(lib.kvsel_select_varlen(_ptr(Qwin), _ptr(K), _ptr(V), _i32_array(cu_L), _i32_array(C), len(C),
                                   W, D, heads, kernel, POOL.get(pooling, pooling), DTYPE.get(dtype, dtype),
                                   _ptr(indices), _ptr(K_out), _ptr(V_out), _ptr(row_stats), _ptr(votes),
                                   _ptr(pooled), _ptr(workspace), ws_bytes, _stream(stream)))


def kvsel_select_lse(Qwin, K, V, row_lse, L, W, C, D, heads, kernel, pooling, dtype, indices, K_out, V_out,
                     votes=None, pooled=None, workspace=None, workspace_bytes=None, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(lib.kvsel_select_lse(_ptr(Qwin), _ptr(K), _ptr(V), _ptr(row_lse), L, W, C, D, heads, kernel,
                                POOL.get(pooling, pooling), DTYPE.get(dtype, dtype),
                                _ptr(indices), _ptr(K_out), _ptr(V_out), _ptr(votes), _ptr(pooled),
                                _ptr(workspace), ws_bytes, _stream(stream)))


def kvsel_select_varlen_lse(Qwin, K, V, row_lse, cu_L, C, W, D, heads, kernel, pooling, dtype, indices, K_out,
                            V_out, votes=None, pooled=None, workspace=None, workspace_bytes=None,
                            stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(lib.kvsel_select_varlen_lse(_ptr(Qwin), _ptr(K), _ptr(V), _ptr(row_lse), _i32_array(cu_L),
                                       _i32_array(C), len(C), W, D, heads, kernel, POOL.get(pooling, pooling),
                                       DTYPE.get(dtype, dtype), _ptr(indices), _ptr(K_out), _ptr(V_out),
                                       _ptr(votes), _ptr(pooled), _ptr(workspace), ws_bytes, _stream(stream)))


def kvsel_gqa_workspace_bytes(q_heads: int, kv_heads: int, L: int, W: int, C: int, D: int, dtype) -> int:
    n = lib.kvsel_gqa_workspace_bytes(q_heads, kv_heads, L, W, C, D, DTYPE.get(dtype, dtype))
    if n == 0:
        raise KvselError(KVSEL_EINVAL, kvsel_last_error())
    return n


def kvsel_select_gqa(Qwin, K, V, row_lse, L, W, C, D, q_heads, kv_heads, kernel, pooling, dtype, indices, K_out,
                     V_out, row_stats=None, votes=None, pooled=None, workspace=None, workspace_bytes=None,
                     stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(lib.kvsel_select_gqa(_ptr(Qwin), _ptr(K), _ptr(V), _ptr(row_lse), L, W, C, D, q_heads, kv_heads, kernel,
                                POOL.get(pooling, pooling), DTYPE.get(dtype, dtype), _ptr(indices), _ptr(K_out),
                                _ptr(V_out), _ptr(row_stats), _ptr(votes), _ptr(pooled), _ptr(workspace), ws_bytes,
                                _stream(stream)))


def kvsel_topk_workspace_bytes(rows: int, n: int) -> int:
    v = lib.kvsel_topk_workspace_bytes(rows, n)
    if v == 0:
        raise KvselError(KVSEL_EINVAL, kvsel_last_error())
    return v


def kvsel_topk(scores, rows, n, count, out, ld_out, workspace=None, workspace_bytes=None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.kvsel_topk(_ptr(scores), rows, n, count, _ptr(out), ld_out, _ptr(workspace), workspace_bytes,
                          _stream(stream)))


def kvsel_refresh_workspace_bytes(rows: int, n: int) -> int:
    v = lib.kvsel_refresh_workspace_bytes(rows, n)
    if v == 0:
        raise KvselError(KVSEL_EINVAL, kvsel_last_error())
    return v


def kvsel_refresh(scores, rows, n, keep, protect_head, protect_tail, K, V, D, dtype, tokens, indices, K_out, V_out,
                  tokens_out, workspace, workspace_bytes=None, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(lib.kvsel_refresh(_ptr(scores), rows, n, keep, protect_head, protect_tail, _ptr(K), _ptr(V), D,
                             DTYPE.get(dtype, dtype), _ptr(tokens), _ptr(indices), _ptr(K_out), _ptr(V_out),
                             _ptr(tokens_out), _ptr(workspace), ws_bytes, _stream(stream)))


def kvsel_jacap_workspace_bytes(heads: int, N: int, D: int) -> int:
    v = lib.kvsel_jacap_workspace_bytes(heads, N, D)
    if v == 0:
        raise KvselError(KVSEL_EINVAL, kvsel_last_error())
    return v


def kvsel_jacap_select(K, V, U, mu_q, lambda_q, tau, heads, N, D, dtype, keep, protect_head, protect_tail, tokens,
                       indices, K_out, V_out, tokens_out, scores, workspace, workspace_bytes=None,
                       stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(lib.kvsel_jacap_select(_ptr(K), _ptr(V), _ptr(U), _ptr(mu_q), _ptr(lambda_q), float(tau), heads, N, D,
                                  DTYPE.get(dtype, dtype), keep, protect_head, protect_tail, _ptr(tokens),
                                  _ptr(indices), _ptr(K_out), _ptr(V_out), _ptr(tokens_out), _ptr(scores),
                                  _ptr(workspace), ws_bytes, _stream(stream)))


def kvsel_pool1d(votes, rows, n, kernel, pooling, pooled, stream=None) -> None:
    _check(lib.kvsel_pool1d(_ptr(votes), rows, n, kernel, POOL.get(pooling, pooling), _ptr(pooled),
                            _stream(stream)))


def kvsel_gather(K, V, indices, ld_idx, heads, L, count, D, dtype, K_out, V_out, stream=None) -> None:
    _check(lib.kvsel_gather(_ptr(K), _ptr(V), _ptr(indices), ld_idx, heads, L, count, D,
                            DTYPE.get(dtype, dtype), _ptr(K_out), _ptr(V_out), _stream(stream)))


# ------------------------------------------------------------ conveniences

def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def select(Qwin: torch.Tensor, K: torch.Tensor, V: torch.Tensor, C: int, kernel: int = 5,
           pooling: str = "avg", with_scores: bool = False, workspace: Optional[torch.Tensor] = None,
           stream=None):
    """Allocate outputs and run kvsel_select on Qwin [H, W, D], K, V [H, L, D].
    Returns (indices [H, C], K_out [H, C, D], V_out [H, C, D]) plus
    (row_stats [H, W, 2], votes [H, P], pooled [H, P]) if with_scores."""
    H, L, D = K.shape
    W = Qwin.shape[1]
    dev = K.device
    ws = workspace if workspace is not None else _workspace(kvsel_workspace_bytes(H, L, W, C, D, K.dtype), dev)
    idx = torch.empty((H, C), dtype=torch.int32, device=dev)
    Ko = torch.empty((H, C, D), dtype=K.dtype, device=dev)
    Vo = torch.empty((H, C, D), dtype=V.dtype, device=dev)
    rs = vt = pl = None
    if with_scores:
        rs = torch.empty((H, W, 2), dtype=torch.float32, device=dev)
        vt = torch.empty((H, max(L - W, 0)), dtype=torch.float32, device=dev)
        pl = torch.empty((H, max(L - W, 0)), dtype=torch.float32, device=dev)
    kvsel_select(Qwin, K, V, L, W, C, D, H, kernel, pooling, K.dtype, idx, Ko, Vo, rs, vt, pl, ws,
                 stream=stream)
    return (idx, Ko, Vo, rs, vt, pl) if with_scores else (idx, Ko, Vo)


class _KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int), ("total_ms", ctypes.c_double)]


lib.kvsel_profile_enable.restype = _i
lib.kvsel_profile_enable.argtypes = [_i]
lib.kvsel_profile_read.restype = _i
lib.kvsel_profile_read.argtypes = [ctypes.POINTER(_KernelTime), _i]


def kvsel_profile_enable(on: bool) -> None:
    _check(lib.kvsel_profile_enable(1 if on else 0))


def kvsel_profile_read() -> dict:
    """{kernel name: (launches, total milliseconds)} since profiling was enabled."""
    buf = (_KernelTime * 64)()
    n = lib.kvsel_profile_read(buf, 64)
    if n < 0:
        raise KvselError(n, kvsel_last_error())
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(min(n, 64))}


KVSEL_OPT_SCORING = 0
KVSEL_OPT_FORCE_FALLBACK = 1
KVSEL_OPT_VALIDATE = 2
KVSEL_OPT_FUSED_SELECT = 3
KVSEL_OPT_SELECT = 4
KVSEL_SELECT_AUTO, KVSEL_SELECT_SPLIT, KVSEL_SELECT_EXCHANGE = 0, 1, 2
SCORING = {"auto": 0, "two_pass": 1, "single_read": 2}
lib.kvsel_set_option.restype = _i
lib.kvsel_set_option.argtypes = [_i, _i]
lib.kvsel_get_option.restype = _i
lib.kvsel_get_option.argtypes = [_i]


def kvsel_set_option(option: int, value: int) -> None:
    _check(lib.kvsel_set_option(option, value))


def kvsel_get_option(option: int) -> int:
    v = lib.kvsel_get_option(option)
    if v < 0:
        raise KvselError(v, kvsel_last_error())
    return v


def kvsel_debug_flags(reset: bool = False, library=None) -> int:
    """The library-wide index-check word of a KVSEL_DEBUG build (then cleared
    if reset); KVSEL_EUNSUPPORTED from a release build."""
    return (library or lib).kvsel_debug_flags(1 if reset else 0)


def debug_library():
    """libkvsel_debug.so with the same C declarations as the release library,
    for checks of the debug build's index flags (a separate handle: its calls
    take raw pointers, as lib's do)."""
    if not os.path.exists(DEBUG_LIB_PATH):
        raise ImportError(f"{DEBUG_LIB_PATH} is missing: build it with `python -m prompt_kv_selection_amd.build`")
    dl = ctypes.CDLL(DEBUG_LIB_PATH)
    for name, f in list(lib.__dict__.items()):
        if name.startswith("kvsel_") and hasattr(f, "argtypes"):
            g = getattr(dl, name)
            g.restype, g.argtypes = f.restype, f.argtypes
    return dl
