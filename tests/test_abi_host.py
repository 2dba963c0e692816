"""Host-side checks of the C ABI, no GPU needed: the library loads, exports
every function include/kvsel.h declares, sizes workspaces, and rejects invalid
arguments before anything is enqueued (no kernel is launched here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvsel.h")


@pytest.fixture(scope="module")
def B():
    from prompt_kv_selection_amd import binding
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvsel_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(B):
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(B.lib, name), name
    out = os.popen(f"nm -D --defined-only {B.LIB_PATH}").read()
    for name in names:
        assert re.search(rf"\bT {name}\b", out), name


def test_version_and_error_string(B):
    assert B.kvsel_version() >= 1
    assert isinstance(B.kvsel_last_error(), str)


def test_workspace_sizes(B):
    n = B.lib.kvsel_workspace_bytes(32, 32768, 32, 1024, 128, 1)
    # header (error flags), two-pass partial (max, sum) per (head, chunk, row), votes, pooled,
    # selection threshold and per-segment counts, single-read exchange slots
    # (per head and 512-position chunk), first-digit histograms, the
    # cooperative selection's status words (one block for each of up to 8
    # launches) and per-row words (histograms,
    # segment counts, candidate entries); then the fused selection's words:
    # a count word and 8 halo words per exchange slot, the arrival tokens,
    # decision and claim counters, per exchange slot 64 + 32 histogram words,
    # per row two completion counters, 8-byte candidates laid out like the
    # votes, and per exchange slot the chunk's 512 pooled scores
    expect_min = (256 + 2 * 32 * 32 * 32 * 4 + 2 * 32 * (32768 - 32) * 4 + 32 * 8 + 32 * 2 * 512 * 4
                  + 32 * 64 * 256 + 32 * 2048 * 4 + 8 * 17 * 256 + 32 * (5120 + 128 + 8192) * 4
                  + 32 * 64 * 8 + 32 * 64 * 8 * 8 + (1024 + 8) * 8 + 32 * 64 * (64 + 32) * 4 + 32 * 2 * 8
                  + 32 * (32768 - 32) * 8 + 32 * 64 * 512 * 4)
    assert expect_min <= n <= expect_min + 13 * 256
    assert n % 256 == 0
    assert B.lib.kvsel_workspace_bytes(32, 100, 32, 32, 128, 1) == 0  # C <= W
    assert "budget" in B.kvsel_last_error()
    cu = (ctypes.c_int32 * 3)(0, 5000, 12000)
    cs = (ctypes.c_int32 * 2)(500, 1200)
    assert B.lib.kvsel_varlen_workspace_bytes(cu, cs, 2, 8, 32, 128, 1) > 0
    # bypassed sequences need no partial stats, still own their vote slots
    cs2 = (ctypes.c_int32 * 2)(6000, 1200)
    assert B.lib.kvsel_varlen_workspace_bytes(cu, cs2, 2, 8, 32, 128, 1) < \
        B.lib.kvsel_varlen_workspace_bytes(cu, cs, 2, 8, 32, 128, 1)


FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every case below fails validation


def call_select(B, **kw):
    args = dict(Q=FAKE, K=FAKE, V=FAKE, L=1024, W=32, C=256, D=128, heads=4, kernel=5, pooling=0, dtype=1,
                idx=FAKE, Ko=FAKE, Vo=FAKE, ws=FAKE, wsb=1 << 30)
    args.update(kw)
    return B.lib.kvsel_select(args["Q"], args["K"], args["V"], args["L"], args["W"], args["C"], args["D"],
                              args["heads"], args["kernel"], args["pooling"], args["dtype"], args["idx"],
                              args["Ko"], args["Vo"], None, None, None, args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(W=0), -1), (dict(W=1025), -1), (dict(C=32), -1), (dict(C=10), -1),
    (dict(kernel=4), -1), (dict(kernel=0), -1), (dict(kernel=-3), -1), (dict(pooling=2), -1),
    (dict(dtype=7), -1), (dict(heads=0), -1), (dict(L=0), -1), (dict(D=0), -1),
    (dict(D=96), -2), (dict(W=129, L=4096, C=512), -2), (dict(kernel=65), -2),
    (dict(Q=None), -1), (dict(K=None), -1), (dict(Vo=None), -1), (dict(idx=None), -1),
    (dict(ws=None), -1), (dict(wsb=1024), -3), (dict(ws=ctypes.c_void_p(0x10010)), -1),
    (dict(K=ctypes.c_void_p(0x10008)), -1),
])
def test_select_argument_errors(B, kw, code):
    assert call_select(B, **kw) == code
    assert B.kvsel_last_error() != ""


def test_lse_argument_errors(B):
    lib = B.lib
    args = [FAKE, FAKE, FAKE]
    tail = [1024, 32, 256, 128, 4, 5, 0, 1, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 30, None]
    assert lib.kvsel_select_lse(*args, None, *tail) == -1 and "row_lse" in B.kvsel_last_error()
    assert lib.kvsel_select_lse(*args, ctypes.c_void_p(0x10002), *tail) == -1
    bad = list(tail)
    bad[2] = 32  # C == W
    assert lib.kvsel_select_lse(*args, FAKE, *bad) == -1
    bad = list(tail)
    bad[-2] = 1024  # workspace too small
    assert lib.kvsel_select_lse(*args, FAKE, *bad) == -3
    cu = (ctypes.c_int32 * 3)(0, 5000, 4000)
    cs = (ctypes.c_int32 * 2)(500, 400)
    rc = lib.kvsel_select_varlen_lse(FAKE, FAKE, FAKE, FAKE, cu, cs, 2, 32, 128, 8, 5, 0, 1, FAKE, FAKE, FAKE,
                                     None, None, FAKE, 1 << 30, None)
    assert rc == -1 and "sequence 1" in B.kvsel_last_error()


def test_gqa_argument_errors(B):
    lib = B.lib
    def gqa(q_heads=8, kv_heads=2, W=32, lse=None, rs=None, wsb=1 << 30):
        return lib.kvsel_select_gqa(FAKE, FAKE, FAKE, lse, 4096, W, 512, 128, q_heads, kv_heads, 5, 0, 1, FAKE, FAKE,
                                    FAKE, rs, None, None, FAKE, wsb, None)
    assert gqa(kv_heads=0) == -1
    assert gqa(kv_heads=3) == -1 and "multiple" in B.kvsel_last_error()
    assert gqa(W=48) == -2                     # grouped heads need W a multiple of 32
    assert gqa(q_heads=10, kv_heads=2) == -2   # group 5: 5 * 32 rows > 128
    assert gqa(lse=FAKE, rs=FAKE) == -1
    assert gqa(wsb=1024) == -3
    assert lib.kvsel_gqa_workspace_bytes(8, 0, 4096, 32, 512, 128, 1) == 0
    # grouped heads score on the two-pass path: no single-read exchange slots
    assert 0 < lib.kvsel_gqa_workspace_bytes(8, 2, 4096, 32, 512, 128, 1) < lib.kvsel_workspace_bytes(8, 4096, 32, 512, 128, 1)
    assert lib.kvsel_gqa_workspace_bytes(8, 8, 4096, 32, 512, 128, 1) == lib.kvsel_workspace_bytes(8, 4096, 32, 512, 128, 1)


def test_varlen_argument_errors(B):
    lib = B.lib
    cu_bad = (ctypes.c_int32 * 3)(0, 5000, 4000)  # negative length
    cs = (ctypes.c_int32 * 2)(500, 400)
    rc = lib.kvsel_select_varlen(FAKE, FAKE, FAKE, cu_bad, cs, 2, 32, 128, 8, 5, 0, 1, FAKE, FAKE, FAKE,
                                 None, None, None, FAKE, 1 << 30, None)
    assert rc == -1 and "sequence 1" in B.kvsel_last_error()
    cu = (ctypes.c_int32 * 3)(1, 5000, 9000)
    rc = lib.kvsel_select_varlen(FAKE, FAKE, FAKE, cu, cs, 2, 32, 128, 8, 5, 0, 1, FAKE, FAKE, FAKE,
                                 None, None, None, FAKE, 1 << 30, None)
    assert rc == -1
    rc = lib.kvsel_select_varlen(FAKE, FAKE, FAKE, None, cs, 2, 32, 128, 8, 5, 0, 1, FAKE, FAKE, FAKE,
                                 None, None, None, FAKE, 1 << 30, None)
    assert rc == -1
    cu = (ctypes.c_int32 * 3)(0, 20, 9000)    # window longer than sequence 0
    rc = lib.kvsel_select_varlen(FAKE, FAKE, FAKE, cu, cs, 2, 32, 128, 8, 5, 0, 1, FAKE, FAKE, FAKE,
                                 None, None, None, FAKE, 1 << 30, None)
    assert rc == -1 and "window" in B.kvsel_last_error()


def test_step_entry_point_errors(B):
    lib = B.lib
    assert lib.kvsel_topk(FAKE, 4, 100, 0, FAKE, 10, None, 0, None) == -1
    assert lib.kvsel_topk(FAKE, 4, 100, 101, FAKE, 200, None, 0, None) == -1
    assert lib.kvsel_topk(FAKE, 4, 100, 10, FAKE, 9, None, 0, None) == -1
    assert lib.kvsel_topk(None, 4, 100, 10, FAKE, 10, None, 0, None) == -1
    assert lib.kvsel_topk(FAKE, 4, 100, 10, FAKE, 10, None, 0, None) == -1          # no workspace
    assert lib.kvsel_topk(FAKE, 4, 100, 10, FAKE, 10, FAKE, 1024, None) == -3       # too small
    # histograms, cut, segment counts, candidate scores (one word per score)
    assert lib.kvsel_topk_workspace_bytes(4, 100) == 4 * 2048 * 4 + 256 + 4 * 2 * 512 * 4 + 1792
    assert lib.kvsel_topk_workspace_bytes(0, 100) == 0
    assert lib.kvsel_pool1d(FAKE, 4, 100, 2, 0, ctypes.c_void_p(0x20000), None) == -1
    assert lib.kvsel_pool1d(FAKE, 4, 100, 3, 0, FAKE, None) == -1  # aliasing
    assert lib.kvsel_pool1d(FAKE, 4, 100, 3, 5, ctypes.c_void_p(0x20000), None) == -1
    assert lib.kvsel_gather(FAKE, FAKE, FAKE, 10, 4, 100, 20, 128, 1, FAKE, FAKE, None) == -1  # ld < count
    assert lib.kvsel_gather(FAKE, FAKE, FAKE, 20, 4, 100, 20, 80, 1, FAKE, FAKE, None) == -2
    assert lib.kvsel_gather(FAKE, FAKE, FAKE, 20, 4, 100, 20, 128, 3, FAKE, FAKE, None) == -1


def test_status_entry_point_errors(B):
    assert B.lib.kvsel_status(None, None) == -1
    assert B.lib.kvsel_status(ctypes.c_void_p(0x10010), None) == -1 and "aligned" in B.kvsel_last_error()
    assert B.KVSEL_ENONFINITE == -5


def test_refresh_argument_errors(B):
    lib = B.lib
    def refresh(n=100, keep=10, head=2, tail=2, D=128, tok=None, tok_out=None, wsb=1 << 30):
        return lib.kvsel_refresh(FAKE, 2, n, keep, head, tail, FAKE, FAKE, D, 1, tok, FAKE, FAKE, FAKE, tok_out,
                                 FAKE, wsb, None)
    assert refresh(keep=0) == -1
    assert refresh(keep=101) == -1
    assert refresh(head=6, tail=5) == -1 and "fit" in B.kvsel_last_error()
    assert refresh(head=-1) == -1
    assert refresh(tok=FAKE) == -1                 # tokens without tokens_out
    assert refresh(D=96) == -2
    assert refresh(wsb=1024) == -3
    assert lib.kvsel_refresh_workspace_bytes(2, 100) == lib.kvsel_topk_workspace_bytes(2, 100)


def test_jacap_argument_errors(B):
    lib = B.lib
    mu = (ctypes.c_float * 128)()

    def jacap(N=100, D=128, dtype=1, keep=10, head=2, tail=2, tau=10.0, tok=None, tok_out=None, wsb=1 << 30,
              U=FAKE, lam=None):
        lam = ctypes.addressof(mu) if lam is None else lam
        return lib.kvsel_jacap_select(FAKE, FAKE, U, ctypes.addressof(mu), lam, tau, 2, N, D, dtype, keep, head,
                                      tail, tok, FAKE, FAKE, FAKE, tok_out, None, FAKE, wsb, None)
    assert jacap(keep=0) == -1
    assert jacap(keep=101) == -1
    assert jacap(head=6, tail=5) == -1 and "fit" in B.kvsel_last_error()
    assert jacap(tau=0.0) == -1 and "temperature" in B.kvsel_last_error()
    assert jacap(tau=float("nan")) == -1
    assert jacap(U=None) == -1
    assert jacap(lam=0) == -1
    assert jacap(tok=FAKE) == -1
    assert jacap(dtype=0) == -2 and "bf16" in B.kvsel_last_error()   # f32 keys are not supported here
    assert jacap(D=96) == -2
    assert jacap(wsb=1024) == -3
    assert lib.kvsel_jacap_workspace_bytes(2, 100, 96) == 0
    a = lib.kvsel_jacap_workspace_bytes(2, 100, 128)
    b = lib.kvsel_jacap_workspace_bytes(2, 5000, 128)
    assert a % 256 == 0 and b > a


def test_options(B):
    lib = B.lib
    assert lib.kvsel_get_option(2) == 0                       # validating mode off
    assert lib.kvsel_set_option(2, 3) == -1
    assert lib.kvsel_set_option(2, 1) == 0 and lib.kvsel_get_option(2) == 1
    assert lib.kvsel_set_option(2, 0) == 0 and lib.kvsel_get_option(2) == 0
    assert lib.kvsel_get_option(0) == 0
    assert lib.kvsel_set_option(0, 3) == -1
    assert lib.kvsel_get_option(1) == 0                       # forced fallback off
    assert lib.kvsel_set_option(1, 2) == -1
    assert lib.kvsel_set_option(1, 1) == 0 and lib.kvsel_get_option(1) == 1
    assert lib.kvsel_set_option(1, 0) == 0 and lib.kvsel_get_option(1) == 0
    assert lib.kvsel_get_option(4) == 0                       # selection kernels: automatic
    assert lib.kvsel_set_option(4, 3) == -1
    assert lib.kvsel_set_option(4, 1) == 0 and lib.kvsel_get_option(4) == 1
    assert lib.kvsel_set_option(4, 2) == 0 and lib.kvsel_get_option(4) == 2
    assert lib.kvsel_set_option(4, 0) == 0 and lib.kvsel_get_option(4) == 0
    assert lib.kvsel_set_option(5, 0) == -1
    assert lib.kvsel_get_option(5) == -1
    assert lib.kvsel_get_option(3) == 0                       # fused selection off
    assert lib.kvsel_set_option(3, 2) == -1
    assert lib.kvsel_set_option(3, 1) == 0 and lib.kvsel_get_option(3) == 1
    assert lib.kvsel_set_option(3, 0) == 0 and lib.kvsel_get_option(3) == 0
    assert lib.kvsel_set_option(0, 1) == 0 and lib.kvsel_get_option(0) == 1
    assert lib.kvsel_set_option(0, 0) == 0 and lib.kvsel_get_option(0) == 0


# ---------------------------------------------------------------- host sanitizers

def _sanitized_plan_check():
    """Build tests/host_check/plan_check.cpp against the library sources with
    AddressSanitizer and UndefinedBehaviorSanitizer on the host code (the
    device code is compiled as usual and never launched), once per source
    digest, into tests/host_check/_build."""
    import hashlib
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc is not installed")
    here = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(here)
    csrc = os.path.join(root, "prompt_kv_selection_amd", "csrc")
    srcs = [os.path.join(csrc, f"kvsel_{s}.hip") for s in ("api", "score", "select", "fused", "jacap", "probe")]
    deps = srcs + [os.path.join(here, "host_check", "plan_check.cpp"), os.path.join(root, "include", "kvsel.h")]
    deps += [os.path.join(csrc, f) for f in sorted(os.listdir(csrc)) if f.endswith(".h")]
    digest = hashlib.sha256(b"".join(open(p, "rb").read() for p in deps)).hexdigest()[:16]
    build = os.path.join(here, "host_check", "_build")
    exe = os.path.join(build, f"plan_check_{digest}")
    if os.path.exists(exe):
        return exe
    os.makedirs(build, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Wno-unused-function",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + os.path.join(root, "include"), "-I" + csrc] + san
    objs, procs = [], []
    for src in srcs + [os.path.join(here, "host_check", "plan_check.cpp")]:
        obj = os.path.join(build, os.path.basename(src) + f".{digest}.o")
        objs.append(obj)
        procs.append(subprocess.Popen([hipcc] + flags + ["-c", src, "-o", obj], stdout=subprocess.PIPE,
                                      stderr=subprocess.STDOUT))
    for p in procs:
        out = p.communicate()[0].decode(errors="replace")
        assert p.returncode == 0, out[-3000:]
    r = subprocess.run([hipcc, "--offload-arch=gfx950"] + san + ["-o", exe] + objs, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    for o in objs:
        os.remove(o)
    return exe


def test_validation_and_planning_under_sanitizers():
    """Argument validation and workspace planning of every entry point run
    clean under ASan and UBSan: no out-of-bounds host access (the cu_L and C
    arrays are exactly sized heap blocks), no signed overflow or other
    undefined behaviour, and the expected return codes.  No call reaches the
    device (invalid arguments, or a workspace one byte short)."""
    import subprocess
    exe = _sanitized_plan_check()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=99",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=98")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "plan_check: 0 unexpected" in out
