"""The C-ABI library loads, exports every entry point of include/qlora.h, and
rejects bad arguments with the documented status before touching the GPU.

These run on a host without a GPU: argument validation lives in a HIP-free
translation unit and happens before any HIP call.
"""
import ctypes
import os
import re

import pytest

import qlora_fine_tuning_linear_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "qlora.h")

OK, INVALID, SHAPE, MISALIGNED, WS_SMALL, DEVICE, HIP = 0, -1, -2, -3, -4, -5, -6


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(q.LIB_PATH):
        pytest.skip("libqlora.so not built")
    return q.load_library()


def header_functions():
    src = open(HDR).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s+([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported(lib):
    declared = header_functions()
    assert set(declared) == set(q.EXPORTED), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_and_strerror(lib):
    assert lib.qlora_abi_version() == 1
    for st in (OK, INVALID, SHAPE, MISALIGNED, WS_SMALL, DEVICE, HIP, 12345):
        assert isinstance(lib.qlora_strerror(st), bytes) and lib.qlora_strerror(st)


FAKE = 0x10000  # a 16-byte-aligned address that validation never dereferences


def nf4(N=128, K=128, dq=0, codes=FAKE, cb=FAKE, absmax=FAKE, blocksize=64):
    c = q.CNf4()
    c.codes, c.codebook, c.N, c.K, c.blocksize, c.dq_group = codes, cb, N, K, blocksize, dq
    if dq:
        c.absmax_q, c.absmax_scale = FAKE, FAKE
    else:
        c.absmax = absmax
    return c


def linear(N=128, K=128, r=8, alpha=16.0, **kw):
    L = q.CLinear()
    L.W0 = nf4(N, K, **kw)
    L.A, L.B, L.r, L.alpha = FAKE, FAKE, r, alpha
    return L


def fwd(lib, L, X=FAKE, M=16, Y=FAKE, XA=FAKE, ws=FAKE, wsb=1 << 30):
    return lib.qlora_linear_fwd(ctypes.byref(L), X, M, Y, XA, ws, wsb, None)


def test_linear_fwd_rejections(lib):
    assert fwd(lib, linear(), X=None) == INVALID
    assert fwd(lib, linear(), M=-1) == INVALID
    assert fwd(lib, linear(alpha=float("nan"))) == INVALID
    assert fwd(lib, linear(alpha=float("inf"))) == INVALID
    assert fwd(lib, linear(K=96)) == SHAPE
    assert fwd(lib, linear(N=100)) == SHAPE
    assert fwd(lib, linear(N=1 << 22)) == SHAPE      # a 256-row bf16 tile must stay below 2 GiB
    assert fwd(lib, linear(K=1 << 22)) == SHAPE
    assert fwd(lib, linear(r=0)) == SHAPE
    assert fwd(lib, linear(r=129)) == SHAPE
    assert fwd(lib, linear(blocksize=32)) == SHAPE
    assert fwd(lib, linear(dq=128)) == SHAPE
    assert fwd(lib, linear(codes=None)) == INVALID
    assert fwd(lib, linear(absmax=None)) == INVALID
    assert fwd(lib, linear(), X=FAKE + 2) == MISALIGNED
    assert fwd(lib, linear(codes=FAKE + 8)) == MISALIGNED
    assert fwd(lib, linear(), XA=FAKE + 4) == MISALIGNED
    assert lib.qlora_linear_fwd(None, FAKE, 16, FAKE, FAKE, FAKE, 1 << 30, None) == INVALID


def test_linear_fwd_static_rejections(lib):
    """The allocation-free forward validates like qlora_linear_fwd and refuses
    a pass whose scratch exceeds the library's static array, before touching
    the device."""
    call = lambda L, M=16, X=FAKE, Y=FAKE, XA=FAKE: lib.qlora_linear_fwd_static(ctypes.byref(L), X, M, Y, XA, None)
    assert call(linear(), X=None) == INVALID
    assert call(linear(), Y=FAKE + 8) == MISALIGNED
    assert call(linear(r=0)) == SHAPE
    assert call(linear(), M=-1) == INVALID
    assert call(linear(), M=0) == OK
    # 4096 tokens of an 8192 x 8192 layer: a 128 MiB bf16 weight copy
    assert call(linear(N=8192, K=8192, r=16), M=4096) == WS_SMALL
    assert lib.qlora_linear_workspace_bytes(ctypes.byref(linear(N=8192, K=8192, r=16)), 4096) > q.QLORA_STATIC_SCRATCH_BYTES
    # small enough: validation passes and the call stops at the device check
    assert call(linear(N=2048, K=1024, r=16), M=40) in (HIP, DEVICE)


def test_debug_force_arch_argument(lib):
    assert lib.qlora_debug_force_arch(b"x" * 64) == INVALID
    assert lib.qlora_debug_force_arch(None) == OK


def test_linear_workspace_rule(lib):
    L = linear(N=28672, K=8192, r=16, dq=256)   # skinny M splits the reduction -> needs workspace
    need = lib.qlora_linear_workspace_bytes(ctypes.byref(L), 64)
    assert need > 0
    assert fwd(lib, L, M=64, wsb=16) == WS_SMALL
    assert fwd(lib, L, M=64, ws=None, wsb=need) == INVALID
    assert fwd(lib, L, M=64, ws=FAKE + 4, wsb=need) == MISALIGNED
    bwd = lambda wsb: lib.qlora_linear_bwd(ctypes.byref(L), FAKE, FAKE, FAKE, 64, FAKE, FAKE, FAKE, FAKE, wsb,
                                           None)
    assert bwd(need - 1) == WS_SMALL  # the query returns what the larger (backward) pass needs


def test_m_zero_forward_is_a_noop(lib):
    # M == 0 returns OK before any device work, even without a GPU
    assert fwd(lib, linear(), M=0, X=None, Y=None, XA=None, ws=None, wsb=0) == OK


def test_linear_bwd_rejections(lib):
    L = linear()
    call = lambda **k: lib.qlora_linear_bwd(ctypes.byref(L), k.get("dY", FAKE), k.get("X", FAKE),
                                            k.get("XA", FAKE), k.get("M", 16), k.get("dX", FAKE),
                                            k.get("dA", FAKE), k.get("dB", FAKE), FAKE, 1 << 30, None)
    assert call(dA=None) == INVALID
    assert call(dB=FAKE + 2) == MISALIGNED
    assert call(dY=None) == INVALID
    assert call(M=-3) == INVALID


def test_quantize_rejections(lib):
    f = lambda **k: lib.nf4_quantize(k.get("W", FAKE), k.get("N", 64), k.get("K", 64), k.get("cb", FAKE),
                                     k.get("bs", 64), k.get("dq", 0), k.get("codes", FAKE),
                                     k.get("absmax", FAKE), k.get("aq", None), k.get("sc", None), None)
    assert f(K=100) == SHAPE
    assert f(bs=128) == SHAPE
    assert f(dq=3) == SHAPE
    assert f(N=-1) == INVALID
    assert f(W=None) == INVALID
    assert f(absmax=None) == INVALID
    assert f(dq=256) == INVALID  # DQ outputs missing
    assert f(codes=FAKE + 1) == MISALIGNED
    assert f(N=0) == OK          # empty weight: nothing to do


def test_dequantize_rejections(lib):
    w = nf4()
    assert lib.nf4_dequantize(ctypes.byref(w), 7, FAKE, None) == INVALID
    assert lib.nf4_dequantize(ctypes.byref(w), 0, None, None) == INVALID
    assert lib.nf4_dequantize(None, 0, FAKE, None) == INVALID


def test_mlp_shape_rules(lib):
    P = q.CMlp(linear(N=256, K=128), linear(N=256, K=128), linear(N=128, K=256))
    S = q.CMlpSaved(FAKE, FAKE, FAKE, FAKE, FAKE)
    call = lambda P: lib.qlora_mlp_fwd(ctypes.byref(P), FAKE, 16, FAKE, ctypes.byref(S), FAKE, 1 << 40, None)
    bad = q.CMlp(linear(N=256, K=128), linear(N=192, K=128), linear(N=128, K=256))
    assert call(bad) == SHAPE
    bad2 = q.CMlp(linear(N=256, K=128), linear(N=256, K=128), linear(N=256, K=256))
    assert call(bad2) == SHAPE
    assert lib.qlora_mlp_fwd(ctypes.byref(P), FAKE, 16, FAKE, None, FAKE, 1 << 40, None) == INVALID
    need = lib.qlora_mlp_workspace_bytes(ctypes.byref(P), 16)
    assert need >= 16 * 256 * 2          # at least the transient H
    assert lib.qlora_mlp_fwd(ctypes.byref(P), FAKE, 16, FAKE, ctypes.byref(S), FAKE, 16 * 256 * 2 - 1,
                             None) == WS_SMALL
    # a well-formed call on a host without a GPU fails at the device check, cleanly
    assert lib.qlora_mlp_fwd(ctypes.byref(P), FAKE, 16, FAKE, ctypes.byref(S), FAKE, need, None) in (HIP, DEVICE)


def test_mlp_rmsnorm_rules(lib):
    """qlora_mlp_fwd_rmsnorm: the MLP forward's rules plus those of rmsnorm_fwd
    (eps finite and >= 0, norm weight and rstd given); Xn is optional."""
    P = q.CMlp(linear(N=256, K=128), linear(N=256, K=128), linear(N=128, K=256))
    S = q.CMlpSaved(FAKE, FAKE, FAKE, FAKE, FAKE)
    need = lib.qlora_mlp_rmsnorm_workspace_bytes(ctypes.byref(P), 16)
    assert need > 16 * 256 * 2  # at least the transient H
    assert lib.qlora_mlp_rmsnorm_workspace_bytes(ctypes.byref(P), 0) == 0

    def call(M=16, X=FAKE, w=FAKE, eps=1e-5, rstd=FAKE, Xn=None, wsb=None, saved=True):
        return lib.qlora_mlp_fwd_rmsnorm(ctypes.byref(P), X, w, eps, M, FAKE, ctypes.byref(S) if saved else None,
                                         rstd, Xn, FAKE, need if wsb is None else wsb, None)

    assert call(eps=-1.0) == INVALID
    assert call(eps=float("nan")) == INVALID
    assert call(w=None) == INVALID
    assert call(rstd=None) == INVALID
    assert call(X=None) == INVALID
    assert call(saved=False) == INVALID
    assert call(Xn=FAKE + 2) == MISALIGNED
    assert call(wsb=need - 1) == WS_SMALL
    assert call(M=0, X=None, rstd=None) == OK
    # well-formed, with and without Xn: fails at the device check on a host without a GPU
    assert call() in (HIP, DEVICE)
    assert call(Xn=FAKE) in (HIP, DEVICE)
    bad = q.CMlp(linear(N=256, K=8200), linear(N=256, K=8200), linear(N=8200, K=256))
    assert lib.qlora_mlp_rmsnorm_workspace_bytes(ctypes.byref(bad), 16) == 0


def test_mlp_intermediate_bound(lib):
    """The backward's [W_g^T | W_u^T] bf16 copy has row stride 2I; a 256-row
    tile of it must stay below 2 GiB, so I is capped at 2097088."""
    S = q.CMlpSaved(FAKE, FAKE, FAKE, FAKE, FAKE)

    def call(I):
        P = q.CMlp(linear(N=I, K=64), linear(N=I, K=64), linear(N=64, K=I))
        return lib.qlora_mlp_fwd(ctypes.byref(P), FAKE, 16, FAKE, ctypes.byref(S), FAKE, 1 << 50, None)

    assert call(2097088 + 64) == SHAPE
    assert call(2097088) in (HIP, DEVICE)


def test_mlp_accepts_combined_rank_above_128(lib):
    """r_g = r_u = 128 is valid (each layer's rank is at most 128; the forward
    then projects X onto A_g and A_u in two passes)."""
    P = q.CMlp(linear(N=256, K=128, r=128), linear(N=256, K=128, r=128), linear(N=128, K=256, r=128))
    S = q.CMlpSaved(FAKE, FAKE, FAKE, FAKE, FAKE)
    need = lib.qlora_mlp_workspace_bytes(ctypes.byref(P), 600)
    assert need > 0
    assert lib.qlora_mlp_fwd(ctypes.byref(P), FAKE, 600, FAKE, ctypes.byref(S), FAKE, need, None) in (HIP, DEVICE)


def test_workspace_grows_with_tokens(lib):
    P = q.CMlp(linear(N=14336, K=4096, r=16), linear(N=14336, K=4096, r=16), linear(N=4096, K=14336, r=16))
    a = lib.qlora_mlp_workspace_bytes(ctypes.byref(P), 1024)
    b = lib.qlora_mlp_workspace_bytes(ctypes.byref(P), 8192)
    assert 0 < a < b
    assert lib.qlora_mlp_workspace_bytes(ctypes.byref(P), 0) == 0


def test_merge_rejections(lib):
    call = lambda L, dt=0, out=FAKE: lib.qlora_merge(ctypes.byref(L), dt, out, None)
    assert call(linear(), dt=1) == INVALID          # fp32 is not a merge output type
    assert call(linear(), dt=7) == INVALID
    assert call(linear(), out=None) == INVALID
    assert call(linear(), out=FAKE + 2) == MISALIGNED
    assert call(linear(K=96)) == SHAPE
    assert call(linear(r=0)) == SHAPE
    assert call(linear(r=129)) == SHAPE
    assert call(linear(alpha=float("nan"))) == INVALID
    assert call(linear(codes=FAKE + 8)) == MISALIGNED
    assert lib.qlora_merge(None, 0, FAKE, None) == INVALID


def test_rmsnorm_rejections(lib):
    fwd = lambda M=16, D=64, eps=1e-5, X=FAKE, w=FAKE, Y=FAKE, r=FAKE: lib.rmsnorm_fwd(X, w, M, D, eps, Y, r, None)
    assert fwd(D=4) == SHAPE
    assert fwd(D=12) == SHAPE
    assert fwd(D=8200) == SHAPE
    assert fwd(M=-1) == INVALID
    assert fwd(eps=-1.0) == INVALID
    assert fwd(eps=float("nan")) == INVALID
    assert fwd(X=None) == INVALID
    assert fwd(Y=FAKE + 2) == MISALIGNED
    assert fwd(M=0, X=None, Y=None) == OK            # empty batch: nothing to check or launch
    assert lib.rmsnorm_bwd_workspace_bytes(16, 64) == 4 * 64 * 4
    assert lib.rmsnorm_bwd_workspace_bytes(10 ** 6, 64) == 256 * 64 * 4
    assert lib.rmsnorm_bwd_workspace_bytes(16, 12) == 0
    bwd = lambda M=16, D=64, dw=FAKE, ws=FAKE, wsb=1 << 20, dX=FAKE: lib.rmsnorm_bwd(
        FAKE, FAKE, FAKE, FAKE, M, D, dX, dw, ws, wsb, None)
    assert bwd(D=12) == SHAPE
    assert bwd(dX=None) == INVALID
    assert bwd(wsb=16) == WS_SMALL
    assert bwd(ws=FAKE + 4) == MISALIGNED
    assert bwd(dw=FAKE + 4) == MISALIGNED


def test_linear_ce_rejections(lib):
    # every call below fails validation, so nothing reaches a device
    ce = lambda T=16, D=64, V=128, chunk=8, X=FAKE, W=FAKE, t=FAKE, loss=FAKE, tl=None, dX=FAKE, ws=FAKE, \
        wsb=1 << 30: lib.qlora_linear_ce(X, T, D, W, V, t, -100, chunk, loss, tl, dX, ws, wsb, None)
    assert ce(D=96) == SHAPE
    assert ce(V=100) == SHAPE
    assert ce(D=0) == INVALID
    assert ce(T=-1) == INVALID
    assert ce(chunk=0) == INVALID
    assert ce(loss=None) == INVALID
    assert ce(X=None) == INVALID
    assert ce(t=None) == INVALID
    assert ce(W=FAKE + 2) == MISALIGNED
    assert ce(dX=FAKE + 4) == MISALIGNED
    assert ce(tl=FAKE + 4) == MISALIGNED
    assert ce(wsb=16) == WS_SMALL
    assert ce(dX=None, wsb=16) == WS_SMALL
    assert ce(ws=FAKE + 4) == MISALIGNED
    assert ce(V=(1 << 22)) == SHAPE               # 256 vocabulary rows of bf16 must stay below 2 GiB
    assert ce(V=2097088 + 64) == SHAPE            # ... also as the logit gradient of row stride 2V
    # workspace: chunk of fp32 logits + per-token losses (+ the dX product's split partials; the
    # head is read as stored, never copied)
    fwd_only = lib.qlora_linear_ce_workspace_bytes(16, 64, 128, 8, 0)
    assert fwd_only == 256 + 256 + 8 * 128 * 4
    with_dx = lib.qlora_linear_ce_workspace_bytes(16, 64, 128, 8, 1)
    assert with_dx >= fwd_only
    big = lib.qlora_linear_ce_workspace_bytes(4096, 4096, 128256, 1024, 1)
    assert big < 256 + 4096 * 4 + 1024 * 128256 * 4 + 128256 * 4096 * 2 // 4  # far below one head copy
    assert lib.qlora_linear_ce_workspace_bytes(16, 96, 128, 8, 1) == 0
    assert lib.qlora_linear_ce_workspace_bytes(4096, 4096, 128256, 1024, 0) == 256 + 4096 * 4 + 1024 * 128256 * 4


def grouped(Ns=(64, 64), rs=(8, 8), N=None, K=128, G=None):
    Q = q.CGrouped()
    Q.W0 = nf4(sum(Ns) if N is None else N, K)
    Q.A = FAKE
    Q.G = len(Ns) if G is None else G
    for g, (n, r) in enumerate(zip(Ns, rs)):
        Q.B[g], Q.N[g], Q.r[g], Q.alpha[g] = FAKE, n, r, 16.0
    return Q


def test_grouped_rejections(lib):
    fwd = lambda Q, M=16: lib.qlora_grouped_fwd(ctypes.byref(Q), FAKE, M, FAKE, FAKE, FAKE, 1 << 30, None)
    assert fwd(grouped(G=0)) == SHAPE
    assert fwd(grouped(G=9)) == SHAPE
    assert fwd(grouped(N=192)) == SHAPE                     # sum of N != W0.N
    assert fwd(grouped(rs=(100, 29))) == SHAPE              # r_total > 128
    Q = grouped()
    Q.B[1] = None
    assert fwd(Q) == INVALID
    Q = grouped()
    Q.B[0] = FAKE + 2
    assert fwd(Q) == MISALIGNED
    assert fwd(grouped(), M=-1) == INVALID
    assert lib.qlora_grouped_fwd(ctypes.byref(grouped()), FAKE, 16, FAKE, FAKE, FAKE, 16, None) == WS_SMALL
    dB = (ctypes.c_void_p * 8)(FAKE, None)
    assert lib.qlora_grouped_bwd(ctypes.byref(grouped()), FAKE, FAKE, FAKE, 16, FAKE, FAKE, dB, FAKE, 1 << 30,
                                 None) == INVALID
    assert lib.qlora_grouped_workspace_bytes(ctypes.byref(grouped()), 64) > 0
    assert lib.qlora_grouped_workspace_bytes(ctypes.byref(grouped(G=0)), 64) == 0


def test_validation_under_address_and_ub_sanitizers(tmp_path):
    """qlora_validate.cpp (argument checks, workspace sizing; no HIP) built with
    -fsanitize=address,undefined and driven over null, misaligned, negative,
    zero and extreme arguments: no sanitizer report, no crash."""
    import shutil
    import subprocess
    if shutil.which("g++") is None:
        pytest.skip("no host C++ compiler")
    csrc = os.path.join(ROOT, "qlora_fine_tuning_linear_amd", "csrc")
    exe = str(tmp_path / "validate_san")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
           os.path.join(csrc, "qlora_validate.cpp"), os.path.join(ROOT, "tests", "abi_validate_driver.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "calls" in r.stdout.splitlines()[-1]


def test_down_projection_partials_fit_the_workspace_bound(tmp_path):
    """The split count of the LoRA down-projection depends on the rank (64
    tokens per workgroup at ranks 33..64), so the workspace sizing uses a bound
    over all ranks up to each site's maximum: checked on the host for token
    counts, reduction lengths and ranks 1..256."""
    import shutil
    import subprocess
    if shutil.which("g++") is None:
        pytest.skip("no host C++ compiler")
    csrc = os.path.join(ROOT, "qlora_fine_tuning_linear_amd", "csrc")
    exe = str(tmp_path / "plan_bound")
    cmd = ["g++", "-std=c++17", "-O1", "-I" + csrc, os.path.join(ROOT, "tests", "plan_bound_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr

