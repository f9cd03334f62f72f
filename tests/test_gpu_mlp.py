"""GPU parity of qlora_mlp_fwd / qlora_mlp_bwd against the fp64 oracle.

Outputs Y, the saved G, U, XA_g, XA_u, HA_d, the input gradient dX and the
six LoRA gradients must be within relative Frobenius error 1e-2.

Small blocks are compared in full.  The two Llama-shaped workloads (M=8192,
4096/14336, r=16; M=4096, 8192/28672, r=64 with double-quantized absmax) run
at full size in the launch configuration bench.py times; the oracle then
checks a sample of token rows: forward outputs row by row, and, with dY
non-zero only on the sampled rows, dX on those rows and the LoRA gradients,
which are then sums over the sampled rows alone (every other row contributes
exactly zero, because dG and dU vanish where dY does).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import qlora as oq

from gpu_util import Guarded, assert_close, bf16_dev, make_linear

pytestmark = pytest.mark.gpu

q = pytest.importorskip("qlora_fine_tuning_linear_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.load_library()


def build(cfg, seed, codebook):
    inp = synth.mlp_inputs(cfg, seed)
    g, Wg = make_linear(q, inp["Wg"], inp["Ag"], inp["Bg"], cfg.alpha, codebook, cfg.dq_group)
    u, Wu = make_linear(q, inp["Wu"], inp["Au"], inp["Bu"], cfg.alpha, codebook, cfg.dq_group)
    d, Wd = make_linear(q, inp["Wd"], inp["Ad"], inp["Bd"], cfg.alpha, codebook, cfg.dq_group)
    for k in ("Wg", "Wu", "Wd"):
        del inp[k]
    return q.QLoraMlp(g, u, d), dict(Wg=Wg, Wu=Wu, Wd=Wd), inp


def oracle_args(W, inp):
    return (W["Wg"], W["Wu"], W["Wd"], inp["Ag"], inp["Bg"], inp["Au"], inp["Bu"], inp["Ad"], inp["Bd"])


SMALL = [
    synth.MlpCfg("m300_d256_i512_r8", M=300, D=256, I=512, r=8, alpha=16.0, dq_group=0),
    synth.MlpCfg("m70_d512_i768_r16_dq", M=70, D=512, I=768, r=16, alpha=16.0, dq_group=256),
    synth.MlpCfg("m1_d128_i256_r4", M=1, D=128, I=256, r=4, alpha=8.0, dq_group=0),
    synth.MlpCfg("m513_d256_i384_r64_dq", M=513, D=256, I=384, r=64, alpha=16.0, dq_group=256),
    synth.MlpCfg("m1100_d320_i448_r16", M=1100, D=320, I=448, r=16, alpha=16.0, dq_group=0),
    synth.MlpCfg("m1537_d192_i576_r32_dq", M=1537, D=192, I=576, r=32, alpha=32.0, dq_group=256),
    # down rank 20: the dH GEMM's fused T^T H runs its second 16-rank frag
    # with four live ranks; ragged token and column tiles
    synth.MlpCfg("m777_d192_i320_r20", M=777, D=192, I=320, r=20, alpha=16.0, dq_group=0),
    # rank 128 on every layer: r_g + r_u = 256 exceeds one down-projection
    # launch, below and above the 512-token switch to the bf16-copy GEMMs
    synth.MlpCfg("m200_d256_i384_r128", M=200, D=256, I=384, r=128, alpha=16.0, dq_group=0),
    synth.MlpCfg("m600_d256_i384_r128_dq", M=600, D=256, I=384, r=128, alpha=32.0, dq_group=256),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_mlp_parity_small(cfg, codebook):
    print("case", cfg.name, flush=True)
    P, W, inp = build(cfg, 3000 + cfg.M, codebook)
    X, dY = bf16_dev(inp["X"]), bf16_dev(inp["dY"])
    g = Guarded()
    M, D, I = cfg.M, cfg.D, cfg.I
    bf, f32 = torch.bfloat16, torch.float32
    S0 = q.MlpSaved(g.empty((M, I), bf), g.empty((M, I), bf), g.empty((M, P.gate.r), f32),
                    g.empty((M, P.up.r), f32), g.empty((M, P.down.r), f32))
    Y, S = q.qlora_mlp_fwd(P, X, Y=g.empty((M, D), bf), saved=S0)
    grads0 = {k: g.empty_like(getattr(P, lay).A if k[1] == "A" else getattr(P, lay).B)
              for k, lay in (("dA_g", "gate"), ("dB_g", "gate"), ("dA_u", "up"), ("dB_u", "up"),
                             ("dA_d", "down"), ("dB_d", "down"))}
    dX, grads = q.qlora_mlp_bwd(P, dY, X, S, dX=g.empty((M, D), bf), grads=grads0)
    g.check()
    f = oq.mlp_forward(inp["X"], *oracle_args(W, inp), cfg.alpha)
    b = oq.mlp_backward(inp["dY"], inp["X"], f["G"], f["U"], *oracle_args(W, inp), cfg.alpha)
    assert_close("Y", Y, f["Y"])
    assert_close("G", S.G, f["G"])
    assert_close("U", S.U, f["U"])
    assert_close("XA_g", S.XA_g, f["XA_g"])
    assert_close("XA_u", S.XA_u, f["XA_u"])
    assert_close("HA_d", S.HA_d, f["HA_d"])
    assert_close("dX", dX, b["dX"])
    for k in ("dA_g", "dB_g", "dA_u", "dB_u", "dA_d", "dB_d"):
        assert_close(k, grads[k], b[k])


def _sample_rows(M, n, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(M, size=n, replace=False))


@pytest.mark.parametrize("idx", [2, 3], ids=["llama3_8b_mlp", "llama3_70b_mlp_dq"])
def test_mlp_parity_full_size_sampled(idx, codebook):
    cfg = synth.CONFIGS[idx]
    print("case", cfg.name, flush=True)
    P, W, inp = build(cfg, synth.seed_of(idx), codebook)
    rows = _sample_rows(cfg.M, 96, idx)
    dY_s = np.zeros_like(inp["dY"])
    dY_s[rows] = inp["dY"][rows]
    X = bf16_dev(inp["X"])
    Y, S = q.qlora_mlp_fwd(P, X)
    dX, grads = q.qlora_mlp_bwd(P, bf16_dev(dY_s), X, S)
    torch.cuda.synchronize()
    Xs, dYs = inp["X"][rows], inp["dY"][rows]
    f = oq.mlp_forward(Xs, *oracle_args(W, inp), cfg.alpha)
    b = oq.mlp_backward(dYs, Xs, f["G"], f["U"], *oracle_args(W, inp), cfg.alpha)
    idx_t = torch.as_tensor(rows, device="cuda")
    assert_close("Y", Y[idx_t], f["Y"])
    assert_close("G", S.G[idx_t], f["G"])
    assert_close("U", S.U[idx_t], f["U"])
    assert_close("XA_g", S.XA_g[idx_t], f["XA_g"])
    assert_close("XA_u", S.XA_u[idx_t], f["XA_u"])
    assert_close("HA_d", S.HA_d[idx_t], f["HA_d"])
    assert_close("dX", dX[idx_t], b["dX"])
    # rows outside the sample have dY == 0, hence dX == X-independent LoRA-free zero
    others = torch.ones(cfg.M, dtype=torch.bool, device="cuda")
    others[idx_t] = False
    assert torch.count_nonzero(dX[others]) == 0
    for k in ("dA_g", "dB_g", "dA_u", "dB_u", "dA_d", "dB_d"):
        assert_close(k, grads[k], b[k])


def test_mlp_parity_full_size_dense_llama3_8b(codebook):
    """The Llama-3-8B-shaped block (M=8192, D=4096, I=14336, r=16) at full
    size with dense dY: every LoRA gradient is a sum over all 8192 tokens,
    compared with the oracle's whole-batch forward + backward (run in token
    chunks; about 6 TFLOP of fp64 host work), and Y and dX on every row."""
    cfg = synth.CONFIGS[2]
    print("case", cfg.name, "dense", flush=True)
    P, W, inp = build(cfg, synth.seed_of(2), codebook)
    X, dY = bf16_dev(inp["X"]), bf16_dev(inp["dY"])
    Y, S = q.qlora_mlp_fwd(P, X)
    dX, grads = q.qlora_mlp_bwd(P, dY, X, S)
    torch.cuda.synchronize()
    ref = oq.mlp_forward_backward_rows(inp["X"], inp["dY"], *oracle_args(W, inp), cfg.alpha, chunk=1024,
                                       keep=("Y", "dX"))
    assert_close("Y", Y, ref["Y"])
    assert_close("dX", dX, ref["dX"])
    for k in ("dA_g", "dB_g", "dA_u", "dB_u", "dA_d", "dB_d"):
        assert_close(k, grads[k], ref[k])



# RMSNorm folded into the block's forward: from 512 tokens the norm weight is
# in the expanded gate/up weights and the inverse RMS scales the gate/up
# product; below, the norm runs as its own pass.  Ranks cover the fused HA_d
# (r_d <= 32) and the separate one (r_d = 64, r_g + r_u = 128).
RMS_CASES = [
    synth.MlpCfg("rms_m600_d256_i384_r16", M=600, D=256, I=384, r=16, alpha=16.0, dq_group=0),
    synth.MlpCfg("rms_m777_d192_i320_r20_dq", M=777, D=192, I=320, r=20, alpha=16.0, dq_group=256),
    synth.MlpCfg("rms_m1100_d320_i448_r64", M=1100, D=320, I=448, r=64, alpha=16.0, dq_group=0),
    synth.MlpCfg("rms_m300_d256_i512_r8", M=300, D=256, I=512, r=8, alpha=16.0, dq_group=0),
]


@pytest.mark.parametrize("want_xn", [False, True], ids=["no_xn", "xn"])
@pytest.mark.parametrize("cfg", RMS_CASES, ids=[c.name for c in RMS_CASES])
def test_mlp_rmsnorm_fused_forward(cfg, want_xn, codebook):
    from oracle import rmsnorm as orn
    print("case", cfg.name, want_xn, flush=True)
    P, W, inp = build(cfg, 5000 + cfg.M, codebook)
    M, D, I = cfg.M, cfg.D, cfg.I
    wn = synth.normal_bf16(5000 + cfg.M, 42, D, 1.0, 0.1)
    eps = 1e-5
    X, wd = bf16_dev(inp["X"]), bf16_dev(wn)
    g = Guarded()
    bf, f32 = torch.bfloat16, torch.float32
    S0 = q.MlpSaved(g.empty((M, I), bf), g.empty((M, I), bf), g.empty((M, P.gate.r), f32),
                    g.empty((M, P.up.r), f32), g.empty((M, P.down.r), f32))
    Y, S, rstd, Xn = q.qlora_mlp_fwd_rmsnorm(P, X, wd, eps, Y=g.empty((M, D), bf), saved=S0,
                                             rstd=g.empty((M,), f32), want_xn=want_xn,
                                             Xn=g.empty((M, D), bf) if want_xn else None)
    g.check()
    Xn_o, rstd_o = orn.rmsnorm_forward(inp["X"], wn, eps)
    f = oq.mlp_forward(Xn_o, *oracle_args(W, inp), cfg.alpha)
    assert_close("rstd", rstd, rstd_o, tol=1e-5)
    if want_xn:
        assert_close("Xn", Xn, Xn_o)
    assert_close("Y", Y, f["Y"])
    assert_close("G", S.G, f["G"])
    assert_close("U", S.U, f["U"])
    assert_close("XA_g", S.XA_g, f["XA_g"])
    assert_close("XA_u", S.XA_u, f["XA_u"])
    assert_close("HA_d", S.HA_d, f["HA_d"])
