"""GPU parity of qlora_linear_fwd / qlora_linear_bwd against the fp64 oracle.

Every floating-point output (Y, XA, dX, dA, dB) must be within relative
Frobenius error 1e-2 of the oracle.  Cases: the single-linear workloads at
their full sizes (M=256 512->512 r=8; M=4096 4096->4096 r=16; M=64
8192->28672 r=16 with double-quantized absmax), ragged token counts and
output widths that leave partial tiles, every rank from 1 to 128, and the
degenerate cases (M=0, alpha=0, B=0).  Launch shapes are the library's own
(the same ones bench.py times).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import qlora as oq

from gpu_util import Guarded, assert_close, bf16_dev, f64_host, make_linear

pytestmark = pytest.mark.gpu

q = pytest.importorskip("qlora_fine_tuning_linear_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.load_library()


def run_case(cfg, seed, codebook, zero_B=False, alpha=None):
    alpha = cfg.alpha if alpha is None else alpha
    inp = synth.linear_inputs(cfg, seed)
    if zero_B:
        inp["B"] = np.zeros_like(inp["B"])
    L, Wh = make_linear(q, inp["W0"], inp["A"], inp["B"], alpha, codebook, cfg.dq_group)
    X, dY = bf16_dev(inp["X"]), bf16_dev(inp["dY"])
    M, K, N, r = cfg.M, cfg.K, cfg.N, cfg.r
    g = Guarded()
    Y, XA = q.qlora_linear_fwd(L, X, Y=g.empty((M, N), torch.bfloat16), XA=g.empty((M, r), torch.float32))
    dX, dA, dB = q.qlora_linear_bwd(L, dY, X, XA, dX=g.empty((M, K), torch.bfloat16),
                                    dA=g.empty((r, K), torch.bfloat16), dB=g.empty((N, r), torch.bfloat16))
    g.check()
    Yr, XAr = oq.linear_forward(inp["X"], Wh, inp["A"], inp["B"], alpha)
    dXr, dAr, dBr = oq.linear_backward(inp["dY"], inp["X"], Wh, inp["A"], inp["B"], alpha)
    return dict(Y=(Y, Yr), XA=(XA, XAr), dX=(dX, dXr), dA=(dA, dAr), dB=(dB, dBr)), L, X, dY


CASES = [
    # the single-linear workloads at full size
    synth.CONFIGS[0],
    synth.CONFIGS[1],
    synth.CONFIGS[4],
    # ragged and odd shapes: partial token tiles, partial column tiles, all ranks
    synth.LinearCfg("m1_64x64_r1", M=1, K=64, N=64, r=1, alpha=2.0, dq_group=0),
    synth.LinearCfg("m33_128x192_r3", M=33, K=128, N=192, r=3, alpha=5.0, dq_group=256),
    synth.LinearCfg("m300_512x320_r16", M=300, K=512, N=320, r=16, alpha=16.0, dq_group=0),
    synth.LinearCfg("m257_256x576_r64", M=257, K=256, N=576, r=64, alpha=16.0, dq_group=256),
    synth.LinearCfg("m129_640x128_r128", M=129, K=640, N=128, r=128, alpha=32.0, dq_group=0),
    synth.LinearCfg("m100_2048x4160_r8", M=100, K=2048, N=4160, r=8, alpha=16.0, dq_group=256),
    synth.LinearCfg("m520_1024x1088_r24", M=520, K=1024, N=1088, r=24, alpha=8.0, dq_group=0),
    synth.LinearCfg("m1300_384x448_r16", M=1300, K=384, N=448, r=16, alpha=16.0, dq_group=256),
    synth.LinearCfg("m2049_192x1216_r40", M=2049, K=192, N=1216, r=40, alpha=20.0, dq_group=0),
    # LoRA-factor transposes above 2 M elements take the tiled form: 64 x 64
    # tiles with 40 live columns (B [53312, 40]) or rows (A [40, 256]), 256 x 16
    # tiles with 12 live columns and a partial last tile (B [200000, 12]), and
    # 16 x 256 tiles (A [12, 256])
    synth.LinearCfg("m300_256x53312_r40", M=300, K=256, N=53312, r=40, alpha=20.0, dq_group=0),
    synth.LinearCfg("m300_256x200000_r12", M=300, K=256, N=200000, r=12, alpha=12.0, dq_group=256),
    # skinny (M <= 64) forward: reduction splits, ragged rows / tokens, wave
    # ranges that leave a partial load ring, the largest rank it takes
    synth.LinearCfg("m16_4096x192_r64", M=16, K=4096, N=192, r=64, alpha=16.0, dq_group=256),
    synth.LinearCfg("m16_256x20032_r8", M=16, K=256, N=20032, r=8, alpha=16.0, dq_group=0),
    synth.LinearCfg("m64_1024x1088_r48", M=64, K=1024, N=1088, r=48, alpha=12.0, dq_group=0),
    synth.LinearCfg("m50_640x4096_r16", M=50, K=640, N=4096, r=16, alpha=16.0, dq_group=256),
    synth.LinearCfg("m7_8192x1024_r32", M=7, K=8192, N=1024, r=32, alpha=8.0, dq_group=0),
    synth.LinearCfg("m64_1024x512_r65", M=64, K=1024, N=512, r=65, alpha=13.0, dq_group=0),
    # skinny backward finish at the largest rank it takes (its LDS is sized
    # by the rank: 66.5 KB at r = 128)
    synth.LinearCfg("m48_1024x2048_r128", M=48, K=1024, N=2048, r=128, alpha=32.0, dq_group=0),
    # skinny forward with 4, 7 and 8 frags of 16 rows per workgroup: tile
    # counts that are not a multiple of 4, ragged rows and tokens, and two
    # reduction splits forced by the absmax staging limit (128 tiles > 124)
    synth.LinearCfg("m64_640x9216_r32", M=64, K=640, N=9216, r=32, alpha=32.0, dq_group=0),
    synth.LinearCfg("m40_1088x16448_r16", M=40, K=1088, N=16448, r=16, alpha=16.0, dq_group=256),
    synth.LinearCfg("m16_8192x32768_r8_split", M=16, K=8192, N=32768, r=8, alpha=16.0, dq_group=0),
    # streaming skinny forward (K a multiple of 256): 1-4 token frags, 1, 2
    # and 7 frags of rows per workgroup, groups of 4 tiles dealt unevenly over
    # the 4 waves (5 groups: 2, 2, 1, 0; 10 groups: 3, 3, 3, 1), reduction
    # splits, ragged rows and tokens, both absmax forms
    synth.LinearCfg("m48_2048x3072_r16", M=48, K=2048, N=3072, r=16, alpha=16.0, dq_group=0),
    synth.LinearCfg("m24_1280x7168_r8_dq", M=24, K=1280, N=7168, r=8, alpha=8.0, dq_group=256),
    synth.LinearCfg("m61_2560x28672_r16", M=61, K=2560, N=28672, r=16, alpha=16.0, dq_group=0),
    synth.LinearCfg("m9_4096x28608_r64_dq", M=9, K=4096, N=28608, r=64, alpha=32.0, dq_group=256),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_linear_parity(cfg, codebook):
    print("case", cfg.name, flush=True)
    out, *_ = run_case(cfg, 2000 + CASES.index(cfg), codebook)
    for k, (g, r) in out.items():
        assert_close(k, g, r)


def test_alpha_zero_is_base_matmul(codebook):
    cfg = synth.LinearCfg("a0", M=96, K=256, N=192, r=8, alpha=0.0, dq_group=0)
    out, *_ = run_case(cfg, 77, codebook)
    assert_close("Y", *out["Y"])
    # with alpha == 0 the LoRA gradients are exactly zero
    for k in ("dA", "dB"):
        assert np.all(f64_host(out[k][0]) == 0)


def test_b_zero_gives_exact_zero_dA(codebook):
    cfg = synth.LinearCfg("b0", M=200, K=256, N=320, r=16, alpha=16.0, dq_group=256)
    out, *_ = run_case(cfg, 78, codebook, zero_B=True)
    assert np.all(f64_host(out["dA"][0]) == 0)
    for k in ("Y", "XA", "dX", "dB"):
        assert_close(k, *out[k])


def test_m_zero(codebook):
    cfg = synth.LinearCfg("m0", M=4, K=128, N=128, r=4, alpha=4.0, dq_group=0)
    inp = synth.linear_inputs(cfg, 5)
    L, _ = make_linear(q, inp["W0"], inp["A"], inp["B"], 4.0, codebook, 0)
    X = torch.empty(0, 128, dtype=torch.bfloat16, device="cuda")
    Y, XA = q.qlora_linear_fwd(L, X)
    assert Y.shape == (0, 128)
    dA = torch.full_like(L.A, 3.0)
    dB = torch.full_like(L.B, 3.0)
    q.qlora_linear_bwd(L, torch.empty(0, 128, dtype=torch.bfloat16, device="cuda"), X, XA, dA=dA, dB=dB)
    torch.cuda.synchronize()
    assert torch.all(dA == 0) and torch.all(dB == 0)


def test_skinny_forward_is_bitwise_deterministic(codebook):
    cfg = synth.LinearCfg("det_skinny", M=48, K=2048, N=640, r=16, alpha=16.0, dq_group=256)
    out, L, X, dY = run_case(cfg, 10, codebook)
    for _ in range(2):
        Y2, XA2 = q.qlora_linear_fwd(L, X)
        assert torch.equal(Y2.view(torch.int16), out["Y"][0].view(torch.int16))
        assert torch.equal(XA2, out["XA"][0])


def test_backward_is_bitwise_deterministic(codebook):
    cfg = synth.LinearCfg("det", M=1000, K=1024, N=768, r=16, alpha=16.0, dq_group=0)
    out, L, X, dY = run_case(cfg, 9, codebook)
    XA = out["XA"][0]
    a = q.qlora_linear_bwd(L, dY, X, XA)
    b = q.qlora_linear_bwd(L, dY, X, XA)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    Y2, XA2 = q.qlora_linear_fwd(L, X)
    assert torch.equal(Y2.view(torch.int16), out["Y"][0].view(torch.int16))
    assert torch.equal(XA2, XA)
