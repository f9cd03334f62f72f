"""GPU parity of the packed-adapter entry points (qlora_grouped_fwd / _bwd)
against the oracle's separate QLoRA linears, one per group.

The packed layer is the row-concatenation of the groups' weights, quantized as
one NF4 tensor (blocks never straddle rows, so its codes are those of the
separate weights); the oracle runs linear_forward / linear_backward on each
group's row block with that group's A, B and alpha, and the expected outputs
are the concatenated Y and XA, the summed dX and the per-group dA, dB.

Cases: the Llama-3-8B q/k/v shapes (K=4096, N = 4096 / 1024 / 1024, r=16) on
both GEMM paths (256 and 1024 tokens); a ragged group set with different
ranks and scales that are not powers of two (so the packed B is rounded);
G = 1; the skinny path (33 tokens); ranks <= 16 with group boundaries on and
off multiples of 128 rows (dB reduced per group, or as the whole
block-diagonal gradient); M = 0.  Bar: relative Frobenius error 1e-2 on every
output.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import nf4 as onf4
from oracle import qlora as oq

from gpu_util import assert_close, bf16_dev, quantize_both, assert_codes_equal

pytestmark = pytest.mark.gpu

q = pytest.importorskip("qlora_fine_tuning_linear_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.load_library()


def _bf16(seed, stream, shape, std=1.0, mean=0.0):
    return synth.normal_bf16(seed, stream, int(np.prod(shape)), mean, std).reshape(shape)


def _case(K, Ns, rs, alphas, M, dq, seed, codebook):
    Nt = sum(Ns)
    W = synth.weight_rows(seed, 2, K, 0, Nt)
    bound = 1.0 / np.sqrt(K)
    A = synth.uniform_bf16(seed, 3, sum(rs) * K, -bound, bound).reshape(sum(rs), K)
    Bs = [_bf16(seed, 10 + g, (Ns[g], rs[g]), 0.01) for g in range(len(Ns))]
    X = _bf16(seed, 4, (M, K))
    dY = _bf16(seed, 5, (M, Nt))
    qw, ow = quantize_both(W, codebook, dq, q)
    assert_codes_equal(qw, ow)
    Wh = onf4.dequantize(ow, codebook).astype(np.float64)
    Q = q.QLoraGrouped(qw, bf16_dev(A), [bf16_dev(B) for B in Bs], list(alphas))
    return Q, Wh, A, Bs, X, dY


def _check(Q, Wh, A, Bs, X, dY, alphas):
    Ns, rs = [B.shape[0] for B in Bs], [B.shape[1] for B in Bs]
    Xd, dYd = bf16_dev(X), bf16_dev(dY)
    Y, XA = q.qlora_grouped_fwd(Q, Xd)
    dX, dA, dBs = q.qlora_grouped_bwd(Q, dYd, Xd, XA)
    torch.cuda.synchronize()
    n0 = r0 = 0
    Yr, XAr, dXr, dAr = [], [], 0.0, []
    for g in range(len(Ns)):
        Wg, Ag = Wh[n0:n0 + Ns[g]], A[r0:r0 + rs[g]]
        y, xa = oq.linear_forward(X, Wg, Ag, Bs[g], alphas[g])
        dx, da, db = oq.linear_backward(dY[:, n0:n0 + Ns[g]], X, Wg, Ag, Bs[g], alphas[g])
        Yr.append(y)
        XAr.append(xa)
        dXr = dXr + dx
        dAr.append(da)
        assert_close("dB_%d" % g, dBs[g], db)
        n0 += Ns[g]
        r0 += rs[g]
    assert_close("Y", Y, np.concatenate(Yr, axis=1))
    assert_close("XA", XA, np.concatenate(XAr, axis=1))
    assert_close("dX", dX, dXr)
    assert_close("dA", dA, np.concatenate(dAr, axis=0))


# (name, K, Ns, rs, alphas, M, dq, seed)
CASES = [
    ("qkv_8b_m256", 4096, [4096, 1024, 1024], [16, 16, 16], [16.0, 16.0, 16.0], 256, 0, 3001),
    ("qkv_8b_m1024", 4096, [4096, 1024, 1024], [16, 16, 16], [16.0, 16.0, 16.0], 1024, 0, 3002),
    ("ragged_scales_dq", 512, [192, 64, 128], [8, 24, 5], [16.0, 8.0, 3.0], 70, 256, 3003),
    ("single_group", 256, [128], [12], [24.0], 100, 0, 3004),
    ("skinny_m33", 1024, [256, 256], [16, 16], [16.0, 32.0], 33, 256, 3005),
    # ranks <= 16 and group boundaries on 128-row multiples: dB reduced per
    # group against its own ranks of XA (last 128-column wave ragged, ragged
    # token tail); then the same ranks with a boundary off the 128 grid
    ("per_group_db_m777", 512, [256, 384, 192], [16, 5, 11], [16.0, 7.0, 3.0], 777, 0, 3007),
    ("unaligned_groups_m300", 512, [192, 320], [16, 8], [16.0, 5.0], 300, 256, 3008),
]


@pytest.mark.parametrize("name,K,Ns,rs,alphas,M,dq,seed", CASES, ids=[c[0] for c in CASES])
def test_grouped_matches_separate_layers(name, K, Ns, rs, alphas, M, dq, seed, codebook):
    print("case", name, flush=True)
    Q, Wh, A, Bs, X, dY = _case(K, Ns, rs, alphas, M, dq, seed, codebook)
    _check(Q, Wh, A, Bs, X, dY, alphas)


def test_grouped_empty_batch(codebook):
    print("case empty", flush=True)
    Q, _, _, _, _, _ = _case(256, [64, 128], [8, 8], [16.0, 16.0], 1, 0, 3006, codebook)
    X = torch.empty(0, 256, dtype=torch.bfloat16, device="cuda")
    Y, XA = q.qlora_grouped_fwd(Q, X)
    assert Y.shape == (0, 192)
    dX, dA, dBs = q.qlora_grouped_bwd(Q, torch.empty(0, 192, dtype=torch.bfloat16, device="cuda"), X, XA)
    assert torch.count_nonzero(dA).item() == 0
    assert all(torch.count_nonzero(b).item() == 0 for b in dBs)
