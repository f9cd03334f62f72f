"""qlora_linear_fwd_static (the entry point that allocates nothing) against
qlora_linear_fwd with a caller workspace: same kernels, same launch plan, so
Y and XA must agree bit for bit, on two calls in a row, the second with fewer
tokens (the library's static scratch then still holds the first call's
partials), and both must meet the oracle's 1e-2 relative Frobenius bar.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import qlora as oq

from gpu_util import assert_close, bf16_dev, make_linear

pytestmark = pytest.mark.gpu

q = pytest.importorskip("qlora_fine_tuning_linear_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.load_library()


def test_static_scratch_forward_matches_workspace_forward(codebook):
    # 300 tokens: the dequant-staged GEMM with two reduction splits (fp32
    # partials in the scratch); 40 tokens: the skinny GEMM with split partials
    # of the rank-r down-projection (also in the scratch)
    base = synth.LinearCfg("static_k1024_n2048_r16", M=300, K=1024, N=2048, r=16, alpha=16.0, dq_group=256)
    inp = synth.linear_inputs(base, 4242)
    L, Wh = make_linear(q, inp["W0"], inp["A"], inp["B"], base.alpha, codebook, base.dq_group)
    for M in (300, 40):
        print("case static forward M=%d" % M, flush=True)
        Xh = inp["X"][:M]
        X = bf16_dev(Xh)
        Ys, XAs = q.qlora_linear_fwd_static(L, X)
        Yw, XAw = q.qlora_linear_fwd(L, X)
        torch.cuda.synchronize()
        assert torch.equal(Ys.view(torch.int16), Yw.view(torch.int16)), "Y differs from the workspace forward"
        assert torch.equal(XAs.view(torch.int32), XAw.view(torch.int32)), "XA differs from the workspace forward"
        Yr, XAr = oq.linear_forward(Xh, Wh, inp["A"], inp["B"], base.alpha)
        assert_close("Y", Ys, Yr)
        assert_close("XA", XAs, XAr)


def test_static_scratch_rejects_oversized_pass():
    # 4096 tokens of an 8192 x 8192 layer: the bf16 weight copy alone is 128 MiB
    w = q.Nf4Weight(torch.empty(8192 * 8192 // 2, dtype=torch.uint8, device="cuda"),
                    torch.empty(8192 * 8192 // 64, dtype=torch.float32, device="cuda"), None, None,
                    torch.empty(16, dtype=torch.float32, device="cuda"), 8192, 8192, 0)
    L = q.QLoraLinear(w, torch.empty(16, 8192, dtype=torch.bfloat16, device="cuda"),
                      torch.empty(8192, 16, dtype=torch.bfloat16, device="cuda"), 16.0)
    X = torch.empty(4096, 8192, dtype=torch.bfloat16, device="cuda")
    Y = torch.full((4096, 8192), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(q.QloraError) as e:
        q.qlora_linear_fwd_static(L, X, Y=Y)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all()), "a rejected call wrote its output"
