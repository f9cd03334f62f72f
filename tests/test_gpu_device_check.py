"""The device check, forced from the host: with the library told that the
device is not a gfx950 (qlora_debug_force_arch), every entry point that would
launch work returns QLORA_ERR_UNSUPPORTED_DEVICE and enqueues nothing (its
outputs keep their contents); restoring the real query makes the same call
work again."""
import numpy as np
import pytest
import torch

import synth

from gpu_util import bf16_dev, make_linear

pytestmark = pytest.mark.gpu

q = pytest.importorskip("qlora_fine_tuning_linear_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.load_library()
    yield
    q.debug_force_arch(None)


def test_forced_other_arch_is_rejected_before_any_work(codebook):
    cfg = synth.LinearCfg("devcheck_m64_256x256_r8", M=64, K=256, N=256, r=8, alpha=16.0, dq_group=0)
    inp = synth.linear_inputs(cfg, 77)
    L, _ = make_linear(q, inp["W0"], inp["A"], inp["B"], cfg.alpha, codebook, 0)
    X, dY = bf16_dev(inp["X"]), bf16_dev(inp["dY"])
    Y = torch.full((cfg.M, cfg.N), 3.0, dtype=torch.bfloat16, device="cuda")
    XA = torch.full((cfg.M, cfg.r), 5.0, dtype=torch.float32, device="cuda")
    dX = torch.full((cfg.M, cfg.K), 3.0, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros(cfg.N, cfg.K, dtype=torch.float32, device="cuda")
    out = torch.full((cfg.N, cfg.K), 2.0, dtype=torch.bfloat16, device="cuda")
    q.debug_force_arch("gfx942")
    try:
        calls = [
            lambda: q.qlora_linear_fwd(L, X, Y=Y, XA=XA),
            lambda: q.qlora_linear_fwd_static(L, X, Y=Y, XA=XA),
            lambda: q.qlora_linear_bwd(L, dY, X, XA, dX=dX),
            lambda: q.nf4_dequantize(L.W0, out=out),
            lambda: q.qlora_merge(L, out=out),
            lambda: q.nf4_quantize(W, L.W0.codebook),
        ]
        for f in calls:
            with pytest.raises(q.QloraError) as e:
                f()
            assert e.value.status == -5, e.value
    finally:
        q.debug_force_arch(None)
    torch.cuda.synchronize()
    assert bool((Y == 3.0).all()) and bool((XA == 5.0).all()) and bool((dX == 3.0).all())
    assert bool((out == 2.0).all())
    # the real device passes again
    Y2, XA2 = q.qlora_linear_fwd(L, X)
    torch.cuda.synchronize()
    assert torch.isfinite(Y2.float()).all()
