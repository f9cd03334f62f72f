"""HIP graph capture of whole QLoRA steps through the C ABI.

A call of the library only enqueues kernels on the caller's stream (no
allocation, no memset, no host synchronization), so a caller can capture a
forward + backward step into a HIP graph and replay it.  Each case captures
one step with every output and workspace preallocated, then replays it
several times with eager work and new input values in between; every replay
must equal an eager run of the same step on the same inputs bit for bit (the
library's kernels are deterministic), which also shows that the graph reads
the buffers' current contents.  Cases cover the three token-count regimes of
the linear layer (skinny <= 64 tokens, in-GEMM expansion, expand once + bf16
GEMM) and of the MLP.
"""
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


def _bits(t):
    return t.contiguous().view(torch.uint8)


def _capture(step):
    """Warm the step up on a side stream, then capture it into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def _check_replays(g, step, inputs, outputs, seed, replays=3):
    rng = np.random.default_rng(seed)
    for it in range(replays):
        # new input values in the captured buffers (eager copies)
        for t in inputs:
            t.copy_(torch.from_numpy(rng.standard_normal(tuple(t.shape)).astype(np.float32)).to(t.device, t.dtype))
        step()
        torch.cuda.synchronize()
        ref = [_bits(o).clone() for o in outputs]
        for o in outputs:
            _bits(o).fill_(0xA5)
        g.replay()
        torch.cuda.synchronize()
        for k, (o, r) in enumerate(zip(outputs, ref)):
            assert torch.equal(_bits(o), r), "replay %d: output %d differs from the eager step" % (it, k)


LIN = [
    synth.LinearCfg("skinny_m48_1024x2048_r16_dq", M=48, K=1024, N=2048, r=16, alpha=16.0, dq_group=256),
    synth.LinearCfg("fused_m200_512x768_r8", M=200, K=512, N=768, r=8, alpha=16.0, dq_group=0),
    synth.LinearCfg("bf16_m600_512x768_r16", M=600, K=512, N=768, r=16, alpha=16.0, dq_group=0),
]


@pytest.mark.parametrize("cfg", LIN, ids=[c.name for c in LIN])
def test_linear_step_replays_match_eager(cfg, codebook):
    print("case", cfg.name, flush=True)
    inp = synth.linear_inputs(cfg, 4100 + cfg.M)
    L, _ = make_linear(q, inp["W0"], inp["A"], inp["B"], cfg.alpha, codebook, cfg.dq_group)
    M, K, N, r = cfg.M, cfg.K, cfg.N, cfg.r
    dev = "cuda"
    X, dY = bf16_dev(inp["X"]), bf16_dev(inp["dY"])
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    XA = torch.empty(M, r, dtype=torch.float32, device=dev)
    dX = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    dA = torch.empty(r, K, dtype=torch.bfloat16, device=dev)
    dB = torch.empty(N, r, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(256, q.qlora_linear_workspace_bytes(L, M)), dtype=torch.uint8, device=dev)

    def step():
        q.qlora_linear_fwd(L, X, Y=Y, XA=XA, ws=ws)
        q.qlora_linear_bwd(L, dY, X, XA, dX=dX, dA=dA, dB=dB, ws=ws)

    g = _capture(step)
    _check_replays(g, step, [X, dY], [Y, XA, dX, dA, dB], seed=cfg.M)


MLP = [
    synth.MlpCfg("fused_m300_d256_i512_r8", M=300, D=256, I=512, r=8, alpha=16.0, dq_group=0),
    synth.MlpCfg("bf16_m520_d256_i384_r16_dq", M=520, D=256, I=384, r=16, alpha=16.0, dq_group=256),
]


@pytest.mark.parametrize("cfg", MLP, ids=[c.name for c in MLP])
def test_mlp_step_replays_match_eager(cfg, codebook):
    print("case", cfg.name, flush=True)
    inp = synth.mlp_inputs(cfg, 4200 + cfg.M)
    gl, _ = make_linear(q, inp["Wg"], inp["Ag"], inp["Bg"], cfg.alpha, codebook, cfg.dq_group)
    ul, _ = make_linear(q, inp["Wu"], inp["Au"], inp["Bu"], cfg.alpha, codebook, cfg.dq_group)
    dl, _ = make_linear(q, inp["Wd"], inp["Ad"], inp["Bd"], cfg.alpha, codebook, cfg.dq_group)
    P = q.QLoraMlp(gl, ul, dl)
    M, D = cfg.M, cfg.D
    dev = "cuda"
    X, dY = bf16_dev(inp["X"]), bf16_dev(inp["dY"])
    Y = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    saved = q.alloc_mlp_saved(P, M, dev)
    dX = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    grads = dict(dA_g=torch.empty_like(gl.A), dB_g=torch.empty_like(gl.B), dA_u=torch.empty_like(ul.A),
                 dB_u=torch.empty_like(ul.B), dA_d=torch.empty_like(dl.A), dB_d=torch.empty_like(dl.B))
    ws = torch.empty(max(256, q.qlora_mlp_workspace_bytes(P, M)), dtype=torch.uint8, device=dev)

    def step():
        q.qlora_mlp_fwd(P, X, Y=Y, saved=saved, ws=ws)
        q.qlora_mlp_bwd(P, dY, X, saved, dX=dX, grads=grads, ws=ws)

    g = _capture(step)
    outs = [Y, saved.G, saved.U, saved.XA_g, saved.XA_u, saved.HA_d, dX] + [grads[k] for k in sorted(grads)]
    _check_replays(g, step, [X, dY], outs, seed=cfg.M)
